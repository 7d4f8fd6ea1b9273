/*
 * moe_q4.h -- C ABI of the MI355X (gfx950) sigmoid-routed Q4 MoE expert layer.
 *
 * The layer (sources are pages of pull-request text, cited by title):
 *   - "feat(laguna): Laguna-S-2.1 decode on the CUDA engine"
 *     (thewafflehaus/butter pull request 69): a hybrid MoE whose router is
 *     a sigmoid top-10 with a score-correction bias, plus an always-on
 *     shared expert; Q4-requantised expert weights; decode runs the experts
 *     as gathered Q4 GEMVs, gate+up fused with SwiGLU, the shared expert in
 *     the same gather.
 *   - "feat(laguna): batched prefill with tensor-core projections, fused
 *     MoE, CTA scheduling" (same pull request; thewafflehaus/FFAI pull
 *     request 70): grouped-GEMM MoE with descriptors built on the device,
 *     fused gate+up expert stacks, descending-size expert order and an
 *     N-banded workgroup order for weight reuse in cache.
 *   - thewafflehaus/FFAI pull request 72, the Nemotron MoE commits: CSR
 *     offsets and router-sorted token indices, gather-on-read, a
 *     deterministic non-atomic scatter-add, routed+shared summed before
 *     anything else ("ffai_add3"), a K-loop that must not read past a
 *     weight buffer (tile-select fix), and no device-to-host copy inside a
 *     captured stream.
 *
 * What one layer call computes, for every token t (x_t in R^d):
 *   l    = W_r x_t                       router logits, fp32 accumulate
 *   s    = 1 / (1 + exp(-l))             sigmoid scores
 *   sel  = the k experts with the largest s + b (ties: lower id first),
 *          listed by descending s + b -- the bias b only selects
 *   w_j  = s[sel_j] / sum_j s[sel_j]    unbiased, normalised to 1
 *   h_e  = silu(W_g[e] x_t) * (W_u[e] x_t),  y_e = W_d[e] h_e
 *   y_t  = (sum_{j=0..k-1} w_j * y_{sel_j}) + y_shared(x_t)
 * Routed terms are summed in j order, then the shared expert is added
 * (moe_q4_forward_residual then adds a residual).
 * No float atomics anywhere: results are bitwise reproducible run to run.
 *
 * Conventions for every call
 *   - Every array argument is a DEVICE pointer owned by the caller, who
 *     keeps it alive until the work enqueued on `stream` has finished.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue kernels: they never allocate, free, synchronise or copy
 *     device-to-host, so they can be captured into a HIP graph.
 *   - All arguments are validated on the host before any HIP call; a
 *     failed check returns a negative MOE_E* code and enqueues nothing.
 *   - MOE_EHIP is returned when a kernel launch is rejected by the runtime
 *     (the error reported by hipGetLastError right after the launch).
 *   - Expert ids passed back in (topk_ids) must lie in [0, E); this is not
 *     checked on the device.
 *   - With MOE_ROCTX=1 in the environment, every call that enqueues work is
 *     wrapped in a roctx range named after it (for rocprofv3
 *     --marker-trace); the roctx library is looked up at run time and the
 *     ranges stay off without it.
 *
 * Storage formats
 *   x         bf16 bit patterns, row-major [T][d]
 *   w_router  float32 [E][d];   bias  float32 [E]
 *   y         float32 [T][d]
 *   Q4 matrix of shape [rows][K] (K % 32 == 0, rows % 16 == 0): 32-element
 *   blocks of 16 code bytes and one fp16 scale, stored in groups of 16 rows
 *   so that the 16 rows x 4 blocks one load instruction needs are one
 *   contiguous KiB (codes) and 128 bytes (scales):
 *     qs      uint8 [rows/16][K/32][16][16]: the 16-byte block b of row r
 *             starts at byte ((r/16)*(K/32) + b)*256 + (r%16)*16; inside a
 *             block, byte i holds element 2i in its low nibble and element
 *             2i+1 in its high nibble
 *     scales  uint16 [rows/16][K/32][16]: IEEE fp16 bits; the scale of row
 *             r, block b is element ((r/16)*(K/32) + b)*16 + r%16
 *     value = (q - 8) * scale          (q the 4-bit code, 0..15)
 *   Both are index permutations of the row-major arrays [rows][K/2] and
 *   [rows][K/32]; moe_q4_pack (below) performs it on the device.
 *   w13  [E][2I][d]  gate rows 0..I-1, up rows I..2I-1 of every expert
 *   w2   [E][d][I]
 *   s13  [2*I_shared][d], s2 [d][I_shared]   (shared expert, same split)
 *
 * Two execution paths, chosen on the host from T alone (or forced by the
 * flags below, identically in all three calls):
 *   small-T path (T <= MOE_GEMV_MAX_T): the router runs as a GEMV, no
 *     routing build is needed, and every (token, expert) pair streams its
 *     expert rows through a fused dequant-GEMV with SwiGLU; the down
 *     projection is fused with the combine.
 *   grouped path (larger T): an MFMA router GEMM, an on-device routing
 *     build (histogram, scan, stable scatter, group order, tile counts),
 *     and grouped GEMMs that dequantise Q4 in registers into fp16 MFMA
 *     operands, with the shared expert as one more always-present group,
 *     then a fixed-order combine.
 *   Both paths round x to fp16 for the expert projections and keep the
 *   SwiGLU outputs in fp16 between the two projections; the grouped path
 *   also stores every expert's down-projection output in fp16 before the
 *   combine.  On both paths the same three quantities -- x as the experts
 *   see it, h, and each expert's output before the routing weight -- are
 *   saturated to the fp16 range: a value beyond +-65504 becomes +-65504,
 *   one inside it is rounded to nearest even.  Finite inputs never give Inf
 *   or NaN; results are accurate while those values stay inside the range
 *   (the router always sees the unsaturated bf16 x).  Inf/NaN inputs are
 *   outside the contract.
 */
#ifndef MOE_Q4_H
#define MOE_Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---------------------------------------------------- */
#define MOE_OK            0
#define MOE_EINVAL       (-1)  /* null pointer, non-positive size, k > E          */
#define MOE_EALIGN       (-2)  /* an array not 16-byte aligned                    */
#define MOE_EUNSUPPORTED (-3)  /* d, I or I_shared not a multiple of 32, E > 1024,
                                  k > 32, or a size beyond the chosen path's range:
                                  small-T path d <= 8192, I, I_shared <= 2048, T <= 64;
                                  grouped path max(I, I_shared) * d < 2^31 (32-bit
                                  offsets into one expert's weights); both paths
                                  (T*k + T) * max(d, I) < 2^31 */
#define MOE_ENOSPACE     (-4)  /* routing workspace or scratch smaller than needed */
#define MOE_EHIP         (-5)  /* the HIP runtime rejected a kernel launch          */

/* ---- flags (pass the same value to all three calls) ------------------- */
#define MOE_FLAG_DEFAULT      0u
#define MOE_FLAG_FORCE_GROUPED 1u  /* grouped path even when T is small            */
#define MOE_FLAG_FORCE_GEMV    2u  /* small-T path even when T is larger (T <= 64)  */
#define MOE_FLAG_ID_ORDER      4u  /* schedule groups in id order, not by size     */
#define MOE_FLAG_NO_BANDING    8u  /* grouped GEMMs: workgroups in plain item order  */
#define MOE_FLAG_BAND_MAJOR   16u  /* grouped GEMMs: N-banded order, all M-tiles of a
                                      weight band on one XCD (weight reuse in L2)  */

#define MOE_GEMV_MAX_T      8    /* default small-T threshold                       */
#define MOE_GEMV_FORCE_MAX_T 64  /* largest T the small-T path accepts              */

typedef struct moe_dims {
  int32_t T;         /* tokens in this call                         */
  int32_t d;         /* hidden size                                 */
  int32_t E;         /* routed experts                              */
  int32_t k;         /* experts chosen per token                    */
  int32_t I;         /* routed expert intermediate size             */
  int32_t I_shared;  /* shared expert intermediate size             */
} moe_dims;

typedef struct moe_q4 {
  const uint8_t*  qs;      /* [rows/16][K/32][16][16] codes, 16-byte aligned */
  const uint16_t* scales;  /* [rows/16][K/32][16] fp16 bits, 16-byte aligned */
} moe_q4;

typedef struct moe_q4_weights {
  moe_q4 w13;  /* [E][2I][d]                */
  moe_q4 w2;   /* [E][d][I]                 */
  moe_q4 s13;  /* [2*I_shared][d]           */
  moe_q4 s2;   /* [d][I_shared]             */
} moe_q4_weights;

/* Byte offsets of the regions inside the routing workspace, so that tests
 * and tools can read what the routing build wrote.  Sizes are in elements.
 * Pairs are p = t*k + j; groups are the E experts plus the shared expert
 * as group E. */
typedef struct moe_routing_layout {
  size_t logits;       /* float [8][T][E]   router logits (scratch of moe_route; the
                          grouped path's router writes 8 partial sums over K) */
  size_t counts;       /* int32 [E+1]       rows per group (group E = T)         */
  size_t offsets;      /* int32 [E+1]       CSR exclusive prefix over experts     */
  size_t sorted_pair;  /* int32 [P]         pair id at each sorted position       */
  size_t pair_pos;     /* int32 [P]         sorted position of each pair          */
  size_t row_expert;   /* int32 [P]         expert of each sorted position        */
  size_t group_order;  /* int32 [E+1]       groups in schedule order              */
  size_t mt_prefix;    /* int32 [E+2]       exclusive prefix of M-tiles per order */
  size_t chunk_counts; /* int32 [chunks][E] per-chunk histogram (build scratch)   */
  size_t total;        /* bytes required                                          */
} moe_routing_layout;

/* 0 when the shape is supported on the path `flags` selects, else a
 * negative code.  Host only. */
int moe_supports(const moe_dims* dims, uint32_t flags);

/* Path `flags` selects for this shape: 0 = small-T GEMV path, 1 = grouped. */
int moe_path(const moe_dims* dims, uint32_t flags);

/* Routing workspace size in bytes (0 if the shape is unsupported). */
size_t moe_routing_bytes(const moe_dims* dims, uint32_t flags);

/* Fill `out` with the routing workspace layout.  Returns MOE_OK or a code. */
int moe_routing_layout_of(const moe_dims* dims, uint32_t flags, moe_routing_layout* out);

/* Scratch size in bytes needed by moe_q4_forward (0 if unsupported). */
size_t moe_scratch_bytes(const moe_dims* dims, uint32_t flags);

/* Router and expert selection: page "feat(laguna): Laguna-S-2.1 decode on
 * the CUDA engine" (thewafflehaus/butter pull request 69), the sigmoid
 * top-10 router with a score-correction bias that only ranks the experts.
 * For every token t: l = W_r x_t (fp32 accumulate), s = sigmoid(l), the k
 * experts with the largest s + b (ties to the lower id) listed by descending
 * s + b, and weights s_j / sum s_j.
 * x_bf16 [T][d] (16-byte aligned), w_router float [E][d] (16-byte aligned),
 * bias float [E]: inputs.  topk_ids int32 [T][k], topk_w float [T][k]:
 * outputs.  routing: the caller's routing workspace (moe_routing_bytes); its
 * logits region is used as scratch.  MOE_EINVAL (NULL pointer, bad dims or
 * flags), MOE_EALIGN, MOE_EUNSUPPORTED, MOE_ENOSPACE, MOE_EHIP. */
int moe_route(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router,
              const float* bias, int32_t* topk_ids, float* topk_w,
              void* routing, size_t routing_bytes, uint32_t flags, void* stream);

/* Routing build for the grouped path: page "feat(laguna): batched prefill
 * with tensor-core projections, fused MoE, CTA scheduling" (grouped-GEMM MoE
 * with descriptors built on the device, descending-size expert order) and
 * the Nemotron MoE commits of thewafflehaus/FFAI pull request 72 (one
 * device-side fill from the router's CSR offsets; router-sorted token
 * indices; the expert id of every sorted row expanded from the offsets).
 * Writes into `routing`: per-expert counts, CSR offsets, the stable (expert,
 * token) order of the pairs and its inverse, the expert of every sorted row,
 * the group schedule order (largest first, ties to the lower id;
 * MOE_FLAG_ID_ORDER: id order) and the M-tile prefix (layout:
 * moe_routing_layout_of).  topk_ids int32 [T][k] is the input (values in
 * [0, E)).  On the small-T path it enqueues nothing and returns MOE_OK.
 * MOE_EINVAL, MOE_EALIGN, MOE_EUNSUPPORTED, MOE_ENOSPACE, MOE_EHIP. */
int moe_build_descriptors(const moe_dims* dims, const int32_t* topk_ids,
                          void* routing, size_t routing_bytes, uint32_t flags,
                          void* stream);

/* Expert computation and combine: page "feat(laguna): Laguna-S-2.1 decode on
 * the CUDA engine" (SwiGLU experts over Q4 weights, gate and up fused, the
 * shared expert always on) and the Nemotron MoE commits of
 * thewafflehaus/FFAI pull request 72 (gather-on-read through the sorted
 * token indices, a deterministic scatter-add, "ffai_add3": routed terms
 * summed first, then the shared expert).  For every token
 *   y_t = (sum_{j=0..k-1} w_tj * W_d[e] (silu(W_g[e] x_t) * (W_u[e] x_t)))
 *         + W_sd (silu(W_sg x_t) * (W_su x_t)),  e = topk_ids[t][j],
 * summed in j order without atomics (bitwise reproducible).
 * x_bf16 [T][d], topk_ids, topk_w [T][k] (as written by moe_route) and the
 * Q4 weights are inputs; y float [T][d] (16-byte aligned) is the output.
 * `routing` must hold what moe_build_descriptors wrote for the same
 * topk_ids (grouped path only; may be NULL on the small-T path); `scratch`
 * holds intermediate activations and per-pair outputs and needs
 * moe_scratch_bytes() bytes.  MOE_EINVAL, MOE_EALIGN, MOE_EUNSUPPORTED,
 * MOE_ENOSPACE, MOE_EHIP. */
int moe_q4_forward(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids,
                   const float* topk_w, const void* routing, size_t routing_bytes,
                   const moe_q4_weights* weights, float* y, void* scratch,
                   size_t scratch_bytes, uint32_t flags, void* stream);

/* moe_q4_forward followed by a residual add, in one pass over y:
 *   y_t = ((sum_j w_j * y_{sel_j}) + y_shared(x_t)) + residual_t
 * (routed and shared summed first, then the residual: page thewafflehaus/FFAI
 * pull request 72, "ffai_add3", whose order keeps the routed + shared sum
 * independent of the residual's magnitude).  `residual` is a DEVICE array
 * float32 [T][d], 16-byte aligned, never NULL; it may be `y` itself (each
 * element is read before it is overwritten, by the same thread).  Every
 * other argument, error and the behaviour are those of moe_q4_forward. */
int moe_q4_forward_residual(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids,
                            const float* topk_w, const void* routing, size_t routing_bytes,
                            const moe_q4_weights* weights, const float* residual, float* y, void* scratch,
                            size_t scratch_bytes, uint32_t flags, void* stream);

/* The whole layer in one call: moe_route, moe_build_descriptors and
 * moe_q4_forward (residual NULL) or moe_q4_forward_residual (residual given,
 * same rules) with the same arguments, giving the same topk_ids, topk_w and
 * y bit for bit.  Page "feat(laguna): Laguna-S-2.1 decode on the CUDA engine"
 * runs the decode layer as one recorded sequence of launches; here, on the
 * small-T (GEMV) path, the top-k is not a launch of its own: every gate+up
 * workgroup of a routed pair selects its token's experts from the router's
 * logits itself (the same selection), and one of them per token writes
 * topk_ids / topk_w, so a decode layer is three launches.  Every argument is
 * checked before the first launch (MOE_EINVAL, MOE_EALIGN, MOE_EUNSUPPORTED,
 * MOE_ENOSPACE as for the separate calls); MOE_EHIP if a launch fails.
 * topk_ids / topk_w are outputs, as for moe_route; routing and scratch are
 * sized by moe_routing_bytes / moe_scratch_bytes. */
int moe_layer_forward(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router, const float* bias,
                      const moe_q4_weights* weights, const float* residual, float* y, int32_t* topk_ids,
                      float* topk_w, void* routing, size_t routing_bytes, void* scratch, size_t scratch_bytes,
                      uint32_t flags, void* stream);

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call without the routing and scratch arguments.  The
 * routing workspace and the scratch live in one device array of the
 * library's own, MOE_NOALLOC_MAX_BYTES per GPU, reserved when the library is
 * loaded and held until the process ends; nothing is allocated or freed.
 * The shape must fit: moe_routing_bytes + moe_scratch_bytes (each rounded
 * up to a multiple of 256) <= MOE_NOALLOC_MAX_BYTES, else MOE_ENOSPACE
 * (64 MiB holds the d = 4096, E = 256, top-10, I = 1024 layer up to about
 * T = 480 tokens).  Every other argument, check, error and result is that of
 * moe_layer_forward, bit for bit.  All calls on one GPU share the array, so
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and give undefined results; calls on different GPUs do not interact.  The
 * first call on a device looks the array up for that device (a HIP runtime
 * query, no allocation); MOE_EHIP if that fails. */
#define MOE_NOALLOC_MAX_BYTES (64ull << 20)
int moe_layer_forward_noalloc(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router,
                              const float* bias, const moe_q4_weights* weights, const float* residual, float* y,
                              int32_t* topk_ids, float* topk_w, uint32_t flags, void* stream);

/* Pre-MoE norm (the step in front of the layer): for each of T rows of d
 * values (d % 8 == 0),
 *     x_t = bf16( h_t / sqrt(mean(h_t^2) + eps) * gamma )
 * rounded to nearest even: the standard RMSNorm.  The pages name RMSNorm
 * (per-head QK RMSNorm in "feat(laguna): Laguna-S-2.1 decode on the CUDA
 * engine", a fused add-RMSNorm op) without defining the norm in front of
 * the MoE block; this is the plain reading.  h float32 [T][d], gamma
 * float32 [d] and x_bf16 uint16 [T][d] are DEVICE arrays, 16-byte aligned;
 * the mean of squares is summed in fp32 in a fixed order (deterministic).
 * MOE_EINVAL: T or d < 1, a NULL pointer, eps negative or not finite;
 * MOE_EUNSUPPORTED: d % 8 != 0 or d > 2^20; MOE_EALIGN; MOE_EHIP. */
int moe_rmsnorm_bf16(int T, int d, const float* h, const float* gamma, float eps, uint16_t* x_bf16,
                     void* stream);

/* ---- Multi-layer decode context ------------------------------------------
 * Page "feat(laguna): Laguna-S-2.1 decode on the CUDA engine" runs decode as
 * one captured graph over every layer, replayed each step, with a persistent
 * workspace.  A context does that for a stack of MoE layers of one shape:
 * the layer input is taken from a residual stream h (float32 [T][d]) and the
 * layer output is added back to it,
 *     for l in 0 .. n_layers-1:   x = bf16(h);   h = moe_layer_l(x) + h
 * with bf16() rounding to nearest even and the residual added after the
 * routed + shared sum (as moe_q4_forward_residual); a layer with a norm
 * weight takes x through the pre-MoE norm instead (moe_rmsnorm_bf16).  The
 * attention blocks a model has between its MoE layers are not part of it. */
typedef struct moe_layer {
  const float* w_router;   /* DEVICE float32 [E][d], 16-byte aligned        */
  const float* bias;       /* DEVICE float32 [E]                              */
  moe_q4_weights weights;  /* DEVICE Q4 stacks as for moe_q4_forward           */
  const float* norm_weight;  /* DEVICE float32 [d] (16-byte aligned), or NULL:
                                with it the layer's input is the pre-MoE norm
                                x = bf16(rmsnorm(h) * norm_weight), see
                                moe_rmsnorm_bf16; without it x = bf16(h)      */
  float norm_eps;          /* eps of that norm (>= 0, finite)                 */
} moe_layer;

typedef struct moe_decode_ctx moe_decode_ctx;  /* opaque */

/* Bytes of the caller-owned device workspace a context needs (0 if the
 * shape or flags are unsupported): the bf16 layer input, the selection, one
 * routing workspace and one scratch buffer, shared by the layers, which run
 * one after another. */
size_t moe_decode_ctx_workspace_bytes(const moe_dims* dims, uint32_t flags);

/* Record the whole stack once into a HIP graph.  `layers` (n_layers >= 1,
 * host array, read during the call only) and every device pointer in it,
 * `h` (DEVICE float32 [T][d], 16-byte aligned) and `workspace` (DEVICE, 16-
 * byte aligned, at least moe_decode_ctx_workspace_bytes) stay owned by the
 * caller and must outlive the context; the graph keeps their addresses.
 * The library allocates no device memory: the context holds only host-side
 * objects (the graph and its executable form).  Every argument is checked
 * before the first HIP call (MOE_EINVAL, MOE_EALIGN, MOE_EUNSUPPORTED,
 * MOE_ENOSPACE as for the layer calls; n_layers outside 1..4096 or a norm
 * eps that is negative or not finite is MOE_EINVAL); a HIP failure while
 * recording gives MOE_EHIP.  The stack is recorded on a stream of the
 * context's own in thread-local capture mode, so the calling thread must not
 * be recording a graph itself.  Nothing runs until moe_decode_ctx_run.  On
 * success *out receives the context. */
int moe_decode_ctx_create(const moe_dims* dims, int n_layers, const moe_layer* layers, float* h, void* workspace,
                          size_t workspace_bytes, uint32_t flags, moe_decode_ctx** out);

/* Enqueue one pass of the recorded stack on `stream` (any stream, also the
 * null stream): h is updated in place.  Passes on one context must not
 * overlap (they share the workspace and h).  MOE_EINVAL for a NULL context,
 * MOE_EHIP if the launch fails. */
int moe_decode_ctx_run(moe_decode_ctx* ctx, void* stream);

/* Release the context's host objects (NULL is allowed).  Work already
 * enqueued by moe_decode_ctx_run completes normally. */
int moe_decode_ctx_destroy(moe_decode_ctx* ctx);

/* Repack Q4 matrices from the plain row-major layout into the 16-row groups
 * every other call reads, on the device (page "feat(laguna): Laguna-S-2.1
 * decode on the CUDA engine" loads its Q4-requantised weights once and keeps
 * them resident; this is the one-time step at load).  n_mats matrices of
 * shape [rows][K], stacked (an expert stack [E][rows][K] is n_mats = E):
 *   qs_in       uint8  [n_mats][rows][K/2]   row-major codes: byte i of a row
 *               holds element 2i (low nibble) and 2i+1 (high nibble)
 *   scales_in   uint16 [n_mats][rows][K/32]  row-major fp16 scale bits
 *   qs_out      uint8  [n_mats][rows/16][K/32][16][16]
 *   scales_out  uint16 [n_mats][rows/16][K/32][16]
 * (the layout of moe_q4 above, per matrix).  A pure permutation of whole
 * 16-byte code blocks and of scales; nothing is computed.  All four are
 * DEVICE arrays owned by the caller; the inputs must not overlap the
 * outputs (out-of-place only).  Enqueued on `stream`; no allocation.
 * MOE_EINVAL: a size < 1, a NULL pointer, or overlapping in/out ranges;
 * MOE_EUNSUPPORTED: rows % 16 != 0, K % 32 != 0, or rows or K > 2^24;
 * MOE_EALIGN: qs_in, qs_out or scales_out not 16-byte aligned, or scales_in
 * not 2-byte aligned; MOE_EHIP. */
int moe_q4_pack(int32_t n_mats, int32_t rows, int32_t K, const uint8_t* qs_in, const uint16_t* scales_in,
                uint8_t* qs_out, uint16_t* scales_out, void* stream);

/* ---- fp8-activation variants: W4A8 and W8A8 ----------------------------
 * Page thewafflehaus/FFAI pull request 72 ("Nemotron-Nano-30B GB10 prefill
 * quality + speed wins") adds W4A8 (fp8 activations x fp4 weights) and
 * W8A8 (fp8 activations x fp8 weights) grouped MoE paths beside the Q4
 * W4A16 one; the fp4 weights are the Q4 weights requantised once to a
 * block-scaled fp4 grid, the fp8 activations carry a per-token scale
 * applied to the product.  Here the weight grids are the block formats the
 * gfx950 block-scaled MFMA multiplies as they are, in the Q4 blocks of 32,
 * each block with a power-of-two scale 2^E stored as the byte E + 127:
 *   MXFP4  e2m1 elements (0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives),
 *          E = floor(log2 max|w|) - 2
 *   MXFP8  e4m3 elements (largest 448), E = floor(log2 max|w|) - 8
 * (E = -127 for an all-zero block; elements round to nearest, ties to the
 * even mantissa, saturating at the largest value).  fp8 activations are
 * e4m3.  Per layer call, for every token t:
 *   routing  as for moe_q4_forward (the same topk_w and routing build);
 *   x8_t     = e4m3(x_t / sx_t),   sx_t = amax(x_t) / 448   (1 if x_t = 0)
 *   h        = fp16(silu(sx_t * (W_g x8_t)) * (sx_t * (W_u x8_t)))
 *   h8       = e4m3(h / sh),       sh = amax(h) / 448 per h row
 *   y_e      = sh * (W_d h8)       (W the requantised matrices, exact
 *                                   products, fp32 accumulation)
 * then the combine of moe_q4_forward.  Both divisions are correctly rounded
 * fp32. */
typedef struct moe_mx {
  const uint8_t* codes;  /* [rows/16][K/32][16][B] element codes, 16-byte
                            aligned: the Q4 code layout with B bytes per
                            block, B = 16 for MXFP4 (element 2i in the low
                            nibble of byte i) and 32 for MXFP8 (element i
                            at byte i)                                    */
  const uint8_t* exps;   /* [rows/16][K/32][16] biased block exponents, the
                            Q4 scale layout with one byte per block      */
} moe_mx;

typedef struct moe_mx_weights {
  moe_mx w13;  /* [E][2I][d]       */
  moe_mx w2;   /* [E][d][I]        */
  moe_mx s13;  /* [2*I_shared][d]  */
  moe_mx s2;   /* [d][I_shared]    */
} moe_mx_weights;

/* Requantise Q4 blocks to MXFP4 (moe_q4_to_mxfp4) or MXFP8 (moe_q4_to_mxfp8)
 * on the device (the one-time load step).  Block b of (qs, scales) becomes
 * block b of (codes_out, exps_out), so it works on the packed 16-row groups
 * (giving the moe_mx layout) and on row-major arrays alike; n_mats * rows *
 * K / 32 blocks in total.  DEVICE arrays owned by the caller: qs and
 * codes_out 16-byte aligned ([blocks][16] in, [blocks][16] or [blocks][32]
 * out), scales uint16 [blocks] (2-byte aligned), exps_out uint8 [blocks];
 * outputs must not overlap inputs.
 * MOE_EINVAL: a size < 1, a NULL pointer, overlapping ranges;
 * MOE_EUNSUPPORTED: rows % 16 != 0, K % 32 != 0, or rows or K > 2^24;
 * MOE_EALIGN; MOE_EHIP. */
int moe_q4_to_mxfp4(int32_t n_mats, int32_t rows, int32_t K, const uint8_t* qs, const uint16_t* scales,
                    uint8_t* codes_out, uint8_t* exps_out, void* stream);
int moe_q4_to_mxfp8(int32_t n_mats, int32_t rows, int32_t K, const uint8_t* qs, const uint16_t* scales,
                    uint8_t* codes_out, uint8_t* exps_out, void* stream);

/* The activation step of the fp8 variants on its own: `rows` rows of K
 * values (bf16 bits, or fp16 bits when in_is_fp16 != 0) -> e4m3 codes
 * (uint8 [rows][K]) and fp32 row scales s = amax / 448 (1 for an all-zero
 * row), code = e4m3(x / s) as above.  DEVICE arrays owned by the caller,
 * 16-byte aligned (scales 4-byte).  MOE_EINVAL: rows or K < 1, a NULL
 * pointer; MOE_EUNSUPPORTED: K % 4 != 0 or rows * K >= 2^31; MOE_EALIGN;
 * MOE_EHIP. */
int moe_rows_to_fp8(int32_t rows, int32_t K, const uint16_t* in, int in_is_fp16, uint8_t* codes_out,
                    float* scales_out, void* stream);

/* Bytes of scratch moe_w4a8_forward / moe_w8a8_forward need (the same for
 * both), 0 if the shape or flags are unsupported (see there). */
size_t moe_w4a8_scratch_bytes(const moe_dims* dims, uint32_t flags);
size_t moe_w8a8_scratch_bytes(const moe_dims* dims, uint32_t flags);

/* The W4A8 (MXFP4 weights from moe_q4_to_mxfp4) and W8A8 (MXFP8 weights
 * from moe_q4_to_mxfp8) expert layers (formula above) on the grouped path.
 * Arguments as for moe_q4_forward; the routing workspace must hold
 * moe_build_descriptors' output for the same topk ids and flags.  topk_ids
 * is checked but not read (the routing build holds it).  MOE_EUNSUPPORTED
 * also when flags select the small-T path (pass MOE_FLAG_FORCE_GROUPED for
 * T <= MOE_GEMV_MAX_T), when d, I or I_shared is not a multiple of 128, and
 * for W8A8 when 2 * max(I, I_shared) * d >= 2^31 (32-bit offsets into one
 * expert's fp8 codes); MOE_EINVAL, MOE_EALIGN (exps need no alignment),
 * MOE_ENOSPACE (scratch below the _scratch_bytes query), MOE_EHIP. */
int moe_w4a8_forward(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids, const float* topk_w,
                     const void* routing, size_t routing_bytes, const moe_mx_weights* w, float* y,
                     void* scratch, size_t scratch_bytes, uint32_t flags, void* stream);
int moe_w8a8_forward(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids, const float* topk_w,
                     const void* routing, size_t routing_bytes, const moe_mx_weights* w, float* y,
                     void* scratch, size_t scratch_bytes, uint32_t flags, void* stream);

/* Static string for a return code; never NULL. */
const char* moe_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* MOE_Q4_H */
