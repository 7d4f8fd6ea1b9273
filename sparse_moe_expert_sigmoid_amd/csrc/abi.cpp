// C ABI of the Q4 MoE expert layer: host-side validation, workspace layouts,
// path selection and kernel dispatch.  Declarations and the contract of every
// entry point are in include/moe_q4.h.
//
// Everything here runs on the host.  Arguments are validated before the
// first HIP call, so a rejected call enqueues nothing; accepted calls only
// enqueue kernels on the caller's stream (no allocation, synchronisation or
// device-to-host copy), which keeps them capturable into a HIP graph.
#include <hip/hip_runtime.h>

#include <dlfcn.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "moe_q4.h"
#include "moe_kernels.hpp"

namespace {

// roctx ranges around the entry points that enqueue work, for rocprofv3 --marker-trace.  Off unless the
// environment sets MOE_ROCTX=1 when the library first needs them; the roctx library is then looked up
// at run time, so nothing links against it and a missing one leaves the ranges off.
struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
  Roctx() {
    const char* on = getenv("MOE_ROCTX");
    if (!on || strcmp(on, "1") != 0) return;
    void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (!h) h = dlopen("libroctx64.so.4", RTLD_NOW | RTLD_LOCAL);
    if (!h) return;
    push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
    pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
    if (!push || !pop) push = nullptr, pop = nullptr;
  }
};
const Roctx& roctx() {
  static const Roctx r;
  return r;
}
struct Range {
  const bool on;
  explicit Range(const char* name) : on(roctx().push != nullptr) {
    if (on) roctx().push(name);
  }
  ~Range() {
    if (on) roctx().pop();
  }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kBuildChunk = 256;
constexpr long long kMaxPairs = 1LL << 26;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// 0 = small-T GEMV path, 1 = grouped path.
int choose_path(const moe_dims* d, uint32_t flags) {
  if (flags & MOE_FLAG_FORCE_GROUPED) return 1;
  if (flags & MOE_FLAG_FORCE_GEMV) return 0;
  return d->T <= MOE_GEMV_MAX_T ? 0 : 1;
}

int check_dims(const moe_dims* d, uint32_t flags) {
  if (!d) return MOE_EINVAL;
  if (d->T < 1 || d->d < 1 || d->E < 1 || d->k < 1 || d->I < 1 || d->I_shared < 1) return MOE_EINVAL;
  if (d->k > d->E) return MOE_EINVAL;
  if ((flags & MOE_FLAG_FORCE_GROUPED) && (flags & MOE_FLAG_FORCE_GEMV)) return MOE_EINVAL;
  if ((flags & MOE_FLAG_NO_BANDING) && (flags & MOE_FLAG_BAND_MAJOR)) return MOE_EINVAL;
  if (flags & ~(uint32_t)(MOE_FLAG_FORCE_GROUPED | MOE_FLAG_FORCE_GEMV | MOE_FLAG_ID_ORDER | MOE_FLAG_NO_BANDING |
                          MOE_FLAG_BAND_MAJOR))
    return MOE_EINVAL;
  if (d->d % 32 || d->I % 32 || d->I_shared % 32) return MOE_EUNSUPPORTED;
  if (d->E > kMaxExperts || d->k > kMaxTopK) return MOE_EUNSUPPORTED;
  const long long P = (long long)d->T * d->k;
  if (P > kMaxPairs || d->d > (1 << 20) || d->I > (1 << 20) || d->I_shared > (1 << 20)) return MOE_EUNSUPPORTED;
  const long long wide = d->d > d->I ? d->d : d->I;
  if ((P + d->T) * wide >= (1LL << 31)) return MOE_EUNSUPPORTED;  // 32-bit row indices in the kernels
  if (choose_path(d, flags) == 0) {
    if (d->d > 8192 || d->I > 2048 || d->I_shared > 2048) return MOE_EUNSUPPORTED;
    if (d->T > MOE_GEMV_FORCE_MAX_T) return MOE_EUNSUPPORTED;
  } else {
    // The grouped GEMMs address one expert's weights through 32-bit buffer offsets: a gate+up stack of
    // 2*I rows by d/2 code bytes (I*d bytes) or a down matrix (d*I/2 bytes) must stay below 2^31.
    const long long Imax = d->I > d->I_shared ? d->I : d->I_shared;
    if (Imax * d->d >= (1LL << 31)) return MOE_EUNSUPPORTED;
  }
  return MOE_OK;
}

struct Layout {
  size_t logits, counts, offsets, sorted_pair, pair_pos, row_expert, group_order, mt_prefix, chunk_counts, total;
};

Layout routing_layout(const moe_dims* d) {
  const size_t T = d->T, E = d->E, P = (size_t)d->T * d->k;
  const size_t nchunks = (T + kBuildChunk - 1) / kBuildChunk;
  Layout L{};
  size_t off = 0;
  L.logits = off;       off += align256((size_t)moe::kRouterParts * T * E * 4);
  L.counts = off;       off += align256((E + 1) * 4);
  L.offsets = off;      off += align256((E + 1) * 4);
  L.sorted_pair = off;  off += align256(P * 4);
  L.pair_pos = off;     off += align256(P * 4);
  L.row_expert = off;   off += align256(P * 4);
  L.group_order = off;  off += align256((E + 1) * 4);
  L.mt_prefix = off;    off += align256((E + 2) * 4);
  L.chunk_counts = off; off += align256(nchunks * E * 4);
  L.total = off;
  return L;
}

struct ScratchLayout {
  size_t x16, h_r, h_s, y_pair, y_s, total;
};

ScratchLayout scratch_layout(const moe_dims* d, int path) {
  const size_t T = d->T, P = (size_t)d->T * d->k;
  ScratchLayout S{};
  size_t off = 0;
  if (path == 0) {
    S.h_r = off; off += align256(P * d->I * 2);
    S.h_s = off; off += align256(T * d->I_shared * 2);
  } else {
    S.x16 = off;    off += align256(T * d->d * 2);
    S.h_r = off;    off += align256(P * d->I * 2);
    S.h_s = off;    off += align256(T * d->I_shared * 2);
    S.y_pair = off; off += align256(P * d->d * 2);
    S.y_s = off;    off += align256(T * d->d * 2);
  }
  S.total = off;
  return S;
}

moe::Routing routing_ptrs(void* base, const Layout& L) {
  char* b = static_cast<char*>(base);
  moe::Routing r;
  r.logits = reinterpret_cast<float*>(b + L.logits);
  r.counts = reinterpret_cast<int*>(b + L.counts);
  r.offsets = reinterpret_cast<int*>(b + L.offsets);
  r.sorted_pair = reinterpret_cast<int*>(b + L.sorted_pair);
  r.pair_pos = reinterpret_cast<int*>(b + L.pair_pos);
  r.row_expert = reinterpret_cast<int*>(b + L.row_expert);
  r.group_order = reinterpret_cast<int*>(b + L.group_order);
  r.mt_prefix = reinterpret_cast<int*>(b + L.mt_prefix);
  r.chunk_counts = reinterpret_cast<int*>(b + L.chunk_counts);
  return r;
}

moe::Shape shape_of(const moe_dims* d) { return moe::Shape{d->T, d->d, d->E, d->k, d->I, d->I_shared}; }

bool q4_ok(const moe_q4& q) { return q.qs && q.scales; }
bool q4_aligned(const moe_q4& q) { return aligned(q.qs, 16) && aligned(q.scales, 16); }

int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// fp8-activation variants: grouped path only, every K a whole number of 128-value MFMA steps; MXFP8
// codes take twice the bytes of Q4 codes, so one expert's gate+up stack (2 I d bytes) must leave 31 bits.
int check_fp8act(const moe_dims* d, uint32_t flags, bool fp8) {
  const int rc = check_dims(d, flags);
  if (rc) return rc;
  if (choose_path(d, flags) != 1) return MOE_EUNSUPPORTED;
  if (d->d % 128 || d->I % 128 || d->I_shared % 128) return MOE_EUNSUPPORTED;
  const long long Imax = d->I > d->I_shared ? d->I : d->I_shared;
  if (fp8 && 2 * Imax * d->d >= (1LL << 31)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

struct W4A8Layout {
  size_t x8, xs, h_r, h_s, h8_r, hs_r, h8_s, hs_s, y_pair, y_s, total;
};

W4A8Layout w4a8_layout(const moe_dims* d) {
  const size_t T = d->T, P = (size_t)d->T * d->k;
  W4A8Layout S{};
  size_t off = 0;
  S.x8 = off;     off += align256(T * d->d);
  S.xs = off;     off += align256(T * 4);
  S.h_r = off;    off += align256(P * d->I * 2);
  S.h_s = off;    off += align256(T * d->I_shared * 2);
  S.h8_r = off;   off += align256(P * d->I);
  S.hs_r = off;   off += align256(P * 4);
  S.h8_s = off;   off += align256(T * d->I_shared);
  S.hs_s = off;   off += align256(T * 4);
  S.y_pair = off; off += align256(P * d->d * 2);
  S.y_s = off;    off += align256(T * d->d * 2);
  S.total = off;
  return S;
}

}  // namespace

extern "C" {

int moe_supports(const moe_dims* dims, uint32_t flags) { return check_dims(dims, flags); }

int moe_path(const moe_dims* dims, uint32_t flags) {
  const int rc = check_dims(dims, flags);
  return rc ? rc : choose_path(dims, flags);
}

size_t moe_routing_bytes(const moe_dims* dims, uint32_t flags) {
  if (check_dims(dims, flags)) return 0;
  return routing_layout(dims).total;
}

int moe_routing_layout_of(const moe_dims* dims, uint32_t flags, moe_routing_layout* out) {
  const int rc = check_dims(dims, flags);
  if (rc) return rc;
  if (!out) return MOE_EINVAL;
  const Layout L = routing_layout(dims);
  out->logits = L.logits;
  out->counts = L.counts;
  out->offsets = L.offsets;
  out->sorted_pair = L.sorted_pair;
  out->pair_pos = L.pair_pos;
  out->row_expert = L.row_expert;
  out->group_order = L.group_order;
  out->mt_prefix = L.mt_prefix;
  out->chunk_counts = L.chunk_counts;
  out->total = L.total;
  return MOE_OK;
}

size_t moe_scratch_bytes(const moe_dims* dims, uint32_t flags) {
  if (check_dims(dims, flags)) return 0;
  return scratch_layout(dims, choose_path(dims, flags)).total;
}

namespace {
// x16 (internal, may be nullptr): on the grouped path the router also writes the fp16 copy of x that the
// gate+up reads (the whole-layer call passes its scratch slot and skips that copy's own pass).  Every
// launch here stays idempotent: replaying any one of them alone rewrites the same values.
int route_impl(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router, const float* bias,
               int32_t* topk_ids, float* topk_w, void* routing, size_t routing_bytes, uint32_t flags, void* stream,
               _Float16* x16) {
  int rc = check_dims(dims, flags);
  if (rc) return rc;
  if (!x_bf16 || !w_router || !bias || !topk_ids || !topk_w || !routing) return MOE_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(w_router, 16) || !aligned(routing, 16) || !aligned(bias, 4) ||
      !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return MOE_EALIGN;
  const Layout L = routing_layout(dims);
  if (routing_bytes < L.total) return MOE_ENOSPACE;
  const moe::Shape s = shape_of(dims);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const moe::Routing r = routing_ptrs(routing, L);
  (void)hipGetLastError();
  const bool gemv = choose_path(dims, flags) == 0;
  hipError_t e = gemv ? moe::launch_router_gemv(s, x_bf16, w_router, r.logits, st)
                      : moe::launch_router_mfma(s, x_bf16, w_router, r.logits, st, x16);
  if (e != hipSuccess) return MOE_EHIP;
  const int nparts = gemv ? 1 : moe::kRouterParts;
  return hip_rc(moe::launch_topk(s, r.logits, nparts, bias, topk_ids, topk_w, st));
}
}  // namespace

int moe_route(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router, const float* bias,
              int32_t* topk_ids, float* topk_w, void* routing, size_t routing_bytes, uint32_t flags, void* stream) {
  const Range range("moe_route");
  return route_impl(dims, x_bf16, w_router, bias, topk_ids, topk_w, routing, routing_bytes, flags, stream, nullptr);
}

int moe_build_descriptors(const moe_dims* dims, const int32_t* topk_ids, void* routing, size_t routing_bytes,
                          uint32_t flags, void* stream) {
  const Range range("moe_build_descriptors");
  int rc = check_dims(dims, flags);
  if (rc) return rc;
  if (!topk_ids || !routing) return MOE_EINVAL;
  if (!aligned(topk_ids, 4) || !aligned(routing, 16)) return MOE_EALIGN;
  const Layout L = routing_layout(dims);
  if (routing_bytes < L.total) return MOE_ENOSPACE;
  if (choose_path(dims, flags) == 0) return MOE_OK;  // the GEMV path reads topk_ids directly
  (void)hipGetLastError();
  return hip_rc(moe::launch_build(shape_of(dims), topk_ids, routing_ptrs(routing, L), flags,
                                  static_cast<hipStream_t>(stream)));
}

namespace {
// y_bf16 (internal, may be nullptr): also write y rounded to bf16, in the pass that writes y.
// x16_ready (internal): the scratch's fp16 copy of x was written by the router of the same layer call.
int forward_impl(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids, const float* topk_w,
                 const void* routing, size_t routing_bytes, const moe_q4_weights* w, const float* residual,
                 float* y, void* scratch, size_t scratch_bytes, uint32_t flags, void* stream,
                 uint16_t* y_bf16 = nullptr, bool x16_ready = false) {
  int rc = check_dims(dims, flags);
  if (rc) return rc;
  const int path = choose_path(dims, flags);
  if (!x_bf16 || !topk_ids || !topk_w || !w || !y || !scratch) return MOE_EINVAL;
  if (!q4_ok(w->w13) || !q4_ok(w->w2) || !q4_ok(w->s13) || !q4_ok(w->s2)) return MOE_EINVAL;
  if (path == 1 && !routing) return MOE_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(y, 16) || !aligned(scratch, 16) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4))
    return MOE_EALIGN;
  if (!q4_aligned(w->w13) || !q4_aligned(w->w2) || !q4_aligned(w->s13) || !q4_aligned(w->s2)) return MOE_EALIGN;
  if (path == 1 && !aligned(routing, 16)) return MOE_EALIGN;
  const Layout L = routing_layout(dims);
  if (path == 1 && routing_bytes < L.total) return MOE_ENOSPACE;
  const ScratchLayout S = scratch_layout(dims, path);
  if (scratch_bytes < S.total) return MOE_ENOSPACE;

  const moe::Shape s = shape_of(dims);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* sb = static_cast<char*>(scratch);
  const moe::Q4 w13{w->w13.qs, w->w13.scales}, w2{w->w2.qs, w->w2.scales};
  const moe::Q4 s13{w->s13.qs, w->s13.scales}, s2{w->s2.qs, w->s2.scales};
  (void)hipGetLastError();
  if (path == 0) {
    _Float16* h_r = reinterpret_cast<_Float16*>(sb + S.h_r);
    _Float16* h_s = reinterpret_cast<_Float16*>(sb + S.h_s);
    if (moe::launch_gemv_gateup(s, x_bf16, topk_ids, w13, s13, h_r, h_s, st) != hipSuccess) return MOE_EHIP;
    return hip_rc(moe::launch_gemv_down_combine(s, topk_ids, topk_w, w2, s2, h_r, h_s, residual, y, y_bf16, st));
  }
  const moe::Routing r = routing_ptrs(const_cast<void*>(routing), L);
  moe::GroupedOut o;
  o.x16 = reinterpret_cast<_Float16*>(sb + S.x16);
  o.h_r = reinterpret_cast<_Float16*>(sb + S.h_r);
  o.h_s = reinterpret_cast<_Float16*>(sb + S.h_s);
  o.y_pair = reinterpret_cast<_Float16*>(sb + S.y_pair);
  o.y_s = reinterpret_cast<_Float16*>(sb + S.y_s);
  if (moe::launch_grouped_gateup(s, x_bf16, r, w13, s13, o, flags, st, x16_ready) != hipSuccess) return MOE_EHIP;
  if (moe::launch_grouped_down(s, r, w2, s2, o, flags, st) != hipSuccess) return MOE_EHIP;
  return hip_rc(moe::launch_combine(s, topk_w, r, o, residual, y, y_bf16, st));
}
}  // namespace

int moe_q4_forward(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids, const float* topk_w,
                   const void* routing, size_t routing_bytes, const moe_q4_weights* w, float* y, void* scratch,
                   size_t scratch_bytes, uint32_t flags, void* stream) {
  const Range range("moe_q4_forward");
  return forward_impl(dims, x_bf16, topk_ids, topk_w, routing, routing_bytes, w, nullptr, y, scratch, scratch_bytes,
                      flags, stream);
}

int moe_q4_forward_residual(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids,
                            const float* topk_w, const void* routing, size_t routing_bytes,
                            const moe_q4_weights* w, const float* residual, float* y, void* scratch,
                            size_t scratch_bytes, uint32_t flags, void* stream) {
  const Range range("moe_q4_forward_residual");
  const int rc = check_dims(dims, flags);
  if (rc) return rc;
  if (!residual) return MOE_EINVAL;
  if (!aligned(residual, 16)) return MOE_EALIGN;
  return forward_impl(dims, x_bf16, topk_ids, topk_w, routing, routing_bytes, w, residual, y, scratch,
                      scratch_bytes, flags, stream);
}

}  // extern "C"

namespace {
// The whole layer in one call.  Every argument is checked before the first launch; on the small-T
// path the router GEMV is followed by the gate+up GEMV that selects its own experts (no top-k
// launch), then the down + combine pass.  y_bf16 as for forward_impl.
int layer_impl(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router, const float* bias,
               const moe_q4_weights* w, const float* residual, float* y, int32_t* topk_ids, float* topk_w,
               void* routing, size_t routing_bytes, void* scratch, size_t scratch_bytes, uint32_t flags,
               void* stream, uint16_t* y_bf16 = nullptr) {
  int rc = check_dims(dims, flags);
  if (rc) return rc;
  if (!x_bf16 || !w_router || !bias || !w || !y || !topk_ids || !topk_w || !routing || !scratch) return MOE_EINVAL;
  if (!q4_ok(w->w13) || !q4_ok(w->w2) || !q4_ok(w->s13) || !q4_ok(w->s2)) return MOE_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(w_router, 16) || !aligned(bias, 4) || !aligned(y, 16) ||
      !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(routing, 16) || !aligned(scratch, 16) ||
      (residual && !aligned(residual, 16)))
    return MOE_EALIGN;
  if (!q4_aligned(w->w13) || !q4_aligned(w->w2) || !q4_aligned(w->s13) || !q4_aligned(w->s2)) return MOE_EALIGN;
  const int path = choose_path(dims, flags);
  const Layout L = routing_layout(dims);
  if (routing_bytes < L.total) return MOE_ENOSPACE;
  const ScratchLayout S = scratch_layout(dims, path);
  if (scratch_bytes < S.total) return MOE_ENOSPACE;
  if (path == 1) {
    _Float16* x16 = reinterpret_cast<_Float16*>(static_cast<char*>(scratch) + S.x16);
    rc = route_impl(dims, x_bf16, w_router, bias, topk_ids, topk_w, routing, routing_bytes, flags, stream, x16);
    if (rc == MOE_OK) rc = moe_build_descriptors(dims, topk_ids, routing, routing_bytes, flags, stream);
    if (rc == MOE_OK)
      rc = forward_impl(dims, x_bf16, topk_ids, topk_w, routing, routing_bytes, w, residual, y, scratch,
                        scratch_bytes, flags, stream, y_bf16, true);
    return rc;
  }
  const moe::Shape s = shape_of(dims);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const moe::Routing r = routing_ptrs(routing, L);
  char* sb = static_cast<char*>(scratch);
  _Float16* h_r = reinterpret_cast<_Float16*>(sb + S.h_r);
  _Float16* h_s = reinterpret_cast<_Float16*>(sb + S.h_s);
  const moe::Q4 w13{w->w13.qs, w->w13.scales}, w2{w->w2.qs, w->w2.scales};
  const moe::Q4 s13{w->s13.qs, w->s13.scales}, s2{w->s2.qs, w->s2.scales};
  (void)hipGetLastError();
  if (moe::launch_router_gemv(s, x_bf16, w_router, r.logits, st) != hipSuccess) return MOE_EHIP;
  if (moe::launch_gemv_gateup_select(s, x_bf16, r.logits, bias, topk_ids, topk_w, w13, s13, h_r, h_s, st) !=
      hipSuccess)
    return MOE_EHIP;
  return hip_rc(moe::launch_gemv_down_combine(s, topk_ids, topk_w, w2, s2, h_r, h_s, residual, y, y_bf16, st));
}
}  // namespace

// Sizes and the entry for the variant that keeps its routing workspace and scratch in device memory of
// the library's own (noalloc.hip).
namespace moe_abi {
int layer_sizes(const moe_dims* dims, uint32_t flags, size_t* routing_bytes, size_t* scratch_bytes) {
  const int rc = check_dims(dims, flags);
  if (rc) return rc;
  *routing_bytes = align256(routing_layout(dims).total);
  *scratch_bytes = align256(scratch_layout(dims, choose_path(dims, flags)).total);
  return MOE_OK;
}
int layer_forward(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router, const float* bias,
                  const moe_q4_weights* w, const float* residual, float* y, int32_t* topk_ids, float* topk_w,
                  void* routing, size_t routing_bytes, void* scratch, size_t scratch_bytes, uint32_t flags,
                  void* stream) {
  const Range range("moe_layer_forward_noalloc");
  return layer_impl(dims, x_bf16, w_router, bias, w, residual, y, topk_ids, topk_w, routing, routing_bytes, scratch,
                    scratch_bytes, flags, stream);
}
int check_layer_args(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router, const float* bias,
                     const moe_q4_weights* w, const float* residual, const float* y, const int32_t* topk_ids,
                     const float* topk_w, uint32_t flags) {
  const int rc = check_dims(dims, flags);
  if (rc) return rc;
  if (!x_bf16 || !w_router || !bias || !w || !y || !topk_ids || !topk_w) return MOE_EINVAL;
  if (!q4_ok(w->w13) || !q4_ok(w->w2) || !q4_ok(w->s13) || !q4_ok(w->s2)) return MOE_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(w_router, 16) || !aligned(bias, 4) || !aligned(y, 16) ||
      !aligned(topk_ids, 4) || !aligned(topk_w, 4) || (residual && !aligned(residual, 16)))
    return MOE_EALIGN;
  if (!q4_aligned(w->w13) || !q4_aligned(w->w2) || !q4_aligned(w->s13) || !q4_aligned(w->s2)) return MOE_EALIGN;
  return MOE_OK;
}
}  // namespace moe_abi

extern "C" {
int moe_layer_forward(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router, const float* bias,
                      const moe_q4_weights* w, const float* residual, float* y, int32_t* topk_ids, float* topk_w,
                      void* routing, size_t routing_bytes, void* scratch, size_t scratch_bytes, uint32_t flags,
                      void* stream) {
  const Range range("moe_layer_forward");
  return layer_impl(dims, x_bf16, w_router, bias, w, residual, y, topk_ids, topk_w, routing, routing_bytes, scratch,
                    scratch_bytes, flags, stream);
}
}  // extern "C"

struct moe_decode_ctx {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace {

struct CtxLayout {
  size_t x, ids, w, routing, scratch, total;
};

CtxLayout ctx_layout(const moe_dims* d, uint32_t flags) {
  const size_t T = d->T, P = (size_t)d->T * d->k;
  CtxLayout C{};
  size_t off = 0;
  C.x = off;       off += align256(T * d->d * 2);
  C.ids = off;     off += align256(P * 4);
  C.w = off;       off += align256(P * 4);
  C.routing = off; off += align256(routing_layout(d).total);
  C.scratch = off; off += align256(scratch_layout(d, choose_path(d, flags)).total);
  C.total = off;
  return C;
}

bool weights_ok(const moe_q4_weights& w) { return q4_ok(w.w13) && q4_ok(w.w2) && q4_ok(w.s13) && q4_ok(w.s2); }
bool weights_aligned(const moe_q4_weights& w) {
  return q4_aligned(w.w13) && q4_aligned(w.w2) && q4_aligned(w.s13) && q4_aligned(w.s2);
}

// Enqueue the whole stack on `st` (the stream being recorded).
int enqueue_stack(const moe_dims* dims, int n_layers, const moe_layer* layers, float* h, char* ws,
                  const CtxLayout& C, uint32_t flags, hipStream_t st) {
  uint16_t* x = reinterpret_cast<uint16_t*>(ws + C.x);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + C.ids);
  float* tw = reinterpret_cast<float*>(ws + C.w);
  void* routing = ws + C.routing;
  void* scratch = ws + C.scratch;
  const size_t rbytes = C.scratch - C.routing, sbytes = C.total - C.scratch;
  (void)hipGetLastError();
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer& L = layers[l];
    // the layer's input: through the norm, or bf16(h) (written by the previous layer's last pass)
    hipError_t e = hipSuccess;
    if (L.norm_weight)
      e = moe::launch_rmsnorm_bf16(h, L.norm_weight, L.norm_eps, x, dims->T, dims->d, st);
    else if (l == 0)
      e = moe::launch_f32_to_bf16(h, x, (size_t)dims->T * dims->d, st);
    if (e != hipSuccess) return MOE_EHIP;
    // h = layer(x) + h; the last pass also writes the next layer's x = bf16(h) unless that layer's
    // input goes through the norm
    const bool fused_next = l + 1 < n_layers && !layers[l + 1].norm_weight;
    const int rc = layer_impl(dims, x, L.w_router, L.bias, &L.weights, h, h, ids, tw, routing, rbytes, scratch,
                              sbytes, flags, st, fused_next ? x : nullptr);
    if (rc != MOE_OK) return rc;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_rmsnorm_bf16(int T, int d, const float* h, const float* gamma, float eps, uint16_t* x_bf16,
                     void* stream) {
  const Range range("moe_rmsnorm_bf16");
  if (T < 1 || d < 1 || !h || !gamma || !x_bf16 || !(isfinite(eps) && eps >= 0.f)) return MOE_EINVAL;
  if (d % 8 || d > (1 << 20)) return MOE_EUNSUPPORTED;
  if (!aligned(h, 16) || !aligned(gamma, 16) || !aligned(x_bf16, 16)) return MOE_EALIGN;
  (void)hipGetLastError();
  return hip_rc(moe::launch_rmsnorm_bf16(h, gamma, eps, x_bf16, T, d, static_cast<hipStream_t>(stream)));
}

size_t moe_decode_ctx_workspace_bytes(const moe_dims* dims, uint32_t flags) {
  if (check_dims(dims, flags)) return 0;
  return ctx_layout(dims, flags).total;
}

int moe_decode_ctx_create(const moe_dims* dims, int n_layers, const moe_layer* layers, float* h, void* workspace,
                          size_t workspace_bytes, uint32_t flags, moe_decode_ctx** out) {
  const Range range("moe_decode_ctx_create");
  const int rc0 = check_dims(dims, flags);
  if (rc0) return rc0;
  if (!layers || !h || !workspace || !out || n_layers < 1 || n_layers > 4096) return MOE_EINVAL;
  for (int l = 0; l < n_layers; ++l) {
    if (!layers[l].w_router || !layers[l].bias || !weights_ok(layers[l].weights)) return MOE_EINVAL;
    if (layers[l].norm_weight && !(isfinite(layers[l].norm_eps) && layers[l].norm_eps >= 0.f)) return MOE_EINVAL;
  }
  if (!aligned(h, 16) || !aligned(workspace, 16)) return MOE_EALIGN;
  for (int l = 0; l < n_layers; ++l)
    if (!aligned(layers[l].w_router, 16) || !aligned(layers[l].bias, 4) || !weights_aligned(layers[l].weights) ||
        !aligned(layers[l].norm_weight, 16))
      return MOE_EALIGN;
  const CtxLayout C = ctx_layout(dims, flags);
  if (workspace_bytes < C.total) return MOE_ENOSPACE;

  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return MOE_EHIP;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int rc = MOE_OK;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    rc = MOE_EHIP;
  } else {
    rc = enqueue_stack(dims, n_layers, layers, h, static_cast<char*>(workspace), C, flags, cs);
    const hipError_t e = hipStreamEndCapture(cs, &graph);  // ends the recording whatever happened
    if (rc == MOE_OK && e != hipSuccess) rc = MOE_EHIP;
    if (rc == MOE_OK && hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) rc = MOE_EHIP;
  }
  (void)hipStreamDestroy(cs);
  if (rc != MOE_OK) {
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
    return rc;
  }
  *out = new moe_decode_ctx{graph, exec};
  return MOE_OK;
}

int moe_decode_ctx_run(moe_decode_ctx* ctx, void* stream) {
  const Range range("moe_decode_ctx_run");
  if (!ctx) return MOE_EINVAL;
  return hip_rc(hipGraphLaunch(ctx->exec, static_cast<hipStream_t>(stream)));
}

int moe_decode_ctx_destroy(moe_decode_ctx* ctx) {
  if (!ctx) return MOE_OK;
  (void)hipGraphExecDestroy(ctx->exec);
  (void)hipGraphDestroy(ctx->graph);
  delete ctx;
  return MOE_OK;
}

int moe_q4_pack(int32_t n_mats, int32_t rows, int32_t K, const uint8_t* qs_in, const uint16_t* scales_in,
                uint8_t* qs_out, uint16_t* scales_out, void* stream) {
  const Range range("moe_q4_pack");
  if (n_mats < 1 || rows < 1 || K < 1 || !qs_in || !scales_in || !qs_out || !scales_out) return MOE_EINVAL;
  if (rows % 16 || K % 32 || rows > (1 << 24) || K > (1 << 24)) return MOE_EUNSUPPORTED;
  if (!aligned(qs_in, 16) || !aligned(qs_out, 16) || !aligned(scales_out, 16) || !aligned(scales_in, 2))
    return MOE_EALIGN;
  const size_t nblocks = (size_t)n_mats * (size_t)rows * (size_t)(K / 32);
  const uintptr_t qi = (uintptr_t)qs_in, qo = (uintptr_t)qs_out, si = (uintptr_t)scales_in,
                  so = (uintptr_t)scales_out;
  const size_t qb = 16 * nblocks, sb = 2 * nblocks;
  auto overlap = [](uintptr_t a, size_t na, uintptr_t b, size_t nb) { return a < b + nb && b < a + na; };
  if (overlap(qo, qb, qi, qb) || overlap(qo, qb, si, sb) || overlap(so, sb, qi, qb) || overlap(so, sb, si, sb) ||
      overlap(qo, qb, so, sb))
    return MOE_EINVAL;
  (void)hipGetLastError();
  return hip_rc(moe::launch_q4_pack((size_t)n_mats, rows, K, qs_in, scales_in, qs_out, scales_out,
                                    static_cast<hipStream_t>(stream)));
}

namespace {
int q4_to_mx(int32_t n_mats, int32_t rows, int32_t K, const uint8_t* qs, const uint16_t* scales, uint8_t* codes_out,
             uint8_t* exps_out, bool fp8, void* stream) {
  if (n_mats < 1 || rows < 1 || K < 1 || !qs || !scales || !codes_out || !exps_out) return MOE_EINVAL;
  if (rows % 16 || K % 32 || rows > (1 << 24) || K > (1 << 24)) return MOE_EUNSUPPORTED;
  if (!aligned(qs, 16) || !aligned(codes_out, 16) || !aligned(scales, 2)) return MOE_EALIGN;
  const size_t nblocks = (size_t)n_mats * (size_t)rows * (size_t)(K / 32);
  const uintptr_t qi = (uintptr_t)qs, si = (uintptr_t)scales, co = (uintptr_t)codes_out, eo = (uintptr_t)exps_out;
  const size_t qb = 16 * nblocks, sb = 2 * nblocks, cb = (fp8 ? 32 : 16) * nblocks, eb = nblocks;
  auto overlap = [](uintptr_t a, size_t na, uintptr_t b, size_t nb) { return a < b + nb && b < a + na; };
  if (overlap(co, cb, qi, qb) || overlap(co, cb, si, sb) || overlap(eo, eb, qi, qb) || overlap(eo, eb, si, sb) ||
      overlap(co, cb, eo, eb))
    return MOE_EINVAL;
  (void)hipGetLastError();
  return hip_rc(moe::launch_q4_to_mx(nblocks, qs, scales, codes_out, exps_out, fp8, static_cast<hipStream_t>(stream)));
}
}  // namespace

int moe_q4_to_mxfp4(int32_t n_mats, int32_t rows, int32_t K, const uint8_t* qs, const uint16_t* scales,
                    uint8_t* codes_out, uint8_t* exps_out, void* stream) {
  const Range range("moe_q4_to_mxfp4");
  return q4_to_mx(n_mats, rows, K, qs, scales, codes_out, exps_out, false, stream);
}

int moe_q4_to_mxfp8(int32_t n_mats, int32_t rows, int32_t K, const uint8_t* qs, const uint16_t* scales,
                    uint8_t* codes_out, uint8_t* exps_out, void* stream) {
  const Range range("moe_q4_to_mxfp8");
  return q4_to_mx(n_mats, rows, K, qs, scales, codes_out, exps_out, true, stream);
}

int moe_rows_to_fp8(int32_t rows, int32_t K, const uint16_t* in, int in_is_fp16, uint8_t* codes_out,
                    float* scales_out, void* stream) {
  const Range range("moe_rows_to_fp8");
  if (rows < 1 || K < 1 || !in || !codes_out || !scales_out) return MOE_EINVAL;
  if (K % 4 || (long long)rows * K >= (1LL << 31)) return MOE_EUNSUPPORTED;
  if (!aligned(in, 16) || !aligned(codes_out, 16) || !aligned(scales_out, 4)) return MOE_EALIGN;
  (void)hipGetLastError();
  return hip_rc(moe::launch_rows_fp8(in, in_is_fp16 != 0, rows, K, codes_out, scales_out,
                                     static_cast<hipStream_t>(stream)));
}

size_t moe_w4a8_scratch_bytes(const moe_dims* dims, uint32_t flags) {
  if (check_fp8act(dims, flags, false)) return 0;
  return w4a8_layout(dims).total;
}

size_t moe_w8a8_scratch_bytes(const moe_dims* dims, uint32_t flags) {
  if (check_fp8act(dims, flags, true)) return 0;
  return w4a8_layout(dims).total;
}

namespace {
int fp8act_forward(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids, const float* topk_w,
                   const void* routing, size_t routing_bytes, const moe_mx_weights* w, float* y, void* scratch,
                   size_t scratch_bytes, uint32_t flags, bool fp8, void* stream) {
  const int rc = check_fp8act(dims, flags, fp8);
  if (rc) return rc;
  if (!x_bf16 || !topk_ids || !topk_w || !routing || !w || !y || !scratch) return MOE_EINVAL;
  const moe_mx* m[4] = {&w->w13, &w->w2, &w->s13, &w->s2};
  for (const moe_mx* p : m)
    if (!p->codes || !p->exps) return MOE_EINVAL;
  if (!aligned(x_bf16, 16) || !aligned(y, 16) || !aligned(scratch, 16) || !aligned(routing, 16) ||
      !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return MOE_EALIGN;
  for (const moe_mx* p : m)
    if (!aligned(p->codes, 16)) return MOE_EALIGN;
  const Layout L = routing_layout(dims);
  if (routing_bytes < L.total) return MOE_ENOSPACE;
  const W4A8Layout S = w4a8_layout(dims);
  if (scratch_bytes < S.total) return MOE_ENOSPACE;
  char* sb = static_cast<char*>(scratch);
  moe::W4A8Scratch o;
  o.x8 = reinterpret_cast<uint8_t*>(sb + S.x8);
  o.xs = reinterpret_cast<float*>(sb + S.xs);
  o.h_r = reinterpret_cast<_Float16*>(sb + S.h_r);
  o.h_s = reinterpret_cast<_Float16*>(sb + S.h_s);
  o.h8_r = reinterpret_cast<uint8_t*>(sb + S.h8_r);
  o.hs_r = reinterpret_cast<float*>(sb + S.hs_r);
  o.h8_s = reinterpret_cast<uint8_t*>(sb + S.h8_s);
  o.hs_s = reinterpret_cast<float*>(sb + S.hs_s);
  o.y_pair = reinterpret_cast<_Float16*>(sb + S.y_pair);
  o.y_s = reinterpret_cast<_Float16*>(sb + S.y_s);
  const moe::MxWeights mw{w->w13.codes, w->w13.exps, w->w2.codes, w->w2.exps,
                          w->s13.codes, w->s13.exps, w->s2.codes, w->s2.exps};
  (void)hipGetLastError();
  return hip_rc(moe::launch_w4a8_forward(shape_of(dims), x_bf16, routing_ptrs(const_cast<void*>(routing), L), mw, o,
                                         topk_w, y, flags, fp8, static_cast<hipStream_t>(stream)));
}
}  // namespace

int moe_w4a8_forward(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids, const float* topk_w,
                     const void* routing, size_t routing_bytes, const moe_mx_weights* w, float* y,
                     void* scratch, size_t scratch_bytes, uint32_t flags, void* stream) {
  const Range range("moe_w4a8_forward");
  return fp8act_forward(dims, x_bf16, topk_ids, topk_w, routing, routing_bytes, w, y, scratch, scratch_bytes, flags,
                        false, stream);
}

int moe_w8a8_forward(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids, const float* topk_w,
                     const void* routing, size_t routing_bytes, const moe_mx_weights* w, float* y,
                     void* scratch, size_t scratch_bytes, uint32_t flags, void* stream) {
  const Range range("moe_w8a8_forward");
  return fp8act_forward(dims, x_bf16, topk_ids, topk_w, routing, routing_bytes, w, y, scratch, scratch_bytes, flags,
                        true, stream);
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer, non-positive size, k > E or conflicting flags)";
    case MOE_EALIGN: return "misaligned array (16-byte alignment required)";
    case MOE_EUNSUPPORTED: return "unsupported shape (d, I, I_shared % 32, E > 1024, k > 32, or beyond the path's range)";
    case MOE_ENOSPACE: return "routing workspace or scratch buffer too small";
    case MOE_EHIP: return "HIP runtime rejected a kernel launch";
    default: return "unknown error code";
  }
}

}  // extern "C"
