// C ABI of the Q4 MoE expert layer: host-side validation, workspace layouts,
// path selection and kernel dispatch.  Declarations and the contract of every
// entry point are in include/moe_q4.h.
//
// Everything here runs on the host.  Arguments are validated before the
// first HIP call, so a rejected call enqueues nothing; accepted calls only
// enqueue kernels on the caller's stream (no allocation, synchronisation or
// device-to-host copy), which keeps them capturable into a HIP graph.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "moe_q4.h"
#include "moe_kernels.hpp"

namespace {

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

int moe_route(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router, const float* bias,
              int32_t* topk_ids, float* topk_w, void* routing, size_t routing_bytes, uint32_t flags, void* stream) {
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
                      : moe::launch_router_mfma(s, x_bf16, w_router, r.logits, st);
  if (e != hipSuccess) return MOE_EHIP;
  const int nparts = gemv ? 1 : moe::kRouterParts;
  return hip_rc(moe::launch_topk(s, r.logits, nparts, bias, topk_ids, topk_w, st));
}

int moe_build_descriptors(const moe_dims* dims, const int32_t* topk_ids, void* routing, size_t routing_bytes,
                          uint32_t flags, void* stream) {
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
int forward_impl(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids, const float* topk_w,
                 const void* routing, size_t routing_bytes, const moe_q4_weights* w, const float* residual,
                 float* y, void* scratch, size_t scratch_bytes, uint32_t flags, void* stream) {
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
    return hip_rc(moe::launch_gemv_down_combine(s, topk_ids, topk_w, w2, s2, h_r, h_s, residual, y, st));
  }
  const moe::Routing r = routing_ptrs(const_cast<void*>(routing), L);
  moe::GroupedOut o;
  o.x16 = reinterpret_cast<_Float16*>(sb + S.x16);
  o.h_r = reinterpret_cast<_Float16*>(sb + S.h_r);
  o.h_s = reinterpret_cast<_Float16*>(sb + S.h_s);
  o.y_pair = reinterpret_cast<_Float16*>(sb + S.y_pair);
  o.y_s = reinterpret_cast<_Float16*>(sb + S.y_s);
  if (moe::launch_grouped_gateup(s, x_bf16, r, w13, s13, o, flags, st) != hipSuccess) return MOE_EHIP;
  if (moe::launch_grouped_down(s, r, w2, s2, o, flags, st) != hipSuccess) return MOE_EHIP;
  return hip_rc(moe::launch_combine(s, topk_w, r, o, residual, y, st));
}
}  // namespace

int moe_q4_forward(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids, const float* topk_w,
                   const void* routing, size_t routing_bytes, const moe_q4_weights* w, float* y, void* scratch,
                   size_t scratch_bytes, uint32_t flags, void* stream) {
  return forward_impl(dims, x_bf16, topk_ids, topk_w, routing, routing_bytes, w, nullptr, y, scratch, scratch_bytes,
                      flags, stream);
}

int moe_q4_forward_residual(const moe_dims* dims, const uint16_t* x_bf16, const int32_t* topk_ids,
                            const float* topk_w, const void* routing, size_t routing_bytes,
                            const moe_q4_weights* w, const float* residual, float* y, void* scratch,
                            size_t scratch_bytes, uint32_t flags, void* stream) {
  const int rc = check_dims(dims, flags);
  if (rc) return rc;
  if (!residual) return MOE_EINVAL;
  if (!aligned(residual, 16)) return MOE_EALIGN;
  return forward_impl(dims, x_bf16, topk_ids, topk_w, routing, routing_bytes, w, residual, y, scratch,
                      scratch_bytes, flags, stream);
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
