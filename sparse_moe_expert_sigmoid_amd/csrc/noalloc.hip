// moe_layer_forward without caller-provided workspaces, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The routing workspace and the scratch the layer's kernels use live in one file-scope device array of
// kNoAllocBytes per GPU, held for the life of the process.  Host code never passes the array's name to
// a kernel: at the first call on a device (with that device current) its device address is looked up
// once with hipGetSymbolAddress and kept per device, and only that address is handed to the kernels,
// exactly as the caller's buffers are by moe_layer_forward.  Calls on one GPU share the array: calls
// that overlap in time on one GPU race.  Nothing in it has to start at zero: every region the kernels
// read is written earlier in the same call (the small-T path's arrival counters start at zero when the
// program is loaded and every call leaves them at zero).
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_q4.h"

namespace moe_abi {
int layer_sizes(const moe_dims* dims, uint32_t flags, size_t* routing_bytes, size_t* scratch_bytes);
int layer_forward(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router, const float* bias,
                  const moe_q4_weights* w, const float* residual, float* y, int32_t* topk_ids, float* topk_w,
                  void* routing, size_t routing_bytes, void* scratch, size_t scratch_bytes, uint32_t flags,
                  void* stream);
int check_layer_args(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router, const float* bias,
                     const moe_q4_weights* w, const float* residual, const float* y, const int32_t* topk_ids,
                     const float* topk_w, uint32_t flags);
}  // namespace moe_abi

namespace {

constexpr size_t kNoAllocBytes = (size_t)MOE_NOALLOC_MAX_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each device, looked up once

// The array's device address on the current device (nullptr on failure).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

int moe_layer_forward_noalloc(const moe_dims* dims, const uint16_t* x_bf16, const float* w_router,
                              const float* bias, const moe_q4_weights* weights, const float* residual, float* y,
                              int32_t* topk_ids, float* topk_w, uint32_t flags, void* stream) {
  int rc = moe_abi::check_layer_args(dims, x_bf16, w_router, bias, weights, residual, y, topk_ids, topk_w, flags);
  if (rc != MOE_OK) return rc;
  size_t rb = 0, sb = 0;
  rc = moe_abi::layer_sizes(dims, flags, &rb, &sb);
  if (rc != MOE_OK) return rc;
  if (rb + sb > kNoAllocBytes) return MOE_ENOSPACE;  // beyond the library's fixed workspace
  char* base = static_cast<char*>(scratch_ptr());
  if (!base) return MOE_EHIP;
  return moe_abi::layer_forward(dims, x_bf16, w_router, bias, weights, residual, y, topk_ids, topk_w, base, rb,
                                base + rb, sb, flags, stream);
}

}  // extern "C"
