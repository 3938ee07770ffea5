// h3attn_forward_noalloc: h3attn_forward with its workspace in a static
// device array instead of a caller buffer, for callers that cannot allocate
// (declared in include/h3attn.h). The kernels are the forward's own; they
// receive the array's device address as their workspace pointer.
#include <mutex>

#include "h3attn.h"
#include "h3attn_internal.h"

#define H3_API extern "C" __attribute__((visibility("default")))

namespace {

// The workspace, one copy per GPU that loads the library (each at its own
// device address, held until the process ends). Host code never uses the
// name `scratch` as an address: on the host it is only a stand-in symbol.
// Every use goes through the device address that hipGetSymbolAddress
// returns for the current device (scratch_address below).
static __device__ __align__(256) uint8_t scratch[H3ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, set on first use

// The current device's address of `scratch`, looked up once per device
// with that device current.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return H3ATTN_ERR_UNSUPPORTED_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return H3ATTN_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return H3ATTN_OK;
}

}  // namespace

H3_API int h3attn_forward_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, int32_t B,
                                  int32_t Sq, int32_t Sk, int32_t H, int32_t head_dim, const float* q_norm_w,
                                  const float* k_norm_w, float eps, const float* rope_cos, const float* rope_sin,
                                  int32_t rope_rows, int32_t q_valid, int32_t kv_valid, float softmax_scale,
                                  void* stream) {
  size_t need = 0;
  if (int st = h3::check_dense_args(q, k, v, o, B, Sq, Sk, H, head_dim, q_norm_w, k_norm_w, eps, rope_cos, rope_sin,
                                    rope_rows, q_valid, kv_valid, softmax_scale, &need))
    return st;
  if (need > H3ATTN_NOALLOC_SCRATCH_BYTES) return H3ATTN_ERR_WORKSPACE;
  if (int st = h3::check_gfx950()) return st;
  void* ws = nullptr;
  if (int st = scratch_address(&ws)) return st;
  return h3::forward_dense(q, k, v, o, B, Sq, Sk, H, head_dim, q_norm_w, k_norm_w, eps, rope_cos, rope_sin, rope_rows,
                           q_valid, kv_valid, softmax_scale, ws, H3ATTN_NOALLOC_SCRATCH_BYTES,
                           H3ATTN_STAGE_PREPARE | H3ATTN_STAGE_ATTEND, stream);
}
