// Microbenchmarks for the achievable roofline denominators on gfx950: the
// sustained bf16 matrix-core rate (with the shader clock under that load),
// the v_exp_f32 rate and a streaming device copy. Entry points and the work
// each launch does are declared in include/h3attn_micro.h.
#include "h3attn_micro.h"

#include "h3attn.h"
#include "h3attn_internal.h"

#define H3_API extern "C" __attribute__((visibility("default")))

namespace h3 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaChains = 8;
constexpr int kExpChains = 8;
// One 16-byte chunk per lane (4 KB per 256-lane workgroup): measured on 1 GiB
// against 2, 4, 8 and 16 chunks per lane, larger workgroups and grid-stride
// loops, cached and non-temporal accesses, the fastest (6.5 TB/s read +
// write; 16 chunks per lane: 5.2 TB/s).
constexpr int kCopyChunksPerLane = 1;

// Four waves per workgroup; each wave issues iters x 8 independent
// 16x16x32 bf16 matrix-core instructions (eight accumulator chains, so the
// matrix core never waits on a result) and times its loop with the shader
// clock and the 100 MHz reference clock.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ sink,
                                                         uint64_t* __restrict__ clocks) {
  const int tid = threadIdx.x, lane = tid & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)((float)((lane + j) & 7) * 0.125f);
    b[j] = (__bf16)((float)((3 * lane + j) & 7) * 0.0625f);
  }
  f32x4_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  // The clocks are read after the sum, which waits for the last results.
  asm volatile("" ::"v"(s));
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[(int64_t)blockIdx.x * 256 + tid] = s;
  if (lane < 2) clocks[((int64_t)blockIdx.x * 4 + (tid >> 6)) * 2 + lane] = lane ? r1 - r0 : c1 - c0;
}

// Every lane runs eight independent chains x <- exp2(-x): one v_exp_f32 per
// exponential (the negation is a source modifier).
__global__ __launch_bounds__(256) void exp_probe_kernel(int iters, float* __restrict__ sink) {
  float x[kExpChains];
#pragma unroll
  for (int c = 0; c < kExpChains; ++c) x[c] = (float)(threadIdx.x + 7 * c) * (1.0f / 1024.0f);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kExpChains; ++c) x[c] = __builtin_amdgcn_exp2f(-x[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kExpChains; ++c) s += x[c];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Streaming copy of n16 16-byte chunks: every lane loads its chunks (stride
// 256 chunks, so each instruction is one 4 KB coalesced access per
// workgroup) before storing any, non-temporally.
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                         int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * (256 * kCopyChunksPerLane) + threadIdx.x;
  u32x4_t v[kCopyChunksPerLane];
#pragma unroll
  for (int j = 0; j < kCopyChunksPerLane; ++j) {
    const int64_t i = base + j * 256;
    if (i < n16) v[j] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int j = 0; j < kCopyChunksPerLane; ++j) {
    const int64_t i = base + j * 256;
    if (i < n16) __builtin_nontemporal_store(v[j], dst + i);
  }
}

// Bounds the work of one launch to about a second at the chip's rate
// (2^32 workgroup-iterations: 2^31 matrix-core cycles per SIMD, or 2^29
// exponential cycles).
bool probe_shape_ok(int32_t blocks, int32_t iters) {
  return blocks >= 1 && blocks <= 65536 && iters >= 1 && iters <= (1 << 24) &&
         (int64_t)blocks * iters <= (int64_t)1 << 32;
}

int status_of(hipError_t e) { return e == hipSuccess ? H3ATTN_OK : H3ATTN_ERR_HIP; }

}  // namespace
}  // namespace h3

H3_API int h3micro_mfma_bf16(int32_t blocks, int32_t iters, float* sink, uint64_t* clocks, void* stream) {
  if (!sink || !clocks) return H3ATTN_ERR_NULL_POINTER;
  if (!h3::probe_shape_ok(blocks, iters)) return H3ATTN_ERR_BAD_SHAPE;
  if ((reinterpret_cast<uintptr_t>(sink) & 3u) || (reinterpret_cast<uintptr_t>(clocks) & 7u))
    return H3ATTN_ERR_BAD_ALIGNMENT;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(sink), s1 = s0 + (size_t)blocks * 256 * 4;
  const uintptr_t c0 = reinterpret_cast<uintptr_t>(clocks), c1 = c0 + (size_t)blocks * 8 * 8;
  if (s0 < c1 && c0 < s1) return H3ATTN_ERR_ALIASING;
  if (int st = h3::check_gfx950()) return st;
  h3::mfma_probe_kernel<<<dim3((unsigned)blocks), 256, 0, (hipStream_t)stream>>>(iters, sink, clocks);
  return h3::status_of(hipGetLastError());
}

H3_API int h3micro_exp(int32_t blocks, int32_t iters, float* sink, void* stream) {
  if (!sink) return H3ATTN_ERR_NULL_POINTER;
  if (!h3::probe_shape_ok(blocks, iters)) return H3ATTN_ERR_BAD_SHAPE;
  if (reinterpret_cast<uintptr_t>(sink) & 3u) return H3ATTN_ERR_BAD_ALIGNMENT;
  if (int st = h3::check_gfx950()) return st;
  h3::exp_probe_kernel<<<dim3((unsigned)blocks), 256, 0, (hipStream_t)stream>>>(iters, sink);
  return h3::status_of(hipGetLastError());
}

H3_API int h3micro_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return H3ATTN_ERR_NULL_POINTER;
  if (bytes == 0 || bytes % 16 != 0 || bytes / 16 >= ((size_t)1 << 31)) return H3ATTN_ERR_BAD_SHAPE;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u))
    return H3ATTN_ERR_BAD_ALIGNMENT;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(src), b0 = reinterpret_cast<uintptr_t>(dst);
  if (a0 < b0 + bytes && b0 < a0 + bytes) return H3ATTN_ERR_ALIASING;
  if (int st = h3::check_gfx950()) return st;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t per_block = 256 * h3::kCopyChunksPerLane;
  const int64_t grid = (n16 + per_block - 1) / per_block;
  h3::copy_probe_kernel<<<dim3((unsigned)grid), 256, 0, (hipStream_t)stream>>>(
      static_cast<const h3::u32x4_t*>(src), static_cast<h3::u32x4_t*>(dst), n16);
  return h3::status_of(hipGetLastError());
}
