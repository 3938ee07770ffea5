// Fused RMSNorm + indexed AdaLN scale/shift for gfx950 (MI355X).
//
// The DiT block's norm before the QKV projection and the final layer's, with
// the AdaLN modulation x * (1 + scale) + shift applied per token from a
// modulation row chosen by an index (TeleFuser PR #37, "2.5 Fuse RMSNorm
// with indexed AdaLN modulation"). The fused kernel keeps every bf16
// rounding of the unfused chain, so its output equals that chain bit for bit:
//   r = fp32(1 / sqrt(mean_c x_c^2 + eps))      per row
//   n = bf16(fp32(x * r) [* w])                 the norm's bf16 output
//   t = bf16(1 + scale[i])
//   u = bf16(n * t)
//   y = bf16(u + shift[i])                      i = clamp(index[b, s], 0, M-1)
// Every operation is an fp32 IEEE operation with round to nearest even, as
// bf16 tensor arithmetic performs it. r comes from an fp64 sum of the
// squares (exact products, ~1e-16 relative error in the sum) and
// correctly rounded fp64 square root and division, so it is the fp32 value
// nearest 1/sqrt(ms + eps) except when that value lies within ~2^-48 of the
// midpoint between two floats.
//
// Schedule. One wave per (b, s) row: the wave issues the loads of its whole
// row (16 bytes per lane per chunk, 1 KB per wave per chunk, coalesced) and,
// for rows of up to 6144 channels, of its modulation rows (shared by every
// token of the same index, so they stay in L2), reduces the sum of squares
// across its 64 lanes, then computes and writes y. The step is bound by HBM:
// x is read once and y written once, 4 bytes per channel per token, both
// with non-temporal accesses (neither is read again by this kernel). A row
// is read in full before any of it is written, so y may be x itself (in
// place).
#include "h3attn_internal.h"

#include <cmath>
#include <type_traits>

namespace h3 {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// The two bf16 values packed in a dword, as fp32 (exact).
__device__ inline float lo_f32(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float hi_f32(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Two fp32 values rounded to bf16 (nearest even, the mode register's
// default) and packed, lo first: one v_cvt_pk_bf16_f32. Written as inline
// asm because the compiler otherwise converts each value on its own when
// the packed result is unpacked again, at twice the conversions.
__device__ inline uint32_t pack_rne(float lo, float hi) {
  uint32_t r;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
  return r;
}

// The modulation of one packed pair: n = bf16 pair of the norm, sc and sh the
// pairs of scale and shift.
__device__ inline uint32_t modulate_pair(uint32_t n, uint32_t sc, uint32_t sh) {
  const uint32_t t = pack_rne(1.0f + lo_f32(sc), 1.0f + hi_f32(sc));
  const uint32_t u = pack_rne(lo_f32(n) * lo_f32(t), hi_f32(n) * hi_f32(t));
  return pack_rne(lo_f32(u) + lo_f32(sh), hi_f32(u) + hi_f32(sh));
}

constexpr int kWavesPerBlock = 4;

// fp64 sum over the 64 lanes of a wave, the same value in every lane: a
// butterfly (each step adds a lane's value and its partner's, so both
// partners compute the same sum) over lane ^ 1, ^ 2 (DPP quad permutes),
// the mirror lane in each 8 and in each 16 (DPP row mirrors), the partner
// row of 16 and the partner half of 32 (permlane swaps).
__device__ inline double wave_sum(double v) {
  auto dpp = [](double x, auto ctrl) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, decltype(ctrl)::value, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), decltype(ctrl)::value, 0xf, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
  };
  v += dpp(v, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
  v += dpp(v, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
  v += dpp(v, std::integral_constant<int, 0x141>{});   // row_half_mirror
  v += dpp(v, std::integral_constant<int, 0x140>{});   // row_mirror
  {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    v = __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi[0] << 32) | (uint32_t)lo[0]) +
        __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi[1] << 32) | (uint32_t)lo[1]);
  }
  {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    v = __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi[0] << 32) | (uint32_t)lo[0]) +
        __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi[1] << 32) | (uint32_t)lo[1]);
  }
  return v;
}

// Raw buffer resource over `bytes` bytes from `base` (wave-uniform, held in
// scalar registers): loads past the range return zeros and stores past it
// are dropped, so a row's ragged last chunk needs no branch.
constexpr int kBufferRsrcWord3 = 0x00020000;   // 32-bit data format, untyped access
__device__ inline __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferRsrcWord3);
}
constexpr int kNonTemporal = 2;   // cache-policy bits of a buffer access: nt

// CPL: 16-byte chunks (8 channels) per lane, enough for the row; chunk c of
// the row is held by lane c % 64 as its chunk c / 64, at byte 16 c of the
// row. Every load is issued before the first is used.
template <int CPL, bool WEIGHT>
__global__ __launch_bounds__(kWavesPerBlock * 64) void scale_shift_kernel(ScaleShiftArgs a) {
  // Wave-uniform (readfirstlane), so the row's buffer resources stay in
  // scalar registers.
  const int row = blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= a.rows) return;   // whole waves only
  const int lane = threadIdx.x & 63;
  const int row_bytes = a.D * 2;

  // The modulation row of this token (the index is wave-uniform).
  const int b = row / a.S;
  int idx = a.index ? __builtin_amdgcn_readfirstlane(a.index[row]) : 0;
  idx = min(max(idx, 0), a.M - 1);
  const int64_t mrow = ((int64_t)b * a.M + idx) * a.D;

  const auto xr = row_rsrc(a.x + (int64_t)row * a.D, row_bytes);
  const auto scr = row_rsrc(a.scale + mrow, row_bytes);
  const auto shr = row_rsrc(a.shift + mrow, row_bytes);
  const int off = lane * 16;
  u32x4_t xv[CPL], sc[CPL], sh[CPL];
  auto load_mod = [&] {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      sc[i] = __builtin_amdgcn_raw_buffer_load_b128(scr, off, i * 1024, 0);
      sh[i] = __builtin_amdgcn_raw_buffer_load_b128(shr, off, i * 1024, 0);
    }
  };
  // Rows of up to 6144 channels also have their modulation rows in flight
  // during the reduction; wider rows load them after it, to stay within
  // the register file.
  constexpr bool kEarlyMod = CPL <= 12;
#pragma unroll
  for (int i = 0; i < CPL; ++i) xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, i * 1024, kNonTemporal);
  if constexpr (kEarlyMod) load_mod();

  // Chunks past the row read as zeros and add nothing.
  double ssq = 0.0;
#pragma unroll
  for (int i = 0; i < CPL; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double lo = lo_f32(xv[i][j]), hi = hi_f32(xv[i][j]);
      ssq = fma(lo, lo, ssq);
      ssq = fma(hi, hi, ssq);
    }
  ssq = wave_sum(ssq);
  const float r = (float)(1.0 / sqrt(ssq / (double)a.D + (double)a.eps));
  if constexpr (!kEarlyMod) {
    __builtin_amdgcn_sched_barrier(0);   // keep the loads after the reduction
    load_mod();
  }

  const auto yr = row_rsrc(a.y + (int64_t)row * a.D, row_bytes);
  const auto wr = row_rsrc(a.w, WEIGHT ? a.D * 4 : 0);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    float w[8];
    if constexpr (WEIGHT) {
      const u32x4_t w0 = __builtin_amdgcn_raw_buffer_load_b128(wr, 2 * off, i * 2048, 0);
      const u32x4_t w1 = __builtin_amdgcn_raw_buffer_load_b128(wr, 2 * off, i * 2048 + 16, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[j] = __uint_as_float(w0[j]);
        w[4 + j] = __uint_as_float(w1[j]);
      }
    }
    u32x4_t out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float n0 = lo_f32(xv[i][j]) * r;
      float n1 = hi_f32(xv[i][j]) * r;
      if constexpr (WEIGHT) {
        n0 *= w[2 * j];
        n1 *= w[2 * j + 1];
      }
      out[j] = modulate_pair(pack_rne(n0, n1), sc[i][j], sh[i][j]);
    }
    // The chunk offset goes in the vector offset, soffset stays the
    // constant 0: with an SGPR soffset the compiler assumes a 16-byte
    // buffer store needs no wait state before a vector instruction rewrites
    // its data registers, and on gfx950 the store then intermittently wrote
    // the new values of the last lanes of each 16.
    __builtin_amdgcn_raw_buffer_store_b128(out, yr, off + i * 1024, 0, kNonTemporal);
  }
}

template <int CPL>
hipError_t launch_cpl(const ScaleShiftArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.rows + kWavesPerBlock - 1) / kWavesPerBlock));
  if (a.w)
    hipLaunchKernelGGL((scale_shift_kernel<CPL, true>), grid, dim3(kWavesPerBlock * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((scale_shift_kernel<CPL, false>), grid, dim3(kWavesPerBlock * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scale_shift(const ScaleShiftArgs& a, hipStream_t stream) {
  const int cpl = (a.D / 8 + 63) / 64;
  if (a.rows <= 0) return hipSuccess;
  if (cpl <= 1) return launch_cpl<1>(a, stream);
  if (cpl <= 2) return launch_cpl<2>(a, stream);
  if (cpl <= 4) return launch_cpl<4>(a, stream);
  if (cpl <= 8) return launch_cpl<8>(a, stream);
  if (cpl <= 12) return launch_cpl<12>(a, stream);
  if (cpl <= 16) return launch_cpl<16>(a, stream);
  if (cpl <= 24) return launch_cpl<24>(a, stream);
  if (cpl <= 32) return launch_cpl<32>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace h3
