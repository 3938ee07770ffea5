// Q/K prologue of the MiniMax-H3 attention step for gfx950, plus the rotary
// table kernel.
//
// The prologue is per-head RMSNorm followed by the rotary embedding on 96 of
// the 128 channels (FastVideo PR #1832, "Preserve H3-specific attention
// behavior"; TeleFuser PR #37, section 2.2, norm then RoPE in one kernel). It
// is HBM-bound: about 7 flop per 4 bytes moved, so the design goal is
// full-width coalesced 16-byte accesses and enough bytes in flight.
//
// The forward path asks for q multiplied by softmax_scale*log2(e) (in fp32,
// before the single bf16 rounding) so the attention kernel's scores come
// out of the matrix core already in exp2 units; the stand-alone entry point
// uses a scale of 1.
//
// Work unit: one (b, s, h) row of 128 bf16 channels (256 B), handled by 8
// lanes. Lane t < 6 holds channel chunks t and t+6, i.e. channels 8t..8t+7
// and their rotate-half partners 48+8t..48+8t+7, so the rotation needs no
// cross-lane traffic. Lanes 6 and 7 hold the pass-through channels 96..127.
// The mean of squares is reduced over the 8 lanes with DPP moves.
#include "h3attn_internal.h"

namespace h3 {
namespace {

struct alignas(16) U4 {
  uint32_t x, y, z, w;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two fp32 values to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline void unpack8(const U4& u, float* f) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
  f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
  f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}

__device__ inline U4 pack8(const float* f) {
  U4 u;
  u.x = pack_bf16x2(f[0], f[1]);
  u.y = pack_bf16x2(f[2], f[3]);
  u.z = pack_bf16x2(f[4], f[5]);
  u.w = pack_bf16x2(f[6], f[7]);
  return u;
}

// Sum over the 8 lanes of an aligned group: quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], then row_half_mirror (lane i <-> 7-i within each 8 lanes).
__device__ inline float sum8(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  return v;
}

struct ProArgs {
  ProTensor t0, t1;
  int32_t nblk0;           // blocks [0, nblk0) serve t0, the rest t1
  int32_t B, H;
  float eps;
  const float* cos;
  const float* sin;
};

constexpr int kProThreads = 256;
constexpr int kUnitsPerThread = 2;
constexpr int kUnitsPerBlock = kProThreads / 8 * kUnitsPerThread;

template <bool NORM, bool ROPE>
__global__ __launch_bounds__(kProThreads) void qk_prologue_kernel(ProArgs a) {
  const bool second = (int32_t)blockIdx.x >= a.nblk0;
  // Field-wise selects keep the argument struct out of scratch memory.
  const uint16_t* in = second ? a.t1.in : a.t0.in;
  uint16_t* out = second ? a.t1.out : a.t0.out;
  const float* w = second ? a.t1.w : a.t0.w;
  const int64_t in_sb = second ? a.t1.in_sb : a.t0.in_sb;
  const int64_t in_ss = second ? a.t1.in_ss : a.t0.in_ss;
  const int64_t in_sh = second ? a.t1.in_sh : a.t0.in_sh;
  const int64_t out_sb = second ? a.t1.out_sb : a.t0.out_sb;
  const int64_t out_ss = second ? a.t1.out_ss : a.t0.out_ss;
  const int64_t out_sh = second ? a.t1.out_sh : a.t0.out_sh;
  const int32_t S_valid = second ? a.t1.S_valid : a.t0.S_valid;
  const int32_t S_out = second ? a.t1.S_out : a.t0.S_out;
  const float out_scale = second ? a.t1.out_scale : a.t0.out_scale;
  const int64_t blk = second ? (int64_t)blockIdx.x - a.nblk0 : (int64_t)blockIdx.x;

  const int t = threadIdx.x & 7;                       // lane within the unit
  const int c0 = t < 6 ? t : 2 * t;                    // 16-byte chunk indices
  const int c1 = t < 6 ? t + 6 : 2 * t + 1;
  const int64_t n_units = (int64_t)a.B * S_out * a.H;
  const int64_t first = blk * kUnitsPerBlock + (threadIdx.x >> 3);

  U4 x0[kUnitsPerThread], x1[kUnitsPerThread];
  int64_t obase[kUnitsPerThread];
  int srow[kUnitsPerThread];
  bool live[kUnitsPerThread], load[kUnitsPerThread];

#pragma unroll
  for (int k = 0; k < kUnitsPerThread; ++k) {
    const int64_t u = first + (int64_t)k * (kProThreads / 8);
    live[k] = u < n_units;
    const int64_t uu = live[k] ? u : 0;
    const int h = (int)(uu % a.H);
    const int64_t rest = uu / a.H;
    const int s = (int)(rest % S_out);
    const int b = (int)(rest / S_out);
    srow[k] = s;
    load[k] = live[k] && s < S_valid;
    obase[k] = b * out_sb + s * out_ss + h * out_sh;
    const int64_t ibase = b * in_sb + s * in_ss + h * in_sh;
    if (load[k]) {
      x0[k] = *reinterpret_cast<const U4*>(in + ibase + c0 * 8);
      x1[k] = *reinterpret_cast<const U4*>(in + ibase + c1 * 8);
    } else {
      x0[k] = U4{0, 0, 0, 0};
      x1[k] = U4{0, 0, 0, 0};
    }
  }

  float w0[8], w1[8];
  if (NORM) {
    const float4* wp = reinterpret_cast<const float4*>(w);
    float4 a0 = wp[c0 * 2], a1 = wp[c0 * 2 + 1], b0 = wp[c1 * 2], b1 = wp[c1 * 2 + 1];
    w0[0] = a0.x; w0[1] = a0.y; w0[2] = a0.z; w0[3] = a0.w;
    w0[4] = a1.x; w0[5] = a1.y; w0[6] = a1.z; w0[7] = a1.w;
    w1[0] = b0.x; w1[1] = b0.y; w1[2] = b0.z; w1[3] = b0.w;
    w1[4] = b1.x; w1[5] = b1.y; w1[6] = b1.z; w1[7] = b1.w;
  }

#pragma unroll
  for (int k = 0; k < kUnitsPerThread; ++k) {
    float f0[8], f1[8];
    unpack8(x0[k], f0);
    unpack8(x1[k], f1);
    if (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(f0[i], f0[i], fmaf(f1[i], f1[i], ss));
      ss = sum8(ss);
      // The output scale rides on the normalisation factor (one fp32 multiply).
      const float r = rsqrtf(ss * (1.0f / 128.0f) + a.eps) * out_scale;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        f0[i] = f0[i] * r * w0[i];
        f1[i] = f1[i] * r * w1[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        f0[i] *= out_scale;
        f1[i] *= out_scale;
      }
    }
    if (ROPE && t < 6 && load[k]) {
      const float4* cp = reinterpret_cast<const float4*>(a.cos + (int64_t)srow[k] * kRopePairs + t * 8);
      const float4* sp = reinterpret_cast<const float4*>(a.sin + (int64_t)srow[k] * kRopePairs + t * 8);
      const float4 ca = cp[0], cb = cp[1], sa = sp[0], sb = sp[1];
      const float cs[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
      const float sn[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = f0[i], q = f1[i];
        f0[i] = p * cs[i] - q * sn[i];
        f1[i] = q * cs[i] + p * sn[i];
      }
    }
    if (live[k]) {
      // Rows past S_valid are zero-filled, never computed from (absent) data.
      const U4 zero = U4{0, 0, 0, 0};
      *reinterpret_cast<U4*>(out + obase[k] + c0 * 8) = load[k] ? pack8(f0) : zero;
      *reinterpret_cast<U4*>(out + obase[k] + c1 * 8) = load[k] ? pack8(f1) : zero;
    }
  }
}

// Rotary tables in fp64, rounded once to fp32. One thread per (row, pair).
__global__ __launch_bounds__(256) void rope_tables_kernel(float* cos_out, float* sin_out, int32_t rows,
                                                          double theta) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)rows * kRopePairs) return;
  const int j = (int)(i % kRopePairs);
  const int64_t p = i / kRopePairs;
  const double inv_freq = pow(theta, -(2.0 * j) / 96.0);
  const double phi = (double)p * inv_freq;
  double s, c;
  sincos(phi, &s, &c);
  cos_out[i] = (float)c;
  sin_out[i] = (float)s;
}

}  // namespace

hipError_t launch_qk_prologue(const ProTensor& t0, const ProTensor& t1, int32_t B, int32_t H,
                              float eps, const float* rope_cos, const float* rope_sin,
                              hipStream_t stream) {
  ProArgs a;
  a.t0 = t0;
  a.t1 = t1;
  a.B = B;
  a.H = H;
  a.eps = eps;
  a.cos = rope_cos;
  a.sin = rope_sin;
  const int64_t u0 = (int64_t)B * t0.S_out * H;
  const int64_t u1 = (int64_t)B * t1.S_out * H;
  const int64_t nb0 = (u0 + kUnitsPerBlock - 1) / kUnitsPerBlock;
  const int64_t nb1 = (u1 + kUnitsPerBlock - 1) / kUnitsPerBlock;
  if (nb0 + nb1 > 0x7fffffffLL) return hipErrorInvalidValue;
  a.nblk0 = (int32_t)nb0;
  const dim3 grid((unsigned)(nb0 + nb1));
  const bool norm = t0.w != nullptr;
  const bool rope = rope_cos != nullptr;
  if (norm && rope)
    qk_prologue_kernel<true, true><<<grid, kProThreads, 0, stream>>>(a);
  else if (norm)
    qk_prologue_kernel<true, false><<<grid, kProThreads, 0, stream>>>(a);
  else if (rope)
    qk_prologue_kernel<false, true><<<grid, kProThreads, 0, stream>>>(a);
  else
    qk_prologue_kernel<false, false><<<grid, kProThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_rope_tables(float* cos_out, float* sin_out, int32_t rows, double theta,
                              hipStream_t stream) {
  const int64_t n = (int64_t)rows * kRopePairs;
  const dim3 grid((unsigned)((n + 255) / 256));
  rope_tables_kernel<<<grid, 256, 0, stream>>>(cos_out, sin_out, rows, theta);
  return hipGetLastError();
}

}  // namespace h3
