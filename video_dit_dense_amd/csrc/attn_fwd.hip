// Dense non-causal attention forward at head_dim 128 for gfx950 (MI355X).
//
// Computes, per (b, h) and query row i < q_valid,
//   o_i = sum_{j < kv_valid} softmax_j(scale * q_i . k_j) v_j
// flash-style: key/value tiles stream through LDS, scores never reach HBM,
// and a running max / running sum per query row rescales the accumulator
// (online softmax). QK^T and PV are bf16 matrix-core contractions
// (v_mfma_f32_32x32x16_bf16) accumulated in fp32; the softmax is fp32.
// The step is the dense attention of FastVideo PR #1832 ("Summary": BSHD,
// head_dim 128, dense non-causal) with the valid-front / zero-tail layout of
// TeleFuser PR #37 (sections 2.3 and 2.4).
//
// Orientation. Each wave owns 32 query rows and computes S^T = K Q^T, so the
// matrix-core result puts one query per lane column: lane l holds 16 of the
// 32 keys of a 32x32 score tile for query l%32, and lane l^32 holds the other
// 16. Row max needs one cross-half exchange per tile; the row sum is kept per
// lane and combined once at the end. P^T then feeds O^T = V^T P^T straight
// from registers: the keys a lane holds are exactly the keys its B operand
// needs, provided V^T's key order inside each 16-key group is permuted by
// sigma (swap bits 2 and 3 of the key index). The v relayout kernel writes
// V^T in that order, so every LDS operand read here is one 16-byte access.
//
// Matrix-core operand layouts used (32x32x16, wave64):
//   A (32 x 16): lane l supplies row l%32, k = 8*(l/32) .. 8*(l/32)+7
//   B (16 x 32): lane l supplies column l%32, k = 8*(l/32) .. +7
//   D (32 x 32): lane l register r holds row 8*(r/4) + 4*(l/32) + r%4, col l%32
#include "h3attn_internal.h"

namespace h3 {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

constexpr int kBK = 64;          // keys per LDS tile
constexpr int kKPitch = 136;     // K tile row pitch in bf16 (272 B: rows shift 4 banks)
constexpr int kVPitch = 72;      // V^T tile row pitch in bf16 (144 B)

template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int KCH = kBK * 16 / NT;     // 16-byte K chunks per thread per tile
  constexpr int VCH = 128 * 8 / NT;      // 16-byte V^T chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBK * kKPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][128 * kVPitch];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int g = lane >> 5;

  // Tile order: blocks are dispatched round-robin over the 8 XCDs, so block
  // `bid` runs on XCD bid%8. Give each XCD a contiguous range of tiles (same
  // head, neighbouring query blocks) so its L2 serves one head's K/V stream.
  const int n_qblocks = (a.Sq + BM - 1) / BM;
  const int n_tiles = a.B * a.H * n_qblocks;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int per = n_tiles >> 3, rem = n_tiles & 7;
  const int tile = xcd * per + min(xcd, rem) + (bid >> 3);
  const int bh = tile / n_qblocks;
  const int qb = tile - bh * n_qblocks;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int q0 = qb * BM;

  const int64_t orow = (int64_t)a.H * 128;
  uint16_t* obase = a.o + ((int64_t)b * a.Sq * a.H + h) * 128;

  if (q0 >= a.q_valid) {
    // Whole block lies in the invalid tail: zero rows [q0, min(q0+BM, Sq)).
    for (int idx = tid; idx < BM * 16; idx += NT) {
      const int q = q0 + (idx >> 4);
      if (q < a.Sq) *reinterpret_cast<u32x4_t*>(obase + q * orow + (idx & 15) * 8) = u32x4_t{0u, 0u, 0u, 0u};
    }
    return;
  }

  // Q fragments (B operand of S^T = K Q^T): lane holds query row lq of this
  // wave, channels 16*kk + 8*g .. +7.
  bf16x8_t qf[8];
  {
    const uint16_t* qp = a.qw + ((int64_t)bh * a.Sq_pad + q0 + wave * 32 + lq) * 128 + g * 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = *reinterpret_cast<const bf16x8_t*>(qp + kk * 16);
  }

  const uint16_t* kw = a.kw + (int64_t)bh * a.Sk_pad * 128;
  const uint16_t* vt = a.vt + (int64_t)bh * 128 * a.Sk_pad;
  u32x4_t kreg[KCH], vreg[VCH];

  auto gload = [&](int j) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int idx = tid + i * NT;
      kreg[i] = *reinterpret_cast<const u32x4_t*>(kw + (int64_t)(j * kBK + (idx >> 4)) * 128 + (idx & 15) * 8);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int idx = tid + i * NT;
      vreg[i] = *reinterpret_cast<const u32x4_t*>(vt + (int64_t)(idx >> 3) * a.Sk_pad + j * kBK + (idx & 7) * 8);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int idx = tid + i * NT;
      *reinterpret_cast<u32x4_t*>(&Ks[buf][(idx >> 4) * kKPitch + (idx & 15) * 8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int idx = tid + i * NT;
      *reinterpret_cast<u32x4_t*>(&Vs[buf][(idx >> 3) * kVPitch + (idx & 7) * 8]) = vreg[i];
    }
  };

  f32x16_t acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
  float m_run = -INFINITY;   // running max of scale*log2(e)*s for this lane's query
  float l_run = 0.f;         // running sum of this lane's bf16 probabilities
  const float c = a.scale_log2e;
  const int ntiles = (a.kv_valid + kBK - 1) / kBK;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  gload(0);
  lstore(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) gload(j + 1);
    const uint16_t* ks = Ks[buf];
    const uint16_t* vs = Vs[buf];

    // S^T for keys 32n..32n+31 of the tile.
    f32x16_t s[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[n][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(ks + (n * 32 + lq) * kKPitch + kk * 16 + g * 8);
        s[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[n], 0, 0, 0);
      }
    }

    if (j == ntiles - 1 && (a.kv_valid % kBK) != 0) {
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * kBK + n * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          if (key >= a.kv_valid) s[n][r] = -INFINITY;
        }
    }

    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 15; r += 2) mx = max3(mx, s[0][r], s[0][r + 1]);
    mx = max3(mx, s[0][15], s[1][0]);
#pragma unroll
    for (int r = 1; r < 15; r += 2) mx = max3(mx, s[1][r], s[1][r + 1]);
    mx = fmaxf(mx, s[1][15]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));

    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    bf16x8_t pf[4];
    float psum = 0.f;
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4) {
      const int n = ks4 >> 1, r0 = (ks4 & 1) * 8;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[n][r0 + i], c, -m_new));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[n][r0 + i + 1], c, -m_new));
        const bf16x2_t pp = {(__bf16)p0, (__bf16)p1};
        psum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, psum, false);
        pf[ks4][i] = pp[0];
        pf[ks4][i + 1] = pp[1];
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;

    // O^T (128 x 32) += V^T (128 x 64) P^T (64 x 32), four 32-row d tiles.
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int ks4 = 0; ks4 < 4; ++ks4) {
        const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(vs + (dt * 32 + lq) * kVPitch + ks4 * 16 + g * 8);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks4], acc[dt], 0, 0, 0);
      }

    if (j + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  const float lsum = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / lsum;
  const int q = q0 + wave * 32 + lq;
  if (q < a.Sq) {
    uint16_t* op = obase + q * orow;
    const bool live = q < a.q_valid;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = dt * 32 + rq * 8 + g * 4;
        uint2 val = make_uint2(0u, 0u);
        if (live) {
          val.x = pack_bf16x2(acc[dt][rq * 4 + 0] * inv, acc[dt][rq * 4 + 1] * inv);
          val.y = pack_bf16x2(acc[dt][rq * 4 + 2] * inv, acc[dt][rq * 4 + 3] * inv);
        }
        *reinterpret_cast<uint2*>(op + d0) = val;
      }
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  constexpr int NW = 4;
  constexpr int BM = NW * 32;
  const int64_t n_tiles = (int64_t)a.B * a.H * ((a.Sq + BM - 1) / BM);
  if (n_tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  attn_fwd_kernel<NW><<<dim3((unsigned)n_tiles), NW * 64, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace h3
