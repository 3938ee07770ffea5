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
// Each (b, s, h) row of 128 bf16 channels (256 B) is handled by 16 lanes
// with full-width coalesced 16-byte accesses; the mean of squares and the
// rotate-half partners move between lanes with DPP. A thread handles the q
// row and the k row at the same (b, s, h), so each rotary table row is read
// once for both; inputs and outputs are streamed with non-temporal loads and
// stores.
#include "h3attn_internal.h"

namespace h3 {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two fp32 values to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Sum over the 16 lanes of a DPP row: quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror (i <-> 7-i), row_mirror (i <-> 15-i).
__device__ inline float sum16(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  return v;
}

// Value of lane i+6 (row_shl:6) or i-6 (row_shr:6) within the DPP row.
__device__ inline float from_lane_plus6(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x106, 0xF, 0xF, false));
}
__device__ inline float from_lane_minus6(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x116, 0xF, 0xF, false));
}

typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));

struct ProArgs {
  ProTensor t0, t1;
  int32_t B, H;            // H = the larger head count of the two tensors
  float eps;
  const float* cos;
  const float* sin;
};

// RMSNorm then the rotary embedding of one lane's 8 channels (8c .. 8c+7)
// of a 128-channel row held by a 16-lane DPP row, in fp32; `scale`
// multiplies the result (it rides on the normalisation factor). The rotated
// lanes (c < 12) take their rotate-half partner from lane c+6 or c-6. Every
// fused multiply-add is written out (fmaf) and no other product meets an
// addition, so every kernel that inlines this computes the same bits.
template <bool NORM, bool ROPE>
__device__ __forceinline__ void norm_rope8(float (&f)[8], const float* w, float eps, float scale,
                                           const float (&cs)[8], const float (&sn)[8], int c) {
  if (NORM) {
    const float4* wp = reinterpret_cast<const float4*>(w + c * 8);
    const float4 w0 = wp[0], w1 = wp[1];
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
    ss = sum16(ss);
    const float r = rsqrtf(fmaf(ss, 1.0f / 128.0f, eps)) * scale;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] * r * wv[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] *= scale;
  }
  if (ROPE) {
    const bool rot = c < 12;
    const float sgn = c < 6 ? -1.0f : 1.0f;   // own*cos + sgn*partner*sin
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float up = from_lane_plus6(f[i]), dn = from_lane_minus6(f[i]);
      const float partner = c < 6 ? up : dn;
      f[i] = rot ? fmaf(sgn * partner, sn[i], f[i] * cs[i]) : f[i];
    }
  }
}

// Loads the 8 rotary pairs of lane c (pairs 8(c mod 6) .. +7) for table row
// `row`, or the identity rotation for the unrotated lanes and rows not loaded.
__device__ __forceinline__ void rope_row8(const float* cos_t, const float* sin_t, int64_t row, int c, bool load,
                                          float (&cs)[8], float (&sn)[8]) {
  if (c < 12 && load) {
    const int jb = (c < 6 ? c : c - 6) * 8;
    const float4* cp = reinterpret_cast<const float4*>(cos_t + row * kRopePairs + jb);
    const float4* sp = reinterpret_cast<const float4*>(sin_t + row * kRopePairs + jb);
    const float4 ca = cp[0], cb = cp[1], sa = sp[0], sb = sp[1];
    cs[0] = ca.x; cs[1] = ca.y; cs[2] = ca.z; cs[3] = ca.w; cs[4] = cb.x; cs[5] = cb.y; cs[6] = cb.z; cs[7] = cb.w;
    sn[0] = sa.x; sn[1] = sa.y; sn[2] = sa.z; sn[3] = sa.w; sn[4] = sb.x; sn[5] = sb.y; sn[6] = sb.z; sn[7] = sb.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) { cs[i] = 1.0f; sn[i] = 0.0f; }
  }
}

__device__ __forceinline__ void unpack8(v4u_t x, float (&f)[8]) {
  f[0] = bf16_lo(x[0]); f[1] = bf16_hi(x[0]);
  f[2] = bf16_lo(x[1]); f[3] = bf16_hi(x[1]);
  f[4] = bf16_lo(x[2]); f[5] = bf16_hi(x[2]);
  f[6] = bf16_lo(x[3]); f[7] = bf16_hi(x[3]);
}

__device__ __forceinline__ v4u_t pack8(const float (&f)[8]) {
  return v4u_t{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

constexpr int kProThreads = 256;
constexpr int kUnitsPerThread = 1;
constexpr int kUnitsPerBlock = kProThreads / 16 * kUnitsPerThread;

// Work unit: one (b, s, h) row of 128 channels. Lane c of a 16-lane DPP row
// holds channels 8c..8c+7, so each wave-wide 16-byte access covers four
// whole rows (1 KB contiguous in BSHD). The rotate-half partner of chunk c
// (c < 6) is chunk c+6, two DPP moves away; chunks 12..15 (channels 96..127)
// are not rotated.
template <bool NORM, bool ROPE>
__global__ __launch_bounds__(kProThreads) void qk_prologue_kernel(ProArgs a) {
  // Each thread takes one (b, s, h) row position and handles the q row and
  // the k row there, so a rotary table row is loaded once for both.
  const int c = threadIdx.x & 15;                      // 16-byte chunk: channels 8c..8c+7
  const int32_t S_all = a.t0.S_out > a.t1.S_out ? a.t0.S_out : a.t1.S_out;
  const int64_t n_units = (int64_t)a.B * S_all * a.H;
  const int64_t first = (int64_t)blockIdx.x * kUnitsPerBlock + (threadIdx.x >> 4);
#pragma unroll
  for (int k = 0; k < kUnitsPerThread; ++k) {
    const int64_t u = first + (int64_t)k * (kProThreads / 16);
    const bool live_u = u < n_units;
    const uint32_t uu = live_u ? (uint32_t)u : 0u;      // unit counts are < 2^31 (host-checked)
    const uint32_t rest = a.t0.div_h.div(uu);
    const int h = (int)(uu - rest * (uint32_t)a.H);
    const uint32_t bq = a.t0.div_s.div(rest);          // div_s divides by S_all
    const int s = (int)(rest - bq * (uint32_t)S_all);
    const int64_t b = (int64_t)bq;
    v4u_t x[2];
    bool live[2], load[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const ProTensor& T = t ? a.t1 : a.t0;
      live[t] = live_u && h < T.H && s < T.S_out;
      load[t] = live[t] && s < item_valid(T.lengths, (int)b, T.which, T.S_valid, T.S_valid);
      // Streamed once: non-temporal loads (measured ~4% faster than cached
      // loads at the full workload).
      x[t] = load[t] ? __builtin_nontemporal_load(
                           reinterpret_cast<const v4u_t*>(T.in + b * T.in_sb + s * T.in_ss + h * T.in_sh + c * 8))
                     : v4u_t{0u, 0u, 0u, 0u};
    }
    float cs[8], sn[8];
    if (ROPE) rope_row8(a.cos, a.sin, s, c, load[0] || load[1], cs, sn);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const ProTensor& T = t ? a.t1 : a.t0;
      float f[8];
      unpack8(x[t], f);
      norm_rope8<NORM, ROPE>(f, T.w, a.eps, T.out_scale, cs, sn, c);
      if (live[t]) {
        // Rows past S_valid are zero-filled, never computed from (absent) data.
        v4u_t r = v4u_t{0u, 0u, 0u, 0u};
        if (load[t]) r = pack8(f);
        __builtin_nontemporal_store(r, reinterpret_cast<v4u_t*>(T.out + b * T.out_sb + s * T.out_ss + h * T.out_sh + c * 8));
      }
    }
  }
}

// The prologue fused with the destination-major Ulysses pack (TeleFuser PR
// #37, section 2.2, step 4). One rank's sequence shard q, k, v [B, S, H, 128]
// (dense BSHD) goes out as P destination chunks per tensor: head h = p Hl + j
// of row (b, s) lands at chunk p, row ((b S + s) Hl + j), so each chunk is one
// contiguous block that an equal-split all-to-all sends to rank p. q and k
// take RMSNorm and the rotary embedding at global position row_offset + s,
// rounded once to bf16; v is copied bit for bit. Same lane layout as the
// prologue: 16 lanes per (b, s, h) row, the q, k and v rows at one (b, s, h)
// in one thread group, so the rotary table row is read once for both.
struct PackArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* q_send;
  uint16_t* k_send;
  uint16_t* v_send;
  const float* w_q;
  const float* w_k;
  const float* cos;
  const float* sin;
  float eps;
  int32_t B, S, H, Hl, row_offset;
  int64_t chunk;           // elements per destination chunk: B * S * Hl * 128
  FastDiv div_h, div_s, div_hl;
};

template <bool NORM, bool ROPE>
__global__ __launch_bounds__(kProThreads) void qkv_pack_kernel(PackArgs a) {
  const int c = threadIdx.x & 15;
  const int64_t n_units = (int64_t)a.B * a.S * a.H;
  const int64_t u = (int64_t)blockIdx.x * kUnitsPerBlock + (threadIdx.x >> 4);
  const bool live = u < n_units;
  const uint32_t uu = live ? (uint32_t)u : 0u;          // unit counts are < 2^31 (host-checked)
  const uint32_t bs = a.div_h.div(uu);                  // b * S + s
  const int h = (int)(uu - bs * (uint32_t)a.H);
  const uint32_t b = a.div_s.div(bs);
  const int s = (int)(bs - b * (uint32_t)a.S);
  const uint32_t p = a.div_hl.div((uint32_t)h);
  const int j = (int)((uint32_t)h - p * (uint32_t)a.Hl);
  const int64_t in_off = (int64_t)uu * kHeadDim + c * 8;
  const int64_t out_off = (int64_t)p * a.chunk + ((int64_t)bs * a.Hl + j) * kHeadDim + c * 8;
  v4u_t xq = v4u_t{0u, 0u, 0u, 0u}, xk = xq, xv = xq;
  if (live) {
    xq = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(a.q + in_off));
    xk = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(a.k + in_off));
    xv = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(a.v + in_off));
  }
  float cs[8], sn[8];
  if (ROPE) rope_row8(a.cos, a.sin, (int64_t)a.row_offset + s, c, live, cs, sn);
  float fq[8], fk[8];
  unpack8(xq, fq);
  unpack8(xk, fk);
  norm_rope8<NORM, ROPE>(fq, a.w_q, a.eps, 1.0f, cs, sn, c);
  norm_rope8<NORM, ROPE>(fk, a.w_k, a.eps, 1.0f, cs, sn, c);
  if (live) {
    __builtin_nontemporal_store(pack8(fq), reinterpret_cast<v4u_t*>(a.q_send + out_off));
    __builtin_nontemporal_store(pack8(fk), reinterpret_cast<v4u_t*>(a.k_send + out_off));
    __builtin_nontemporal_store(xv, reinterpret_cast<v4u_t*>(a.v_send + out_off));
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

// The prepare stage for head dims other than 128, which have neither H3's
// norm nor its rotary embedding: each thread moves one 16-byte chunk (8
// channels) of one (b, s, h) row of t into the head-major workspace,
// multiplied by t.out_scale in fp32 before the bf16 rounding; rows at or
// past the valid length are written as zeros. Rows are numbered
// r = (b * S_out + s) * H + h (below 2^31, host-checked).
template <int D>
__global__ __launch_bounds__(256) void qk_copy_kernel(ProTensor t, int32_t B) {
  constexpr int CPR = D / 8;   // chunks per row
  const int64_t n = (int64_t)B * t.S_out * t.H * CPR;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= n) return;
  const int c = (int)(u % CPR);
  const int r = (int)(u / CPR);
  const int h = r % t.H;
  const int bs = r / t.H;
  const int s = bs % t.S_out;
  const int b = bs / t.S_out;
  v4u_t x = v4u_t{0u, 0u, 0u, 0u};
  if (s < item_valid(t.lengths, b, t.which, t.S_valid, t.S_valid)) {
    x = __builtin_nontemporal_load(
        reinterpret_cast<const v4u_t*>(t.in + b * t.in_sb + s * t.in_ss + h * t.in_sh + c * 8));
    if (t.out_scale != 1.0f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = pack_bf16x2(bf16_lo(x[i]) * t.out_scale, bf16_hi(x[i]) * t.out_scale);
    }
  }
  *reinterpret_cast<v4u_t*>(t.out + b * t.out_sb + s * t.out_ss + h * t.out_sh + c * 8) = x;
}

// The largest norm of the prepared key rows in each chunk of kKnChunk rows
// of one (b, kv head): D/8 lanes per row (16 bytes each), the squares of the
// bf16 values summed in fp32 and over the row's lanes, the maximum over the
// chunk's rows through the waves and LDS, one sqrt.
template <int D>
__global__ __launch_bounds__(256) void key_norm_kernel(const uint16_t* __restrict__ kw, float* __restrict__ kn,
                                                       int32_t Sk_pad, int32_t kn_chunks) {
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int RPI = 256 / CPR;    // rows per iteration of the block
  __shared__ float wave_max[4];
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int c = threadIdx.x % CPR;
  const int r1 = min((chunk + 1) * kKnChunk, Sk_pad);
  const uint16_t* base = kw + (int64_t)bh * Sk_pad * D + c * 8;
  float mx = 0.f;
  for (int r = chunk * kKnChunk + (int)threadIdx.x / CPR; r < r1; r += RPI) {
    const v4u_t x = *reinterpret_cast<const v4u_t*>(base + (int64_t)r * D);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = bf16_lo(x[i]), hi = bf16_hi(x[i]);
      ss = fmaf(lo, lo, ss);
      ss = fmaf(hi, hi, ss);
    }
#pragma unroll
    for (int o = 1; o < CPR; o <<= 1) ss += __shfl_xor(ss, o);
    mx = fmaxf(mx, ss);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0)
    kn[(int64_t)bh * kn_chunks + chunk] = sqrtf(fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3])));
}

template <int D>
hipError_t launch_copy_d(const ProTensor& t, int32_t B, hipStream_t stream) {
  const int64_t n = (int64_t)B * t.S_out * t.H * (D / 8);
  if ((int64_t)B * t.S_out * t.H >= (1ll << 31)) return hipErrorInvalidValue;
  if (n > 0) qk_copy_kernel<D><<<dim3((unsigned)((n + 255) / 256)), 256, 0, stream>>>(t, B);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_prologue(const ProTensor& t0, const ProTensor& t1, int32_t B,
                              float eps, const float* rope_cos, const float* rope_sin,
                              hipStream_t stream) {
  ProArgs a;
  a.t0 = t0;
  a.t1 = t1;
  a.B = B;
  const int32_t H = t0.H > t1.H ? t0.H : t1.H;
  a.H = H;
  a.eps = eps;
  a.cos = rope_cos;
  a.sin = rope_sin;
  const int32_t S_all = t0.S_out > t1.S_out ? t0.S_out : t1.S_out;
  const int64_t units = (int64_t)B * S_all * H;
  if (units >= (1ll << 31)) return hipErrorInvalidValue;
  a.t0.div_h = FastDiv::make((uint32_t)H);
  a.t0.div_s = FastDiv::make((uint32_t)S_all);
  a.t1.div_h = a.t0.div_h;
  a.t1.div_s = a.t0.div_s;
  const dim3 grid((unsigned)((units + kUnitsPerBlock - 1) / kUnitsPerBlock));
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

hipError_t launch_qk_copy(const ProTensor& t0, const ProTensor& t1, int32_t B, int32_t D,
                          hipStream_t stream) {
  for (const ProTensor* t : {&t0, &t1}) {
    hipError_t e;
    switch (D) {
      case 64: e = launch_copy_d<64>(*t, B, stream); break;
      case 256: e = launch_copy_d<256>(*t, B, stream); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_qkv_pack(const QkvPack& t, hipStream_t stream) {
  PackArgs a;
  a.q = t.q;
  a.k = t.k;
  a.v = t.v;
  a.q_send = t.q_send;
  a.k_send = t.k_send;
  a.v_send = t.v_send;
  a.w_q = t.w_q;
  a.w_k = t.w_k;
  a.cos = t.rope_cos;
  a.sin = t.rope_sin;
  a.eps = t.eps;
  a.B = t.B;
  a.S = t.S;
  a.H = t.H;
  a.Hl = t.H / t.P;
  a.row_offset = t.row_offset;
  a.chunk = (int64_t)t.B * t.S * a.Hl * kHeadDim;
  const int64_t units = (int64_t)t.B * t.S * t.H;
  if (units >= (1ll << 31) || a.Hl < 1 || a.Hl * t.P != t.H) return hipErrorInvalidValue;
  a.div_h = FastDiv::make((uint32_t)t.H);
  a.div_s = FastDiv::make((uint32_t)t.S);
  a.div_hl = FastDiv::make((uint32_t)a.Hl);
  const dim3 grid((unsigned)((units + kUnitsPerBlock - 1) / kUnitsPerBlock));
  const bool norm = t.w_q != nullptr;
  const bool rope = t.rope_cos != nullptr;
  if (norm && rope)
    qkv_pack_kernel<true, true><<<grid, kProThreads, 0, stream>>>(a);
  else if (norm)
    qkv_pack_kernel<true, false><<<grid, kProThreads, 0, stream>>>(a);
  else if (rope)
    qkv_pack_kernel<false, true><<<grid, kProThreads, 0, stream>>>(a);
  else
    qkv_pack_kernel<false, false><<<grid, kProThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_key_norms(const uint16_t* kw, float* kn, int32_t BH, int32_t Sk_pad, int32_t kn_chunks, int32_t D,
                            hipStream_t stream) {
  const dim3 grid((unsigned)kn_chunks, (unsigned)BH);
  switch (D) {
    case 64: key_norm_kernel<64><<<grid, 256, 0, stream>>>(kw, kn, Sk_pad, kn_chunks); break;
    case 128: key_norm_kernel<128><<<grid, 256, 0, stream>>>(kw, kn, Sk_pad, kn_chunks); break;
    case 256: key_norm_kernel<256><<<grid, 256, 0, stream>>>(kw, kn, Sk_pad, kn_chunks); break;
    default: return hipErrorInvalidValue;
  }
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
