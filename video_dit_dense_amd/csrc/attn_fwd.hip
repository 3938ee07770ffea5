// Attention forward for gfx950 (MI355X): the dense step and its variants.
//
// Computes, per (b, h) and query row i < q_valid,
//   o_i = sum_{j visible to i} softmax_j(scale * q_i . k_j) v_j
// flash-style: key/value blocks stream through LDS, scores never reach HBM,
// and each row's softmax offset is either an a priori bound of its scores or
// a running maximum that rescales the accumulator (online softmax). QK^T and
// PV are bf16 matrix-core contractions (v_mfma_f32_16x16x32_bf16, wave64)
// accumulated in fp32; the softmax is fp32.
// The main step is the dense attention of FastVideo PR #1832 ("Summary":
// BSHD, head_dim 128, dense non-causal) with the valid-front / zero-tail
// layout of TeleFuser PR #37 (sections 2.3 and 2.4): key j is visible to
// row i iff j < kv_valid. The variants narrow that set: the causal mask
// (j <= i), per-item valid lengths and grouped key/value heads (FastVideo PR
// #1799, "Implementation"), and a frame window with anchor frames (SGLang PR
// #37903, "Modifications", hybrid_window_attn_h3), whose optional softmax
// gate multiplies each output row by sigmoid(g). Head dims 64, 128 and 256
// share the code through the Geo<D, QT> tiling constants.
//
// Orientation. Each wave owns QT 16-row query tiles (four at head dim 64;
// two or three at 128, chosen per launch; at 256 a pair of waves shares two)
// and computes S^T = K Q^T: K comes from LDS as the A operand and Q stays in
// registers as the B operand, so each lane holds 8 scores of each query
// tile, and P^T feeds O^T = V^T P^T straight from registers. V^T's keys are
// permuted inside each 32-key sub-tile (key_of_position) so that the keys a
// lane holds are the ones its PV operand needs. The operand layouts are
// described where the fragments are built.
//
// Schedule. A workgroup is eight waves, one workgroup per CU, so every SIMD
// runs two waves. Keys are processed in 32-key sub-tiles u, and step u is
// split by workgroup barriers into two phases:
//   X: matrix-core work only: QK^T of sub-tile u+1 and PV of sub-tile u;
//   Y: vector and LDS work: the exponentials and row sums that turn the
//      scores of u+1 into the next PV operand (and, on the online path, the
//      row maxima), the first fragment reads of the next X phase and the
//      ring refills.
// The two waves of a SIMD run the phases in opposition (the second passes
// one extra barrier first), so while one feeds the matrix core the other does
// the softmax: a ping-pong. Both run the same instructions in the same
// order, so the result does not depend on which wave runs which phase.
// Sub-tiles land in an LDS ring (eight slots at head dims 64 and 128, four
// at 256) through direct buffer->LDS loads issued several sub-tiles ahead;
// the loads use buffer resources in scalar registers, so they cost no
// vector instructions. The chip runs this kernel at its power limit, so
// every vector instruction and LDS byte per step costs clock: the step
// keeps them few.
//
// Chip schedule. A workgroup owns one (b, h, query block) tile and one CU,
// so tiles run in rounds of one per CU. In the uniform mode (no causal mask,
// per-item lengths or window), when the last round is only partly full, its
// tiles are not run whole: their 32-key steps are divided evenly over up to
// one workgroup per CU, each workgroup writes an fp32 partial result
// (un-normalised accumulator, offset, row sum) per tile it touches, and
// attn_merge_kernel combines them. Tiles wholly past q_valid only write
// zeros. The general mode (the other variants) runs one workgroup per tile,
// each finding its own key ranges. Short key ranges at head dim 128 keep
// their keys resident in LDS instead (attn_resident_kernel).
//
// Exponent arithmetic. q arrives pre-multiplied by softmax_scale*log2(e)
// (applied in fp32 by the prologue before its single bf16 rounding), so
// scores leave the matrix core in exp2 units and p = exp2(s - m).
//
// Workspace layouts read here (written by the prologue and the relayout):
//   qw [B*H][Sq_pad][D]            rows >= q_valid zero
//   kw [B*Hkv][Sk_pad][D]          rows >= kv_valid zero
//   vt [B*Hkv][Sk_pad/32][D][32]   vt[.., x, d, p] = v[key 32x + key_of_position(p)][d], zero past kv_valid
#include "h3attn_internal.h"

#include <algorithm>
#include <atomic>
#include <functional>
#include <mutex>
#include <numeric>
#include <queue>
#include <vector>
#include <type_traits>
#include <utility>

namespace h3 {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
// Word 3 of a raw (stride 0) buffer resource on gfx9: 32-bit data format,
// untyped loads.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Direct global->LDS load of 16 bytes per lane: lane i's bytes land at
// dst + 16 i. `base` must be wave-uniform; the buffer resource built from it
// lives in SGPRs and covers `bytes` bytes, so the only per-lane operand is the
// 32-bit byte offset.
__device__ __forceinline__ void load_lds16(const void* base, int bytes, int byte_off, uint8_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferRsrcWord3), (lds_void_t*)dst, 16,
      byte_off, 0, 0, 0);
}

// The same load with the buffer's sub-block in the scalar offset: base and
// bytes fixed for a whole segment, so the resource is built once.
__device__ __forceinline__ void load_lds16_soff(const void* base, int bytes, int byte_off, int soff, uint8_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferRsrcWord3), (lds_void_t*)dst, 16,
      byte_off, soff, 0, 0);
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Compiles to v_max3_f32 (scores are finite or -inf; built with
// -fno-honor-nans, so no NaN canonicalisation is emitted). Written in C++
// rather than inline asm so the compiler sees the read of matrix-core
// results and inserts the required wait states.
__device__ inline float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Maximum / sum of x over the lane pair (l, l^32) with v_permlane32_swap.
__device__ inline float max_lane_pair(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
}
__device__ inline float sum_lane_pair(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
}

// Maximum of x over the whole wave, in every lane: within each 16-lane row
// by DPP (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror), then
// over the four rows with v_permlane16_swap and v_permlane32_swap.
__device__ inline float wave_max(float x) {
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false)));
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false)));
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return max_lane_pair(fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1])));
}

// The largest prepared key norm of key/value head bh_kv (the maximum over
// its chunks' maxima), in every lane of the wave.
__device__ inline float key_norm_max(const AttnArgs& a, int bh_kv) {
  const float* kn = a.knorm + (int64_t)bh_kv * a.kn_chunks;
  float x = 0.f;
  for (int i = (int)(threadIdx.x & 63); i < a.kn_chunks; i += 64) x = fmaxf(x, kn[i]);
  return wave_max(x);
}

// Sum of squares of bf16 values, in fp32.
__device__ inline float sum_sq(const bf16x8_t& v, float ss) {
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf((float)v[e], (float)v[e], ss);
  return ss;
}

// Lazy rescaling: the running max m used in p = exp2(s - m) is only raised
// when a score exceeds it by more than 2^kRescaleLog2 (in the exp2 domain), so
// p <= 2^8 and the fp32 accumulator is rescaled only a handful of times per
// row. The result o = O / l does not depend on m; bf16 rounding of p is
// relative, so neither does its accuracy.
constexpr float kRescaleLog2 = 8.0f;
// The largest a priori score bound M (exp2 units) the fixed-offset softmax
// takes: scores then lie in [-M, M], so exp2(s - M) >= 2^-120 stays a normal
// fp32 and bf16 number and no row sum can underflow.
constexpr float kBoundMax = 60.0f;
// Relative slack of the data-derived bound |q_i| max_j |k_j|: the fp32 sums
// of squares and square roots of bf16 rows and the matrix core's fp32
// accumulation of the score each err by far less.
constexpr float kBoundSlack = 1.0f + 1.0f / 1024.0f;
constexpr int kSub = 32;                       // keys per sub-tile

// Tiling by head dim D (64, 128 or 256) and query tiles per wave QT_: eight
// waves per workgroup, two per SIMD, 16x16x32 matrix-core instructions on QT
// 16-row query tiles per wave (four at 64, so 512 rows per workgroup; two or
// three at 128, 256 or 384 rows; two at 256). At 256 the
// waves work in pairs (kCS): both waves of a pair hold the same 32 query
// rows; each computes the scores of half of every sub-tile's keys and the
// output of half of the channels, so that its accumulators and fragment
// reads are those of head dim 128, and the pair exchanges probabilities
// through LDS (128 rows per workgroup).
template <int D, int QT_>
struct Geo {
  static_assert(D == 64 || D == 128 || D == 256, "head dim");
  static_assert(QT_ >= attn_qt_min(D) && QT_ <= attn_qt_max(D), "query tiles per wave");
  static constexpr int NW = 8;                          // waves per workgroup
  static constexpr int WPE = 2;                         // waves per SIMD
  static constexpr bool kCS = D == 256;                 // channel-split wave pairs
  static constexpr int DW = kCS ? D / 2 : D;            // channels per wave
  static constexpr int QT = QT_;                        // 16-row query tiles per wave
  static constexpr int WROWS = 16 * QT;                 // query rows per wave (per pair when kCS)
  static constexpr int BM = (kCS ? NW / 2 : NW) * WROWS;   // query rows per workgroup
  static constexpr int kRing = D <= 128 ? 8 : 4;        // ring depth (sub-tiles)
  static constexpr int kKBytes = kSub * D * 2;          // K sub-tile: 32 rows x 2D bytes
  static constexpr int kVBytes = D * kSub * 2;          // V^T sub-tile: D rows x 64 B
  static constexpr int kBufBytes = kKBytes + kVBytes;   // one ring slot
  static constexpr int kSwz = (D / 8 < 16 ? D / 8 : 16) - 1;   // K chunk swizzle mask
  static constexpr int nK = kKBytes / 1024;             // 1 KB direct loads per sub-tile (K)
  static constexpr int LDPS = (kKBytes + kVBytes) / 1024 / NW;   // per wave per sub-tile
  // LDS: the ring (K sub-tiles, then V^T sub-tiles), for kCS the pairs'
  // exchange areas (row maxima and sums: 512 B per wave; probabilities: 1 KB
  // per wave), then one int per wave (its SIMD).
  static constexpr int kXOff = kRing * kBufBytes;
  static constexpr int kXScores = kCS ? NW * 512 : 0;
  static constexpr int kXProbs = kCS ? NW * 1024 : 0;
  static constexpr int kSimdOff = kXOff + kXScores + kXProbs;
  static constexpr int kLdsBytes = kSimdOff + NW * 4;
  // Partial record layout per thread: kRecA accumulator floats, then QT row
  // offsets and QT partial sums.
  static constexpr int kRecA = WROWS * DW / 64;
  static_assert(LDPS * NW * 1024 == kKBytes + kVBytes, "tile split");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
  static_assert(BM == attn_rows(D, QT) && NW * 64 == attn_threads(D), "tiling constants");
  static_assert(kRing * kKBytes <= 65536, "K sub-tiles within the first 64 KB");
  // Floats each thread writes to a partial record fill exactly the record
  // size the host reserves per record.
  static constexpr int kRecFloats = attn_part_floats(D, QT);
  static_assert((kRecA + 2 * QT) * NW * 64 == kRecFloats && kRecFloats <= attn_part_floats_max(D),
                "partial record size");
};

// LDS layouts (no padding). A ds_read_b128 is served in four passes of 16
// lanes, 256 bytes (all 64 banks) each; lanes 0-31 split by the parity of
// lane bits 2..4 ({0-3, 12-15, 20-27} and the rest), lanes 32-63 likewise
// (measured with the bank-conflict counter on single lane pairs). The XOR
// swizzles put the 16 lanes of every pass of a fragment read on 16 distinct
// 16-byte bank groups:
//   K:   row r (key), 16-byte chunk c (channels 8c..8c+7) at r*2D + (c ^ (r & kSwz))*16
//   V^T: row d (channel), chunk c (positions 8c..8c+7) at d*64 + (c ^ vt_swz(d))*16
// In a V^T fragment read lane (l16, g4) takes chunk g4 of row 16 ct + l16,
// i.e. bank group 4 (l16 & 3) + (g4 ^ vt_swz(l16)); a pass holds two values
// of l16 >> 2 for each of two g4, and vt_swz maps them to four distinct
// offsets (a swizzle of (d >> 2) & 3 itself leaves two-way conflicts).
__host__ __device__ constexpr int vt_swz(int d) { return (4 - ((d >> 2) & 3)) & 3; }

// Writes NT16 x 16 channels of one query row of a finished tile (obase
// points at the first of them): o = acc * inv rounded to bf16, or +0.0 for
// rows at or past q_valid. With a gate (gate_row: the head's gate column of
// the batch item, stride H) the row is also multiplied by sigmoid(gate), the
// softmax gate epilogue. In the 16x16 output layout lane (l, register r of
// acc[ct]) holds channel 16 ct + 4 (l/16) + r (g4 = l/16). For each pair of
// channel tiles (2m, 2m + 1) the lanes l and l ^ 16 (same row) trade halves
// with v_permlane16_swap, so that every lane then holds 8 consecutive
// channels, 16 ct + 8 (g4 >> 1) with ct = 2m + (g4 & 1): each store
// instruction writes 64 contiguous bytes of each of 16 rows (the row's
// lanes are active or inactive together), streamed past the caches.
template <int D, int NT16>
__device__ inline void store_row16(const AttnArgs& a, uint16_t* obase, int q, int g4, const f32x4_t* acc,
                                   float inv, int q_valid, const uint16_t* gate_row) {
  uint16_t* op = obase + q * ((int64_t)a.H * D);
  const bool live = q < q_valid;
  if (gate_row && live) {
    const float gv = __uint_as_float((uint32_t)gate_row[(int64_t)q * a.H] << 16);
    inv *= 1.0f / (1.0f + __expf(-gv));
  }
#pragma unroll
  for (int m = 0; m < NT16 / 2; ++m) {
    uint32_t e0 = 0u, e1 = 0u, o0 = 0u, o1 = 0u;
    if (live) {
      e0 = pack_bf16x2(acc[2 * m][0] * inv, acc[2 * m][1] * inv);
      e1 = pack_bf16x2(acc[2 * m][2] * inv, acc[2 * m][3] * inv);
      o0 = pack_bf16x2(acc[2 * m + 1][0] * inv, acc[2 * m + 1][1] * inv);
      o1 = pack_bf16x2(acc[2 * m + 1][2] * inv, acc[2 * m + 1][3] * inv);
    }
    const auto s0 = __builtin_amdgcn_permlane16_swap(e0, o0, false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(e1, o1, false, false);
    const int ch = 16 * (2 * m + (g4 & 1)) + 8 * (g4 >> 1);
    const u32x4_t val = {(uint32_t)s0[0], (uint32_t)s1[0], (uint32_t)s0[1], (uint32_t)s1[1]};
    if (q < a.Sq) __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(op + ch));
  }
}

// store_row16 through a buffer resource covering the batch item's output rows
// [0, Sq): rows at or past Sq fall outside it and the hardware drops their
// stores, so the stores need no branch. ob: byte offset of the head's
// channel 0 in row 0; gmul: the row's gate factor sigmoid(g), or 1. Without
// a branch around them the stores leave the compiler's count of outstanding
// memory operations exact, so a later wait for loads issued before them does
// not also wait for the stores.
template <int D, int NT16>
__device__ inline void store_row16_rsrc(const AttnArgs& a, __amdgpu_buffer_rsrc_t rsrc, uint32_t ob, int q, int g4,
                                        const f32x4_t* acc, float inv, int q_valid) {
  const uint32_t orow = ob + (uint32_t)q * (uint32_t)(a.H * D * 2);
  const bool live = q < q_valid;
#pragma unroll
  for (int m = 0; m < NT16 / 2; ++m) {
    uint32_t e0 = 0u, e1 = 0u, o0 = 0u, o1 = 0u;
    if (live) {
      e0 = pack_bf16x2(acc[2 * m][0] * inv, acc[2 * m][1] * inv);
      e1 = pack_bf16x2(acc[2 * m][2] * inv, acc[2 * m][3] * inv);
      o0 = pack_bf16x2(acc[2 * m + 1][0] * inv, acc[2 * m + 1][1] * inv);
      o1 = pack_bf16x2(acc[2 * m + 1][2] * inv, acc[2 * m + 1][3] * inv);
    }
    const auto s0 = __builtin_amdgcn_permlane16_swap(e0, o0, false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(e1, o1, false, false);
    const int ch = 16 * (2 * m + (g4 & 1)) + 8 * (g4 >> 1);
    const u32x4_t val = {(uint32_t)s0[0], (uint32_t)s1[0], (uint32_t)s0[1], (uint32_t)s1[1]};
    __builtin_amdgcn_raw_buffer_store_b128(val, rsrc, orow + ch * 2, 0, 0);
  }
}

// Partial record of a split tile, per logical thread t (64 lwave + lane) of
// the workgroup (fp32, thread-contiguous so every access is coalesced):
// accumulator register r at [r * 512 + t] (kRecA of them), then the QT row
// offsets and the QT partial row sums.

// f(integral_constant<int, K>) for each K of the sequence, in order.
template <int... K, typename F>
__device__ __forceinline__ void for_each_index(std::integer_sequence<int, K...>, F&& f) {
  (f(std::integral_constant<int, K>{}), ...);
}

// Workgroup barrier without a memory fence: the callers order LDS traffic
// through the ring schedule and their own vmcnt waits. The "memory" clobber
// keeps the compiler from moving memory operations across it.
__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }

// D: the head dim. QT_: query tiles per wave. WIN: the frame-window variant
// (general mode with a.win_F > 0); the other modes are compiled without its
// per-lane window bounds and first-key bookkeeping, which would cost
// registers in the steady state.
template <int D, int QT_, bool WIN>
__global__ __launch_bounds__((Geo<D, QT_>::NW * 64))
__attribute__((amdgpu_waves_per_eu(Geo<D, QT_>::WPE, Geo<D, QT_>::WPE)))
void attn_fwd_kernel(AttnArgs a) {
  using G = Geo<D, QT_>;
  constexpr int NW = G::NW;
  constexpr int BM = G::BM;
  constexpr int T = NW * 64;
  constexpr int LDPS = G::LDPS;                // 1 KB load instructions per wave per sub-tile
  constexpr int kRing = G::kRing;
  constexpr int kKBytes = G::kKBytes;
  constexpr int kBufBytes = G::kBufBytes;
  // One LDS object only: the ring, then the per-wave SIMD ids. (With a
  // second LDS variable the compiler can no longer tell fragment reads from
  // the ring's DMA writes and waits for every load in flight before each.)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[G::kLdsBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  // Role of this wave among the waves that share its SIMD (HW_ID bits 5:4
  // name the SIMD): the second one of each SIMD runs one phase behind.
  // Channel-split pairs (head dim 256) must run in the same phase: when every
  // SIMD holds two waves, the waves of one role (one per SIMD) pair up by
  // SIMD (0 with 1, 2 with 3); otherwise every wave takes role 0 (no phase
  // offset) and waves 2p and 2p + 1 pair up. pair: the wave's (or pair's)
  // query rows; half: its channel half.
  int role = 0, pair = wave, half = 0;
  {
    int* simd_of = reinterpret_cast<int*>(lds + G::kSimdOff);
    if (lane == 0) simd_of[wave] = (int)(__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4) & 3);
    __syncthreads();
    const int mine = simd_of[wave];
    int on_simd[4] = {0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      role += (w < wave && simd_of[w] == mine) ? 1 : 0;
      on_simd[simd_of[w] & 3] += 1;
    }
    role = __builtin_amdgcn_readfirstlane(role & 1);
    if constexpr (G::kCS) {
      const bool regular = on_simd[0] == 2 && on_simd[1] == 2 && on_simd[2] == 2 && on_simd[3] == 2;
      if (regular) {
        pair = 2 * role + (mine >> 1);
        half = mine & 1;
      } else {
        role = 0;
        pair = wave >> 1;
        half = wave & 1;
      }
      pair = __builtin_amdgcn_readfirstlane(pair);
      half = __builtin_amdgcn_readfirstlane(half);
      role = __builtin_amdgcn_readfirstlane(role);
    }
  }
  // Logical wave: the position of this wave's rows and channels in the
  // workgroup's tile, which indexes its share of a partial record.
  const int lwave = G::kCS ? 2 * pair + half : wave;

  const int n_qblocks = (a.Sq + BM - 1) / BM;
  const int bid = blockIdx.x;
  // Zero rows [q0, min(q0 + BM, Sq)) of head bh: a tile with no valid query
  // row or no valid key.
  auto zero_tile = [&](int bh, int q0) {
    const int b = bh / a.H, h = bh - b * a.H;
    uint16_t* obase = a.o + ((int64_t)b * a.Sq * a.H + h) * D;
    const int64_t orow = (int64_t)a.H * D;
    constexpr int CPR = D / 8;   // 16-byte chunks per row
    for (int idx = tid; idx < BM * CPR; idx += T) {
      const int q = q0 + idx / CPR;
      if (q < a.Sq) *reinterpret_cast<u32x4_t*>(obase + q * orow + (idx % CPR) * 8) = u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  // This block's work: one or two segments, each a query tile (head bh,
  // first row q0) and its sub-tiles [xb, xe), finished either into o
  // (rec < 0) or into partial record rec. Per segment also: the valid query
  // rows qv (rows at or past it are written as zeros) and the valid keys kvv.
  int bh0, q00, xb0, xe0, rec0, bh1 = 0, q01 = 0, xb1 = 0, xe1 = 0, rec1 = -1, nseg = 1;
  int qv_t = a.q_valid, kvv_t = a.kv_valid;
  // Frame window: virtual steps v < wn1 read sub-tile v, later ones sub-tile
  // v + ws2; win_fast when every row of the tile sees the same whole
  // sub-tiles (only the key-padding end needs the mask).
  int wn1 = 0x7fffffff, ws2 = 0, win_cap = 0;
  bool win_fast = true;
  if (a.general) {
    // One tile per block. With the causal mask a tile's work grows with its
    // query block, so blocks take the longest tiles first.
    const int nbh = a.B * a.H;
    int qb;
    if (a.causal) {
      int rank;
      spread_tile(bid, n_qblocks, nbh, a.lengths != nullptr, rank, bh0);
      qb = n_qblocks - 1 - rank;
    } else if (WIN) {
      // Block bid takes rank r and head bh from spread_tile. The query block
      // of rank r is r (increasing order: the anchor frames, whose dense rows
      // see the most keys, first) or, when the launcher found that it
      // shortens the schedule, the block of rank r in the order of
      // decreasing sub-tile count (ties by index) of its batch item, ranked
      // in LDS before the ring is filled.
      int rank;
      spread_tile(bid, n_qblocks, nbh, a.lengths != nullptr, rank, bh0);
      qb = rank;
      if (a.win_longest_first && n_qblocks <= kWinOrderMax) {
        const int b = bh0 / a.H;
        const int qv = item_valid(a.lengths, b, 0, a.q_valid, a.Sq);
        const int kvv = item_valid(a.lengths, b, 1, a.kv_valid, a.Sk);
        // Unique keys (win_rank_key), so the block of rank r has exactly r
        // larger keys; a padding key of zero is below them all.
        uint32_t* key = reinterpret_cast<uint32_t*>(lds);   // [n4] keys, then the chosen block
        const int n4 = (n_qblocks + 3) & ~3;
        for (int j = tid; j < n4; j += T) {
          uint32_t k = 0;
          if (j < n_qblocks) {
            const int xe = (j * BM >= qv || kvv == 0) ? 0 : win_span(a.win_F, a.win_C, a.win_R, a.win_A, BM, j * BM, qv, kvv).xe;
            k = win_rank_key(xe, j);
          }
          key[j] = k;
        }
        __syncthreads();
        // One pass over the keys counts, for each of this thread's blocks
        // j = tid + m T, the larger ones (several reads in flight).
        constexpr int JM = (kWinOrderMax + T - 1) / T;
        uint32_t kj[JM];
        int rj[JM];
#pragma unroll
        for (int m = 0; m < JM; ++m) {
          const int j = tid + m * T;
          kj[m] = j < n_qblocks ? key[j] : 0xffffffffu;
          rj[m] = 0;
        }
#pragma unroll 4
        for (int i = 0; i < n4; i += 4) {
          const u32x4_t k4 = *reinterpret_cast<const u32x4_t*>(key + i);
#pragma unroll
          for (int m = 0; m < JM; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) rj[m] += k4[e] > kj[m] ? 1 : 0;
        }
#pragma unroll
        for (int m = 0; m < JM; ++m)
          if (tid + m * T < n_qblocks && rj[m] == rank) key[n4] = (uint32_t)(tid + m * T);
        __syncthreads();
        qb = __builtin_amdgcn_readfirstlane((int)key[n4]);
        __syncthreads();   // the ring fill overwrites the keys
      }
    } else {
      bh0 = bid / n_qblocks;
      qb = bid - bh0 * n_qblocks;
    }
    q00 = qb * BM;
    const int b = bh0 / a.H;
    qv_t = item_valid(a.lengths, b, 0, a.q_valid, a.Sq);
    kvv_t = item_valid(a.lengths, b, 1, a.kv_valid, a.Sk);
    if (q00 >= qv_t || kvv_t == 0) {
      zero_tile(bh0, q00);
      return;
    }
    // Keys [0, key_end): with the causal mask no row of the tile sees a key
    // at or past its last row + 1.
    const int key_end = a.causal ? min(kvv_t, q00 + BM) : kvv_t;
    xb0 = 0;
    xe0 = (key_end + kSub - 1) / kSub;
    rec0 = -1;
    if constexpr (WIN) {
      const WinSpan w = win_span(a.win_F, a.win_C, a.win_R, a.win_A, BM, q00, qv_t, kvv_t);
      win_cap = w.cap;
      wn1 = w.wn1;
      ws2 = w.ws2;
      xe0 = w.xe;
      win_fast = w.fast;
      if (xe0 == 0) {
        zero_tile(bh0, q00);
        return;
      }
    }
  } else {
    const int NU = (a.kv_valid + kSub - 1) / kSub;   // sub-tiles with at least one valid key
    int g0 = 0, g1 = 0;
    if (bid < a.n_whole) {
      g0 = xcd_order(bid, a.n_whole);
      xb0 = 0;
      xe0 = NU;
      rec0 = -1;
    } else if (bid < a.n_whole + a.n_split_blocks) {
      // Split tiles (split_segments): block j takes its share of the split
      // tiles' steps, at most NU steps over at most two tiles.
      const SplitSeg sg = split_segments(xcd_order(bid - a.n_whole, a.n_split_blocks), a.n_split, NU,
                                         a.n_split_blocks);
      g0 = a.n_whole + sg.tile;
      xb0 = sg.kb0;
      xe0 = sg.kb0 + (sg.xe0 - sg.xb0);
      rec0 = sg.rec0;
      if (sg.nseg == 2) {
        nseg = 2;
        g1 = g0 + 1;
        xb1 = sg.kb1;
        xe1 = sg.kb1 + sg.xe1;
        rec1 = sg.rec1;
      }
    } else {
      // A tile wholly past q_valid.
      const int nqz = n_qblocks - a.nqv;
      const int z = bid - a.n_whole - a.n_split_blocks;
      const int bh = z / nqz;
      zero_tile(bh, (a.nqv + (z - bh * nqz)) * BM);
      return;
    }
    bh0 = g0 / a.nqv;
    q00 = (g0 - bh0 * a.nqv) * BM;
    bh1 = g1 / a.nqv;
    q01 = (g1 - bh1 * a.nqv) * BM;
  }

#pragma nounroll
  for (int si = 0; si < nseg; ++si) {
  const int bh = si ? bh1 : bh0;
  const int q0 = si ? q01 : q00;
  const int xb = si ? xb1 : xb0;
  const int xe = si ? xe1 : xe0;
  const int rec = si ? rec1 : rec0;
  const int qv_seg = qv_t;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int bh_kv = b * a.Hkv + h / (a.H / a.Hkv);
  uint16_t* obase = a.o + ((int64_t)b * a.Sq * a.H + h) * D;
  const uint16_t* gate_row = a.gate ? a.gate + (int64_t)b * a.Sq * a.H + h : nullptr;
  // All head dims on v_mfma_f32_16x16x32_bf16 (A 16 x 32: lane l supplies
  // row l%16, k = 8(l/16) .. +7; B 32 x 16: column l%16, the same k; D 16 x
  // 16: lane l register r holds row 4(l/16) + r, column l%16). The smaller
  // shape sustains more flops at the chip's power limit. Each wave keeps its
  // 16 QT query rows as QT 16-row tiles qt and works on DW channels: QK^T is 2
  // key tiles x QT query tiles x DW/32 channel chunks (each K fragment serves
  // every query tile), so lane l holds, for query row 16 qt + l%16, the 8
  // keys 16 kt + 4 g4 + r (g4 = l/16, r < 4); a row's 32 keys are spread over
  // the four lanes l%16 + 16 j. PV takes those 8 keys as positions 8 g4 .. 8
  // g4 + 7 of the sub-tile, with V^T's keys permuted to match (position 8g + j
  // holds key 16 (j/4) + 4g + j%4), and is DW/16 channel tiles x QT query
  // tiles (each V^T fragment serves every query tile). Head dim 64 holds four
  // query tiles (64 rows) per wave, so that each fragment read and each
  // step's softmax feed as many matrix-core cycles as at 128. Head dim 128
  // holds two or three (the launcher picks per launch): three feed each
  // fragment read and each direct load to a third more matrix-core
  // instructions, in 384-row query blocks that fill the chip's rounds
  // differently from 256-row ones.
  //
  // Head dim 256 (CS): the two waves of a pair hold the same 32 rows. Wave
  // `half` computes the full scores (all 256 channels) of key tile kt = half
  // of each sub-tile and their probabilities, and the output of its channel
  // half (DW = 128) from all 32 keys: it writes its 16 keys' probabilities to
  // LDS and reads the partner's 16 before its PV. So each wave holds the Q
  // of every channel but only half of the accumulators, issues as many
  // matrix-core instructions and fragment reads per step as at head dim 128,
  // and computes half of the exponentials. The pair runs in one phase of the
  // ping-pong, so the barriers that separate the phases also order the
  // exchange: probabilities are written in Y and read at the start of the
  // next X.
  //
  // Schedule (ping-pong): the two waves of a SIMD alternate an X phase
  // (matrix-core work only: QK^T of sub-tile u+1 and PV of sub-tile u, the
  // wave reading its own fragments four ahead in fenced groups) and a Y
  // phase (softmax of u+1, the first fragment reads of the next X, one ring
  // refill), separated by workgroup barriers, so one wave feeds the matrix
  // core while the other computes the softmax.
  constexpr bool CS = G::kCS;
  constexpr int DW = G::DW;          // channels of this wave
  constexpr int NC = DW / 32;        // 32-channel chunks of this wave's output channels
  constexpr int NCQ = CS ? D / 32 : NC;   // 32-channel chunks of its QK^T
  constexpr int NKF = CS ? NCQ : 2 * NC;  // K fragments per sub-tile (CS: one key tile)
  constexpr int NT16 = DW / 16;      // 16-channel output tiles
  const int l16 = lane & 15, g4 = lane >> 4;
  constexpr int QT = G::QT;          // 16-row query tiles per wave
  int rowq[QT], limq[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    rowq[qt] = q0 + pair * G::WROWS + qt * 16 + l16;
    limq[qt] = a.causal ? min(rowq[qt], kvv_t - 1) : kvv_t - 1;
  }
  auto xmap = [&](int v) __attribute__((always_inline)) {
    if constexpr (WIN) return v < wn1 ? v : v + ws2;
    else return v;
  };
  int x_mask = min(a.causal ? q0 / kSub : 0x7fffffff, (kvv_t % kSub) ? kvv_t / kSub : 0x7fffffff);
  int c_row[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) c_row[qt] = -1;
  if constexpr (WIN) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int f = rowq[qt] / a.win_F;
      c_row[qt] = f < a.win_A ? -1 : (f - a.win_A) / a.win_C;
    }
    x_mask = !win_fast ? 0 : ((kvv_t % kSub) && xmap(xe - 1) == kvv_t / kSub ? xe - 1 : 0x7fffffff);
  }

  // Q fragments (B operand of S^T = K Q^T): query row 16 qt + l%16 of the
  // wave, channels 32 cc + 8 g4 .. +7. Loaded before the ring fill.
  bf16x8_t qf[QT][NCQ];
  {
    const uint16_t* qp = a.qw + ((int64_t)bh * a.Sq_pad + q0 + pair * G::WROWS + l16) * D + g4 * 8;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int cc = 0; cc < NCQ; ++cc) qf[qt][cc] = *reinterpret_cast<const bf16x8_t*>(qp + qt * 16 * D + cc * 32);
  }

  // Direct loads: the ring keeps all K sub-tiles in its first kRing kKBytes
  // and all V^T sub-tiles after them (slot s: K at s * kKBytes, V^T at kRing
  // * kKBytes + s * kKBytes), so every fragment offset fits the instruction's
  // 16-bit field from one base register per operand. Load i of this wave
  // fills LDS bytes [1024 j, 1024 j + 1024) of the slot's K (j < nK) or V^T
  // (j - nK), j = wave + NW i; the lane that fills LDS chunk Q fetches the
  // logical chunk the swizzle puts there.
  const uint16_t* kw = a.kw + (int64_t)bh_kv * a.Sk_pad * D;
  const uint16_t* vt = a.vt + (int64_t)bh_kv * a.Sk_pad * D;
  int loff[LDPS];
#pragma unroll
  for (int i = 0; i < LDPS; ++i) {
    const int j = wave + NW * i;
    if (j < G::nK) {
      const int Q = j * 64 + lane;
      const int r = Q / (D / 8), p = Q % (D / 8);
      loff[i] = (r * D + ((p ^ (r & G::kSwz)) * 8)) * 2;
    } else {
      const int Q = (j - G::nK) * 64 + lane;
      const int d = Q >> 2, p = Q & 3;
      loff[i] = (d * kSub + ((p ^ vt_swz(d)) * 8)) * 2;
    }
  }
  // Head dims 64 and 128 build one buffer resource per operand for the
  // segment (the head's prepared K or V^T, Sk_pad keys; the host keeps that
  // below 2 GB) and give a load's sub-tile as its scalar offset; a load past
  // the segment's last sub-tile re-reads sub-tile 0 into a slot that is never
  // read, so every access stays inside the head's rows. Head dim 256 builds a
  // resource per sub-tile instead (an empty one past the end): its loop has
  // no scalar registers to spare for two resources held across the segment,
  // and the spills cost more than the per-load set-up.
  const int kv_bytes = a.Sk_pad * D * 2;
  // Loads of sub-tile x into its slot: i in [i0, i1) of this wave's LDPS
  // loads (the first LDPS / 2 fill K, the others V^T, as j = wave + NW i).
  auto issue_part = [&](int x, int i0, int i1) __attribute__((always_inline)) {
    const int sl = (x - xb) & (kRing - 1);
    const bool live = x < xe;
    const int xs = live ? xmap(x) : 0;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int j = wave + NW * i;
      uint8_t* dst = j < G::nK ? lds + sl * kKBytes + j * 1024 : lds + (kRing + sl) * kKBytes + (j - G::nK) * 1024;
      if constexpr (G::kCS) {
        const uint16_t* src = (j < G::nK ? kw : vt) + (int64_t)xs * (kSub * D);
        load_lds16(src, live ? kKBytes : 0, loff[i], dst);
      } else {
        load_lds16_soff(j < G::nK ? kw : vt, kv_bytes, loff[i], xs * kKBytes, dst);
      }
    }
  };
  static_assert(G::nK == NW * LDPS / 2, "half of each wave's loads fill K");
  auto issue_loads = [&](int x) __attribute__((always_inline)) { issue_part(x, 0, LDPS); };
  auto issue_k = [&](int x) __attribute__((always_inline)) { issue_part(x, 0, LDPS / 2); };
  auto issue_v = [&](int x) __attribute__((always_inline)) { issue_part(x, LDPS / 2, LDPS); };
  // Ring refills. Sub-tile x is first read in the Y phase of step x - 2 (K)
  // and x - 1 (V^T); its slot's K part is free once every wave has done
  // step x - kRing - 1's X phase, its V^T part one step later.
  // Head dims 64 and 128 (eight slots): step u refills the slot of u - 1
  // with u - 1 + kRing and each Y phase ends waiting for the loads of u + 3.
  // Head dim 256 (four slots) refills K a step ahead of V^T: in step u the
  // waves of role 0 load K(u + 4) and V^T(u + 3) and, at the end of each X
  // phase, wait for the loads of two steps before; the waves of role 1, which
  // run a phase later, load K(u + 5) and V^T(u + 4) and wait at the end of
  // each Y phase for the loads of two steps before. Either way every wave's
  // share of a sub-tile has landed at the barrier before its first read, and
  // each load has two to three phases to land.
  const bool early = CS && role;
  auto fill_ring = [&]() __attribute__((always_inline)) {
    if constexpr (CS) {
      // Role 0: K and V^T of xb .. xb + 2, K of xb + 3; role 1: K and V^T of
      // xb .. xb + 3 (its K of xb + 4 follows once the prologue has read K of
      // xb).
#pragma unroll
      for (int i = 0; i < kRing - 1; ++i) issue_loads(xb + i);
      if (early) issue_loads(xb + kRing - 1);
      else issue_k(xb + kRing - 1);
    } else {
#pragma unroll
      for (int i = 0; i < kRing - 1; ++i) issue_loads(xb + i);
    }
  };
  fill_ring();

  // Accumulator tiles (qt, ct) live as 4-register slices of 16-register
  // tuples (tile i = qt NT16 + ct in tuple i/4, slice i%4): with the tiles as
  // separate 4-register values the register allocator writes most results to
  // fresh registers instead of in place and doubles them.
  constexpr int NA = QT * NT16 / 4;
  f32x16_t accq[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) accq[i][r] = 0.f;
  auto acc_mfma = [&](int qt, int ct, bf16x8_t va_, bf16x8_t vb_) __attribute__((always_inline)) {
    const int i = qt * NT16 + ct;
    f32x16_t& t = accq[i >> 2];
    const int o = (i & 3) * 4;
    f32x4_t c = {t[o], t[o + 1], t[o + 2], t[o + 3]};
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va_, vb_, c, 0, 0, 0);
    t[o] = c[0]; t[o + 1] = c[1]; t[o + 2] = c[2]; t[o + 3] = c[3];
  };
  auto acc_get = [&](int qt, int ct) __attribute__((always_inline)) -> f32x4_t {
    const int i = qt * NT16 + ct;
    const int o = (i & 3) * 4;
    return f32x4_t{accq[i >> 2][o], accq[i >> 2][o + 1], accq[i >> 2][o + 2], accq[i >> 2][o + 3]};
  };
  float m_run[QT];      // row offsets (exp2 units), shared by the row's four lanes
  float l_run[QT];      // this lane's share of each row sum
  bool seen[QT];        // the row has met a visible key
  f32x4_t msplat[QT];   // -m_run: the QK^T accumulators' initial value
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = l_run[qt] = 0.f;
    seen[qt] = true;
    msplat[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

  // Pair exchange areas (CS): row values (maxima, sums) that wave (pair, h)
  // reads at xs(pair, h) (its partner writes them there), probabilities that
  // wave (pair, h) writes at xp(pair, h); per lane QT floats and 8 bf16.
  uint8_t* const xs_out = lds + G::kXOff + (pair * 2 + (1 - half)) * 512 + lane * 8;
  const uint8_t* const xs_in = lds + G::kXOff + (pair * 2 + half) * 512 + lane * 8;
  uint8_t* const xp_out = lds + G::kXOff + G::kXScores + (pair * 2 + half) * 1024 + lane * 16;
  const uint8_t* const xp_in = lds + G::kXOff + G::kXScores + (pair * 2 + (1 - half)) * 1024 + lane * 16;
  // Barrier with this wave's LDS writes complete (the pair's exchanges at
  // points where every wave of the workgroup is in step).
  auto pair_sync = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // Sets this lane's scores of key tile kt of query tile qt in sub-tile x
  // that its row does not see to -inf.
  auto mask_kt = [&](f32x4_t& sk, int x, int qt, int kt) __attribute__((always_inline)) {
    int a_end = 0x7fffffff, w_lo = 0, w_hi = 0;
    if constexpr (WIN) {
      if (c_row[qt] >= 0) {
        a_end = a.win_A * a.win_F;
        w_lo = (a.win_A + a.win_C * max(c_row[qt] - a.win_R, 0)) * a.win_F;
        w_hi = (a.win_A + a.win_C * min(c_row[qt] + a.win_R + 1, win_cap)) * a.win_F;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = x * kSub + kt * 16 + g4 * 4 + r;
      if constexpr (WIN) {
        // Bitwise, not short-circuit, so it compiles to compares and one
        // select instead of branches.
        const bool hidden = (key > limq[qt]) | ((key >= a_end) & ((key < w_lo) | (key >= w_hi)));
        sk[r] = hidden ? -INFINITY : sk[r];
      } else {
        if (key > limq[qt]) sk[r] = -INFINITY;
      }
    }
  };
  auto mask16 = [&](f32x4_t* sq, int x, int qt) __attribute__((always_inline)) {
    mask_kt(sq[0], x, qt, 0);
    mask_kt(sq[1], x, qt, 1);
  };
  // This lane's maximum of the 8 scores of query tile qt in sub-tile x; with
  // MASK, keys its row does not see are set to -inf first.
  auto rowmax16 = [&](f32x4_t* sq, int x, int qt, auto mask) __attribute__((always_inline)) {
    if constexpr (decltype(mask)::value) mask16(sq, x, qt);
    return fmaxf(max3(max3(sq[0][0], sq[0][1], sq[0][2]), sq[0][3], sq[1][0]), max3(sq[1][1], sq[1][2], sq[1][3]));
  };
  // Maximum / sum over the four lanes of a row (l, l^16, l^32, l^48).
  auto max_row16 = [](float x) __attribute__((always_inline)) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto sw = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return max_lane_pair(fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1])));
  };
  auto sum_row16 = [](float x) __attribute__((always_inline)) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto sw = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return sum_lane_pair(__builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]));
  };
  // A priori score bound. After H3's RMSNorm (weight w) a row y of 128
  // channels has |y| <= sqrt(128) max|w| (r^2 sum x^2 = 128 ms / (ms + eps));
  // the rotary embedding keeps |y|, q carries the factor c = scale log2(e)
  // and the bf16 rounding grows a norm by at most 2^-8, so by Cauchy-Schwarz
  // every score (exp2 units) lies in [-M, M] with
  //   M = c * 128 * max|w_q| * max|w_k| * (1 + 2^-6)
  // (2^-6 covers the roundings and the fp32 sums with room to spare). When
  // M <= kBoundMax the fixed offset m = M serves every row: p = exp2(s - M)
  // lies in [2^-2M, 1], finite and normal in fp32 and bf16, so the running
  // maximum, its wave-wide check and the rescale drop out of every step and
  // o = O / l is unchanged (softmax does not depend on the offset; bf16
  // rounding of p is relative). Otherwise (unnormalised inputs, large
  // weights) the online maximum runs as before.
  // Without the norm, the bound comes from the data: row i's scores lie in
  // [-m_i, m_i] with m_i = |q_i| max_j |k_j| (Cauchy-Schwarz on the bf16
  // rows the matrix core reads; q carries c already), each row taking its own
  // m_i as its offset when every row of the wave has m_i <= kBoundMax (at
  // head dim 256 both waves of a pair hold every channel of their rows, so
  // they take the same offsets).
  bool bounded = false;
  if (a.wq != nullptr) {
    auto wmax = [&](const float* w) __attribute__((always_inline)) {
      return wave_max(fmaxf(fabsf(w[lane]), fabsf(w[lane + 64])));
    };
    const float M = a.c_log2 * 128.0f * wmax(a.wq) * wmax(a.wk) * (1.0f + 1.0f / 64.0f);
    const float Mu = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, M)));
    bounded = Mu <= kBoundMax;
    if (bounded) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        m_run[qt] = Mu;
        msplat[qt] = f32x4_t{-Mu, -Mu, -Mu, -Mu};
      }
    }
  } else if (a.knorm != nullptr) {
    const float kmax = key_norm_max(a, bh_kv);
    float ss[QT], m[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      ss[qt] = 0.f;
#pragma unroll
      for (int cc = 0; cc < NCQ; ++cc) ss[qt] = sum_sq(qf[qt][cc], ss[qt]);
      ss[qt] = sum_row16(ss[qt]);
    }
    bool over = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      m[qt] = sqrtf(ss[qt]) * kmax * kBoundSlack;
      over = over | !(m[qt] <= kBoundMax);
    }
    bounded = __builtin_amdgcn_ballot_w64(over) == 0;
    if constexpr (CS) {
      // Without the bound the pairs run an extra pass with barriers of its
      // own, so the whole workgroup takes one decision: bounded only if
      // every wave is. (The SIMD-id slots are free after the kernel start;
      // the next segment writes them after a barrier.)
      int* flag = reinterpret_cast<int*>(lds + G::kSimdOff);
      if (lane == 0) flag[wave] = bounded ? 1 : 0;
      pair_sync();
      int all = 1;
#pragma unroll
      for (int w = 0; w < NW; ++w) all &= flag[w];
      bounded = __builtin_amdgcn_readfirstlane(all) != 0;
    }
    if (bounded) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        m_run[qt] = m[qt];
        msplat[qt] = f32x4_t{-m[qt], -m[qt], -m[qt], -m[qt]};
      }
    }
  }

  using NoMask = std::integral_constant<bool, false>;
  using Mask = std::integral_constant<bool, true>;
  // Scores arrive as s - m_run. If some row of the wave exceeds its offset by
  // more than 2^kRescaleLog2 (rare), raise the offsets by the rows' excess,
  // shift the scores and rescale the accumulators and partial sums; with
  // MASK, a row that saw no key before takes its first keys' maximum.
  auto maybe_rescale16 = [&](f32x4_t (&s)[QT][2], const float* mx, auto mask) __attribute__((always_inline)) {
    bool trigger = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      trigger = trigger | (mx[qt] > kRescaleLog2);
      if constexpr (WIN && decltype(mask)::value) trigger = trigger | (!seen[qt] & (mx[qt] != -INFINITY));
    }
    if (__builtin_amdgcn_ballot_w64(trigger) != 0) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        float delta = max_row16(mx[qt]);
        float alpha;
        if constexpr (WIN && decltype(mask)::value) {
          const bool fresh = !seen[qt] && delta != -INFINITY;
          seen[qt] = seen[qt] || fresh;
          delta = fresh ? delta : fmaxf(delta, 0.f);
          alpha = fresh ? 1.f : __builtin_amdgcn_exp2f(-delta);
        } else {
          delta = fmaxf(delta, 0.f);
          alpha = __builtin_amdgcn_exp2f(-delta);
        }
        m_run[qt] += delta;
        l_run[qt] *= alpha;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[qt][0][r] -= delta;
          s[qt][1][r] -= delta;
          msplat[qt][r] -= delta;
        }
#pragma unroll
        for (int ct = 0; ct < NT16; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) accq[(qt * NT16 + ct) >> 2][((qt * NT16 + ct) & 3) * 4 + r] *= alpha;
      }
    }
  };
  // bf16 probabilities p = exp2(s) as the PV operand of each query tile
  // (element j: key 16 (j/4) + 4 g4 + j%4), and this lane's share of the sums.
  auto probs16 = [&](const f32x4_t (&s)[QT][2], bf16x8_t* pf) __attribute__((always_inline)) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[qt][j] = (__bf16)__builtin_amdgcn_exp2f(s[qt][j >> 2][j & 3]);
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const bf16x2_t pp = {pf[qt][j], pf[qt][j + 1]};
        l_run[qt] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run[qt], false);
      }
    }
  };

  // Fragment reads. K fragment (kt, cc): key row 16 kt + l%16 (CS: kt =
  // half), chunk 4 cc + g4, stored at (4 cc + g4) ^ s = (g4 ^ s) ^ 4 cc (s =
  // l%16 & kSwz), so one address register per cc; V^T fragment ct: channel
  // row half DW + 16 ct + l%16, chunk g4. The V^T base (kRing K sub-tiles
  // in) is hidden from the compiler so that it stays in the register and out
  // of the offset field.
  bf16x8_t pf[QT];
  const uint32_t kb16 = (l16 + (CS ? 16 * half : 0)) * (2 * D) + ((g4 ^ (l16 & G::kSwz)) * 16);
  uint32_t ka[NCQ];
#pragma unroll
  for (int cc = 0; cc < NCQ; ++cc) ka[cc] = kb16 ^ (64u * cc);
  uint32_t va = kRing * kKBytes + half * (DW * 64) + l16 * 64 + ((g4 ^ vt_swz(l16)) * 16);
  asm("" : "+v"(va));
  // Fragment g of a step: g < NKF is K fragment (kt, cc) = (g % 2, g / 2)
  // (CS: (half, g)) of the sub-tile in slot_k, the others V^T fragment ct =
  // g - NKF of the one in slot_v. Each feeds QT matrix-core instructions.
  auto frag = [&](int g, auto slot_k, auto slot_v) __attribute__((always_inline)) -> bf16x8_t {
    int sk, sv;
    if constexpr (std::is_integral_v<decltype(slot_k)>) sk = slot_k;
    else sk = decltype(slot_k)::value;
    if constexpr (std::is_integral_v<decltype(slot_v)>) sv = slot_v;
    else sv = decltype(slot_v)::value;
    if (g < NKF) {
      if constexpr (CS) return *reinterpret_cast<const bf16x8_t*>(lds + sk * kKBytes + ka[g]);
      else return *reinterpret_cast<const bf16x8_t*>(lds + sk * kKBytes + (g & 1) * (16 * 2 * D) + ka[g >> 1]);
    }
    return *reinterpret_cast<const bf16x8_t*>(lds + sv * kKBytes + (g - NKF) * 1024 + va);
  };
  constexpr int NG = NKF + NT16;   // fragments per step
  auto rslot = [&](int x) { return (x - xb) & (kRing - 1); };
  // One X phase: QK^T into s (K fragments of slot_k) and, with PV, PV into
  // acc (V^T fragments of slot_v, probabilities pf), in fenced groups of the
  // instructions that use fragment g and the read of fragment g + 4; fr holds
  // the first four fragments, read by the caller.
  bf16x8_t fr[4];
  auto xphase = [&](f32x4_t (&s)[QT][2], auto slot_k, auto slot_v, auto pv, auto hf) __attribute__((always_inline)) {
    constexpr bool PV = decltype(pv)::value;
    constexpr int H = decltype(hf)::value;
    constexpr int NGX = PV ? NG : NKF;
    bf16x8_t gf[NG];
#pragma unroll
    for (int g = 0; g < 4; ++g) gf[g] = fr[g];
    for_each_index(std::make_integer_sequence<int, NGX>{}, [&](auto gc) __attribute__((always_inline)) {
      constexpr int g = decltype(gc)::value;
      if constexpr (g + 4 < NGX) gf[g + 4] = frag(g + 4, slot_k, slot_v);
      if constexpr (g < NKF) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          if constexpr (CS) s[qt][H] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gf[g], qf[qt][g], s[qt][H], 0, 0, 0);
          else s[qt][g & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gf[g], qf[qt][g >> 1], s[qt][g & 1], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) acc_mfma(qt, g - NKF, gf[g], pf[qt]);
      }
      fence();
    });
  };

  // Probabilities of key tile H (elements 4H .. 4H + 3 of each query tile's
  // PV operand) and this lane's share of the sums; written for the partner.
  auto probs_own = [&](const f32x4_t (&s)[QT][2], auto hf) __attribute__((always_inline)) {
    constexpr int H = decltype(hf)::value;
    uint32_t w[QT * 2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) pf[qt][4 * H + j] = (__bf16)__builtin_amdgcn_exp2f(s[qt][H][j]);
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const bf16x2_t pp = {pf[qt][4 * H + j], pf[qt][4 * H + j + 1]};
        l_run[qt] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run[qt], false);
        w[qt * 2 + j / 2] = __builtin_bit_cast(uint32_t, pp);
      }
    }
    static_assert(!CS || QT == 2, "one 16-byte exchange per lane");
    *reinterpret_cast<u32x4_t*>(xp_out) = u32x4_t{w[0], w[1], w[2], w[3]};
  };
  // The partner's probabilities (key tile 1 - H) into the PV operands.
  auto probs_in = [&](auto hf) __attribute__((always_inline)) {
    constexpr int H = decltype(hf)::value;
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(xp_in);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      u32x4_t p = __builtin_bit_cast(u32x4_t, pf[qt]);
      p[2 * (1 - H)] = w[2 * qt];
      p[2 * (1 - H) + 1] = w[2 * qt + 1];
      pf[qt] = __builtin_bit_cast(bf16x8_t, p);
    }
  };
  // Largest score of key tile H per lane (the max pass).
  auto max_own = [&](const f32x4_t (&s)[QT][2], float* mx, auto hf) __attribute__((always_inline)) {
    constexpr int H = decltype(hf)::value;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) mx[qt] = fmaxf(mx[qt], fmaxf(max3(s[qt][H][0], s[qt][H][1], s[qt][H][2]), s[qt][H][3]));
  };

  // The rest of the tile. MODE 0: the online maximum with lazy rescale;
  // MODE 1: the fixed offsets msplat (a bound, or the exact row maxima), no
  // row maximum, wave-wide check or rescale in the steps; MODE 2 (CS only):
  // the max pass, QK^T only, each row's largest visible score into mxp.
  // hf: this wave's channel half (CS; 0 otherwise).
  float mxp[QT];
  auto run_tile = [&](auto mode, auto hf, auto rf) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode)::value;
    constexpr int H = decltype(hf)::value;
    // Role as a constant (CS: the pair's waits and refills depend on it, and
    // branches on it would split the unrolled steps into many blocks).
    constexpr int RF = decltype(rf)::value;
    const bool role1 = CS ? RF == 1 : role != 0;
    constexpr bool ONLINE = MODE == 0, MAXP = MODE == 2;
    static_assert(!(CS && ONLINE) && (CS || !MAXP), "modes");
    // QK^T accumulators start from -m: scores arrive relative to the row
    // offset.
    auto s_init = [&](int qt) __attribute__((always_inline)) -> f32x4_t {
      if constexpr (ONLINE) return f32x4_t{0.f, 0.f, 0.f, 0.f};
      else return msplat[qt];
    };
    // Prologue: scores of xb set each row's offset to its exact maximum
    // (online path), or start from the fixed offset.
    // Wait for K and V^T of xb and xb + 1 (and, in role 1, K of xb + 2).
    if constexpr (CS) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * LDPS / 2) : "memory");
    else asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kRing - 4) * LDPS) : "memory");
    __syncthreads();
    f32x4_t s[QT][2];
    {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) s[qt][kt] = s_init(qt);
#pragma unroll
      for (int g = 0; g < NKF; ++g) {
        const bf16x8_t kfr = frag(g, 0, 0);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          if constexpr (CS) s[qt][H] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr, qf[qt][g], s[qt][H], 0, 0, 0);
          else s[qt][g & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfr, qf[qt][g >> 1], s[qt][g & 1], 0, 0, 0);
        }
      }
      if constexpr (CS) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) mask_kt(s[qt][H], xmap(xb), qt, H);
        if constexpr (MAXP) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) mxp[qt] = -INFINITY;
          max_own(s, mxp, hf);
        } else {
          probs_own(s, hf);
        }
        pair_sync();
        if constexpr (RF == 1) issue_k(xb + kRing);   // every wave has read K of xb
        if constexpr (!MAXP) probs_in(hf);
      } else {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          if constexpr (!ONLINE) {
            mask16(s[qt], xmap(xb), qt);
          } else {
            m_run[qt] = max_row16(rowmax16(s[qt], xmap(xb), qt, Mask{}));
            if constexpr (WIN) {
              seen[qt] = m_run[qt] != -INFINITY;
              if (!seen[qt]) m_run[qt] = 0.f;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              s[qt][0][r] -= m_run[qt];
              s[qt][1][r] -= m_run[qt];
              msplat[qt][r] = -m_run[qt];
            }
          }
        }
        probs16(s, pf);
      }
    }
    // The first fragments of the first X phase: K(xb+1), V(xb).
#pragma unroll
    for (int g = 0; g < 4; ++g) fr[g] = frag(g, rslot(min(xb + 1, xe - 1)), 0);

    // Step u: X = QK^T of u+1 and PV of u; Y = fragment reads of K(u+2) and
    // V(u+1), a ring refill, the softmax of u+1.
    // slot_vc, slot_kc: V(u) and K(u+1), read by this X phase; slot_vn,
    // slot_kn: V(u+1) and K(u+2), whose first fragments the Y phase reads.
    auto step = [&](int u, auto mask_next, auto slot_vn, auto slot_kn, auto slot_vc, auto slot_kc) __attribute__((always_inline)) {
      fence();
      if constexpr (CS && !MAXP) probs_in(hf);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) s[qt][kt] = CS ? s_init(qt) : msplat[qt];
      xphase(s, slot_kc, slot_vc, std::integral_constant<bool, !MAXP>{}, hf);
      if constexpr (CS && RF == 0) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(LDPS) : "memory");
      else bar();
      fence();
      if constexpr (CS) {
        // The probabilities go out first, then the next X phase's first
        // fragment reads: LDS operations complete in order, so waiting until
        // at most those four reads are outstanding publishes the write at
        // the barrier while the reads stay in flight.
        if constexpr (decltype(mask_next)::value) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) mask_kt(s[qt][H], xmap(u + 1), qt, H);
        }
        if constexpr (MAXP) max_own(s, mxp, hf);
        else probs_own(s, hf);
        fence();
#pragma unroll
        for (int g = 0; g < 4; ++g) fr[g] = frag(g, slot_kn, slot_vn);
        if constexpr (RF == 1) {
          issue_k(u + kRing + 1);
          issue_v(u + kRing);
        } else {
          issue_k(u + kRing);
          issue_v(u + kRing - 1);
        }
        fence();
        if constexpr (RF == 1) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(4)\n\ts_barrier" ::"n"(2 * LDPS) : "memory");
        else asm volatile("s_waitcnt lgkmcnt(4)\n\ts_barrier" ::: "memory");
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) fr[g] = frag(g, slot_kn, slot_vn);
        issue_loads(u - 1 + kRing);
        if constexpr (!ONLINE) {
          if constexpr (decltype(mask_next)::value) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) mask16(s[qt], xmap(u + 1), qt);
          }
        } else {
          float mx[QT];
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) mx[qt] = rowmax16(s[qt], xmap(u + 1), qt, mask_next);
          maybe_rescale16(s, mx, mask_next);
        }
        probs16(s, pf);
        fence();
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((kRing - 4) * LDPS) : "memory");
      }
      fence();
    };

    if (role1) bar();
    int u = xb;
    for (; u + kRing <= min(xe - 2, x_mask - 1); u += kRing) {
      for_each_index(std::make_integer_sequence<int, kRing>{}, [&](auto k) __attribute__((always_inline)) {
        constexpr int K = decltype(k)::value;
        step(u + K, NoMask{}, std::integral_constant<int, (K + 1) % kRing>{},
             std::integral_constant<int, (K + 2) % kRing>{}, std::integral_constant<int, K % kRing>{},
             std::integral_constant<int, (K + 1) % kRing>{});
      });
    }
    for (; u < xe - 1; ++u) step(u, Mask{}, rslot(u + 1), rslot(min(u + 2, xe - 1)), rslot(u), rslot(u + 1));
    // Last X phase: PV of the last sub-tile only.
    if constexpr (!MAXP) {
      if constexpr (CS) probs_in(hf);
      const int vs = rslot(xe - 1);
#pragma unroll
      for (int ct = 0; ct < NT16; ++ct) {
        const bf16x8_t vfr = frag(2 * NC + ct, 0, vs);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) acc_mfma(qt, ct, vfr, pf[qt]);
      }
    }
    if (!role1) bar();
    // The ring holds refills that nobody reads; let them retire so no LDS
    // write is pending when the workgroup ends or the ring restarts.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  if constexpr (CS) {
    // Without a usable bound, a max pass over the keys finds each row's
    // largest score first (the pair's two key tiles combined), and the
    // second pass runs with those exact maxima as fixed offsets.
    auto both = [&](auto hf, auto rf) __attribute__((always_inline)) {
      if (!bounded) {
        run_tile(std::integral_constant<int, 2>{}, hf, rf);
        float mr[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) mr[qt] = max_row16(mxp[qt]);
        __syncthreads();
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) reinterpret_cast<float*>(xs_out)[qt] = mr[qt];
        pair_sync();
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          float m = fmaxf(mr[qt], reinterpret_cast<const float*>(xs_in)[qt]);
          m = m == -INFINITY ? 0.f : m;   // a row that sees no key: l = 0, written as 0
          m_run[qt] = m;
          msplat[qt] = f32x4_t{-m, -m, -m, -m};
        }
        pair_sync();
        fill_ring();
      }
      run_tile(std::integral_constant<int, 1>{}, hf, rf);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    if (role) {
      if (half) both(I1{}, I1{});
      else both(I0{}, I1{});
    } else {
      if (half) both(I1{}, I0{});
      else both(I0{}, I0{});
    }
    // Each lane's row-sum share over both key tiles: add the partner's.
    __syncthreads();
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) reinterpret_cast<float*>(xs_out)[qt] = l_run[qt];
    pair_sync();
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) l_run[qt] += reinterpret_cast<const float*>(xs_in)[qt];
  } else {
    using I0 = std::integral_constant<int, 0>;
    if (bounded) run_tile(std::integral_constant<int, 1>{}, I0{}, I0{});
    else run_tile(std::integral_constant<int, 0>{}, I0{}, I0{});
  }

  if (rec < 0) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float l = sum_row16(l_run[qt]);
      f32x4_t at[NT16];
#pragma unroll
      for (int ct = 0; ct < NT16; ++ct) at[ct] = acc_get(qt, ct);
      store_row16<D, NT16>(a, obase + half * DW, rowq[qt], g4, at, (!WIN || l > 0.f) ? 1.0f / l : 0.f, qv_seg,
                           gate_row);
    }
  } else {
    float* pr = a.part + (int64_t)rec * G::kRecFloats + lwave * 64 + lane;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int ct = 0; ct < NT16; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[((qt * NT16 + ct) * 4 + r) * T] = accq[(qt * NT16 + ct) >> 2][((qt * NT16 + ct) & 3) * 4 + r];
      pr[(G::kRecA + qt) * T] = m_run[qt];
      pr[(G::kRecA + QT + qt) * T] = l_run[qt];
    }
  }
  if (si + 1 < nseg) __syncthreads();   // the next segment refills the LDS ring
  }
}

// Short key ranges at head dim 128 (cross-attention against a few hundred
// text keys): when the valid keys of a (b, kv head) fill at most kResMaxSub
// sub-tiles, their K and V^T (8 KB each per sub-tile, 160 KB at 10) stay
// resident in LDS. A workgroup of eight waves then owns one (b, h) and one
// residue class of its query tiles (tiles gi, gi + G, ...): it loads the keys
// once, and each tile costs only its Q fragments (loaded a tile ahead, into
// registers) and its output, instead of a launch, a ring fill and a drain.
// The arithmetic is the main kernel's on 16x16x32 instructions: per
// sub-tile, QK^T from the Q fragments and the K fragments in LDS, p =
// exp2(s - m) rounded to bf16, PV into fp32 accumulators; o = O / l. With
// the a priori bound (norm weights, or the key-norm maxima) m is the row's
// fixed bound; otherwise a first pass over the resident keys finds each
// row's exact maximum (two QK^T passes, no rescale). The LDS layouts are
// the ring slots' (K rows and V^T rows swizzled as there), filled by plain
// loads and stores.
constexpr int kResMaxSub = 10;
constexpr int kResRows = 256;   // query rows per tile: eight waves of two 16-row tiles

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_resident_kernel(AttnArgs a, int32_t G) {
  constexpr int D = 128;
  using Gm = Geo<D, 2>;
  constexpr int BM = kResRows, T = Gm::NW * 64, NC = D / 32, NT16 = D / 16;
  constexpr int kKB = Gm::kKBytes;                 // one K or V^T sub-tile (8 KB)
  constexpr int kVBase = kResMaxSub * kKB;         // V^T region
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kResMaxSub * kKB];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
  const int bh = blockIdx.x / G, gi = blockIdx.x - bh * G;
  const int b = bh / a.H, h = bh - b * a.H;
  const int bh_kv = b * a.Hkv + h / (a.H / a.Hkv);
  const int kvv = a.kv_valid, NU = (kvv + kSub - 1) / kSub;
  const int nq = (a.Sq + BM - 1) / BM, nqv = (a.q_valid + BM - 1) / BM;
  // The batch item's output rows; the host keeps Sq * H * D * 2 below 2^31.
  const __amdgpu_buffer_rsrc_t orsrc =
      __builtin_amdgcn_make_buffer_rsrc(a.o + (int64_t)b * a.Sq * a.H * D, 0, (int)((int64_t)a.Sq * a.H * D * 2),
                                        kBufferRsrcWord3);
  const uint16_t* gate_row = a.gate ? a.gate + (int64_t)b * a.Sq * a.H + h : nullptr;

  // Resident keys: LDS byte P of sub-tile x (K at x kKB, V^T at kVBase + x
  // kKB) holds the 16 bytes that the ring's direct loads would put there:
  // chunk Q = P / 16 comes from sub-tile byte offset loff(Q) below.
  {
    const uint16_t* kw = a.kw + (int64_t)bh_kv * a.Sk_pad * D;
    const uint16_t* vt = a.vt + (int64_t)bh_kv * a.Sk_pad * D;
    constexpr int CH = kKB / 16;                   // 512 chunks per sub-tile and operand
    constexpr int kFill = 2 * kResMaxSub * CH / T; // chunks per thread (all loads issued before any store)
    u32x4_t tmp[kFill];
    int dst[kFill];
#pragma unroll
    for (int k = 0; k < kFill; ++k) {
      const int i = tid + k * T;
      const int x = i / (2 * CH), rem = i - x * 2 * CH;
      const bool is_v = rem >= CH;
      const int Q = is_v ? rem - CH : rem;
      int off;
      if (!is_v) {
        const int r = Q / (D / 8), pp = Q % (D / 8);
        off = (r * D + ((pp ^ (r & Gm::kSwz)) * 8)) * 2;
      } else {
        const int d = Q >> 2, pp = Q & 3;
        off = (d * kSub + ((pp ^ vt_swz(d)) * 8)) * 2;
      }
      dst[k] = (is_v ? kVBase : 0) + x * kKB + Q * 16;
      if (x < NU)
        tmp[k] = *reinterpret_cast<const u32x4_t*>(
            reinterpret_cast<const uint8_t*>((is_v ? vt : kw) + (int64_t)x * (kSub * D)) + off);
    }
#pragma unroll
    for (int k = 0; k < kFill; ++k)
      if ((tid + k * T) / (2 * CH) < NU) *reinterpret_cast<u32x4_t*>(lds + dst[k]) = tmp[k];
  }

  // Fragment addresses as in the main kernel's 16x16x32 path.
  const uint32_t kb16 = l16 * (2 * D) + ((g4 ^ (l16 & Gm::kSwz)) * 16);
  const uint32_t va = kVBase + l16 * 64 + ((g4 ^ vt_swz(l16)) * 16);
  auto kfrag = [&](int x, int g) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8_t*>(lds + x * kKB + (g & 1) * (16 * 2 * D) + (kb16 ^ (64u * (g >> 1))));
  };
  auto vfrag = [&](int x, int ct) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8_t*>(lds + x * kKB + ct * 1024 + va);
  };
  // Q fragments of tile t: query row 16 qt + l%16 of the wave, channels
  // 32 cc + 8 g4 .. +7 (rows past the workspace's valid rows are zero).
  bf16x8_t qn[2][NC];
  auto load_q = [&](int t) __attribute__((always_inline)) {
    const uint16_t* qp = a.qw + ((int64_t)bh * a.Sq_pad + t * BM + wave * 32 + l16) * D + g4 * 8;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) qn[qt][cc] = *reinterpret_cast<const bf16x8_t*>(qp + qt * 16 * D + cc * 32);
  };
  int t = gi;
  if (t < nqv) load_q(t);
  __syncthreads();

  // A priori bound with H3's norm weights (uniform), else per row from the
  // key-norm maxima and the Q fragments; INFINITY when neither applies.
  float w_bound = INFINITY, kmax = INFINITY;
  if (a.wq != nullptr) {
    w_bound = a.c_log2 * 128.0f * wave_max(fmaxf(fabsf(a.wq[lane]), fabsf(a.wq[lane + 64]))) *
              wave_max(fmaxf(fabsf(a.wk[lane]), fabsf(a.wk[lane + 64]))) * (1.0f + 1.0f / 64.0f);
  } else if (a.knorm != nullptr) {
    kmax = key_norm_max(a, bh_kv);
  }
  auto sum_row16 = [](float x) __attribute__((always_inline)) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto sw = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return sum_lane_pair(__builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]));
  };
  auto max_row16 = [](float x) __attribute__((always_inline)) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto sw = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return max_lane_pair(fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1])));
  };
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  for (; t < nq; t += G) {
    if (t >= nqv) {
      // Query tile wholly past q_valid: zeros.
      constexpr int CPR = D / 8;
      for (int idx = tid; idx < BM * CPR; idx += T) {
        const int q = t * BM + idx / CPR;
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{0u, 0u, 0u, 0u}, orsrc,
                                               (uint32_t)(((q * a.H + h) * D + (idx % CPR) * 8) * 2), 0, 0);
      }
      continue;
    }
    bf16x8_t qf[2][NC];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) qf[qt][cc] = qn[qt][cc];
    // The next tile's Q (this tile's again when there is none, from L2): the
    // load is issued on every path, so the wait for it at the next tile
    // counts only this tile's stores after it.
    load_q(t + G < nqv ? t + G : t);
    // Gate values of this wave's two rows (rows past q_valid read the last
    // valid row's and are written as zeros), loaded with the Q prefetch and
    // first used at the stores.
    uint32_t graw[2] = {0u, 0u};
    if (gate_row) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        graw[qt] = gate_row[(int64_t)min(t * BM + wave * 32 + qt * 16 + l16, a.q_valid - 1) * a.H];
    }

    // QK^T of sub-tile x into s (initial value sinit); keys at or past kvv set to -inf.
    auto scores = [&](int x, const f32x4_t* sinit, f32x4_t (&s)[2][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        s[qt][0] = sinit[qt];
        s[qt][1] = sinit[qt];
      }
#pragma unroll
      for (int g = 0; g < 2 * NC; ++g) {
        const bf16x8_t kf = kfrag(x, g);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          s[qt][g & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qt][g >> 1], s[qt][g & 1], 0, 0, 0);
      }
      if (x == NU - 1 && (kvv % kSub) != 0) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (x * kSub + kt * 16 + g4 * 4 + r >= kvv) s[qt][kt][r] = -INFINITY;
      }
    };

    // Row offsets: the bound when it is known and at most kBoundMax for every
    // row of the wave, else the exact row maxima from a first pass.
    float m[2];
    bool have = false;
    if (a.wq != nullptr) {
      m[0] = m[1] = w_bound;
      have = __builtin_amdgcn_readfirstlane(w_bound <= kBoundMax ? 1 : 0) != 0;
    } else if (a.knorm != nullptr) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float ss = 0.f;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) ss = sum_sq(qf[qt][cc], ss);
        m[qt] = sqrtf(sum_row16(ss)) * kmax * kBoundSlack;
      }
      have = __builtin_amdgcn_ballot_w64(!(m[0] <= kBoundMax) | !(m[1] <= kBoundMax)) == 0;
    }
    if (!have) {
      const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
      const f32x4_t z[2] = {zero4, zero4};
      float mx[2] = {-INFINITY, -INFINITY};
      for (int x = 0; x < NU; ++x) {
        f32x4_t s[2][2];
        scores(x, z, s);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          mx[qt] = fmaxf(mx[qt], fmaxf(max3(max3(s[qt][0][0], s[qt][0][1], s[qt][0][2]), s[qt][0][3], s[qt][1][0]),
                                       max3(s[qt][1][1], s[qt][1][2], s[qt][1][3])));
      }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) m[qt] = max_row16(mx[qt]);
    }
    const f32x4_t msplat[2] = {f32x4_t{-m[0], -m[0], -m[0], -m[0]}, f32x4_t{-m[1], -m[1], -m[1], -m[1]}};

    f32x4_t acc[2][NT16];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int ct = 0; ct < NT16; ++ct) acc[qt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float l_run[2] = {0.f, 0.f};
    // Pipeline over the resident sub-tiles, one scheduling region per phase:
    // step x reads x's eight V^T fragments first (the exponentials that
    // follow hide their latency), computes x's probabilities, reads the K
    // fragments of x + 1 (PV hides their latency), runs PV of x and then
    // QK^T of x + 1, whose scores the next step's exponentials take.
    bf16x8_t kf[2 * NC];
    auto read_k = [&](int x) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < 2 * NC; ++g) kf[g] = kfrag(x, g);
    };
    auto qk = [&](f32x4_t (&s)[2][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        s[qt][0] = msplat[qt];
        s[qt][1] = msplat[qt];
      }
#pragma unroll
      for (int g = 0; g < 2 * NC; ++g)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          s[qt][g & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[g], qf[qt][g >> 1], s[qt][g & 1], 0, 0, 0);
    };
    f32x4_t s[2][2];
    bf16x8_t vf[NT16];
    read_k(0);
#pragma unroll
    for (int ct = 0; ct < NT16; ++ct) vf[ct] = vfrag(0, ct);
    qk(s);
    for (int x = 0; x < NU; ++x) {
      if (x == NU - 1 && (kvv % kSub) != 0) {
        const int lim = kvv - x * kSub - g4 * 4;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kt * 16 + r >= lim) {
              s[0][kt][r] = -INFINITY;
              s[1][kt][r] = -INFINITY;
            }
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8_t pf[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[qt][j] = (__bf16)__builtin_amdgcn_exp2f(s[qt][j >> 2][j & 3]);
      __builtin_amdgcn_sched_barrier(0);
      if (x + 1 < NU) read_k(x + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ct = 0; ct < NT16; ++ct)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) acc[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[ct], pf[qt], acc[qt][ct], 0, 0, 0);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const bf16x2_t pp = {pf[qt][j], pf[qt][j + 1]};
          l_run[qt] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run[qt], false);
        }
      __builtin_amdgcn_sched_barrier(0);
      if (x + 1 < NU) {
#pragma unroll
        for (int ct = 0; ct < NT16; ++ct) vf[ct] = vfrag(x + 1, ct);
        qk(s);
      }
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float inv = 1.0f / sum_row16(l_run[qt]);
      if (gate_row) inv *= 1.0f / (1.0f + __expf(-__uint_as_float(graw[qt] << 16)));
      store_row16_rsrc<D, NT16>(a, orsrc, (uint32_t)(h * D * 2), t * BM + wave * 32 + qt * 16 + l16, g4, acc[qt], inv,
                                a.q_valid);
    }
  }
}

// Merge of a split tile t (tile n_whole + t): the blocks whose step ranges
// meet the tile each left one partial record (O_i, m_i, l_i) with O_i and l_i
// relative to their own offset m_i; with M = max m_i the tile's result is
// sum 2^(m_i - M) O_i / sum 2^(m_i - M) l_i (scores are in exp2 units).
template <int D, int QT_>
__global__ __launch_bounds__(64) void attn_merge_kernel(AttnArgs a) {
  // One workgroup per (split tile, logical wave): a single wave merges the
  // rows (and at head dim 256 the channel half) that logical wave lw of the
  // split blocks held, so the grid has NW workgroups per split tile.
  using G = Geo<D, QT_>;
  constexpr int BM = G::BM;
  constexpr int T = G::NW * 64;
  constexpr int QT = G::QT;
  constexpr int NT16 = G::DW / 16;   // 16-channel output tiles per thread
  constexpr int NR = G::kRecA + 2 * QT;   // floats per thread in a record
  const int lane = threadIdx.x;
  const int t = blockIdx.x / G::NW;
  const int lw = blockIdx.x - t * G::NW;   // logical wave: its rows (and channel half at 256)
  const int tid = lw * 64 + lane;          // its thread index within a record
  const int pair = G::kCS ? lw >> 1 : lw, half = G::kCS ? lw & 1 : 0;
  const int NU = (a.kv_valid + kSub - 1) / kSub;
  const int tg = a.n_whole + t;
  const int bh = tg / a.nqv;
  const int q0 = (tg - bh * a.nqv) * BM;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  uint16_t* obase = a.o + ((int64_t)b * a.Sq * a.H + h) * D + half * G::DW;

  // The blocks j0 .. j1 that touch tile t, and block j's record for it.
  int j0, j1;
  merge_blocks(t, a.n_split, NU, a.n_split_blocks, j0, j1);
  auto record = [&](int j) {
    return a.part + (int64_t)merge_record(j, t, a.n_split, NU, a.n_split_blocks) * G::kRecFloats + tid;
  };
  const uint16_t* gate_row = a.gate ? a.gate + (int64_t)b * a.Sq * a.H + h : nullptr;
  // Records in the 16x16 layout: QT query tiles x NT16 tiles x 4 registers,
  // then the QT rows' offsets and the QT partial sums. Each record is read
  // whole into registers (all loads in flight together, coalesced across
  // the wave), then folded into the running result.
  f32x4_t acc[QT][NT16];
  float M[QT], l[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    M[qt] = -INFINITY;
    l[qt] = 0.f;
    for (int j = j0; j <= j1; ++j) M[qt] = fmaxf(M[qt], record(j)[(G::kRecA + qt) * T]);
#pragma unroll
    for (int ct = 0; ct < NT16; ++ct) acc[qt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int j = j0; j <= j1; ++j) {
    const float* pr = record(j);
    float v[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) v[r] = __builtin_nontemporal_load(pr + r * T);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float w = __builtin_amdgcn_exp2f(v[G::kRecA + qt] - M[qt]);
      l[qt] += w * v[G::kRecA + QT + qt];
#pragma unroll
      for (int ct = 0; ct < NT16; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[qt][ct][r] += w * v[(qt * NT16 + ct) * 4 + r];
    }
  }
  const int l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const uint32_t u = __builtin_bit_cast(uint32_t, l[qt]);
    const auto sw = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float lr = sum_lane_pair(__builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]));
    store_row16<D, NT16>(a, obase, q0 + pair * G::WROWS + qt * 16 + l16, g4, acc[qt], 1.0f / lr, a.q_valid, gate_row);
  }
}

// Key held at position p (< 32) of a V^T sub-tile: position 8g + j holds
// key 16 (j/4) + 4g + j%4, the keys whose probabilities lane group g of the
// 16x16x32 PV operand supplies.
template <int D>
__device__ inline int key_of_position(int p) {
  return ((p & 4) << 2) | ((p & 0x18) >> 1) | (p & 3);
}

// Transposed, key-blocked copy of v for the PV operand: a block moves 64 keys
// (two sub-tiles) x D channels of one (b, h) through LDS, reading 2D-byte
// rows of v and writing one contiguous block of 128 D bytes of vt. Keys at or
// past kv_valid are written as zeros and never read.
template <int D>
__global__ __launch_bounds__(256) void v_relayout_kernel(const uint16_t* __restrict__ v, int64_t sb,
                                                         int64_t ss, int64_t sh,
                                                         uint16_t* __restrict__ vt, int32_t H,
                                                         int32_t Sk, int32_t kv_valid,
                                                         const int32_t* __restrict__ lengths,
                                                         int32_t Sk_pad) {
  constexpr int kPitch = D + 8;   // row pitch in elements: 16 bytes of padding
  constexpr int CPR = D / 8;      // 16-byte chunks per row of v
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kPitch];
  const int p0 = blockIdx.x * 64;
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x;
  const int32_t valid = item_valid(lengths, b, 1, kv_valid, Sk);
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const int idx = tid + 256 * i;
    const int key = idx / CPR, ch = idx % CPR;
    u32x4_t val = u32x4_t{0u, 0u, 0u, 0u};
    if (p0 + key < valid)
      val = *reinterpret_cast<const u32x4_t*>(v + (int64_t)b * sb + (int64_t)(p0 + key) * ss + (int64_t)h * sh + ch * 8);
    *reinterpret_cast<u32x4_t*>(&tile[key * kPitch + ch * 8]) = val;
  }
  __syncthreads();
  // Output chunk idx covers sub-tile xs = idx/(4D), channel d, positions 8pc..8pc+7.
  uint16_t* out = vt + ((int64_t)bh * Sk_pad + p0) * D;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const int idx = tid + 256 * i;
    const int xs = idx / (4 * D), d = (idx >> 2) % D, pc = idx & 3;
    uint32_t packed[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int pa = pc * 8 + e, pb = pa + 1;
      const int ka = xs * kSub + key_of_position<D>(pa);
      const int kb = xs * kSub + key_of_position<D>(pb);
      packed[e / 2] = (uint32_t)tile[ka * kPitch + d] | ((uint32_t)tile[kb * kPitch + d] << 16);
    }
    *reinterpret_cast<u32x4_t*>(out + idx * 8) = u32x4_t{packed[0], packed[1], packed[2], packed[3]};
  }
}

}  // namespace

namespace {

// Compute units of the current device (cached per device; 0 if unknown).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace

namespace {

// Frame window: whether handing the query blocks out longest first (as the
// kernel ranks them) shortens a greedy schedule of the tiles, one per CU at
// a time in rank order, by more than 1% against increasing order. Tiles in
// the increasing order share their windows' keys in L2 more, so the ranked
// order pays only where the tile lengths leave the last round uneven. With
// per-item lengths (on the device) the tile lengths are unknown here:
// increasing order. The decision for the last geometry is kept.
bool win_longest_first(const AttnArgs& a, int BM, int64_t nq, int cus) {
  const int64_t nbh = (int64_t)a.B * a.H;
  if (a.lengths != nullptr || cus <= 0 || nq > kWinOrderMax || nq * nbh > (1 << 16)) return false;
  static std::mutex mu;
  static int64_t last_key[12] = {-1};
  static bool last = false;
  const int64_t key[12] = {a.B, a.H, a.Sq, a.Sk, a.q_valid, a.kv_valid, a.win_F, a.win_C, a.win_R, a.win_A, BM, cus};
  std::lock_guard<std::mutex> lock(mu);
  if (std::equal(key, key + 12, last_key)) return last;
  std::vector<int64_t> len(nq);
  for (int64_t j = 0; j < nq; ++j)
    len[j] = j * BM >= a.q_valid ? 0 : win_span(a.win_F, a.win_C, a.win_R, a.win_A, BM, (int)(j * BM), a.q_valid, a.kv_valid).xe;
  auto makespan = [&](const std::vector<int>& order) {
    std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
    for (int c = 0; c < cus; ++c) free_at.push(0);
    int64_t end = 0;
    for (const int j : order)
      for (int64_t h = 0; h < nbh; ++h) {
        const int64_t t = free_at.top() + len[j] + 1;
        free_at.pop();
        free_at.push(t);
        end = std::max(end, t);
      }
    return end;
  };
  std::vector<int> plain(nq);
  std::iota(plain.begin(), plain.end(), 0);
  std::vector<int> ranked = plain;
  std::stable_sort(ranked.begin(), ranked.end(), [&](int x, int y) { return len[x] > len[y]; });
  last = makespan(ranked) * 100 < makespan(plain) * 99;
  std::copy(key, key + 12, last_key);
  return last;
}

// The launch at QT query tiles per wave, on the schedule plan_attention
// made: general mode, or the uniform schedule of whole rounds and a split
// last round.
template <int D, int QT>
hipError_t launch_attention_q(AttnArgs a, const AttnPlan& p, hipStream_t stream) {
  using G = Geo<D, QT>;
  constexpr int NW = G::NW;
  static_assert(kAttnSub == kSub, "tiling constants");
  if (p.rows != G::BM || p.grid > 0x7fffffffLL || p.nqv > 0x7fffffffLL) return hipErrorInvalidValue;
  a.nqv = (int32_t)p.nqv;
  a.n_whole = (int32_t)p.n_whole;
  a.n_split = (int32_t)p.n_split;
  a.n_split_blocks = (int32_t)p.n_blocks;
  if (a.general) {
    a.win_longest_first = a.win_F > 0 && win_longest_first(a, G::BM, p.nqv, device_cus()) ? 1 : 0;
    if (p.grid > 0) {
      if (a.win_F > 0)
        attn_fwd_kernel<D, QT, true><<<dim3((unsigned)p.grid), NW * 64, 0, stream>>>(a);
      else
        attn_fwd_kernel<D, QT, false><<<dim3((unsigned)p.grid), NW * 64, 0, stream>>>(a);
    }
    return hipGetLastError();
  }
  if (p.grid > 0) attn_fwd_kernel<D, QT, false><<<dim3((unsigned)p.grid), NW * 64, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 0) return e;
  attn_merge_kernel<D, QT><<<dim3((unsigned)(p.n_split * NW)), 64, 0, stream>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_attention_d(const AttnArgs& a, const AttnPlan& p, hipStream_t stream) {
  if constexpr (D == 128) {
    if (p.resident) {
      if (p.grid > 0x7fffffffLL) return hipErrorInvalidValue;
      attn_resident_kernel<<<dim3((unsigned)p.grid), Geo<D, 2>::NW * 64, 0, stream>>>(a, (int32_t)(p.grid / ((int64_t)a.B * a.H)));
      return hipGetLastError();
    }
  }
  constexpr int lo = attn_qt_min(D), hi = attn_qt_max(D);
  if (p.query_tiles == hi) return launch_attention_q<D, hi>(a, p, stream);
  if constexpr (lo != hi) {
    if (p.query_tiles == lo) return launch_attention_q<D, lo>(a, p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

AttnPlan plan_attention(const AttnArgs& a, int cus) {
  AttnPlan p{};
  const bool general = a.causal || a.lengths != nullptr || a.win_F > 0;
  const int64_t NU = (a.kv_valid + kSub - 1) / kSub;
  const int64_t bh = (int64_t)a.B * a.H;
  if (a.D == 128 && !general && NU <= kResMaxSub && (int64_t)a.Sq * a.H * 128 * 2 < (1ll << 31)) {
    // Keys resident in LDS: one workgroup per (b, h) and residue class of its
    // query tiles, G classes per head so that the grid covers the CUs.
    const int64_t nq = (a.Sq + kResRows - 1) / kResRows;
    const int64_t G = std::max<int64_t>(1, std::min<int64_t>(nq, (std::max(cus, 1) + bh - 1) / bh));
    p.resident = 1;
    p.query_tiles = 2;
    p.rows = kResRows;
    p.nqv = (a.q_valid + kResRows - 1) / kResRows;
    p.tiles = bh * p.nqv;
    p.grid = bh * G;
    return p;
  }
  p.query_tiles = a.query_tiles != 0 ? a.query_tiles
                                     : choose_query_tiles(a.D, general, bh, general ? a.Sq : a.q_valid, NU, cus,
                                                          a.part_slots);
  p.rows = attn_rows(a.D, p.query_tiles);
  const int64_t nq = (a.Sq + p.rows - 1) / p.rows;
  if (general) {
    // One block per (b, h, query block); each finds its own valid rows and
    // key range, so nothing is split.
    p.nqv = nq;
    p.tiles = bh * nq;
    p.grid = p.tiles;
    return p;
  }
  // One tile per CU at a time: the last round holds n_valid % cus tiles. When
  // that round is partial, split its tiles' steps over more blocks (at most
  // one per CU, each at least kSplitMinSteps steps, and more blocks than
  // tiles so no block spans more than two tiles). Tiles wholly past q_valid
  // only write zeros.
  p.nqv = (a.q_valid + p.rows - 1) / p.rows;
  p.tiles = bh * p.nqv;
  const SplitPlan sp = split_plan(p.tiles, NU, cus, a.part_slots);
  p.n_whole = sp.n_whole;
  p.n_split = sp.n_split;
  p.n_blocks = sp.n_blocks;
  p.grid = sp.n_whole + sp.n_blocks + bh * (nq - p.nqv);
  return p;
}

hipError_t launch_attention(AttnArgs a, hipStream_t stream) {
  a.general = (a.causal || a.lengths != nullptr || a.win_F > 0) ? 1 : 0;
  const AttnPlan p = plan_attention(a, device_cus());
  switch (a.D) {
    case 64: return launch_attention_d<64>(a, p, stream);
    case 128: return launch_attention_d<128>(a, p, stream);
    case 256: return launch_attention_d<256>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_v_relayout(const uint16_t* v, int64_t sb, int64_t ss, int64_t sh, uint16_t* vt,
                             int32_t B, int32_t Sk, int32_t H, int32_t kv_valid,
                             const int32_t* lengths, int32_t Sk_pad, int32_t D, hipStream_t stream) {
  const dim3 grid((unsigned)(Sk_pad / 64), (unsigned)(B * H));
  switch (D) {
    case 64: v_relayout_kernel<64><<<grid, 256, 0, stream>>>(v, sb, ss, sh, vt, H, Sk, kv_valid, lengths, Sk_pad); break;
    case 128: v_relayout_kernel<128><<<grid, 256, 0, stream>>>(v, sb, ss, sh, vt, H, Sk, kv_valid, lengths, Sk_pad); break;
    case 256: v_relayout_kernel<256><<<grid, 256, 0, stream>>>(v, sb, ss, sh, vt, H, Sk, kv_valid, lengths, Sk_pad); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace h3
