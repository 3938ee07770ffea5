// Internal launch interface between the C-ABI layer (h3attn_api.cpp) and the
// gfx950 kernels. Arguments reaching these functions are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_sched.h"

namespace h3 {

constexpr int kHeadDim = 128;
constexpr int kRopePairs = 48;      // rotate-half pairs (j, j+48), j < 48
constexpr int kRowPad = 256;        // workspace rows are padded to this multiple

// Exact unsigned division by a runtime divisor d >= 1 for dividends below
// 2^31: q = (n * m) >> p with p = 31 + ceil(log2 d), m = ceil(2^p / d).
// (m <= 2^32 + 1, so n * m fits in 64 bits; the error term m*d - 2^p < d
// keeps floor exact for every n < 2^31.)
struct FastDiv {
  uint64_t m;
  uint32_t p, d;
  static FastDiv make(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    FastDiv f;
    f.d = d;
    f.p = 31 + l;
    f.m = (uint64_t)(((((unsigned __int128)1) << f.p) + d - 1) / d);
    return f;
  }
  __device__ __host__ uint32_t div(uint32_t n) const { return (uint32_t)(((uint64_t)n * m) >> p); }
};

// Valid length of batch item b from an optional device array of per-item
// lengths (q at [2b], kv at [2b+1]), clamped to [0, limit]; `uniform` when
// there is no array. Clamping keeps every access in bounds whatever the
// array holds.
__device__ inline int32_t item_valid(const int32_t* lengths, int b, int which, int32_t uniform,
                                     int32_t limit) {
  if (lengths == nullptr) return uniform;
  const int32_t v = lengths[2 * b + which];
  return v < 0 ? 0 : (v > limit ? limit : v);
}

// One tensor handled by the prologue kernel. Strides are in elements and
// describe a [B, S, H, D] view (channel stride 1); the norm and rotary
// prologue takes D = 128, the copy of the other head dims 64 and 256.
struct ProTensor {
  const uint16_t* in;
  uint16_t* out;
  const float* w;          // RMSNorm weight [128] or nullptr (no norm; always for the copy)
  int64_t in_sb, in_ss, in_sh;
  int64_t out_sb, out_ss, out_sh;
  int32_t S_valid;         // rows s < S_valid are read and transformed
  int32_t S_out;           // rows S_valid <= s < S_out are written as zeros
  float out_scale;         // outputs are multiplied by this in fp32 before the bf16 rounding
  const int32_t* lengths;  // optional per-item lengths (device); item b then uses
  int32_t which;           //   item_valid(lengths, b, which, S_valid, S_valid) as its S_valid
  int32_t H;               // heads of this tensor
  FastDiv div_h, div_s;    // set by launch_qk_prologue: division by the larger H and by S_out
};

// h3attn_forward_stages with every argument validated first (the C-ABI
// entry points share it): returns an h3attn status code.
int forward_dense(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, int32_t B, int32_t Sq,
                  int32_t Sk, int32_t H, int32_t head_dim, const float* q_norm_w, const float* k_norm_w, float eps,
                  const float* rope_cos, const float* rope_sin, int32_t rope_rows, int32_t q_valid, int32_t kv_valid,
                  float softmax_scale, void* workspace, size_t workspace_bytes, uint32_t stages, void* stream);

// Validates h3attn_forward's arguments other than the workspace, without
// the device gate; on success sets the workspace bytes the call needs.
int check_dense_args(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, int32_t B, int32_t Sq,
                     int32_t Sk, int32_t H, int32_t head_dim, const float* q_norm_w, const float* k_norm_w,
                     float eps, const float* rope_cos, const float* rope_sin, int32_t rope_rows, int32_t q_valid,
                     int32_t kv_valid, float softmax_scale, size_t* workspace_bytes);

// H3ATTN_OK when the current device is gfx950, else the h3attn status the
// entry points return (UNSUPPORTED_DEVICE, or HIP when the query fails).
int check_gfx950();

// Enqueues the fused RMSNorm + partial-rotary prologue over up to two tensors
// (t1 may have S_out == 0; the two may have different head counts).
// rope_cos/rope_sin == nullptr disables rotary.
hipError_t launch_qk_prologue(const ProTensor& t0, const ProTensor& t1, int32_t B,
                              float eps, const float* rope_cos, const float* rope_sin,
                              hipStream_t stream);

// Writes the transposed, key-blocked copy of v ([B, Sk, H, D] with element
// strides sb, ss, sh) that the attention kernel reads (layout in
// attn_fwd.hip); keys at or past the valid length (kv_valid, or the item's
// entry of `lengths` when given) are written as zeros and never read.
hipError_t launch_v_relayout(const uint16_t* v, int64_t sb, int64_t ss, int64_t sh, uint16_t* vt,
                             int32_t B, int32_t Sk, int32_t H, int32_t kv_valid,
                             const int32_t* lengths, int32_t Sk_pad, int32_t D, hipStream_t stream);

// The largest norm of the prepared key rows kw [BH][Sk_pad][D] in each chunk
// of kKnChunk rows: kn[bh * kn_chunks + chunk] (rows past the valid length
// are zero in kw and do not count).
hipError_t launch_key_norms(const uint16_t* kw, float* kn, int32_t BH, int32_t Sk_pad, int32_t kn_chunks, int32_t D,
                            hipStream_t stream);

// The prepare stage for head dims other than 128 (no norm, no rotary): copies
// t0 and t1 ([B, S, H, D] views) into the head-major workspace, multiplying
// by out_scale in fp32 before the bf16 rounding and zero-filling rows at or
// past the valid length. The ProTensor strides are in elements.
hipError_t launch_qk_copy(const ProTensor& t0, const ProTensor& t1, int32_t B, int32_t D,
                          hipStream_t stream);

hipError_t launch_rope_tables(float* cos_out, float* sin_out, int32_t rows, double theta,
                              hipStream_t stream);

// The prologue fused with the destination-major Ulysses pack of one rank's
// sequence shard (dense [B, S, H, 128] q, k, v in; three [P][B][S][H/P][128]
// send buffers out; rotary position row_offset + s; w_q == nullptr: no norm,
// rope_cos == nullptr: no rotary).
struct QkvPack {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* q_send;
  uint16_t* k_send;
  uint16_t* v_send;
  const float* w_q;
  const float* w_k;
  float eps;
  const float* rope_cos;
  const float* rope_sin;
  int32_t B, S, H, P, row_offset;
};
hipError_t launch_qkv_pack(const QkvPack& t, hipStream_t stream);

struct AttnArgs {
  int32_t D;               // head dim: 64, 128 or 256
  const uint16_t* qw;      // [B*H][Sq_pad][D] scaled by softmax_scale*log2(e), rows >= q_valid zero
  const uint16_t* kw;      // [B*Hkv][Sk_pad][D], rows >= kv_valid are zero
  const uint16_t* vt;      // [B*Hkv][Sk_pad/32][D][32], see attn_fwd.hip; keys >= kv_valid zero
  uint16_t* o;             // [B][Sq][H][D]
  float* part;             // partial records for split tiles
  int64_t part_slots;      // records available at part
  int32_t B, H, Sq, Sk, Sq_pad, Sk_pad, q_valid, kv_valid;
  int32_t Hkv;             // key/value heads; query head h reads kv head h / (H / Hkv)
  int32_t causal;          // key j visible to query row i only if j <= i
  const int32_t* lengths;  // optional per-item valid lengths (device), see item_valid()
  // Frame window (win_F > 0): row or key i is in frame i / win_F; frames
  // below win_A are anchors whose queries see every key; frame f >= win_A is
  // in chunk (f - win_A) / win_C, and its queries see the anchor frames and
  // the chunks within win_R of their own.
  int32_t win_F, win_C, win_R, win_A;
  const uint16_t* gate;    // optional [B][Sq][H] bf16: o *= sigmoid(gate)
  // H3's Q/K RMSNorm weights ([128] fp32 each, or nullptr when q and k were
  // not normalised) and the factor c = softmax_scale * log2(e) the prologue
  // multiplied q by: with them every score (in exp2 units) is bounded by
  // c * 128 * max|w_q| * max|w_k| (see attn_fwd.hip).
  const float* wq;
  const float* wk;
  float c_log2;
  // Without the norm (wq == nullptr): the largest prepared key norm of each
  // chunk of kKnChunk keys, [B*Hkv][kn_chunks] fp32 (key_norm_kernel), from
  // which the kernel bounds each row's scores by |q_i| max_j |k_j|.
  const float* knorm;
  int32_t kn_chunks;
  // Query tiles per wave (2 or 3 at head dim 128, the only count elsewhere),
  // or 0: the launcher chooses (choose_query_tiles in attn_sched.h).
  int32_t query_tiles;
  // Schedule, filled in by launch_attention. Uniform mode (no causal mask,
  // no per-item lengths): valid tiles (query block below q_valid) are
  // numbered g = (b*H + h) * nqv + query block; tiles g < n_whole run whole,
  // the n_split tiles after them are split over n_split_blocks workgroups;
  // tiles past q_valid only write zeros. General mode (causal mask,
  // per-item lengths or frame window): one workgroup per (b, h, query
  // block), each finding its own key ranges.
  int32_t general;
  int32_t nqv, n_whole, n_split, n_split_blocks;
  // Frame window: 1 when workgroups take the query blocks longest first
  // (set by the launcher when that shortens the schedule), else 0.
  int32_t win_longest_first;
};

// The schedule of one attention launch on a device with `cus` compute units
// (host arithmetic only): which kernel, its query tiles per wave and rows
// per tile, the valid query blocks per (b, h), the tiles with work, the
// uniform schedule's whole tiles, split tiles and split blocks, and the grid.
struct AttnPlan {
  int32_t resident;      // 1: keys resident in LDS (attn_resident_kernel)
  int32_t query_tiles;
  int32_t rows;
  int64_t nqv, tiles, n_whole, n_split, n_blocks, grid;
};
AttnPlan plan_attention(const AttnArgs& a, int cus);

// Enqueues the attention kernel (and, when the schedule splits tiles, the
// merge of their partial records) on `stream`.
hipError_t launch_attention(AttnArgs a, hipStream_t stream);

// RMSNorm + indexed scale/shift (scale_shift.hip). x and y [rows = B*S, D]
// bf16, scale and shift [B, M, D] bf16, index [B*S] int32 or null (row 0),
// w fp32 [D] or null. D is a multiple of 8 and at most kScaleShiftMaxD.
constexpr int kScaleShiftMaxD = 16384;
struct ScaleShiftArgs {
  const uint16_t* x;
  uint16_t* y;
  const uint16_t* scale;
  const uint16_t* shift;
  const int32_t* index;
  const float* w;
  float eps;
  int32_t rows, S, D, M;
};
hipError_t launch_scale_shift(const ScaleShiftArgs& a, hipStream_t stream);

}  // namespace h3
