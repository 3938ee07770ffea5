// Internal launch interface between the C-ABI layer (h3attn_api.cpp) and the
// gfx950 kernels. Arguments reaching these functions are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// One tensor handled by the prologue kernel. Strides are in elements and
// describe a [B, S, H, 128] view (channel stride 1).
struct ProTensor {
  const uint16_t* in;
  uint16_t* out;
  const float* w;          // RMSNorm weight [128] or nullptr (no norm)
  int64_t in_sb, in_ss, in_sh;
  int64_t out_sb, out_ss, out_sh;
  int32_t S_valid;         // rows s < S_valid are read and transformed
  int32_t S_out;           // rows S_valid <= s < S_out are written as zeros
  float out_scale;         // outputs are multiplied by this in fp32 before the bf16 rounding
  FastDiv div_h, div_s;    // set by launch_qk_prologue: division by H and by S_out
};

// Enqueues the fused RMSNorm + partial-rotary prologue over up to two tensors
// (t1 may have S_out == 0). rope_cos/rope_sin == nullptr disables rotary.
hipError_t launch_qk_prologue(const ProTensor& t0, const ProTensor& t1, int32_t B, int32_t H,
                              float eps, const float* rope_cos, const float* rope_sin,
                              hipStream_t stream);

// Writes the transposed, key-blocked copy of v that the attention kernel
// reads (layout in attn_fwd.hip); keys >= kv_valid are written as zeros.
hipError_t launch_v_relayout(const uint16_t* v, uint16_t* vt, int32_t B, int32_t Sk, int32_t H,
                             int32_t kv_valid, int32_t Sk_pad, hipStream_t stream);

hipError_t launch_rope_tables(float* cos_out, float* sin_out, int32_t rows, double theta,
                              hipStream_t stream);

// Attention tiling: a workgroup of kAttnWaves waves (32 query rows each) owns
// kAttnRows query rows of one (b, h) and walks the keys in kAttnSub-key
// sub-tiles.
constexpr int kAttnWaves = 8;
constexpr int kAttnRows = kAttnWaves * 32;
constexpr int kAttnSub = 32;

// Load balancing of the last, partial round of query tiles (stream-K): those
// tiles' sub-tile steps are split evenly over up to kSplitMaxBlocks
// workgroups, each taking at least kSplitMinSteps steps and touching at most
// two tiles; each writes one partial record per tile it touches and a second
// kernel merges them. A record holds the un-normalised fp32 accumulator (64
// values per lane) plus the lane's running max and partial row sum.
constexpr int kSplitMaxBlocks = 256;
constexpr int kSplitMinSteps = 16;
constexpr int kPartFloats = (64 + 2) * kAttnWaves * 64;
constexpr size_t kPartBytes = sizeof(float) * kPartFloats;

// Partial records the forward workspace reserves for these sizes: two per
// split workgroup, for the largest split the launcher can choose.
inline int64_t split_part_slots(int32_t B, int32_t Sq, int32_t Sk, int32_t H) {
  const int64_t tiles = (int64_t)B * H * ((Sq + kAttnRows - 1) / kAttnRows);
  const int64_t steps = tiles * ((Sk + kAttnSub - 1) / kAttnSub);
  const int64_t blocks = steps / kSplitMinSteps < kSplitMaxBlocks ? steps / kSplitMinSteps : kSplitMaxBlocks;
  return 2 * blocks;
}

struct AttnArgs {
  const uint16_t* qw;      // [B*H][Sq_pad][128] scaled by softmax_scale*log2(e), rows >= q_valid zero
  const uint16_t* kw;      // [B*H][Sk_pad][128], rows >= kv_valid are zero
  const uint16_t* vt;      // [B*H][Sk_pad/32][128][32], see attn_fwd.hip; keys >= kv_valid zero
  uint16_t* o;             // [B][Sq][H][128]
  float* part;             // partial records for split tiles
  int64_t part_slots;      // records available at part
  int32_t B, H, Sq, Sq_pad, Sk_pad, q_valid, kv_valid;
  // Schedule, filled in by launch_attention: valid tiles (query block below
  // q_valid) are numbered g = (b*H + h) * nqv + query block; tiles g < n_whole
  // run whole, the n_split tiles after them are split over n_split_blocks
  // workgroups; tiles past q_valid only write zeros.
  int32_t nqv, n_whole, n_split, n_split_blocks;
};

// Enqueues the attention kernel (and, when the schedule splits tiles, the
// merge of their partial records) on `stream`.
hipError_t launch_attention(AttnArgs a, hipStream_t stream);

}  // namespace h3
