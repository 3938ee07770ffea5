/*
 * h3attn: the MiniMax-H3 video-DiT attention step on AMD Instinct MI355X (gfx950).
 *
 * The step (FastVideo PR #1832 "Add FlashInfer attention backend support for
 * MiniMax H3", sections "Summary" and "Preserve H3-specific attention
 * behavior"; TeleFuser PR #37, section 2.2): per-head RMSNorm of q and k, a
 * rotary embedding on 96 of the 128 head channels, then dense non-causal
 * scaled-dot-product attention over BSHD tensors at head_dim 128 in bf16,
 * with an optional valid front / padded tail (TeleFuser PR #37, sections 2.3
 * and 2.4; FastVideo PR #1799, section "Implementation", padding masks).
 * Beside it, the DiT block's RMSNorm with indexed AdaLN scale/shift that
 * feeds the QKV projection (TeleFuser PR #37, section 2.5).
 *
 * Conventions shared by every entry point
 *  - bf16 tensors are passed as uint16_t bit patterns. Every pointer is a
 *    caller-owned device pointer unless stated otherwise. q, k, v and o are
 *    dense, contiguous [B, S, H, 128] (BSHD, channel fastest).
 *  - Every device pointer must be 16-byte aligned.
 *  - The library allocates no device memory at run time and keeps no caller
 *    pointer after a call returns (h3attn_forward_noalloc's workspace is a
 *    static array of the loaded library). Work is enqueued asynchronously on
 *    `stream` (a hipStream_t passed as void*; NULL is the null stream).
 *  - All arguments are validated before anything is enqueued: when a call
 *    returns an error, nothing has run and no output was touched.
 *  - Device faults, like any asynchronous HIP error, surface at the caller's
 *    next synchronisation, not as a return value.
 *  - The library runs on gfx950 only. On any other device the call returns
 *    H3ATTN_ERR_UNSUPPORTED_DEVICE; there is no fallback path.
 *  - There is no backward pass: the step is inference-only (FastVideo PR
 *    #1799, section "Failure behavior").
 */
#ifndef H3ATTN_H_
#define H3ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum h3attn_status {
  H3ATTN_OK = 0,
  H3ATTN_ERR_NULL_POINTER = 1,      /* a required pointer is NULL, or only one of a pair is given */
  H3ATTN_ERR_BAD_SHAPE = 2,         /* a size is out of range (head_dim, S < 1, valid lengths, table rows) */
  H3ATTN_ERR_BAD_ALIGNMENT = 3,     /* a pointer is not 16-byte aligned */
  H3ATTN_ERR_ALIASING = 4,          /* an output overlaps an input (other than an exact in-place prologue) */
  H3ATTN_ERR_BAD_VALUE = 5,         /* eps, theta or softmax_scale not finite / out of range */
  H3ATTN_ERR_WORKSPACE = 6,         /* workspace missing or smaller than h3attn_forward_workspace_bytes() */
  H3ATTN_ERR_UNSUPPORTED_DEVICE = 7,/* the current device is not gfx950, or there is no device */
  H3ATTN_ERR_HIP = 8                /* a HIP runtime call or a kernel launch failed */
};

#define H3ATTN_HEAD_DIM 128
#define H3ATTN_ROPE_DIM 96     /* channels 0..95 are rotated as 48 rotate-half pairs (j, j+48) */
#define H3ATTN_ROPE_PAIRS 48

/* A static, NUL-terminated description of a status code. Never NULL. */
const char* h3attn_status_string(int status);

/*
 * Rotary tables for the 96/128 partial rotary embedding (FastVideo PR #1832,
 * "Preserve H3-specific attention behavior").
 *
 * Writes cos_out[p*48 + j] = cos(phi) and sin_out[p*48 + j] = sin(phi) with
 * phi = p * theta^(-2j/96), for rows p = 0 .. rows-1 and pairs j = 0..47.
 * Angles, cosines and sines are evaluated in fp64 on the device and rounded
 * once to fp32.
 *   cos_out, sin_out: device fp32 [rows, 48], disjoint, 16-byte aligned.
 *   rows >= 1; theta finite and > 1.
 * Errors: NULL_POINTER, BAD_SHAPE (rows < 1), BAD_VALUE (theta), ALIGNMENT,
 * ALIASING (cos/sin overlap), UNSUPPORTED_DEVICE, HIP.
 */
int h3attn_rope_tables(float* cos_out, float* sin_out, int32_t rows, double theta, void* stream);

/*
 * The fused Q/K prologue: per-head RMSNorm followed by the partial rotary
 * embedding, rounded once to bf16 (round to nearest even).
 *
 * For every (b, s, h) row x of 128 channels of q (weight q_norm_w) and of k
 * (weight k_norm_w):
 *   y_c = x_c * (mean_c x_c^2 + eps)^(-1/2) * w_c            (fp32)
 *   for j in 0..47, (a, b) = (y_j, y_{j+48}), c = cos[s*48+j], n = sin[s*48+j]:
 *   y_j <- a*c - b*n,  y_{j+48} <- b*c + a*n;  channels 96..127 unchanged.
 * (TeleFuser PR #37 section 2.2, steps 1 and 3; FastVideo PR #1832,
 * "Preserve H3-specific attention behavior".)
 *
 *   q_in [B,Sq,H,128], k_in [B,Sk,H,128]: device bf16, read only.
 *   q_out, k_out: device bf16, same shapes. Each may equal its input exactly
 *     (in place) or be disjoint from every other tensor.
 *   head_dim: must be 128.
 *   q_norm_w, k_norm_w: device fp32 [128]; both NULL disables the norm.
 *   eps: finite, >= 0 (the configurations use 1e-6).
 *   rope_cos, rope_sin: device fp32 [rope_rows, 48] (see h3attn_rope_tables);
 *     both NULL disables the rotary embedding; row s serves token s.
 *   rope_rows: >= max(Sq, Sk) when the rotary embedding is on.
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_ALIGNMENT, ALIASING, BAD_VALUE,
 * UNSUPPORTED_DEVICE, HIP.
 */
int h3attn_qk_prologue(const uint16_t* q_in, const uint16_t* k_in,
                       uint16_t* q_out, uint16_t* k_out,
                       int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t head_dim,
                       const float* q_norm_w, const float* k_norm_w, float eps,
                       const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                       void* stream);

/*
 * The prologue fused with the destination-major Ulysses pack, for one rank
 * of P that hold sequence shards (TeleFuser PR #37, section 2.2: Q/K
 * RMSNorm, rounding, RoPE and destination-major Q/K/V packing in one
 * kernel; section 2.1: the packed buffers feed the all-to-all that turns
 * sequence shards into head shards). This rank holds rows row_offset ..
 * row_offset + S_local - 1 of the sequence for all H heads; destination
 * rank p takes heads p*H/P .. (p+1)*H/P - 1. With Hl = H / P:
 *   q_send[p][b][s][j][:] = prologue(q)[b][s][p*Hl + j][:]
 *   k_send[p][b][s][j][:] = prologue(k)[b][s][p*Hl + j][:]
 *   v_send[p][b][s][j][:] = v[b][s][p*Hl + j][:]          (bit for bit)
 * where prologue() is h3attn_qk_prologue's RMSNorm + rotary embedding, one
 * bf16 rounding, with rotary table row row_offset + s serving local row s.
 * Chunk p of each buffer (B * S_local * Hl * 128 elements, contiguous) is
 * what rank p receives from this rank: after an equal-split all-to-all of
 * the three buffers, rank p holds [P][B][S_local][Hl][128] in source-rank
 * order, which for B = 1 is the whole sequence of its heads as dense BSHD
 * [1, P * S_local, Hl, 128] (h3attn_forward's layout). The layout of the
 * chunks is this library's reading; the pages name the packing only.
 *
 *   q, k, v: device bf16 [B, S_local, H, 128], dense, read only.
 *   q_send, k_send, v_send: device bf16 [P, B, S_local, Hl, 128], dense,
 *     disjoint from each other and from every input (no in-place form: the
 *     layouts differ).
 *   head_dim: 128.  P >= 1 and H a multiple of P.  row_offset >= 0.
 *   q_norm_w, k_norm_w, eps, rope_cos, rope_sin: as for h3attn_qk_prologue
 *     (both weights NULL: no norm; both tables NULL: no rotary); with the
 *     rotary embedding, rope_rows >= row_offset + S_local.
 *   B * S_local * H < 2^31.
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_ALIGNMENT, ALIASING, BAD_VALUE,
 * UNSUPPORTED_DEVICE, HIP.
 */
int h3attn_qkv_pack(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    uint16_t* q_send, uint16_t* k_send, uint16_t* v_send,
                    int32_t B, int32_t S_local, int32_t H, int32_t P, int32_t head_dim, int32_t row_offset,
                    const float* q_norm_w, const float* k_norm_w, float eps,
                    const float* rope_cos, const float* rope_sin, int32_t rope_rows, void* stream);

/*
 * Bytes of device workspace h3attn_forward needs for these sizes: the
 * normalised q and k and a key-major copy of v, each padded to whole tiles,
 * then room for the partial results of query tiles whose keys the forward
 * splits over several workgroups (it does so when the last round of tiles
 * would leave compute units idle; two fp32 records of 204 KB per split
 * workgroup, at most 512 records), then one fp32 per (b, head, 4096 keys):
 * the largest key norm of each chunk, which bounds the scores when q and k
 * are not normalised. Returns 0 when a size is < 1 or the result would
 * overflow.
 */
size_t h3attn_forward_workspace_bytes(int32_t B, int32_t Sq, int32_t Sk, int32_t H);

/*
 * The attention step: the prologue above on q and k (when enabled), then dense
 * non-causal attention
 *   o_i = sum_{j < kv_valid} softmax_j(softmax_scale * q_i . k_j) v_j   for i < q_valid,
 *   o_i = 0                                                             for q_valid <= i < Sq,
 * per (b, h), with QK^T and PV as bf16 matrix-core contractions accumulated
 * in fp32 and the softmax in fp32. Keys at or past kv_valid are never read.
 *
 *   q [B,Sq,H,128], k and v [B,Sk,H,128]: device bf16, read only.
 *   o [B,Sq,H,128]: device bf16, written in full; disjoint from all inputs
 *     and from the workspace.
 *   head_dim: must be 128.
 *   q_norm_w, k_norm_w, eps: as for h3attn_qk_prologue (both NULL: q and k
 *     are used as given).
 *   rope_cos, rope_sin, rope_rows: as for h3attn_qk_prologue (both NULL: no
 *     rotary embedding; cross-attention uses this).
 *   q_valid: -1 means Sq; else 0..Sq. Rows >= q_valid are written as +0.0.
 *   kv_valid: -1 means Sk; else 1..Sk.
 *   softmax_scale: finite and > 0 (the configurations use 1/sqrt(128)).
 *   workspace: device memory of at least
 *     h3attn_forward_workspace_bytes(B, Sq, Sk, H) bytes, 256-byte aligned,
 *     disjoint from every tensor; its contents on entry do not matter and are
 *     clobbered. Required.
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_ALIGNMENT, ALIASING, BAD_VALUE,
 * WORKSPACE, UNSUPPORTED_DEVICE, HIP.
 */
int h3attn_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                   int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t head_dim,
                   const float* q_norm_w, const float* k_norm_w, float eps,
                   const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                   int32_t q_valid, int32_t kv_valid, float softmax_scale,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * h3attn_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation with the same kernels, with the workspace in a
 * static device array of the library instead of a caller buffer. The call
 * allocates nothing: no hipMalloc or hipFree and no allocating library
 * routine. The array is H3ATTN_NOALLOC_SCRATCH_BYTES on every GPU that
 * loads the library, held until the process ends; the first call on a
 * device looks up its device address (hipGetSymbolAddress).
 *
 * Arguments, results and errors are those of h3attn_forward without
 * workspace and workspace_bytes. Sizes whose workspace
 * (h3attn_forward_workspace_bytes) exceeds H3ATTN_NOALLOC_SCRATCH_BYTES are
 * rejected with H3ATTN_ERR_WORKSPACE before anything is enqueued: the tiny,
 * mid (8192 x 8 heads, 158 MB) and cross-attention (32760 x 8 heads against
 * 512 keys, 177 MB) shapes fit; padded (32768 x 8, 309 MB) and the full
 * 104448 x 6 share (588 MB) do not.
 *
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents; nothing in it needs to start at zero (every call writes
 * what it reads). Calls ordered on one stream are safe; calls that overlap
 * on one GPU (different streams, or host threads without ordering between
 * their launches) race on the array and their outputs are undefined.
 */
#define H3ATTN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int h3attn_forward_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t head_dim,
                           const float* q_norm_w, const float* k_norm_w, float eps,
                           const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                           int32_t q_valid, int32_t kv_valid, float softmax_scale, void* stream);

/*
 * h3attn_forward split into its two stages, for callers that time them
 * separately or prepare k/v once and attend several times.
 *   stages & H3ATTN_STAGE_PREPARE: the prologue on q and k and the key-major
 *     copy of v, written into the workspace (all other tensors read only).
 *   stages & H3ATTN_STAGE_ATTEND: attention from the prepared workspace into o
 *     (one kernel, plus a second that merges split tiles when the schedule
 *     splits any).
 * Arguments and errors are those of h3attn_forward; stages must be 1, 2 or 3
 * (else BAD_VALUE). A call with only H3ATTN_STAGE_ATTEND must follow, in
 * stream order, a PREPARE call with the same sizes, valid lengths and
 * workspace; q, k and v are then not read (but must still be valid
 * pointers, for validation). h3attn_forward(...) equals this with stages = 3.
 */
#define H3ATTN_STAGE_PREPARE 1u
#define H3ATTN_STAGE_ATTEND 2u
int h3attn_forward_stages(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                          int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t head_dim,
                          const float* q_norm_w, const float* k_norm_w, float eps,
                          const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                          int32_t q_valid, int32_t kv_valid, float softmax_scale,
                          void* workspace, size_t workspace_bytes, uint32_t stages, void* stream);

/*
 * The attention step with the variants of the FastVideo PR #1799 dense
 * backend (section "Implementation": MHA and GQA, causal attention, padding
 * and causal masks combined), plus strided inputs and per-item valid
 * lengths. Everything h3attn_forward_stages does, generalised:
 *
 *   o[b, i, h] = sum_{j in V(b, i)} softmax_j(softmax_scale * q[b,i,h] . k[b,j,h/G]) v[b,j,h/G]
 *                for i < q_valid(b), with G = Hq / Hkv (grouped heads; G = 1 is MHA),
 *   V(b, i) = { j < kv_valid(b) }, and with causal also j <= i (the lower
 *             triangle of row indices; for Sq != Sk this is the top-left
 *             alignment of torch's scaled_dot_product_attention),
 *   o[b, i, h] = 0 for q_valid(b) <= i < Sq.
 *
 * q, k, v are views: element strides along batch, sequence and head (the
 * channel stride is 1), for instance slices of a fused QKV projection. All
 * three strides 0 means dense BSHD. Strides must be >= 0 and multiples of 8
 * (every row 16-byte aligned). Views may overlap each other (they are only
 * read) but not o, the workspace or the valid-length array.
 *
 * valid_lengths: NULL, or a device int32 array [2*B] holding q_valid(b) at
 *   [2b] and kv_valid(b) at [2b+1]; q_valid and kv_valid are then ignored.
 *   The kernels clamp each entry to [0, Sq] / [0, Sk]; an item with
 *   kv_valid(b) = 0 has no keys and its rows are written as +0.0. Without
 *   the array, q_valid (-1 = Sq, else 0..Sq) and kv_valid (-1 = Sk, else
 *   1..Sk) apply to every item.
 * causal: 0 or 1. Keys masked by the causal mask still enter the
 *   contraction with weight 0, so a non-finite value there propagates (as
 *   in torch's SDPA); keys at or past kv_valid(b) are never read.
 * head_dim: 64, 128 or 256 (the head dims FastVideo PR #1799,
 *   "Implementation", validates). q, k, v and o are [.., head_dim]; strides
 *   are in elements as above. The norm and rotary arguments (H3's prologue,
 *   defined on 128 channels) must be NULL unless head_dim is 128, else
 *   BAD_SHAPE. Hq must be a multiple of Hkv. Norm, rotary and softmax_scale
 *   arguments are those of h3attn_forward; the rotary table rows serve
 *   sequence positions of q and k alike.
 * Work split: the attention kernel's workgroup owns a query block of one
 *   (b, h): 512 rows at head_dim 64, 256 or 384 at 128 (two or three 16-row
 *   tiles per wave, chosen per launch from the schedule each gives; see
 *   query_tiles), 128 at 256. No causal mask, no valid_lengths and no
 *   window uses the schedule of h3attn_forward (whole rounds of query
 *   blocks, the last round's key steps split over all compute units; at
 *   head_dim 128 with at most 320 valid keys and an item's output below
 *   2^31 bytes, the keys stay resident in LDS and each workgroup streams
 *   several 256-row blocks past them); otherwise
 *   one workgroup per (b, h, query block), the longest first under the
 *   causal mask and the frame window. h3attn_forward_ex_plan() reports the
 *   schedule a call takes.
 *
 * h3attn_forward_ex_workspace_bytes() gives the workspace these arguments
 * need (0 if a size is invalid); stages are those of h3attn_forward_stages
 * (an ATTEND-only call must follow a PREPARE call with the same arguments).
 * Size limits (BAD_SHAPE past them): B * Hq <= 65535; Sq, Sk <= 2^30;
 * B * S * H < 2^31 for q and for k; and one head's prepared keys, Sk rounded
 * up to a multiple of 256 times head_dim * 2 bytes, below 2^31 bytes (the
 * attention kernel addresses them with 32-bit offsets).
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_ALIGNMENT (pointers, strides),
 * ALIASING, BAD_VALUE (causal not 0/1, stages, scale, eps), WORKSPACE,
 * UNSUPPORTED_DEVICE, HIP.
 */
typedef struct h3attn_forward_args {
  const uint16_t* q;          /* [B, Sq, Hq, 128] view */
  const uint16_t* k;          /* [B, Sk, Hkv, 128] view */
  const uint16_t* v;          /* [B, Sk, Hkv, 128] view */
  uint16_t* o;                /* [B, Sq, Hq, 128], dense, written in full */
  int64_t q_stride[3];        /* element strides: batch, sequence, head */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int32_t B, Sq, Sk, Hq, Hkv, head_dim;
  const float* q_norm_w;      /* fp32 [128] each, both NULL: no norm */
  const float* k_norm_w;
  float eps;
  int32_t rope_rows;
  const float* rope_cos;      /* fp32 [rope_rows, 48] each, both NULL: no rotary */
  const float* rope_sin;
  int32_t q_valid;
  int32_t kv_valid;
  const int32_t* valid_lengths;
  int32_t causal;
  float softmax_scale;
  /* Frame-window attention (SGLang PR #37903, "Modifications",
   * hybrid_window_attn_h3: a chunk-5 / radius-1 window with anchor frames,
   * dense-query rows against all keys). Row or key i lies in frame
   * i / window_frame_rows. Frames below window_anchor_frames are anchor
   * frames: their queries see every key. Frame f >= window_anchor_frames is in
   * chunk (f - window_anchor_frames) / window_chunk_frames; its queries see
   * the anchor frames and the frames of the chunks within window_radius of
   * their own. Composed with the valid lengths like the other masks; a row
   * that sees no key is written as 0. window_frame_rows = 0 turns the window
   * off (the other three fields must then be 0); otherwise
   * window_chunk_frames >= 1, window_radius >= 0, window_anchor_frames >= 0,
   * and causal must be 0. */
  int32_t window_frame_rows;
  int32_t window_chunk_frames;
  int32_t window_radius;
  int32_t window_anchor_frames;
  /* Softmax gate epilogue: NULL, or bf16 [B, Sq, Hq] contiguous (2-byte
   * aligned, disjoint from o); each output row (b, i, h) is multiplied by
   * sigmoid(gate[b, i, h]) = 1 / (1 + exp(-gate)) before its bf16 rounding.
   * Rows at or past q_valid stay +0.0. */
  const uint16_t* gate;
  /* Query tiles per wave of the attention kernel: 0 (a zeroed descriptor)
   * lets the library choose; otherwise 2 or 3 at head_dim 128 and the one
   * count of the other head dims (4 at 64, 2 at 256), else BAD_VALUE. An
   * override for tuning and tests: every row's arithmetic is the same at
   * either count, so tiles that run whole give bit-identical rows; the
   * split last round divides its keys differently (same accuracy). Ignored
   * when the keys are resident in LDS. The workspace does not depend on
   * it. */
  int32_t query_tiles;
} h3attn_forward_args;

size_t h3attn_forward_ex_workspace_bytes(const h3attn_forward_args* args);
int h3attn_forward_ex(const h3attn_forward_args* args, void* workspace, size_t workspace_bytes,
                      uint32_t stages, void* stream);

/*
 * The schedule h3attn_forward_ex(args) launches on a device with `cus`
 * compute units (cus <= 0: the current device's), written to *plan. Host
 * arithmetic only: nothing is enqueued, and with cus > 0 no device is
 * needed. Arguments are checked as for h3attn_forward_ex, except the
 * workspace and the device (pointers are not dereferenced).
 * Errors: NULL_POINTER (plan or args), the argument errors of
 * h3attn_forward_ex, UNSUPPORTED_DEVICE or HIP when cus <= 0 and there is no
 * usable device.
 */
typedef struct h3attn_plan {
  int32_t kernel;         /* 0: the ring kernel; 1: keys resident in LDS */
  int32_t query_tiles;    /* 16-row query tiles per wave */
  int32_t rows_per_tile;  /* query rows per workgroup tile */
  int32_t reserved;       /* 0 */
  int64_t tiles;          /* tiles with valid rows (every tile in general mode) */
  int64_t whole_tiles;    /* uniform schedule: tiles run whole */
  int64_t split_tiles;    /* uniform schedule: last-round tiles split over split_blocks workgroups */
  int64_t split_blocks;
  int64_t grid;           /* workgroups of the attention kernel */
} h3attn_plan;
int h3attn_forward_ex_plan(const h3attn_forward_args* args, int32_t cus, h3attn_plan* plan);

/*
 * Fused RMSNorm + indexed AdaLN scale/shift, the DiT block's norm before the
 * QKV projection (TeleFuser PR #37, "2.5 Fuse RMSNorm with indexed AdaLN
 * modulation"). It keeps every bf16 rounding of the unfused chain
 * "RMSNorm, then x * (1 + scale) + shift", so the result equals that chain
 * computed with bf16 tensor arithmetic bit for bit. For token (b, s) with
 * channels x_c, c < D, and i = index[b*S + s] clamped to [0, M-1] (0 when
 * index is NULL):
 *   r   = 1 / sqrt(mean_c x_c^2 + eps), rounded to the nearest fp32
 *   n_c = bf16(fp32(x_c * r) * w_c)            (without "* w_c" when norm_w is NULL)
 *   t_c = bf16(1 + scale[b, i, c])
 *   u_c = bf16(n_c * t_c)
 *   y_c = bf16(u_c + shift[b, i, c])
 * where every operation is one fp32 IEEE operation and bf16() rounds to
 * nearest, ties to even. r is computed from an fp64 sum of squares, so it is
 * the nearest fp32 value except when 1/sqrt(.) lies within ~2^-48 (relative)
 * of a point halfway between two fp32 values, where either neighbour may
 * result. NaN or infinity in a row of x makes that whole row NaN; NaN in
 * scale or shift makes that channel NaN.
 *   x, y:         bf16 [B, S, D], contiguous. y == x (in place) or y disjoint
 *                 from every input.
 *   norm_w:       fp32 [D] or NULL (no weight, the usual DiT block norm).
 *   eps:          finite, >= 0.
 *   scale, shift: bf16 [B, M, D], contiguous, M >= 1.
 *   index:        int32 [B, S], contiguous, or NULL; values outside [0, M)
 *                 are clamped (never read out of bounds).
 *   B, S >= 1; D a multiple of 8, 8 <= D <= 16384; B*S < 2^31.
 * Alignment: x, y, scale, shift, norm_w 16 bytes; index 4 bytes.
 * Errors: NULL_POINTER, BAD_SHAPE, BAD_ALIGNMENT, ALIASING, BAD_VALUE (eps),
 * UNSUPPORTED_DEVICE, HIP.
 */
int h3attn_rmsnorm_scale_shift(const uint16_t* x, uint16_t* y, int32_t B, int32_t S, int32_t D,
                               const float* norm_w, float eps, const uint16_t* scale,
                               const uint16_t* shift, int32_t M, const int32_t* index, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* H3ATTN_H_ */
