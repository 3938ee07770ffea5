// C-ABI layer of the h3attn library: argument validation, the gfx950 device
// gate, workspace carving and kernel orchestration. Every check runs before
// anything is enqueued, so an error return means no work was done.
#include "h3attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "h3attn_internal.h"

#define H3_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture.
std::atomic<int> g_device_kind[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return H3ATTN_ERR_UNSUPPORTED_DEVICE;
  if (dev >= kMaxDevices) return H3ATTN_ERR_UNSUPPORTED_DEVICE;
  int kind = g_device_kind[dev].load(std::memory_order_relaxed);
  if (kind == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return H3ATTN_ERR_HIP;
    kind = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_kind[dev].store(kind, std::memory_order_relaxed);
  }
  return kind == 1 ? H3ATTN_OK : H3ATTN_ERR_UNSUPPORTED_DEVICE;
}

}  // namespace

int h3::check_gfx950() { return check_device(); }

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Bytes of a [B, S, H, D] bf16 tensor, or 0 on overflow.
size_t bshd_bytes(int32_t B, int32_t S, int32_t H, int32_t D = h3::kHeadDim) {
  const unsigned __int128 n = (unsigned __int128)B * (unsigned __int128)S * (unsigned __int128)H * (unsigned)D * 2u;
  if (n > (unsigned __int128)(INT64_MAX / 4)) return 0;
  return (size_t)n;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int status_from(hipError_t e) { return e == hipSuccess ? H3ATTN_OK : H3ATTN_ERR_HIP; }

// Shared validation of the prologue arguments (both entry points).
int check_prologue_args(int32_t Sq, int32_t Sk, const float* wq, const float* wk, float eps,
                        const float* rc, const float* rs, int32_t rope_rows) {
  if ((wq == nullptr) != (wk == nullptr)) return H3ATTN_ERR_NULL_POINTER;
  if ((rc == nullptr) != (rs == nullptr)) return H3ATTN_ERR_NULL_POINTER;
  if (wq && !(std::isfinite(eps) && eps >= 0.f)) return H3ATTN_ERR_BAD_VALUE;
  if (wq && (!aligned16(wq) || !aligned16(wk))) return H3ATTN_ERR_BAD_ALIGNMENT;
  if (rc) {
    if (rope_rows < Sq || rope_rows < Sk) return H3ATTN_ERR_BAD_SHAPE;
    if (!aligned16(rc) || !aligned16(rs)) return H3ATTN_ERR_BAD_ALIGNMENT;
    const size_t tb = (size_t)rope_rows * h3::kRopePairs * sizeof(float);
    if (overlap(range_of(rc, tb), range_of(rs, tb))) return H3ATTN_ERR_ALIASING;
  }
  return H3ATTN_OK;
}

struct WorkspaceLayout {
  int64_t Sq_pad, Sk_pad, part_slots, kn_chunks;
  size_t q_off, k_off, v_off, part_off, kn_off, total;
};

// Workspace of a forward with Hq query heads and Hkv key/value heads; the
// partial records of split tiles are only needed by the uniform schedule
// (no causal mask, no per-item lengths).
bool workspace_layout(int32_t B, int32_t Sq, int32_t Sk, int32_t Hq, int32_t Hkv, bool uniform, int32_t D,
                      WorkspaceLayout* w) {
  if (B < 1 || Sq < 1 || Sk < 1 || Hq < 1 || Hkv < 1) return false;
  if (D != 64 && D != 128 && D != 256) return false;
  // Query rows pad to whole query blocks of every tiling a launch may take:
  // the ring kernel's (512 rows at head dim 64, 256 or 384 at 128, 128 at
  // 256) and the resident-key kernel's (256).
  w->Sq_pad = std::max({round_up(Sq, h3::attn_rows(D, h3::attn_qt_min(D))),
                        round_up(Sq, h3::attn_rows(D, h3::attn_qt_max(D))), round_up(Sq, h3::kRowPad)});
  w->Sk_pad = round_up(Sk, h3::kRowPad);
  const unsigned row = 2u * (unsigned)D;
  const unsigned __int128 qb = (unsigned __int128)B * (unsigned __int128)Hq * (unsigned __int128)w->Sq_pad * row;
  const unsigned __int128 kb = (unsigned __int128)B * (unsigned __int128)Hkv * (unsigned __int128)w->Sk_pad * row;
  w->part_slots = uniform ? h3::split_part_slots(B, Sq, Sk, Hq, D) : 0;
  const unsigned __int128 pb = (unsigned __int128)w->part_slots * (sizeof(float) * h3::attn_part_floats_max(D));
  // Key-norm maxima (fp32 per chunk of keys of each (b, kv head)), padded to 256 bytes.
  w->kn_chunks = h3::key_norm_chunks(w->Sk_pad);
  const unsigned __int128 nb = ((unsigned __int128)B * Hkv * w->kn_chunks * sizeof(float) + 255) / 256 * 256;
  const unsigned __int128 tot = qb + 2 * kb + pb + nb;
  if (tot > (unsigned __int128)(INT64_MAX / 4)) return false;
  w->q_off = 0;
  w->k_off = (size_t)qb;
  w->v_off = (size_t)(qb + kb);
  w->part_off = (size_t)(qb + 2 * kb);
  w->kn_off = (size_t)(qb + 2 * kb + pb);
  w->total = (size_t)tot;
  return true;
}

// Element strides of a [B, S, H, D] view: all three 0 means dense.
void resolve_strides(const int64_t in[3], int32_t S, int32_t H, int32_t D, int64_t out[3]) {
  if (in[0] == 0 && in[1] == 0 && in[2] == 0) {
    out[2] = D;
    out[1] = (int64_t)H * D;
    out[0] = (int64_t)S * out[1];
  } else {
    out[0] = in[0];
    out[1] = in[1];
    out[2] = in[2];
  }
}

// Byte range [lo, hi) a [B, S, H, D] view with non-negative strides can
// touch, or false on overflow.
bool view_range(const void* p, const int64_t st[3], int32_t B, int32_t S, int32_t H, int32_t D, Range* r) {
  const unsigned __int128 last = (unsigned __int128)(B - 1) * (uint64_t)st[0] + (unsigned __int128)(S - 1) * (uint64_t)st[1] +
                                 (unsigned __int128)(H - 1) * (uint64_t)st[2] + (unsigned)D;
  const unsigned __int128 bytes = last * 2u;
  if (bytes > (unsigned __int128)(INT64_MAX / 4)) return false;
  *r = range_of(p, (size_t)bytes);
  return true;
}

}  // namespace

H3_API const char* h3attn_status_string(int status) {
  switch (status) {
    case H3ATTN_OK: return "ok";
    case H3ATTN_ERR_NULL_POINTER: return "a required pointer is NULL (or only one of a pair was given)";
    case H3ATTN_ERR_BAD_SHAPE: return "a size is out of range (head_dim 128, or 64/256 without norm and rotary; S, H, B >= 1; valid lengths; rotary table rows)";
    case H3ATTN_ERR_BAD_ALIGNMENT: return "a pointer is not 16-byte aligned (workspace: 256-byte)";
    case H3ATTN_ERR_ALIASING: return "an output overlaps an input or another output";
    case H3ATTN_ERR_BAD_VALUE: return "eps, theta or softmax_scale is not finite or out of range";
    case H3ATTN_ERR_WORKSPACE: return "workspace missing or smaller than h3attn_forward_workspace_bytes()";
    case H3ATTN_ERR_UNSUPPORTED_DEVICE: return "the current device is not gfx950 (MI355X), or no device is present";
    case H3ATTN_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    default: return "unknown h3attn status";
  }
}

H3_API int h3attn_rope_tables(float* cos_out, float* sin_out, int32_t rows, double theta, void* stream) {
  if (!cos_out || !sin_out) return H3ATTN_ERR_NULL_POINTER;
  if (rows < 1 || (int64_t)rows * h3::kRopePairs > INT32_MAX) return H3ATTN_ERR_BAD_SHAPE;
  if (!std::isfinite(theta) || !(theta > 1.0)) return H3ATTN_ERR_BAD_VALUE;
  if (!aligned16(cos_out) || !aligned16(sin_out)) return H3ATTN_ERR_BAD_ALIGNMENT;
  const size_t tb = (size_t)rows * h3::kRopePairs * sizeof(float);
  if (overlap(range_of(cos_out, tb), range_of(sin_out, tb))) return H3ATTN_ERR_ALIASING;
  if (int st = check_device()) return st;
  return status_from(h3::launch_rope_tables(cos_out, sin_out, rows, theta, (hipStream_t)stream));
}

H3_API int h3attn_qk_prologue(const uint16_t* q_in, const uint16_t* k_in, uint16_t* q_out, uint16_t* k_out,
                              int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t head_dim,
                              const float* q_norm_w, const float* k_norm_w, float eps,
                              const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                              void* stream) {
  if (!q_in || !k_in || !q_out || !k_out) return H3ATTN_ERR_NULL_POINTER;
  if (head_dim != h3::kHeadDim || B < 1 || Sq < 1 || Sk < 1 || H < 1) return H3ATTN_ERR_BAD_SHAPE;
  const size_t qbytes = bshd_bytes(B, Sq, H), kbytes = bshd_bytes(B, Sk, H);
  if (qbytes == 0 || kbytes == 0) return H3ATTN_ERR_BAD_SHAPE;
  if ((int64_t)B * Sq * H >= (1ll << 31) || (int64_t)B * Sk * H >= (1ll << 31)) return H3ATTN_ERR_BAD_SHAPE;
  if (int st = check_prologue_args(Sq, Sk, q_norm_w, k_norm_w, eps, rope_cos, rope_sin, rope_rows)) return st;
  if (!aligned16(q_in) || !aligned16(k_in) || !aligned16(q_out) || !aligned16(k_out))
    return H3ATTN_ERR_BAD_ALIGNMENT;
  const Range qi = range_of(q_in, qbytes), ki = range_of(k_in, kbytes);
  const Range qo = range_of(q_out, qbytes), ko = range_of(k_out, kbytes);
  if (q_out != q_in && (overlap(qo, qi) || overlap(qo, ki))) return H3ATTN_ERR_ALIASING;
  if (k_out != k_in && (overlap(ko, ki) || overlap(ko, qi))) return H3ATTN_ERR_ALIASING;
  if (overlap(qo, ko)) return H3ATTN_ERR_ALIASING;
  if (q_out == q_in && overlap(qi, ki)) return H3ATTN_ERR_ALIASING;
  if (int st = check_device()) return st;

  const int64_t row = (int64_t)H * h3::kHeadDim;
  h3::ProTensor tq{q_in, q_out, q_norm_w, (int64_t)Sq * row, row, h3::kHeadDim,
                   (int64_t)Sq * row, row, h3::kHeadDim, Sq, Sq, 1.0f, nullptr, 0, H};
  h3::ProTensor tk{k_in, k_out, k_norm_w, (int64_t)Sk * row, row, h3::kHeadDim,
                   (int64_t)Sk * row, row, h3::kHeadDim, Sk, Sk, 1.0f, nullptr, 1, H};
  return status_from(h3::launch_qk_prologue(tq, tk, B, eps, rope_cos, rope_sin, (hipStream_t)stream));
}

H3_API int h3attn_qkv_pack(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* q_send,
                           uint16_t* k_send, uint16_t* v_send, int32_t B, int32_t S_local, int32_t H, int32_t P,
                           int32_t head_dim, int32_t row_offset, const float* q_norm_w, const float* k_norm_w,
                           float eps, const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                           void* stream) {
  if (!q || !k || !v || !q_send || !k_send || !v_send) return H3ATTN_ERR_NULL_POINTER;
  if (head_dim != h3::kHeadDim || B < 1 || S_local < 1 || H < 1 || P < 1 || H % P != 0 || row_offset < 0)
    return H3ATTN_ERR_BAD_SHAPE;
  const size_t bytes = bshd_bytes(B, S_local, H);
  if (bytes == 0 || (int64_t)B * S_local * H >= (1ll << 31)) return H3ATTN_ERR_BAD_SHAPE;
  if (rope_cos && (int64_t)rope_rows < (int64_t)row_offset + S_local) return H3ATTN_ERR_BAD_SHAPE;
  if (int st = check_prologue_args(1, 1, q_norm_w, k_norm_w, eps, rope_cos, rope_sin, rope_rows)) return st;
  const void* ptrs[6] = {q, k, v, q_send, k_send, v_send};
  for (const void* p : ptrs)
    if (!aligned16(p)) return H3ATTN_ERR_BAD_ALIGNMENT;
  for (int i = 3; i < 6; ++i)
    for (int j = 0; j < 6; ++j)
      if (i != j && overlap(range_of(ptrs[i], bytes), range_of(ptrs[j], bytes))) return H3ATTN_ERR_ALIASING;
  for (int i = 3; i < 6; ++i) {
    const Range o = range_of(ptrs[i], bytes);
    if (q_norm_w && (overlap(o, range_of(q_norm_w, 512)) || overlap(o, range_of(k_norm_w, 512))))
      return H3ATTN_ERR_ALIASING;
    if (rope_cos) {
      const size_t tb = (size_t)rope_rows * h3::kRopePairs * sizeof(float);
      if (overlap(o, range_of(rope_cos, tb)) || overlap(o, range_of(rope_sin, tb))) return H3ATTN_ERR_ALIASING;
    }
  }
  if (int st = check_device()) return st;
  h3::QkvPack t{q, k, v, q_send, k_send, v_send, q_norm_w, k_norm_w, eps, rope_cos, rope_sin,
                B, S_local, H, P, row_offset};
  return status_from(h3::launch_qkv_pack(t, (hipStream_t)stream));
}

H3_API size_t h3attn_forward_workspace_bytes(int32_t B, int32_t Sq, int32_t Sk, int32_t H) {
  WorkspaceLayout w;
  if (!workspace_layout(B, Sq, Sk, H, H, true, h3::kHeadDim, &w)) return 0;
  return w.total;
}

namespace {

bool uniform_schedule(const h3attn_forward_args* a) {
  return !a->causal && a->valid_lengths == nullptr && a->window_frame_rows == 0;
}

// Validates every argument of a forward before anything is enqueued; on
// success fills the resolved strides and the workspace layout.
// With with_workspace false, the workspace and the device gate are not
// checked (a caller that brings its own workspace checks them after).
int check_forward(const h3attn_forward_args* a, size_t workspace_bytes, const void* workspace, uint32_t stages,
                  int64_t qs[3], int64_t ks[3], int64_t vs[3], WorkspaceLayout* wl, bool with_workspace = true) {
  if (!a) return H3ATTN_ERR_NULL_POINTER;
  if (!a->q || !a->k || !a->v || !a->o) return H3ATTN_ERR_NULL_POINTER;
  if (stages == 0 || stages > (H3ATTN_STAGE_PREPARE | H3ATTN_STAGE_ATTEND)) return H3ATTN_ERR_BAD_VALUE;
  const int32_t B = a->B, Sq = a->Sq, Sk = a->Sk, Hq = a->Hq, Hkv = a->Hkv;
  if ((a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256) || B < 1 || Sq < 1 || Sk < 1 || Hq < 1 ||
      Hkv < 1)
    return H3ATTN_ERR_BAD_SHAPE;
  // The Q/K norm and the partial rotary embedding are H3's, defined on 128 channels.
  if (a->head_dim != h3::kHeadDim && (a->q_norm_w || a->k_norm_w || a->rope_cos || a->rope_sin))
    return H3ATTN_ERR_BAD_SHAPE;
  if (Hq % Hkv != 0) return H3ATTN_ERR_BAD_SHAPE;
  if ((int64_t)B * Hq > 65535 || Sq > (1 << 30) || Sk > (1 << 30)) return H3ATTN_ERR_BAD_SHAPE;
  const int32_t D = a->head_dim;
  const size_t obytes = bshd_bytes(B, Sq, Hq, D);
  if (obytes == 0 || bshd_bytes(B, Sk, Hkv, D) == 0) return H3ATTN_ERR_BAD_SHAPE;
  if (a->causal != 0 && a->causal != 1) return H3ATTN_ERR_BAD_VALUE;
  if (a->window_frame_rows < 0) return H3ATTN_ERR_BAD_VALUE;
  if (a->window_frame_rows == 0) {
    if (a->window_chunk_frames || a->window_radius || a->window_anchor_frames) return H3ATTN_ERR_BAD_VALUE;
  } else if (a->window_chunk_frames < 1 || a->window_radius < 0 || a->window_anchor_frames < 0 || a->causal) {
    return H3ATTN_ERR_BAD_VALUE;
  } else if (Sq >= (1 << 28) || Sk >= (1 << 28)) {
    return H3ATTN_ERR_BAD_SHAPE;   // keeps the window's row arithmetic in 32 bits
  }
  if (!a->valid_lengths) {
    const int32_t qv = a->q_valid == -1 ? Sq : a->q_valid;
    const int32_t kvv = a->kv_valid == -1 ? Sk : a->kv_valid;
    if (qv < 0 || qv > Sq || kvv < 1 || kvv > Sk) return H3ATTN_ERR_BAD_SHAPE;
  }
  if (!std::isfinite(a->softmax_scale) || !(a->softmax_scale > 0.f)) return H3ATTN_ERR_BAD_VALUE;
  if (a->query_tiles != 0 && (a->query_tiles < h3::attn_qt_min(a->head_dim) || a->query_tiles > h3::attn_qt_max(a->head_dim)))
    return H3ATTN_ERR_BAD_VALUE;
  if (int st = check_prologue_args(Sq, Sk, a->q_norm_w, a->k_norm_w, a->eps, a->rope_cos, a->rope_sin, a->rope_rows))
    return st;
  for (int i = 0; i < 3; ++i)
    if (a->q_stride[i] < 0 || a->k_stride[i] < 0 || a->v_stride[i] < 0) return H3ATTN_ERR_BAD_SHAPE;
  resolve_strides(a->q_stride, Sq, Hq, D, qs);
  resolve_strides(a->k_stride, Sk, Hkv, D, ks);
  resolve_strides(a->v_stride, Sk, Hkv, D, vs);
  for (int i = 0; i < 3; ++i)
    if ((qs[i] | ks[i] | vs[i]) & 7) return H3ATTN_ERR_BAD_ALIGNMENT;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o)) return H3ATTN_ERR_BAD_ALIGNMENT;
  if (a->valid_lengths && (reinterpret_cast<uintptr_t>(a->valid_lengths) & 3u)) return H3ATTN_ERR_BAD_ALIGNMENT;
  if (a->gate && (reinterpret_cast<uintptr_t>(a->gate) & 1u)) return H3ATTN_ERR_BAD_ALIGNMENT;
  if (!workspace_layout(B, Sq, Sk, Hq, Hkv, uniform_schedule(a), D, wl)) return H3ATTN_ERR_BAD_SHAPE;
  if ((int64_t)B * Hq * wl->Sq_pad >= (1ll << 31) || (int64_t)B * Hkv * wl->Sk_pad >= (1ll << 31))
    return H3ATTN_ERR_BAD_SHAPE;
  // One head's prepared keys are addressed with 32-bit byte offsets.
  if ((int64_t)wl->Sk_pad * D * 2 >= (1ll << 31)) return H3ATTN_ERR_BAD_SHAPE;
  if ((int64_t)B * Sq * Hq >= (1ll << 31) || (int64_t)B * Sk * Hkv >= (1ll << 31)) return H3ATTN_ERR_BAD_SHAPE;
  Range rq, rk, rv;
  if (!view_range(a->q, qs, B, Sq, Hq, D, &rq) || !view_range(a->k, ks, B, Sk, Hkv, D, &rk) ||
      !view_range(a->v, vs, B, Sk, Hkv, D, &rv))
    return H3ATTN_ERR_BAD_SHAPE;
  if (with_workspace) {
    if (!workspace || workspace_bytes < wl->total) return H3ATTN_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return H3ATTN_ERR_BAD_ALIGNMENT;
  }
  const Range oq = range_of(a->o, obytes);
  const Range ws = with_workspace ? range_of(workspace, wl->total) : Range{0, 0};
  if (overlap(oq, rq) || overlap(oq, rk) || overlap(oq, rv) || overlap(oq, ws)) return H3ATTN_ERR_ALIASING;
  if (overlap(ws, rq) || overlap(ws, rk) || overlap(ws, rv)) return H3ATTN_ERR_ALIASING;
  if (a->q_norm_w) {
    const Range w1 = range_of(a->q_norm_w, 512), w2 = range_of(a->k_norm_w, 512);
    if (overlap(ws, w1) || overlap(ws, w2) || overlap(oq, w1) || overlap(oq, w2)) return H3ATTN_ERR_ALIASING;
  }
  if (a->rope_cos) {
    const size_t tb = (size_t)a->rope_rows * h3::kRopePairs * sizeof(float);
    const Range c1 = range_of(a->rope_cos, tb), c2 = range_of(a->rope_sin, tb);
    if (overlap(ws, c1) || overlap(ws, c2) || overlap(oq, c1) || overlap(oq, c2)) return H3ATTN_ERR_ALIASING;
  }
  if (a->valid_lengths) {
    const Range lr = range_of(a->valid_lengths, (size_t)B * 2 * sizeof(int32_t));
    if (overlap(ws, lr) || overlap(oq, lr)) return H3ATTN_ERR_ALIASING;
  }
  if (a->gate) {
    const Range gr = range_of(a->gate, (size_t)B * Sq * Hq * sizeof(uint16_t));
    if (overlap(ws, gr) || overlap(oq, gr)) return H3ATTN_ERR_ALIASING;
  }
  return with_workspace ? check_device() : H3ATTN_OK;
}

// The attention kernel's arguments for a checked forward, less the
// workspace pointers and the key-norm maxima.
h3::AttnArgs attn_args(const h3attn_forward_args* a, const WorkspaceLayout& wl) {
  const int32_t Sq = a->Sq, Sk = a->Sk;
  h3::AttnArgs at{};
  at.D = a->head_dim;
  at.o = a->o;
  at.part_slots = wl.part_slots;
  at.B = a->B;
  at.H = a->Hq;
  at.Sq = Sq;
  at.Sk = Sk;
  at.Sq_pad = (int32_t)wl.Sq_pad;
  at.Sk_pad = (int32_t)wl.Sk_pad;
  at.q_valid = a->valid_lengths ? Sq : (a->q_valid == -1 ? Sq : a->q_valid);
  at.kv_valid = a->valid_lengths ? Sk : (a->kv_valid == -1 ? Sk : a->kv_valid);
  at.Hkv = a->Hkv;
  at.causal = a->causal;
  at.lengths = a->valid_lengths;
  if (a->window_frame_rows > 0) {
    // Clamp the geometry to the sequence without changing which keys a row
    // sees: a frame longer than the sequence is one frame, and counts of
    // anchor frames, chunk frames or radius chunks beyond the sequence's
    // frames cover everything. With S < 2^28 the kernel's products
    // (A + C*(c + R + 1)) * F then stay below 2^31.
    const int32_t S = std::max(Sq, Sk);
    const int32_t F = std::min(a->window_frame_rows, S);
    const int32_t n_frames = (S + F - 1) / F;
    at.win_F = F;
    at.win_C = std::min(a->window_chunk_frames, n_frames);
    at.win_R = std::min(a->window_radius, n_frames);
    at.win_A = std::min(a->window_anchor_frames, n_frames);
  }
  at.gate = a->gate;
  at.wq = a->q_norm_w;
  at.wk = a->k_norm_w;
  at.kn_chunks = (int32_t)wl.kn_chunks;
  at.query_tiles = a->query_tiles;
  return at;
}

int run_forward(const h3attn_forward_args* a, void* workspace, size_t workspace_bytes, uint32_t stages,
                void* stream) {
  int64_t qs[3], ks[3], vs[3];
  WorkspaceLayout wl;
  if (int st = check_forward(a, workspace_bytes, workspace, stages, qs, ks, vs, &wl)) return st;
  const int32_t B = a->B, Sq = a->Sq, Sk = a->Sk, Hq = a->Hq, Hkv = a->Hkv;
  const int32_t q_valid = a->valid_lengths ? Sq : (a->q_valid == -1 ? Sq : a->q_valid);
  const int32_t kv_valid = a->valid_lengths ? Sk : (a->kv_valid == -1 ? Sk : a->kv_valid);

  hipStream_t s = (hipStream_t)stream;
  uint16_t* wsb = static_cast<uint16_t*>(workspace);
  uint16_t* qw = wsb + wl.q_off / 2;
  uint16_t* kw = wsb + wl.k_off / 2;
  uint16_t* vt = wsb + wl.v_off / 2;
  float* kn = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + wl.kn_off);

  // Prologue into the head-major workspace: rows past the valid length are
  // zero-filled so the attention kernel can read whole tiles.
  // q is written pre-multiplied by softmax_scale*log2(e) (fp32, before its
  // one bf16 rounding), so the attention kernel's scores are in exp2 units.
  const float c = (float)((double)a->softmax_scale * 1.4426950408889634);
  const int32_t D = a->head_dim;
  h3::ProTensor tq{a->q, qw, a->q_norm_w, qs[0], qs[1], qs[2],
                   (int64_t)Hq * wl.Sq_pad * D, D, wl.Sq_pad * D,
                   q_valid, (int32_t)wl.Sq_pad, c, a->valid_lengths, 0, Hq};
  h3::ProTensor tk{a->k, kw, a->k_norm_w, ks[0], ks[1], ks[2],
                   (int64_t)Hkv * wl.Sk_pad * D, D, wl.Sk_pad * D,
                   kv_valid, (int32_t)wl.Sk_pad, 1.0f, a->valid_lengths, 1, Hkv};
  if (stages & H3ATTN_STAGE_PREPARE) {
    // Head dim 128 runs H3's norm + rotary prologue (each part optional);
    // other head dims have neither and only copy (q scaled) into the layout.
    hipError_t e = D == h3::kHeadDim ? h3::launch_qk_prologue(tq, tk, B, a->eps, a->rope_cos, a->rope_sin, s)
                                     : h3::launch_qk_copy(tq, tk, B, D, s);
    if (e != hipSuccess) return H3ATTN_ERR_HIP;
    e = h3::launch_v_relayout(a->v, vs[0], vs[1], vs[2], vt, B, Sk, Hkv, kv_valid, a->valid_lengths,
                              (int32_t)wl.Sk_pad, D, s);
    if (e != hipSuccess) return H3ATTN_ERR_HIP;
    // Without H3's norm the score bound comes from the data: the largest
    // prepared key norm of each chunk of keys.
    if (a->k_norm_w == nullptr) {
      e = h3::launch_key_norms(kw, kn, B * Hkv, (int32_t)wl.Sk_pad, (int32_t)wl.kn_chunks, D, s);
      if (e != hipSuccess) return H3ATTN_ERR_HIP;
    }
  }
  if (!(stages & H3ATTN_STAGE_ATTEND)) return H3ATTN_OK;

  h3::AttnArgs at = attn_args(a, wl);
  at.qw = qw;
  at.kw = kw;
  at.vt = vt;
  at.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + wl.part_off);
  at.c_log2 = c;
  at.knorm = a->k_norm_w == nullptr ? kn : nullptr;
  return status_from(h3::launch_attention(at, s));
}

h3attn_forward_args dense_args(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, int32_t B,
                               int32_t Sq, int32_t Sk, int32_t H, int32_t head_dim, const float* q_norm_w,
                               const float* k_norm_w, float eps, const float* rope_cos, const float* rope_sin,
                               int32_t rope_rows, int32_t q_valid, int32_t kv_valid, float softmax_scale) {
  h3attn_forward_args a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.B = B;
  a.Sq = Sq;
  a.Sk = Sk;
  a.Hq = H;
  a.Hkv = H;
  a.head_dim = head_dim;
  a.q_norm_w = q_norm_w;
  a.k_norm_w = k_norm_w;
  a.eps = eps;
  a.rope_rows = rope_rows;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.q_valid = q_valid;
  a.kv_valid = kv_valid;
  a.valid_lengths = nullptr;
  a.causal = 0;
  a.softmax_scale = softmax_scale;
  return a;
}

}  // namespace

int h3::check_dense_args(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, int32_t B,
                         int32_t Sq, int32_t Sk, int32_t H, int32_t head_dim, const float* q_norm_w,
                         const float* k_norm_w, float eps, const float* rope_cos, const float* rope_sin,
                         int32_t rope_rows, int32_t q_valid, int32_t kv_valid, float softmax_scale,
                         size_t* workspace_bytes) {
  const h3attn_forward_args a = dense_args(q, k, v, o, B, Sq, Sk, H, head_dim, q_norm_w, k_norm_w, eps, rope_cos,
                                           rope_sin, rope_rows, q_valid, kv_valid, softmax_scale);
  int64_t qs[3], ks[3], vs[3];
  WorkspaceLayout wl;
  const int st = check_forward(&a, 0, nullptr, H3ATTN_STAGE_PREPARE | H3ATTN_STAGE_ATTEND, qs, ks, vs, &wl, false);
  if (st == H3ATTN_OK) *workspace_bytes = wl.total;
  return st;
}

int h3::forward_dense(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, int32_t B, int32_t Sq,
                      int32_t Sk, int32_t H, int32_t head_dim, const float* q_norm_w, const float* k_norm_w, float eps,
                      const float* rope_cos, const float* rope_sin, int32_t rope_rows, int32_t q_valid,
                      int32_t kv_valid, float softmax_scale, void* workspace, size_t workspace_bytes, uint32_t stages,
                      void* stream) {
  const h3attn_forward_args a = dense_args(q, k, v, o, B, Sq, Sk, H, head_dim, q_norm_w, k_norm_w, eps, rope_cos,
                                           rope_sin, rope_rows, q_valid, kv_valid, softmax_scale);
  return run_forward(&a, workspace, workspace_bytes, stages, stream);
}

H3_API int h3attn_forward(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                          int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t head_dim,
                          const float* q_norm_w, const float* k_norm_w, float eps,
                          const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                          int32_t q_valid, int32_t kv_valid, float softmax_scale,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const h3attn_forward_args a = dense_args(q, k, v, o, B, Sq, Sk, H, head_dim, q_norm_w, k_norm_w, eps, rope_cos,
                                           rope_sin, rope_rows, q_valid, kv_valid, softmax_scale);
  return run_forward(&a, workspace, workspace_bytes, H3ATTN_STAGE_PREPARE | H3ATTN_STAGE_ATTEND, stream);
}

H3_API int h3attn_forward_stages(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                                 int32_t B, int32_t Sq, int32_t Sk, int32_t H, int32_t head_dim,
                                 const float* q_norm_w, const float* k_norm_w, float eps,
                                 const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                                 int32_t q_valid, int32_t kv_valid, float softmax_scale,
                                 void* workspace, size_t workspace_bytes, uint32_t stages, void* stream) {
  const h3attn_forward_args a = dense_args(q, k, v, o, B, Sq, Sk, H, head_dim, q_norm_w, k_norm_w, eps, rope_cos,
                                           rope_sin, rope_rows, q_valid, kv_valid, softmax_scale);
  return run_forward(&a, workspace, workspace_bytes, stages, stream);
}

H3_API size_t h3attn_forward_ex_workspace_bytes(const h3attn_forward_args* args) {
  if (!args || args->Hkv < 1 || args->Hq < 1 || args->Hq % args->Hkv != 0) return 0;
  WorkspaceLayout w;
  if (!workspace_layout(args->B, args->Sq, args->Sk, args->Hq, args->Hkv, uniform_schedule(args), args->head_dim,
                        &w))
    return 0;
  return w.total;
}

H3_API int h3attn_forward_ex(const h3attn_forward_args* args, void* workspace, size_t workspace_bytes,
                             uint32_t stages, void* stream) {
  return run_forward(args, workspace, workspace_bytes, stages, stream);
}

H3_API int h3attn_forward_ex_plan(const h3attn_forward_args* args, int32_t cus, h3attn_plan* plan) {
  if (!plan) return H3ATTN_ERR_NULL_POINTER;
  int64_t qs[3], ks[3], vs[3];
  WorkspaceLayout wl;
  if (int st = check_forward(args, 0, nullptr, H3ATTN_STAGE_PREPARE | H3ATTN_STAGE_ATTEND, qs, ks, vs, &wl, false))
    return st;
  if (cus <= 0) {
    if (int st = check_device()) return st;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return H3ATTN_ERR_HIP;
  }
  const h3::AttnPlan p = h3::plan_attention(attn_args(args, wl), cus);
  plan->kernel = p.resident;
  plan->query_tiles = p.query_tiles;
  plan->rows_per_tile = p.rows;
  plan->reserved = 0;
  plan->tiles = p.tiles;
  plan->whole_tiles = p.n_whole;
  plan->split_tiles = p.n_split;
  plan->split_blocks = p.n_blocks;
  plan->grid = p.grid;
  return H3ATTN_OK;
}

H3_API int h3attn_rmsnorm_scale_shift(const uint16_t* x, uint16_t* y, int32_t B, int32_t S, int32_t D,
                                      const float* norm_w, float eps, const uint16_t* scale,
                                      const uint16_t* shift, int32_t M, const int32_t* index, void* stream) {
  if (!x || !y || !scale || !shift) return H3ATTN_ERR_NULL_POINTER;
  if (B < 1 || S < 1 || M < 1 || D < 8 || D % 8 != 0 || D > h3::kScaleShiftMaxD) return H3ATTN_ERR_BAD_SHAPE;
  if ((int64_t)B * S >= (1ll << 31) || (int64_t)B * M >= (1ll << 31)) return H3ATTN_ERR_BAD_SHAPE;
  if (!std::isfinite(eps) || !(eps >= 0.f)) return H3ATTN_ERR_BAD_VALUE;
  if (!aligned16(x) || !aligned16(y) || !aligned16(scale) || !aligned16(shift)) return H3ATTN_ERR_BAD_ALIGNMENT;
  if (norm_w && !aligned16(norm_w)) return H3ATTN_ERR_BAD_ALIGNMENT;
  if (index && (reinterpret_cast<uintptr_t>(index) & 3u)) return H3ATTN_ERR_BAD_ALIGNMENT;
  const size_t xbytes = (size_t)B * S * D * 2, mbytes = (size_t)B * M * D * 2;
  const Range xr = range_of(x, xbytes), yr = range_of(y, xbytes);
  if (y != x && overlap(yr, xr)) return H3ATTN_ERR_ALIASING;
  if (overlap(yr, range_of(scale, mbytes)) || overlap(yr, range_of(shift, mbytes))) return H3ATTN_ERR_ALIASING;
  if (norm_w && overlap(yr, range_of(norm_w, (size_t)D * 4))) return H3ATTN_ERR_ALIASING;
  if (index && overlap(yr, range_of(index, (size_t)B * S * 4))) return H3ATTN_ERR_ALIASING;
  if (int st = check_device()) return st;
  h3::ScaleShiftArgs a;
  a.x = x;
  a.y = y;
  a.scale = scale;
  a.shift = shift;
  a.index = index;
  a.w = norm_w;
  a.eps = eps;
  a.rows = B * S;
  a.S = S;
  a.D = D;
  a.M = M;
  return status_from(h3::launch_scale_shift(a, reinterpret_cast<hipStream_t>(stream)));
}
