// C ABI of libhvattn: argument validation, launch geometry, status codes.
// Every check runs on the host before the first HIP call, so each error path
// can be exercised without a GPU.
#include <math.h>
#include <string.h>

#include <mutex>

#include "hv_internal.h"

namespace {

constexpr int64_t kRowElems = (int64_t)HV_HEADS * HV_HEAD_DIM;  // 3072

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Validate a layout; on success *extent is the number of elements a tensor
// spans from its base pointer.
int check_layout(const hv_layout* lay, int64_t* extent) {
  if (!lay) return HV_ERR_INVALID_ARG;
  if (lay->batch < 0 || lay->seq_len < 0 || lay->heads <= 0 || lay->head_dim <= 0)
    return HV_ERR_INVALID_ARG;
  if (lay->heads != HV_HEADS || lay->head_dim != HV_HEAD_DIM) return HV_ERR_UNSUPPORTED;
  if (lay->batch > HV_MAX_BATCH || lay->seq_len > HV_MAX_SEQ) return HV_ERR_UNSUPPORTED;
  if (lay->stride_l < kRowElems || (lay->stride_l & 7) != 0) return HV_ERR_INVALID_ARG;
  // per-lane offsets inside a 64-row tile are 32-bit: 64 * 2 * stride_l < 2^32
  if (lay->stride_l > HV_MAX_TOKEN_STRIDE) return HV_ERR_UNSUPPORTED;
  if ((lay->stride_b & 7) != 0) return HV_ERR_INVALID_ARG;
  if (lay->batch > 1 && lay->stride_b < (int64_t)lay->seq_len * lay->stride_l)
    return HV_ERR_INVALID_ARG;
  if (lay->batch == 0 || lay->seq_len == 0) {
    *extent = 0;
  } else {
    *extent = (int64_t)(lay->batch - 1) * lay->stride_b +
              (int64_t)(lay->seq_len - 1) * lay->stride_l + kRowElems;
  }
  return HV_OK;
}

// Do two tensors with the same layout, based at a and b, share an element?
// Disjoint address ranges never do.  Otherwise, when every row starts at a
// multiple of stride_l (one batch entry, or stride_b a multiple of stride_l),
// the rows of b sit at a fixed offset r (mod stride_l) from the rows of a and
// the tensors are disjoint exactly when both row segments fit side by side:
// r >= 3072 and stride_l - r >= 3072 (e.g. q, k, v sliced from one fused
// [B][L][3][24][128] buffer).  Any other overlapping case counts as aliasing.
bool overlap(const void* a, const void* b, const hv_layout* lay, int64_t elems) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  const uintptr_t n = (uintptr_t)elems * sizeof(hv_bf16);
  if (!(x < y + n && y < x + n)) return false;
  const uintptr_t dbytes = x > y ? x - y : y - x;
  if (dbytes % sizeof(hv_bf16) != 0) return true;
  const int64_t d = (int64_t)(dbytes / sizeof(hv_bf16));
  const int64_t sl = lay->stride_l;
  if (lay->batch > 1 && lay->stride_b % sl != 0) return true;
  const int64_t r = d % sl;
  return !(r >= kRowElems && sl - r >= kRowElems);
}

// Do the byte ranges [a, a + na) and [b, b + nb) meet?
bool ranges_meet(const void* a, uintptr_t na, const void* b, uintptr_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na != 0 && nb != 0 && x < y + nb && y < x + na;
}

// Overlap of two bf16 tensors that may have different layouts: disjoint
// ranges never overlap; same layouts use the exact row-interleave test;
// anything else that shares bytes counts as overlapping.
bool overlap_any(const void* a, int64_t ea, const void* b, int64_t eb, const hv_layout* la,
                 const hv_layout* lb) {
  if (!ranges_meet(a, (uintptr_t)ea * 2, b, (uintptr_t)eb * 2)) return false;
  const bool same = la->batch == lb->batch && la->seq_len == lb->seq_len &&
                    la->stride_b == lb->stride_b && la->stride_l == lb->stride_l;
  return same ? overlap(a, b, la, ea) : true;
}

// The packed-V workspace of a forward call: enough bytes for the segments of
// p, 16-byte aligned and disjoint from the n byte ranges [ptr, ptr + len).
// A NULL workspace selects the in-place V path and needs nothing.
int check_workspace(const hv::AttnParams& p, const void* ws, int64_t ws_bytes,
                    const void* const* ptrs, const uintptr_t* lens, int n) {
  if (ws_bytes < 0) return HV_ERR_INVALID_ARG;
  if (ws == nullptr) return HV_OK;
  if (!aligned16(ws) || ws_bytes < hv::attn_workspace_bytes(p)) return HV_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (ptrs[i] && ranges_meet(ws, (uintptr_t)ws_bytes, ptrs[i], lens[i])) return HV_ERR_INVALID_ARG;
  return HV_OK;
}

float scale_log2(float softmax_scale) {
  float scale = softmax_scale;
  if (!(scale > 0.f) || !isfinite(scale)) scale = 1.0f / sqrtf((float)HV_HEAD_DIM);
  return (float)((double)scale * 1.4426950408889634);  // log2(e)
}

// Pointers, alignment and overlap of the backward's arguments (shared by the
// padded and the packed forms).  lse holds batch * 24 * seq_len floats; delta
// twice as many, followed by 256 bytes of work counters.
// A NULL delta is accepted only with own_delta == false (the allocation-free
// form, whose delta is the library's static scratch and meets no argument).
int check_bwd_buffers(const hv_bf16* q, const hv_bf16* k, const hv_bf16* v, const hv_bf16* out,
                      const hv_bf16* dout, const float* lse, hv_bf16* dq, hv_bf16* dk, hv_bf16* dv,
                      float* delta, const hv_layout* layout, bool own_delta = true) {
  int64_t extent = 0;
  int st = check_layout(layout, &extent);
  if (st != HV_OK) return st;
  const hv_bf16* ins[5] = {q, k, v, out, dout};
  hv_bf16* outs[3] = {dq, dk, dv};
  for (const hv_bf16* t : ins)
    if (!t || !aligned16(t)) return HV_ERR_INVALID_ARG;
  for (const hv_bf16* t : outs)
    if (!t || !aligned16(t)) return HV_ERR_INVALID_ARG;
  if (!lse || ((uintptr_t)lse & 3u) != 0) return HV_ERR_INVALID_ARG;
  if (own_delta && (!delta || ((uintptr_t)delta & 3u) != 0)) return HV_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i) {
    for (const hv_bf16* t : ins)
      if (overlap(outs[i], t, layout, extent)) return HV_ERR_INVALID_ARG;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j], layout, extent)) return HV_ERR_INVALID_ARG;
  }
  const uintptr_t vb = (uintptr_t)layout->batch * HV_HEADS * layout->seq_len * sizeof(float);
  // -D, -lse/scale, the two work counters (none of the caller's when the
  // library's scratch holds them)
  const uintptr_t db = own_delta ? 2 * vb + hv::kCounterBytes : 0;
  const uintptr_t tb = (uintptr_t)extent * sizeof(hv_bf16);
  if (ranges_meet(delta, db, lse, vb)) return HV_ERR_INVALID_ARG;
  for (const hv_bf16* t : ins)
    if (ranges_meet(delta, db, t, tb) || ranges_meet(lse, vb, t, tb)) return HV_ERR_INVALID_ARG;
  for (const hv_bf16* t : outs)
    if (ranges_meet(delta, db, t, tb) || ranges_meet(lse, vb, t, tb)) return HV_ERR_INVALID_ARG;
  return HV_OK;
}

// Fill the parts of BwdParams shared by both forms and launch.
int launch_bwd(hv::BwdParams& p, const hv_bf16* q, const hv_bf16* k, const hv_bf16* v,
               const hv_bf16* out, const hv_bf16* dout, const float* lse, hv_bf16* dq,
               hv_bf16* dk, hv_bf16* dv, float* delta, const hv_layout* layout,
               float softmax_scale, void* stream) {
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = out;
  p.dout = dout;
  p.lse = lse;
  p.delta = delta;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.stride_b = layout->stride_b;
  p.stride_l = layout->stride_l;
  p.v_hstride = layout->seq_len;
  p.batch = layout->batch;
  p.seq_len = layout->seq_len;
  p.scale_log2 = scale_log2(softmax_scale);
  p.scale = (float)((double)p.scale_log2 / 1.4426950408889634);
  const hipError_t e = hv::launch_attn_bwd(p, (hipStream_t)stream);
  return e == hipSuccess ? HV_OK : HV_ERR_HIP;
}

int check_grid(const hv_grid* g) {
  if (!g) return HV_ERR_INVALID_ARG;
  if (g->gt <= 0 || g->gh <= 0 || g->gw <= 0) return HV_ERR_INVALID_ARG;
  if (g->n_video != (int64_t)g->gt * g->gh * g->gw) return HV_ERR_INVALID_ARG;
  return HV_OK;
}

// The 64 rotation frequencies of a head, pair p = 0..63: pairs 0..7 form the
// time block (width 16), 8..35 height (56), 36..63 width (56);
// freq = theta^(-2j/width) with j the pair's index inside its block.
void rope_frequencies(float theta, float* freq) {
  const int widths[3] = {16, 56, 56};
  int pair = 0;
  for (int a = 0; a < 3; ++a)
    for (int j = 0; j < widths[a] / 2; ++j)
      freq[pair++] = (float)pow((double)theta, -2.0 * j / widths[a]);
}

// Segment table of the padded batch for the backward: entry b's queries
// attend to its first n_video + text_valid_len[b] keys.
int padded_bwd_segments(hv::BwdParams& p, const int32_t* text_valid_len, int64_t n_video,
                        const hv_layout* layout) {
  if (n_video < 0 || n_video > layout->seq_len) return HV_ERR_INVALID_ARG;
  memset(&p, 0, sizeof(p));
  const int64_t text_cap = layout->seq_len - n_video;
  const int L = layout->seq_len;
  for (int b = 0; b < layout->batch; ++b) {
    const int64_t valid = text_valid_len ? text_valid_len[b] : text_cap;
    if (valid < 0 || valid > text_cap) return HV_ERR_INVALID_ARG;
    if (n_video + valid < 1) return HV_ERR_INVALID_ARG;
    hv::BwdSegment& sg = p.seg[b];
    sg.q_off = sg.k_off = (int64_t)b * layout->stride_b;
    sg.v_off = (int64_t)b * HV_HEADS * L;
    sg.q_len = sg.k_rows = L;
    sg.k_len = (int32_t)(n_video + valid);
  }
  p.n_seg = layout->batch;
  return HV_OK;
}

// Scratch of hv_joint_attention_bwd_noalloc: what the delta workspace of
// hv_joint_attention_bwd holds (-D, -lse/scale, the two work counters), in a
// fixed array of device memory.  Every GPU the library runs on has its own
// copy at its own address, kept until the process ends; in host code the
// array's name is not a device address, so it is only reached through the
// per-device addresses below.
static __device__ __align__(256) unsigned char scratch[HV_NOALLOC_BWD_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch on the current device, looked up once per
// device (with that device current) and kept.
int bwd_scratch_of_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return HV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return HV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return HV_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return HV_OK;
}

}  // namespace

extern "C" {

int hv_version(void) { return 10200; }

int64_t hv_attention_workspace_bytes(int64_t n_keys, int32_t n_segments) {
  if (n_keys < 0 || n_segments < 0) return 0;
  const int64_t tiles = (n_keys + 63 * (int64_t)n_segments) / 64;
  return tiles > 0 ? tiles * HV_HEADS * hv::kVtTileElems * 2 + hv::kCounterBytes : 0;
}

const char* hv_status_string(int status) {
  switch (status) {
    case HV_OK: return "HV_OK: success";
    case HV_ERR_INVALID_ARG: return "HV_ERR_INVALID_ARG: invalid argument (NULL, size, range, alignment or overlap)";
    case HV_ERR_UNSUPPORTED: return "HV_ERR_UNSUPPORTED: unsupported shape (heads must be 24, head_dim 128, batch/seq within limits)";
    case HV_ERR_HIP: return "HV_ERR_HIP: HIP launch failed";
    default: return "unknown hv status";
  }
}

int hv_token_grid(int32_t frames, int32_t height, int32_t width, hv_grid* out) {
  if (!out) return HV_ERR_INVALID_ARG;
  if (frames <= 0 || height <= 0 || width <= 0) return HV_ERR_INVALID_ARG;
  if ((frames - 1) % 4 != 0) return HV_ERR_INVALID_ARG;
  if (height % 16 != 0 || width % 16 != 0) return HV_ERR_INVALID_ARG;
  hv_grid g;
  memset(&g, 0, sizeof(g));
  g.frames = frames;
  g.height = height;
  g.width = width;
  g.t_lat = (frames - 1) / 4 + 1;  // causal VAE keeps the first frame, then 4x in time
  g.h_lat = height / 8;            // 8x in space
  g.w_lat = width / 8;
  g.gt = g.t_lat;                  // 1x2x2 patches
  g.gh = g.h_lat / 2;
  g.gw = g.w_lat / 2;
  g.n_video = (int64_t)g.gt * g.gh * g.gw;
  *out = g;
  return HV_OK;
}

int hv_rope3d_apply(hv_bf16* q, hv_bf16* k, const hv_layout* layout, const hv_grid* grid,
                    float theta, void* stream) {
  int64_t extent = 0;
  int st = check_layout(layout, &extent);
  if (st != HV_OK) return st;
  st = check_grid(grid);
  if (st != HV_OK) return st;
  if (!(theta > 0.f) || !isfinite(theta)) return HV_ERR_INVALID_ARG;
  if (grid->n_video > layout->seq_len) return HV_ERR_INVALID_ARG;
  if (!q || !k) return HV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k)) return HV_ERR_INVALID_ARG;
  if (overlap(q, k, layout, extent)) return HV_ERR_INVALID_ARG;
  if (layout->batch == 0 || layout->seq_len == 0 || grid->n_video == 0) return HV_OK;

  hv::RopeParams p;
  memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.stride_b = layout->stride_b;
  p.stride_l = layout->stride_l;
  p.batch = layout->batch;
  p.n_video = (int32_t)grid->n_video;
  p.gh = grid->gh;
  p.gw = grid->gw;
  rope_frequencies(theta, p.freq);
  const hipError_t e = hv::launch_rope3d(p, (hipStream_t)stream);
  return e == hipSuccess ? HV_OK : HV_ERR_HIP;
}

int hv_qk_norm_rope3d_apply(hv_bf16* q, hv_bf16* k, const hv_layout* layout, const hv_grid* grid,
                            float theta, const hv_bf16* gamma_q, const hv_bf16* gamma_k,
                            const hv_bf16* gamma_q_text, const hv_bf16* gamma_k_text, float eps,
                            void* stream) {
  int64_t extent = 0;
  int st = check_layout(layout, &extent);
  if (st != HV_OK) return st;
  st = check_grid(grid);
  if (st != HV_OK) return st;
  if (!(theta > 0.f) || !isfinite(theta)) return HV_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !isfinite(eps)) return HV_ERR_INVALID_ARG;
  if (grid->n_video > layout->seq_len) return HV_ERR_INVALID_ARG;
  if (!q || !k || !gamma_q || !gamma_k) return HV_ERR_INVALID_ARG;
  if (!gamma_q_text) gamma_q_text = gamma_q;
  if (!gamma_k_text) gamma_k_text = gamma_k;
  if (!aligned16(q) || !aligned16(k) || !aligned16(gamma_q) || !aligned16(gamma_k) ||
      !aligned16(gamma_q_text) || !aligned16(gamma_k_text))
    return HV_ERR_INVALID_ARG;
  if (overlap(q, k, layout, extent)) return HV_ERR_INVALID_ARG;
  // the weights are read while q and k are written: they must lie outside both
  const uintptr_t gbytes = HV_HEAD_DIM * sizeof(hv_bf16);
  const uintptr_t tbytes = (uintptr_t)extent * sizeof(hv_bf16);
  const void* gammas[4] = {gamma_q, gamma_k, gamma_q_text, gamma_k_text};
  for (const void* g : gammas) {
    const uintptr_t x = (uintptr_t)g;
    for (const void* t : {(const void*)q, (const void*)k}) {
      const uintptr_t y = (uintptr_t)t;
      if (x < y + tbytes && y < x + gbytes) return HV_ERR_INVALID_ARG;
    }
  }
  if (layout->batch == 0 || layout->seq_len == 0) return HV_OK;

  hv::QkNormParams p;
  memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.gamma_q = gamma_q;
  p.gamma_k = gamma_k;
  p.gamma_q_text = gamma_q_text;
  p.gamma_k_text = gamma_k_text;
  p.stride_b = layout->stride_b;
  p.stride_l = layout->stride_l;
  p.batch = layout->batch;
  p.seq_len = layout->seq_len;
  p.n_video = (int32_t)grid->n_video;
  p.gh = grid->gh;
  p.gw = grid->gw;
  p.eps = eps;
  rope_frequencies(theta, p.freq);
  const hipError_t e = hv::launch_qknorm_rope3d(p, (hipStream_t)stream);
  return e == hipSuccess ? HV_OK : HV_ERR_HIP;
}

int hv_joint_attention_fwd(const hv_bf16* q, const hv_bf16* k, const hv_bf16* v,
                           const int32_t* text_valid_len, hv_bf16* out,
                           const hv_layout* layout, int64_t n_video, float softmax_scale,
                           void* workspace, int64_t workspace_bytes, void* stream) {
  int64_t extent = 0;
  int st = check_layout(layout, &extent);
  if (st != HV_OK) return st;
  if (n_video < 0 || n_video > layout->seq_len) return HV_ERR_INVALID_ARG;
  if (!q || !k || !v || !out) return HV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return HV_ERR_INVALID_ARG;
  if (overlap(out, q, layout, extent) || overlap(out, k, layout, extent) ||
      overlap(out, v, layout, extent))
    return HV_ERR_INVALID_ARG;
  if (layout->batch == 0 || layout->seq_len == 0) return HV_OK;

  hv::AttnParams p;
  memset(&p, 0, sizeof(p));
  const int64_t text_cap = layout->seq_len - n_video;
  for (int b = 0; b < layout->batch; ++b) {
    const int64_t valid = text_valid_len ? text_valid_len[b] : text_cap;
    if (valid < 0 || valid > text_cap) return HV_ERR_INVALID_ARG;
    if (n_video + valid < 1) return HV_ERR_INVALID_ARG;
    hv::AttnSegment& sg = p.seg[b];
    sg.q_off = sg.k_off = sg.o_off = (int64_t)b * layout->stride_b;
    sg.q_len = layout->seq_len;
    sg.k_len = (int32_t)(n_video + valid);
  }
  p.n_seg = layout->batch;
  {
    const void* ptrs[4] = {q, k, v, out};
    const uintptr_t n = (uintptr_t)extent * 2;
    const uintptr_t lens[4] = {n, n, n, n};
    st = check_workspace(p, workspace, workspace_bytes, ptrs, lens, 4);
    if (st != HV_OK) return st;
  }
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.vt = (uint16_t*)workspace;
  p.q_sl = p.kv_sl = p.o_sl = layout->stride_l;
  p.scale_log2 = scale_log2(softmax_scale);
  const hipError_t e = hv::launch_attn_fwd(p, (hipStream_t)stream);
  return e == hipSuccess ? HV_OK : HV_ERR_HIP;
}

int hv_attention_fwd_lse(const hv_bf16* q, const hv_layout* q_layout, const hv_bf16* k,
                         const hv_bf16* v, const hv_layout* kv_layout,
                         const int32_t* kv_valid_len, hv_bf16* out, float* lse,
                         float softmax_scale, void* workspace, int64_t workspace_bytes,
                         void* stream) {
  int64_t qext = 0, kvext = 0;
  int st = check_layout(q_layout, &qext);
  if (st != HV_OK) return st;
  st = check_layout(kv_layout, &kvext);
  if (st != HV_OK) return st;
  if (kv_layout->batch != q_layout->batch) return HV_ERR_INVALID_ARG;
  if (!q || !k || !v || !out) return HV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return HV_ERR_INVALID_ARG;
  if (lse && ((uintptr_t)lse & 3u) != 0) return HV_ERR_INVALID_ARG;
  const int B = q_layout->batch, Lq = q_layout->seq_len;
  if (overlap(out, q, q_layout, qext) || overlap_any(out, qext, k, kvext, q_layout, kv_layout) ||
      overlap_any(out, qext, v, kvext, q_layout, kv_layout))
    return HV_ERR_INVALID_ARG;
  if (lse) {
    const int64_t n = (int64_t)B * HV_HEADS * Lq;
    const uintptr_t lb = (uintptr_t)n * sizeof(float);
    if (ranges_meet(lse, lb, q, qext * 2) || ranges_meet(lse, lb, out, qext * 2) ||
        ranges_meet(lse, lb, k, kvext * 2) || ranges_meet(lse, lb, v, kvext * 2))
      return HV_ERR_INVALID_ARG;
  }
  if (B == 0 || Lq == 0) return HV_OK;

  hv::AttnParams p;
  memset(&p, 0, sizeof(p));
  for (int b = 0; b < B; ++b) {
    const int64_t n = kv_valid_len ? kv_valid_len[b] : kv_layout->seq_len;
    if (n < 1 || n > kv_layout->seq_len) return HV_ERR_INVALID_ARG;
    hv::AttnSegment& sg = p.seg[b];
    sg.q_off = sg.o_off = (int64_t)b * q_layout->stride_b;
    sg.k_off = (int64_t)b * kv_layout->stride_b;
    sg.lse_off = (int64_t)b * HV_HEADS * Lq;
    sg.q_len = Lq;
    sg.k_len = (int32_t)n;
  }
  p.n_seg = B;
  {
    const void* ptrs[5] = {q, k, v, out, lse};
    const uintptr_t lens[5] = {(uintptr_t)qext * 2, (uintptr_t)kvext * 2, (uintptr_t)kvext * 2,
                               (uintptr_t)qext * 2, (uintptr_t)B * HV_HEADS * Lq * sizeof(float)};
    st = check_workspace(p, workspace, workspace_bytes, ptrs, lens, 5);
    if (st != HV_OK) return st;
  }
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.vt = (uint16_t*)workspace;
  p.q_sl = p.o_sl = q_layout->stride_l;
  p.kv_sl = kv_layout->stride_l;
  p.lse_hstride = Lq;
  p.scale_log2 = scale_log2(softmax_scale);
  const hipError_t e = hv::launch_attn_fwd(p, (hipStream_t)stream);
  return e == hipSuccess ? HV_OK : HV_ERR_HIP;
}

int hv_joint_attention_varlen_fwd(const hv_bf16* q, const hv_bf16* k, const hv_bf16* v,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                  int32_t n_segments, hv_bf16* out, float* lse,
                                  const hv_layout* layout, float softmax_scale, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
  int64_t extent = 0;
  int st = check_layout(layout, &extent);
  if (st != HV_OK) return st;
  if (layout->batch != 1) return HV_ERR_INVALID_ARG;
  if (n_segments < 1 || n_segments > HV_MAX_SEGMENTS) return HV_ERR_INVALID_ARG;
  if (!cu_seqlens_q || !cu_seqlens_k) return HV_ERR_INVALID_ARG;
  if (!q || !k || !v || !out) return HV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return HV_ERR_INVALID_ARG;
  if (lse && ((uintptr_t)lse & 3u) != 0) return HV_ERR_INVALID_ARG;
  if (overlap(out, q, layout, extent) || overlap(out, k, layout, extent) ||
      overlap(out, v, layout, extent))
    return HV_ERR_INVALID_ARG;
  const int T = layout->seq_len;
  if (lse) {
    const uintptr_t lb = (uintptr_t)HV_HEADS * T * sizeof(float);
    if (ranges_meet(lse, lb, q, extent * 2) || ranges_meet(lse, lb, out, extent * 2) ||
        ranges_meet(lse, lb, k, extent * 2) || ranges_meet(lse, lb, v, extent * 2))
      return HV_ERR_INVALID_ARG;
  }
  hv::AttnParams p;
  memset(&p, 0, sizeof(p));
  if (cu_seqlens_q[0] < 0 || cu_seqlens_k[0] < 0) return HV_ERR_INVALID_ARG;
  for (int s = 0; s < n_segments; ++s) {
    const int32_t q0 = cu_seqlens_q[s], q1 = cu_seqlens_q[s + 1];
    const int32_t k0 = cu_seqlens_k[s], k1 = cu_seqlens_k[s + 1];
    if (q1 < q0 || k1 < k0 || q1 > T || k1 > T) return HV_ERR_INVALID_ARG;
    if (q1 > q0 && k1 == k0) return HV_ERR_INVALID_ARG;  // queries with no key
    hv::AttnSegment& sg = p.seg[s];
    sg.q_off = sg.o_off = (int64_t)q0 * layout->stride_l;
    sg.k_off = (int64_t)k0 * layout->stride_l;
    sg.lse_off = q0;
    sg.q_len = q1 - q0;
    sg.k_len = k1 - k0;
  }
  if (T == 0) return HV_OK;
  p.n_seg = n_segments;
  {
    const void* ptrs[5] = {q, k, v, out, lse};
    const uintptr_t n = (uintptr_t)extent * 2;
    const uintptr_t lens[5] = {n, n, n, n, (uintptr_t)HV_HEADS * T * sizeof(float)};
    st = check_workspace(p, workspace, workspace_bytes, ptrs, lens, 5);
    if (st != HV_OK) return st;
  }
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.vt = (uint16_t*)workspace;
  p.q_sl = p.kv_sl = p.o_sl = layout->stride_l;
  p.lse_hstride = T;
  p.scale_log2 = scale_log2(softmax_scale);
  const hipError_t e = hv::launch_attn_fwd(p, (hipStream_t)stream);
  return e == hipSuccess ? HV_OK : HV_ERR_HIP;
}

int hv_joint_attention_bwd(const hv_bf16* q, const hv_bf16* k, const hv_bf16* v,
                           const hv_bf16* out, const hv_bf16* dout, const float* lse,
                           const int32_t* text_valid_len, int64_t n_video, hv_bf16* dq,
                           hv_bf16* dk, hv_bf16* dv, float* delta, const hv_layout* layout,
                           float softmax_scale, void* stream) {
  int st = check_bwd_buffers(q, k, v, out, dout, lse, dq, dk, dv, delta, layout);
  if (st != HV_OK) return st;
  if (layout->batch == 0 || layout->seq_len == 0) {
    if (n_video < 0 || n_video > layout->seq_len) return HV_ERR_INVALID_ARG;
    return HV_OK;
  }
  hv::BwdParams p;
  st = padded_bwd_segments(p, text_valid_len, n_video, layout);
  if (st != HV_OK) return st;
  return launch_bwd(p, q, k, v, out, dout, lse, dq, dk, dv, delta, layout, softmax_scale, stream);
}

int hv_joint_attention_bwd_noalloc(const hv_bf16* q, const hv_bf16* k, const hv_bf16* v,
                                   const hv_bf16* out, const hv_bf16* dout, const float* lse,
                                   const int32_t* text_valid_len, int64_t n_video, hv_bf16* dq,
                                   hv_bf16* dk, hv_bf16* dv, const hv_layout* layout,
                                   float softmax_scale, void* stream) {
  int st = check_bwd_buffers(q, k, v, out, dout, lse, dq, dk, dv, nullptr, layout, false);
  if (st != HV_OK) return st;
  if (layout->batch == 0 || layout->seq_len == 0) {
    if (n_video < 0 || n_video > layout->seq_len) return HV_ERR_INVALID_ARG;
    return HV_OK;
  }
  hv::BwdParams p;
  st = padded_bwd_segments(p, text_valid_len, n_video, layout);
  if (st != HV_OK) return st;
  // -D and -lse/scale for every (batch, head, row), then the counters
  const int64_t need = 2 * (int64_t)layout->batch * HV_HEADS * layout->seq_len * (int64_t)sizeof(float) +
                       hv::kCounterBytes;
  if (need > HV_NOALLOC_BWD_SCRATCH_BYTES) return HV_ERR_UNSUPPORTED;
  float* scratch_ptr = nullptr;
  st = bwd_scratch_of_current_device(&scratch_ptr);
  if (st != HV_OK) return st;
  return launch_bwd(p, q, k, v, out, dout, lse, dq, dk, dv, scratch_ptr, layout, softmax_scale,
                    stream);
}

int hv_joint_attention_varlen_bwd(const hv_bf16* q, const hv_bf16* k, const hv_bf16* v,
                                  const hv_bf16* out, const hv_bf16* dout, const float* lse,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                  int32_t n_segments, hv_bf16* dq, hv_bf16* dk, hv_bf16* dv,
                                  float* delta, const hv_layout* layout, float softmax_scale,
                                  void* stream) {
  int st = check_bwd_buffers(q, k, v, out, dout, lse, dq, dk, dv, delta, layout);
  if (st != HV_OK) return st;
  if (layout->batch != 1) return HV_ERR_INVALID_ARG;
  if (n_segments < 1 || n_segments > HV_MAX_SEGMENTS) return HV_ERR_INVALID_ARG;
  if (!cu_seqlens_q || !cu_seqlens_k) return HV_ERR_INVALID_ARG;
  if (cu_seqlens_q[0] < 0 || cu_seqlens_k[0] < 0) return HV_ERR_INVALID_ARG;
  const int T = layout->seq_len;
  hv::BwdParams p;
  memset(&p, 0, sizeof(p));
  for (int s = 0; s < n_segments; ++s) {
    const int32_t q0 = cu_seqlens_q[s], q1 = cu_seqlens_q[s + 1];
    const int32_t k0 = cu_seqlens_k[s], k1 = cu_seqlens_k[s + 1];
    if (q1 < q0 || k1 < k0 || q1 > T || k1 > T) return HV_ERR_INVALID_ARG;
    if (q1 > q0 && k1 == k0) return HV_ERR_INVALID_ARG;  // queries with no key
    hv::BwdSegment& sg = p.seg[s];
    sg.q_off = (int64_t)q0 * layout->stride_l;
    sg.k_off = (int64_t)k0 * layout->stride_l;
    sg.v_off = q0;
    sg.q_len = q1 - q0;
    sg.k_rows = sg.k_len = k1 - k0;
  }
  if (T == 0) return HV_OK;
  p.n_seg = n_segments;
  return launch_bwd(p, q, k, v, out, dout, lse, dq, dk, dv, delta, layout, softmax_scale, stream);
}

int hv_attention_merge(const hv_bf16* const* outs, const float* const* lses, int32_t n_parts,
                       hv_bf16* out, float* lse_out, const hv_layout* layout, void* stream) {
  int64_t extent = 0;
  int st = check_layout(layout, &extent);
  if (st != HV_OK) return st;
  if (n_parts < 1 || n_parts > HV_MAX_MERGE_PARTS) return HV_ERR_INVALID_ARG;
  if (!outs || !lses || !out) return HV_ERR_INVALID_ARG;
  if (!aligned16(out)) return HV_ERR_INVALID_ARG;
  if (lse_out && ((uintptr_t)lse_out & 3u) != 0) return HV_ERR_INVALID_ARG;
  const int64_t nl = (int64_t)layout->batch * HV_HEADS * layout->seq_len;
  const uintptr_t lb = (uintptr_t)nl * sizeof(float);
  for (int i = 0; i < n_parts; ++i) {
    if (!outs[i] || !lses[i]) return HV_ERR_INVALID_ARG;
    if (!aligned16(outs[i]) || ((uintptr_t)lses[i] & 3u) != 0) return HV_ERR_INVALID_ARG;
    if (overlap(out, outs[i], layout, extent)) return HV_ERR_INVALID_ARG;
    if (ranges_meet(lses[i], lb, out, extent * 2)) return HV_ERR_INVALID_ARG;
    if (lse_out && (ranges_meet(lse_out, lb, lses[i], lb) ||
                    ranges_meet(lse_out, lb, outs[i], extent * 2)))
      return HV_ERR_INVALID_ARG;
  }
  if (lse_out && ranges_meet(lse_out, lb, out, extent * 2)) return HV_ERR_INVALID_ARG;
  if (layout->batch == 0 || layout->seq_len == 0) return HV_OK;

  hv::MergeParams p;
  memset(&p, 0, sizeof(p));
  for (int i = 0; i < n_parts; ++i) {
    p.outs[i] = outs[i];
    p.lses[i] = lses[i];
  }
  p.n_parts = n_parts;
  p.out = out;
  p.lse_out = lse_out;
  p.stride_b = layout->stride_b;
  p.stride_l = layout->stride_l;
  p.batch = layout->batch;
  p.seq_len = layout->seq_len;
  const hipError_t e = hv::launch_attn_merge(p, (hipStream_t)stream);
  return e == hipSuccess ? HV_OK : HV_ERR_HIP;
}

}  // extern "C"
