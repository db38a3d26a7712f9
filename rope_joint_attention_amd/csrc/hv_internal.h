// Internal declarations shared by the libhvattn translation units.
// Kernel launchers take already-validated arguments; validation lives in
// hvattn_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hvattn.h"

namespace hv {

// ---- 3D RoPE --------------------------------------------------------------
// 64 rotation frequencies per head, one per channel pair p = 0..63:
// pairs 0..7 belong to the time block (d = 16), 8..35 to height (d = 56),
// 36..63 to width (d = 56); freq[p] = theta^(-2j/d) with j the pair index
// inside its block.  Computed on the host in double, stored as float.
struct RopeParams {
  uint16_t* q;
  uint16_t* k;
  int64_t stride_b;  // elements
  int64_t stride_l;  // elements
  int32_t batch;
  int32_t n_video;
  int32_t gh;        // token grid height
  int32_t gw;        // token grid width
  float freq[64];
};

hipError_t launch_rope3d(const RopeParams& p, hipStream_t stream);

// ---- QK-norm + 3D RoPE prologue ---------------------------------------------
// Per-head RMSNorm of every row of q and k (video rows with gamma_q/gamma_k,
// text rows with gamma_q_text/gamma_k_text, which the host sets to the video
// weights when the caller passes none), then the rotation of RopeParams on
// the video rows.
struct QkNormParams {
  uint16_t* q;
  uint16_t* k;
  const uint16_t* gamma_q;
  const uint16_t* gamma_k;
  const uint16_t* gamma_q_text;
  const uint16_t* gamma_k_text;
  int64_t stride_b;  // elements
  int64_t stride_l;  // elements
  int32_t batch;
  int32_t seq_len;
  int32_t n_video;
  int32_t gh;        // token grid height
  int32_t gw;        // token grid width
  float eps;
  float freq[64];    // as in RopeParams
};

hipError_t launch_qknorm_rope3d(const QkNormParams& p, hipStream_t stream);

// ---- attention forward ------------------------------------------------------
// The kernel works on segments: segment s holds q_len query rows starting at
// element q_off of q (token stride q_sl) and k_len keys starting at element
// k_off of k and v (token stride kv_sl); its output rows start at element
// o_off of out (stride o_sl).  A batch entry of the padded joint layout, a
// packed clip and a (query rows, K/V block) pair of a ring step are all one
// segment.  Query blocks of 256 rows are numbered segment by segment, head by
// head: segment s owns logical blocks [blk_begin, blk_begin + 24 * nqb).
constexpr int kMaxSegments = HV_MAX_SEGMENTS;

struct AttnSegment {
  int64_t q_off;     // elements
  int64_t k_off;     // elements (k and v)
  int64_t o_off;     // elements
  int64_t lse_off;   // index of (head 0, row 0) in lse
  int64_t vt_off;    // elements: the segment's packed V in the workspace
  int32_t q_len;     // query rows
  int32_t k_len;     // keys, >= 1 when q_len > 0
  int32_t blk_begin; // first logical block
  int32_t nqb;       // query blocks per head
};

// Packed V (optional workspace): for every segment with query rows, head h
// and 64-key tile t, a contiguous 16 KB block at
//   vt + vt_off + (h * ntiles + t) * 8192 elements,  ntiles = ceil(k_len / 64),
// followed by 256 bytes that hold the attention's work counter,
// holding the tile channel-major: row d (0..127) is 64 bf16, position p of
// the row is key 64t + kv_key_of_pos(p) of channel d; keys >= k_len are 0.
// Inside each group of 16 keys the positions swap bits 2 and 3 of the key
// index, which puts the 8 keys one lane needs for an MFMA operand (the order
// the probabilities come out of the score MFMA) next to each other.
constexpr int kVtTileElems = 64 * HV_HEAD_DIM;  // 8192 elements = 16 KB

__host__ __device__ constexpr int kv_key_of_pos(int p) {
  return (p & ~15) | (p & 3) | (((p >> 3) & 1) << 2) | (((p >> 2) & 1) << 3);
}

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;          // natural-log log-sum-exp per (head, row); may be null
  uint16_t* vt;        // packed V workspace; null: V is read in place
  int* counter;        // next query block of the persistent workgroups (packed path)
  int64_t q_sl;        // token strides, elements
  int64_t kv_sl;
  int64_t o_sl;
  int64_t lse_hstride; // lse elements between heads
  int32_t n_seg;
  int32_t n_blocks;    // total logical blocks
  float scale_log2;    // softmax scale * log2(e)
  int32_t pad_;
  AttnSegment seg[kMaxSegments];
};

// Workspace bytes that the segments of p need: packed V (segments without
// query rows need none) and the 256-byte work counter.
constexpr int64_t kCounterBytes = 256;
inline int64_t attn_workspace_bytes(const AttnParams& p) {
  int64_t tiles = 0;
  for (int i = 0; i < p.n_seg; ++i)
    if (p.seg[i].q_len > 0) tiles += (p.seg[i].k_len + 63) / 64;
  return tiles > 0 ? tiles * HV_HEADS * kVtTileElems * 2 + kCounterBytes : 0;
}

// Fills blk_begin / nqb / n_blocks from q_len (and vt_off when p.vt is set),
// packs V into p.vt when it is set, and launches the attention.
hipError_t launch_attn_fwd(AttnParams& p, hipStream_t stream);

// ---- V packing for the attention forward --------------------------------------
struct VtSegment {
  int64_t k_off;     // elements of v
  int64_t vt_off;    // elements of vt
  int32_t k_len;
  int32_t ntiles;    // ceil(k_len / 64)
  int32_t blk_begin; // first block: blocks run head-major over the tiles
  int32_t pad_;
};

struct VtParams {
  const uint16_t* v;
  uint16_t* vt;
  int* counter;        // the attention's work counter: set to zero here
  int64_t kv_sl;       // token stride of v, elements
  int32_t n_seg;
  int32_t n_blocks;
  VtSegment seg[kMaxSegments];
};

hipError_t launch_v_pack(const VtParams& p, hipStream_t stream);

// ---- merge of partial attention results -------------------------------------
// n_parts outputs over disjoint key blocks (same layout as out) and their
// log-sum-exps ([batch][24][seq_len] fp32) combine into out / lse_out.
struct MergeParams {
  const uint16_t* outs[HV_MAX_MERGE_PARTS];
  const float* lses[HV_MAX_MERGE_PARTS];
  uint16_t* out;
  float* lse_out;      // may be null
  int64_t stride_b;    // elements
  int64_t stride_l;    // elements
  int32_t batch;
  int32_t seq_len;
  int32_t n_parts;
  int32_t pad_;
};

hipError_t launch_attn_merge(const MergeParams& p, hipStream_t stream);

// ---- attention backward -----------------------------------------------------
// Segments as in the forward: segment s has q_len query rows from element
// q_off (q, o, dout, dq) and k_rows key rows from element k_off (k, v, dk,
// dv), of which the first k_len are valid keys; the rest get zero dk, dv.
// Its lse / delta values sit at v_off + head * v_hstride + row.
struct BwdSegment {
  int64_t q_off;
  int64_t k_off;
  int64_t v_off;
  int32_t q_len;
  int32_t k_rows;
  int32_t k_len;     // >= 1 when q_len > 0
  int32_t q_blk;     // first block of the dq kernel
  int32_t k_blk;     // first block of the dkdv kernel
  int32_t nqb;       // dq blocks per head
  int32_t nkb;       // dkdv blocks per head
  int32_t pad_;
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;    // natural log, per (head, row) as the segments place it
  float* delta;        // -D, same placement, written by the first kernel
  float* nls;          // -lse / scale, same placement, written by the first kernel
  int* counters;       // next block of the dK/dV [0] and dQ [1] persistent workgroups
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int64_t stride_b;    // elements, shared by all bf16 tensors (delta pass)
  int64_t stride_l;
  int64_t v_hstride;   // lse / delta elements between heads
  int32_t batch;       // the delta pass covers batch x seq_len rows,
  int32_t seq_len;     // delta[(b * 24 + h) * seq_len + n]
  float scale;         // softmax scale
  float scale_log2;    // scale * log2(e)
  int32_t n_seg;
  int32_t n_q_blocks;  // dq workgroups
  int32_t n_kv_blocks; // dkdv workgroups
  int32_t pad_;
  BwdSegment seg[kMaxSegments];
};

hipError_t launch_attn_bwd(BwdParams& p, hipStream_t stream);

// Kernel arguments are passed by value; keep them within 4 KB.
static_assert(sizeof(AttnParams) <= 4096, "attention kernel arguments exceed 4 KB");
static_assert(sizeof(BwdParams) <= 4096, "backward kernel arguments exceed 4 KB");
static_assert(sizeof(MergeParams) <= 4096, "merge kernel arguments exceed 4 KB");
static_assert(sizeof(VtParams) <= 4096, "V packing kernel arguments exceed 4 KB");

}  // namespace hv
