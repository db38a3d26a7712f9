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

// ---- joint attention forward ----------------------------------------------
struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  int64_t stride_b;    // elements
  int64_t stride_l;    // elements
  int32_t batch;
  int32_t seq_len;
  int32_t n_qblocks;   // query blocks per (batch, head)
  int32_t n_blocks;    // batch * heads * n_qblocks
  float scale_log2;    // softmax scale * log2(e)
  int32_t pad_;
  int32_t lk[HV_MAX_BATCH];  // valid keys per batch entry (n_video + valid text)
};

hipError_t launch_attn_fwd(AttnParams& p, hipStream_t stream);

}  // namespace hv
