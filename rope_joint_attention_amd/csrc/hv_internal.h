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
