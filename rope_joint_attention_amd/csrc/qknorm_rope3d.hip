// QK-norm prologue of the joint attention, in place: per-head RMSNorm of every
// row of Q and K, then the 3D rotary embedding of the video rows.
//
// What is computed (HunyuanVideo notes page "HunyuanVideo 模型结构与数学原理"):
//   section 5.4: each 128-channel head x of Q and K becomes
//       gamma * x / sqrt(mean(x^2) + eps);
//   section 5.2: the double-stream blocks keep separate weights for the video
//       and text streams, so video rows take gamma_video and text rows
//       gamma_text (one vector per tensor);
//   section 5.5: video rows are then rotated exactly as hv_rope3d_apply does
//       (channel blocks 16/56/56 for t/h/w, adjacent pairs, theta^(-2j/d)).
// The normalised value is kept in fp32 and rounded to bf16 once, after the
// rotation.
//
// HBM-bound design for gfx950 (one read and one write of every Q and K row,
// the same traffic as the RoPE alone, which it replaces):
//   * one thread owns one (row, 16-byte channel chunk) and walks all 24 heads
//     of q and k; 16 consecutive lanes cover one 256-byte head row, so the
//     sum of squares of a head is 16 in-lane partial sums reduced with four
//     DPP steps inside a 16-lane row (quad swaps, half mirror, mirror) and
//     every lane of the row ends with the total;
//   * 8 heads of q and k (16 vector loads) are in flight per thread before
//     the first reduction;
//   * the weights of the row's stream (8 channels each of gamma_q, gamma_k)
//     and, for video rows, the 4 (cos, sin) pairs of the chunk are loaded or
//     computed once per thread and reused over the 24 heads.
#include "hv_internal.h"

namespace hv {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kHeads = HV_HEADS;
constexpr int kGroup = 8;  // heads per load batch

// DPP controls (GFX9 encoding): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int Ctrl>
__device__ __forceinline__ float dpp_sum_step(float v) {
  const int o = __builtin_amdgcn_mov_dpp(__float_as_int(v), Ctrl, 0xF, 0xF, true);
  return v + __int_as_float(o);
}

// Sum over the 16 lanes of a DPP row; every lane receives the total.
__device__ __forceinline__ float row16_sum(float v) {
  v = dpp_sum_step<kDppQuadXor1>(v);
  v = dpp_sum_step<kDppQuadXor2>(v);
  v = dpp_sum_step<kDppHalfMirror>(v);
  return dpp_sum_step<kDppMirror>(v);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float chunk_sumsq(u32x4 w) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = lo(w[i]), b = hi(w[i]);
    s = fmaf(a, a, s);
    s = fmaf(b, b, s);
  }
  return s;
}

// Scale the chunk's 8 channels by inv * gamma, rotate its 4 pairs when
// `rotate`, round to bf16.
__device__ __forceinline__ u32x4 norm_chunk(u32x4 w, float inv, const float* g, bool rotate,
                                            const float* c, const float* s) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = lo(w[i]) * inv * g[2 * i];
    const float x1 = hi(w[i]) * inv * g[2 * i + 1];
    if (rotate)
      r[i] = pack_bf16(x0 * c[i] - x1 * s[i], x0 * s[i] + x1 * c[i]);
    else
      r[i] = pack_bf16(x0, x1);
  }
  return r;
}

__global__ __launch_bounds__(kThreads) void qknorm_rope3d_kernel(QkNormParams p) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int chunk = (int)(gid & 15);
  const int64_t row = gid >> 4;  // b * seq_len + n
  // Whole 16-lane rows leave together, so the DPP rows below are complete.
  if (row >= (int64_t)p.batch * p.seq_len) return;
  const int b = (int)(row / p.seq_len);
  const int n = (int)(row - (int64_t)b * p.seq_len);
  const bool video = n < p.n_video;

  // this chunk's 8 weights of the row's stream
  float gq[8], gk[8];
  {
    const uint16_t* gqp = (video ? p.gamma_q : p.gamma_q_text) + chunk * 8;
    const uint16_t* gkp = (video ? p.gamma_k : p.gamma_k_text) + chunk * 8;
    const u32x4 wq = *reinterpret_cast<const u32x4*>(gqp);
    const u32x4 wk = *reinterpret_cast<const u32x4*>(gkp);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gq[2 * i] = lo(wq[i]);
      gq[2 * i + 1] = hi(wq[i]);
      gk[2 * i] = lo(wk[i]);
      gk[2 * i + 1] = hi(wk[i]);
    }
  }

  float c[4] = {1.f, 1.f, 1.f, 1.f}, s[4] = {0.f, 0.f, 0.f, 0.f};
  if (video) {
    // patch coordinates of video token n (time-major, then rows, then columns);
    // chunk c holds pairs 4c..4c+3: chunks 0-1 time, 2-8 height, 9-15 width
    const int plane = p.gh * p.gw;
    const int t = n / plane;
    const int rem = n - t * plane;
    const int h = rem / p.gw;
    const int w = rem - h * p.gw;
    const int pos = chunk < 2 ? t : (chunk < 9 ? h : w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ang = (float)pos * p.freq[4 * chunk + i];
      sincosf(ang, &s[i], &c[i]);
    }
  }

  const int64_t base = (int64_t)b * p.stride_b + (int64_t)n * p.stride_l + chunk * 8;
  u32x4* qp = reinterpret_cast<u32x4*>(p.q + base);
  u32x4* kp = reinterpret_cast<u32x4*>(p.k + base);
  // head stride is 128 bf16 = 16 vectors of 16 bytes
#pragma unroll
  for (int g = 0; g < kHeads; g += kGroup) {
    u32x4 vq[kGroup], vk[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      vq[i] = qp[(g + i) * 16];
      vk[i] = kp[(g + i) * 16];
    }
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const float ssq = row16_sum(chunk_sumsq(vq[i]));
      const float ssk = row16_sum(chunk_sumsq(vk[i]));
      const float invq = rsqrtf(fmaf(ssq, 1.0f / HV_HEAD_DIM, p.eps));
      const float invk = rsqrtf(fmaf(ssk, 1.0f / HV_HEAD_DIM, p.eps));
      qp[(g + i) * 16] = norm_chunk(vq[i], invq, gq, video, c, s);
      kp[(g + i) * 16] = norm_chunk(vk[i], invk, gk, video, c, s);
    }
  }
}

}  // namespace

hipError_t launch_qknorm_rope3d(const QkNormParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.batch * p.seq_len * 16;
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(qknorm_rope3d_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hv
