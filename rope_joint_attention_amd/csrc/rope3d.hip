// 3D rotary position embedding on the video rows of Q and K, in place.
//
// What is computed (HunyuanVideo notes page "HunyuanVideo 模型结构与数学原理",
// section 5.5): each 128-channel head is split (16, 56, 56) over the time,
// height and width axes and every adjacent channel pair (2j, 2j+1) of an axis
// block is rotated by pos_axis * theta^(-2j/d_axis).  Text rows are skipped.
//
// HBM-bound design for gfx950:
//   * one thread owns one (token, 16-byte channel chunk) and walks all 24
//     heads of q and k, so its 4 (cos, sin) pairs are computed once per token
//     and reused 48 times (sin/cos per (t, h, w) coordinate, fp32);
//   * 16 consecutive threads cover one head row (256 contiguous bytes), every
//     access is a 16-byte vector load or store;
//   * 8 heads of q and k (16 loads) are in flight per thread before any
//     rotation, which is enough outstanding traffic to stream HBM.
// Chunk c holds pairs 4c..4c+3; chunks 0-1 are the time block, 2-8 height,
// 9-15 width (block boundaries at pairs 8 and 36 fall on chunk boundaries).
#include "hv_internal.h"

namespace hv {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kHeads = HV_HEADS;
constexpr int kGroup = 8;  // heads per load batch

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, r);
}

// One 32-bit word holds a channel pair: x0 in the low half, x1 in the high.
__device__ __forceinline__ uint32_t rotate_pair(uint32_t w, float c, float s) {
  const float x0 = __uint_as_float(w << 16);
  const float x1 = __uint_as_float(w & 0xffff0000u);
  return pack_bf16(x0 * c - x1 * s, x0 * s + x1 * c);
}

__device__ __forceinline__ u32x4 rotate_chunk(u32x4 w, const float* c, const float* s) {
  u32x4 r;
  r.x = rotate_pair(w.x, c[0], s[0]);
  r.y = rotate_pair(w.y, c[1], s[1]);
  r.z = rotate_pair(w.z, c[2], s[2]);
  r.w = rotate_pair(w.w, c[3], s[3]);
  return r;
}

__global__ __launch_bounds__(kThreads) void rope3d_kernel(RopeParams p) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int chunk = (int)(gid & 15);
  const int64_t row = gid >> 4;  // b * n_video + n
  if (row >= (int64_t)p.batch * p.n_video) return;
  const int b = (int)(row / p.n_video);
  const int n = (int)(row - (int64_t)b * p.n_video);

  // patch coordinates of video token n (time-major, then rows, then columns)
  const int plane = p.gh * p.gw;
  const int t = n / plane;
  const int rem = n - t * plane;
  const int h = rem / p.gw;
  const int w = rem - h * p.gw;
  const int pos = chunk < 2 ? t : (chunk < 9 ? h : w);

  float c[4], s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float ang = (float)pos * p.freq[4 * chunk + i];
    sincosf(ang, &s[i], &c[i]);
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
      qp[(g + i) * 16] = rotate_chunk(vq[i], c, s);
      kp[(g + i) * 16] = rotate_chunk(vk[i], c, s);
    }
  }
}

}  // namespace

hipError_t launch_rope3d(const RopeParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.batch * p.n_video * 16;
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(rope3d_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hv
