// Exact merge of attention results computed over disjoint key blocks.
//
// What is computed (HunyuanVideo notes page "HunyuanVideo 模型结构与数学原理",
// section 9.2: Ring Attention keeps each rank's query rows and passes K/V
// blocks around the ring, so every rank holds one partial result per block):
// for parts i with outputs O_i and log-sum-exps lse_i of one (row, head),
//     lse = log sum_i e^(lse_i),   O = sum_i e^(lse_i - lse) O_i,
// which is the softmax over the union of the blocks, because part i's
// unnormalised numerator is e^(lse_i) O_i.  fp32 arithmetic, O rounded to
// bf16 once.
//
// HBM-bound: one thread per (row, head, 16-byte channel chunk); 16 lanes share
// a head row, read its P log-sum-exps (one broadcast load each) and the P
// 16-byte chunks of their channels, all loads issued before any arithmetic.
#include "hv_internal.h"

namespace hv {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, r);
}

template <int P>
__device__ __forceinline__ void merge_chunk(const MergeParams& p, int64_t row_off, int64_t lse_idx,
                                            int64_t elem, bool write_lse) {
  float l[P];
  u32x4 w[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    l[i] = p.lses[i][lse_idx];
    w[i] = *reinterpret_cast<const u32x4*>(p.outs[i] + row_off + elem);
  }
  float top = l[0];
#pragma unroll
  for (int i = 1; i < P; ++i) top = fmaxf(top, l[i]);
  float tot = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const float wt = __expf(l[i] - top);
    tot += wt;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = fmaf(wt, __uint_as_float(w[i][j] << 16), acc[2 * j]);
      acc[2 * j + 1] = fmaf(wt, __uint_as_float(w[i][j] & 0xffff0000u), acc[2 * j + 1]);
    }
  }
  const float inv = 1.0f / tot;
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = pack_bf16(acc[2 * j] * inv, acc[2 * j + 1] * inv);
  *reinterpret_cast<u32x4*>(p.out + row_off + elem) = r;
  if (write_lse) p.lse_out[lse_idx] = top + __logf(tot);
}

__global__ __launch_bounds__(kThreads) void attn_merge_kernel(MergeParams p) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int chunk = (int)(gid & 15);
  const int64_t rh = gid >> 4;  // (b * seq_len + n) * 24 + head
  if (rh >= (int64_t)p.batch * p.seq_len * HV_HEADS) return;
  const int head = (int)(rh % HV_HEADS);
  const int64_t row = rh / HV_HEADS;
  const int b = (int)(row / p.seq_len);
  const int n = (int)(row - (int64_t)b * p.seq_len);
  const int64_t row_off = (int64_t)b * p.stride_b + (int64_t)n * p.stride_l;
  const int64_t lse_idx = ((int64_t)b * HV_HEADS + head) * p.seq_len + n;
  const int64_t elem = (int64_t)head * HV_HEAD_DIM + chunk * 8;
  const bool wl = p.lse_out != nullptr && chunk == 0;
  switch (p.n_parts) {
#define HV_MERGE_CASE(P) case P: merge_chunk<P>(p, row_off, lse_idx, elem, wl); break;
    HV_MERGE_CASE(1) HV_MERGE_CASE(2) HV_MERGE_CASE(3) HV_MERGE_CASE(4)
    HV_MERGE_CASE(5) HV_MERGE_CASE(6) HV_MERGE_CASE(7) HV_MERGE_CASE(8)
    HV_MERGE_CASE(9) HV_MERGE_CASE(10) HV_MERGE_CASE(11) HV_MERGE_CASE(12)
    HV_MERGE_CASE(13) HV_MERGE_CASE(14) HV_MERGE_CASE(15) HV_MERGE_CASE(16)
#undef HV_MERGE_CASE
    default: break;
  }
}

}  // namespace

hipError_t launch_attn_merge(const MergeParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.batch * p.seq_len * HV_HEADS * 16;
  const int64_t blocks = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hv
