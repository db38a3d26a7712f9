// V packing for the attention forward on gfx950 (MI355X).
//
// The product P V of the attention (HunyuanVideo notes page "HunyuanVideo 模型结构与数学原理",
// section 5.2) contracts over keys, and an MFMA operand wants the contracted
// index contiguous in each lane: 8 keys of one channel.  V arrives token-major
// ([token][head][channel]), so without this pass every operand is gathered with
// two transposing LDS reads instead of one plain 16-byte read.  This kernel
// rewrites V once per call, tile by tile, channel-major
// (layout in hv_internal.h); the attention then streams 16 KB blocks into LDS
// and reads each operand with one ds_read_b128.  The pass moves 2 x |V| bytes
// through HBM, about 0.2 % of the attention's time at the largest sizes.
//
// One workgroup = (segment, head, 64-key tile), 256 threads:
//   1. each thread loads 64 bytes of one key row (keys past k_len are zeros)
//      and stores them to LDS as 16 channel pairs; the pair column is XORed
//      with bits 2, 4 and 5 of the key so that step 2 reads without bank
//      conflicts;
//   2. each thread builds two units of (channel pair, 8 positions): eight
//      32-bit LDS reads give the pair for 8 keys, which split into one 16-byte
//      row piece for each of the two channels.  Eight consecutive lanes write
//      one whole 128-byte row.
// Block 0 also zeroes the attention's work counter, which follows the packed
// tiles in the workspace (a kernel write, so no memset node is recorded when
// the caller captures the calls in a graph).
#include "hv_internal.h"

namespace hv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTileKeys = 64;
constexpr int kPairs = HV_HEAD_DIM / 2;  // 64 channel pairs = one 256-byte LDS row

// Pair-column XOR of a key row: bit 2 of the key -> bit 3, bits 4..5 -> 4..5.
__device__ __forceinline__ int pair_swz(int key) {
  return (((key >> 2) & 1) << 3) | (((key >> 4) & 3) << 4);
}

__global__ __launch_bounds__(kThreads) void v_pack_kernel(VtParams p) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[kTileKeys * kPairs];

  int si = 0;  // segment of this block (uniform scan over at most 64 entries)
  for (int i = 1; i < p.n_seg; ++i)
    if ((int)blockIdx.x >= p.seg[i].blk_begin) si = i;
  const VtSegment& sg = p.seg[si];
  const int rel = blockIdx.x - sg.blk_begin;
  const int head = rel / sg.ntiles;
  const int t = rel - head * sg.ntiles;
  const int tid = threadIdx.x;
  // the attention that follows on the stream hands out query blocks from here
  if (blockIdx.x == 0 && tid == 0) *p.counter = 0;

  // 1. key row r, channel pairs 16 q4 .. 16 q4 + 15 (four 16-byte chunks)
  {
    const int r = tid >> 2, q4 = tid & 3;
    const int key = t * kTileKeys + r;
    u32x4 d[4];
    if (key < sg.k_len) {
      const u32x4* src = reinterpret_cast<const u32x4*>(p.v + sg.k_off + (int64_t)key * p.kv_sl +
                                                         (int64_t)head * HV_HEAD_DIM) + 4 * q4;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = src[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = (u32x4){0u, 0u, 0u, 0u};
    }
    const int sw = pair_swz(r);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&tile[r * kPairs + ((16 * q4 + 4 * i) ^ sw)]) = d[i];
  }
  __syncthreads();

  // 2. unit u: row piece cp (positions 8cp .. 8cp+7) of channels 2j and 2j+1
  uint16_t* dst = p.vt + sg.vt_off + ((int64_t)head * sg.ntiles + t) * kVtTileElems;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int u = it * kThreads + tid;
    const int cp = u & 7, j = u >> 3;
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = kv_key_of_pos(8 * cp + e);
      w[e] = tile[key * kPairs + (j ^ pair_swz(key))];
    }
    u32x4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = (w[2 * i] & 0xffffu) | (w[2 * i + 1] << 16);
      hi[i] = (w[2 * i] >> 16) | (w[2 * i + 1] & 0xffff0000u);
    }
    *reinterpret_cast<u32x4*>(dst + (2 * j) * kTileKeys + 8 * cp) = lo;
    *reinterpret_cast<u32x4*>(dst + (2 * j + 1) * kTileKeys + 8 * cp) = hi;
  }
}

}  // namespace

hipError_t launch_v_pack(const VtParams& p, hipStream_t stream) {
  if (p.n_blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(v_pack_kernel, dim3((unsigned)p.n_blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hv
