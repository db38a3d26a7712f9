// Joint [video; text] attention forward for gfx950 (MI355X).
//
// What is computed (HunyuanVideo notes page "HunyuanVideo 模型结构与数学原理",
// section 5.2): per (batch, head), O = softmax(Q K^T / sqrt(128)) V over the
// concatenated sequence, with text keys beyond the valid length left out.
// The attention is exact (section 9.1 stresses that IO-aware tiling does not
// change the result), so the kernel is a tiled exact softmax: scores are
// never written to memory.
//
// Work decomposition
//   * one workgroup = (batch, head, 256 query rows); 8 waves, 32 rows each,
//     two waves per SIMD so one wave's softmax overlaps the other's MFMA;
//   * key/value tiles of 64 rows are staged through LDS, double buffered:
//     the next tile's global loads are issued before the current tile's
//     math and written to the other LDS buffer after it;
//   * workgroup ids are remapped so that consecutive query blocks of one
//     (batch, head) run on the same XCD and share its L2 for K/V.
//
// Per wave and tile, in MFMA 32x32x16 bf16 (fp32 accumulate):
//   S^T (64 keys x 32 queries) = K_tile * Q^T   -- lane l owns query l%32, so
//       row statistics are 32 in-register values plus one exchange between
//       the two 32-lane halves (v_permlane32_swap);
//   online softmax in the log2 domain with exp2; the running reference m is
//       only raised when a row maximum exceeds it by more than 8 (factor 256),
//       which keeps every probability <= 256 and the result exact, while
//       skipping almost all accumulator rescales;
//   O^T (128 channels x 32 queries) += V^T_tile * P^T -- P^T stays in the
//       registers the softmax produced (converted to bf16); V is written to
//       LDS transposed, with the key order inside each 16-key group permuted
//       to match the register layout of P^T.
// The padded-key mask is a loop bound plus a predicate on the last tile;
// K and V rows at or beyond the valid length are never read (zeros are
// staged instead), so garbage in padded rows cannot reach the output.
#include "hv_internal.h"

namespace hv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = HV_HEAD_DIM;  // 128
constexpr int BN = 64;          // keys per tile
constexpr int NW = 8;           // waves per workgroup
constexpr int QPW = 32;         // query rows per wave
constexpr int BM = NW * QPW;    // 256 query rows per workgroup
constexpr int NT = NW * 64;     // 512 threads
constexpr int KS = D + 8;       // K tile row stride in LDS (bf16): 272 B, conflict-free reads
constexpr int VS = BN + 8;      // V^T tile row stride in LDS (bf16): 144 B
constexpr float kRescaleLog2 = 8.0f;

// Position of key `key` (0..63 inside a tile) in a V^T row.  Inside every
// group of 16 keys, bits 2 and 3 of the key index are swapped: the P^T
// operand register of lane-half h, slot e holds key 8*(e/4) + 4h + e%4 of its
// 16-key group, so V^T must hold that key at position 8h + e.
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);  // nearest even
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& s, int base) {
  u32x4 w;
  w.x = pack_bf16(s[base + 0], s[base + 1]);
  w.y = pack_bf16(s[base + 2], s[base + 3]);
  w.z = pack_bf16(s[base + 4], s[base + 5]);
  w.w = pack_bf16(s[base + 6], s[base + 7]);
  return __builtin_bit_cast(bf16x8, w);
}

struct Stage {
  u32x4 k0, k1, v0, v1;
};

__global__ __launch_bounds__(NT, 1) void attn_fwd_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * VS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous range of (batch, head, query-block) ids so that the query
  // blocks resident on one XCD stream the same K/V through its L2.
  const int nb = p.n_blocks;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int per = nb >> 3, extra = nb & 7;
  const int logical = xcd * per + min(xcd, extra) + (bid >> 3);
  const int qb = logical % p.n_qblocks;
  const int bh = logical / p.n_qblocks;
  const int head = bh % HV_HEADS;
  const int b = bh / HV_HEADS;

  const int L = p.seq_len;
  const int Lk = p.lk[b];
  const int64_t sl = p.stride_l;
  const int64_t hbase = (int64_t)b * p.stride_b + (int64_t)head * D;
  const uint16_t* Kg = p.k + hbase;
  const uint16_t* Vg = p.v + hbase;

  // Q^T operand: lane holds query row q0 + l32, channels 16*kc + 8*hh .. +7.
  const int q0 = qb * BM + wave * QPW;
  const int qrow = min(q0 + l32, L - 1);  // rows past the end are computed, never stored
  bf16x8 qf[8];
  {
    const uint16_t* qptr = p.q + hbase + (int64_t)qrow * sl + hh * 8;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) qf[kc] = *reinterpret_cast<const bf16x8*>(qptr + kc * 16);
  }

  // Staging roles.  K: thread -> rows (tid/16, tid/16 + 32), 16-byte chunk tid%16
  // (coalesced).  V: lane -> key pair (lane%32), channel chunk 2*wave + lane/32,
  // so that the transposed LDS writes of a wave cover 32 consecutive dwords
  // in two rows 8 channels apart (no bank conflicts).
  const int k_row = tid >> 4;
  const int k_c = tid & 15;
  const int v_kp = lane & 31;
  const int v_c = wave * 2 + hh;

  auto load_stage = [&](int tile, Stage& st) {
    const int kb = tile * BN;
    const int r0 = kb + k_row, r1 = r0 + 32;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    st.k0 = r0 < Lk ? *reinterpret_cast<const u32x4*>(Kg + (int64_t)r0 * sl + k_c * 8) : zero;
    st.k1 = r1 < Lk ? *reinterpret_cast<const u32x4*>(Kg + (int64_t)r1 * sl + k_c * 8) : zero;
    const int v0r = kb + 2 * v_kp, v1r = v0r + 1;
    st.v0 = v0r < Lk ? *reinterpret_cast<const u32x4*>(Vg + (int64_t)v0r * sl + v_c * 8) : zero;
    st.v1 = v1r < Lk ? *reinterpret_cast<const u32x4*>(Vg + (int64_t)v1r * sl + v_c * 8) : zero;
  };

  auto store_stage = [&](int buf, const Stage& st) {
    *reinterpret_cast<u32x4*>(&sK[buf][k_row * KS + k_c * 8]) = st.k0;
    *reinterpret_cast<u32x4*>(&sK[buf][(k_row + 32) * KS + k_c * 8]) = st.k1;
    uint32_t* vt = reinterpret_cast<uint32_t*>(&sV[buf][0]);
    const int col = vt_pos(2 * v_kp);  // even: keys 2kp, 2kp+1 are adjacent
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = st.v0[e >> 1], c = st.v1[e >> 1];
      const uint32_t w = (e & 1) ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
      vt[((8 * v_c + e) * VS + col) >> 1] = w;
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;
  float m_run = -INFINITY;  // running reference, log2 domain
  float l_run = 0.f;        // this lane's share of the softmax denominator
  const float c2 = p.scale_log2;

  const int ntiles = (Lk + BN - 1) / BN;
  Stage st;
  load_stage(0, st);
  store_stage(0, st);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool has_next = t + 1 < ntiles;
    if (has_next) load_stage(t + 1, st);

    // ---- S^T = K Q^T for the two 32-key halves of the tile
    f32x16 s0, s1;
#pragma unroll
    for (int v = 0; v < 16; ++v) { s0[v] = 0.f; s1[v] = 0.f; }
    const uint16_t* kt = &sK[buf][0];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kt + l32 * KS + kc * 16 + hh * 8);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kt + (l32 + 32) * KS + kc * 16 + hh * 8);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kc], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kc], s1, 0, 0, 0);
    }

    // ---- padded keys of the last tile: s = -inf
    const int lim = Lk - t * BN;
    if (lim < BN) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = 8 * (v >> 2) + 4 * hh + (v & 3);
        if (key >= lim) s0[v] = -INFINITY;
        if (key + 32 >= lim) s1[v] = -INFINITY;
      }
    }

    // ---- row maximum (16 + 16 values in lane, then across the halves)
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(s0[v], s1[v]));
    mx = max_across_halves(mx) * c2;

    const bool need = mx > m_run + kRescaleLog2;
    if (__any(need)) {
      const float m_new = need ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }

    // ---- probabilities p = 2^(s*c2 - m)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s0[v] = __builtin_amdgcn_exp2f(fmaf(s0[v], c2, -m_run));
      s1[v] = __builtin_amdgcn_exp2f(fmaf(s1[v], c2, -m_run));
      l_run += s0[v] + s1[v];
    }
    bf16x8 pb[4];
    pb[0] = to_bf16x8(s0, 0);
    pb[1] = to_bf16x8(s0, 8);
    pb[2] = to_bf16x8(s1, 0);
    pb[3] = to_bf16x8(s1, 8);

    // ---- O^T += V^T P^T, 16 keys per MFMA
    const uint16_t* vt = &sV[buf][0];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (dt * 32 + l32) * VS + mm * 16 + hh * 8);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[mm], o[dt], 0, 0, 0);
      }
    }

    if (has_next) store_stage(buf ^ 1, st);
    __syncthreads();
  }

  // ---- epilogue: O / l, round to bf16, store rows that exist
  const float inv = 1.0f / sum_across_halves(l_run);
  const int orow = q0 + l32;
  if (orow < L) {
    uint16_t* op = p.out + hbase + (int64_t)orow * sl;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w.x = pack_bf16(o[dt][4 * j + 0] * inv, o[dt][4 * j + 1] * inv);
        w.y = pack_bf16(o[dt][4 * j + 2] * inv, o[dt][4 * j + 3] * inv);
        *reinterpret_cast<u32x2*>(op + dt * 32 + 8 * j + 4 * hh) = w;
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd(AttnParams& p, hipStream_t stream) {
  p.n_qblocks = (p.seq_len + BM - 1) / BM;
  p.n_blocks = p.batch * HV_HEADS * p.n_qblocks;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)p.n_blocks), dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hv
