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
#include <type_traits>

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

// ---- scheduling hints -------------------------------------------------------
// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedVALU = 0x002;
constexpr int kSchedMFMA = 0x008;
constexpr int kSchedDSRead = 0x100;
constexpr int kSchedDSWrite = 0x200;
constexpr int kSchedVMEMRead = 0x020;
#ifndef HV_ATTN_SCHED
#define HV_ATTN_SCHED 1
#endif
#if HV_ATTN_SCHED
#define HV_SCHED_GROUP(mask, n, id) __builtin_amdgcn_sched_group_barrier(mask, n, id)
#else
#define HV_SCHED_GROUP(mask, n, id) ((void)0)
#endif

// ---- per-step building blocks --------------------------------------------------

struct KStage {
  u32x4 r0, r1;
};
struct VStage {
  u32x4 a, b;
};

// Row maximum of a score tile (32 in-lane values, then across the two halves),
// in the log2 domain.  Masked keys must already be -inf.
__device__ __forceinline__ float tile_max(const f32x16& s0, const f32x16& s1, float c2) {
  float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
  for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(s0[v], s1[v]));
  return max_across_halves(mx) * c2;
}

__device__ __forceinline__ void mask_tile(f32x16& s0, f32x16& s1, int lim, int hh) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int key = 8 * (v >> 2) + 4 * hh + (v & 3);
    if (key >= lim) s0[v] = -INFINITY;
    if (key + 32 >= lim) s1[v] = -INFINITY;
  }
}

// Raise the running reference to the tile maximum when it exceeds it by more
// than 2^8; rescale the accumulators accordingly (rare after the first tiles).
__device__ __forceinline__ void update_reference(float mx, float& m_run, float& l_run,
                                                 f32x16 (&o)[4]) {
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
}

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
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // K rows past the valid keys are clamped to the last valid row: they are
  // always in bounds, and their scores are replaced by -inf on the last tile.
  // V rows past the valid keys (last tile only) are clamped and zeroed, so
  // padding contents (even NaN) never meet a zero weight.
  auto load_k = [&](int tile, KStage& st) {
    const int r0 = min(tile * BN + k_row, Lk - 1), r1 = min(tile * BN + k_row + 32, Lk - 1);
    st.r0 = *reinterpret_cast<const u32x4*>(Kg + (int64_t)r0 * sl + k_c * 8);
    st.r1 = *reinterpret_cast<const u32x4*>(Kg + (int64_t)r1 * sl + k_c * 8);
  };
  auto store_k = [&](int buf, const KStage& st) {
    *reinterpret_cast<u32x4*>(&sK[buf][k_row * KS + k_c * 8]) = st.r0;
    *reinterpret_cast<u32x4*>(&sK[buf][(k_row + 32) * KS + k_c * 8]) = st.r1;
  };
  auto load_v = [&](int tile, VStage& st) {  // tile fully inside the valid keys
    const int r0 = tile * BN + 2 * v_kp;
    st.a = *reinterpret_cast<const u32x4*>(Vg + (int64_t)r0 * sl + v_c * 8);
    st.b = *reinterpret_cast<const u32x4*>(Vg + (int64_t)(r0 + 1) * sl + v_c * 8);
  };
  auto load_v_last = [&](int tile, VStage& st) {  // may run past the valid keys
    const int r0 = tile * BN + 2 * v_kp, r1 = r0 + 1;
    st.a = *reinterpret_cast<const u32x4*>(Vg + (int64_t)min(r0, Lk - 1) * sl + v_c * 8);
    st.b = *reinterpret_cast<const u32x4*>(Vg + (int64_t)min(r1, Lk - 1) * sl + v_c * 8);
    if (r0 >= Lk) st.a = zero;
    if (r1 >= Lk) st.b = zero;
  };
  auto store_v = [&](int buf, const VStage& st) {
    uint32_t* vt = reinterpret_cast<uint32_t*>(&sV[buf][0]);
    const int col = vt_pos(2 * v_kp);  // even: keys 2kp, 2kp+1 are adjacent
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = st.a[e >> 1], c = st.b[e >> 1];
      const uint32_t w = (e & 1) ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
      vt[((8 * v_c + e) * VS + col) >> 1] = w;
    }
  };
  auto k_frag = [&](const uint16_t* kt, int half, int kc) {
    return *reinterpret_cast<const bf16x8*>(kt + (half * 32 + l32) * KS + kc * 16 + hh * 8);
  };
  auto v_frag = [&](const uint16_t* vt, int dt, int mm) {
    return *reinterpret_cast<const bf16x8*>(vt + (dt * 32 + l32) * VS + mm * 16 + hh * 8);
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;
  float m_run = -INFINITY;  // running reference, log2 domain
  float l_run = 0.f;        // this lane's share of the denominator (bf16-rounded weights)
  const float c2 = p.scale_log2;
  const int ntiles = (Lk + BN - 1) / BN;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // exp2 of scores e0, e0+1 of tile registers s (in place)
  auto exp_pair = [&](f32x16 (&s)[2], int e0) {
#pragma unroll
    for (int e = e0; e < e0 + 2; ++e)
      s[e >> 4][e & 15] = __builtin_amdgcn_exp2f(fmaf(s[e >> 4][e & 15], c2, -m_run));
  };
  // bf16 P^T operand for keys 16*i .. 16*i+15 and its share of the denominator.
  // The four packed words are built as separate 32-bit values and fed to
  // v_dot2 before they are assembled into the MFMA operand: taking them back
  // out of the 128-bit operand (as vector elements) makes this compiler encode
  // the first word for all four v_dot2c_f32_bf16 operands.
  auto pack_p = [&](f32x16 (&s)[2], int i) {
    const f32x16& src = s[i >> 1];
    const int base = (i & 1) * 8;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack_bf16(src[base + 2 * j], src[base + 2 * j + 1]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[j]), ones, l_run, false);
    const u32x4 v = {w[0], w[1], w[2], w[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  // ---- prologue: K tiles 0 and 1, V tile 0; scores and reference of tile 0
  {
    KStage ks;
    VStage vs;
    load_k(0, ks);
    if (ntiles == 1) load_v_last(0, vs); else load_v(0, vs);
    store_k(0, ks);
    store_v(0, vs);
    if (ntiles > 1) {
      load_k(1, ks);
      store_k(1, ks);
    }
  }
  __syncthreads();
  f32x16 sa[2], sb[2];
#pragma unroll
  for (int v = 0; v < 16; ++v) { sa[0][v] = 0.f; sa[1][v] = 0.f; }
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    sa[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(&sK[0][0], 0, kc), qf[kc], sa[0], 0, 0, 0);
    sa[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(&sK[0][0], 1, kc), qf[kc], sa[1], 0, 0, 0);
  }
  if (ntiles == 1) mask_tile(sa[0], sa[1], Lk, hh);
  update_reference(tile_max(sa[0], sa[1], c2), m_run, l_run, o);
  __syncthreads();  // every wave has read K tile 0 before its buffer is refilled

  // ---- steady state.  Step t (tile t+1 exists):
  //   phase 1: QK^T MFMAs of tile t+1, interleaved with the exp2 / bf16 / sum
  //            work of tile t (independent VALU that runs under the MFMAs);
  //   phase 2: PV MFMAs of tile t, interleaved with the row maximum of tile t+1;
  //   then the staged K tile t+2 and V tile t+1 go to the free LDS buffers,
  //   one barrier, and the reference update for tile t+1 (rarely taken).
  auto step = [&](auto last, int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    constexpr bool kLast = decltype(last)::value;  // tile t+1 is the last tile
    KStage ks;
    VStage vs;
    if constexpr (!kLast) {
      load_k(t + 2, ks);
      load_v(t + 1, vs);
    } else {
      load_v_last(t + 1, vs);
    }
    const uint16_t* kt = &sK[(t + 1) & 1][0];
    const uint16_t* vt = &sV[t & 1][0];
#pragma unroll
    for (int v = 0; v < 16; ++v) { nxt[0][v] = 0.f; nxt[1][v] = 0.f; }
    bf16x8 pb[4];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      nxt[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(kt, 0, kc), qf[kc], nxt[0], 0, 0, 0);
      exp_pair(cur, 4 * kc);
      nxt[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(kt, 1, kc), qf[kc], nxt[1], 0, 0, 0);
      exp_pair(cur, 4 * kc + 2);
      if (kc & 1) pb[kc >> 1] = pack_p(cur, kc >> 1);
    }
    HV_SCHED_GROUP(kSchedVMEMRead, 4, 0);
    HV_SCHED_GROUP(kSchedDSRead, 4, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      HV_SCHED_GROUP(kSchedMFMA, 1, 0);
      HV_SCHED_GROUP(kSchedVALU, 6, 0);
      HV_SCHED_GROUP(kSchedDSRead, 1, 0);
      HV_SCHED_GROUP(kSchedMFMA, 1, 0);
      HV_SCHED_GROUP(kSchedVALU, 6, 0);
      HV_SCHED_GROUP(kSchedDSRead, 1, 0);
    }

    if constexpr (kLast) mask_tile(nxt[0], nxt[1], Lk - (t + 1) * BN, hh);

#pragma unroll
    for (int mm = 0; mm < 4; ++mm)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(vt, dt, mm), pb[mm], o[dt], 0, 0, 0);
    const float mx = tile_max(nxt[0], nxt[1], c2);
    if constexpr (!kLast) store_k(t & 1, ks);
    store_v((t + 1) & 1, vs);
    HV_SCHED_GROUP(kSchedDSRead, 4, 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      HV_SCHED_GROUP(kSchedMFMA, 1, 1);
      HV_SCHED_GROUP(kSchedDSRead, 1, 1);
    }
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      HV_SCHED_GROUP(kSchedMFMA, 1, 1);
      HV_SCHED_GROUP(kSchedVALU, 3, 1);
      HV_SCHED_GROUP(kSchedDSRead, 1, 1);
    }
    HV_SCHED_GROUP(kSchedDSWrite, 10, 1);
    __syncthreads();
    update_reference(mx, m_run, l_run, o);
  };

  using Plain = std::integral_constant<bool, false>;
  using Last = std::integral_constant<bool, true>;
  int t = 0;
  for (; t + 3 < ntiles; t += 2) {
    step(Plain{}, t, sa, sb);
    step(Plain{}, t + 1, sb, sa);
  }
  if (t + 2 < ntiles) {
    step(Plain{}, t, sa, sb);
    step(Last{}, t + 1, sb, sa);
    t += 2;
  } else if (t + 1 < ntiles) {
    step(Last{}, t, sa, sb);
    ++t;
#pragma unroll
    for (int v = 0; v < 16; ++v) { sa[0][v] = sb[0][v]; sa[1][v] = sb[1][v]; }
  }

  // ---- last tile: softmax and PV only
  {
    const uint16_t* vt = &sV[t & 1][0];
    bf16x8 pb[4];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      exp_pair(sa, 4 * kc);
      exp_pair(sa, 4 * kc + 2);
      if (kc & 1) pb[kc >> 1] = pack_p(sa, kc >> 1);
    }
#pragma unroll
    for (int mm = 0; mm < 4; ++mm)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(vt, dt, mm), pb[mm], o[dt], 0, 0, 0);
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
