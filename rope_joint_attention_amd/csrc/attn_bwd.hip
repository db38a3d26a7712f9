// Gradients of the joint [video; text] attention for gfx950 (MI355X).
//
// What is computed: the attention of the HunyuanVideo notes page ("HunyuanVideo
// 模型结构与数学原理", section 5.2) differentiated by the chain rule through the
// softmax; the report summary page (zhao9797.github.io, "hunyuan-video", Infra
// section, training) names fused attention as the training bottleneck.  Per
// (batch, head), with P = softmax(scale * Q K^T) over the valid keys and the
// upstream gradient dO:
//     D_i = sum_c dO_ic O_ic             (= rowsum(P * dP), since O = P V)
//     dV  = P^T dO,   dP = dO V^T,   dS = P * (dP - D),
//     dQ  = scale * dS K,   dK = scale * dS^T Q.
// P is recomputed from the forward's log-sum-exp: P_ij = exp(scale s_ij - lse_i),
// so no running maximum is needed.  Padded keys get zero dK, dV.
//
// Three kernels, all MFMA 32x32x16 bf16 with fp32 accumulation:
//   * delta: D per (row, head), one thread per 16-byte chunk, 16-lane DPP sum,
//            stored negated: -D is where every dP accumulation starts, so the
//            MFMAs yield dP - D directly; it also writes -lse/scale, where the
//            dkdv kernel's S chains start, so the exponent is one multiply away;
//   * dkdv:  a block is (batch, head, 128 keys), 4 waves of 32 keys,
//            K and V of its keys held in registers as MFMA operands; it walks
//            all query tiles of 64 rows (Q, dO, lse, D staged in LDS by
//            global->LDS loads, two stages) and accumulates dV^T += dO^T P and
//            dK^T += Q^T dS in registers; the two 32-query units of a tile
//            are staggered so one unit's exp/dS work runs under the other's
//            MFMAs;
//   * dq:    a block is (batch, head, 256 queries), 8 waves of 32
//            queries (two per SIMD) with Q and dO in registers; it walks the key tiles of 64
//            rows (K, V staged the same way) and accumulates dQ^T += K^T dS^T.
// The dkdv and dq grids are persistent: one workgroup per CU, each taking
// (batch, head, rows) blocks in order from a work counter until none is left.
// dQ is computed in its own pass (recomputing S and dP) instead of by atomics
// from the key-block kernel: no fp32 scratch, deterministic results.
//
// Orientation.  Scores are formed so that the lane owns the row whose
// statistics it needs: in dq, S^T = K Q^T (lane = query, one lse and one D per
// lane); in dkdv, S = Q K^T (lane = key), and the per-query lse and D of the
// 16 rows a lane holds are read from LDS as four 16-byte vectors.  The
// operand that has to be transposed (K^T in dq, dO^T and Q^T in dkdv) comes
// from LDS through ds_read_b64_tr_b16, as V^T does in the forward kernel.
//
// LDS tiles are 64 rows of 256 bytes; the 16-byte chunk c of row r is stored
// at slot c ^ f(r mod 16) with f(r) = 4(r mod 4) + (r div 4) mod 4.  Sixteen
// consecutive rows at one chunk (the row-operand reads) hit 16 distinct slots,
// and eight rows (a multiple of 8 onwards) by four chunks (the transposing
// reads) hit 16 distinct slots twice each, so both read patterns are free of
// bank conflicts on the same tile.
#include <type_traits>

#include "hv_internal.h"

namespace hv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define HV_LDS __attribute__((address_space(3)))

constexpr int D = HV_HEAD_DIM;   // 128
constexpr int ROWB = D * 2;      // bytes per tile row
constexpr int TR = 64;           // rows per staged tile
constexpr int TILEB = TR * ROWB; // 16 KB
constexpr float kLog2e = 1.4426950408889634f;

constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// Barrier without the fence of __syncthreads(): the caller's own global->LDS
// loads are waited for explicitly (vmcnt 0), the barrier makes every wave's
// loads visible and orders this step's reads before the next refill.
__device__ __forceinline__ void barrier_loads_done(void) {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int tile_off(int r, int c) { return r * ROWB + ((c ^ swz(r & 15)) << 4); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);  // nearest even
  return __builtin_bit_cast(uint32_t, r);
}

// bf16 operand from 8 score registers base .. base+7 of a 32x32 result: the
// contraction slots of the other operand are ordered to match (see tr_offsets).
__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int base) {
  const u32x4 w = {pack_bf16(s[base], s[base + 1]), pack_bf16(s[base + 2], s[base + 3]),
                   pack_bf16(s[base + 4], s[base + 5]), pack_bf16(s[base + 6], s[base + 7])};
  return __builtin_bit_cast(bf16x8, w);
}

// Row-operand offsets: row l32 (plus 32 * half as an immediate), chunk 2kc + hh.
__device__ __forceinline__ void row_offsets(int l32, int hh, int (&off)[8]) {
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) off[kc] = tile_off(l32, 2 * kc + hh);
}

// Transposing-read offsets for an operand whose rows are the contraction
// (rows 16mm + 8(e/4) + 4hh + e%4 in slot e) and whose m index is the channel
// 32dt + l32.  ds_read_b64_tr_b16: in each group of 16 lanes, lane j receives
// element j%4 of the 8-byte rows that lanes j/4, j/4+4, j/4+8, j/4+12
// address.  Lane p of a group addresses row base + p/4, channels
// d0 + 4(p%4) .. +3, so lane j ends up with channel d0 + j of rows base..+3.
__device__ __forceinline__ void tr_offsets(int lane, int (&off)[8]) {
  const int hh = lane >> 5;
  const int tr_row = 4 * hh + ((lane & 15) >> 2);
  const int tr_ch = 16 * ((lane & 31) >> 4) + 4 * (lane & 3);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int ch = 32 * dt + tr_ch;
      off[2 * dt + q] = tile_off(tr_row + 8 * q, ch >> 3) + 2 * (ch & 7);
    }
}

__device__ __forceinline__ bf16x8 tr_operand(const unsigned char* tile, const int (&off)[8], int dt,
                                             int row0) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HV_LDS i16x4*)(tile + off[2 * dt] + row0 * ROWB));
  const i16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HV_LDS i16x4*)(tile + off[2 * dt + 1] + row0 * ROWB));
  const u32x4 w = {__builtin_bit_cast(u32x2, a)[0], __builtin_bit_cast(u32x2, a)[1],
                   __builtin_bit_cast(u32x2, c)[0], __builtin_bit_cast(u32x2, c)[1]};
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ bf16x8 row_operand(const unsigned char* tile, const int (&off)[8], int kc,
                                              int row0) {
  return *reinterpret_cast<const bf16x8*>(tile + off[kc] + row0 * ROWB);
}

// Persistent workgroups, one per CU, take blocks in order from a counter
// (zeroed by the delta kernel that runs first): under MFMA load the XCDs settle
// at different clocks, and a fixed share of blocks per XCD would let the
// slowest one set the time.  Returns the next block, or a value >= nb when
// the work is done.  The first barrier makes sure every wave is done with the
// previous block's LDS before the caller stages new tiles.
__device__ __forceinline__ int next_block(int* counter, int& slot) {
  __syncthreads();
  if (threadIdx.x == 0) slot = atomicAdd(counter, 1);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(slot);
}

// Stage one 64-row tile (rows row0.. of a [rows][stride] bf16 tensor, last
// valid row `last`) into LDS with global->LDS loads: the wave issues `n`
// 1-KB instructions starting at instruction i0; instruction i fills rows
// 4i .. 4i+3, lane l slot l%16 of row 4i + l/16 with the chunk that the row's
// swizzle puts there.
__device__ __forceinline__ void stage_tile(const uint16_t* base, int64_t stride, int row0, int last,
                                           unsigned char* tile, int i0, int n, int lane) {
  for (int j = 0; j < n; ++j) {
    const int i = i0 + j;
    const int r = 4 * i + (lane >> 4);
    const int c = (lane & 15) ^ swz(r & 15);
    const int grow = min(row0 + r, last);
    const unsigned char* src = (const unsigned char*)(base + (int64_t)grow * stride) + c * 16;
    __builtin_amdgcn_global_load_lds(src, (HV_LDS void*)(tile + i * 1024), 16, 0, 0);
  }
}

// Per-lane byte offsets, from the first row of a full tile, of the `n`
// staging instructions i0 .. i0+n-1 (the same rows and slots as stage_tile).
template <int N>
__device__ __forceinline__ void stage_offsets(int64_t stride, int i0, int lane, uint32_t (&off)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const int r = 4 * (i0 + j) + (lane >> 4);
    const int c = (lane & 15) ^ swz(r & 15);
    off[j] = (uint32_t)(r * stride * 2) + c * 16;
  }
}

// stage_tile for a tile whose 64 rows all exist: a scalar tile address plus
// the precomputed 32-bit lane offsets, no per-lane address arithmetic.
template <int N>
__device__ __forceinline__ void stage_full_tile(const uint16_t* base, int64_t stride, int row0,
                                                unsigned char* tile, int i0, uint32_t (&off)[N]) {
  const unsigned char* tb = (const unsigned char*)(base + (int64_t)row0 * stride);
#pragma unroll
  for (int j = 0; j < N; ++j) {
    asm volatile("" : "+v"(off[j]));  // keeps the scalar base + 32-bit offset form
    __builtin_amdgcn_global_load_lds(tb + off[j], (HV_LDS void*)(tile + (i0 + j) * 1024), 16, 0, 0);
  }
}

// 64 consecutive fp32 values (rows row0.., clamped to `last`) of a row vector.
__device__ __forceinline__ void stage_vec(const float* base, int row0, int last, float* dst,
                                          int lane) {
  const float* src = base + min(row0 + lane, last);
  __builtin_amdgcn_global_load_lds(src, (HV_LDS void*)dst, 4, 0, 0);
}

// ---------------------------------------------------------------- delta ----
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
  return v;
}

__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(BwdParams p) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {  // work counters of the two gradient kernels
    p.counters[0] = 0;
    p.counters[1] = 0;
  }
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int chunk = (int)(gid & 15);
  const int64_t row = gid >> 4;  // b * seq_len + n
  if (row >= (int64_t)p.batch * p.seq_len) return;  // whole 16-lane rows leave together
  const int b = (int)(row / p.seq_len);
  const int n = (int)(row - (int64_t)b * p.seq_len);
  const int64_t base = (int64_t)b * p.stride_b + (int64_t)n * p.stride_l + chunk * 8;
  const float nis = -1.0f / p.scale;
  const u32x4* op = reinterpret_cast<const u32x4*>(p.o + base);
  const u32x4* gp = reinterpret_cast<const u32x4*>(p.dout + base);
#pragma unroll
  for (int h0 = 0; h0 < HV_HEADS; h0 += 8) {
    u32x4 ov[8], gv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ov[i] = op[(h0 + i) * 16];
      gv[i] = gp[(h0 + i) * 16];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s = fmaf(__uint_as_float(ov[i][j] << 16), __uint_as_float(gv[i][j] << 16), s);
        s = fmaf(__uint_as_float(ov[i][j] & 0xffff0000u), __uint_as_float(gv[i][j] & 0xffff0000u), s);
      }
      s = row16_sum(s);
      // stored negated: it is the starting accumulator of the dP products;
      // -lse/scale likewise starts the S products of the dK/dV kernel
      if (chunk == 0) {
        const int64_t at = ((int64_t)b * HV_HEADS + h0 + i) * p.seq_len + n;
        p.delta[at] = -s;
        p.nls[at] = p.lse[at] * nis;
      }
    }
  }
}

// ----------------------------------------------------------------- dK, dV --
constexpr int KV_WAVES = 4;
constexpr int KV_KEYS = KV_WAVES * 32;  // keys per workgroup

__global__ __launch_bounds__(KV_WAVES * 64, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char sQ0[TILEB], sQ1[TILEB], sG0[TILEB], sG1[TILEB];
  __shared__ __attribute__((aligned(16))) float sL0[TR], sL1[TR], sD0[TR], sD1[TR];
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto qbuf = [&](auto st) -> unsigned char* { if constexpr (decltype(st)::value == 0) return sQ0; else return sQ1; };
  auto gbuf = [&](auto st) -> unsigned char* { if constexpr (decltype(st)::value == 0) return sG0; else return sG1; };
  auto lbuf = [&](auto st) -> float* { if constexpr (decltype(st)::value == 0) return sL0; else return sL1; };
  auto dbuf = [&](auto st) -> float* { if constexpr (decltype(st)::value == 0) return sD0; else return sD1; };

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  __shared__ int s_block;
  for (;;) {
  const int logical = next_block(p.counters + 0, s_block);
  if (logical >= p.n_kv_blocks) break;
  int si = 0;  // segment of this block (uniform scan over at most 64 entries)
  for (int i = 1; i < p.n_seg; ++i)
    if (logical >= p.seg[i].k_blk) si = i;
  const BwdSegment& sg = p.seg[si];
  const int rel = logical - sg.k_blk;
  const int head = rel / sg.nkb;
  const int kb = rel - head * sg.nkb;
  const int L = sg.q_len;    // query rows
  const int Lk = sg.k_len;   // valid keys
  const int64_t sl = p.stride_l;
  const int64_t qbase = sg.q_off + (int64_t)head * D;
  const int64_t kbase = sg.k_off + (int64_t)head * D;
  const int64_t vbase = sg.v_off + (int64_t)head * p.v_hstride;  // lse / delta row 0

  // K and V of this lane's key as the B operands (n = key, k = channels
  // 16kc + 8hh .. +7); keys past the valid ones read the last valid row and
  // are masked out of P and dS below.
  const int key = kb * KV_KEYS + wave * 32 + l32;
  const bool key_ok = key < Lk;
  bf16x8 kf[8], vf[8];
  {
    const int64_t r = kbase + (int64_t)min(key, Lk - 1) * sl + hh * 8;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      kf[kc] = *reinterpret_cast<const bf16x8*>(p.k + r + kc * 16);
      vf[kc] = *reinterpret_cast<const bf16x8*>(p.v + r + kc * 16);
      // K and V are only ever MFMA operands: keep them in AGPRs, which
      // leaves the VGPRs to the accumulators (with VGPR-form MFMAs the
      // softmax then reads S and dP without a copy per value)
      asm volatile("" : "+a"(kf[kc]), "+a"(vf[kc]));
    }
  }
  int roff[8], troff[8];
  row_offsets(l32, hh, roff);
  tr_offsets(lane, troff);

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) dk[dt][v] = dv[dt][v] = 0.f;
  const float c2 = p.scale_log2;
  // a block of padded keys only has zero gradients: skip the query loop
  const int nq = kb * KV_KEYS >= Lk || L == 0 ? 0 : (L + TR - 1) / TR;

  // 16 instructions per 64-row tile and tensor: wave w issues 4w .. 4w+3
  uint32_t soff[4];
  stage_offsets(sl, 4 * wave, lane, soff);
  auto load = [&](auto st, int t) {
    if (t * TR + TR <= L) {
      stage_full_tile(p.q + qbase, sl, t * TR, qbuf(st), 4 * wave, soff);
      stage_full_tile(p.dout + qbase, sl, t * TR, gbuf(st), 4 * wave, soff);
    } else {
      stage_tile(p.q + qbase, sl, t * TR, L - 1, qbuf(st), 4 * wave, 4, lane);
      stage_tile(p.dout + qbase, sl, t * TR, L - 1, gbuf(st), 4 * wave, 4, lane);
    }
    if (wave == 0) stage_vec(p.nls + vbase, t * TR, L - 1, lbuf(st), lane);
    if (wave == 1) stage_vec(p.delta + vbase, t * TR, L - 1, dbuf(st), lane);
  };

  // One 64-query tile in two units of 32 queries.  Per unit: S = Q K^T and
  // dP = dO V^T (16 MFMAs), then P and dS (VALU), then dV^T += dO^T P and
  // dK^T += Q^T dS (16 MFMAs).  The units are staggered so that the VALU work
  // of one runs under the MFMAs of the other:
  //   A0 | A1 + V0 | B0 + V1 | B1
  // kMask: the tile may hold query rows past L or this block keys past Lk.
  // Full tiles of a block whose keys are all valid skip the per-element mask.
  // mid: called once inside the tile (the next tile's request, or nothing).
  auto tile = [&](auto st, auto masked, int t, auto mid) {
    constexpr bool kMask = decltype(masked)::value;
    const unsigned char* qt = qbuf(st);
    const unsigned char* gt = gbuf(st);
    const float* lt = lbuf(st);
    const float* dtv = dbuf(st);
    f32x16 s0, d0, s1, d1;
    // Starting accumulators of unit u, row by row (register v of a unit holds
    // query 32u + 8(v/4) + 4hh + v%4 of the tile): -lse/scale for S, so that
    // scale*log2(e) times the result is the log2 of P, and -D for dP, so that
    // the result is dP - D.
    f32x16 si[2], di[2];
    auto stats = [&](int u) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = 32 * u + 8 * g + 4 * hh;
        const f32x4 l = *reinterpret_cast<const f32x4*>(lt + r);  // -lse/scale
        const f32x4 d = *reinterpret_cast<const f32x4*>(dtv + r);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          si[u][4 * g + j] = l[j];
          di[u][4 * g + j] = d[j];
        }
      }
    };
    // P and dS of scores 2w, 2w+1 of unit u, rounded to bf16 straight into
    // word w of the unit's dV and dK operands (the accumulators are only read)
    uint32_t pw[2][8], dw[2][8];
    auto grad = [&](const f32x16& sv, const f32x16& dv_, int u, int w) __attribute__((always_inline)) {
      float p0 = __builtin_amdgcn_exp2f(sv[2 * w] * c2);
      float p1 = __builtin_amdgcn_exp2f(sv[2 * w + 1] * c2);
      float g0 = p0 * dv_[2 * w];
      float g1 = p1 * dv_[2 * w + 1];
      if constexpr (kMask) {
        const int r = 32 * u + 8 * (w >> 1) + 4 * hh + 2 * (w & 1);  // rows r, r + 1
        const bool ok0 = key_ok && (t * TR + r < L);
        const bool ok1 = key_ok && (t * TR + r + 1 < L);
        p0 = ok0 ? p0 : 0.f;
        g0 = ok0 ? g0 : 0.f;
        p1 = ok1 ? p1 : 0.f;
        g1 = ok1 ? g1 : 0.f;
      }
      pw[u][w] = pack_bf16(p0, p1);
      dw[u][w] = pack_bf16(g0, g1);
    };
    auto words = [&](const uint32_t (&wd)[8], int h) __attribute__((always_inline)) {
      const u32x4 v = {wd[4 * h], wd[4 * h + 1], wd[4 * h + 2], wd[4 * h + 3]};
      return __builtin_bit_cast(bf16x8, v);
    };
    // The tile is 32 MFMA pairs: 0..7 S, dP of unit 0 (rows of Q, dO); 8..15
    // the same for unit 1, with the probabilities and dS of unit 0 computed
    // under them; 16..23 dV, dK of unit 0 (transposed dO, Q) with unit 1's
    // softmax under them; 24..31 dV, dK of unit 1.  Each pair's two LDS
    // operands are read two pairs ahead, the row statistics four pairs ahead.
    auto ops = [&](int i, bf16x8& a, bf16x8& b) __attribute__((always_inline)) {
      if (i < 16) {
        const int kc = i & 7, row0 = 32 * (i >> 3);
        a = row_operand(qt, roff, kc, row0);
        b = row_operand(gt, roff, kc, row0);
      } else {
        const int u = (i - 16) >> 3, j = (i - 16) & 7;
        const int mm = j >> 2, dt = j & 3;
        a = tr_operand(gt, troff, dt, 32 * u + 16 * mm);
        b = tr_operand(qt, troff, dt, 32 * u + 16 * mm);
      }
    };
    bf16x8 ca, cb, na, nb, xa, xb, pb0[2], db0[2], pb1[2], db1[2];
    ops(0, ca, cb);
    ops(1, na, nb);
    stats(0);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + 2 < 32) ops(i + 2, xa, xb);
      if (i == 6) mid();  // the next tile's request (measured: cheapest at pair 6)
      if (i == 4) stats(1);
      if (i == 16) {
        pb0[0] = words(pw[0], 0); pb0[1] = words(pw[0], 1);
        db0[0] = words(dw[0], 0); db0[1] = words(dw[0], 1);
      }
      if (i == 24) {
        pb1[0] = words(pw[1], 0); pb1[1] = words(pw[1], 1);
        db1[0] = words(dw[1], 0); db1[1] = words(dw[1], 1);
      }
      if (i < 8) {  // the first MFMA of each chain takes the starting accumulator
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca, kf[i], i ? s0 : si[0], 0, 0, 0);
        d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb, vf[i], i ? d0 : di[0], 0, 0, 0);
      } else if (i < 16) {
        const int kc = i - 8;
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca, kf[kc], kc ? s1 : si[1], 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb, vf[kc], kc ? d1 : di[1], 0, 0, 0);
        grad(s0, d0, 0, kc);
      } else if (i < 24) {
        const int j = i - 16, mm = j >> 2, dt = j & 3;
        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca, pb0[mm], dv[dt], 0, 0, 0);
        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb, db0[mm], dk[dt], 0, 0, 0);
        grad(s1, d1, 1, j);
      } else {
        const int j = i - 24, mm = j >> 2, dt = j & 3;
        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca, pb1[mm], dv[dt], 0, 0, 0);
        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb, db1[mm], dk[dt], 0, 0, 0);
      }
      ca = na;
      cb = nb;
      na = xa;
      nb = xb;
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  using Unmasked = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  // pairs of full tiles without masks while the block's keys are all valid,
  // then the rest (a full tile, the partial last one, or all tiles of a block
  // that holds padded keys) with masks
  const int n_unmasked = (kb + 1) * KV_KEYS <= Lk ? L / TR : 0;
  if (nq > 0) load(I0{}, 0);
  int t = 0;
  // In the unmasked loop the next tile is requested from inside the tile (at
  // its seventh MFMA pair) rather than right after the barrier: its stage was
  // freed by that barrier either way, and the later request costs less.
  auto none = [] {};
  for (; t + 2 <= n_unmasked; t += 2) {
    barrier_loads_done();
    tile(I0{}, Unmasked{}, t, [&] { load(I1{}, t + 1); });
    barrier_loads_done();
    tile(I1{}, Unmasked{}, t + 1, [&] { if (t + 2 < nq) load(I0{}, t + 2); });
  }
  for (; t + 2 <= nq; t += 2) {
    barrier_loads_done();
    load(I1{}, t + 1);
    tile(I0{}, Masked{}, t, none);
    barrier_loads_done();
    if (t + 2 < nq) load(I0{}, t + 2);
    tile(I1{}, Masked{}, t + 1, none);
  }
  if (t < nq) {
    barrier_loads_done();
    tile(I0{}, Masked{}, t, none);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

  // lane owns key `key`, channels 32dt + 8j + 4hh .. +3 (register 4j .. 4j+3)
  if (key < sg.k_rows) {
    const float sc = p.scale;
    uint16_t* kp = p.dk + kbase + (int64_t)key * sl;
    uint16_t* vp = p.dv + kbase + (int64_t)key * sl;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 wk, wv;
        wk.x = pack_bf16(dk[dt][4 * j] * sc, dk[dt][4 * j + 1] * sc);
        wk.y = pack_bf16(dk[dt][4 * j + 2] * sc, dk[dt][4 * j + 3] * sc);
        wv.x = pack_bf16(dv[dt][4 * j], dv[dt][4 * j + 1]);
        wv.y = pack_bf16(dv[dt][4 * j + 2], dv[dt][4 * j + 3]);
        *reinterpret_cast<u32x2*>(kp + dt * 32 + 8 * j + 4 * hh) = wk;
        *reinterpret_cast<u32x2*>(vp + dt * 32 + 8 * j + 4 * hh) = wv;
      }
  }
  }  // block loop
}

// --------------------------------------------------------------------- dQ --
constexpr int Q_WAVES = 8;
constexpr int Q_ROWS = Q_WAVES * 32;  // queries per workgroup

__global__ __launch_bounds__(Q_WAVES * 64, 1) void attn_bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char sK0[TILEB], sK1[TILEB], sV0[TILEB], sV1[TILEB];
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto kbuf = [&](auto st) -> unsigned char* { if constexpr (decltype(st)::value == 0) return sK0; else return sK1; };
  auto vbuf = [&](auto st) -> unsigned char* { if constexpr (decltype(st)::value == 0) return sV0; else return sV1; };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar: DMA destinations (M0) from the scalar unit
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  __shared__ int s_block;
  for (;;) {
  const int logical = next_block(p.counters + 1, s_block);
  if (logical >= p.n_q_blocks) break;
  int si = 0;
  for (int i = 1; i < p.n_seg; ++i)
    if (logical >= p.seg[i].q_blk) si = i;
  const BwdSegment& sg = p.seg[si];
  const int rel = logical - sg.q_blk;
  const int head = rel / sg.nqb;
  const int qb = rel - head * sg.nqb;
  const int L = sg.q_len;
  const int Lk = sg.k_len;
  const int64_t sl = p.stride_l;
  const int64_t qbase = sg.q_off + (int64_t)head * D;
  const int64_t kbase = sg.k_off + (int64_t)head * D;
  const int64_t vbase = sg.v_off + (int64_t)head * p.v_hstride;

  // Q and dO of this lane's query as B operands (n = query, k = channels)
  const int q0 = qb * Q_ROWS + wave * 32;
  const int qrow = min(q0 + l32, L - 1);  // rows past the end are computed, never stored
  bf16x8 qf[8], gf[8];
  {
    const int64_t r = qbase + (int64_t)qrow * sl + hh * 8;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      qf[kc] = *reinterpret_cast<const bf16x8*>(p.q + r + kc * 16);
      gf[kc] = *reinterpret_cast<const bf16x8*>(p.dout + r + kc * 16);
    }
  }
  const float lse2 = p.lse[vbase + qrow] * kLog2e;
  f32x16 neg_d;  // -D of this lane's query (as stored): the dP^T chains start from it
  {
    const float nd = p.delta[vbase + qrow];
#pragma unroll
    for (int v = 0; v < 16; ++v) neg_d[v] = nd;
  }
  int roff[8], troff[8];
  row_offsets(l32, hh, roff);
  tr_offsets(lane, troff);

  f32x16 dq[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) dq[dt][v] = 0.f;
  const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float c2 = p.scale_log2;
  const int nk = (Lk + TR - 1) / TR;

  // 16 instructions per tile and tensor, split evenly over the waves
  constexpr int per_wave = 16 / Q_WAVES;
  uint32_t soff[per_wave];
  stage_offsets(sl, per_wave * wave, lane, soff);
  auto load = [&](auto st, int t) {
    if (t * TR + TR <= Lk) {
      stage_full_tile(p.k + kbase, sl, t * TR, kbuf(st), per_wave * wave, soff);
      stage_full_tile(p.v + kbase, sl, t * TR, vbuf(st), per_wave * wave, soff);
    } else {
      stage_tile(p.k + kbase, sl, t * TR, Lk - 1, kbuf(st), per_wave * wave, per_wave, lane);
      stage_tile(p.v + kbase, sl, t * TR, Lk - 1, vbuf(st), per_wave * wave, per_wave, lane);
    }
  };

  // kMask: the tile holds keys past Lk (only the last one can); mid: called
  // once between the two halves (the next tile's request, or nothing)
  auto tile = [&](auto st, auto masked, int t, auto mid) {
    constexpr bool kMask = decltype(masked)::value;
    const unsigned char* kt = kbuf(st);
    const unsigned char* vt = vbuf(st);
    const int lim = Lk - t * TR;
    // two halves of 32 keys, one after the other (keeps the wave within 256
    // registers, so two waves share each SIMD)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1) mid();  // the next tile's request, between the halves (measured)
      // S^T = K Q^T and dP^T = V dO^T: 32 keys x this wave's 32 queries
      f32x16 s, dp;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {  // S^T starts from zero, dP^T from -D
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand(kt, roff, kc, 32 * h), qf[kc], kc ? s : zero16, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand(vt, roff, kc, 32 * h), gf[kc], kc ? dp : neg_d, 0, 0, 0);
      }
      // key of register v: 32h + 8(v/4) + 4hh + v%4
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float ds = __builtin_amdgcn_exp2f(fmaf(s[v], c2, -lse2)) * dp[v];  // dS^T
        if constexpr (kMask) {
          const bool ok = 32 * h + 8 * (v >> 2) + 4 * hh + (v & 3) < lim;
          s[v] = ok ? ds : 0.f;
        } else {
          s[v] = ds;
        }
      }
      // dQ^T += K^T dS^T, keys in groups of 16
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const bf16x8 db = pack8(s, 8 * m2);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(kt, troff, dt, 32 * h + 16 * m2), db, dq[dt], 0, 0, 0);
      }
    }
  };

  using Unmasked = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  const int n_full = Lk / TR;  // key tiles with every key valid
  load(I0{}, 0);
  int t = 0;
  // In the loop over full tiles the next tile is requested between the two
  // halves of the tile rather than right after the barrier (cheaper, measured).
  auto none = [] {};
  for (; t + 2 <= n_full; t += 2) {
    barrier_loads_done();
    tile(I0{}, Unmasked{}, t, [&] { load(I1{}, t + 1); });
    barrier_loads_done();
    tile(I1{}, Unmasked{}, t + 1, [&] { if (t + 2 < nk) load(I0{}, t + 2); });
  }
  // at most one full tile and the partial one remain
  for (; t + 2 <= nk; t += 2) {
    barrier_loads_done();
    load(I1{}, t + 1);
    tile(I0{}, Masked{}, t, none);
    barrier_loads_done();
    if (t + 2 < nk) load(I0{}, t + 2);
    tile(I1{}, Masked{}, t + 1, none);
  }
  if (t < nk) {
    barrier_loads_done();
    tile(I0{}, Masked{}, t, none);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

  const int orow = q0 + l32;
  if (orow < L) {
    const float sc = p.scale;
    uint16_t* op = p.dq + qbase + (int64_t)orow * sl;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w.x = pack_bf16(dq[dt][4 * j] * sc, dq[dt][4 * j + 1] * sc);
        w.y = pack_bf16(dq[dt][4 * j + 2] * sc, dq[dt][4 * j + 3] * sc);
        *reinterpret_cast<u32x2*>(op + dt * 32 + 8 * j + 4 * hh) = w;
      }
  }
  }  // block loop
}

}  // namespace

hipError_t launch_attn_bwd(BwdParams& p, hipStream_t stream) {
  int qblocks = 0, kblocks = 0;
  for (int i = 0; i < p.n_seg; ++i) {
    BwdSegment& sg = p.seg[i];
    sg.nqb = (sg.q_len + Q_ROWS - 1) / Q_ROWS;
    sg.nkb = (sg.k_rows + KV_KEYS - 1) / KV_KEYS;  // also zero-fills keys nobody attends to
    sg.q_blk = qblocks;
    sg.k_blk = kblocks;
    qblocks += HV_HEADS * sg.nqb;
    kblocks += HV_HEADS * sg.nkb;
  }
  p.n_q_blocks = qblocks;
  p.n_kv_blocks = kblocks;
  if (qblocks == 0 && kblocks == 0) return hipSuccess;
  // the caller's workspace: -D, then -lse/scale, then the two work counters
  const int64_t nrows = (int64_t)p.batch * HV_HEADS * p.seq_len;
  p.nls = p.delta + nrows;
  p.counters = reinterpret_cast<int*>(p.delta + 2 * nrows);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipGetLastError();
  if (cus <= 0) return hipErrorInvalidDevice;
  // D for every row (and the counters' reset): it runs first on the stream
  const int64_t threads = (int64_t)p.batch * p.seq_len * 16;
  hipLaunchKernelGGL(attn_bwd_delta_kernel, dim3((unsigned)std::max<int64_t>(1, (threads + 255) / 256)),
                     dim3(256), 0, stream, p);
  // one persistent workgroup per CU (each kernel's LDS or registers allow one)
  if (kblocks > 0)
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel, dim3((unsigned)std::min(kblocks, cus)), dim3(KV_WAVES * 64), 0,
                       stream, p);
  if (qblocks > 0)
    hipLaunchKernelGGL(attn_bwd_dq_kernel, dim3((unsigned)std::min(qblocks, cus)), dim3(Q_WAVES * 64), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace hv
