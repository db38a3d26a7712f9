// Joint [video; text] attention forward for gfx950 (MI355X).
//
// What is computed (HunyuanVideo notes page "HunyuanVideo 模型结构与数学原理",
// section 5.2): per (batch, head), O = softmax(Q K^T / sqrt(128)) V over the
// concatenated sequence, with text keys beyond the valid length left out.
// The attention is exact (section 9.1 stresses that IO-aware tiling does not
// change the result), so the kernel is a tiled exact softmax: scores are
// never written to memory.
//
// The same kernel serves the padded batch, packed segments (variable-length
// clips, section 9.1) and one query block against one K/V block of a
// sequence-parallel ring (section 9.2): its work list is a table of segments
// (query rows, key rows, output rows), and it can also write the natural-log
// log-sum-exp of every row, which lets results over disjoint K/V blocks be
// merged exactly.
//
// Work decomposition
//   * one query block = (segment, head, 256 query rows); 8 waves of 32 rows,
//     two waves per SIMD, one workgroup per CU (calls small enough that
//     blocks of 128 rows all run at once use those instead, 4 waves, one per
//     SIMD: see kWavesSmall).  With a workspace the
//     workgroups are persistent (one per CU) and take query blocks from a
//     counter; without one each workgroup does one block;
//   * K and V tiles of 64 keys reach LDS by direct global->LDS loads
//     (global_load_lds_dwordx4: no registers, fully coalesced 1 KB per wave
//     instruction) into four LDS stages each for K and V; K tile t+4 and
//     V tile t+3 are requested during step t, and each wave waits only for
//     its own oldest loads (s_waitcnt vmcnt) before the step's one barrier;
//   * blocks are numbered segment by segment and head by head, so the blocks
//     in flight stream the same K/V; without a workspace (one block per
//     workgroup) workgroup ids are remapped so that consecutive query blocks
//     of one (batch, head) run on the same XCD and share its L2.
//
// Per wave and step, in MFMA 32x32x16 bf16 (fp32 accumulate):
//   S^T (64 keys x 32 queries) = K_tile * Q^T   -- lane l owns query l%32, so
//       row statistics are 32 in-register values plus one exchange between
//       the two 32-lane halves (v_permlane32_swap);
//   online softmax in the log2 domain with exp2.  The reference m of a row
//       is its maximum over the first tile; later tiles compute no maximum:
//       the row's running sum of weights bounds every weight, and when it
//       passes 2^40 the reference rises by 32 (the accumulators are scaled
//       by 2^-32 exactly).  A block whose weights still overflow is redone
//       with the reference following each tile's maximum (raised only when
//       it exceeds the reference by more than 8, so weights stay <= 256);
//       either way the result is exact;
//   O^T (128 channels x 32 queries) += V^T_tile * P^T -- P^T stays in the
//       registers the softmax produced (bf16).  The V^T operand wants 8 keys
//       of one channel per lane.  With a workspace, V is first packed
//       channel-major tile by tile (v_pack.hip) and each operand is one
//       16-byte LDS read; without one, V stays in its natural [key][channel]
//       layout and the operand is gathered with the gfx950 transposing read
//       ds_read_b64_tr_b16 (two per operand).
//   The step is software-pipelined: the QK^T MFMAs of tile t+1 run under the
//   softmax VALU work of tile t, the PV MFMAs of tile t under the row maximum
//   of tile t+1.
// LDS rows are 256 bytes; 16-byte chunks are XOR-swizzled within a row (K:
// slot c ^ (r % 16), V: slot c ^ 4(r % 4)) so that both the K operand reads
// and the transposing V reads run without bank conflicts.  A packed V tile
// has 128 rows of 128 bytes (one per channel) with slot c ^ ((r / 2) % 8).
// The padded-key mask is a loop bound plus a predicate on the last tile.  Rows
// past the valid keys are never read: their loads are clamped to the last
// valid row, whose scores are masked to -inf (K) or whose weights are exactly
// zero (V; packed V holds zeros there instead), so padding contents cannot
// reach the output.
#include <type_traits>

#include "hv_internal.h"

namespace hv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define HV_LDS __attribute__((address_space(3)))

constexpr int D = HV_HEAD_DIM;  // 128
constexpr int BN = 64;          // keys per tile
constexpr int QPW = 32;         // query rows per wave
// Waves per workgroup: 8 (256 query rows, two waves per SIMD) for every call
// whose blocks take more than one round of workgroups; 4 (128 rows, one wave
// per SIMD) when even the 128-row blocks all run in the first round, where a
// block's time is the chain of its key tiles and one wave per SIMD runs each
// tile in half the time.
constexpr int kWavesLarge = 8;
constexpr int kWavesSmall = 4;
// Per wave count W: 1-KB load instructions per wave and tile, and the tile
// rows each wave loads.  (Namespace-scope templates rather than constants
// local to the kernel: the host pass of this compiler fails to instantiate a
// kernel template whose lambdas use such local constants, and then silently
// emits no launch stub for it.)
template <int W> constexpr int kLoadsPerWave = 16 / W;
template <int W> constexpr int kRowsPerWave = 64 / W;
// Per-lane load offsets are held in arrays of the largest count (the 8-wave
// kernel leaves the upper half unused): with a bound that depends on the
// kernel's wave count, the host pass drops the kernel as well.
constexpr int kMaxLoadsPerWave = 16 / kWavesSmall;
constexpr int NSTAGE = 4;       // K/V tiles resident in LDS (each)
constexpr int ROWB = D * 2;     // bytes per K/V row in LDS (no padding; swizzled)
constexpr int TILEB = BN * ROWB;                 // 16 KB per K or V tile
constexpr int KAHEAD = 4;       // K tile t+KAHEAD is requested in step t
constexpr int VAHEAD = 3;       // V tile t+VAHEAD is requested in step t
constexpr float kRescaleLog2 = 8.0f;

// s_waitcnt immediate for gfx9: vmcnt in bits [3:0] and [15:14], expcnt
// [6:4] (left at its maximum), lgkmcnt [11:8].
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// Byte offset of 16-byte chunk c of row r inside a K tile: slot c ^ (r % 16).
// The 16-byte K operand reads take 16 consecutive rows at one chunk: they hit
// all 16 slots.
__device__ __forceinline__ int kswz(int r, int c) { return r * ROWB + ((c ^ (r & 15)) << 4); }
// Same for a V tile: slot c ^ 4(r % 4).  One transposing read covers 8
// consecutive rows (a multiple of 8 onwards) and 4 consecutive chunks (a
// multiple of 4 onwards): 32 (row, chunk) pairs that land on every slot
// exactly twice, the minimum for 512 bytes.
__device__ __forceinline__ int vswz(int r, int c) { return r * ROWB + ((c ^ ((r & 3) << 2)) << 4); }

// Maximum that propagates NaN (IEEE maximum): it lowers to gfx950's
// v_maximum3_f32 with no input quieting, unlike fmaxf.  Scores are never NaN
// unless an input is, and then the row's output is NaN either way.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);  // nearest even
  return __builtin_bit_cast(uint32_t, r);
}

// Workgroup barrier without the memory fence __syncthreads() implies: the
// fence would drain the in-flight global->LDS loads of later tiles.  The
// caller waits for exactly the loads and LDS operations that must be
// complete; the empty asm statements keep the compiler from moving memory
// accesses across the barrier.
template <int kVm, int kLgkm = 0>
__device__ __forceinline__ void barrier_after(void) {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(kVm, kLgkm));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Row maximum of a score tile (32 in-lane values, then across the two halves),
// in the log2 domain.  Masked keys must already be -inf.
__device__ __forceinline__ float tile_max(const f32x16& s0, const f32x16& s1, float c2) {
  float mx = vmax(s0[0], s1[0]);
#pragma unroll
  for (int v = 1; v < 16; ++v) mx = vmax(vmax(mx, s0[v]), s1[v]);
  return max_across_halves(mx) * c2;
}

// Scores of keys >= lim (tile-relative) become -inf.  Register v of a lane
// holds key 8(v/4) + 4hh + v%4; the lane-dependent part is moved to the
// limit, so every compare is against an immediate (with the key index as the
// loop-invariant operand the compiler keeps 32 key indices in registers for
// the whole key loop).
__device__ __forceinline__ void mask_tile(f32x16& s0, f32x16& s1, int lim, int hh) {
  const int rel = lim - 4 * hh;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int key = 8 * (v >> 2) + (v & 3);
    if (key >= rel) s0[v] = -INFINITY;
    if (key + 32 >= rel) s1[v] = -INFINITY;
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

// Without per-tile maxima: the sum of a row's weights bounds each of them,
// so when it passes 2^40 the reference rises by 32 and the accumulators are
// scaled by 2^-32 (exactly).  The two lanes of a row decide on their joint
// sum, so they keep one reference.
__device__ __forceinline__ void bound_weights(float& m_run, float& l_run, f32x16 (&o)[4]) {
  const bool need = sum_across_halves(l_run) > 0x1p40f;
  if (__any(need)) {
    const float alpha = need ? 0x1p-32f : 1.0f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
    l_run *= alpha;
    if (need) m_run += 32.0f;
  }
}

template <bool kPackedV, int kNW>
__global__ __launch_bounds__(kNW * 64, 1) void attn_fwd_kernel(AttnParams p) {
  // One LDS array per stage: with every access naming its array at compile
  // time, the compiler can tell the tile being loaded from the tiles being
  // read and does not drain the in-flight global->LDS loads before the
  // transposing reads (which it must otherwise assume to alias them).
  __shared__ __attribute__((aligned(1024))) unsigned char sK0[TILEB], sK1[TILEB], sK2[TILEB], sK3[TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char sV0[TILEB], sV1[TILEB], sV2[TILEB], sV3[TILEB];
  auto kbuf = [&](auto st) -> unsigned char* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return sK0; else if constexpr (S == 1) return sK1;
    else if constexpr (S == 2) return sK2; else return sK3;
  };
  auto vbuf = [&](auto st) -> unsigned char* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return sV0; else if constexpr (S == 1) return sV1;
    else if constexpr (S == 2) return sV2; else return sV3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  const int tid = threadIdx.x;
  // wave index as a scalar: the LDS destinations of the tile loads (M0) are
  // then computed on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int nb = p.n_blocks;
  // block ids of the persistent workgroups: slot iter % 2 holds this
  // iteration's, slot (iter + 1) % 2 receives the next one
  __shared__ int s_block[2];
  for (int iter = 0;; ++iter) {
  int logical;
  int next_block = 0;  // thread 0: the id taken for the next iteration
  if constexpr (kPackedV) {
    // Persistent workgroups, one per CU, take query blocks in order from a
    // counter in the workspace (zeroed by the packing kernel).  Under MFMA
    // load the eight XCDs settle at different clocks (measured 1.68-1.85 GHz
    // on one part); with a fixed share of blocks per XCD the slowest one sets
    // the time, with the counter the faster ones take more blocks.  Blocks are
    // numbered segment by segment, head by head, so the 256 blocks in flight
    // share one head's K/V.  The next block is taken as soon as this one
    // starts (its round trip overlaps the block's first loads) and published
    // in LDS at the end of the block, before the barrier of the end-of-block
    // check, which orders it before the next iteration's read; the next
    // iteration publishes into the other slot.
    if (iter == 0) {
      if (tid == 0) s_block[0] = atomicAdd(p.counter, 1);
      __syncthreads();
    }
    logical = __builtin_amdgcn_readfirstlane(s_block[iter & 1]);
    if (logical >= nb) break;
    if (tid == 0) next_block = atomicAdd(p.counter, 1);
  } else {
    // One block per workgroup.  Workgroups are dealt round-robin to the 8
    // XCDs; give each XCD a contiguous range of (segment, head, query-block)
    // ids so that the query blocks resident on one XCD stream the same K/V
    // through its L2.
    if (iter) break;
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int per = nb >> 3, extra = nb & 7;
    logical = xcd * per + min(xcd, extra) + (bid >> 3);
  }
  int si = 0;  // segment of this block (uniform scan over at most 64 entries)
  for (int i = 1; i < p.n_seg; ++i)
    if (logical >= p.seg[i].blk_begin) si = i;
  const AttnSegment& sg = p.seg[si];
  const int rel = logical - sg.blk_begin;
  const int head = rel / sg.nqb;
  const int qb = rel - head * sg.nqb;

  const int L = sg.q_len;
  const int Lk = sg.k_len;
  const int64_t sl = p.kv_sl;
  const uint16_t* Kg = p.k + sg.k_off + (int64_t)head * D;
  const uint16_t* Vg = p.v + sg.k_off + (int64_t)head * D;
  const int ntiles = (Lk + BN - 1) / BN;
  // packed V: this head's tiles, 16 KB apart
  const uint16_t* Vt = kPackedV ? p.vt + sg.vt_off + (int64_t)head * ntiles * kVtTileElems : nullptr;

  // Q^T operand: lane holds query row q0 + l32, channels 16*kc + 8*hh .. +7.
  const int q0 = qb * (kNW * QPW) + wave * QPW;
  const int qrow = min(q0 + l32, L - 1);  // rows past the end are computed, never stored
  bf16x8 qf[8];
  {
    const uint16_t* qptr = p.q + sg.q_off + (int64_t)head * D + (int64_t)qrow * p.q_sl + hh * 8;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) qf[kc] = *reinterpret_cast<const bf16x8*>(qptr + kc * 16);
  }

  // ---- global -> LDS tile loads.  A tile is 16 wave instructions of 4 rows
  // (1 KB); with n = 16 / kNW instructions per wave (2 for 8 waves, 4 for 4),
  // wave w issues instructions n*w .. n*w + n-1 of each K and V tile, whose
  // rows are (64 / kNW)*w + 4j + l/16 for its instruction j.
  // Lane l of an instruction fills LDS slot l%16 of row 4i + l/16, i.e. it
  // loads the chunk the row's swizzle puts in that slot; the 16 lanes of a row
  // still read its 256 contiguous bytes.  Byte offsets from the tile's first
  // row are fixed per lane (32 bits: a tile spans 64 rows), so a full tile
  // costs no vector arithmetic; only the last, partial tile clamps its rows.
  const int ld_row0 = kRowsPerWave<kNW> * wave + (lane >> 4);
  const uint32_t row_bytes = (uint32_t)(sl * 2);
  int ld_kc[kMaxLoadsPerWave], ld_vc[kMaxLoadsPerWave];
  uint32_t lk[kMaxLoadsPerWave], lv[kMaxLoadsPerWave];
#pragma unroll
  for (int j = 0; j < kLoadsPerWave<kNW>; ++j) {
    ld_kc[j] = (lane & 15) ^ ((ld_row0 + 4 * j) & 15);
    ld_vc[j] = (lane & 15) ^ ((ld_row0 & 3) << 2);  // rows 4 apart swizzle alike
    lk[j] = (ld_row0 + 4 * j) * row_bytes + ld_kc[j] * 16;
    lv[j] = (ld_row0 + 4 * j) * row_bytes + ld_vc[j] * 16;
  }
  auto load_tile = [&](const uint16_t* g, unsigned char* buf, int tile, const uint32_t (&o)[kMaxLoadsPerWave],
                       const int (&c)[kMaxLoadsPerWave]) {
    const unsigned char* tb = (const unsigned char*)(g + (int64_t)tile * BN * sl);
    unsigned char* dst = buf + wave * (kLoadsPerWave<kNW> * 1024);
    if (tile * BN + BN > Lk) {  // partial last tile: clamp to the last valid row
      const int lim = Lk - 1 - tile * BN;
      uint32_t co[kMaxLoadsPerWave];
#pragma unroll
      for (int j = 0; j < kLoadsPerWave<kNW>; ++j) co[j] = (uint32_t)min(ld_row0 + 4 * j, lim) * row_bytes + c[j] * 16;
#pragma unroll
      for (int j = 0; j < kLoadsPerWave<kNW>; ++j)
        __builtin_amdgcn_global_load_lds(tb + co[j], (HV_LDS void*)(dst + j * 1024), 16, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < kLoadsPerWave<kNW>; ++j)
        __builtin_amdgcn_global_load_lds(tb + o[j], (HV_LDS void*)(dst + j * 1024), 16, 0, 0);
    }
  };
  auto load_k = [&](auto st, int tile) { load_tile(Kg, kbuf(st), tile, lk, ld_kc); };
  // Packed V tile: 128 rows of 128 bytes, instruction i = kLoadsPerWave<kNW>*w + j covers
  // rows 8i .. 8i+7; lane l fills slot l%8 of row 8i + l/8 with the chunk the
  // row's swizzle (slot c ^ ((row / 2) % 8)) puts there.  Full tiles only:
  // keys past the end are zeros in the workspace.
  uint32_t lt[kMaxLoadsPerWave];
#pragma unroll
  for (int j = 0; j < kLoadsPerWave<kNW>; ++j)
    lt[j] = (8 * (kLoadsPerWave<kNW> * wave + j) + (lane >> 3)) * 128 + (((lane & 7) ^ ((4 * j + (lane >> 4)) & 7)) << 4);
  auto load_v = [&](auto st, int tile) {
    if constexpr (kPackedV) {
      // opaque per call: keeps the scalar tile base + 32-bit lane offset form
      // instead of 64-bit per-lane addresses hoisted out of the loop
#pragma unroll
      for (int j = 0; j < kLoadsPerWave<kNW>; ++j) asm volatile("" : "+v"(lt[j]));
      const unsigned char* tb = (const unsigned char*)(Vt + (int64_t)tile * kVtTileElems);
      unsigned char* dst = vbuf(st) + wave * (kLoadsPerWave<kNW> * 1024);
#pragma unroll
      for (int j = 0; j < kLoadsPerWave<kNW>; ++j)
        __builtin_amdgcn_global_load_lds(tb + lt[j], (HV_LDS void*)(dst + j * 1024), 16, 0, 0);
    } else {
      load_tile(Vg, vbuf(st), tile, lv, ld_vc);
    }
  };

  // Operand offsets inside a tile.  The swizzle only depends on the row modulo
  // 16, so moving 16 rows (V key groups) or 32 rows (K halves) is a plain
  // immediate; the lane-dependent XOR is folded into 16 per-lane offsets.
  //
  // K operand (rows half*32 + l32, channel chunk 2kc + hh): one 16-byte read.
  int koff[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) koff[kc] = kswz(l32, 2 * kc + hh);
  // V^T operand for channels 32dt + l32 and keys 16mm + 8(e/4) + 4hh + e%4
  // (slot e), matching the register layout of P^T.  The offsets include the
  // LDS address of the first V stage (the V stages lie above 64 KB), so that
  // stage and dt/mm offsets fold into the instruction's offset field.
  const int vbase = (int)(uint32_t)(uintptr_t)(HV_LDS unsigned char*)sV0;
  int voff[4];
  if constexpr (kPackedV) {
    // packed tile: row 32dt + l32, 16-byte chunk 2mm + hh (positions 16mm + 8hh
    // .. +7, i.e. exactly the slot-e keys above) at slot (2mm + hh) ^ ((l32 / 2) % 8);
    // dt moves 32 rows = 4 KB, an immediate
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) voff[mm] = vbase + l32 * 128 + (((2 * mm + hh) ^ ((l32 >> 1) & 7)) << 4);
  } else {
    // ds_read_b64_tr_b16: in each group of 16 lanes, lane j receives element
    // j%4 of the 8-byte rows that lanes j/4, j/4+4, j/4+8, j/4+12 address.
    // Lane p of a group addresses key (base + p/4), channels d0 + 4(p%4) ..
    // +3, so lane j ends up with channel d0 + j of keys base .. base+3.  Keys 8
    // further are 8 rows = 2 KB further with the same swizzle (an immediate);
    // only dt changes the swizzled slot.
    const int tr_key = 4 * hh + ((lane & 15) >> 2);
    const int tr_ch = 16 * ((lane & 31) >> 4) + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int ch = 32 * dt + tr_ch;
      voff[dt] = vbase + vswz(tr_key, ch >> 3) + 2 * (ch & 7);
    }
  }
  // Re-declared opaque once per step, so the compiler keeps the 16 offsets in
  // registers and folds array base + stage-free immediates into the ds_read
  // offset fields, instead of hoisting every (offset + immediate) sum.
  auto refresh_offsets = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(koff[i]));
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(voff[i]));
  };
  auto k_frag = [&](auto st, int half, int kc) {
    return *reinterpret_cast<const bf16x8*>(kbuf(st) + koff[kc] + half * 32 * ROWB);
  };
  auto v_frag = [&](auto st, int dt, int mm) {
    unsigned char* vb = vbuf(st) - vbase;
    if constexpr (kPackedV) {
      return *(const HV_LDS bf16x8*)(HV_LDS unsigned char*)(vb + voff[mm] + dt * 32 * 128);
    } else {
      const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HV_LDS i16x4*)(vb + voff[dt] + mm * 16 * ROWB));
      const i16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HV_LDS i16x4*)(vb + voff[dt] + 8 * ROWB + mm * 16 * ROWB));
      const u32x4 w = {__builtin_bit_cast(u32x2, a)[0], __builtin_bit_cast(u32x2, a)[1],
                       __builtin_bit_cast(u32x2, c)[0], __builtin_bit_cast(u32x2, c)[1]};
      return __builtin_bit_cast(bf16x8, w);
    }
  };

  f32x16 o[4];
  float m_run;  // reference, log2 domain
  float l_run;  // this lane's share of the denominator (bf16-rounded weights)
  const float c2 = p.scale_log2;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

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

  // The block's computation, in one of two modes.
  //   kTrack = false (every block starts here): the reference m starts at
  //     the row maximum of tile 0; no later tile's maximum is computed.
  //     Instead the row's sum of weights, which bounds each weight, is kept
  //     below 2^40 by raising m in steps of 32 (bound_weights): one compare
  //     per step instead of a 32-value maximum.  The weights stay finite
  //     unless a tile's scores jump far (over 2^80) above everything before
  //     them, and the result is exact either way (every weight of a row
  //     carries the row's reference, which cancels in O / l).
  //   kTrack = true: the reference follows the row maximum tile by tile
  //     (raised lazily, see update_reference), so every weight is <= 2^8.
  //     A block whose sum of weights is not below 2^64 (or not finite) after
  //     the fast mode is run again in this mode.
  auto run = [&](auto track) __attribute__((always_inline)) {
  constexpr bool kTrack = decltype(track)::value;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;
  m_run = -INFINITY;
  l_run = 0.f;

  // ---- prologue: K tiles 0..3 and V tiles 0..2 requested; scores of tile 0
  load_k(I0{}, 0);
  load_k(I1{}, min(1, ntiles - 1));
  load_k(I2{}, min(2, ntiles - 1));
  load_k(I3{}, min(3, ntiles - 1));
  load_v(I0{}, 0);
  load_v(I1{}, min(1, ntiles - 1));
  load_v(I2{}, min(2, ntiles - 1));
  // Each wave's loads complete in the order issued: its eight Q loads, then
  // kLoadsPerWave<kNW> instructions per tile, K 0..3 and V 0..2.  Tile 0's scores wait only
  // for Q and K tile 0 (six tiles may still be in flight), so the first
  // MFMAs start one tile's latency after the block begins instead of seven.
  barrier_after<6 * kLoadsPerWave<kNW>>();
  f32x16 sa[2], sb[2];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    sa[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(I0{}, 0, kc), qf[kc], kc ? sa[0] : zero16, 0, 0, 0);
    sa[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(I0{}, 1, kc), qf[kc], kc ? sa[1] : zero16, 0, 0, 0);
  }
  if (ntiles == 1) mask_tile(sa[0], sa[1], Lk, hh);
  update_reference(tile_max(sa[0], sa[1], c2), m_run, l_run, o);
  barrier_after<5 * kLoadsPerWave<kNW>>();  // K tile 1 in place
  // K operands of the first step (tile 1) are read, and its first two QK^T
  // MFMAs issued, before its barrier (see the end of a step)
  bf16x8 kf[4];
  kf[0] = k_frag(I1{}, 0, 0);
  kf[1] = k_frag(I1{}, 1, 0);
  kf[2] = k_frag(I1{}, 0, 1);
  kf[3] = k_frag(I1{}, 1, 1);
  sb[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qf[0], zero16, 0, 0, 0);
  sb[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[1], qf[0], zero16, 0, 0, 0);
  kf[0] = k_frag(I1{}, 0, 2);
  kf[1] = k_frag(I1{}, 1, 2);
  // K tiles 2, 3 and V tile 0 in place for the first step (V tiles 1 and 2 may
  // still be in flight: the first step's barrier waits for them), and every
  // wave has read K tile 0 before its buffer is refilled
  barrier_after<2 * kLoadsPerWave<kNW>>();

  // ---- steady state.  Step t (tile t+1 exists; U = t % 4 at compile time),
  // in fixed instruction order (sched_barrier fences between bundles keep the
  // compiler from regrouping):
  //   phase 1: QK^T MFMAs of tile t+1 (its first chunk was issued before the
  //            previous barrier, the operands of the next two were read there,
  //            the rest two chunks ahead), interleaved with the exp2 / bf16 /
  //            sum work for keys 0..31 of tile t, spread evenly over the chunks;
  //   phase 2: PV MFMAs of tile t (V operands read two MFMAs ahead, the first
  //            two already during phase 1); the first ten carry the exp2
  //            work for keys 32..63 (with the two packs in slots of their
  //            own), the last eight the row maximum of tile t+1, so the VALU
  //            work is spread over the whole phase; the first K
  //            operands of tile t+2 are read at its 11th MFMA and the requests
  //            for K tile t+4 and V tile t+3 go out at its 13th and 15th;
  //   then the first chunk of QK^T MFMAs of tile t+2 (into the score
  //   registers of tile t, free by then), so that the MFMA pipe has work
  //   queued while the waves meet at the barrier, and the operands of its
  //   second and third chunks; one barrier and the reference update.
  // K tile t+1 and V tile t were requested three steps earlier (or in the
  // prologue); every barrier waits for the loads of the step before it, so a
  // tile is complete and visible from the barrier that follows its request
  // step by one.
  auto step = [&](auto u, int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    constexpr int U = decltype(u)::value;
    using KS = std::integral_constant<int, (U + 1) % NSTAGE>;   // K tile t+1
    using VS = std::integral_constant<int, U>;                  // V tile t
    using KN = std::integral_constant<int, (U + 2) % NSTAGE>;   // K tile t+2
    using KL = std::integral_constant<int, U>;                  // K tile t+4 goes here
    using VL = std::integral_constant<int, (U + 3) % NSTAGE>;   // V tile t+3 goes here
    refresh_offsets();
    bf16x8 pb[4];
    bf16x8 vf[2];  // V operands, two MFMAs ahead in the PV phase
#pragma unroll
    for (int kc = 1; kc < 8; ++kc) {  // chunk 0 was issued before the barrier
      __builtin_amdgcn_sched_barrier(0);
      const int sl0 = 2 * (kc & 1);
      nxt[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[sl0], qf[kc], nxt[0], 0, 0, 0);
      // keys 0..31 of tile t: pairs 0,1 | 2,3 | pack | 4 | 5 | 6,7 | pack
      if (kc == 1) { exp_pair(cur, 0); exp_pair(cur, 2); }
      if (kc == 2) { exp_pair(cur, 4); exp_pair(cur, 6); }
      if (kc == 4) exp_pair(cur, 8);
      if (kc == 5) exp_pair(cur, 10);
      if (kc == 6) { exp_pair(cur, 12); exp_pair(cur, 14); }
      nxt[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[sl0 + 1], qf[kc], nxt[1], 0, 0, 0);
      if (kc == 5) {  // the first two V operands of the PV phase (tile t is visible)
        vf[0] = v_frag(VS{}, 0, 0);
        vf[1] = v_frag(VS{}, 1, 0);
      }
      if (kc == 3) pb[0] = pack_p(cur, 0);
      if (kc == 7) pb[1] = pack_p(cur, 1);
      if (kc + 2 < 8) {
        kf[sl0] = k_frag(KS{}, 0, kc + 2);
        kf[sl0 + 1] = k_frag(KS{}, 1, kc + 2);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // keep phase-1 results where they are computed (not sunk past the branch)
    asm volatile("" ::"v"(pb[0]), "v"(pb[1]));
    if (t + 2 == ntiles) mask_tile(nxt[0], nxt[1], Lk - (t + 1) * BN, hh);

    float part_run = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const int mm = i >> 2, dt = i & 3;
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i & 1], pb[mm], o[dt], 0, 0, 0);
      if (i + 2 < 16) vf[i & 1] = v_frag(VS{}, (i + 2) & 3, (i + 2) >> 2);
      // keys 32..63 of tile t, packed before PV chunks 2 and 3 need them
      if (i < 4) exp_pair(cur, 16 + 2 * i);
      if (i == 4) pb[2] = pack_p(cur, 2);
      if (i >= 5 && i < 9) exp_pair(cur, 16 + 2 * (i - 1));
      if (i == 9) pb[3] = pack_p(cur, 3);
      // requests for K tile t+4 and V tile t+3 (their stages, of K tile t and
      // V tile t-1, are free since the last barrier); placed late in the PV
      // phase, where they cost least (measured)
      if (i == 12) load_k(KL{}, min(t + KAHEAD, ntiles - 1));
      if (i == 14) load_v(VL{}, min(t + VAHEAD, ntiles - 1));
      if (i == 10) {  // first K operands of tile t+2 (the QK^T phase is done with kf)
        kf[0] = k_frag(KN{}, 0, 0);
        kf[1] = k_frag(KN{}, 1, 0);
        kf[2] = k_frag(KN{}, 0, 1);
        kf[3] = k_frag(KN{}, 1, 1);
      }
      if (kTrack && i >= 8) {  // row maximum of tile t+1, in eight pieces of one chain
        const int j = i - 8;
        const f32x16& sv = nxt[j >> 2];
        const int b = 4 * (j & 3);
        float m = j ? vmax(vmax(part_run, sv[b]), sv[b + 1]) : vmax(sv[b], sv[b + 1]);
        m = vmax(vmax(m, sv[b + 2]), sv[b + 3]);
        part_run = m;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    const float mx = kTrack ? max_across_halves(part_run) * c2 : 0.f;
    __builtin_amdgcn_sched_barrier(0);
    // chunk 0 of tile t+2 (after the last step: a tile that is never used)
    cur[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qf[0], zero16, 0, 0, 0);
    cur[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[1], qf[0], zero16, 0, 0, 0);
    kf[0] = k_frag(KN{}, 0, 2);
    kf[1] = k_frag(KN{}, 1, 2);
    __builtin_amdgcn_sched_barrier(0);
    // the loads just issued (two tiles) stay in flight, and so may the two reads of K
    // tile t+2 (its stage is not refilled before the next barrier)
    barrier_after<2 * kLoadsPerWave<kNW>, 2>();
    if constexpr (kTrack) update_reference(mx, m_run, l_run, o);
    else bound_weights(m_run, l_run, o);
  };

  const int last = ntiles - 1;  // steps run for t = 0 .. last-1
  int t = 0;
  for (; t + 4 <= last; t += 4) {  // branch-free body: four full steps
    step(I0{}, t, sa, sb);
    step(I1{}, t + 1, sb, sa);
    step(I2{}, t + 2, sa, sb);
    step(I3{}, t + 3, sb, sa);
  }
  if (t < last) step(I0{}, t, sa, sb);
  if (t + 1 < last) step(I1{}, t + 1, sb, sa);
  if (t + 2 < last) step(I2{}, t + 2, sa, sb);
  // scores of the last tile: sa if it is tile 0, 2, 4, ...
  if (last & 1) {
#pragma unroll
    for (int v = 0; v < 16; ++v) { sa[0][v] = sb[0][v]; sa[1][v] = sb[1][v]; }
  }

  // ---- last tile: softmax and PV only
  {
    bf16x8 pb[4];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      exp_pair(sa, 4 * kc);
      exp_pair(sa, 4 * kc + 2);
      if (kc & 1) pb[kc >> 1] = pack_p(sa, kc >> 1);
    }
    auto final_pv = [&](auto st) {
#pragma unroll
      for (int mm = 0; mm < 4; ++mm)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(st, dt, mm), pb[mm], o[dt], 0, 0, 0);
    };
    switch (last % NSTAGE) {
      case 0: final_pv(I0{}); break;
      case 1: final_pv(I1{}); break;
      case 2: final_pv(I2{}); break;
      default: final_pv(I3{}); break;
    }
  }
  // no LDS access follows; drain the remaining (dead) tile loads
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  };  // run

  run(std::false_type{});
  if constexpr (kPackedV) {
    if (tid == 0) s_block[(iter + 1) & 1] = next_block;
  }
  float l_tot = sum_across_halves(l_run);
  // every wave of the block joins (the waves share the K/V tiles in LDS)
  if (__syncthreads_or(!(l_tot < 0x1p64f))) {
    run(std::true_type{});
    l_tot = sum_across_halves(l_run);
    // the next block's first tile loads must not overwrite LDS that a slower
    // wave of this block still reads
    __syncthreads();
  }

  // ---- epilogue: O / l, round to bf16, store rows that exist; optionally
  // the natural-log log-sum-exp of the row's logits: the weights summed in l
  // are 2^(s*c2 - m), so sum_j e^(scale*s_j) = 2^m * l.
  const float inv = 1.0f / l_tot;
  const int orow = q0 + l32;
  if (orow < L) {
    uint16_t* op = p.out + sg.o_off + (int64_t)head * D + (int64_t)orow * p.o_sl;
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
    if (p.lse != nullptr && hh == 0)
      p.lse[sg.lse_off + (int64_t)head * p.lse_hstride + orow] =
          (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
  }  // block loop
}

}  // namespace

hipError_t launch_attn_fwd(AttnParams& p, hipStream_t stream) {
  int blocks = 0;
  int64_t vt_elems = 0;
  VtParams vp;
  vp.v = p.v;
  vp.vt = p.vt;
  vp.counter = nullptr;
  vp.kv_sl = p.kv_sl;
  vp.n_seg = p.n_seg;
  vp.n_blocks = 0;
  // query blocks of 128 rows (kWavesSmall) and of 256 rows (kWavesLarge)
  int64_t blocks_small = 0, blocks_large = 0;
  for (int i = 0; i < p.n_seg; ++i) {
    blocks_small += HV_HEADS * ((p.seg[i].q_len + kWavesSmall * QPW - 1) / (kWavesSmall * QPW));
    blocks_large += HV_HEADS * ((p.seg[i].q_len + kWavesLarge * QPW - 1) / (kWavesLarge * QPW));
  }
  int cus = 0;
  if (blocks_large > 0) {
    // compute units of the current device, looked up once per device
    static int cu_count[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
    cus = dev >= 0 && dev < 64 ? __atomic_load_n(&cu_count[dev], __ATOMIC_RELAXED) : 0;
    if (cus <= 0) {
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipGetLastError();
      if (cus <= 0) return hipErrorInvalidDevice;
      if (dev >= 0 && dev < 64) __atomic_store_n(&cu_count[dev], cus, __ATOMIC_RELAXED);
    }
  }
  // blocks of 128 query rows when they all fit in one round of workgroups
  const bool small = blocks_small <= cus;
  const int bm = (small ? kWavesSmall : kWavesLarge) * QPW;
  for (int i = 0; i < p.n_seg; ++i) {
    AttnSegment& sg = p.seg[i];
    sg.nqb = (sg.q_len + bm - 1) / bm;
    sg.blk_begin = blocks;
    blocks += HV_HEADS * sg.nqb;
    // packed V only for segments with query rows
    const int nt = sg.q_len > 0 ? (sg.k_len + BN - 1) / BN : 0;
    sg.vt_off = vt_elems;
    VtSegment& vs = vp.seg[i];
    vs.k_off = sg.k_off;
    vs.vt_off = vt_elems;
    vs.k_len = sg.k_len;
    vs.ntiles = nt;
    vs.blk_begin = vp.n_blocks;
    vs.pad_ = 0;
    vp.n_blocks += HV_HEADS * nt;
    vt_elems += (int64_t)HV_HEADS * nt * kVtTileElems;
  }
  p.n_blocks = blocks;
  if (blocks == 0) return hipSuccess;
  // A call whose blocks all run in the first round (one workgroup per CU)
  // gains nothing from sharing them out by a counter, and V packing (one more
  // launch and pass over V) costs it more than the transposing reads do: it
  // reads V in place (bitwise the same results).
  if (blocks <= cus) p.vt = nullptr;
  if (p.vt != nullptr) {
    // the work counter follows the packed tiles
    p.counter = vp.counter = reinterpret_cast<int*>(p.vt + vt_elems);
    const hipError_t e = launch_v_pack(vp, stream);
    if (e != hipSuccess) return e;
    // one persistent workgroup per CU (128 KB of LDS: one fits per CU)
    attn_fwd_kernel<true, kWavesLarge><<<dim3((unsigned)min(blocks, cus)), dim3(kWavesLarge * 64), 0, stream>>>(p);
  } else if (small) {
    attn_fwd_kernel<false, kWavesSmall><<<dim3((unsigned)blocks), dim3(kWavesSmall * 64), 0, stream>>>(p);
  } else {
    attn_fwd_kernel<false, kWavesLarge><<<dim3((unsigned)blocks), dim3(kWavesLarge * 64), 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace hv
