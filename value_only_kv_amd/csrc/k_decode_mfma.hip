// k_decode_mfma.hip - matrix-core split decode for Grouped Value Attention (bf16 cache, gfx950).
//
// What is computed (same as the vector-ALU kernel): for head h of group g = g(h) and cached
// position j, the score q~_h . v_{j,g} + r_h . kr_j ("GVA：KV 缓存里的 Key 其实可以不存",
// shibing624.github.io review of arXiv:2609.13285, sections 关键技巧一 and 关键技巧二), a softmax
// over the positions and the weighted sum of the same cached values (agihunt.info summary of
// the paper). All H/G heads of a group share one value stream, so a tile of V is read from HBM
// once and serves every head of its group; the positional key is shared by all groups.
//
// Why matrix cores: per cached bf16 element the H/G heads of a group need H/G multiply-adds for
// the scores and H/G for the weighted sum; at H/G = 4 that is 4 FMA per byte, which the vector
// ALU cannot sustain at HBM speed. Both products are dense [H/G x d] x [d x tokens] contractions
// and go to v_mfma_f32_16x16x32_bf16.
//
// Layout facts of v_mfma_f32_16x16x32_bf16 used below (checked on the hardware):
//   A[i][k]: lane i + 16 (k / 8), element k % 8;  B[k][j]: lane j + 16 (k / 8), element k % 8;
//   D[i][j]: lane j + 16 (i / 4), register i % 4.
// Write n = lane % 16 (a row of 16 lanes) and q = lane / 16.
//
// One wave per (chunk, group). Chunks come from one of two work plans (see the kernel):
// per-sequence splits, or equal ranges over the tiles of all sequences (balanced). In the
// balanced plan with G a multiple of 8, a work-group holds eight groups of the same range (one
// work-group per CU) and only its wave 0 fetches the shared positional key; it passes each tile's
// key to the other seven through LDS, one barrier per tile. Concurrent misses on the same line
// are not merged by the caches, so letting every wave fetch the key read it two to three times
// from HBM (2.9% more traffic on the ragged batch). Otherwise a work-group holds four groups
// and every wave fetches the key, and the work-groups of one chunk take ids 8 apart so that they
// run on the same XCD. A chunk is walked in tiles of 32 positions, two blocks of 16 (tb = 0, 1):
//   1. V rows go straight from HBM into registers in A-operand form: lane (n, q) loads 16 bytes,
//      8 consecutive dims 32 ks + 8 q .. of position 16 tb + n, for every k-step ks.
//   2. Scores S^T[t][c] = sum_k V[t][k] Q[c][k]. The query keeps ~16 significant bits by being
//      split into bf16 hi + lo parts. With NH heads per group (NH <= 8) column c < NH holds
//      head c's hi part and column NH + c its lo part, so one MFMA forms both; a row shift by NH
//      lanes (DPP) adds them, and lane (NH + c, q) then owns head c's scores of positions
//      16 tb + 4 q + r, r = 0..3. (Other head counts use separate hi and lo MFMAs; then lane
//      (c, q) owns head c.)
//   3. Online softmax per head in the base-2 domain; the tile max needs two lane exchanges.
//   4. The weighted sum O^T[d][c] = sum_t V[t][d] P[c][t] contracts over positions, so V is
//      needed with positions along K. The wave copies its tile rows to a private LDS area and
//      reads them back with the transposing LDS load (ds_read_b64_tr_b16), which yields V^T in
//      A-operand form with K order (q, e) -> 16 (e / 4) + 4 q + e % 4. That is exactly the order
//      in which each lane already holds its probabilities, so the B operand (P split into hi and
//      lo parts, laid out like the query columns) is built from registers, with one more row
//      shift to place the hi parts.
//   5. O^T accumulates in registers: lane (n, q) holds column n, dims 16 nb + 4 q + r; the hi
//      and lo columns are added once, at the end.
// The four-wave layout needs 168 registers at d_h = 128, so three work-groups share a compute
// unit (transposing V with selection-matrix MFMAs instead of the LDS load needed 250); the
// eight-wave layout is alone on its CU and may use up to 256.
//
// The same template, with GQA = true, decodes the comparator cache of a matched grouped-query
// model (G keys and G values per token): the score then contracts key rows loaded beside the
// value rows, and there is no positional term.
#include <hip/hip_runtime.h>

#include <math.h>

#include "gva_device.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kTile = 32;
constexpr int kGroupWaves = gva::kDecodeGroupWaves;

// Per-wave LDS copy of one tile: 32 rows (positions) of d_h bf16 values, each row padded by 32
// bytes. The padding puts the four rows that one transposing read touches in every group of 16
// lanes on different banks.
template <int KS>
struct TileLds {
  static constexpr int kRow = 64 * KS + 32;   // bytes per row
  static constexpr int kWave = kTile * kRow;  // bytes per wave
};

// ds_read_b64_tr_b16 (checked on the hardware): in each group of 16 lanes, lanes 4 e + k
// (k = 0..3) address 4 consecutive 16-bit elements each, together one row of 16; lane i of the
// group receives element e of its result from row e, column i. So lane L addressing row L / 4,
// columns 4 (L % 4) .. + 3 of a row-major tile receives column L % 16 of rows 4 (L / 16) .. + 3.
__device__ __forceinline__ i16x4 read_tr(const uint8_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16(const u32x4 &u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ unsigned pack2(float x, float y) {
  const f32x2 v = {x, y};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));  // RNE, x in low half
}

__device__ __forceinline__ float low_bf16(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float high_bf16(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Lane i of each row of 16 receives lane i - S (row_shr) or i + S (row_shl); lanes with no
// source receive 0.
template <int S>
__device__ __forceinline__ unsigned row_shr(unsigned v) {
  return static_cast<unsigned>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x110 + S, 0xf, 0xf, true));
}
template <int S>
__device__ __forceinline__ unsigned row_shl(unsigned v) {
  return static_cast<unsigned>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x100 + S, 0xf, 0xf, true));
}
template <int S>
__device__ __forceinline__ float row_shr_f(float v) {
  return __uint_as_float(row_shr<S>(__float_as_uint(v)));
}
template <int S>
__device__ __forceinline__ float row_shl_f(float v) {
  return __uint_as_float(row_shl<S>(__float_as_uint(v)));
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): ~16 significant bits in two bf16 values.
__device__ __forceinline__ void split8(const float (&x)[8], u32x4 &hi, u32x4 &lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned w = pack2(x[2 * i], x[2 * i + 1]);
    hi[i] = w;
    lo[i] = pack2(x[2 * i] - low_bf16(w), x[2 * i + 1] - high_bf16(w));
  }
}

// GQA == true is the comparator: a cache of G keys and G values per token, where the score
// contracts the key rows (d_h wide) instead of [value row | positional key row].
template <int KS, bool GQA>
struct Tile {
  u32x4 v[2][KS];                  // V rows in A-operand form, per position block and k-step
  u32x4 x[2][GQA ? KS : 1];        // GVA: positional key rows; GQA: key rows, like v
};

// A 16-byte load of cache rows that this launch reads once, marked non-temporal. Measured on a
// plain streaming read of the ragged batch's 9.35 GB: 6.23 TB/s with ordinary loads, 7.10 TB/s
// with non-temporal ones, but only when every load instruction covers whole 128-byte lines
// (with the matrix-operand layout, where an instruction reads 64 bytes of each of 16 rows, the
// non-temporal loads were no faster, and the decode was slower: the second half of each line
// was fetched again). Hence the line layout below.
__device__ __forceinline__ u32x4 stream_load(const uint16_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Line layout of a 16-position block's value loads, for d_h = 32 KS with KS a power of two:
// a row is 64 KS bytes (4 KS chunks of 16), and load k of lane L reads chunk L mod 4 KS of row
// k (16 / KS) + L / (4 KS). Each load instruction then reads whole rows (1 KiB of consecutive
// chunks when the group's rows are adjacent, whole 128-byte lines of each row otherwise, for
// d_h >= 64). The rows go to the wave's LDS tile as they are, and the score operand is read
// back from there in the matrix-operand layout.
template <int KS>
constexpr bool kLine = (KS & (KS - 1)) == 0;
template <int KS>
__device__ __forceinline__ int line_chunk(int lane) { return lane & (4 * KS - 1); }
template <int KS>
__device__ __forceinline__ int line_row(int lane, int k) { return k * (16 / KS) + lane / (4 * KS); }

// Block-table entries of the two 16-position blocks of the tile at t0 (clamped to c1 - 1):
// even lanes hold the first block's entry, odd lanes the second's. The per-lane address makes
// this a vector load, so it completes in order with the V loads; it is issued a tile ahead and
// ordered before the previous tile's V loads, so waiting for it never waits for V data in
// flight. (A scalar load here would share the counter of the cross-lane exchanges and stall.)
__device__ __forceinline__ int32_t load_pages(const int32_t *__restrict__ bt, int log2_bs, int t0,
                                              int c1, int lane) {
  return bt[min(t0 + 16 * (lane & 1), c1 - 1) >> log2_bs];
}

// Loads the 32 positions starting at t0 as two blocks of 16. Every load is issued
// unconditionally, so the number of loads in flight is the same on every path and each tile
// waits only for its own data. A block lies inside one cache block (block_size >= 16 and t0 is a
// multiple of 16), so one table entry serves all of its lanes. Positions >= c1 read position
// c1 - 1 instead (finite data from a block that is cached already); their scores are masked, so
// they add exactly zero. vgrp is the value group's element offset, klane the lane-invariant
// part of the positional key's. V is loaded in the line layout when kLine<KS> (T.v[tb][k] =
// load k of block tb), else in the matrix-operand layout (T.v[tb][ks] = dims 32 ks + 8 q ..
// of row n); the keys of the comparator (GQA) always in the operand layout.
// SHARE: only the waves with fetch_key read the positional key (the others read a row of their
// own work-group, kown, which stays in cache, and take the key from LDS instead); every load is
// still issued, so the loads in flight stay the same on every path.
template <int KS, bool GQA, bool SHARE>
__device__ __forceinline__ void load_tile(const gva::DecodeArgs &a, int32_t P, int t0, int c1,
                                          int n, int64_t vgrp, int64_t klane, Tile<KS, GQA> &T,
                                          bool &bad, bool fetch_key, int64_t kown) {
  const int mask = (1 << a.log2_bs) - 1;
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const uint16_t *vbase = static_cast<const uint16_t *>(a.v);
  const uint16_t *kbase = static_cast<const uint16_t *>(a.kr);
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int32_t pb = __builtin_amdgcn_readlane(P, tb);
    const bool ok = pb >= 0 && static_cast<int64_t>(pb) < a.num_blocks;
    bad |= !ok;
    const int64_t blk = ok ? pb : 0;
    const int f = min(t0 + 16 * tb, c1 - 1);          // first position read by this block
    const int lim = c1 - 1 - f;                        // rows past it read row lim
    const int rn = min(n, lim);                        // the operand layout's row (clamped)
    const int64_t row = static_cast<int64_t>((f & mask) + rn);
    const uint16_t *vblk = vbase + blk * a.v_sb + static_cast<int64_t>(f & mask) * a.v_st + vgrp;
    if constexpr (kLine<KS>) {
      const int ch = 8 * line_chunk<KS>(lane);
#pragma unroll
      for (int k = 0; k < KS; ++k)
        T.v[tb][k] = stream_load(vblk + static_cast<int64_t>(min(line_row<KS>(lane, k), lim)) * a.v_st + ch);
    } else {
      const uint16_t *vp = vblk + static_cast<int64_t>(rn) * a.v_st + 8 * q;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) T.v[tb][ks] = *reinterpret_cast<const u32x4 *>(vp + 32 * ks);
    }
    if constexpr (GQA) {
      const uint16_t *kp = static_cast<const uint16_t *>(a.k) + blk * a.v_sb + row * a.v_st + vgrp + 8 * q;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) T.x[tb][ks] = *reinterpret_cast<const u32x4 *>(kp + 32 * ks);
      (void)kbase;
      (void)klane;
      (void)fetch_key;
      (void)kown;
    } else {
      const int64_t koff = !SHARE || fetch_key ? blk * a.kr_sb + row * a.kr_st : kown;
      T.x[tb][0] = *reinterpret_cast<const u32x4 *>(kbase + koff + klane);
    }
  }
}

// Per-wave state of the online softmax and the accumulators.
template <int KS>
struct Acc {
  f32x4 O[2 * KS];
  float m;
  float lsum;
};

// One tile: scores, online softmax and the weighted sum. NH > 0: merged hi/lo columns (see the
// file comment); NH == 0: separate hi and lo MFMAs with QX = hi and QY = lo.
// SHARE: the positional key comes from the work-group's LDS copy (this lane's 16 bytes of
// block 0 at kx, of block 1 at kx + 1024) instead of the tile's registers.
template <int KS, int NH, bool GQA, bool SHARE>
__device__ __forceinline__ void tile_step(const Tile<KS, GQA> &cur, int t0, int c1, int n, int q,
                                          const bf16x8 (&QX)[KS], const bf16x8 (&QY)[KS],
                                          const bf16x8 &RX, const bf16x8 &RY, uint8_t *lw_wr,
                                          uint8_t *lw_line, const uint8_t *lw_rd, Acc<KS> &acc,
                                          const uint8_t *kx) {
  constexpr int SH = NH > 0 ? NH : 1;
  using L = TileLds<KS>;
  // the tile's V rows go to the wave's LDS copy (row-major, rows of L::kRow bytes), to be read
  // back transposed for the weighted sum: from the line layout (lane's chunk of rows
  // line_row(k), at lw_line) or from the operand layout (row 16 tb + n, columns 32 ks + 8 q ..)
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (kLine<KS>)
        *reinterpret_cast<u32x4 *>(lw_line + (16 * tb + ks * (16 / KS)) * L::kRow) = cur.v[tb][ks];
      else
        *reinterpret_cast<u32x4 *>(lw_wr + tb * 16 * L::kRow + 64 * ks) = cur.v[tb][ks];
    }
  f32x4 S[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
    // the score operand: the value rows plus the positional key (GVA) or the key rows (GQA);
    // in the line layout the value rows are read back from LDS in the operand layout (the
    // wave's own LDS writes above complete first: LDS serves a wave's accesses in order)
    u32x4 vop[KS];
    if constexpr (kLine<KS> && !GQA) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        vop[ks] = *reinterpret_cast<const u32x4 *>(lw_wr + tb * 16 * L::kRow + 64 * ks);
    }
    const u32x4 *sx = GQA ? cur.x[tb] : (kLine<KS> ? vop : cur.v[tb]);
    // the positional key rows (GVA)
    const u32x4 kx_tb = SHARE ? *reinterpret_cast<const u32x4 *>(kx + 1024 * tb) : cur.x[tb][0];
    if (NH > 0) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s0 = mfma(as_bf16(sx[ks]), QX[ks], s0);
      if (!GQA) s0 = mfma(as_bf16(kx_tb), RX, s0);
#pragma unroll
      for (int r = 0; r < 4; ++r) s0[r] += row_shr_f<SH>(s0[r]);
    } else {
      f32x4 s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s0 = mfma(as_bf16(sx[ks]), QX[ks], s0);
        s1 = mfma(as_bf16(sx[ks]), QY[ks], s1);
      }
      if (!GQA) {
        s0 = mfma(as_bf16(kx_tb), RX, s0);
        s1 = mfma(as_bf16(kx_tb), RY, s1);
      }
      s0 += s1;
    }
    S[tb] = s0;
  }
  if (t0 + kTile > c1) {  // the last tile of the chunk: mask positions >= c1
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (t0 + 16 * tb + 4 * q + r >= c1) S[tb][r] = -INFINITY;
  }
  float mt = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                   fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float mn = fmaxf(acc.m, mt);
  float alpha = __builtin_amdgcn_exp2f(acc.m - mn);
  float p[8];
  float ps = 0.0f;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[4 * tb + r] = __builtin_amdgcn_exp2f(S[tb][r] - mn);
      ps += p[4 * tb + r];
    }
  acc.lsum = acc.lsum * alpha + ps;
  acc.m = mn;
  u32x4 ph, pl;
  split8(p, ph, pl);
  if (NH > 0) {
    // hi columns c < NH take the hi parts (and alpha) from their owner lanes NH + c
    const bool hi_col = n < NH;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned h = row_shl<SH>(ph[i]);
      pl[i] = hi_col ? h : pl[i];
    }
    const float a2 = row_shl_f<SH>(alpha);
    alpha = hi_col ? a2 : alpha;
  }
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) acc.O[i] *= alpha;
  }
  const bf16x8 PX = as_bf16(NH > 0 ? pl : ph);
  const bf16x8 PY = as_bf16(pl);
  // V^T in A-operand form, dims 16 nb + n, K order (q, e) -> position 16 (e / 4) + 4 q + e % 4:
  // the first read gives positions 4 q .. + 3 of block 0, the second the same of block 1.
#pragma unroll
  for (int nb = 0; nb < 2 * KS; ++nb) {
    const i16x4 v0 = read_tr(lw_rd + 32 * nb);
    const i16x4 v1 = read_tr(lw_rd + 16 * L::kRow + 32 * nb);
    const bf16x8 VT = __builtin_bit_cast(
        bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    acc.O[nb] = mfma(VT, PX, acc.O[nb]);
    if (NH == 0) acc.O[nb] = mfma(VT, PY, acc.O[nb]);
  }
}

// Waves per SIMD the register allocation must allow: three where the kernel fits in 168
// registers without spilling (d_h <= 64, or d_h = 128 with merged hi/lo columns), else two.
template <int KS, int NH, bool GQA, int WAVES>
constexpr int min_waves_per_simd() {
  // an 8-wave work-group is alone on its CU (two waves per SIMD) whatever its registers
  return WAVES == 8 ? 2 : !GQA && (KS <= 2 || (KS == 4 && NH > 0)) ? 3 : 2;
}

// The head in slot h0 + c of a.head_of, for a group of NH slots (1, 2, 4 or 8) starting at h0,
// a multiple of NH the whole wave agrees on. The slots are read as aligned 32-bit words with a
// uniform index, which compiles to scalar loads (a byte load from the kernel arguments, or a
// per-lane index, is a vector memory round trip), and the lane's byte is shifted out.
template <int NH>
__device__ __forceinline__ int slot_head(const gva::DecodeArgs &a, int h0, int c) {
  static_assert(NH == 1 || NH == 2 || NH == 4 || NH == 8, "slot_head: NH");
  const uint32_t *w = reinterpret_cast<const uint32_t *>(a.head_of) + (h0 >> 2);
  uint32_t word = w[0];
  if (NH == 8) word = (c & 4) ? w[1] : word;
  return static_cast<int>((word >> (8 * ((h0 & 3) + (c & 3)))) & 0xffu);
}

// The head of this lane's query column in group g: column n of the merged hi/lo layout reads
// slot g (H / G) + c, c = n mod NH (lanes past the columns read slot c = 0). With NH = 0 (more
// heads per group than merged columns) column n reads slot g (H / G) + n, a per-lane index.
template <int NH>
__device__ __forceinline__ int lane_head(const gva::DecodeArgs &a, int g, int n) {
  const int nhg = a.H / a.G;
  const int h0 = g * nhg;
  if constexpr (NH == 0) {
    return a.head_of[h0 + (n < nhg ? n : 0)];
  } else {
    const int c = n < NH ? n : (n < 2 * NH ? n - NH : 0);
    return slot_head<NH>(a, h0, c);
  }
}

// One chunk of positions [c0, c1) of sequence b for value group g (one wave): scores, online
// softmax and weighted sum over its tiles, then the partial (m, l, o) of each of the group's heads
// h at workspace row prow0 + h or, when `direct`, the final output row. len_bad makes the output
// row NaN (its chunk is empty). lds is the work-group's LDS tile area.
template <int KS, int NH, bool GQA, bool SHARE>
__device__ __forceinline__ void run_chunk(const gva::DecodeArgs &a, int b, int g, int c0, int c1,
                                          bool len_bad, bool direct, int64_t prow0,
                                          uint8_t *lds, uint8_t *kbuf) {
  constexpr int SH = NH > 0 ? NH : 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int q = lane >> 4;
  const int nhg = a.H / a.G;
  const bool col_ok = NH > 0 ? (n < 2 * NH) : (n < nhg);
  const bool use_lo = NH > 0 && n >= NH;
  const int head_lane = lane_head<NH>(a, __builtin_amdgcn_readfirstlane(g), n);
  // the lanes that own a head's softmax state and output
  const bool owner = NH > 0 ? (n >= NH && n < 2 * NH) : (n < nhg);
  const int row_len = a.d_h + a.d_r;
  const float qnan = __int_as_float(0x7fc00000);

  Acc<KS> acc;
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i) acc.O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  acc.m = -INFINITY;
  acc.lsum = 0.0f;
  bool bad = false;

  if (c0 < c1) {
    // ---- query operands (B layout: column n, K group q) ----
    // Every lane loads (lanes without a column read their group's first head; d_r is a
    // multiple of 8, so a lane's eight positional elements are all inside the row or all past
    // it, and the latter re-read the last eight) and masks with a bitwise and: a select on a
    // loaded value is compiled as a branch around the load with a wait inside, which would
    // serialise the query loads.
    bf16x8 QX[KS], QY[KS], RX, RY;
    const float *qp = a.q_abs + (static_cast<int64_t>(b) * a.H + head_lane) * row_len;
    const int col_mask = col_ok ? -1 : 0;
    float4 qraw[2 * KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 *src = reinterpret_cast<const float4 *>(qp + 32 * ks + 8 * q);
      qraw[2 * ks] = src[0];
      qraw[2 * ks + 1] = src[1];
    }
    const float4 *rsrc = reinterpret_cast<const float4 *>(qp + a.d_h + 8 * min(q, (a.d_r >> 3) - 1));
    const float4 r0 = rsrc[0], r1 = rsrc[1];
    const float rraw[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    const int r_mask = 8 * q < a.d_r ? col_mask : 0;
    // the first two tiles' block-table entries go out behind the query rows: the split below
    // waits for the query only (loads complete in order), so their round trips overlap
    const int32_t *__restrict__ bt = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
    const int lb = a.log2_bs;
    int32_t PA = load_pages(bt, lb, c0, c1, lane);
    int32_t PB = load_pages(bt, lb, c0 + kTile, c1, lane);
    auto masked = [](float v, int m) { return __int_as_float(__float_as_int(v) & m); };
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 x0 = qraw[2 * ks], x1 = qraw[2 * ks + 1];
      float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = masked(x[e], col_mask) * a.qscale;
      u32x4 hi, lo;
      split8(x, hi, lo);
      QX[ks] = as_bf16(use_lo ? lo : hi);
      QY[ks] = as_bf16(lo);
    }
    {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = masked(rraw[e], r_mask) * a.qscale;
      u32x4 hi, lo;
      split8(x, hi, lo);
      RX = as_bf16(use_lo ? lo : hi);
      RY = as_bf16(lo);
    }
    // this wave's LDS tile: lane (n, q) writes row n, columns 8 q ..; lane L reads row L / 4,
    // columns 4 (L % 4) .. (see read_tr)
    using L = TileLds<KS>;
    uint8_t *lw_wr = lds + wave * L::kWave + n * L::kRow + 16 * q;
    const uint8_t *lw_rd = lds + wave * L::kWave + (lane >> 2) * L::kRow + 8 * (lane & 3);

    // lane-invariant parts of the element offsets (positional K groups beyond d_r read the
    // row's last 8 elements; they meet zeros in the query operand)
    const int64_t vgrp = static_cast<int64_t>(g) * a.v_sg;
    uint8_t *lw_line = lds + wave * L::kWave + (lane / (4 * KS)) * L::kRow + 16 * line_chunk<KS>(lane);
    const int64_t klane = min(8 * q, a.d_r - 8);

    // Two tile buffers in ping-pong (A, Bt): while one tile is computed the other one's loads
    // are in flight, and no register copies are needed. Issue order per half-step: V loads of
    // the next tile, then the page entries two tiles ahead, then the math of the current tile.
    // (A third buffer, tried for grids of at most two work-groups per CU, gained nothing: the
    // loop runs near the streaming rate already.)
    // SHARE: wave 0 fetches each tile's positional key and stores it in the work-group's key
    // buffer (two tiles, 2 KB each: block tb, lane l at 1024 tb + 16 l); one barrier per tile
    // publishes it. The buffer of tile t + 1 is written after tile t's step and after every
    // wave has passed the barrier that ended tile t - 1, its last reader.
    const bool fetch_key = wave == 0;
    const int64_t kown = SHARE ? static_cast<int64_t>(blockIdx.x % a.num_blocks) * a.kr_sb : 0;
    uint8_t *kb0 = kbuf;
    uint8_t *kb1 = kbuf + 2048;
    auto publish = [&](uint8_t *kb, const Tile<KS, GQA> &T) {
      if constexpr (SHARE) {
        if (fetch_key) {
          *reinterpret_cast<u32x4 *>(kb + 16 * lane) = T.x[0][0];
          *reinterpret_cast<u32x4 *>(kb + 1024 + 16 * lane) = T.x[1][0];
        }
        __syncthreads();
      }
    };
    Tile<KS, GQA> A, Bt;
    load_tile<KS, GQA, SHARE>(a, PA, c0, c1, n, vgrp, klane, A, bad, fetch_key, kown);
    PA = load_pages(bt, lb, c0 + 2 * kTile, c1, lane);
    publish(kb0, A);
    for (int t0 = c0; t0 < c1; t0 += 2 * kTile) {
      const int t1 = t0 + kTile;
      load_tile<KS, GQA, SHARE>(a, PB, t1, c1, n, vgrp, klane, Bt, bad, fetch_key, kown);
      PB = load_pages(bt, lb, t1 + 2 * kTile, c1, lane);
      tile_step<KS, NH, GQA, SHARE>(A, t0, c1, n, q, QX, QY, RX, RY, lw_wr, lw_line, lw_rd, acc,
                                    kb0 + 16 * lane);
      publish(kb1, Bt);
      load_tile<KS, GQA, SHARE>(a, PA, t1 + kTile, c1, n, vgrp, klane, A, bad, fetch_key, kown);
      PA = load_pages(bt, lb, t1 + 3 * kTile, c1, lane);
      if (t1 < c1)                                     // uniform per work-group
        tile_step<KS, NH, GQA, SHARE>(Bt, t1, c1, n, q, QX, QY, RX, RY, lw_wr, lw_line, lw_rd, acc,
                                      kb1 + 16 * lane);
      publish(kb0, A);
    }
  }

  // ---- epilogue: the owner lanes of head c; dims 16 nb + 4 q + r ----
  if (NH > 0) {
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc.O[i][r] += row_shr_f<SH>(acc.O[i][r]);
  }
  float ltot = acc.lsum + __shfl_xor(acc.lsum, 16, 64);
  ltot += __shfl_xor(ltot, 32, 64);
  const bool any_bad = __any(bad);
  if (lane == 0 && any_bad) gvad::raise_err(a.err_flag, GVA_DEVERR_BLOCK);
  const bool poison = any_bad || len_bad;
  if (!owner) return;
  // empty chunks (past the end of a sequence, or of a sequence with a bad length) are never
  // read by the combine
  if (!direct && c0 >= c1) return;
  const int h = head_lane;                 // the owner lane's column is its head's
  if (direct) {
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    float *dst = a.out + (static_cast<int64_t>(b) * a.H + h) * a.d_h + 4 * q;
#pragma unroll
    for (int nb = 0; nb < 2 * KS; ++nb) {
      f32x4 v = acc.O[nb] * inv;
      if (poison) v = f32x4{qnan, qnan, qnan, qnan};
      *reinterpret_cast<f32x4 *>(dst + 16 * nb) = v;
    }
    if (a.lse && q == 0) {
      const float v = ltot > 0.0f ? (acc.m + log2f(ltot)) * gvad::kLn2 : -INFINITY;
      a.lse[static_cast<int64_t>(b) * a.H + h] = poison ? qnan : v;
    }
  } else {
    const int64_t prow = prow0 + h;
    float *dst = a.part_o + prow * a.d_h + 4 * q;
#pragma unroll
    for (int nb = 0; nb < 2 * KS; ++nb) *reinterpret_cast<f32x4 *>(dst + 16 * nb) = acc.O[nb];
    if (q == 0) {
      a.part_m[prow] = poison ? qnan : acc.m;
      a.part_l[prow] = ltot;
    }
  }
}


// Values the whole wave agrees on, moved to scalar registers (they come out of LDS or from
// per-lane arithmetic, so the compiler cannot know they are uniform).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ int tiles_of(const gva::DecodeArgs &a, int b, int cap) {
  const int len = a.seq_len[b];
  return (len >= 0 && len <= a.max_len && len <= cap) ? (len + kTile - 1) / kTile : 0;
}

// WAVES: the most waves (value groups) a work-group has; 8 only for the GVA balanced plan,
// whose work-groups then share the positional key through LDS (SHARE).
template <int KS, int NH, bool BALANCED, bool GQA, int WAVES>
__global__ __launch_bounds__(64 * WAVES, (min_waves_per_simd<KS, NH, GQA, WAVES>())) void
k_decode_mfma(gva::DecodeArgs a) {
  using L = TileLds<KS>;
  constexpr bool SHARE = WAVES == 8 && BALANCED && !GQA;
  __shared__ __align__(16) uint8_t lds[WAVES * L::kWave];
  __shared__ __align__(16) uint8_t kbuf[SHARE ? 4096 : 16];
  __shared__ int64_t s_part[WAVES];
  __shared__ int32_t s_found_b;
  __shared__ int32_t s_len[64 * WAVES];
  __shared__ int64_t s_found_p;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // Work-groups are dealt to the 8 XCDs in turn (XCD = id % 8). The nz work-groups that share
  // one work item (they cover the same positions for different value groups) take ids 8 apart,
  // so they run on the same XCD at about the same time (their reads of the shared positional key
  // still miss together about half the time).
  const int wpg = blockDim.x >> 6;
  const int nz = a.G / wpg;
  const int id = blockIdx.x;
  const int r8 = id >> 3;
  const int g = (r8 % nz) * wpg + wave;
  const int item = (r8 / nz) * 8 + (id & 7);
  const int cap = a.max_blocks << a.log2_bs;

  if constexpr (!BALANCED) {
    // Split grid: item = (split s, sequence b) with b fastest, so every XCD receives an even
    // share of each split column (early columns are almost always non-empty, late ones often
    // empty). Chunk s covers positions [s chunk, (s + 1) chunk).
    if (item >= a.B * a.num_splits) return;
    const int b = item % a.B;
    const int s = item / a.B;
    const int len = a.seq_len[b];
    const bool len_bad = len < 0 || len > a.max_len || len > cap;
    if (len_bad && s == 0 && g == 0 && lane == 0) gvad::raise_err(a.err_flag, GVA_DEVERR_LENGTH);
    const int c0 = s * a.chunk;
    const int c1 = len_bad ? c0 : min(c0 + a.chunk, len);
    run_chunk<KS, NH, GQA, SHARE>(a, b, g, c0, c1, len_bad, a.num_splits == 1,
                      (static_cast<int64_t>(b) * a.num_splits + s) * a.H, lds, kbuf);
  } else {

  // Balanced ranges: the 32-position tiles of all sequences, concatenated in sequence order
  // (T of them), are cut into Re = min(num_ranges, T) equal ranges; range r = item covers tiles
  // [r T / Re, (r + 1) T / Re), never empty. A range that spans several sequences does one chunk per sequence;
  // the chunk of range r in sequence b writes its partials at workspace rows (r + b) H + h, so
  // the chunks of one sequence occupy consecutive rows. Range 0 of the first group block also
  // writes the tile prefix P[b] (and P[B] = T) for the combine.
  const int R = a.num_ranges;
  if (item >= R) return;
  const bool writer = item == 0 && r8 % nz == 0;
  const int nthr = blockDim.x;
  // total tile count (with at most one sequence per thread, each length is read once and kept:
  // in a register for the scans, in LDS for the walk over the ranges)
  const bool one_pass = a.B <= nthr;
  int t_own = 0;
  int64_t mine = 0;
  if (one_pass) {
    if (tid < a.B) {
      const int len = a.seq_len[tid];
      s_len[tid] = len;
      t_own = (len >= 0 && len <= a.max_len && len <= cap) ? (len + kTile - 1) / kTile : 0;
    }
    mine = t_own;
  } else {
    for (int b = tid; b < a.B; b += nthr) mine += tiles_of(a, b, cap);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mine += __shfl_xor(mine, o, 64);
  if (lane == 0) s_part[wave] = mine;
  if (tid == 0) s_found_b = -1;
  __syncthreads();
  int64_t T = 0;
  for (int w = 0; w < wpg; ++w) T += s_part[w];
  T = uniform(T);
  // with fewer tiles than ranges, one tile per range (no range is empty)
  const int64_t Re = T < R ? T : R;
  const bool has_range = item < Re;
  const int64_t start = has_range ? static_cast<int64_t>(item) * T / Re : 0;
  const int64_t end = has_range ? static_cast<int64_t>(item + 1) * T / Re : 0;
  if (!writer && !has_range) return;                   // uniform per work-group
  // the sequence holding tile `start`: a running block-wide prefix over the sequences
  int64_t base = 0;
  for (int b0 = 0; b0 < a.B; b0 += nthr) {
    __syncthreads();                                   // s_part reuse
    const int b = b0 + tid;
    const int t = one_pass ? t_own : (b < a.B ? tiles_of(a, b, cap) : 0);
    int incl = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (lane == 63) s_part[wave] = incl;
    __syncthreads();
    int64_t before = base;
    int64_t chunk_total = 0;
    for (int w = 0; w < wpg; ++w) {
      if (w < wave) before += s_part[w];
      chunk_total += s_part[w];
    }
    const int64_t p_excl = before + incl - t;
    if (writer && b < a.B) a.tile_prefix[b] = static_cast<int32_t>(p_excl);
    if (has_range && t > 0 && p_excl <= start && start < p_excl + t) {
      s_found_b = b;
      s_found_p = p_excl;
    }
    base += chunk_total;
    __syncthreads();
    if (!writer && s_found_b >= 0) break;              // uniform per work-group
  }
  if (writer && tid == 0) a.tile_prefix[a.B] = static_cast<int32_t>(T);
  if (!has_range) return;
  auto len_of = [&](int b) { return uniform(one_pass ? s_len[b] : a.seq_len[b]); };
  auto tiles_b_of = [&](int b) {
    const int len = len_of(b);
    return (len >= 0 && len <= a.max_len && len <= cap) ? (len + kTile - 1) / kTile : 0;
  };
  int b = uniform(s_found_b);
  int64_t pb = uniform(s_found_p);                     // first tile of sequence b
  int64_t t = start;
  while (t < end) {
    const int tiles_b = tiles_b_of(b);
    const int64_t seg_end = min(end, pb + tiles_b);
    const int len = len_of(b);
    const int c0 = static_cast<int>(t - pb) * kTile;
    const int c1 = min(static_cast<int>(seg_end - pb) * kTile, len);
    run_chunk<KS, NH, GQA, SHARE>(a, b, g, c0, c1, false, false, static_cast<int64_t>(item + b) * a.H,
                                  lds, kbuf);
    t = seg_end;
    pb += tiles_b;
    ++b;
    while (t < end && tiles_b_of(b) == 0) ++b;        // sequences without tiles hold no range
  }
  }
}

template <int NH, bool BAL, bool GQA, int W>
hipError_t launch_mode(const gva::DecodeArgs &a, dim3 grid, dim3 block, hipStream_t stream) {
  switch (a.d_h / 32) {
    case 1: hipLaunchKernelGGL((k_decode_mfma<1, NH, BAL, GQA, W>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((k_decode_mfma<2, NH, BAL, GQA, W>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((k_decode_mfma<3, NH, BAL, GQA, W>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((k_decode_mfma<4, NH, BAL, GQA, W>), grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL((k_decode_mfma<5, NH, BAL, GQA, W>), grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL((k_decode_mfma<6, NH, BAL, GQA, W>), grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL((k_decode_mfma<7, NH, BAL, GQA, W>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((k_decode_mfma<8, NH, BAL, GQA, W>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int NH>
hipError_t launch_nh(const gva::DecodeArgs &a, dim3 grid, dim3 block, hipStream_t stream) {
  if (a.k) {
    return a.num_ranges > 0 ? launch_mode<NH, true, true, kGroupWaves>(a, grid, block, stream)
                            : launch_mode<NH, false, true, kGroupWaves>(a, grid, block, stream);
  }
  if (a.num_ranges == 0) return launch_mode<NH, false, false, kGroupWaves>(a, grid, block, stream);
  return block.x == 64u * gva::kSharedKeyWaves
             ? launch_mode<NH, true, false, gva::kSharedKeyWaves>(a, grid, block, stream)
             : launch_mode<NH, true, false, kGroupWaves>(a, grid, block, stream);
}

// ---- the decode step in one launch (small batches) -------------------------------------------
//
// K work-groups per (sequence b, value group g), W waves each. In one launch they do what the
// append, the absorption and the decode of a step do for the group:
//   1. absorption: q~ of the group's heads with float32 multiply-adds in the same order as
//      gva_absorb_query (so q_abs is bit-identical), the rows of M staged through LDS with
//      coalesced loads; the positional slice rotated in float64 at the token's position;
//   2. append: the token's values for group g (and, in group 0's work-group, its rotated
//      positional key) rounded once and written to the cache, as gva_cache_append writes them,
//      and kept in LDS: a wave whose tile holds position pos[b] takes the token from there
//      instead of the cache, which this launch is writing (every work-group of the sequence
//      rounds the positional key itself);
//   3. decode: the K W waves split the sequence's tiles into contiguous chunks and stream them
//      as the split decode does (scores, online softmax, weighted sum on the matrix cores);
//   4. merge: each wave leaves its (m, l, o) per head in LDS and the work-group merges them
//      through their log-sum-exp. With K = 1 that is the output. With K > 1 each work-group
//      writes its merged partial with device-scope stores (they write through to memory, so no
//      cache write-back is needed), waits for them to complete, and takes a ticket (a relaxed
//      device-scope atomic); the work-group that draws the last ticket reads the K partials with
//      device-scope loads, merges them into the output rows and puts the ticket back to zero.
// No work-group waits on another, and nothing is left for a second launch. (Ordering the merge
// with release/acquire fences instead writes back and invalidates whole L2 caches: measured
// 18 to 270 microseconds per launch here, against under 2 for the write-through pattern.)
// STEP == false is the decode alone with the same split and merge (gva_decode's plan for small
// batches): steps 1 and 2 are skipped, and each wave loads its query rows from q_abs, as the
// split decode does, with its first tiles.
template <int KS>
constexpr int step_waves() { return 8; }   // gva::step_waves_of(32 KS)
constexpr int kStepRegionBytes = 144 * 1024;   // staging of M, then tile copies, then the merge

// Loads the tile at t0 of a run ending at c1 as load_tile does, for block-table entries P read
// at positions clamped to the run's end at max_len instead of c1 (they were fetched before the
// sequence length was known). A 16-position block that starts at or past c1 was then looked up
// at a position that may lie in another block: it is not checked, and fix_tile zeroes its data
// before use, so only blocks holding positions of the run can raise the bad flag.
template <int KS>
__device__ __forceinline__ void load_tile_run(const gva::DecodeArgs &a, int32_t pb0, int32_t pb1,
                                              int t0, int c1, int n, int64_t vgrp, int klane,
                                              Tile<KS, false> &T, bool &bad) {
  static_assert(kLine<KS>, "the one-launch kernels load V in the line layout");
  const int mask = (1 << a.log2_bs) - 1;
  const int lane = threadIdx.x & 63;
  const int ch = 8 * line_chunk<KS>(lane);
  const uint16_t *vbase = static_cast<const uint16_t *>(a.v);
  const uint16_t *kbase = static_cast<const uint16_t *>(a.kr);
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int32_t pb = tb == 0 ? pb0 : pb1;
    const bool ok = pb >= 0 && static_cast<int64_t>(pb) < a.num_blocks;
    bad |= !ok && t0 + 16 * tb < c1;
    const int64_t blk = ok ? pb : 0;
    const int f = min(t0 + 16 * tb, c1 - 1);
    const int lim = c1 - 1 - f;
    const int64_t row = static_cast<int64_t>((f & mask) + min(n, lim));
    const uint16_t *vblk = vbase + blk * a.v_sb + static_cast<int64_t>(f & mask) * a.v_st + vgrp;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      T.v[tb][k] = stream_load(vblk + static_cast<int64_t>(min(line_row<KS>(lane, k), lim)) * a.v_st + ch);
    T.x[tb][0] = *reinterpret_cast<const u32x4 *>(kbase + blk * a.kr_sb + row * a.kr_st + klane);
  }
}

template <int KS, int NH, int W, bool STEP>
__global__ __launch_bounds__(64 * W, 1) void k_step_fused(gva::StepArgs s) {
  constexpr int DH = 32 * KS;
  using L = TileLds<KS>;
  static_assert(W * L::kWave <= kStepRegionBytes, "tile copies exceed the region");
  static_assert(W * NH * (DH + 2) * 4 <= kStepRegionBytes, "merge area exceeds the region");
  static_assert(32 * NH * (DH + 2) * 4 + 64 + 64 * 16 <= kStepRegionBytes,
                "K <= 32 partials (and the spare slots) exceed the region");
  __shared__ __align__(16) uint8_t region[kStepRegionBytes];
  __shared__ __align__(16) float q_lds[STEP ? NH : 1][DH + 32];  // q~ (DH), then r (d_r <= 32)
  __shared__ __align__(16) uint16_t tok_v[DH];                   // the new token's values, group g
  __shared__ __align__(16) uint16_t tok_kr[32];          // its rotated positional key (padded)
  __shared__ int s_bad;
  __shared__ int s_last;
  const gva::DecodeArgs &a = s.a;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int q = lane >> 4;
  // work-group -> (item, group) with item = (sequence b, part kk of K): items are dealt to the 8
  // XCDs in turn and the G work-groups of an item take ids 8 apart, so they run on one XCD at
  // about the same time and its L2 serves the positional keys they all read
  const int id = blockIdx.x;
  const int r8 = id >> 3;
  const int g = r8 % a.G;
  const int item = (r8 / a.G) * 8 + (id & 7);
  const int K = s.K;
  const int b = item / K;
  const int kk = item - b * K;
  if (b >= a.B) return;                                  // uniform per work-group
  if (tid == 0) s_bad = 0;
  // the group's heads: slot_head reads the group's slots with uniform (scalar) loads
  const int gh = __builtin_amdgcn_readfirstlane(g * NH);
  auto head = [&](int c) { return slot_head<NH>(a, gh, c); };
  const int d_r = a.d_r;
  const int d_n = s.d_n;
  const int row_len = DH + d_r;
  const float qnan = __int_as_float(0x7fc00000);
  const int p = STEP ? s.pos[b] : 0;
  const int len = a.seq_len[b];
  const int cap = a.max_blocks << a.log2_bs;

  // This wave's run: runs of tiles_per_wave tiles are cut from max_len, so the run's first
  // position, and the block-table entries of its first two tiles, are known before the
  // sequence's length arrives; the run ends at c1 = min(its end, len).
  const int c0 = (kk * W + wave) * s.tiles_per_wave * kTile;
  const int cend = min(c0 + s.tiles_per_wave * kTile, a.max_len);
  const int32_t *__restrict__ bt = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
  const int lb = a.log2_bs;
  // the first two tiles' entries, one per 16-position block, as scalar loads: they do not
  // queue behind the vector loads that stage M
  int32_t pa0 = 0, pa1 = 0, pb0 = 0, pb1 = 0;
  if (c0 < cend) {                                       // uniform per wave
    pa0 = bt[c0 >> lb];
    pa1 = bt[min(c0 + 16, cend - 1) >> lb];
    pb0 = bt[min(c0 + kTile, cend - 1) >> lb];
    pb1 = bt[min(c0 + kTile + 16, cend - 1) >> lb];
  }
  int32_t PA = 0, PB = 0;                                // later tiles' entries (vector loads)
  const bool len_bad = len < 0 || len > a.max_len || len > cap;
  const bool rope_bad = STEP && (p < 0 || p >= s.max_pos);  // the absorbed query is NaN
  // the append's inputs go out now too: the token's block-table entry, its values (one pair per
  // lane below d_h / 2) and its positional key pairs with their (cos, sin)
  int32_t aerr = 0;
  if constexpr (STEP) {
    if (p < 0) aerr = GVA_DEVERR_LENGTH;
    else if (p >= cap) aerr = GVA_DEVERR_CAPACITY;
    else if (p >= s.max_pos) aerr = GVA_DEVERR_ROPE;
  }
  const int32_t pblk = (!STEP || aerr) ? 0 : bt[p >> lb];
  const int half_r = d_r >> 1;
  float2 tok_x = {0.f, 0.f}, tok_k = {0.f, 0.f};
  double2 tok_cs = {1.0, 0.0};
  if (STEP && !aerr) {
    if (tid < DH / 2)
      tok_x = reinterpret_cast<const float2 *>(s.v_new + (static_cast<int64_t>(b) * a.G + g) * DH)[tid];
    if (tid < half_r) {
      tok_k = reinterpret_cast<const float2 *>(s.kr_raw + static_cast<int64_t>(b) * d_r)[tid];
      tok_cs = reinterpret_cast<const double2 *>(s.rope)[static_cast<int64_t>(p) * half_r + tid];
    }
  }
  // and so do the positional query pairs of the group's heads with their (cos, sin) at p
  // (lane t < NH d_r / 2 rotates pair t % (d_r / 2) of head t / (d_r / 2))
  float2 rq = {0.f, 0.f};
  double2 rq_cs = {1.0, 0.0};
  if (STEP && !rope_bad && tid < NH * half_r) {
    const int c = tid / half_r;
    const int k = tid - c * half_r;
    rq = reinterpret_cast<const float2 *>(s.q_rope + (static_cast<int64_t>(b) * a.H + head(c)) * d_r)[k];
    rq_cs = reinterpret_cast<const double2 *>(s.rope)[static_cast<int64_t>(p) * half_r + k];
  }
  const int c1 = len_bad ? c0 : min(cend, len);
  const int64_t vgrp = static_cast<int64_t>(g) * a.v_sg;
  const int klane = min(8 * q, d_r - 8);
  bool bad = false;
  Tile<KS, false> A, Bt;
  bool tile_a_issued = false;
  // the run's first tile, issued between the first staging loads and their LDS stores so that
  // waiting for the staged rows does not wait for it
  auto issue_tile_a = [&]() {
    if (c0 < c1) load_tile_run<KS>(a, pa0, pa1, c0, c1, n, vgrp, klane, A, bad);
    if (c0 + kTile < c1) {
      load_tile_run<KS>(a, pb0, pb1, c0 + kTile, c1, n, vgrp, klane, Bt, bad);
      if (c0 + 2 * kTile < c1) PA = load_pages(bt, lb, c0 + 2 * kTile, c1, lane);
    }
    tile_a_issued = true;
  };
  // decode only: the query rows (q~ | r) of this lane's column, as the split decode reads them
  // (lanes without a column read their group's first head and are masked with a bitwise and)
  const int cq = n < NH ? n : (n < 2 * NH ? n - NH : 0);
  const int col_mask = n < 2 * NH ? -1 : 0;
  float4 qraw[2 * KS], rraw[2];
  if constexpr (!STEP) {
    const float *qp = a.q_abs + (static_cast<int64_t>(b) * a.H + head(cq)) * row_len;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 *src = reinterpret_cast<const float4 *>(qp + 32 * ks + 8 * q);
      qraw[2 * ks] = src[0];
      qraw[2 * ks + 1] = src[1];
    }
    const float4 *rsrc = reinterpret_cast<const float4 *>(qp + DH + 8 * min(q, (d_r >> 3) - 1));
    rraw[0] = rsrc[0];
    rraw[1] = rsrc[1];
    issue_tile_a();
    __syncthreads();                                     // s_bad is cleared
  }

  // ---- 1. absorption (q~ in the order of gva_absorb_query, so q_abs is bit-identical) ----
  if constexpr (STEP) {
    float *mst = reinterpret_cast<float *>(region);
    const int d4 = d_n >> 2;
    const int stride4 = d4 + 1;                          // rows padded by 16 bytes
    const int qn_off = kStepRegionBytes / 4 - NH * d_n;  // q_nope of the group's heads
    const int rows_per_pass = qn_off / (4 * stride4);
    constexpr int kBatch = 8;                            // 16-byte loads in flight per lane
    for (int o0 = 0; o0 < NH * DH; o0 += rows_per_pass) {
      const int rows = min(rows_per_pass, NH * DH - o0);
      // pass 0 also stages q_nope: its float4 follow the rows' in the index space
      const int n_rows4 = rows * d4;
      const int n4 = n_rows4 + (o0 == 0 ? NH * d4 : 0);
      if (o0 > 0) __syncthreads();                       // the previous pass's rows are used
      for (int e0 = tid; e0 < n4; e0 += kBatch * 64 * W) {
        float4 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int e = e0 + u * 64 * W;
          v[u] = float4{0.f, 0.f, 0.f, 0.f};
          if (e < n_rows4) {
            const int rr = e / d4;
            const int o = o0 + rr;
            const int c = o / DH;
            v[u] = reinterpret_cast<const float4 *>(
                s.M + (static_cast<int64_t>(head(c)) * DH + (o - c * DH)) * d_n)[e - rr * d4];
          } else if (e < n4) {
            const int f = e - n_rows4;
            const int c = f / d4;
            v[u] = reinterpret_cast<const float4 *>(
                s.q_nope + (static_cast<int64_t>(b) * a.H + head(c)) * d_n)[f - c * d4];
          }
        }
        if (!tile_a_issued) issue_tile_a();              // uniform
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int e = e0 + u * 64 * W;
          if (e < n_rows4) {
            const int rr = e / d4;
            reinterpret_cast<float4 *>(mst)[rr * stride4 + (e - rr * d4)] = v[u];
          } else if (e < n4) {
            reinterpret_cast<float4 *>(mst + qn_off)[e - n_rows4] = v[u];
          }
        }
      }
      __syncthreads();
      for (int o = o0 + tid; o < o0 + rows; o += 64 * W) {
        const int c = o / DH;
        const int i = o - c * DH;
        const float4 *mr = reinterpret_cast<const float4 *>(mst) + (o - o0) * stride4;
        const float4 *qr = reinterpret_cast<const float4 *>(mst + qn_off) + c * d4;
        float acc = 0.0f;
#pragma unroll 8
        for (int j4 = 0; j4 < d4; ++j4) {
          const float4 m4 = mr[j4];
          const float4 q4 = qr[j4];
          acc = fmaf(m4.x, q4.x, acc);
          acc = fmaf(m4.y, q4.y, acc);
          acc = fmaf(m4.z, q4.z, acc);
          acc = fmaf(m4.w, q4.w, acc);
        }
        const float v = rope_bad ? qnan : acc;
        q_lds[c][i] = v;
        if (kk == 0) s.q_abs[(static_cast<int64_t>(b) * a.H + head(c)) * row_len + i] = v;
      }
    }
    if (!tile_a_issued) issue_tile_a();
    if (tid < NH * half_r) {                             // NH d_r / 2 <= 128 < 64 W
      const int c = tid / half_r;
      const int k = tid - c * half_r;
      const int h = head(c);
      float y0f = qnan, y1f = qnan;
      if (!rope_bad) {
        double y0, y1;
        gvad::rotate_pair_f64(static_cast<double>(rq.x), static_cast<double>(rq.y), rq_cs.x, rq_cs.y,
                              &y0, &y1);
        y0f = gvad::f64_to_f32(y0);
        y1f = gvad::f64_to_f32(y1);
      }
      q_lds[c][DH + 2 * k] = y0f;
      q_lds[c][DH + 2 * k + 1] = y1f;
      if (kk == 0) {
        float *dst = s.q_abs + (static_cast<int64_t>(b) * a.H + h) * row_len + DH + 2 * k;
        dst[0] = y0f;
        dst[1] = y1f;
      }
    }
  }

  // ---- 2. append (the checks and arithmetic of gva_cache_append) ----
  int64_t blk = -1;
  bool tok_ok = false;                                   // decode only: no token
  if constexpr (STEP) {
    if (!aerr) {
      if (pblk < 0 || static_cast<int64_t>(pblk) >= a.num_blocks) aerr = GVA_DEVERR_BLOCK;
      else blk = pblk;
    }
    tok_ok = aerr == 0;
  }
  if (g == 0 && kk == 0 && tid == 0) {
    if (aerr) gvad::raise_err(a.err_flag, aerr);
    if (rope_bad) gvad::raise_err(a.err_flag, GVA_DEVERR_ROPE);
    if (len_bad) gvad::raise_err(a.err_flag, GVA_DEVERR_LENGTH);
  }
  if (tok_ok) {
    const int64_t off = p & ((1 << a.log2_bs) - 1);
    uint32_t *v32 = reinterpret_cast<uint32_t *>(const_cast<void *>(a.v));
    if (tid < DH / 2) {                                  // 64 W > DH / 2
      const uint32_t w = gvad::f64_to_bf16_bits(static_cast<double>(tok_x.x)) |
                         (static_cast<uint32_t>(gvad::f64_to_bf16_bits(static_cast<double>(tok_x.y))) << 16);
      if (kk == 0) v32[(blk * a.v_sb + off * a.v_st + static_cast<int64_t>(g) * a.v_sg + 2 * tid) >> 1] = w;
      reinterpret_cast<uint32_t *>(tok_v)[tid] = w;
    }
    uint32_t *k32 = reinterpret_cast<uint32_t *>(const_cast<void *>(a.kr));
    if (tid < 16) {
      uint32_t w = 0;
      if (tid < half_r) {
        double y0, y1;
        gvad::rotate_pair_f64(static_cast<double>(tok_k.x), static_cast<double>(tok_k.y), tok_cs.x,
                              tok_cs.y, &y0, &y1);
        w = gvad::f64_to_bf16_bits(y0) | (static_cast<uint32_t>(gvad::f64_to_bf16_bits(y1)) << 16);
        if (g == 0 && kk == 0) k32[(blk * a.kr_sb + off * a.kr_st + 2 * tid) >> 1] = w;
      }
      reinterpret_cast<uint32_t *>(tok_kr)[tid] = w;
    }
  }
  if constexpr (STEP) __syncthreads();                   // q~, r and the token are in LDS

  // ---- 3. decode the wave's run of tiles ----
  constexpr int SH = NH;
  const int c = n < NH ? n : n - NH;                     // the query column's head
  const bool col_ok = n < 2 * NH;
  const bool use_lo = n >= NH;
  const bool owner = n >= NH && n < 2 * NH;
  Acc<KS> acc;
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i) acc.O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  acc.m = -INFINITY;
  acc.lsum = 0.0f;
  if (c0 < c1) {                                         // uniform per wave
    bf16x8 QX[KS], QY[KS], RX, RY;
    if constexpr (STEP) {
      const float *qp = q_lds[col_ok ? c : 0];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float x[8];
        const float4 x0 = *reinterpret_cast<const float4 *>(qp + 32 * ks + 8 * q);
        const float4 x1 = *reinterpret_cast<const float4 *>(qp + 32 * ks + 8 * q + 4);
        x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
        x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = col_ok ? x[e] * a.qscale : 0.0f;
        u32x4 hi, lo;
        split8(x, hi, lo);
        QX[ks] = as_bf16(use_lo ? lo : hi);
        QY[ks] = as_bf16(lo);
      }
      {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * q + e;
          x[e] = (col_ok && i < d_r) ? qp[DH + i] * a.qscale : 0.0f;
        }
        u32x4 hi, lo;
        split8(x, hi, lo);
        RX = as_bf16(use_lo ? lo : hi);
        RY = as_bf16(lo);
      }
    } else {
      // the rows loaded at the start, masked (a bitwise and) and scaled as the split decode does
      auto masked = [](float v, int m) { return __int_as_float(__float_as_int(v) & m); };
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const float4 x0 = qraw[2 * ks], x1 = qraw[2 * ks + 1];
        float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = masked(x[e], col_mask) * a.qscale;
        u32x4 hi, lo;
        split8(x, hi, lo);
        QX[ks] = as_bf16(use_lo ? lo : hi);
        QY[ks] = as_bf16(lo);
      }
      {
        const int r_mask = 8 * q < d_r ? col_mask : 0;
        const float4 r0 = rraw[0], r1 = rraw[1];
        float x[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = masked(x[e], r_mask) * a.qscale;
        u32x4 hi, lo;
        split8(x, hi, lo);
        RX = as_bf16(use_lo ? lo : hi);
        RY = as_bf16(lo);
      }
    }
    uint8_t *lw_wr = region + wave * L::kWave + n * L::kRow + 16 * q;
    uint8_t *lw_line =
        region + wave * L::kWave + (lane / (4 * KS)) * L::kRow + 16 * line_chunk<KS>(lane);
    const uint8_t *lw_rd = region + wave * L::kWave + (lane >> 2) * L::kRow + 8 * (lane & 3);
    const u32x4 tvl = *reinterpret_cast<const u32x4 *>(tok_v + 8 * line_chunk<KS>(lane));
    const u32x4 tk = *reinterpret_cast<const u32x4 *>(tok_kr + klane);
    // Before a tile is used: the lanes that read position p take the new token from LDS (this
    // launch is writing it to the cache), and a block lying wholly past c1 is zeroed (it may
    // have been read from another block; its scores are masked, and its values must be finite).
    auto fix_tile = [&](Tile<KS, false> &T, int t0) {
      if (t0 + kTile > c1) {                             // the run's last tile; uniform
        const bool past = t0 + 16 >= c1;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) T.v[1][ks] = past ? u32x4{0u, 0u, 0u, 0u} : T.v[1][ks];
        T.x[1][0] = past ? u32x4{0u, 0u, 0u, 0u} : T.x[1][0];
      }
      if (!tok_ok || p < t0 || p >= t0 + kTile) return;  // uniform
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int f = min(t0 + 16 * tb, c1 - 1);
        const bool in_run = t0 + 16 * tb < c1;
        // V in the line layout: load k of this lane read row line_row(k) (clamped), at this
        // lane's chunk; the positional key in the operand layout: row n (clamped)
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          const bool at_p = in_run && f + min(line_row<KS>(lane, k), c1 - 1 - f) == p;
          T.v[tb][k] = at_p ? tvl : T.v[tb][k];
        }
        const bool at_p = in_run && f + min(n, c1 - 1 - f) == p;
        T.x[tb][0] = at_p ? tk : T.x[tb][0];
      }
    };
    // two tile buffers in ping-pong, the first two tiles already in flight; nothing is loaded
    // past c1 (the page entries of a tile go out with the data of the tile before it)
    int t0 = c0;
    bool first = true;
    while (true) {
      const int t1 = t0 + kTile;
      if (!first && t1 < c1) {                           // uniform
        load_tile_run<KS>(a, __builtin_amdgcn_readlane(PB, 0), __builtin_amdgcn_readlane(PB, 1), t1,
                          c1, n, vgrp, klane, Bt, bad);
        if (t1 + kTile < c1) PA = load_pages(bt, lb, t1 + kTile, c1, lane);
      }
      first = false;
      fix_tile(A, t0);
      tile_step<KS, NH, false, false>(A, t0, c1, n, q, QX, QY, RX, RY, lw_wr, lw_line, lw_rd, acc,
                                      nullptr);
      if (t1 >= c1) break;
      const int t2 = t1 + kTile;
      if (t2 < c1) {
        load_tile_run<KS>(a, __builtin_amdgcn_readlane(PA, 0), __builtin_amdgcn_readlane(PA, 1), t2,
                          c1, n, vgrp, klane, A, bad);
        if (t2 + kTile < c1) PB = load_pages(bt, lb, t2 + kTile, c1, lane);
      }
      fix_tile(Bt, t1);
      tile_step<KS, NH, false, false>(Bt, t1, c1, n, q, QX, QY, RX, RY, lw_wr, lw_line, lw_rd, acc,
                                      nullptr);
      if (t2 >= c1) break;
      t0 = t2;
    }
  }

  // ---- 4. merge the waves' partials in LDS ----
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc.O[i][r] += row_shr_f<SH>(acc.O[i][r]);
  float ltot = acc.lsum + __shfl_xor(acc.lsum, 16, 64);
  ltot += __shfl_xor(ltot, 32, 64);
  if (__any(bad) && lane == 0) {
    s_bad = 1;
    gvad::raise_err(a.err_flag, GVA_DEVERR_BLOCK);
  }
  __syncthreads();                                       // every wave is done with its tile copy
  float *pm = reinterpret_cast<float *>(region);         // [W][NH]
  float *pl = pm + W * NH;                               // [W][NH]
  float *po = pl + W * NH;                               // [W][NH][DH]
  if (owner) {
#pragma unroll
    for (int nb = 0; nb < 2 * KS; ++nb)
      *reinterpret_cast<f32x4 *>(po + (wave * NH + c) * DH + 16 * nb + 4 * q) = acc.O[nb];
    if (q == 0) {
      pm[wave * NH + c] = acc.m;
      pl[wave * NH + c] = ltot;
    }
  }
  __syncthreads();
  // a NaN query (a position outside the RoPE table) or a NaN partial makes the row NaN, as in
  // the separate calls
  const bool poison = len_bad || rope_bad || s_bad != 0;
  for (int o = tid; o < NH * DH; o += 64 * W) {
    const int ch = o / DH;
    const int d = o - ch * DH;
    float ms = -INFINITY;
    bool nan_in = false;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      ms = fmaxf(ms, pm[w * NH + ch]);
      nan_in = nan_in || pl[w * NH + ch] != pl[w * NH + ch];
    }
    float lt = 0.0f, ov = 0.0f;
    if (ms != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float f = __builtin_amdgcn_exp2f(pm[w * NH + ch] - ms);
        lt += pl[w * NH + ch] * f;
        ov += po[(w * NH + ch) * DH + d] * f;
      }
    }
    const bool nan_row = poison || nan_in;
    if (K == 1) {
      const int64_t orow = static_cast<int64_t>(b) * a.H + head(ch);
      a.out[orow * DH + d] = nan_row ? qnan : (lt > 0.0f ? ov / lt : 0.0f);
      if (d == 0 && a.lse)
        a.lse[orow] = nan_row ? qnan : (lt > 0.0f ? (ms + log2f(lt)) * gvad::kLn2 : -INFINITY);
    } else {
      // this work-group's partial: unnormalised o, m (NaN when poisoned) and l
      const int64_t prow = (static_cast<int64_t>(b * a.G + g) * K + kk) * NH + ch;
      __hip_atomic_store(s.part_o + prow * DH + d, ov, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0) {
        __hip_atomic_store(s.part_m + prow, nan_row ? qnan : ms, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(s.part_l + prow, lt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (K == 1) return;
  // every lane's partial stores have completed at device scope before the ticket is taken
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int32_t *ticket = s.ticket + b * a.G + g;
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == K - 1;
  __syncthreads();
  if (!s_last) return;                                   // uniform per work-group
  // the last work-group merges the K partials of (b, g): one round of device-scope loads stages
  // them in LDS (rows prow0 .. prow0 + K NH - 1 are contiguous), then the merge reads LDS
  const int64_t prow0 = static_cast<int64_t>(b * a.G + g) * K * NH;
  const int kn4 = (K * NH + 3) & ~3;                     // keeps go 16-byte aligned
  float *gm = reinterpret_cast<float *>(region);         // [K][NH]
  float *gl = gm + kn4;                                  // [K][NH]
  float *go = gl + kn4;                                  // [K][NH][DH], then 64 spare slots
  {
    // buffer loads with the device-scope cache policy (sc1): they read past this XCD's L2 like
    // the atomic loads would, but several can be in flight; the ranges end at this pair's rows
    constexpr int kSc1 = 16;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        s.part_o + prow0 * DH, 0, static_cast<int>(K * NH * DH * 4), 0x00020000);
    const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
        s.part_m + prow0, 0, static_cast<int>(K * NH * 4), 0x00020000);
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
        s.part_l + prow0, 0, static_cast<int>(K * NH * 4), 0x00020000);
    // K NH <= 256 < 64 W: one m and one l per thread, issued before the o rows
    const bool has_ml = tid < K * NH;
    uint32_t mv = 0, lv = 0;
    if (has_ml) {
      mv = __builtin_amdgcn_raw_buffer_load_b32(rm, 4 * tid, 0, kSc1);
      lv = __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * tid, 0, kSc1);
    }
    // the o rows in batches of 8 loads per lane (K NH DH / 4 <= 32 * 8 * 16 = 8 * 512: one
    // batch), all in flight before the first LDS store (loads past the range return zero; their
    // stores go to a spare slot per lane after the rows, so every store is made, no load is held
    // back behind a branch, and no two lanes of a store share an address)
    const int n4 = K * NH * DH / 4;
    constexpr int kBatchM = 8;
    for (int e0 = tid; e0 < n4; e0 += kBatchM * 64 * W) {
      u32x4 v[kBatchM];
#pragma unroll
      for (int u = 0; u < kBatchM; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(ro, 16 * (e0 + u * 64 * W), 0, kSc1);
#pragma unroll
      for (int u = 0; u < kBatchM; ++u) {
        const int e = e0 + u * 64 * W;
        reinterpret_cast<u32x4 *>(go)[e < n4 ? e : n4 + lane] = v[u];
      }
    }
    if (has_ml) {
      gm[tid] = __uint_as_float(mv);
      gl[tid] = __uint_as_float(lv);
    }
  }
  __syncthreads();
  // a thread per four dims of a head: the K partials' m and l are LDS broadcasts to the head's
  // threads, and the loops are unrolled so that their LDS reads are in flight together (k in
  // ascending order, so the sums are those of the one-dim-per-thread form)
  constexpr int D4 = DH / 4;
  for (int o4 = tid; o4 < NH * D4; o4 += 64 * W) {
    const int ch = o4 / D4;
    const int d4 = o4 - ch * D4;
    float ms = -INFINITY;
    bool nan_in = false;
#pragma unroll 8
    for (int k = 0; k < K; ++k) {
      const float mk = gm[k * NH + ch];
      nan_in = nan_in || mk != mk;
      ms = fmaxf(ms, mk);
    }
    float lt = 0.0f;
    f32x4 ov = {0.f, 0.f, 0.f, 0.f};
    if (ms != -INFINITY && !nan_in) {
#pragma unroll 8
      for (int k = 0; k < K; ++k) {
        const float f = __builtin_amdgcn_exp2f(gm[k * NH + ch] - ms);
        lt += gl[k * NH + ch] * f;
        const f32x4 ok = *reinterpret_cast<const f32x4 *>(go + (k * NH + ch) * DH + 4 * d4);
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[r] += ok[r] * f;
      }
    }
    const int64_t orow = static_cast<int64_t>(b) * a.H + head(ch);
    f32x4 res;
#pragma unroll
    for (int r = 0; r < 4; ++r) res[r] = nan_in ? qnan : (lt > 0.0f ? ov[r] / lt : 0.0f);
    *reinterpret_cast<f32x4 *>(a.out + orow * DH + 4 * d4) = res;
    if (d4 == 0 && a.lse)
      a.lse[orow] = nan_in ? qnan : (lt > 0.0f ? (ms + log2f(lt)) * gvad::kLn2 : -INFINITY);
  }
  if (tid == 0) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int KS, int NH, bool STEP>
hipError_t launch_step_ks(const gva::StepArgs &s, hipStream_t stream) {
  constexpr int W = step_waves<KS>();
  const int64_t items = static_cast<int64_t>(s.a.B) * s.K;
  const dim3 grid(static_cast<unsigned>((items + 7) / 8 * 8 * s.a.G));
  hipLaunchKernelGGL((k_step_fused<KS, NH, W, STEP>), grid, dim3(64 * W), 0, stream, s);
  return hipGetLastError();
}

template <int NH>
hipError_t launch_step_nh(const gva::StepArgs &s, hipStream_t stream) {
  switch (s.a.d_h / 32) {
    case 1: return launch_step_ks<1, NH, true>(s, stream);
    case 2: return launch_step_ks<2, NH, true>(s, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int NH>
hipError_t launch_merged_nh(const gva::StepArgs &s, hipStream_t stream) {
  switch (s.a.d_h) {
    case 32: return launch_step_ks<1, NH, false>(s, stream);
    case 64: return launch_step_ks<2, NH, false>(s, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

namespace gva {

hipError_t launch_step_fused(const StepArgs &s, hipStream_t stream) {
  switch (s.a.H / s.a.G) {
    case 1: return launch_step_nh<1>(s, stream);
    case 2: return launch_step_nh<2>(s, stream);
    case 4: return launch_step_nh<4>(s, stream);
    case 8: return launch_step_nh<8>(s, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_merged(const StepArgs &s, hipStream_t stream) {
  switch (s.a.H / s.a.G) {
    case 1: return launch_merged_nh<1>(s, stream);
    case 2: return launch_merged_nh<2>(s, stream);
    case 4: return launch_merged_nh<4>(s, stream);
    case 8: return launch_merged_nh<8>(s, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t stream) {
  // the GVA balanced plan's layout (as plan_decode chose it), else four-wave work-groups
  const int64_t tiles_max = static_cast<int64_t>(a.B) * ((a.max_len + kTile - 1) / kTile);
  const int wpg = a.num_ranges > 0 && !a.k ? balanced_layout(a.G, true, tiles_max).waves
                                           : decode_waves_per_group(a.G);
  const int64_t items = a.num_ranges > 0 ? a.num_ranges : static_cast<int64_t>(a.B) * a.num_splits;
  const dim3 grid(static_cast<unsigned>(((items + 7) / 8) * 8 * (a.G / wpg)));
  const dim3 block(64 * wpg);
  switch (a.H / a.G) {
    case 1: return launch_nh<1>(a, grid, block, stream);
    case 2: return launch_nh<2>(a, grid, block, stream);
    case 4: return launch_nh<4>(a, grid, block, stream);
    case 8: return launch_nh<8>(a, grid, block, stream);
    default: return launch_nh<0>(a, grid, block, stream);
  }
}

}  // namespace gva
