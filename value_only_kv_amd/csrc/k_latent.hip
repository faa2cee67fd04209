// k_latent.hip - decode of the MLA-style latent comparator on matrix cores (gfx950).
//
// MLA caches one joint latent of width d_c per token plus a shared, already rotated positional
// key of width d_r, and projects keys and values back up from the latent at decode
// ("GVA：KV 缓存里的 Key 其实可以不存", shibing624.github.io review of arXiv:2609.13285, section
// 问题: T (d_c + d_r) scalars). With the key up-projection folded into the query, the step is
// the absorbed decode of a single group whose cached value is the latent:
//   s_j = scale (q~_h . c_j + r_h . kr_j),   out_h = sum_j softmax_j(s) c_j   (width d_c),
// the value up-projection acting on out_h afterwards, outside this call. Unlike the GVA value
// groups, every head reads the same latent, and d_c is wide (512 in the DeepSeek-V2 example of
// the [mla] page), so the latent tile is staged once in LDS and shared by all the waves.
//
// Work-group: one (sequence, chunk) of the split plan, H / 8 waves of 8 heads each. Per tile of
// 32 positions:
//   * the natural rows [c (d_c) | kr (d_r, padded to a multiple of 32)] go straight from HBM
//     into LDS (global_load_lds_dwordx4, a ring of three or four buffers, two or three tiles
//     ahead): a unit of 16 keys x
//     32 elements is one wave instruction that writes 1 KB, lane i's 16 bytes at 16 i, which is
//     exactly the score product's A-operand form;
//   * scores S^T[key][col] on v_mfma_f32_16x16x32_bf16, B = the absorbed query in its 16
//     columns: column n < 8 the bf16 hi part of head 8 w + n, column n + 8 its lo part; a row
//     rotation by 8 lanes (DPP) adds the two;
//   * online softmax per head in the base-2 domain, with a lazily raised reference maximum;
//   * weighted sum O^T[dim][col] += C^T P^T with the probabilities as a bf16 hi (columns < 8) and
//     lo (columns >= 8) pair and C^T read from the units with the transposing LDS load, whose
//     per-lane addresses follow each key's two 8-element pieces.
// Partials (m, l, o) go to the split-grid rows the decode combine reads; one chunk per sequence
// writes the output directly.
#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

#include "gva_device.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int kTile = 32;
constexpr float kLazyRescale = 8.0f;   // the reference moves when a score passes it by more

__device__ __forceinline__ f32x4 mfma(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ unsigned pack2(float x, float y) {
  const f32x2 v = {x, y};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));  // RNE, x low
}
__device__ __forceinline__ float low_bf16(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float high_bf16(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
// value of the lane 8 places along in its row of 16 (DPP row rotation)
__device__ __forceinline__ float ror8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
}
__device__ __forceinline__ float max4(const f32x4 &v) { return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])); }
// s_waitcnt limiting only the vector-memory counter to N (its low 4 bits at [3:0], high 2 at
// [15:14]; expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt limiting only the LDS / scalar-memory counter to zero
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}
// work-group barrier after this wave's own LDS reads; unlike a fenced barrier it does not wait
// for the transfers into LDS still in flight (later tiles'), whose completion the caller orders
// with wait_vmcnt. The clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS tile: unit (kb, ks) = keys 16 kb .. + 16, elements 32 ks .. + 32 of the natural rows,
// 1 KB: key n, elements 8 q .. + 8 in slot (n ^ 8 (q & 1)) + 16 q of 16 bytes. Within each
// group of 16 slots the keys are permuted, so the score product's operand reads stay
// conflict-free, and the transposing reads, whose 32 lanes per cycle take two pieces of 8 keys,
// cover all 64 banks instead of meeting two by two.
template <int KS, int RS>
struct LatentTile {
  static constexpr int kSteps = KS + RS;             // k-steps of a natural row
  static constexpr int kUnits = 2 * kSteps;
  static constexpr int kBytes = kUnits * 1024;
};
// LDS buffers of the staging ring (tiles in flight + the one being read): up to four, as many as
// 160 KB of LDS holds and as the 6-bit vector-memory counter can wait on ((bufs - 2) tiles of
// transfers outstanding while the next is awaited), at least three
template <int KS, int RS, int NW>
constexpr int latent_bufs() {
  constexpr int units = LatentTile<KS, RS>::kUnits, bytes = LatentTile<KS, RS>::kBytes;
  constexpr int per = (units + NW - 1) / NW;
  int n = 4;
  while (n > 3 && (n * bytes > 160 * 1024 - 1024 || (n - 2) * per > 63)) --n;
  return n;
}
__device__ __forceinline__ int unit_off(int kb, int ks, int steps) { return (kb * steps + ks) * 1024; }

template <int KS, int RS, int NW>
__global__ __launch_bounds__(64 * NW) void k_latent_decode(gva::DecodeArgs a) {
  using L = LatentTile<KS, RS>;
  constexpr int kSteps = L::kSteps;
  constexpr int kPer = (L::kUnits + NW - 1) / NW;    // units each wave stages per tile
  constexpr int kBufs = latent_bufs<KS, RS, NW>();
  constexpr int kDepth = kBufs - 1;                  // tiles staged ahead of the one read
  static_assert(kBufs >= 3 && kBufs <= 4 && kBufs * L::kBytes <= 160 * 1024 - 1024 &&
                (kDepth - 1) * kPer < 64, "ring");
  // one array per buffer: distinct objects, so that the compiler can tell a tile's LDS reads
  // from the transfers into the other buffers
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[L::kBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[L::kBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[L::kBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[kBufs > 3 ? L::kBytes : 1024];
  auto ring = [&](auto I) __attribute__((always_inline)) -> uint8_t * {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return lds0;
    else if constexpr (i == 1) return lds1;
    else if constexpr (i == 2) return lds2;
    else return lds3;
  };
  const int S = a.num_splits;
  const int d_c = a.d_h;
  const int cap = a.max_blocks << a.log2_bs;
  const float qnan = __int_as_float(0x7fc00000);
  // Work queue: the resident work-groups take (sequence, chunk) items from a counter, chunk by
  // chunk (every sequence's first chunk, then every second one, ...), so the work spreads over
  // all CUs whatever the lengths, and the short last chunks come last. No work-group waits for
  // another: each leaves when the queue is empty.
  const int items = a.B * S;
  __shared__ int s_item;
  for (;;) {
  if (threadIdx.x == 0) s_item = atomicAdd(a.work_next, 1);
  __syncthreads();
  const int item = s_item;
  __syncthreads();
  if (item >= items) break;                            // uniform per work-group
  // (the lane's indices are derived anew for every item from a value the compiler cannot see
  // through, so that nothing lane-dependent is kept live across the items)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int q = lane >> 4;
  const int hcol = 8 * wave + (n & 7);                // the head of this lane's column
  const bool lo_col = n >= 8;
  const int b = item % a.B;
  const int s = item / a.B;
  const int len = a.seq_len[b];
  const int64_t orow = static_cast<int64_t>(b) * a.H + hcol;
  const int64_t prow = (static_cast<int64_t>(b) * S + s) * a.H + hcol;
  const int c0 = s * a.chunk;
  int err = 0;
  if (len < 0 || len > a.max_len) err = GVA_DEVERR_LENGTH;
  else if (len > cap) err = GVA_DEVERR_CAPACITY;
  if (err) {                                           // uniform per work-group
    if (threadIdx.x == 0 && s == 0) gvad::raise_err(a.err_flag, err);
    if (S == 1 && !lo_col) {
      for (int d = 4 * q; d < d_c; d += 16) *reinterpret_cast<f32x4 *>(a.out + orow * d_c + d) = f32x4{qnan, qnan, qnan, qnan};
      if (a.lse && q == 0) a.lse[orow] = qnan;
    }
    continue;                                          // S > 1: the combine checks the length
  }
  if (c0 >= len) {                                     // uniform per work-group
    if (S == 1 && !lo_col) {                           // len == 0
      for (int d = 4 * q; d < d_c; d += 16) *reinterpret_cast<f32x4 *>(a.out + orow * d_c + d) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (a.lse && q == 0) a.lse[orow] = -INFINITY;
    }
    continue;                                          // past the end: the combine skips it
  }
  const int c1 = min(len, c0 + a.chunk);

  // absorbed query, B-operand form: column n holds head hcol, elements 32 ks + 8 q .. + 8, as
  // the bf16 hi part (n < 8) or lo part (n >= 8); positional padding is zero
  // (all of the row's loads are issued before any conversion; the lo part subtracts the hi
  // part's value, zero on the hi columns, so that no lane takes a branch)
  u32x4 Q[kSteps];
  {
    const float *qp = a.q_abs + orow * (d_c + a.d_r);
    float x[kSteps][8];
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (ks < KS) {
          x[ks][i] = qp[32 * ks + 8 * q + i];
        } else {
          const int e = 32 * (ks - KS) + 8 * q + i;
          const float v = qp[d_c + min(e, a.d_r - 1)];
          x[ks][i] = e < a.d_r ? v : 0.0f;
        }
      }
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = x[ks][2 * i] * a.qscale;
        const float x1 = x[ks][2 * i + 1] * a.qscale;
        const unsigned w = pack2(x0, x1);
        const float r0 = lo_col ? low_bf16(w) : 0.0f;
        const float r1 = lo_col ? high_bf16(w) : 0.0f;
        Q[ks][i] = pack2(x0 - r0, x1 - r1);
      }
  }

  // staging: wave w loads units w, w + NW, ... of a tile (keys past the chunk repeat its last
  // key; waves past the last unit load it again: the same bytes to the same place). Blocks hold
  // at least 16 positions and tiles start at multiples of 16, so each of a tile's two 16-key
  // blocks lies in one page (a clamped key stays in its block's page): the entries are uniform,
  // loaded two tiles ahead of their staging into one of kBufs register sets.
  // (read through the constant address space: the table does not change during the call, and
  // its uniform loads become scalar ones, which leave the vector-memory counter to the staging)
  typedef __attribute__((address_space(4))) const int32_t cint32;
  cint32 *bt = (cint32 *)(a.block_table + static_cast<int64_t>(b) * a.max_blocks);
  const int pos_mask = (1 << a.log2_bs) - 1;
  bool bad = false;
  int32_t pgs[kBufs][2];
  auto pages = [&](int32_t (&pg)[2], int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) pg[kb] = bt[min(j0 + 16 * kb, c1 - 1) >> a.log2_bs];
  };
  // (a single wave stages the whole tile: its address arithmetic is unrolled in part only)
  constexpr int kStageUnroll = kPer <= 12 ? kPer : 6;
  // stage_part issues transfers i0 .. i1 - 1 of this wave's kPer for a tile
  auto stage_part = [&](auto I0, auto I1, uint8_t *buf, int32_t pg0, int32_t pg1,
                        int j0) __attribute__((always_inline)) {
#pragma unroll kStageUnroll
    for (int i = decltype(I0)::value; i < decltype(I1)::value; ++i) {
      const int unit = min(wave + NW * i, L::kUnits - 1);
      const int kb = unit / kSteps;
      const int ks = unit - kb * kSteps;
      // (this lane's 16 bytes land in slot lane: key n ^ 8 (q & 1) of piece q)
      const int j = min(j0 + 16 * kb + (n ^ (8 * (q & 1))), c1 - 1);
      const int32_t blk = kb ? pg1 : pg0;
      const bool ok = blk >= 0 && static_cast<int64_t>(blk) < a.num_blocks;
      bad = bad || !ok;
      const int64_t bb = ok ? static_cast<int64_t>(blk) : 0;
      const int64_t row = j & pos_mask;
      const uint16_t *src;
      if (ks < KS) {
        src = static_cast<const uint16_t *>(a.v) + bb * a.v_sb + row * a.v_st + 32 * ks + 8 * q;
      } else {
        // positional elements past d_r read the row's last 8 (finite values, met by zeros in Q)
        const int e = min(32 * (ks - KS) + 8 * q, a.d_r - 8);
        src = static_cast<const uint16_t *>(a.kr) + bb * a.kr_sb + row * a.kr_st + e;
      }
      __builtin_amdgcn_global_load_lds((glb_void *)src, (lds_void *)(buf + unit_off(kb, ks, kSteps)),
                                       16, 0, 2);   // non-temporal (nt)
    }
  };
  auto stage = [&](uint8_t *buf, int32_t pg0, int32_t pg1, int j0) __attribute__((always_inline)) {
    stage_part(std::integral_constant<int, 0>{}, std::integral_constant<int, kPer>{}, buf, pg0,
               pg1, j0);
  };

  // transposing-read address of this lane within a unit: key lane / 4, and of its 16-dim
  // block's two 8-element pieces the one of column chunk lane % 4
  const int tr_key = lane >> 2;
  const int tr_k = lane & 3;
  const int sw_lane = 16 * (lane ^ (8 * ((lane >> 4) & 1)));   // slot of (key n, piece q)
  f32x4 O[2 * KS];
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref = -INFINITY, lsum = 0.0f;

  // tile(base, j0, hook): hook(1) runs after the scores, hook(2) after the first half of the
  // weighted sum (compile-time points of the unrolled code, so no branch is added)
  auto tile = [&](const uint8_t *base, int j0, auto &&hook) __attribute__((always_inline)) {
    const float negm = (mref == -INFINITY || lo_col) ? 0.0f : -mref;
    f32x4 Sc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      Sc[tb] = f32x4{negm, negm, negm, negm};
      // all of a key block's A operands are read before its products, so one wait covers them
      u32x4 ka[kSteps];
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks)
        ka[ks] = *reinterpret_cast<const u32x4 *>(base + unit_off(tb, ks, kSteps) + sw_lane);
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) Sc[tb] = mfma(ka[ks], Q[ks], Sc[tb]);
      // hi + lo columns: every lane of the row pair (n, n + 8) holds head hcol's score
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Sc[tb][e] += ror8(Sc[tb][e]);
        if (j0 + 16 * tb + 4 * q + e >= c1) Sc[tb][e] = -INFINITY;
      }
    }
    hook(std::integral_constant<int, 1>{});
    // tile maximum relative to the reference, over the head's 32 keys (4 rows of 16 lanes)
    const float mt = gvad::xor32_max(gvad::xor16_max(fmaxf(max4(Sc[0]), max4(Sc[1]))));
    // bitwise, so that the test compiles to one compare chain with no branch
    const bool raise = (mt > kLazyRescale) | ((mref == -INFINITY) & (mt != -INFINITY));
    if (__any(raise)) {                                // rare after the first tiles
      const float delta = raise ? mt : 0.0f;
      const float mnew = mref == -INFINITY ? mt : mref + delta;
      const float alpha = raise ? __builtin_amdgcn_exp2f(mref - mnew) : 1.0f;   // 0 from -inf
      mref = raise ? mnew : mref;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) O[i] *= alpha;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) Sc[tb] -= delta;
    }
    float pv[8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv[4 * tb + e] = __builtin_amdgcn_exp2f(Sc[tb][e]);
        lsum += pv[4 * tb + e];
      }
    u32x4 PB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned w = pack2(pv[2 * i], pv[2 * i + 1]);
      const float r0 = lo_col ? low_bf16(w) : 0.0f;
      const float r1 = lo_col ? high_bf16(w) : 0.0f;
      PB[i] = pack2(pv[2 * i] - r0, pv[2 * i + 1] - r1);
    }
    // O^T[dim][col] += C^T[dim][key] P^T[key][col]; dims 16 nb .. belong to unit step nb / 2,
    // pieces 2 (nb % 2) and + 1; the first read gives keys 4 q .. + 3 of block 0, the second the
    // same of block 1 (the order the lane holds its probabilities in)
    // (in groups of eight 16-dim blocks: their transposing reads first, then their products)
    constexpr int kGroup = 8;
    static_assert((2 * KS) % kGroup == 0, "whole groups of 16-dim blocks");
#pragma unroll
    for (int g0 = 0; g0 < 2 * KS; g0 += kGroup) {
      i16x4 v0[kGroup], v1[kGroup];
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const int nb = g0 + i;
        const int piece = 2 * (nb & 1) + (tr_k >> 1);
        const int off = 16 * ((tr_key ^ (8 * (tr_k >> 1))) + 16 * piece) + 8 * (tr_k & 1);
        v0[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(base + unit_off(0, nb >> 1, kSteps) + off));
        v1[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(base + unit_off(1, nb >> 1, kSteps) + off));
      }
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const bf16x8 VT = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(v0[i], v1[i], 0, 1, 2, 3, 4, 5, 6, 7));
        O[g0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(VT, __builtin_bit_cast(bf16x8, PB),
                                                            O[g0 + i], 0, 0, 0);
      }
      if (g0 + kGroup == KS) hook(std::integral_constant<int, 2>{});
    }
  };

  // Ring of kBufs buffers, kDepth tiles in flight: step t loads the entries of tile t + kDepth + 2,
  // stages tile t + kDepth into the buffer tile t - 1 was read from (every wave passed the
  // barrier after it), reads tile t, then waits for tile t + 1. Tiles past the chunk's end are
  // staged too (their keys repeat the last one), so every step issues the same transfers and
  // the wait is a fixed count: each step issues at least kPer vector-memory operations, so at
  // most (kDepth - 1) kPer may follow tile t + 1's. The buffer and entry-set indices are
  // compile-time constants of the unrolled ring, which lets the compiler see that a tile's LDS
  // reads do not overlap the transfers in flight.
  const int ntiles = (c1 - c0 + kTile - 1) / kTile;
  using std::integral_constant;
  auto prime = [&](auto U) __attribute__((always_inline)) {      // U < kDepth
    constexpr int u = decltype(U)::value;
    pages(pgs[(u + 2) % kBufs], c0 + (u + 2) * kTile);
    stage(ring(U), pgs[u][0], pgs[u][1], c0 + u * kTile);
  };
  auto step = [&](auto U, int t) __attribute__((always_inline)) {  // t % kBufs == U
    constexpr int u = decltype(U)::value;
    constexpr int sb = (u + kDepth) % kBufs;
    pages(pgs[(u + kDepth + 2) % kBufs], c0 + (t + kDepth + 2) * kTile);
    // tile t + kDepth's transfers in three parts: before the tile, after its scores and halfway
    // through its weighted sum, so that the waves of a CU do not all wait on one burst
    uint8_t *const sbuf = ring(integral_constant<int, sb>{});
    const int js = c0 + (t + kDepth) * kTile;
    constexpr int k1 = kPer / 3, k2 = 2 * kPer / 3;
    stage_part(integral_constant<int, 0>{}, integral_constant<int, k1>{}, sbuf, pgs[sb][0],
               pgs[sb][1], js);
    wait_lgkm0();                                      // the entries, before the tile's LDS reads
    tile(ring(U), c0 + t * kTile, [&](auto P) __attribute__((always_inline)) {
      if constexpr (decltype(P)::value == 1)
        stage_part(integral_constant<int, k1>{}, integral_constant<int, k2>{}, sbuf, pgs[sb][0],
                   pgs[sb][1], js);
      else
        stage_part(integral_constant<int, k2>{}, integral_constant<int, kPer>{}, sbuf,
                   pgs[sb][0], pgs[sb][1], js);
    });
    wait_vmcnt<(kDepth - 1) * kPer>();                 // tile t + 1's units are in LDS
    ring_barrier();
  };
  pages(pgs[0], c0);
  pages(pgs[1], c0 + kTile);
  prime(integral_constant<int, 0>{});
  prime(integral_constant<int, 1>{});
  if constexpr (kDepth > 2) prime(integral_constant<int, 2>{});
  wait_vmcnt<(kDepth - 1) * kPer>();                   // tile 0's units are in LDS
  ring_barrier();
  // whole turns of the ring, then the last ntiles % kBufs tiles (a loop without early exits:
  // the compiler then keeps track of which buffer each transfer in flight writes)
  int t0 = 0;
  for (; t0 + kBufs <= ntiles; t0 += kBufs) {          // uniform per work-group
    step(integral_constant<int, 0>{}, t0);
    step(integral_constant<int, 1>{}, t0 + 1);
    step(integral_constant<int, 2>{}, t0 + 2);
    if constexpr (kBufs > 3) step(integral_constant<int, 3>{}, t0 + 3);
  }
  if (t0 < ntiles) {
    step(integral_constant<int, 0>{}, t0);
    if (t0 + 1 < ntiles) {
      step(integral_constant<int, 1>{}, t0 + 1);
      if constexpr (kBufs > 3) {
        if (t0 + 2 < ntiles) step(integral_constant<int, 2>{}, t0 + 2);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);                       // no transfer into LDS outlives the loop
  __shared__ int bad_lds;
  if (threadIdx.x == 0) bad_lds = 0;
  __syncthreads();
  if (bad) {
    bad_lds = 1;
    gvad::raise_err(a.err_flag, GVA_DEVERR_BLOCK);
  }
  __syncthreads();
  const bool poisoned = bad_lds != 0;

  // head totals: the hi and lo columns' sums added (row rotation by 8), the probability sum
  // taken over the four rows (lsum counts each key once per column pair: use the hi lanes')
  // (the rotations read the lo lanes, so they run before those lanes stop)
  const float l = gvad::xor32_sum(gvad::xor16_sum(lo_col ? 0.0f : lsum));
  const float lt = l + ror8(l);                        // the lo lanes held 0
#pragma unroll
  for (int nb = 0; nb < 2 * KS; ++nb)
#pragma unroll
    for (int e = 0; e < 4; ++e) O[nb][e] += ror8(O[nb][e]);
  if (!lo_col) {
    const float inv = 1.0f / lt;
    float *dst = S == 1 ? a.out + orow * d_c : a.part_o + prow * d_c;
#pragma unroll
    for (int nb = 0; nb < 2 * KS; ++nb) {
      f32x4 v = O[nb];
      if (S == 1) v *= inv;
      if (poisoned) v = f32x4{qnan, qnan, qnan, qnan};
      *reinterpret_cast<f32x4 *>(dst + 16 * nb + 4 * q) = v;
    }
    if (q == 0) {
      if (S == 1) {
        if (a.lse) a.lse[orow] = poisoned ? qnan : (mref + log2f(lt)) * gvad::kLn2;
      } else {
        a.part_m[prow] = poisoned ? qnan : mref;
        a.part_l[prow] = lt;
      }
    }
  }
  }  // the work queue
}

// Empties the work queue's counter before the decode launch (a kernel rather than a memset, so
// the pair can be captured in a graph).
__global__ void k_latent_queue_reset(int32_t *next) {
  if (threadIdx.x == 0) *next = 0;
}

// Work-groups one CU holds by LDS (the registers allow as many for these kernels).
template <int KS, int RS, int NW>
constexpr int latent_groups_per_cu() {
  constexpr int lds = latent_bufs<KS, RS, NW>() * LatentTile<KS, RS>::kBytes + 1024;
  return (160 * 1024) / lds > 0 ? (160 * 1024) / lds : 1;
}

}  // namespace

namespace gva {

hipError_t launch_latent_decode(const DecodeArgs &a, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(a.B) * a.num_splits;
  if (items < 1 || items > INT32_MAX || a.H % 8 != 0 || !a.work_next) return hipErrorInvalidValue;
  const int nw = a.H / 8;
  const int rs = (a.d_r + 31) / 32;
  hipLaunchKernelGGL(k_latent_queue_reset, dim3(1), dim3(64), 0, stream, a.work_next);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
#define GVA_LATENT_CASE(KS, RS, NW)                                                           \
  if (a.d_h == 32 * KS && rs == RS && nw == NW) {                                             \
    const int64_t resident = static_cast<int64_t>(kPlanCUs) * latent_groups_per_cu<KS, RS, NW>(); \
    const dim3 grid(static_cast<unsigned>(items < resident ? items : resident));              \
    hipLaunchKernelGGL((k_latent_decode<KS, RS, NW>), grid, dim3(64 * NW), 0, stream, a);     \
    return hipGetLastError();                                                                 \
  }
  GVA_LATENT_CASE(8, 1, 1) GVA_LATENT_CASE(8, 1, 2) GVA_LATENT_CASE(8, 1, 4)
  GVA_LATENT_CASE(8, 2, 1) GVA_LATENT_CASE(8, 2, 2) GVA_LATENT_CASE(8, 2, 4)
  GVA_LATENT_CASE(16, 1, 1) GVA_LATENT_CASE(16, 1, 2) GVA_LATENT_CASE(16, 1, 4)
  GVA_LATENT_CASE(16, 2, 1) GVA_LATENT_CASE(16, 2, 2) GVA_LATENT_CASE(16, 2, 4)
#undef GVA_LATENT_CASE
  return hipErrorInvalidValue;
}

}  // namespace gva
