// k_prefill.hip - chunked causal prefill for Grouped Value Attention on matrix cores (gfx950).
//
// A chunk of C new tokens per sequence is appended to the cache first (values and the rotated
// shared positional key, exactly as the cache-append entry point writes them). Query i of
// sequence b sits at position start_b + i and attends to positions 0 .. start_b + i, inclusive,
// with the decode score q~_h . v_{j,g(h)} + r_h . kr_j ("GVA：KV 缓存里的 Key 其实可以不存",
// shibing624.github.io review of arXiv:2609.13285, sections 关键技巧一 and 关键技巧二). Prefill
// is a dense, matrix-heavy pass (agihunt.info summary of the paper): the score and the weighted
// sum are [rows x (d_h + d_r)] x [(d_h + d_r) x keys] and [rows x keys] x [keys x d_h] products
// with rows = (query, head) pairs of one value group.
//
// Work-group: 8 waves of one (sequence, group), two per SIMD, rows ordered (query, head) with
// the head fastest. Up to d_h = 128 each wave owns two tiles of 16 rows, so every operand it
// reads from LDS feeds the products of both (half the LDS instructions per product of one tile
// per wave); above, one. Keys are walked in tiles of 32 positions,
// loaded two tiles ahead into registers and staged once per work-group in LDS as natural rows
// [v (d_h) | kr (d_r, zero-padded to 32)] (double-buffered, one barrier per tile). They serve
//   * the scores S^T[key][row] = sum_k K[key][k] Q[row][k]: A = the natural rows, B = the
//     absorbed query as a bf16 hi + lo pair (two products), and
//   * the weighted sum O^T[dim][row] += sum_key V^T[dim][key] P^T[key][row]: A = V^T, read
//     from the same rows with the transposing LDS load (ds_read_b64_tr_b16), B = P in bf16.
// Each lane holds row n = lane % 16 of each of its wave's row tiles and keys 16 tb + 4 q + r of each 16-key
// block (q = lane / 16), which is the K order (q, e) -> 16 (e / 4) + 4 q + e % 4 in which the
// transposing load delivers V^T, so P feeds the second product from the lane's own registers.
// Accumulation and the online softmax (base-2 domain) are float32. The softmax keeps a lazily
// raised reference maximum per row: the scores accumulate on top of minus the reference, and the
// reference (with the rescaling of the sums) moves only when a score passes it by more than 8.
#include <hip/hip_runtime.h>

#include <math.h>

#include "gva_device.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Eight waves per work-group, two per SIMD (up to 256 registers each). Each wave owns RT row
// tiles of 16 rows: two up to d_h = 128, so that every LDS read of a key or V^T operand feeds
// the products of both, and one above, where the query and the accumulators need the
// registers.
constexpr int kWaves = 8;
template <int KS>
constexpr int row_tiles() { return KS <= 4 ? 2 : 1; }
template <int KS>
constexpr int rows_per_group() { return kWaves * 16 * row_tiles<KS>(); }
constexpr int kKeyTile = 32;

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

// ds_read_b64_tr_b16 (checked on the hardware): in each group of 16 lanes, lanes 4 e + k
// (k = 0..3) address 4 consecutive 16-bit elements each, together one row of 16; lane i of the
// group receives element e of its result from row e, column i.
__device__ __forceinline__ i16x4 read_tr(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
}

// Plain v_max_f32 / v_max3_f32: scores come straight from the matrix cores or are -inf, never
// signalling NaNs, so the operand canonicalisation the compiler adds around fmaxf is not needed.
__device__ __forceinline__ float max2(float x, float y) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ float max3(float x, float y, float z) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}
// Row maximum over the 16-lane groups (lanes n, n + 16, n + 32, n + 48 hold one row).
__device__ __forceinline__ float row_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

// The reference maximum of a row is raised only when a score passes it by more than this
// (base-2 domain), so the unnormalised probabilities stay below 2^8.
constexpr float kLazyRescale = 8.0f;

// ---- appending the chunk -----------------------------------------------------------------

// Token k of the chunk belongs to sequence k / C at position start[k / C] + k % C. The
// arithmetic is the cache-append kernel's: one rounding of each value; the positional key
// rotated in float64 (no fused multiply-add) and rounded once.
__global__ __launch_bounds__(256) void k_append_chunk(gva::DecodeArgs a, int32_t C,
                                                      const int32_t *start, const float *v_new,
                                                      const float *kr_raw, const double *rope,
                                                      int32_t max_pos) {
  const int k = blockIdx.x;
  const int b = k / C;
  const int p = start[b] + (k - b * C);
  const int cap = a.max_blocks << a.log2_bs;
  int32_t err = 0;
  if (start[b] < 0 || p < 0) err = GVA_DEVERR_LENGTH;
  else if (p >= cap) err = GVA_DEVERR_CAPACITY;
  else if (p >= max_pos) err = GVA_DEVERR_ROPE;
  int64_t blk = -1;
  if (!err) {
    blk = gvad::block_of(a, b, p);
    if (blk < 0) err = GVA_DEVERR_BLOCK;
  }
  if (err) {
    if (threadIdx.x == 0) gvad::raise_err(a.err_flag, err);
    return;
  }
  const int64_t off = p & ((1 << a.log2_bs) - 1);
  const int half_h = a.d_h >> 1;
  const float2 *src = reinterpret_cast<const float2 *>(v_new + static_cast<int64_t>(k) * a.G * a.d_h);
  uint32_t *v32 = reinterpret_cast<uint32_t *>(const_cast<void *>(a.v));
  for (int idx = threadIdx.x; idx < a.G * half_h; idx += blockDim.x) {
    const int g = idx / half_h;
    const int i = (idx - g * half_h) * 2;
    const float2 x = src[idx];
    const int64_t o = blk * a.v_sb + off * a.v_st + static_cast<int64_t>(g) * a.v_sg + i;
    v32[o >> 1] = gvad::f64_to_bf16_bits(static_cast<double>(x.x)) |
                  (static_cast<uint32_t>(gvad::f64_to_bf16_bits(static_cast<double>(x.y))) << 16);
  }
  const int half_r = a.d_r >> 1;
  const float2 *ksrc = reinterpret_cast<const float2 *>(kr_raw + static_cast<int64_t>(k) * a.d_r);
  const double2 *cs = reinterpret_cast<const double2 *>(rope) + static_cast<int64_t>(p) * half_r;
  uint32_t *k32 = reinterpret_cast<uint32_t *>(const_cast<void *>(a.kr));
  for (int i = threadIdx.x; i < half_r; i += blockDim.x) {
    const float2 x = ksrc[i];
    const double2 t = cs[i];
    double y0, y1;
    gvad::rotate_pair_f64(static_cast<double>(x.x), static_cast<double>(x.y), t.x, t.y, &y0, &y1);
    const int64_t o = blk * a.kr_sb + off * a.kr_st + 2 * i;
    k32[o >> 1] = gvad::f64_to_bf16_bits(y0) |
                  (static_cast<uint32_t>(gvad::f64_to_bf16_bits(y1)) << 16);
  }
}

// ---- attention -----------------------------------------------------------------------------

// LDS tile: 32 natural rows of (KS + 1) * 32 elements, each padded by 16 elements so that the
// four rows one transposing read touches in a group of 16 lanes fall on different banks.
template <int KS>
struct TileLds {
  static constexpr int kNatStride = (KS + 1) * 32 + 16;
  static constexpr int kElems = kKeyTile * kNatStride;
};

// A unit is 16 keys x 32 elements of the natural rows (k-step ks of key block kb); units
// ks < KS are values, unit ks == KS the positional key. Wave w stages units w, w + waves, ...;
// waves past the last unit load a copy of it and store nothing. Each lane holds 16 bytes in
// A-operand form: key 16 kb + n, elements 32 ks + 8 q .. + 8. Every load is unconditional
// (keys past the end repeat the last), so the compiler can count the loads in flight exactly
// and wait only for the one it needs.
template <int KS, int W>
struct Stage {
  static constexpr int kUnits = 2 * (KS + 1);
  static constexpr int kPerWave = (kUnits + W - 1) / W;
  u32x4 u[kPerWave];
};

// Block-table entries of the keys a wave's units read in one tile. They are loaded one stage
// before the data loads that use them, so that waiting for them does not also wait for the
// tile still in flight (memory loads complete in order).
template <int KS, int W>
struct StagePages {
  int32_t pb[Stage<KS, W>::kPerWave];
};

template <int KS, int W>
__device__ __forceinline__ int stage_unit(int wave, int i) {
  return min(wave + W * i, Stage<KS, W>::kUnits - 1);
}
// keys past the end repeat the last
__device__ __forceinline__ int stage_key(int kt0, int unit, int n, int kend) {
  return min(kt0 + 16 * (unit & 1) + n, kend - 1);
}

template <int KS, int W>
__device__ __forceinline__ void stage_pages(const gva::DecodeArgs &a, const int32_t *__restrict__ bt,
                                            int kt0, int kend, int wave, int n,
                                            StagePages<KS, W> &pg) {
#pragma unroll
  for (int i = 0; i < Stage<KS, W>::kPerWave; ++i)
    pg.pb[i] = bt[stage_key(kt0, stage_unit<KS, W>(wave, i), n, kend) >> a.log2_bs];
}

// Where this lane's units read: a fixed base pointer and the per-block and per-token strides of
// the value or positional-key rows (the units, and so the choice, are fixed per wave).
template <int KS, int W>
struct StageSrc {
  const uint16_t *base[Stage<KS, W>::kPerWave];
  int64_t sb[Stage<KS, W>::kPerWave], st[Stage<KS, W>::kPerWave];
};

// The positional key's k-step holds 32 elements. With d_r <= 16 its upper 16 hold a copy of the
// lower 16, and the query's operand there holds the lo parts of the positional query, so one
// product adds both kr . hi and kr . lo (the lo product of that step is left out); above 16 the
// step holds kr zero-padded to 32 and takes a hi and a lo product like the value steps. Lane
// (n, q) holds elements 8 rope_lane(q) .. + 7 of the key.
__device__ __forceinline__ int rope_lane(int q, int d_r) { return d_r <= 16 ? (q & 1) : q; }

template <int KS, int W>
__device__ __forceinline__ StageSrc<KS, W> stage_src(const gva::DecodeArgs &a, int g, int wave,
                                                     int q) {
  StageSrc<KS, W> src;
#pragma unroll
  for (int i = 0; i < Stage<KS, W>::kPerWave; ++i) {
    const int ks = stage_unit<KS, W>(wave, i) >> 1;
    if (ks < KS) {
      src.base[i] = static_cast<const uint16_t *>(a.v) + static_cast<int64_t>(g) * a.v_sg + 32 * ks + 8 * q;
      src.sb[i] = a.v_sb;
      src.st[i] = a.v_st;
    } else {
      // elements 8 rope_lane(q) ..: lanes past d_r read the last 8 positional-key elements and
      // the store zeroes them
      src.base[i] = static_cast<const uint16_t *>(a.kr) + min(8 * rope_lane(q, a.d_r), a.d_r - 8);
      src.sb[i] = a.kr_sb;
      src.st[i] = a.kr_st;
    }
  }
  return src;
}

// A block-table entry outside the pool is read as block 0 (so the load stays in bounds) and the
// lowest such key is kept in bad_key: the rows whose causal window reaches it become NaN.
template <int KS, int W>
__device__ __forceinline__ void stage_load(const gva::DecodeArgs &a, const StageSrc<KS, W> &src,
                                           const StagePages<KS, W> &pg, int kt0, int kend,
                                           int wave, int n, Stage<KS, W> &st, int &bad_key) {
  const int mask = (1 << a.log2_bs) - 1;
#pragma unroll
  for (int i = 0; i < Stage<KS, W>::kPerWave; ++i) {
    const int32_t pb = pg.pb[i];
    // block ids are below 2^31 (checked on the host): one unsigned compare covers both ends
    const bool ok = static_cast<uint32_t>(pb) < static_cast<uint32_t>(a.num_blocks);
    const int64_t blk = ok ? pb : 0;
    const int key = stage_key(kt0, stage_unit<KS, W>(wave, i), n, kend);
    bad_key = ok ? bad_key : min(bad_key, key);
    const int64_t row = key & mask;
    st.u[i] = *reinterpret_cast<const u32x4 *>(src.base[i] + blk * src.sb[i] + row * src.st[i]);
  }
}

template <int KS, int W>
__device__ __forceinline__ void stage_store(uint16_t *nat, int wave, int n, int q, int d_r,
                                            const Stage<KS, W> &st) {
  using L = TileLds<KS>;
#pragma unroll
  for (int i = 0; i < Stage<KS, W>::kPerWave; ++i) {
    const int unit = wave + W * i;
    if (unit >= Stage<KS, W>::kUnits) break;           // uniform per wave
    const int kb = unit & 1;
    const int ks = unit >> 1;
    u32x4 w = st.u[i];
    if (ks == KS && 8 * rope_lane(q, d_r) >= d_r) w = u32x4{0u, 0u, 0u, 0u};   // zero padding
    *reinterpret_cast<u32x4 *>(nat + (16 * kb + n) * L::kNatStride + 32 * ks + 8 * q) = w;
  }
}

template <int KS>
__global__ __launch_bounds__(64 * kWaves) void k_prefill(gva::PrefillArgs p) {
  using L = TileLds<KS>;
  constexpr int W = kWaves;
  constexpr int RT = row_tiles<KS>();
  constexpr int kRows = rows_per_group<KS>();
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][L::kElems];
  __shared__ int s_bad_key;                // lowest key read from a bad block (INT_MAX: none)
  const gva::DecodeArgs &a = p.kv;
  if (threadIdx.x == 0) s_bad_key = INT_MAX;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int n = lane & 15;
  const int q = lane >> 4;
  const int nhg = a.H / a.G;
  const int C = p.chunk_len;
  // Work-group -> (row block, group, sequence). Work-groups are dealt to the 8 XCDs in turn;
  // when the number of (sequence, group) pairs is a multiple of 8, the ids are arranged so that
  // all row blocks of one pair land on the same XCD, back to back, and share its L2 for the
  // keys and values they all read.
  const int nrows = C * nhg;
  const int nrb = (nrows + kRows - 1) / kRows;
  const int npairs = a.B * a.G;
  const int wg = blockIdx.x;
  int rb, pair;
  if ((npairs & 7) == 0) {
    const int j = wg >> 3;
    rb = j % nrb;
    pair = (wg & 7) + 8 * (j / nrb);
  } else {
    rb = wg % nrb;
    pair = wg / nrb;
  }
  const int g = pair % a.G;
  const int b = pair / a.G;
  const int row0 = rb * kRows;
  if (row0 >= nrows) return;                           // uniform per work-group
  const int P0 = p.start[b];
  const int row_len = a.d_h + a.d_r;
  const bool rope_packed = a.d_r <= 16;                // one product for the positional step
  const float qnan = __int_as_float(0x7fc00000);
  const int cap = a.max_blocks << a.log2_bs;
  // A bad start, or a chunk that does not fit the block table or the RoPE table (the chunk
  // append skipped those tokens), makes every row of the sequence NaN.
  int32_t seq_err = 0;
  if (P0 < 0 || P0 > p.max_start) seq_err = GVA_DEVERR_LENGTH;
  else if (P0 + C > cap) seq_err = GVA_DEVERR_CAPACITY;
  else if (P0 + C > p.max_pos) seq_err = GVA_DEVERR_ROPE;
  const bool seq_bad = seq_err != 0;

  // Row tile rt of this wave: rows row0 + 16 (RT wave + rt) + 0..15; this lane's row (the B
  // column) is n of each.
  int qpos[RT];                            // position of this lane's query in row tile rt
  bf16x8 QH[RT][KS + 1], QL[RT][KS + 1];   // query hi and lo parts (B operand)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = row0 + 16 * (RT * wave + rt) + n;
    const int rc = r < nrows ? r : nrows - 1;
    const int qi = rc / nhg;
    const int h = a.head_of[g * nhg + (rc - qi * nhg)];
    qpos[rt] = P0 + qi;
    const float *qp = p.q_abs + ((static_cast<int64_t>(b) * C + qi) * a.H + h) * row_len;
#pragma unroll
    for (int ks = 0; ks <= KS; ++ks) {
      u32x4 hi, lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x0, x1;
        if (ks < KS) {
          x0 = qp[32 * ks + 8 * q + 2 * i];
          x1 = qp[32 * ks + 8 * q + 2 * i + 1];
        } else {
          const int e = 8 * rope_lane(q, a.d_r) + 2 * i;
          x0 = e < a.d_r ? qp[a.d_h + e] : 0.0f;
          x1 = e + 1 < a.d_r ? qp[a.d_h + e + 1] : 0.0f;
        }
        x0 *= a.qscale;
        x1 *= a.qscale;
        const unsigned w = pack2(x0, x1);
        hi[i] = w;
        lo[i] = pack2(x0 - low_bf16(w), x1 - high_bf16(w));
      }
      // the packed positional step: the upper half of the operand (q >= 2) is the lo part
      QH[rt][ks] = as_bf16(ks == KS && rope_packed && q >= 2 ? lo : hi);
      QL[rt][ks] = as_bf16(lo);
    }
  }

  f32x4 O[RT][2 * KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) O[rt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Online softmax with a lazily raised reference: mref is the row's reference maximum (base 2),
  // -inf until the row's first unmasked key. The scores of a tile accumulate on top of negm =
  // -mref (0 while mref = -inf), so the probabilities are exp2 of the accumulators directly.
  float mref[RT], lsum[RT], negm[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    mref[rt] = -INFINITY;
    lsum[rt] = 0.0f;
    negm[rt] = 0.0f;
  }

  // keys 0 .. kend - 1 are seen by some row of this work-group
  const int last_row = min(row0 + kRows, nrows) - 1;
  const int kend = seq_bad ? 0 : P0 + last_row / nhg + 1;
  const int first_q = P0 + row0 / nhg;                 // every key below it is seen by all rows
  const int32_t *__restrict__ bt = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
  // transposing-read address of this lane: row lane / 4, columns 4 (lane % 4) ..
  const int tr_off = (lane >> 2) * L::kNatStride + 4 * (lane & 3);

  int bad_key = INT_MAX;                   // this lane's lowest key read from a bad block
  f32x4 S[RT][2];   // scores of the current tile, from its products to its softmax
  u32x4 PB[RT];     // its probabilities (bf16 pairs), from its softmax to its weighted sum

  // Score products of the tile in nat (starting at key kt0), and its causal mask.
  auto scores = [&](const uint16_t *nat, int kt0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) S[rt][0] = S[rt][1] = f32x4{negm[rt], negm[rt], negm[rt], negm[rt]};
#pragma unroll
    for (int ks = 0; ks <= KS; ++ks) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const u32x4 ka = *reinterpret_cast<const u32x4 *>(nat + (16 * tb + n) * L::kNatStride +
                                                          32 * ks + 8 * q);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          S[rt][tb] = mfma(as_bf16(ka), QH[rt][ks], S[rt][tb]);
          if (ks < KS || !rope_packed)                   // uniform
            S[rt][tb] = mfma(as_bf16(ka), QL[rt][ks], S[rt][tb]);
        }
      }
    }
    // causal mask (only tiles that reach past the first query)
    if (kt0 + kKeyTile - 1 > first_q) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kt0 + 16 * tb + 4 * q + e > qpos[rt]) S[rt][tb][e] = -INFINITY;
    }
  };
  // Online softmax of the scores S into PB (and the rare move of the reference).
  auto softmax = [&]() {
    // Each lane tests its own eight scores: a row's reference can only move when one of its
    // lanes holds a score above kLazyRescale (or the row's first unmasked score arrives), so the
    // exact row maximum, a cross-lane reduction, is formed only on that rare path. The test is
    // bitwise, one compare chain with no branch per row tile.
    float lm[RT];
    bool need = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const f32x4 &s0 = S[rt][0], &s1 = S[rt][1];
      lm[rt] = max2(max3(s0[0], s0[1], s0[2]), max3(s0[3], s1[0], max3(s1[1], s1[2], s1[3])));
      need = need | (lm[rt] > kLazyRescale) | ((mref[rt] == -INFINITY) & (lm[rt] != -INFINITY));
    }
    if (__any(need)) {   // rare after the first tiles: move the reference to the tile maximum
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float mt = row_max(lm[rt]);
        const bool raise = (mt > kLazyRescale) | ((mref[rt] == -INFINITY) & (mt != -INFINITY));
        const float delta = raise ? mt : 0.0f;
        const float mnew = mref[rt] == -INFINITY ? mt : mref[rt] + delta;
        const float alpha = raise ? __builtin_amdgcn_exp2f(mref[rt] - mnew) : 1.0f;   // 0 from -inf
        mref[rt] = raise ? mnew : mref[rt];
        negm[rt] = raise ? -mnew : negm[rt];
        lsum[rt] *= alpha;
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) O[rt][i] *= alpha;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) S[rt][tb] -= delta;
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float pv[8];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[4 * tb + e] = __builtin_amdgcn_exp2f(S[rt][tb][e]);
          lsum[rt] += pv[4 * tb + e];
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) PB[rt][i] = pack2(pv[2 * i], pv[2 * i + 1]);
    }
  };
  // Weighted sum of the tile in nat with PB: O^T[dim][row] += V^T[dim][key] P^T[key][row]; V^T
  // of dims 16 nb .. read transposed: the first read gives keys 4 q .. + 3 of block 0, the
  // second the same of block 1.
  auto weighted_sum = [&](const uint16_t *nat) {
#pragma unroll
    for (int nb = 0; nb < 2 * KS; ++nb) {
      const i16x4 v0 = read_tr(nat + tr_off + 16 * nb);
      const i16x4 v1 = read_tr(nat + tr_off + 16 * L::kNatStride + 16 * nb);
      const bf16x8 VT = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) O[rt][nb] = mfma(VT, as_bf16(PB[rt]), O[rt][nb]);
    }
  };

  if (kend > 0) {
    // Tiles are loaded two ahead: while tile i is computed, tile i + 1 waits in registers (to
    // be stored into the other LDS buffer) and tile i + 2 is in flight. The two register stages
    // alternate roles, so the loop runs over pairs of tiles; it has no early exit, so that the
    // number of loads in flight is the same on every path into its head, and the last one or
    // two tiles follow it. Loads past the last tile read its keys again and are not used.
    auto tile = [&](const uint16_t *nat, int kt0) {
      scores(nat, kt0);
      softmax();
      weighted_sum(nat);
    };
    const int ntiles = (kend + kKeyTile - 1) / kKeyTile;
    const StageSrc<KS, W> src = stage_src<KS, W>(a, g, wave, q);
    Stage<KS, W> s0, s1;
    StagePages<KS, W> p0, p1;
    stage_pages<KS, W>(a, bt, 0, kend, wave, n, p0);
    stage_pages<KS, W>(a, bt, kKeyTile, kend, wave, n, p1);
    stage_load<KS, W>(a, src, p0, 0, kend, wave, n, s0, bad_key);
    stage_pages<KS, W>(a, bt, 2 * kKeyTile, kend, wave, n, p0);
    stage_load<KS, W>(a, src, p1, kKeyTile, kend, wave, n, s1, bad_key);
    stage_pages<KS, W>(a, bt, 3 * kKeyTile, kend, wave, n, p1);
    stage_store<KS, W>(lds[0], wave, n, q, a.d_r, s0);
    __syncthreads();
    int t = 0;
    for (; t + 2 < ntiles; t += 2) {
      const int kt0 = t * kKeyTile;
      // tile t in lds[0]; tile t + 1 in s1; s0 free; p0 holds the pages of tile t + 2
      stage_load<KS, W>(a, src, p0, kt0 + 2 * kKeyTile, kend, wave, n, s0, bad_key);
      stage_pages<KS, W>(a, bt, kt0 + 4 * kKeyTile, kend, wave, n, p0);
      tile(lds[0], kt0);
      stage_store<KS, W>(lds[1], wave, n, q, a.d_r, s1);
      __syncthreads();
      // tile t + 1 in lds[1]; tile t + 2 in s0; s1 free; p1 holds the pages of tile t + 3
      stage_load<KS, W>(a, src, p1, kt0 + 3 * kKeyTile, kend, wave, n, s1, bad_key);
      stage_pages<KS, W>(a, bt, kt0 + 5 * kKeyTile, kend, wave, n, p1);
      tile(lds[1], kt0 + kKeyTile);
      stage_store<KS, W>(lds[0], wave, n, q, a.d_r, s0);
      __syncthreads();
    }
    // one or two tiles left: tile t in lds[0], tile t + 1 (if any) in s1
    tile(lds[0], t * kKeyTile);
    if (t + 1 < ntiles) {                              // uniform per work-group
      stage_store<KS, W>(lds[1], wave, n, q, a.d_r, s1);
      __syncthreads();
      tile(lds[1], (t + 1) * kKeyTile);
    }
  }

  // the work-group's lowest bad key (every wave has passed the barrier after s_bad_key's
  // initialisation when any lane holds one: loads happen only when kend > 0, whose loop has one)
  {
    int m = bad_key;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = min(m, __shfl_xor(m, o, 64));
    if (lane == 0 && m != INT_MAX) atomicMin(&s_bad_key, m);
    __syncthreads();
  }
  const int wg_bad_key = s_bad_key;
  if (wg_bad_key != INT_MAX && threadIdx.x == 0) gvad::raise_err(a.err_flag, GVA_DEVERR_BLOCK);

  // ---- epilogue: lane (n, q) holds row n of each row tile, dims 16 nb + 4 q + e ----
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float lt = gvad::xor32_sum(gvad::xor16_sum(lsum[rt]));
    const int r = row0 + 16 * (RT * wave + rt) + n;
    if (r < nrows) {
      const int qi = r / nhg;
      const int h = a.head_of[g * nhg + (r - qi * nhg)];
      const int64_t orow = (static_cast<int64_t>(b) * C + qi) * a.H + h;
      float *dst = p.out + orow * a.d_h + 4 * q;
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      // the row sees keys 0 .. P0 + qi: a bad block among them poisons it
      const bool poison = seq_bad || wg_bad_key <= P0 + qi;
#pragma unroll
      for (int nb = 0; nb < 2 * KS; ++nb) {
        f32x4 v = O[rt][nb] * inv;
        if (poison) v = f32x4{qnan, qnan, qnan, qnan};
        *reinterpret_cast<f32x4 *>(dst + 16 * nb) = v;
      }
      if (p.lse && q == 0)
        p.lse[orow] = poison ? qnan : (lt > 0.0f ? (mref[rt] + log2f(lt)) * gvad::kLn2 : -INFINITY);
    }
  }
  if (seq_bad && threadIdx.x == 0 && rb == 0 && g == 0) gvad::raise_err(a.err_flag, seq_err);
}

}  // namespace

namespace gva {

hipError_t launch_prefill(const PrefillArgs &p, hipStream_t stream) {
  const DecodeArgs &a = p.kv;
  const int C = p.chunk_len;
  hipLaunchKernelGGL(k_append_chunk, dim3(a.B * C), dim3(256), 0, stream, a, C, p.start, p.v_new,
                     p.kr_raw, p.rope, p.max_pos);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nrows = C * (a.H / a.G);
  const int64_t pairs = static_cast<int64_t>(a.G) * a.B;
  auto grid = [&](int rows) { return dim3(static_cast<unsigned>((nrows + rows - 1) / rows * pairs)); };
#define GVA_PREFILL_CASE(KS)                                                                  \
  case KS:                                                                                    \
    hipLaunchKernelGGL(k_prefill<KS>, grid(rows_per_group<KS>()), dim3(64 * kWaves), 0,       \
                       stream, p);                                                            \
    break;
  switch (a.d_h / 32) {
    GVA_PREFILL_CASE(1)
    GVA_PREFILL_CASE(2)
    GVA_PREFILL_CASE(3)
    GVA_PREFILL_CASE(4)
    GVA_PREFILL_CASE(5)
    GVA_PREFILL_CASE(6)
    GVA_PREFILL_CASE(7)
    GVA_PREFILL_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef GVA_PREFILL_CASE
  return hipGetLastError();
}

}  // namespace gva
