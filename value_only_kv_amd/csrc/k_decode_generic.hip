// k_decode_generic.hip - vector-ALU split decode for Grouped Value Attention, any supported
// shape and cache type (float32 or bfloat16), and the log-sum-exp combine of the splits.
//
// Score of cached position j for head h: q~_h . v_{j,g(h)} + r_h . kr_j, with q~_h the absorbed
// content query and r_h the rotated positional query ("GVA：KV 缓存里的 Key 其实可以不存",
// shibing624.github.io review of arXiv:2609.13285, sections 关键技巧一 and 关键技巧二), then a
// softmax over the cached positions and a weighted sum of the same cached values (agihunt.info
// summary of the paper; "KV Cache 优化（一）", liumengxuan04.github.io, section 1).
//
// One wave per (split, sequence, group, head pass). A chunk is walked in tiles of 64 positions:
// lane t scores position t of the tile for every head of the pass (one lane per position, no
// cross-lane reduction), the wave then updates the running max / sum of each head, and the
// weighted sum runs with lanes over the value dimensions. Scores live in the base-2 domain
// (the query is pre-multiplied by scale * log2 e), so exponentials are exp2.
#include <hip/hip_runtime.h>

#include <math.h>

#include "gva_device.h"

namespace {

constexpr int kHeadsPerPass = 16;   // heads of one group handled by one wave
constexpr int kTile = 64;           // positions per tile (one per lane)
constexpr int kPvBatch = 16;        // positions whose values are loaded together

template <bool BF16>
__device__ __forceinline__ float2 load_pair(const void *base, int64_t off) {
  if (BF16) {
    const uint32_t w = reinterpret_cast<const uint32_t *>(base)[off >> 1];
    return make_float2(gvad::bf16_bits_to_f32(w & 0xffffu), gvad::bf16_bits_to_f32(w >> 16));
  }
  return *reinterpret_cast<const float2 *>(reinterpret_cast<const float *>(base) + off);
}

template <bool BF16>
__device__ __forceinline__ float load_one(const void *base, int64_t off) {
  if (BF16) return gvad::bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(base)[off]);
  return reinterpret_cast<const float *>(base)[off];
}

// Writes the (m, l, o) of a finished chunk, or the final row when there is a single split.
// o holds DPL values per lane: dims lane, lane + 64, ...
template <int DPL>
__device__ __forceinline__ void store_rows(const gva::DecodeArgs &a, int b, int s, int h0, int nh,
                                           const float *m, const float *l,
                                           const float (*o)[DPL], bool poison) {
  const int lane = threadIdx.x;
  const float qnan = __int_as_float(0x7fc00000);
  for (int hh = 0; hh < nh; ++hh) {
    const int h = a.head_of[h0 + hh];
    if (a.num_splits == 1) {
      const float inv = l[hh] > 0.0f ? 1.0f / l[hh] : 0.0f;
      float *dst = a.out + (static_cast<int64_t>(b) * a.H + h) * a.d_h;
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int d = lane + 64 * k;
        if (d < a.d_h) dst[d] = poison ? qnan : o[hh][k] * inv;
      }
      if (a.lse && lane == 0) {
        float v = l[hh] > 0.0f ? (m[hh] + log2f(l[hh])) * gvad::kLn2 : -INFINITY;
        a.lse[static_cast<int64_t>(b) * a.H + h] = poison ? qnan : v;
      }
    } else {
      const int64_t row = (static_cast<int64_t>(b) * a.num_splits + s) * a.H + h;
      float *dst = a.part_o + row * a.d_h;
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int d = lane + 64 * k;
        if (d < a.d_h) dst[d] = o[hh][k];
      }
      if (lane == 0) {
        a.part_m[row] = poison ? qnan : m[hh];
        a.part_l[row] = l[hh];
      }
    }
  }
}

// NHP: heads per wave, a power of two covering the group's heads of this pass; the heads past
// nh are computed with a zero query and never stored, so the loops over heads have no branches.
template <bool BF16, int DPL, int NHP>
__global__ __launch_bounds__(64) void k_decode_generic(gva::DecodeArgs a, int head_passes) {
  __shared__ float q_s[NHP][gva::kMaxDh + gva::kMaxDr];
  __shared__ float p_s[NHP][kTile];
  __shared__ int64_t vo_s[kTile];
  const int s = blockIdx.x;
  const int b = blockIdx.y;
  const int g = blockIdx.z / head_passes;
  const int hp = blockIdx.z - g * head_passes;
  const int hpg = a.H / a.G;
  const int h0 = g * hpg + hp * kHeadsPerPass;     // first slot of this pass in a.head_of
  const int nh = min(kHeadsPerPass, hpg - hp * kHeadsPerPass);
  const int lane = threadIdx.x;
  const int d_h = a.d_h, d_r = a.d_r, row = d_h + d_r;

  float m[NHP], l[NHP], o[NHP][DPL];
#pragma unroll
  for (int hh = 0; hh < NHP; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[hh][k] = 0.0f;
  }

  const int len = a.seq_len[b];
  const int cap = a.max_blocks << a.log2_bs;
  bool poison = false;
  if (len < 0 || len > a.max_len || len > cap) {
    if (lane == 0 && s == 0 && blockIdx.z == 0) gvad::raise_err(a.err_flag, GVA_DEVERR_LENGTH);
    store_rows<DPL>(a, b, s, h0, nh, m, l, o, true);
    return;
  }
  const int c0 = s * a.chunk;
  const int c1 = min(c0 + a.chunk, len);
  if (c0 >= c1) {
    store_rows<DPL>(a, b, s, h0, nh, m, l, o, false);
    return;
  }

  for (int idx = lane; idx < NHP * row; idx += 64) {
    const int hh = idx / row;
    const int e = idx - hh * row;
    q_s[hh][e] = hh < nh ? a.q_abs[(static_cast<int64_t>(b) * a.H + a.head_of[h0 + hh]) * row + e] * a.qscale
                         : 0.0f;
  }
  __syncthreads();

  const int bs_mask = (1 << a.log2_bs) - 1;
  for (int t0 = c0; t0 < c1; t0 += kTile) {
    // ---- scores: one position per lane ----
    const int t = t0 + lane;
    const bool valid = t < c1;
    const int tc = valid ? t : c1 - 1;
    const int64_t blk = gvad::block_of(a, b, tc);
    if (blk < 0) poison = true;
    const int64_t blk_s = blk < 0 ? 0 : blk;
    const int64_t voff = blk_s * a.v_sb + static_cast<int64_t>(tc & bs_mask) * a.v_st +
                         static_cast<int64_t>(g) * a.v_sg;
    const int64_t koff = blk_s * a.kr_sb + static_cast<int64_t>(tc & bs_mask) * a.kr_st;
    vo_s[lane] = voff;                         // the weighted sum reads the rows from here
    float sc[NHP];
#pragma unroll
    for (int hh = 0; hh < NHP; ++hh) sc[hh] = 0.0f;
#pragma unroll 16
    for (int i = 0; i < d_h; i += 2) {
      const float2 x = load_pair<BF16>(a.v, voff + i);
#pragma unroll
      for (int hh = 0; hh < NHP; ++hh) sc[hh] = fmaf(q_s[hh][i], x.x, fmaf(q_s[hh][i + 1], x.y, sc[hh]));
    }
#pragma unroll 4
    for (int i = 0; i < d_r; i += 2) {
      const float2 x = load_pair<BF16>(a.kr, koff + i);
#pragma unroll
      for (int hh = 0; hh < NHP; ++hh)
        sc[hh] = fmaf(q_s[hh][d_h + i], x.x, fmaf(q_s[hh][d_h + i + 1], x.y, sc[hh]));
    }
    // ---- online softmax over the tile, per head ----
#pragma unroll
    for (int hh = 0; hh < NHP; ++hh) {
      const float sv = valid ? sc[hh] : -INFINITY;
      const float mn = fmaxf(m[hh], gvad::wave_max(sv));
      const float alpha = exp2f(m[hh] - mn);
      const float p = exp2f(sv - mn);
      l[hh] = l[hh] * alpha + gvad::wave_sum(p);
      m[hh] = mn;
      p_s[hh][lane] = p;
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[hh][k] *= alpha;
    }
    __syncthreads();
    // ---- weighted sum: lanes over value dimensions ----
    // The row offsets come from LDS (no block-table lookups in this loop), and the values of 16
    // positions are loaded before their products, so a tile costs four load round trips.
    const int nt = min(kTile, c1 - t0);
    for (int j0 = 0; j0 < nt; j0 += kPvBatch) {
      float x[kPvBatch][DPL];
#pragma unroll
      for (int u = 0; u < kPvBatch; ++u)
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
          const int d = lane + 64 * k;
          x[u][k] = (j0 + u < nt && d < d_h) ? load_one<BF16>(a.v, vo_s[j0 + u] + d) : 0.0f;
        }
#pragma unroll
      for (int u = 0; u < kPvBatch; ++u) {
        if (j0 + u < nt) {
#pragma unroll
          for (int hh = 0; hh < NHP; ++hh) {
            const float pj = p_s[hh][j0 + u];
#pragma unroll
            for (int k = 0; k < DPL; ++k) o[hh][k] = fmaf(pj, x[u][k], o[hh][k]);
          }
        }
      }
    }
    __syncthreads();
  }
  // a poisoned split is reported once per wave
  const bool any_poison = __any(poison);
  if (any_poison && lane == 0) gvad::raise_err(a.err_flag, GVA_DEVERR_BLOCK);
  store_rows<DPL>(a, b, s, h0, nh, m, l, o, any_poison);
}

// Combine: m* = max over a sequence's non-empty chunks, L = sum l_c 2^(m_c - m*),
// out = sum o_c 2^(m_c - m*) / L and lse = (m* + log2 L) ln 2. One work-group per
// (64-dim slice, head, sequence) with nw waves (1 .. 16, growing with the split count): the
// chunk weights 2^(m_c - m*) are formed once in LDS, wave w sums chunks w, w + nw, ... with its
// lanes over the slice's dims, and the waves' sums meet in LDS.
constexpr int kCombineMaxWaves = 16;
// partial rows per sequence up to which the combine takes one wave per (sequence, head)
constexpr int kCombineWaveRows = 16;
// o rows per lane of k_combine loaded in the first round
constexpr int kCombineRows = 16;
// partial rows per lane of k_combine_slice at most (8 lanes share a slice's rows)
constexpr int kCombineSliceMaxK = 32;

__device__ __forceinline__ float block_reduce(float v, float *scratch, int nw, bool is_max) {
  v = is_max ? gvad::wave_max(v) : gvad::wave_sum(v);
  if (nw == 1) return v;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  float r = scratch[0];
  for (int i = 1; i < nw; ++i) r = is_max ? fmaxf(r, scratch[i]) : r + scratch[i];
  __syncthreads();
  return r;
}

// The partial rows of (sequence b, head h): rows row0 + s H for s < ns.
__device__ __forceinline__ void partial_rows(const gva::DecodeArgs &a, int b, int h, int len,
                                             int &ns, int64_t &row0) {
  if (a.num_ranges > 0) {
    // balanced mode: the ranges holding tiles [P[b], P[b + 1]) are those containing its first
    // and last tile (with Re = min(R, T) ranges, range r starts at tile r T / Re and is never
    // empty), and range r wrote row (r + b) H + h
    const int64_t pb = a.tile_prefix[b];
    const int64_t pe = a.tile_prefix[b + 1];
    const int64_t T = a.tile_prefix[a.B];
    const int64_t Re = T < a.num_ranges ? T : a.num_ranges;
    if (pe <= pb) {
      ns = 0;
      row0 = 0;
    } else {
      const int64_t r_first = ((pb + 1) * Re - 1) / T;
      const int64_t r_last = (pe * Re - 1) / T;
      ns = static_cast<int>(r_last - r_first + 1);
      row0 = (r_first + b) * a.H + h;
    }
  } else {
    ns = min(a.num_splits, (len + a.chunk - 1) / a.chunk);
    row0 = static_cast<int64_t>(b) * a.num_splits * a.H + h;
  }
}

__global__ __launch_bounds__(64 * kCombineMaxWaves) void k_combine(gva::DecodeArgs a) {
  __shared__ float w_s[gva::kMaxSplits];
  __shared__ float part[kCombineMaxWaves][64];
  __shared__ float scratch[kCombineMaxWaves];
  const int d0 = 64 * blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int nthr = blockDim.x;
  const int d = d0 + lane;
  const bool dim_ok = d < a.d_h;
  const float qnan = __int_as_float(0x7fc00000);
  float *dst = a.out + (static_cast<int64_t>(b) * a.H + h) * a.d_h;
  const bool write_lse = a.lse && tid == 0 && blockIdx.x == 0;
  const int cap = a.max_blocks << a.log2_bs;
  // Every partial this thread needs goes out before any is used: split tid's m and l, and the
  // first kCombineRows of this wave's o rows wave, wave + nw, ... (loads past the last row
  // re-read it; what they bring is never used). In the split grid the rows (row0 + s H,
  // s < num_splits) are known before the length, so these loads go out with it: one round of
  // loads in all; the balanced plan needs the tile prefix first. The arithmetic and its order
  // do not depend on this. Split counts above the block's threads, and rows past the first
  // kCombineRows, are read in further passes.
  const bool split = a.num_ranges == 0;
  const int64_t step = static_cast<int64_t>(a.H) * a.d_h;
  int64_t row0 = split ? static_cast<int64_t>(b) * a.num_splits * a.H + h : 0;
  float m0 = 0.0f, l0 = 0.0f;
  float ov[kCombineRows];
  const float *po = a.part_o;
  auto issue = [&](int nload) {
    const int sm = min(tid, nload - 1);
    m0 = a.part_m[row0 + static_cast<int64_t>(sm) * a.H];
    l0 = a.part_l[row0 + static_cast<int64_t>(sm) * a.H];
    po = a.part_o + row0 * a.d_h + (dim_ok ? d : 0);
#pragma unroll
    for (int j = 0; j < kCombineRows; ++j)
      ov[j] = po[static_cast<int64_t>(min(wave + nw * j, nload - 1)) * step];
  };
  if (split) issue(a.num_splits);
  const int len = a.seq_len[b];
  if (len < 0 || len > a.max_len || len > cap) {
    if (wave == 0 && dim_ok) dst[d] = qnan;
    if (write_lse) a.lse[static_cast<int64_t>(b) * a.H + h] = qnan;
    if (a.num_ranges > 0 && tid == 0 && blockIdx.x == 0 && h == 0)
      gvad::raise_err(a.err_flag, GVA_DEVERR_LENGTH);
    return;
  }
  int ns;
  partial_rows(a, b, h, len, ns, row0);
  if (ns == 0) {
    if (wave == 0 && dim_ok) dst[d] = 0.0f;
    if (write_lse) a.lse[static_cast<int64_t>(b) * a.H + h] = -INFINITY;
    return;
  }
  if (!split) issue(ns);
  const int keep = tid < ns ? -1 : 0;                  // a bitwise blend, not a select on a load
  float mx = fmaxf(-INFINITY, __int_as_float((__float_as_int(m0) & keep) |
                                             (__float_as_int(-INFINITY) & ~keep)));
  float bad = (tid < ns && isnan(m0)) ? 1.0f : 0.0f;
  for (int s = tid + nthr; s < ns; s += nthr) {
    const float ms = a.part_m[row0 + static_cast<int64_t>(s) * a.H];
    bad += isnan(ms) ? 1.0f : 0.0f;
    mx = fmaxf(mx, ms);
    w_s[s] = ms;
  }
  mx = block_reduce(mx, scratch, nw, true);
  const bool poison = block_reduce(bad, scratch, nw, false) > 0.0f;
  float L = 0.0f;
  {
    const float f = exp2f(m0 - mx);
    if (tid < ns) w_s[tid] = f;
    L = __int_as_float(__float_as_int(l0 * f) & keep);
  }
  for (int s = tid + nthr; s < ns; s += nthr) {
    const float f = exp2f(w_s[s] - mx);
    w_s[s] = f;
    L += a.part_l[row0 + static_cast<int64_t>(s) * a.H] * f;
  }
  L = block_reduce(L, scratch, nw, false);
  if (nw == 1) __syncthreads();  // the w_s writes of other lanes must be visible
  float acc = 0.0f;
  if (dim_ok) {
#pragma unroll
    for (int j = 0; j < kCombineRows; ++j) {
      const int s = wave + nw * j;
      if (s < ns) acc = fmaf(ov[j], w_s[s], acc);      // uniform per wave
    }
#pragma unroll 8
    for (int s = wave + nw * kCombineRows; s < ns; s += nw) acc = fmaf(po[s * step], w_s[s], acc);
  }
  if (nw > 1) {
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
      acc = 0.0f;
      for (int w = 0; w < nw; ++w) acc += part[w][lane];
    }
  }
  if (wave == 0 && dim_ok) dst[d] = poison ? qnan : acc / L;
  if (write_lse) a.lse[static_cast<int64_t>(b) * a.H + h] = poison ? qnan : (mx + log2f(L)) * gvad::kLn2;
}


// Split-grid combine of one sequence over 17 .. 8 K chunks, one wave per (32-dim slice, head),
// with no LDS and no barriers. Lane r + 8 c holds the partial rows s = r + 8 k (k < K) of dims
// 32 j + 4 c .. + 3, with their m and l: the 8 lanes of a row read its slice's 128 bytes, one
// whole line, so each load instruction reads 8 whole lines. The rows are known before the
// sequence's length and its chunks are usually all in use, so every load goes out with the
// length's; rows at or past the chunk count are loaded but dropped by a bitwise blend (their
// workspace rows may hold anything). The maximum, the sum of l 2^(m - max) and the weighted rows
// meet through cross-lane reductions. Same formulas as k_combine (base-2 m and lse, weights
// 2^(m_s - max)); the order of the sums differs. Batches keep k_combine: there the chunk counts
// differ per sequence, and it reads only the rows in use, in whole 256-byte pieces.
template <int K>
__global__ __launch_bounds__(64) void k_combine_slice(gva::DecodeArgs a) {
  const int lane = threadIdx.x;
  const int r = lane & 7;
  const int c = lane >> 3;
  const int j = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int S = a.num_splits;
  const int64_t row0 = static_cast<int64_t>(b) * S * a.H + h;
  const int d = 32 * j + 4 * c;
  float4 o[K];
  float m[K], l[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t row = row0 + static_cast<int64_t>(min(r + 8 * k, S - 1)) * a.H;
    m[k] = a.part_m[row];
    l[k] = a.part_l[row];
    o[k] = *reinterpret_cast<const float4 *>(a.part_o + row * a.d_h + d);
  }
  const int len = a.seq_len[b];
  float *dst = a.out + (static_cast<int64_t>(b) * a.H + h) * a.d_h + d;
  float *lse = (a.lse && j == 0 && lane == 0) ? a.lse + static_cast<int64_t>(b) * a.H + h : nullptr;
  const float qnan = __int_as_float(0x7fc00000);
  const int cap = a.max_blocks << a.log2_bs;
  if (len < 0 || len > a.max_len || len > cap) {
    if (r == 0) *reinterpret_cast<float4 *>(dst) = make_float4(qnan, qnan, qnan, qnan);
    if (lse) *lse = qnan;
    return;
  }
  const int ns = min(S, (len + a.chunk - 1) / a.chunk);
  if (ns == 0) {
    if (r == 0) *reinterpret_cast<float4 *>(dst) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lse) *lse = -INFINITY;
    return;
  }
  float mx = -INFINITY;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int keep = r + 8 * k < ns ? -1 : 0;
    m[k] = __int_as_float((__float_as_int(m[k]) & keep) | (__float_as_int(-INFINITY) & ~keep));
    l[k] = __int_as_float(__float_as_int(l[k]) & keep);
    o[k] = make_float4(__int_as_float(__float_as_int(o[k].x) & keep),
                       __int_as_float(__float_as_int(o[k].y) & keep),
                       __int_as_float(__float_as_int(o[k].z) & keep),
                       __int_as_float(__float_as_int(o[k].w) & keep));
    bad = bad || isnan(m[k]);
    mx = fmaxf(mx, m[k]);
  }
  mx = gvad::wave_max(mx);
  const bool poison = __any(bad);
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const float f = exp2f(m[k] - mx);               // 0 for dropped rows
    L = fmaf(l[k], f, L);
    acc.x = fmaf(o[k].x, f, acc.x);
    acc.y = fmaf(o[k].y, f, acc.y);
    acc.z = fmaf(o[k].z, f, acc.z);
    acc.w = fmaf(o[k].w, f, acc.w);
  }
  // sums over r (the 8 lanes of a group hold the same dims); every group of 8 holds all partial
  // rows' l once, so L is summed over the lanes of one group
#pragma unroll
  for (int x = 1; x < 8; x <<= 1) {
    L += __shfl_xor(L, x, 64);
    acc.x += __shfl_xor(acc.x, x, 64);
    acc.y += __shfl_xor(acc.y, x, 64);
    acc.z += __shfl_xor(acc.z, x, 64);
    acc.w += __shfl_xor(acc.w, x, 64);
  }
  if (r == 0) {
    *reinterpret_cast<float4 *>(dst) =
        poison ? make_float4(qnan, qnan, qnan, qnan)
               : make_float4(acc.x / L, acc.y / L, acc.z / L, acc.w / L);
  }
  if (lse) *lse = poison ? qnan : (mx + log2f(L)) * gvad::kLn2;
}

// One wave per (sequence, head), four heads per work-group, for sequences with few partial rows
// (the balanced plan gives about R / B + 1 of them): no LDS and no barriers. The length and the
// tile prefix are loaded together; then m, l and the first kPre rows of o are all in flight at
// once (rows past the last read the last row again, with weight 0), so the common case waits
// for two rounds of loads. Lane s holds row s's m and l (rows are taken 64 at a time); lane i
// accumulates dims i, i + 64, ... of the output. Same arithmetic as k_combine: m and lse in the
// base-2 domain, weights 2^(m_s - max).
template <int DPL>
__global__ __launch_bounds__(256) void k_combine_wave(gva::DecodeArgs a) {
  constexpr int kPre = 4;
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (h >= a.H) return;                                // uniform per wave
  const float qnan = __int_as_float(0x7fc00000);
  float *dst = a.out + (static_cast<int64_t>(b) * a.H + h) * a.d_h;
  float *lse = a.lse ? a.lse + static_cast<int64_t>(b) * a.H + h : nullptr;
  const int len = a.seq_len[b];
  int ns;
  int64_t row0;
  partial_rows(a, b, h, len, ns, row0);
  const int cap = a.max_blocks << a.log2_bs;
  const bool bad = len < 0 || len > a.max_len || len > cap;
  if (bad || ns == 0) {                                // NaN for a bad length, else empty: 0, -inf
#pragma unroll
    for (int k = 0; k < DPL; ++k)
      if (lane + 64 * k < a.d_h) dst[lane + 64 * k] = bad ? qnan : 0.0f;
    if (lse && lane == 0) *lse = bad ? qnan : -INFINITY;
    if (bad && a.num_ranges > 0 && lane == 0 && h == 0) gvad::raise_err(a.err_flag, GVA_DEVERR_LENGTH);
    return;
  }
  const int64_t step = a.H;                            // rows of one (sequence, head) are H apart
  const float *po = a.part_o + row0 * a.d_h + lane;
  const int64_t ostep = step * a.d_h;
  // first rows of o, in flight together with m and l
  float opre[kPre][DPL];
#pragma unroll
  for (int j = 0; j < kPre; ++j)
#pragma unroll
    for (int k = 0; k < DPL; ++k)
      opre[j][k] = lane + 64 * k < a.d_h ? po[min(j, ns - 1) * ostep + 64 * k] : 0.0f;
  float ms = lane < ns ? a.part_m[row0 + lane * step] : -INFINITY;
  float ls = lane < ns ? a.part_l[row0 + lane * step] : 0.0f;
  // maximum of m over all rows (and whether any is NaN)
  bool poison = __any(isnan(ms));
  float mx = gvad::wave_max(ms);
  for (int s0 = 64; s0 < ns; s0 += 64) {
    const float m2 = s0 + lane < ns ? a.part_m[row0 + (s0 + lane) * step] : -INFINITY;
    poison |= __any(isnan(m2));
    mx = fmaxf(mx, gvad::wave_max(m2));
  }
  float acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.0f;
  float L = 0.0f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    if (s0 > 0) {
      ms = s0 + lane < ns ? a.part_m[row0 + (s0 + lane) * step] : -INFINITY;
      ls = s0 + lane < ns ? a.part_l[row0 + (s0 + lane) * step] : 0.0f;
    }
    const float w = s0 + lane < ns ? exp2f(ms - mx) : 0.0f;
    L += ls * w;
    const int nc = min(64, ns - s0);
    int j = 0;
    if (s0 == 0) {
#pragma unroll
      for (; j < kPre; ++j) {
        const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(opre[j][k], wj, acc[k]);
      }
    }
#pragma unroll 4
    for (; j < nc; ++j) {
      const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
#pragma unroll
      for (int k = 0; k < DPL; ++k)
        if (lane + 64 * k < a.d_h) acc[k] = fmaf(po[(s0 + j) * ostep + 64 * k], wj, acc[k]);
    }
  }
  L = gvad::wave_sum(L);
#pragma unroll
  for (int k = 0; k < DPL; ++k)
    if (lane + 64 * k < a.d_h) dst[lane + 64 * k] = poison ? qnan : acc[k] / L;
  if (lse && lane == 0) *lse = poison ? qnan : (mx + log2f(L)) * gvad::kLn2;
}

// ---- the decode step in one launch, vector-ALU path (small batches, short sequences) ---------
//
// One work-group of kSmallWaves waves per (sequence b, value group g) does what the append, the
// absorption and the decode of one step do for that group:
//   1. absorption: q~ of the group's NH heads, float32 multiply-adds in the order of
//      gva_absorb_query (so q_abs is bit-identical), the rows of M and q_nope staged through
//      LDS; the positional slice rotated in float64 at the token's position and rounded once;
//   2. append: the token's values for group g (and, in group 0's work-group, its rotated
//      positional key) rounded once and written as gva_cache_append writes them, and kept in
//      LDS, where the decode takes the token from (this launch is writing it to the cache);
//   3. decode: wave w takes the w-th of kSmallWaves equal ranges of positions, cut from max_len
//      so that its first block-table entries are read at the start, and runs the vector-ALU
//      decode on it: lane-per-position scores, online softmax per head, lanes over the value
//      dimensions for the weighted sum;
//   4. merge: the waves' (m, l, o) meet in LDS through their log-sum-exp; the result is the
//      output row and its lse.
// Every input that does not depend on another load is requested at the start. No work-group
// waits on another. The host takes this path when the matrix-core kernel does not serve the
// shape (float32 caches among them), with at most kPlanCUs (sequence, group) pairs, sequences
// of at most kSmallMaxLen positions and the group's rows of M within the LDS region.
constexpr int kSmallWaves = 8;
using gva::kSmallRegionBytes;

// alt where mask is all ones, else loaded: a bitwise blend, because a select between a loaded
// value and another one is compiled as a branch around the load with a wait inside, which
// would serialise the loads of a batch
__device__ __forceinline__ float blend(float loaded, float alt, int mask) {
  return __int_as_float((__float_as_int(loaded) & ~mask) | (__float_as_int(alt) & mask));
}

template <bool BF16, int NH, int DPL>
__global__ __launch_bounds__(64 * kSmallWaves) void k_step_small(gva::StepArgs s) {
  constexpr int PV = 64 / DPL;                           // positions per weighted-sum batch
  __shared__ __align__(16) float region[kSmallRegionBytes / 4];   // M and q_nope, then the merge
  __shared__ float q_s[NH][gva::kMaxDh + gva::kMaxDr];   // q~ | r, times scale log2(e)
  __shared__ float tok_v[gva::kMaxDh];                   // the token's values (group g), rounded
  __shared__ float tok_kr[gva::kMaxDr];                  // its rotated positional key, rounded
  __shared__ __align__(16) float p_s[kSmallWaves][NH][kTile];
  __shared__ int64_t vo_s[kSmallWaves][kTile];
  __shared__ int s_bad;
  const gva::DecodeArgs &a = s.a;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x / a.G;
  const int g = blockIdx.x - b * a.G;
  const int d_h = a.d_h, d_r = a.d_r, d_n = s.d_n, row = d_h + d_r;
  const int half_r = d_r >> 1;
  const int lb = a.log2_bs;
  const int bs_mask = (1 << lb) - 1;
  const float qnan = __int_as_float(0x7fc00000);
  if (tid == 0) s_bad = 0;
  // the group's heads, slots g NH .. g NH + NH - 1 of a.head_of: read as aligned 32-bit words
  // with uniform indices (scalar loads), the lane's byte shifted out, so that no load has to
  // wait for a per-lane lookup
  const int h0 = g * NH;
  const uint32_t *hw = reinterpret_cast<const uint32_t *>(a.head_of) + (h0 >> 2);
  const uint32_t hw0 = hw[0];
  const uint32_t hw1 = NH == 8 ? hw[1] : 0u;
  auto head = [&](int c) {
    return static_cast<int>((((c & 4) ? hw1 : hw0) >> (8 * ((h0 & 3) + (c & 3)))) & 0xffu);
  };
  const int32_t *__restrict__ bt = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
  // this wave's range [c0, cend) of positions, cut from max_len; the entry of position
  // min(c0 + lane, cend - 1) for its first tile is requested now
  const int chunk = (a.max_len + kSmallWaves - 1) / kSmallWaves;
  const int c0 = wave * chunk;
  const int cend = min(c0 + chunk, a.max_len);
  int32_t pe0 = 0;
  if (c0 < cend) pe0 = bt[min(c0 + lane, cend - 1) >> lb];   // uniform per wave
  const int p = s.pos[b];
  const int len = a.seq_len[b];
  const int cap = a.max_blocks << a.log2_bs;
  const bool len_bad = len < 0 || len > a.max_len || len > cap;
  const bool rope_bad = p < 0 || p >= s.max_pos;         // the absorbed query is NaN
  int32_t aerr = 0;
  if (p < 0) aerr = GVA_DEVERR_LENGTH;
  else if (p >= cap) aerr = GVA_DEVERR_CAPACITY;
  else if (p >= s.max_pos) aerr = GVA_DEVERR_ROPE;
  // the token's table entry, values and positional key pairs with their (cos, sin), and the
  // positional query pairs of the group's heads with theirs, all requested now
  const int32_t pblk = aerr ? 0 : bt[p >> lb];
  float2 tok_x = {0.f, 0.f}, tok_k = {0.f, 0.f}, rq = {0.f, 0.f};
  double2 tok_cs = {1.0, 0.0}, rq_cs = {1.0, 0.0};
  if (!aerr) {
    if (tid < (d_h >> 1))
      tok_x = reinterpret_cast<const float2 *>(s.v_new + (static_cast<int64_t>(b) * a.G + g) * d_h)[tid];
    if (tid < half_r) {
      tok_k = reinterpret_cast<const float2 *>(s.kr_raw + static_cast<int64_t>(b) * d_r)[tid];
      tok_cs = reinterpret_cast<const double2 *>(s.rope)[static_cast<int64_t>(p) * half_r + tid];
    }
  }
  if (!rope_bad && tid < NH * half_r) {                  // NH d_r / 2 <= 256 <= 64 kSmallWaves
    const int c = tid / half_r;
    const int k = tid - c * half_r;
    rq = reinterpret_cast<const float2 *>(s.q_rope + (static_cast<int64_t>(b) * a.H + head(c)) * d_r)[k];
    rq_cs = reinterpret_cast<const double2 *>(s.rope)[static_cast<int64_t>(p) * half_r + k];
  }

  // ---- 1. absorption ----
  // the q_abs values this thread forms, written after the barrier that publishes them in LDS
  // (a barrier waits for the stores before it)
  float qa_val[4] = {0.f, 0.f, 0.f, 0.f};
  float2 qr_val = {0.f, 0.f};
  {
    const int d4 = d_n >> 2;
    const int stride4 = d4 + 1;                          // rows padded by 16 bytes
    const int nrows = NH * d_h;
    float4 *mst = reinterpret_cast<float4 *>(region);
    float4 *qst = mst + nrows * stride4;                 // q_nope of the group's heads
    // Thread t stages element t % d4 of rows t / d4, t / d4 + q, ... of each head's block of M
    // (q = threads / d4 rows per pass): no division in the loops, and every load and store is
    // made (row indices are clamped; a duplicate writes the same value to the same place), so
    // the loads of a head are in flight together.
    const int q4 = (64 * kSmallWaves) / d4;
    const int my_r = tid / d4;
    const int my_j = tid - my_r * d4;
    const int nk = (d_h + q4 - 1) / q4;
#pragma unroll
    for (int c = 0; c < NH; ++c) {
      const float4 *Mc = reinterpret_cast<const float4 *>(s.M + static_cast<int64_t>(head(c)) * d_h * d_n);
      float4 *dc = mst + c * d_h * stride4;
#pragma unroll 4
      for (int k = 0; k < nk; ++k) {
        const int i = min(my_r + k * q4, d_h - 1);
        dc[i * stride4 + my_j] = Mc[i * d4 + my_j];
      }
    }
    for (int e = tid; e < NH * d4; e += 64 * kSmallWaves) {
      const int c = e / d4;
      qst[e] = reinterpret_cast<const float4 *>(
          s.q_nope + (static_cast<int64_t>(b) * a.H + head(c)) * d_n)[e - c * d4];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {                        // nrows <= 8 x 256 = 4 x 512
      const int o = tid + u * 64 * kSmallWaves;
      if (o >= nrows) break;
      const int c = o / d_h;
      const int i = o - c * d_h;
      const float4 *mr = mst + o * stride4;
      const float4 *qr = qst + c * d4;
      float acc = 0.0f;
      for (int j4 = 0; j4 < d4; ++j4) {
        const float4 m4 = mr[j4];
        const float4 q4v = qr[j4];
        acc = fmaf(m4.x, q4v.x, acc);
        acc = fmaf(m4.y, q4v.y, acc);
        acc = fmaf(m4.z, q4v.z, acc);
        acc = fmaf(m4.w, q4v.w, acc);
      }
      const float v = rope_bad ? qnan : acc;
      qa_val[u] = v;
      q_s[c][i] = v * a.qscale;
    }
    if (tid < NH * half_r) {
      const int c = tid / half_r;
      const int k = tid - c * half_r;
      float y0f = qnan, y1f = qnan;
      if (!rope_bad) {
        double y0, y1;
        gvad::rotate_pair_f64(static_cast<double>(rq.x), static_cast<double>(rq.y), rq_cs.x,
                              rq_cs.y, &y0, &y1);
        y0f = gvad::f64_to_f32(y0);
        y1f = gvad::f64_to_f32(y1);
      }
      qr_val = make_float2(y0f, y1f);
      q_s[c][d_h + 2 * k] = y0f * a.qscale;
      q_s[c][d_h + 2 * k + 1] = y1f * a.qscale;
    }
  }

  // ---- 2. append (the checks and arithmetic of gva_cache_append) ----
  int64_t blk = -1;
  if (!aerr) {
    if (pblk < 0 || static_cast<int64_t>(pblk) >= a.num_blocks) aerr = GVA_DEVERR_BLOCK;
    else blk = pblk;
  }
  const bool tok_ok = aerr == 0;
  if (g == 0 && tid == 0) {
    if (aerr) gvad::raise_err(a.err_flag, aerr);
    if (rope_bad) gvad::raise_err(a.err_flag, GVA_DEVERR_ROPE);
    if (len_bad) gvad::raise_err(a.err_flag, GVA_DEVERR_LENGTH);
  }
  // the rounded token (cache bits) this thread writes after the barrier
  uint2 wv = {0u, 0u}, wk = {0u, 0u};
  if (tok_ok) {
    if (tid < (d_h >> 1)) {                              // d_h / 2 <= 128 < 64 kSmallWaves
      if (BF16) {
        wv.x = gvad::f64_to_bf16_bits(static_cast<double>(tok_x.x));
        wv.y = gvad::f64_to_bf16_bits(static_cast<double>(tok_x.y));
        tok_v[2 * tid] = gvad::bf16_bits_to_f32(wv.x);
        tok_v[2 * tid + 1] = gvad::bf16_bits_to_f32(wv.y);
      } else {
        wv.x = gvad::f64_to_f32_bits(static_cast<double>(tok_x.x));
        wv.y = gvad::f64_to_f32_bits(static_cast<double>(tok_x.y));
        tok_v[2 * tid] = __uint_as_float(wv.x);
        tok_v[2 * tid + 1] = __uint_as_float(wv.y);
      }
    }
    if (tid < half_r) {
      double y0, y1;
      gvad::rotate_pair_f64(static_cast<double>(tok_k.x), static_cast<double>(tok_k.y), tok_cs.x,
                            tok_cs.y, &y0, &y1);
      if (BF16) {
        wk.x = gvad::f64_to_bf16_bits(y0);
        wk.y = gvad::f64_to_bf16_bits(y1);
        tok_kr[2 * tid] = gvad::bf16_bits_to_f32(wk.x);
        tok_kr[2 * tid + 1] = gvad::bf16_bits_to_f32(wk.y);
      } else {
        wk.x = gvad::f64_to_f32_bits(y0);
        wk.y = gvad::f64_to_f32_bits(y1);
        tok_kr[2 * tid] = __uint_as_float(wk.x);
        tok_kr[2 * tid + 1] = __uint_as_float(wk.y);
      }
    }
  }
  __syncthreads();                                       // q~, r and the token are in LDS

  // ---- 3. decode the wave's range [c0, c1) ----
  float m[NH], l[NH], o[NH][DPL];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.0f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[hh][k] = 0.0f;
  }
  bool bad = false;
  const int c1 = len_bad ? c0 : min(cend, len);
  for (int t0 = c0; t0 < c1; t0 += kTile) {
    // ---- scores: one position per lane; the token's position reads it from LDS ----
    // lane reads position tp = min(t0 + lane, cend - 1) (inside the table; its entry is only
    // checked, and used, for positions of the sequence)
    const int t = t0 + lane;
    const bool valid = t < c1;
    const int tp = min(t, cend - 1);
    const int32_t pe = t0 == c0 ? pe0 : bt[tp >> lb];
    const bool pe_ok = pe >= 0 && static_cast<int64_t>(pe) < a.num_blocks;
    const bool mine = tok_ok && valid && t == p;
    if (valid && !pe_ok && !mine) bad = true;
    const int mmask = mine ? -1 : 0;
    const int64_t blk_s = pe_ok ? pe : 0;
    const int64_t voff = blk_s * a.v_sb + static_cast<int64_t>(tp & bs_mask) * a.v_st +
                         static_cast<int64_t>(g) * a.v_sg;
    const int64_t koff = blk_s * a.kr_sb + static_cast<int64_t>(tp & bs_mask) * a.kr_st;
    vo_s[wave][lane] = voff;
    float sc[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) sc[hh] = 0.0f;
#pragma unroll 8
    for (int i = 0; i < d_r; i += 2) {
      const float2 y = load_pair<BF16>(a.kr, koff + i);
      const float2 x = make_float2(blend(y.x, tok_kr[i], mmask), blend(y.y, tok_kr[i + 1], mmask));
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
        sc[hh] = fmaf(q_s[hh][d_h + i], x.x, fmaf(q_s[hh][d_h + i + 1], x.y, sc[hh]));
    }
#pragma unroll 32
    for (int i = 0; i < d_h; i += 2) {
      const float2 y = load_pair<BF16>(a.v, voff + i);
      const float2 x = make_float2(blend(y.x, tok_v[i], mmask), blend(y.y, tok_v[i + 1], mmask));
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) sc[hh] = fmaf(q_s[hh][i], x.x, fmaf(q_s[hh][i + 1], x.y, sc[hh]));
    }
    // ---- online softmax over the tile, per head ----
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const float sv = valid ? sc[hh] : -INFINITY;
      const float mn = fmaxf(m[hh], gvad::wave_max(sv));
      const float alpha = exp2f(m[hh] - mn);
      const float pr = exp2f(sv - mn);
      l[hh] = l[hh] * alpha + gvad::wave_sum(pr);
      m[hh] = mn;
      p_s[wave][hh][lane] = pr;
#pragma unroll
      for (int k = 0; k < DPL; ++k) o[hh][k] *= alpha;
    }
    // ---- weighted sum: lanes over value dimensions (the wave's own LDS rows: no barrier) ----
    // every load is issued (positions past the tile's end read a row of the range again, dims
    // past d_h its last element; neither is used); the token's row comes from LDS
    const int nt = min(kTile, c1 - t0);
    const int tokj = tok_ok && p >= t0 && p < t0 + nt ? p - t0 : -1;
    float tokd[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) tokd[k] = tok_v[min(lane + 64 * k, d_h - 1)];
    for (int j0 = 0; j0 < nt; j0 += PV) {
      float x[PV][DPL];
#pragma unroll
      for (int u = 0; u < PV; ++u) {
        const int64_t vo = vo_s[wave][j0 + u];
        const int tmask = j0 + u == tokj ? -1 : 0;
        const int vmask = j0 + u < nt ? -1 : 0;         // rows past nt may hold anything
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
          const float xv = blend(load_one<BF16>(a.v, vo + min(lane + 64 * k, d_h - 1)), tokd[k], tmask);
          x[u][k] = __int_as_float(__float_as_int(xv) & vmask);
        }
      }
      // positions past nt have zero values and zero probabilities (scores of -inf), so every
      // product is taken; four positions' probabilities per 16-byte LDS read
#pragma unroll
      for (int u4 = 0; u4 < PV / 4; ++u4) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          const float4 pj = *reinterpret_cast<const float4 *>(&p_s[wave][hh][j0 + 4 * u4]);
#pragma unroll
          for (int k = 0; k < DPL; ++k) {
            o[hh][k] = fmaf(pj.x, x[4 * u4][k], o[hh][k]);
            o[hh][k] = fmaf(pj.y, x[4 * u4 + 1][k], o[hh][k]);
            o[hh][k] = fmaf(pj.z, x[4 * u4 + 2][k], o[hh][k]);
            o[hh][k] = fmaf(pj.w, x[4 * u4 + 3][k], o[hh][k]);
          }
        }
      }
    }
  }
  if (__any(bad) && lane == 0) {
    atomicOr(&s_bad, 1);
    gvad::raise_err(a.err_flag, GVA_DEVERR_BLOCK);
  }

  // ---- 4. merge the waves' (m, l, o) in LDS (the region's M rows are no longer read) ----
  float *mo = region;                                    // [kSmallWaves][NH][d_h]
  float *mm = mo + kSmallWaves * NH * d_h;               // [kSmallWaves][NH]
  float *ml = mm + kSmallWaves * NH;                     // [kSmallWaves][NH]
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int d = lane + 64 * k;
      if (d < d_h) mo[(wave * NH + hh) * d_h + d] = o[hh][k];
    }
    if (lane == 0) {
      mm[wave * NH + hh] = m[hh];
      ml[wave * NH + hh] = l[hh];
    }
  }
  __syncthreads();
  // the global writes of the absorption and the append, which nothing in this launch reads
  // back (the decode took q~, r and the token from LDS): q_abs, and the token into the cache as
  // gva_cache_append writes it. They go out last, beside the output rows: before a barrier
  // they would be waited for there, and before the decode's loads they would be waited for
  // with them (stores and loads are counted in order).
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int o = tid + u * 64 * kSmallWaves;
    if (o >= NH * d_h) break;
    const int c = o / d_h;
    s.q_abs[(static_cast<int64_t>(b) * a.H + head(c)) * row + (o - c * d_h)] = qa_val[u];
  }
  if (tid < NH * half_r) {
    const int c = tid / half_r;
    const int k = tid - c * half_r;
    *reinterpret_cast<float2 *>(s.q_abs + (static_cast<int64_t>(b) * a.H + head(c)) * row + d_h + 2 * k) =
        qr_val;
  }
  if (tok_ok) {
    const int64_t off = p & bs_mask;
    if (tid < (d_h >> 1)) {
      const int64_t o = blk * a.v_sb + off * a.v_st + static_cast<int64_t>(g) * a.v_sg + 2 * tid;
      if (BF16) reinterpret_cast<uint32_t *>(const_cast<void *>(a.v))[o >> 1] = wv.x | (wv.y << 16);
      else *reinterpret_cast<uint2 *>(reinterpret_cast<uint32_t *>(const_cast<void *>(a.v)) + o) = wv;
    }
    if (g == 0 && tid < half_r) {
      const int64_t o = blk * a.kr_sb + off * a.kr_st + 2 * tid;
      if (BF16) reinterpret_cast<uint32_t *>(const_cast<void *>(a.kr))[o >> 1] = wk.x | (wk.y << 16);
      else *reinterpret_cast<uint2 *>(reinterpret_cast<uint32_t *>(const_cast<void *>(a.kr)) + o) = wk;
    }
  }
  const bool poison = len_bad || s_bad != 0;
  for (int idx = tid; idx < NH * d_h; idx += 64 * kSmallWaves) {
    const int hh = idx / d_h;
    const int d = idx - hh * d_h;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) mx = fmaxf(mx, mm[w * NH + hh]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) {
      const float mw = mm[w * NH + hh];
      const float e = mw == -INFINITY ? 0.0f : exp2f(mw - mx);
      L = fmaf(ml[w * NH + hh], e, L);
      acc = fmaf(mo[(w * NH + hh) * d_h + d], e, acc);
    }
    const int h = head(hh);
    a.out[(static_cast<int64_t>(b) * a.H + h) * d_h + d] = poison ? qnan : (L > 0.0f ? acc / L : 0.0f);
    if (a.lse && d == 0)
      a.lse[static_cast<int64_t>(b) * a.H + h] =
          poison ? qnan : (L > 0.0f ? (mx + log2f(L)) * gvad::kLn2 : -INFINITY);
  }
}

}  // namespace

namespace gva {

template <bool BF16, int DPL>
void launch_generic_nhp(const DecodeArgs &a, dim3 grid, int head_passes, int nhp,
                        hipStream_t stream) {
  switch (nhp) {
    case 1: hipLaunchKernelGGL((k_decode_generic<BF16, DPL, 1>), grid, dim3(64), 0, stream, a, head_passes); break;
    case 2: hipLaunchKernelGGL((k_decode_generic<BF16, DPL, 2>), grid, dim3(64), 0, stream, a, head_passes); break;
    case 4: hipLaunchKernelGGL((k_decode_generic<BF16, DPL, 4>), grid, dim3(64), 0, stream, a, head_passes); break;
    case 8: hipLaunchKernelGGL((k_decode_generic<BF16, DPL, 8>), grid, dim3(64), 0, stream, a, head_passes); break;
    default: hipLaunchKernelGGL((k_decode_generic<BF16, DPL, 16>), grid, dim3(64), 0, stream, a, head_passes); break;
  }
}

template <bool BF16>
void launch_generic_dpl(const DecodeArgs &a, dim3 grid, int head_passes, int nhp,
                        hipStream_t stream) {
  switch ((a.d_h + 63) / 64) {
    case 1: launch_generic_nhp<BF16, 1>(a, grid, head_passes, nhp, stream); break;
    case 2: launch_generic_nhp<BF16, 2>(a, grid, head_passes, nhp, stream); break;
    case 3: launch_generic_nhp<BF16, 3>(a, grid, head_passes, nhp, stream); break;
    default: launch_generic_nhp<BF16, 4>(a, grid, head_passes, nhp, stream); break;
  }
}

hipError_t launch_decode_generic(const DecodeArgs &a, bool bf16, hipStream_t stream) {
  const int hpg = a.H / a.G;
  const int head_passes = (hpg + kHeadsPerPass - 1) / kHeadsPerPass;
  const dim3 grid(a.num_splits, a.B, a.G * head_passes);
  const int nh_max = hpg < kHeadsPerPass ? hpg : kHeadsPerPass;
  int nhp = 1;
  while (nhp < nh_max) nhp <<= 1;
  if (bf16) launch_generic_dpl<true>(a, grid, head_passes, nhp, stream);
  else launch_generic_dpl<false>(a, grid, head_passes, nhp, stream);
  return hipGetLastError();
}

template <bool BF16, int NH>
hipError_t launch_small_dpl(const StepArgs &sa, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(sa.a.B * sa.a.G));
  const dim3 block(64 * kSmallWaves);
  switch ((sa.a.d_h + 63) / 64) {
    case 1: hipLaunchKernelGGL((k_step_small<BF16, NH, 1>), grid, block, 0, stream, sa); break;
    case 2: hipLaunchKernelGGL((k_step_small<BF16, NH, 2>), grid, block, 0, stream, sa); break;
    case 3: hipLaunchKernelGGL((k_step_small<BF16, NH, 3>), grid, block, 0, stream, sa); break;
    default: hipLaunchKernelGGL((k_step_small<BF16, NH, 4>), grid, block, 0, stream, sa); break;
  }
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_small_nh(const StepArgs &sa, hipStream_t stream) {
  switch (sa.a.H / sa.a.G) {
    case 1: return launch_small_dpl<BF16, 1>(sa, stream);
    case 2: return launch_small_dpl<BF16, 2>(sa, stream);
    case 4: return launch_small_dpl<BF16, 4>(sa, stream);
    case 8: return launch_small_dpl<BF16, 8>(sa, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_step_small(const StepArgs &sa, bool bf16, hipStream_t stream) {
  return bf16 ? launch_small_nh<true>(sa, stream) : launch_small_nh<false>(sa, stream);
}

hipError_t launch_combine(const DecodeArgs &a, hipStream_t stream) {
  // waves grow with the partials per sequence (balanced mode: about R / B + 1 of them); with
  // few of them, one wave per (sequence, head)
  const int per_seq = a.num_ranges > 0 ? a.num_ranges / a.B + 1 : a.num_splits;
  if (per_seq <= kCombineWaveRows && a.d_h <= 256) {   // the one-wave combine holds 256 dims
    const dim3 grid((a.H + 3) / 4, a.B);
    switch ((a.d_h + 63) / 64) {
      case 1: hipLaunchKernelGGL(k_combine_wave<1>, grid, dim3(256), 0, stream, a); break;
      case 2: hipLaunchKernelGGL(k_combine_wave<2>, grid, dim3(256), 0, stream, a); break;
      case 3: hipLaunchKernelGGL(k_combine_wave<3>, grid, dim3(256), 0, stream, a); break;
      default: hipLaunchKernelGGL(k_combine_wave<4>, grid, dim3(256), 0, stream, a); break;
    }
    return hipGetLastError();
  }
  if (a.num_ranges == 0 && a.B == 1 && a.num_splits <= 8 * kCombineSliceMaxK && a.d_h % 32 == 0) {
    const dim3 grid(a.d_h / 32, a.H, 1);
    const int k = (a.num_splits + 7) / 8;
    if (k <= 4) hipLaunchKernelGGL(k_combine_slice<4>, grid, dim3(64), 0, stream, a);
    else if (k <= 8) hipLaunchKernelGGL(k_combine_slice<8>, grid, dim3(64), 0, stream, a);
    else if (k <= 16) hipLaunchKernelGGL(k_combine_slice<16>, grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL(k_combine_slice<32>, grid, dim3(64), 0, stream, a);
    return hipGetLastError();
  }
  int nw = per_seq / 16;
  nw = nw < 1 ? 1 : (nw > kCombineMaxWaves ? kCombineMaxWaves : nw);
  hipLaunchKernelGGL(k_combine, dim3((a.d_h + 63) / 64, a.H, a.B), dim3(64 * nw), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gva
