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
    const int h = h0 + hh;
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
  const int h0 = g * hpg + hp * kHeadsPerPass;
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
    q_s[hh][e] = hh < nh ? a.q_abs[(static_cast<int64_t>(b) * a.H + h0 + hh) * row + e] * a.qscale
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
  const int len = a.seq_len[b];
  const int cap = a.max_blocks << a.log2_bs;
  if (len < 0 || len > a.max_len || len > cap) {
    if (wave == 0 && dim_ok) dst[d] = qnan;
    if (write_lse) a.lse[static_cast<int64_t>(b) * a.H + h] = qnan;
    if (a.num_ranges > 0 && tid == 0 && blockIdx.x == 0 && h == 0)
      gvad::raise_err(a.err_flag, GVA_DEVERR_LENGTH);
    return;
  }
  int ns;
  int64_t row0;
  partial_rows(a, b, h, len, ns, row0);
  if (ns == 0) {
    if (wave == 0 && dim_ok) dst[d] = 0.0f;
    if (write_lse) a.lse[static_cast<int64_t>(b) * a.H + h] = -INFINITY;
    return;
  }
  float mx = -INFINITY;
  float bad = 0.0f;
  for (int s = tid; s < ns; s += nthr) {
    const float ms = a.part_m[row0 + static_cast<int64_t>(s) * a.H];
    bad += isnan(ms) ? 1.0f : 0.0f;
    mx = fmaxf(mx, ms);
    w_s[s] = ms;
  }
  mx = block_reduce(mx, scratch, nw, true);
  const bool poison = block_reduce(bad, scratch, nw, false) > 0.0f;
  float L = 0.0f;
  for (int s = tid; s < ns; s += nthr) {
    const float f = exp2f(w_s[s] - mx);
    w_s[s] = f;
    L += a.part_l[row0 + static_cast<int64_t>(s) * a.H] * f;
  }
  L = block_reduce(L, scratch, nw, false);
  if (nw == 1) __syncthreads();  // the w_s writes of other lanes must be visible
  float acc = 0.0f;
  if (dim_ok) {
    const float *po = a.part_o + row0 * a.d_h + d;
    const int64_t step = static_cast<int64_t>(a.H) * a.d_h;
#pragma unroll 8
    for (int s = wave; s < ns; s += nw) acc = fmaf(po[s * step], w_s[s], acc);
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
  int nw = per_seq / 16;
  nw = nw < 1 ? 1 : (nw > kCombineMaxWaves ? kCombineMaxWaves : nw);
  hipLaunchKernelGGL(k_combine, dim3((a.d_h + 63) / 64, a.H, a.B), dim3(64 * nw), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gva
