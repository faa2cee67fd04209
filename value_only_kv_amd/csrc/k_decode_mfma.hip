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
// Write n = lane % 16 and q = lane / 16.
//
// One wave per (chunk, sequence, group); a work-group holds several groups of the same chunk,
// so their reads of the shared positional key hit in cache. A chunk is walked in tiles of 32
// positions, two blocks of 16 (tb = 0, 1):
//   1. V rows go straight from HBM into registers in A-operand form: lane (n, q) loads 16 bytes,
//      8 consecutive dims 32 ks + 8 q .. of position 16 tb + n, for every k-step ks.
//   2. Scores S^T[t][h] = sum_k V[t][k] Q[h][k] (B = the absorbed query, one column per head).
//      The query is split into bf16 hi + lo parts, two MFMAs, so it keeps ~16 mantissa bits.
//      Lane (n, q) then holds head n's scores of positions 16 tb + 4 q + r, r = 0..3.
//   3. Online softmax per head in the base-2 domain; the tile max needs two lane exchanges.
//   4. The weighted sum O^T[d][h] = sum_t V[t][d] P[h][t] contracts over positions, so V is
//      needed with positions along K. The matrix core transposes the registers it already has:
//      V x E, with E a 0/1 selection matrix, returns V[t][d] in D layout (lane (n, q) gets
//      positions 4 q + r of dim n), exactly, since each output is one product by 1.0. Packing
//      the two position blocks gives the A operand with K order (q, e) -> 16 (e / 4) + 4 q + e % 4,
//      which is exactly the order in which each lane already holds its probabilities, so the
//      B operand (P, hi + lo parts) is built from the lane's own registers.
//   5. O^T accumulates in registers: lane (n, q) holds head n, dims 16 nb + 4 q + r.
#include <hip/hip_runtime.h>

#include <math.h>

#include "gva_device.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kTile = 32;

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

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): ~16 significant bits in two bf16 operands.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned w = pack2(x[2 * i], x[2 * i + 1]);
    h[i] = w;
    l[i] = pack2(x[2 * i] - low_bf16(w), x[2 * i + 1] - high_bf16(w));
  }
  hi = as_bf16(h);
  lo = as_bf16(l);
}

template <int KS>
struct Tile {
  u32x4 v[2][KS];   // V rows in A-operand form, per position block and k-step
  u32x4 kr[2];      // positional key rows in A-operand form (zero where 8 q >= d_r)
};

// Loads the 32 positions starting at t0 (positions >= c1 read position c1 - 1 instead; their
// scores are masked). Sets *bad when a block-table entry is outside the pool.
template <int KS>
__device__ __forceinline__ void load_tile(const gva::DecodeArgs &a, int b, int g, int t0, int c1,
                                          int n, int q, Tile<KS> &T, bool &bad) {
  const int mask = (1 << a.log2_bs) - 1;
  const uint16_t *vbase = static_cast<const uint16_t *>(a.v);
  const uint16_t *kbase = static_cast<const uint16_t *>(a.kr);
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = t0 + 16 * tb + n;
    const int tc = t < c1 ? t : c1 - 1;
    const int32_t pb = a.block_table[static_cast<int64_t>(b) * a.max_blocks + (tc >> a.log2_bs)];
    const bool ok = pb >= 0 && static_cast<int64_t>(pb) < a.num_blocks;
    bad |= !ok;
    const int64_t blk = ok ? pb : 0;
    const int64_t off = static_cast<int64_t>(tc & mask);
    const uint16_t *vp = vbase + blk * a.v_sb + off * a.v_st + static_cast<int64_t>(g) * a.v_sg + 8 * q;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) T.v[tb][ks] = *reinterpret_cast<const u32x4 *>(vp + 32 * ks);
    if (8 * q < a.d_r) {
      T.kr[tb] = *reinterpret_cast<const u32x4 *>(kbase + blk * a.kr_sb + off * a.kr_st + 8 * q);
    } else {
      T.kr[tb] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int KS>
__global__ __launch_bounds__(512) void k_decode_mfma(gva::DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int q = lane >> 4;
  const int s = blockIdx.x;
  const int b = blockIdx.y;
  const int g = blockIdx.z * (blockDim.x >> 6) + wave;
  const int nhg = a.H / a.G;
  const int h0 = g * nhg;
  const bool head_ok = n < nhg;
  const int row = a.d_h + a.d_r;
  const float qnan = __int_as_float(0x7fc00000);

  const int len = a.seq_len[b];
  const int cap = a.max_blocks << a.log2_bs;
  const bool len_bad = len < 0 || len > a.max_len || len > cap;
  const int c0 = s * a.chunk;
  const int c1 = len_bad ? c0 : min(c0 + a.chunk, len);

  f32x4 O[2 * KS];
#pragma unroll
  for (int i = 0; i < 2 * KS; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.0f;
  bool bad = false;

  if (c0 < c1) {
    // ---- query operands (B layout: column n = head, K group q) ----
    bf16x8 QH[KS], QL[KS], RH, RL, SEL[2];
    const float *qp = a.q_abs + (static_cast<int64_t>(b) * a.H + h0 + n) * row;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = head_ok ? qp[32 * ks + 8 * q + e] * a.qscale : 0.0f;
      split8(x, QH[ks], QL[ks]);
    }
    {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * q + e;
        x[e] = (head_ok && i < a.d_r) ? qp[a.d_h + i] * a.qscale : 0.0f;
      }
      split8(x, RH, RL);
    }
    // selection matrices E_half[k][j] = 1 if k == 16 half + j (B layout)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned lo = (8 * q + 2 * i == 16 * half + n) ? 0x3f80u : 0u;
        const unsigned hi = (8 * q + 2 * i + 1 == 16 * half + n) ? 0x3f80u : 0u;
        w[i] = lo | (hi << 16);
      }
      SEL[half] = as_bf16(w);
    }

    Tile<KS> cur;
    load_tile<KS>(a, b, g, c0, c1, n, q, cur, bad);
    for (int t0 = c0; t0 < c1; t0 += kTile) {
      const bool more = t0 + kTile < c1;
      Tile<KS> nxt;
      if (more) load_tile<KS>(a, b, g, t0 + kTile, c1, n, q, nxt, bad);

      // ---- scores ----
      f32x4 S[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          acc = mfma(as_bf16(cur.v[tb][ks]), QH[ks], acc);
          acc = mfma(as_bf16(cur.v[tb][ks]), QL[ks], acc);
        }
        acc = mfma(as_bf16(cur.kr[tb]), RH, acc);
        acc = mfma(as_bf16(cur.kr[tb]), RL, acc);
        S[tb] = acc;
      }
      // ---- online softmax (head n; positions t0 + 16 tb + 4 q + r) ----
      float mt = -INFINITY;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (t0 + 16 * tb + 4 * q + r >= c1) S[tb][r] = -INFINITY;
          mt = fmaxf(mt, S[tb][r]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mn = fmaxf(m, mt);
      const float alpha = exp2f(m - mn);
      float p[8];
      float ps = 0.0f;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[4 * tb + r] = exp2f(S[tb][r] - mn);
          ps += p[4 * tb + r];
        }
      lsum = lsum * alpha + ps;
      m = mn;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) O[i] *= alpha;
      }
      bf16x8 PH, PL;
      split8(p, PH, PL);
      // ---- weighted sum: transpose V by the matrix core, then O^T += V^T P^T ----
#pragma unroll
      for (int nb = 0; nb < 2 * KS; ++nb) {
        const int ks = nb >> 1;
        const int half = nb & 1;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 T0 = mfma(as_bf16(cur.v[0][ks]), SEL[half], z);
        const f32x4 T1 = mfma(as_bf16(cur.v[1][ks]), SEL[half], z);
        u32x4 w;
        w[0] = pack2(T0[0], T0[1]);
        w[1] = pack2(T0[2], T0[3]);
        w[2] = pack2(T1[0], T1[1]);
        w[3] = pack2(T1[2], T1[3]);
        const bf16x8 VT = as_bf16(w);
        O[nb] = mfma(VT, PH, O[nb]);
        O[nb] = mfma(VT, PL, O[nb]);
      }
      if (more) cur = nxt;
    }
  }

  // ---- epilogue: head n's row; dims 16 nb + 4 q + r ----
  float ltot = lsum + __shfl_xor(lsum, 16, 64);
  ltot += __shfl_xor(ltot, 32, 64);
  const bool any_bad = __any(bad);
  if (lane == 0) {
    if (any_bad) gvad::raise_err(a.err_flag, GVA_DEVERR_BLOCK);
    if (len_bad && s == 0 && g == 0) gvad::raise_err(a.err_flag, GVA_DEVERR_LENGTH);
  }
  const bool poison = any_bad || len_bad;
  if (!head_ok) return;
  const int h = h0 + n;
  if (a.num_splits == 1) {
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    float *dst = a.out + (static_cast<int64_t>(b) * a.H + h) * a.d_h + 4 * q;
#pragma unroll
    for (int nb = 0; nb < 2 * KS; ++nb) {
      f32x4 v = O[nb] * inv;
      if (poison) v = f32x4{qnan, qnan, qnan, qnan};
      *reinterpret_cast<f32x4 *>(dst + 16 * nb) = v;
    }
    if (a.lse && q == 0) {
      const float v = ltot > 0.0f ? (m + log2f(ltot)) * gvad::kLn2 : -INFINITY;
      a.lse[static_cast<int64_t>(b) * a.H + h] = poison ? qnan : v;
    }
  } else {
    const int64_t prow = (static_cast<int64_t>(b) * a.num_splits + s) * a.H + h;
    float *dst = a.part_o + prow * a.d_h + 4 * q;
#pragma unroll
    for (int nb = 0; nb < 2 * KS; ++nb) *reinterpret_cast<f32x4 *>(dst + 16 * nb) = O[nb];
    if (q == 0) {
      a.part_m[prow] = poison ? qnan : m;
      a.part_l[prow] = ltot;
    }
  }
}

}  // namespace

namespace gva {

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t stream) {
  // waves per work-group: the largest divisor of G that is at most 8
  int wpg = 1;
  for (int w = 8; w >= 1; --w)
    if (a.G % w == 0) {
      wpg = w;
      break;
    }
  const dim3 grid(a.num_splits, a.B, a.G / wpg);
  const dim3 block(64 * wpg);
  switch (a.d_h / 32) {
    case 1: hipLaunchKernelGGL(k_decode_mfma<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(k_decode_mfma<2>, grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL(k_decode_mfma<3>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(k_decode_mfma<4>, grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL(k_decode_mfma<5>, grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL(k_decode_mfma<6>, grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL(k_decode_mfma<7>, grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(k_decode_mfma<8>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gva
