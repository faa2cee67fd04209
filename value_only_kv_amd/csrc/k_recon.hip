// k_recon.hip - decode of the non-absorbable comparator on matrix cores (gfx950).
//
// The scale-matched GVA row rotates the reconstructed content key with ordinary RoPE, so its map
// cannot be folded into the query (agihunt.info summary of arXiv:2609.13285, the scale-matched +
// query RMSNorm row; "GVA：KV 缓存里的 Key 其实可以不存", shibing624.github.io review, section
// 第二次尝试: K_h = V_g M_h). Every decode step therefore rebuilds each head's keys from the
// cached values and rotates them at their own positions:
//   k_{h,j} = R_j (M_h^T v_j),   s_j = scale (R_p q_h) . k_{h,j},   o_h = sum_j softmax_j(s) v_j.
// That per-token d_h x d_n product per head is the cost absorption avoids.
//
// Work-group: one (sequence, chunk, group), two waves per head of the group (H / G <= 4, two
// waves per SIMD), with the group's maps M_h^T resident in LDS for the whole chunk. Keys are
// walked in steps of two tiles of 32 positions, one tile for each half of the waves:
//   * a step's value rows are staged once in LDS (the next step's rows are loaded from HBM into
//     registers while the current one is computed; one barrier per tile);
//   * each wave rebuilds its head's keys, K^T[dim][key] = M_h^T V^T, on
//     v_mfma_f32_16x16x32_bf16 (A = M_h^T from LDS, B = the value rows; both operands are exact
//     bf16 and the products accumulate in float32);
//   * the rotation is split as R_j = R_{j0} R_delta (j0 the tile's first position, delta < 32),
//     so s_j = (R_{p - j0} q) . (R_delta k_j): the lane that holds key delta of a tile knows delta,
//     and the cos/sin of delta * theta_i for its pairs stay in registers for the whole chunk,
//     while the query is rotated once per tile by p - j0 (one table row per tile, staged in LDS
//     as float32);
//   * the score is summed in float32 on the vector ALU over the lane's dims and then over the
//     four lanes that hold one key; the softmax (base 2) and the weighted sum follow: the lane's
//     two probabilities (keys delta and delta + 16) as a bf16 pair against the same dim of both
//     value rows (v_dot2_f32_bf16, float32 accumulation, the value registers of the rebuild),
//     into per-lane partial sums that are reduced at the end of the chunk.
// At the end of the chunk the two waves of a head merge their (m, l, o) through LDS. Partials go
// to the split-grid rows the decode combine reads; a single chunk per sequence writes the output
// directly.
#include <hip/hip_runtime.h>

#include <math.h>

#include "gva_device.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) double f64x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int kTile = 32;

__device__ __forceinline__ f32x4 mfma(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Reductions over the 16 lanes of a row by row rotation (DPP row_ror); every lane of the row
// ends with the result.
template <int K>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + K, 0xf, 0xf,
                                                    false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  return fmaxf(v, row_ror<1>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  return v + row_ror<1>(v);
}

// (x, y) rounded to bf16 (nearest-even) and packed, x in the low half
__device__ __forceinline__ unsigned pack2(float x, float y) {
  const f32x2 v = {x, y};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}
// a.lo * b.lo + a.hi * b.hi + c for bf16 pairs, accumulated in float32
__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

template <int DH, int DN, int NH>
__global__ __launch_bounds__(128 * NH) void k_recon_decode(gva::ReconArgs r) {
  constexpr int KSTEPS = DH / 32;          // k-steps of the key rebuild
  constexpr int NB = DN / 16;              // 16-dim blocks of a key
  constexpr int kStride = DH + 8;          // LDS row (M^T row, value row) in elements: 16 B pad
  constexpr int kStep = 2 * kTile;         // positions staged per step: one tile per half
  constexpr int kUnits = kStep * DH / 8;   // 16-byte pieces of a step's value rows
  constexpr int kThreads = 128 * NH;
  constexpr int kPer = (kUnits + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t m_lds[NH * DN * kStride];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kStep * kStride];
  __shared__ __attribute__((aligned(16))) float cs_lds[2][DN];   // (cos, sin) of DN / 2 pairs
  __shared__ int bad_lds;

  const gva::DecodeArgs &a = r.kv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = wave / NH;              // which tile of each step this wave takes
  const int hw = wave - half * NH;         // head within the group
  const int n = lane & 15;
  const int kq = lane >> 4;
  const int S = a.num_splits;
  // work-group -> (group fastest, then chunk, then sequence): with G = 8 the work-groups of a
  // group share one XCD, and its maps stay in that XCD's L2
  int id = blockIdx.x;
  const int g = id % a.G;
  id /= a.G;
  const int s = id % S;
  const int b = id / S;
  const int h = a.head_of[g * NH + hw];
  const int len = a.seq_len[b];
  const int p = r.q_pos[b];
  const int cap = a.max_blocks << a.log2_bs;
  const float qnan = __int_as_float(0x7fc00000);
  const int64_t orow = static_cast<int64_t>(b) * a.H + h;
  const int64_t prow = (static_cast<int64_t>(b) * S + s) * a.H + h;
  int err = 0;
  if (len < 0 || len > a.max_len) err = GVA_DEVERR_LENGTH;
  else if (len > cap) err = GVA_DEVERR_CAPACITY;
  else if (p < 0 || p >= r.max_pos || len > r.max_pos) err = GVA_DEVERR_ROPE;
  const int c0 = s * a.chunk;
  if (err) {                                           // uniform per work-group
    if (threadIdx.x == 0 && s == 0 && g == 0) gvad::raise_err(a.err_flag, err);
    if (half == 0 && S == 1) {
      for (int d = lane; d < DH; d += 64) a.out[orow * DH + d] = qnan;
      if (a.lse && lane == 0) a.lse[orow] = qnan;
    } else if (half == 0 && err == GVA_DEVERR_ROPE && c0 < len && lane == 0) {
      a.part_m[prow] = qnan;                           // the combine reads this chunk
    }
    return;
  }
  if (c0 >= len) {                                     // uniform per work-group
    if (half == 0 && S == 1) {                         // len == 0
      for (int d = lane; d < DH; d += 64) a.out[orow * DH + d] = 0.0f;
      if (a.lse && lane == 0) a.lse[orow] = -INFINITY;
    }
    return;                                            // past the end: the combine skips it
  }
  const int c1 = min(len, c0 + a.chunk);

  // the maps of the group's heads: LDS row (head, k) = Mt[a.head_of[g NH + head]][k][0 .. DH)
  {
    for (int c = threadIdx.x; c < NH * DN * (DH / 8); c += kThreads) {
      const int row = c / (DH / 8);
      const int col = (c - row * (DH / 8)) * 8;
      const int hh = row / DN;
      const uint16_t *msrc =
          r.Mt + (static_cast<int64_t>(a.head_of[g * NH + hh]) * DN + (row - hh * DN)) * DH;
      *reinterpret_cast<u32x4 *>(m_lds + row * kStride + col) =
          *reinterpret_cast<const u32x4 *>(msrc + col);
    }
  }
  if (threadIdx.x == 0) bad_lds = 0;

  // the query of head h: lane (n, kq) keeps dims 16 nb + 4 kq + e, the key dims it rebuilds
  float qv[NB][4];
  {
    const float *qp = r.q + orow * DN;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const f32x4 t = *reinterpret_cast<const f32x4 *>(qp + 16 * nb + 4 * kq);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[nb][e] = t[e];
    }
  }
  // cos / sin of delta * theta_i for the lane's keys delta = 16 tb + n and pairs 8 nb + 2 kq + u
  float rc[2][NB][2], rsn[2][NB][2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f64x2 t = *reinterpret_cast<const f64x2 *>(
            r.rope + (static_cast<int64_t>(16 * tb + n) * (DN / 2) + 8 * nb + 2 * kq + u) * 2);
        rc[tb][nb][u] = static_cast<float>(t[0]);
        rsn[tb][nb][u] = static_cast<float>(t[1]);
      }

  // staging of one step (two tiles, 64 positions from j0): value rows (keys past the chunk
  // repeat its last key) and, for each tile, the angle row of p - its first position (a
  // negative offset uses the row of its magnitude with the sine negated)
  const int32_t *bt = a.block_table + static_cast<int64_t>(b) * a.max_blocks;
  const int pos_mask = (1 << a.log2_bs) - 1;
  const uint16_t *vbase = static_cast<const uint16_t *>(a.v) + static_cast<int64_t>(g) * a.v_sg;
  u32x4 stv[kPer];
  f64x2 sta = {0.0, 0.0};
  bool bad = false;
  auto load_step = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int unit = threadIdx.x + kThreads * i;
      if (kUnits % kThreads == 0 || unit < kUnits) {
        const int key = unit / (DH / 8);
        const int col = (unit - key * (DH / 8)) * 8;
        const int j = min(j0 + key, c1 - 1);
        const int32_t blk = bt[j >> a.log2_bs];
        const bool ok = blk >= 0 && static_cast<int64_t>(blk) < a.num_blocks;
        bad = bad || !ok;
        const int64_t off = (ok ? static_cast<int64_t>(blk) : 0) * a.v_sb +
                            static_cast<int64_t>(j & pos_mask) * a.v_st + col;
        stv[i] = *reinterpret_cast<const u32x4 *>(vbase + off);
      }
    }
    if (threadIdx.x < DN) {                          // thread t: tile t / (DN/2), pair t % (DN/2)
      const int d = p - j0 - kTile * (threadIdx.x / (DN / 2));
      // inside the table for every tile that exists (|d| < len <= max_pos); the clamp only
      // keeps the unused row of a missing second tile in bounds
      const int row = min(d < 0 ? -d : d, r.max_pos - 1);
      sta = *reinterpret_cast<const f64x2 *>(
          r.rope + (static_cast<int64_t>(row) * (DN / 2) + threadIdx.x % (DN / 2)) * 2);
      if (d < 0) sta[1] = -sta[1];
    }
  };
  auto store_step = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int unit = threadIdx.x + kThreads * i;
      if (kUnits % kThreads == 0 || unit < kUnits) {
        const int key = unit / (DH / 8);
        const int col = (unit - key * (DH / 8)) * 8;
        *reinterpret_cast<u32x4 *>(&v_lds[key * kStride + col]) = stv[i];
      }
    }
    if (threadIdx.x < DN) {
      float *dst = cs_lds[threadIdx.x / (DN / 2)] + 2 * (threadIdx.x % (DN / 2));
      dst[0] = static_cast<float>(sta[0]);
      dst[1] = static_cast<float>(sta[1]);
    }
  };

  float m_run = -INFINITY, l_part = 0.0f;
  float o_part[KSTEPS][8];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) o_part[ks][e] = 0.0f;
  const uint16_t *mh = m_lds + hw * DN * kStride;

  // This wave's tile of the step (first position j0): rebuild the keys, rotate, score, softmax,
  // weighted sum.
  auto compute = [&](int j0) __attribute__((always_inline)) {
    const uint16_t *vt = v_lds + half * kTile * kStride;
    const float *cs = cs_lds[half];
    // B operands: lane (n, kq) holds key 16 tb + n, dims 32 ks + 8 kq .. + 8
    u32x4 vb[2][KSTEPS];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        vb[tb][ks] = *reinterpret_cast<const u32x4 *>(vt + (16 * tb + n) * kStride + 32 * ks + 8 * kq);
    // (cos, sin) of (p - j0) theta for the lane's pairs 8 nb + 2 kq and + 1
    f32x4 c4[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) c4[nb] = *reinterpret_cast<const f32x4 *>(cs + 2 * (8 * nb + 2 * kq));
    // A operands (M_h^T rows) of one 16-dim block, read one block ahead of its products
    u32x4 am[2][KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      am[0][ks] = *reinterpret_cast<const u32x4 *>(mh + n * kStride + 32 * ks + 8 * kq);
    float sp[2] = {0.0f, 0.0f};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (nb + 1 < NB) {
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
          am[(nb + 1) & 1][ks] = *reinterpret_cast<const u32x4 *>(
              mh + (16 * (nb + 1) + n) * kStride + 32 * ks + 8 * kq);
      }
      // K^T[16 nb + i][key] for both key blocks: lane (n, kq) gets dims 16 nb + 4 kq + 0..3
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        acc[0] = mfma(am[nb & 1][ks], vb[0][ks], acc[0]);
        acc[1] = mfma(am[nb & 1][ks], vb[1][ks], acc[1]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float c0 = c4[nb][2 * u], s0 = c4[nb][2 * u + 1];
        const float x0 = qv[nb][2 * u], x1 = qv[nb][2 * u + 1];
        const float q0 = c0 * x0 - s0 * x1;            // R_{p - j0} q
        const float q1 = s0 * x0 + c0 * x1;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          // q . R_delta k = cos (q0 k0 + q1 k1) + sin (q1 k0 - q0 k1)
          const float k0 = acc[tb][2 * u], k1 = acc[tb][2 * u + 1];
          const float dot = fmaf(k1, q1, k0 * q0);
          const float crs = fmaf(-k1, q0, k0 * q1);
          sp[tb] = fmaf(rc[tb][nb][u], dot, sp[tb]);
          sp[tb] = fmaf(rsn[tb][nb][u], crs, sp[tb]);
        }
      }
    }
    // sum over the four lanes (rows of 16) that hold one key; scores in the base-2 domain
    float sc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sc[tb] = gvad::xor32_sum(gvad::xor16_sum(sp[tb])) * a.qscale;
      if (j0 + 16 * tb + n >= c1) sc[tb] = -INFINITY;
    }
    // tile maximum: the same in every lane (exact max of identical sums), read as a scalar
    const float mtf = __int_as_float(
        __builtin_amdgcn_readfirstlane(__float_as_int(row16_max(fmaxf(sc[0], sc[1])))));
    if (mtf > m_run) {                                 // uniform per wave
      const float alpha = __builtin_amdgcn_exp2f(m_run - mtf);   // 0 from -inf
      l_part *= alpha;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) o_part[ks][e] *= alpha;
      m_run = mtf;
    }
    const float p0 = __builtin_amdgcn_exp2f(sc[0] - m_run);
    const float p1 = __builtin_amdgcn_exp2f(sc[1] - m_run);
    l_part += p0 + p1;
    // weighted sum: the probabilities of keys n and 16 + n as a bf16 pair against the same
    // dim of both keys' value rows (v_dot2, float32 accumulation)
    const unsigned pp = pack2(p0, p1);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const unsigned x0 = vb[0][ks][w2], x1 = vb[1][ks][w2];
        o_part[ks][2 * w2] = dot2(pp, __builtin_amdgcn_perm(x1, x0, 0x05040100u), o_part[ks][2 * w2]);
        o_part[ks][2 * w2 + 1] = dot2(pp, __builtin_amdgcn_perm(x1, x0, 0x07060302u), o_part[ks][2 * w2 + 1]);
      }
  };

  const int nsteps = (c1 - c0 + kStep - 1) / kStep;
  load_step(c0);
  for (int t = 0; t < nsteps; ++t) {
    const int j0 = c0 + t * kStep;
    store_step();
    __syncthreads();
    if (t + 1 < nsteps) load_step(j0 + kStep);         // uniform per work-group
    const int jw = j0 + half * kTile;
    if (jw < c1) compute(jw);                          // uniform per wave
    __syncthreads();
  }
  if (bad) {
    bad_lds = 1;
    gvad::raise_err(a.err_flag, GVA_DEVERR_BLOCK);
  }

  // reduce over the 16 lanes of a row (the keys); row kq holds dims 32 ks + 8 kq + e
  float l = row16_sum(l_part);
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) o_part[ks][e] = row16_sum(o_part[ks][e]);
  // merge the two halves of each head through LDS (the value rows are no longer needed):
  // half 1 leaves m, l and its sums; half 0 rescales both to the larger m and adds
  float *mo = reinterpret_cast<float *>(v_lds);        // [NH][DH]
  float *mm = mo + NH * DH;                            // [NH]
  float *ml = mm + NH;                                 // [NH]
  if (half == 1) {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (n != ks) continue;
      float *dst = mo + hw * DH + 32 * ks + 8 * kq;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = o_part[ks][e];
    }
    if (lane == 0) {
      mm[hw] = m_run;
      ml[hw] = l;
    }
  }
  __syncthreads();
  if (half == 1) return;
  const bool poisoned = bad_lds != 0;
  const float m1 = mm[hw];
  const float mx = fmaxf(m_run, m1);                  // finite: half 0 saw the chunk's first tile
  const float a0 = __builtin_amdgcn_exp2f(m_run - mx);
  const float a1 = __builtin_amdgcn_exp2f(m1 - mx);   // 0 when half 1 had no tile
  l = l * a0 + ml[hw] * a1;
  const float inv = 1.0f / l;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    if (n != ks) continue;                             // lane (ks, kq) writes dims 32 ks + 8 kq ..
    const float *src = mo + hw * DH + 32 * ks + 8 * kq;
    f32x4 w0, w1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w0[e] = o_part[ks][e] * a0 + src[e] * a1;
      w1[e] = o_part[ks][4 + e] * a0 + src[4 + e] * a1;
    }
    if (S == 1) {
      w0 *= inv;
      w1 *= inv;
    }
    if (poisoned) w0 = w1 = f32x4{qnan, qnan, qnan, qnan};
    float *dst = (S == 1 ? a.out + orow * DH : a.part_o + prow * DH) + 32 * ks + 8 * kq;
    *reinterpret_cast<f32x4 *>(dst) = w0;
    *reinterpret_cast<f32x4 *>(dst + 4) = w1;
  }
  if (lane == 0) {
    if (S == 1) {
      if (a.lse) a.lse[orow] = poisoned ? qnan : (mx + log2f(l)) * gvad::kLn2;
    } else {
      a.part_m[prow] = poisoned ? qnan : mx;
      a.part_l[prow] = l;
    }
  }
}

template <int DH, int DN>
hipError_t launch_dn(const gva::ReconArgs &r, dim3 grid, int nh, hipStream_t stream) {
  switch (nh) {
    case 1: hipLaunchKernelGGL((k_recon_decode<DH, DN, 1>), grid, dim3(128), 0, stream, r); break;
    case 2: hipLaunchKernelGGL((k_recon_decode<DH, DN, 2>), grid, dim3(256), 0, stream, r); break;
    case 3: hipLaunchKernelGGL((k_recon_decode<DH, DN, 3>), grid, dim3(384), 0, stream, r); break;
    case 4: hipLaunchKernelGGL((k_recon_decode<DH, DN, 4>), grid, dim3(512), 0, stream, r); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

namespace gva {

hipError_t launch_recon_decode(const ReconArgs &r, hipStream_t stream) {
  const DecodeArgs &a = r.kv;
  const int nh = a.H / a.G;
  const int64_t blocks = static_cast<int64_t>(a.B) * a.num_splits * a.G;
  if (blocks < 1 || blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (a.d_h == 64 && r.d_n == 64) return launch_dn<64, 64>(r, grid, nh, stream);
  if (a.d_h == 64 && r.d_n == 128) return launch_dn<64, 128>(r, grid, nh, stream);
  if (a.d_h == 128 && r.d_n == 64) return launch_dn<128, 64>(r, grid, nh, stream);
  if (a.d_h == 128 && r.d_n == 128) return launch_dn<128, 128>(r, grid, nh, stream);
  return hipErrorInvalidValue;
}

}  // namespace gva
