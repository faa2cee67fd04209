// k_append_absorb.hip - cache append (values and the shared rotated positional key) and query
// absorption for Grouped Value Attention.
//
// Append: the cache keeps G grouped values and one positional key per token, the latter
// stored already rotated to the token's position ("GVA：KV 缓存里的 Key 其实可以不存",
// shibing624.github.io review of arXiv:2609.13285, section 关键技巧二; section 缓存账本).
// Absorption: q~_h = q_nope_h M_h^T, formed once per query token (same review, section
// 关键技巧一, the absorption identity).
#include <hip/hip_runtime.h>

#include "gva_device.h"

namespace {

using gvad::f64_to_bf16_bits;
using gvad::f64_to_f32_bits;

// One work-group per appended token. Threads stride over the G*d_h/2 value pairs, then over
// the d_r/2 positional pairs. Values take one rounding fp32 -> cache type (through an exact
// float64 widening); the positional key is rotated in float64 and rounded once. Token k of the
// inputs goes to sequence b (checked by the caller to lie in [0, B)) at position p.
template <bool BF16>
__device__ __forceinline__ void append_one(const gva::DecodeArgs &a, int k, int b, int p,
                                           const float *v_new, const float *kr_raw,
                                           const double *rope, int32_t max_pos) {
  const int cap = a.max_blocks << a.log2_bs;
  int32_t err = 0;
  if (p < 0) err = GVA_DEVERR_LENGTH;
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
  const int G = a.G, d_h = a.d_h, d_r = a.d_r;
  const int half_h = d_h >> 1;
  const float2 *src = reinterpret_cast<const float2 *>(v_new + static_cast<int64_t>(k) * G * d_h);
  for (int idx = threadIdx.x; idx < G * half_h; idx += blockDim.x) {
    const int g = idx / half_h;
    const int i = (idx - g * half_h) * 2;
    const float2 x = src[idx];
    const int64_t o = blk * a.v_sb + off * a.v_st + static_cast<int64_t>(g) * a.v_sg + i;
    if (BF16) {
      const uint32_t lo = f64_to_bf16_bits(static_cast<double>(x.x));
      const uint32_t hi = f64_to_bf16_bits(static_cast<double>(x.y));
      reinterpret_cast<uint32_t *>(const_cast<void *>(a.v))[o >> 1] = lo | (hi << 16);
    } else {
      uint2 w;
      w.x = f64_to_f32_bits(static_cast<double>(x.x));
      w.y = f64_to_f32_bits(static_cast<double>(x.y));
      *reinterpret_cast<uint2 *>(reinterpret_cast<uint32_t *>(const_cast<void *>(a.v)) + o) = w;
    }
  }
  const int half_r = d_r >> 1;
  const float2 *ksrc = reinterpret_cast<const float2 *>(kr_raw + static_cast<int64_t>(k) * d_r);
  const double2 *cs = reinterpret_cast<const double2 *>(rope) + static_cast<int64_t>(p) * half_r;
  for (int i = threadIdx.x; i < half_r; i += blockDim.x) {
    const float2 x = ksrc[i];
    const double2 t = cs[i];
    double y0, y1;
    gvad::rotate_pair_f64(static_cast<double>(x.x), static_cast<double>(x.y), t.x, t.y, &y0, &y1);
    const int64_t o = blk * a.kr_sb + off * a.kr_st + 2 * i;
    if (BF16) {
      const uint32_t lo = f64_to_bf16_bits(y0);
      const uint32_t hi = f64_to_bf16_bits(y1);
      reinterpret_cast<uint32_t *>(const_cast<void *>(a.kr))[o >> 1] = lo | (hi << 16);
    } else {
      uint2 w;
      w.x = f64_to_f32_bits(y0);
      w.y = f64_to_f32_bits(y1);
      *reinterpret_cast<uint2 *>(reinterpret_cast<uint32_t *>(const_cast<void *>(a.kr)) + o) = w;
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_append(gva::DecodeArgs a, int32_t B, const int32_t *seq,
                                                const int32_t *pos, const float *v_new,
                                                const float *kr_raw, const double *rope,
                                                int32_t max_pos) {
  const int k = blockIdx.x;
  const int b = seq[k];
  if (b < 0 || b >= B) {
    if (threadIdx.x == 0) gvad::raise_err(a.err_flag, GVA_DEVERR_SEQ);
    return;
  }
  append_one<BF16>(a, k, b, pos[k], v_new, kr_raw, rope, max_pos);
}

// Absorption, q~[t][i] = sum_j M_h[i][j] q_nope[t][h][j]: for every head a small GEMM of the
// d_h x d_n map by the d_n x n queries. Work-group (head h, tile of kAbsQ query tokens, tile of
// kAbsRows rows of M_h): both operand tiles are staged in LDS, 128 columns at a time, with
// coalesced loads (rows padded by 4 floats so that the 16-byte reads of 8 consecutive rows hit
// 8 different bank groups);
// thread (i, tq) forms q~ for row i and tokens tq, tq + 8, tq + 16, tq + 24, accumulating the
// float32 products in order j = 0 .. d_n - 1. The work-groups with row tile 0 also rotate the
// positional slice at the token's position in float64 and round it once to float32.
constexpr int kAbsQ = 32;
constexpr int kAbsRows = 32;
constexpr int kAbsThreads = 256;

struct AbsorbArgs {
  int32_t H, d_h, d_n, d_r, n_q;
  const float *q_nope, *q_rope;
  const int32_t *q_pos;
  const float *M;
  const double *rope;
  int32_t max_pos;
  float *q_abs;
  int32_t *err_flag;
};

// Tile (head h, query tile ty, row tile tz) of the absorption.
__device__ __forceinline__ void absorb_tile(const AbsorbArgs &x, int h, int ty, int tz) {
  constexpr int kJ4 = 32;                      // d_n is walked in chunks of 128 (32 float4)
  constexpr int kStride4 = kJ4 + 1;            // row stride in float4 (4 floats of padding)
  __shared__ float4 qs[kAbsQ * kStride4];
  __shared__ float4 ms[kAbsRows * kStride4];
  const int H = x.H, d_h = x.d_h, d_n = x.d_n, d_r = x.d_r, n_q = x.n_q;
  const float *q_nope = x.q_nope, *q_rope = x.q_rope, *M = x.M;
  const int32_t *q_pos = x.q_pos;
  const double *rope = x.rope;
  const int32_t max_pos = x.max_pos;
  float *q_abs = x.q_abs;
  int32_t *err_flag = x.err_flag;
  const int k0 = ty * kAbsQ;
  const int i0 = tz * kAbsRows;
  const int nt = min(kAbsQ, n_q - k0);
  const int ni = min(kAbsRows, d_h - i0);
  const int dn4 = d_n >> 2;
  const int row = d_h + d_r;
  const int tid = threadIdx.x;
  const int i = tid >> 3;                      // row of the tile
  const int tq = tid & 7;                      // tokens tq + 8 k
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  // the positions of this thread's tokens, requested before anything waits
  int32_t tpos[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) tpos[k] = tq + 8 * k < nt ? q_pos[k0 + tq + 8 * k] : 0;
  const float4 *Mh = reinterpret_cast<const float4 *>(M + (static_cast<int64_t>(h) * d_h + i0) * d_n);
  // each thread stages kStage float4 of either operand per chunk; all of its loads go out
  // before the first LDS store (one round of loads per chunk, not one per float4)
  constexpr int kStage = kAbsQ * kJ4 / kAbsThreads;
  static_assert(kAbsQ == kAbsRows && kStage * kAbsThreads == kAbsQ * kJ4, "staging map");
  for (int jc = 0; jc < dn4; jc += kJ4) {
    const int nj = min(kJ4, dn4 - jc);
    float4 vq[kStage], vm[kStage];
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      const int idx = tid + u * kAbsThreads;
      const int t = idx / kJ4;                  // token (q_nope) or row (M) of the tile
      const int j4 = idx - t * kJ4;
      vq[u] = float4{0.f, 0.f, 0.f, 0.f};
      vm[u] = float4{0.f, 0.f, 0.f, 0.f};
      if (t < nt && j4 < nj)
        vq[u] = reinterpret_cast<const float4 *>(q_nope + (static_cast<int64_t>(k0 + t) * H + h) * d_n)[jc + j4];
      if (t < ni && j4 < nj) vm[u] = Mh[static_cast<int64_t>(t) * dn4 + jc + j4];
    }
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      const int idx = tid + u * kAbsThreads;
      const int t = idx / kJ4;
      const int j4 = idx - t * kJ4;
      qs[t * kStride4 + j4] = vq[u];
      ms[t * kStride4 + j4] = vm[u];
    }
    __syncthreads();
    for (int j4 = 0; j4 < nj; ++j4) {
      const float4 m = ms[i * kStride4 + j4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 q = qs[(tq + 8 * k) * kStride4 + j4];
        acc[k] = fmaf(m.x, q.x, acc[k]);
        acc[k] = fmaf(m.y, q.y, acc[k]);
        acc[k] = fmaf(m.z, q.z, acc[k]);
        acc[k] = fmaf(m.w, q.w, acc[k]);
      }
    }
    __syncthreads();
  }
  if (i < ni) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = tq + 8 * k;
      if (t >= nt) continue;
      const int p = tpos[k];
      const bool bad = p < 0 || p >= max_pos;
      q_abs[(static_cast<int64_t>(k0 + t) * H + h) * row + i0 + i] = bad ? __int_as_float(0x7fc00000) : acc[k];
    }
  }
  if (tz != 0) return;
  const int half_r = d_r >> 1;
  for (int idx = tid; idx < nt * half_r; idx += kAbsThreads) {
    const int t = idx / half_r;
    const int r = idx - t * half_r;
    const int k = k0 + t;
    const int p = q_pos[k];
    float2 y;
    if (p < 0 || p >= max_pos) {
      y.x = y.y = __int_as_float(0x7fc00000);
      if (r == 0 && err_flag) atomicOr(err_flag, GVA_DEVERR_ROPE);
    } else {
      const float2 x = reinterpret_cast<const float2 *>(q_rope + (static_cast<int64_t>(k) * H + h) * d_r)[r];
      const double2 t2 = reinterpret_cast<const double2 *>(rope)[static_cast<int64_t>(p) * half_r + r];
      double y0, y1;
      gvad::rotate_pair_f64(static_cast<double>(x.x), static_cast<double>(x.y), t2.x, t2.y, &y0, &y1);
      y.x = gvad::f64_to_f32(y0);
      y.y = gvad::f64_to_f32(y1);
    }
    float *dst = q_abs + (static_cast<int64_t>(k) * H + h) * row + d_h + 2 * r;
    dst[0] = y.x;
    dst[1] = y.y;
  }
}

__global__ __launch_bounds__(kAbsThreads) void k_absorb(AbsorbArgs x) {
  absorb_tile(x, blockIdx.x, blockIdx.y, blockIdx.z);
}

// The append and the absorption of one decode step in one launch (they touch disjoint data):
// work-group k < B appends token k to sequence k at position pos[k]; the others are the
// absorption's tiles, head fastest, then query tile, then row tile (query k sits at pos[k]).
template <bool BF16>
__global__ __launch_bounds__(256) void k_step_prep(gva::DecodeArgs a, int32_t B, const int32_t *pos,
                                                   const float *v_new, const float *kr_raw,
                                                   const double *rope, int32_t max_pos,
                                                   AbsorbArgs x, int32_t n_qt) {
  const int id = blockIdx.x;
  if (id < B) {
    append_one<BF16>(a, id, id, pos[id], v_new, kr_raw, rope, max_pos);
    return;
  }
  const int r = id - B;
  const int h = r % x.H;
  const int ty = (r / x.H) % n_qt;
  const int tz = r / (x.H * n_qt);
  absorb_tile(x, h, ty, tz);
}

}  // namespace

namespace gva {

hipError_t launch_append(const gva_dims *d, const gva_cache *c, int32_t B, int32_t n_tok,
                         const int32_t *seq, const int32_t *pos, const float *v_new,
                         const float *kr_raw, hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  DecodeArgs a{};
  a.v = c->v;
  a.kr = c->kr;
  a.v_sb = c->v_stride_block;
  a.v_st = c->v_stride_token;
  a.v_sg = c->v_stride_group;
  a.kr_sb = c->kr_stride_block;
  a.kr_st = c->kr_stride_token;
  a.num_blocks = c->num_blocks;
  a.log2_bs = __builtin_ctz(static_cast<unsigned>(c->block_size));
  a.max_blocks = c->max_blocks;
  a.block_table = c->block_table;
  a.err_flag = c->err_flag;
  a.H = d->H;
  a.G = d->G;
  a.d_h = d->d_h;
  a.d_r = d->d_r;
  const int threads = 256;
  if (c->dtype == GVA_DTYPE_BF16)
    hipLaunchKernelGGL(k_append<true>, dim3(n_tok), dim3(threads), 0, stream, a, B, seq, pos, v_new,
                       kr_raw, c->rope, c->max_pos);
  else
    hipLaunchKernelGGL(k_append<false>, dim3(n_tok), dim3(threads), 0, stream, a, B, seq, pos,
                       v_new, kr_raw, c->rope, c->max_pos);
  return hipGetLastError();
}

hipError_t launch_absorb(const gva_dims *d, int32_t n_q, const float *q_nope, const float *q_rope,
                         const int32_t *q_pos, const float *M, const double *rope,
                         int32_t max_pos, float *q_abs, int32_t *err_flag, hipStream_t stream) {
  if (n_q == 0) return hipSuccess;
  const dim3 grid(d->H, (n_q + kAbsQ - 1) / kAbsQ, (d->d_h + kAbsRows - 1) / kAbsRows);
  const AbsorbArgs x{d->H, d->d_h, d->d_n, d->d_r, n_q, q_nope, q_rope, q_pos, M, rope, max_pos,
                     q_abs, err_flag};
  hipLaunchKernelGGL(k_absorb, grid, dim3(kAbsThreads), 0, stream, x);
  return hipGetLastError();
}

hipError_t launch_step_prep(const DecodeArgs &a, bool bf16, int32_t B, const int32_t *pos,
                            const float *v_new, const float *kr_raw, const double *rope,
                            int32_t max_pos, int32_t d_n, const float *q_nope, const float *q_rope,
                            const float *M, float *q_abs, hipStream_t stream) {
  const int n_qt = (B + kAbsQ - 1) / kAbsQ;
  const int n_rt = (a.d_h + kAbsRows - 1) / kAbsRows;
  const AbsorbArgs x{a.H, a.d_h, d_n, a.d_r, B, q_nope, q_rope, pos, M, rope, max_pos, q_abs,
                     a.err_flag};
  const dim3 grid(static_cast<unsigned>(B + a.H * n_qt * n_rt));
  if (bf16)
    hipLaunchKernelGGL(k_step_prep<true>, grid, dim3(256), 0, stream, a, B, pos, v_new, kr_raw,
                       rope, max_pos, x, n_qt);
  else
    hipLaunchKernelGGL(k_step_prep<false>, grid, dim3(256), 0, stream, a, B, pos, v_new, kr_raw,
                       rope, max_pos, x, n_qt);
  return hipGetLastError();
}

}  // namespace gva
