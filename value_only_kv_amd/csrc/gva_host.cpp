// gva_host.cpp - host side of the GVA library that needs no GPU: argument validation,
// split planning, the RoPE table and the diagnostics. Compiled by the host C++ compiler;
// nothing here calls HIP, so every check can be exercised on a machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "gva_internal.h"

namespace gva {

namespace {
thread_local std::string g_last_error;

// The table holds exactly what the C library's separate cos and sin return. Calling them through
// volatile pointers keeps the compiler from fusing the pair into one sincos call, whose last bit
// can differ from cos for some arguments.
double (*volatile g_libm_cos)(double) = cos;
double (*volatile g_libm_sin)(double) = sin;
double (*volatile g_libm_pow)(double, double) = pow;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
}  // namespace

const char *last_error_cstr() { return g_last_error.c_str(); }

gva_status fail(gva_status status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

gva_status check_dims(const gva_dims *d) {
  if (!d) return fail(GVA_ERR_INVALID_ARG, "dims is NULL");
  if (d->H < 1 || d->H > kMaxH) return fail(GVA_ERR_INVALID_ARG, "H=%d outside [1, %d]", d->H, kMaxH);
  if (d->G < 1 || d->G > d->H) return fail(GVA_ERR_INVALID_ARG, "G=%d outside [1, H=%d]", d->G, d->H);
  if (d->H % d->G != 0) return fail(GVA_ERR_INVALID_ARG, "H=%d is not a multiple of G=%d", d->H, d->G);
  if (d->d_h < 2 || d->d_h > kMaxDh || d->d_h % 2 != 0)
    return fail(GVA_ERR_INVALID_ARG, "d_h=%d must be even and in [2, %d]", d->d_h, kMaxDh);
  if (d->d_n < 1 || d->d_n > kMaxDn)
    return fail(GVA_ERR_INVALID_ARG, "d_n=%d outside [1, %d]", d->d_n, kMaxDn);
  if (d->d_r < 2 || d->d_r > kMaxDr || d->d_r % 2 != 0)
    return fail(GVA_ERR_INVALID_ARG, "d_r=%d must be even and in [2, %d]", d->d_r, kMaxDr);
  if (d->g_of_h) {
    int count[kMaxH] = {0};
    for (int h = 0; h < d->H; ++h) {
      const int32_t g = d->g_of_h[h];
      if (g < 0 || g >= d->G)
        return fail(GVA_ERR_INVALID_ARG, "g_of_h[%d]=%d outside [0, G=%d)", h, g, d->G);
      ++count[g];
    }
    for (int g = 0; g < d->G; ++g)
      if (count[g] != d->H / d->G)
        return fail(GVA_ERR_INVALID_ARG, "g_of_h gives group %d %d heads, not H/G=%d", g, count[g],
                    d->H / d->G);
  }
  return GVA_OK;
}

void group_order(const gva_dims *d, uint8_t *head_of) {
  const int per = d->H / d->G;
  if (!d->g_of_h) {
    for (int h = 0; h < d->H; ++h) head_of[h] = static_cast<uint8_t>(h);
    return;
  }
  int next[kMaxH] = {0};
  for (int h = 0; h < d->H; ++h) {
    const int g = d->g_of_h[h];
    head_of[g * per + next[g]++] = static_cast<uint8_t>(h);
  }
}

gva_status check_cache(const gva_dims *d, const gva_cache *c) {
  if (!c) return fail(GVA_ERR_INVALID_ARG, "cache is NULL");
  if (c->dtype != GVA_DTYPE_F32 && c->dtype != GVA_DTYPE_BF16)
    return fail(GVA_ERR_INVALID_ARG, "unknown cache dtype %d", (int)c->dtype);
  if (!c->v || !c->kr) return fail(GVA_ERR_INVALID_ARG, "cache v or kr is NULL");
  if (!aligned(c->v, 16) || !aligned(c->kr, 16))
    return fail(GVA_ERR_INVALID_ARG, "cache v and kr must be 16-byte aligned");
  if (!c->block_table) return fail(GVA_ERR_INVALID_ARG, "block_table is NULL");
  if (!c->rope) return fail(GVA_ERR_INVALID_ARG, "rope table is NULL");
  if (!aligned(c->rope, 16)) return fail(GVA_ERR_INVALID_ARG, "rope table must be 16-byte aligned");
  if (c->max_pos < 1) return fail(GVA_ERR_INVALID_ARG, "max_pos=%d must be >= 1", c->max_pos);
  if (c->num_blocks < 1) return fail(GVA_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (c->num_blocks > (int64_t)INT32_MAX)
    return fail(GVA_ERR_INVALID_ARG, "num_blocks exceeds the int32 block ids of the table");
  if (!pow2(c->block_size) || c->block_size > (1 << 30))
    return fail(GVA_ERR_INVALID_ARG, "block_size=%d must be a power of two", c->block_size);
  if (c->max_blocks < 1) return fail(GVA_ERR_INVALID_ARG, "max_blocks must be >= 1");
  if ((int64_t)c->max_blocks * c->block_size > (int64_t)INT32_MAX)
    return fail(GVA_ERR_INVALID_ARG, "max_blocks * block_size exceeds int32 positions");
  const int64_t s[5] = {c->v_stride_block, c->v_stride_token, c->v_stride_group,
                        c->kr_stride_block, c->kr_stride_token};
  for (int i = 0; i < 5; ++i) {
    if (s[i] < 0) return fail(GVA_ERR_INVALID_ARG, "cache strides must be >= 0");
    if (s[i] % 2 != 0) return fail(GVA_ERR_INVALID_ARG, "cache strides must be even");
  }
  // Each row must fit between its neighbours: a token row of a group holds d_h elements and a
  // positional row d_r elements. (Overlapping layouts are the caller's mistake; these checks
  // catch the common ones.)
  if (c->v_stride_group < d->d_h && d->G > 1 && c->v_stride_token < d->d_h)
    return fail(GVA_ERR_INVALID_ARG, "v strides overlap rows");
  if (c->kr_stride_token < d->d_r && c->block_size > 1)
    return fail(GVA_ERR_INVALID_ARG, "kr_stride_token=%lld < d_r=%d",
                (long long)c->kr_stride_token, d->d_r);
  return GVA_OK;
}

gva_status check_append(const gva_dims *d, const gva_cache *c, int32_t B, int32_t n_tok,
                        const int32_t *seq, const int32_t *pos, const float *v_new,
                        const float *kr_raw) {
  gva_status st = check_dims(d);
  if (st != GVA_OK) return st;
  if ((st = check_cache(d, c)) != GVA_OK) return st;
  if (B < 1) return fail(GVA_ERR_INVALID_ARG, "B=%d must be >= 1", B);
  if (n_tok < 0) return fail(GVA_ERR_INVALID_ARG, "n_tok=%d must be >= 0", n_tok);
  if (n_tok == 0) return GVA_OK;
  if (!seq || !pos || !v_new || !kr_raw) return fail(GVA_ERR_INVALID_ARG, "append input is NULL");
  if (!aligned(v_new, 8) || !aligned(kr_raw, 8))
    return fail(GVA_ERR_INVALID_ARG, "v_new and kr_raw must be 8-byte aligned");
  return GVA_OK;
}

gva_status check_absorb(const gva_dims *d, int32_t n_q, const float *q_nope, const float *q_rope,
                        const int32_t *q_pos, const float *M, const double *rope, int32_t max_pos,
                        const float *q_abs) {
  gva_status st = check_dims(d);
  if (st != GVA_OK) return st;
  if (n_q < 0) return fail(GVA_ERR_INVALID_ARG, "n_q=%d must be >= 0", n_q);
  if (n_q == 0) return GVA_OK;
  if (!q_nope || !q_rope || !q_pos || !M || !rope || !q_abs)
    return fail(GVA_ERR_INVALID_ARG, "absorb argument is NULL");
  if (max_pos < 1) return fail(GVA_ERR_INVALID_ARG, "max_pos=%d must be >= 1", max_pos);
  if (!aligned(q_nope, 16) || !aligned(q_rope, 8) || !aligned(M, 16) || !aligned(q_abs, 8) ||
      !aligned(rope, 16))
    return fail(GVA_ERR_INVALID_ARG,
                "absorb buffers misaligned (q_nope and M need 16 bytes, q_rope and q_abs 8)");
  if (d->d_n % 4 != 0) return fail(GVA_ERR_UNSUPPORTED, "absorb needs d_n %% 4 == 0 (d_n=%d)", d->d_n);
  return GVA_OK;
}

bool mfma_supported(const gva_dims *d, const gva_cache *c, const char **why) {
  const char *w = nullptr;
  const int hpg = d->H / d->G;
  if (c->dtype != GVA_DTYPE_BF16) w = "the matrix-core kernel needs a bf16 cache";
  else if (d->d_h % 32 != 0 || d->d_h > 256) w = "the matrix-core kernel needs d_h % 32 == 0, <= 256";
  else if (d->d_r % 8 != 0 || d->d_r > 32) w = "the matrix-core kernel needs d_r % 8 == 0, <= 32";
  else if (hpg > 16) w = "the matrix-core kernel needs H / G <= 16";
  else if (d->G > 16) w = "the matrix-core kernel needs G <= 16";
  else if (c->block_size < 16) w = "the matrix-core kernel needs block_size >= 16";
  else if (c->v_stride_block % 8 || c->v_stride_token % 8 || c->v_stride_group % 8 ||
           c->kr_stride_block % 8 || c->kr_stride_token % 8)
    w = "the matrix-core kernel needs strides that are multiples of 8 elements";
  if (why) *why = w;
  return w == nullptr;
}

static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool plan_decode(const gva_dims *d, int32_t B, int32_t max_len, int32_t num_splits,
                 bool balanced, DecodePlan *plan, bool share_key) {
  if (!d || B < 1 || max_len < 0 || num_splits < 0 || num_splits > kMaxSplits) return false;
  *plan = DecodePlan{};
  if (balanced && share_key && num_splits == 0 && decode_merged_shape(d, B)) {
    // small batch: K work-groups per (sequence, group) merge their partials themselves
    StepPlan sp;
    if (!plan_step(d, B, max_len, &sp)) return false;
    plan->merged_K = sp.K;
    const int64_t kw = static_cast<int64_t>(sp.K) * step_waves_of(d->d_h);
    const int64_t tiles = (static_cast<int64_t>(max_len) + kTilePositions - 1) / kTilePositions;
    plan->tiles_per_wave = static_cast<int32_t>((tiles + kw - 1) / kw);
    plan->off_o = sp.off_po;
    plan->off_m = sp.off_pm;
    plan->off_l = sp.off_pl;
    plan->ws_bytes = sp.ws_bytes;
    return true;
  }
  const int64_t tiles_max = static_cast<int64_t>(B) * ((max_len + kTilePositions - 1) / kTilePositions);
  if (balanced && num_splits == 0 && B > 1 && tiles_max > 0 &&
      tiles_max < (int64_t(1) << 31) && d->G > 0) {
    // Equal ranges over all sequences' tiles: at most one pass of work-groups over the device;
    // fewer for small batches, down to one work-group per compute unit (kPlanCUs / nz ranges)
    // or ranges of kMinTilesPerRange tiles (assuming every sequence at max_len), whichever is
    // more. A single sequence gets the same cut from the split grid, without the search for
    // its range.
    const BalancedLayout lay = balanced_layout(d->G, share_key, tiles_max);
    const int64_t nz = d->G / lay.waves;
    const int64_t by_size = (tiles_max + kMinTilesPerRange - 1) / kMinTilesPerRange;
    int64_t R = by_size > kPlanCUs / nz ? by_size : kPlanCUs / nz;
    if (R > kPlanCUs * lay.groups_per_cu / nz) R = kPlanCUs * lay.groups_per_cu / nz;
    if (R > tiles_max) R = tiles_max;
    if (R > kMaxSplits) R = kMaxSplits;
    if (R < 1) R = 1;
    plan->num_ranges = (int32_t)R;
    const size_t rows = (size_t)(R + B) * (size_t)d->H;
    plan->off_o = kWsHeader;
    plan->off_m = plan->off_o + round_up(rows * (size_t)d->d_h * 4, 256);
    plan->off_l = plan->off_m + round_up(rows * 4, 256);
    plan->off_prefix = plan->off_l + round_up(rows * 4, 256);
    plan->ws_bytes = plan->off_prefix + round_up((size_t)(B + 1) * 4, 256);
    return true;
  }
  const int64_t q = kChunkQuantum;
  int64_t S = num_splits;
  if (S == 0) {
    // Chunks of at most 2048 positions for long sequences, and at least kPlanCUs / 2
    // (sequence, chunk) items when the batch is small, down to chunks of kChunkQuantum
    // positions (short sequences are latency-bound: more, shorter chunks finish sooner).
    const int64_t by_len = (max_len + 2047) / 2048;
    const int64_t by_cus = (kPlanCUs / 2 + B - 1) / B;
    S = by_len > by_cus ? by_len : by_cus;
    const int64_t cap = (max_len + q - 1) / q;
    if (S > cap) S = cap;
    if (S < 1) S = 1;
    if (S > kMaxSplits) S = kMaxSplits;
  }
  int64_t chunk = max_len > 0 ? (max_len + S - 1) / S : q;
  chunk = (chunk + q - 1) / q * q;
  if (max_len > 0) S = (max_len + chunk - 1) / chunk;  // no chunk starts at or after max_len
  if (S < 1) S = 1;
  plan->num_splits = (int32_t)S;
  plan->chunk = (int32_t)chunk;
  if (S == 1) return true;
  const size_t rows = (size_t)B * (size_t)S * (size_t)d->H;
  plan->off_o = kWsHeader;
  plan->off_m = plan->off_o + round_up(rows * (size_t)d->d_h * 4, 256);
  plan->off_l = plan->off_m + round_up(rows * 4, 256);
  plan->ws_bytes = plan->off_l + round_up(rows * 4, 256);
  return true;
}

gva_status check_decode(const gva_dims *d, const gva_cache *c, int32_t B,
                        const int32_t *seq_len, int32_t max_len, const float *q_abs,
                        float scale, int32_t num_splits, int32_t kernel, const void *workspace,
                        size_t workspace_bytes, const float *out, DecodePlan *plan,
                        bool *use_mfma, bool share_key) {
  gva_status st = check_dims(d);
  if (st != GVA_OK) return st;
  if ((st = check_cache(d, c)) != GVA_OK) return st;
  if (B < 1) return fail(GVA_ERR_INVALID_ARG, "B=%d must be >= 1", B);
  if (!seq_len || !q_abs || !out) return fail(GVA_ERR_INVALID_ARG, "decode argument is NULL");
  if (!aligned(q_abs, 16) || !aligned(out, 16))
    return fail(GVA_ERR_INVALID_ARG, "q_abs and out must be 16-byte aligned");
  if (max_len < 0) return fail(GVA_ERR_INVALID_ARG, "max_len=%d must be >= 0", max_len);
  if ((int64_t)max_len > (int64_t)c->max_blocks * c->block_size)
    return fail(GVA_ERR_INVALID_ARG, "max_len=%d exceeds the block table's capacity", max_len);
  if (!(scale > 0.0f) || !isfinite(scale))
    return fail(GVA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(GVA_ERR_INVALID_ARG, "num_splits=%d outside [0, %d]", num_splits, kMaxSplits);
  if (kernel < GVA_KERNEL_AUTO || kernel > GVA_KERNEL_MFMA)
    return fail(GVA_ERR_INVALID_ARG, "unknown kernel selector %d", kernel);
  const char *why = nullptr;
  const bool can = mfma_supported(d, c, &why);
  if (kernel == GVA_KERNEL_MFMA && !can) return fail(GVA_ERR_UNSUPPORTED, "%s", why);
  *use_mfma = (kernel == GVA_KERNEL_MFMA) || (kernel == GVA_KERNEL_AUTO && can);
  if (!plan_decode(d, B, max_len, num_splits, *use_mfma, plan, share_key))
    return fail(GVA_ERR_INVALID_ARG, "cannot plan the decode split");
  if (plan->ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan->ws_bytes)
      return fail(GVA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan->ws_bytes,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(GVA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  return GVA_OK;
}

gva_status check_step(const gva_dims *d, const gva_cache *c, int32_t B, const int32_t *pos,
                      const float *v_new, const float *kr_raw, const float *q_nope,
                      const float *q_rope, const float *M, const float *q_abs) {
  gva_status st = check_dims(d);
  if (st != GVA_OK) return st;
  if ((st = check_cache(d, c)) != GVA_OK) return st;
  if (B < 1) return fail(GVA_ERR_INVALID_ARG, "B=%d must be >= 1", B);
  if (!pos || !v_new || !kr_raw) return fail(GVA_ERR_INVALID_ARG, "step append input is NULL");
  if (!aligned(v_new, 8) || !aligned(kr_raw, 8))
    return fail(GVA_ERR_INVALID_ARG, "v_new and kr_raw must be 8-byte aligned");
  return check_absorb(d, B, q_nope, q_rope, pos, M, c->rope, c->max_pos, q_abs);
}

bool step_fused_supported(const gva_dims *d, const gva_cache *c, int32_t B, int32_t max_len,
                          int32_t num_splits, bool use_mfma) {
  // One work-group per (sequence, group) holds a whole sequence, so the batch must fill at most
  // one work-group per compute unit and each sequence must be short enough for one unit
  // (at most 4 MiB of values per group).
  const int hpg = d->H / d->G;
  if (!use_mfma || num_splits != 0) return false;
  // d_h <= 64: every work-group forms its group's q~ itself, reading H / G rows of d_h x d_n
  // map; at d_h = 128 that redundant read (256 KiB per work-group) costs more than the launches
  // it saves (a B = 4, 8705-position step: 40 us in one launch against 31 us in two)
  if (d->d_h != 32 && d->d_h != 64) return false;
  if (hpg != 1 && hpg != 2 && hpg != 4 && hpg != 8) return false;
  if (d->d_n % 4 != 0) return false;
  if (static_cast<int64_t>(B) * d->G > kPlanCUs) return false;
  if (static_cast<int64_t>(max_len) * d->d_h * 2 > (int64_t{4} << 20)) return false;
  (void)c;
  return true;
}

bool decode_merged_shape(const gva_dims *d, int32_t B) {
  const int hpg = d->H / d->G;
  if (d->d_h != 32 && d->d_h != 64) return false;
  if (hpg != 1 && hpg != 2 && hpg != 4 && hpg != 8) return false;
  return static_cast<int64_t>(B) * d->G <= kPlanCUs;
}

bool step_small_supported(const gva_dims *d, const gva_cache *c, int32_t B, int32_t max_len,
                          int32_t num_splits, bool use_mfma) {
  // one work-group per (sequence, group) walks the whole sequence with four waves, so the batch
  // fills at most one work-group per compute unit and the sequences are short
  (void)c;
  if (use_mfma || num_splits != 0) return false;
  const int hpg = d->H / d->G;
  if (hpg != 1 && hpg != 2 && hpg != 4 && hpg != 8) return false;
  if (d->d_n % 4 != 0 || d->d_h > kMaxDh) return false;
  if (static_cast<int64_t>(B) * d->G > kPlanCUs || max_len > kSmallMaxLen) return false;
  // the rows of M (padded by 16 bytes) and q_nope of the group's heads are staged in LDS
  const int64_t m_bytes = static_cast<int64_t>(hpg) * d->d_h * (d->d_n / 4 + 1) * 16 +
                          static_cast<int64_t>(hpg) * d->d_n * 4;
  return m_bytes <= kSmallRegionBytes;
}

bool plan_step(const gva_dims *d, int32_t B, int32_t max_len, StepPlan *plan) {
  if (!d || B < 1 || max_len < 0 || d->G < 1) return false;
  *plan = StepPlan{};
  const int64_t pairs = static_cast<int64_t>(B) * d->G;
  if (pairs > kPlanCUs) return false;
  const int64_t waves = step_waves_of(d->d_h);
  const int64_t tiles = (max_len + kTilePositions - 1) / kTilePositions;
  int64_t K = kPlanCUs / pairs;
  const int64_t by_tiles = (tiles + waves - 1) / waves;        // at least one tile per wave
  if (K > by_tiles) K = by_tiles;
  if (K > 32) K = 32;
  if (K < 1) K = 1;
  plan->K = static_cast<int32_t>(K);
  if (K == 1) return true;
  const size_t rows = static_cast<size_t>(pairs * K) * static_cast<size_t>(d->H / d->G);
  plan->off_po = kWsHeader;
  plan->off_pm = plan->off_po + round_up(rows * static_cast<size_t>(d->d_h) * 4, 256);
  plan->off_pl = plan->off_pm + round_up(rows * 4, 256);
  plan->ws_bytes = plan->off_pl + round_up(rows * 4, 256);
  return true;
}

bool recon_supported(const gva_dims *d, const char **why) {
  const char *w = nullptr;
  if (d->d_h != 64 && d->d_h != 128) w = "the comparator kernel needs d_h of 64 or 128";
  else if (d->d_n != 64 && d->d_n != 128) w = "the comparator kernel needs d_n of 64 or 128";
  else if (d->H / d->G > 4) w = "the comparator kernel needs H / G <= 4";
  if (why) *why = w;
  return w == nullptr;
}

gva_status check_recon(const gva_dims *d, const gva_cache *c, int32_t B, const int32_t *seq_len,
                       int32_t max_len, const float *q, const int32_t *q_pos, const uint16_t *Mt,
                       const double *rope, int32_t max_pos, float scale, int32_t num_splits,
                       const void *workspace, size_t workspace_bytes, const float *out,
                       DecodePlan *plan) {
  if (!d) return fail(GVA_ERR_INVALID_ARG, "dims is NULL");
  gva_dims dd = *d;
  dd.d_r = 2;                              // not used by this entry point
  gva_status st = check_dims(&dd);
  if (st != GVA_OK) return st;
  const char *why = nullptr;
  if (!recon_supported(d, &why)) return fail(GVA_ERR_UNSUPPORTED, "%s", why);
  if (!c) return fail(GVA_ERR_INVALID_ARG, "cache is NULL");
  if (c->dtype != GVA_DTYPE_BF16) return fail(GVA_ERR_UNSUPPORTED, "the comparator needs a bf16 cache");
  if (!c->v || !aligned(c->v, 16)) return fail(GVA_ERR_INVALID_ARG, "cache v must be a 16-byte aligned pointer");
  if (!c->block_table) return fail(GVA_ERR_INVALID_ARG, "block_table is NULL");
  if (c->num_blocks < 1 || c->num_blocks > (int64_t)INT32_MAX)
    return fail(GVA_ERR_INVALID_ARG, "num_blocks must be in [1, 2^31)");
  if (!pow2(c->block_size) || c->block_size > (1 << 30))
    return fail(GVA_ERR_INVALID_ARG, "block_size=%d must be a power of two", c->block_size);
  if (c->max_blocks < 1) return fail(GVA_ERR_INVALID_ARG, "max_blocks must be >= 1");
  if ((int64_t)c->max_blocks * c->block_size > (int64_t)INT32_MAX)
    return fail(GVA_ERR_INVALID_ARG, "max_blocks * block_size exceeds int32 positions");
  const int64_t vs[3] = {c->v_stride_block, c->v_stride_token, c->v_stride_group};
  for (int i = 0; i < 3; ++i)
    if (vs[i] < 0 || vs[i] % 8 != 0)
      return fail(GVA_ERR_INVALID_ARG, "v strides must be >= 0 and multiples of 8 elements");
  if (c->v_stride_group < d->d_h && d->G > 1 && c->v_stride_token < d->d_h)
    return fail(GVA_ERR_INVALID_ARG, "v strides overlap rows");
  if (B < 1) return fail(GVA_ERR_INVALID_ARG, "B=%d must be >= 1", B);
  if (!seq_len || !q || !q_pos || !Mt || !rope || !out)
    return fail(GVA_ERR_INVALID_ARG, "comparator argument is NULL");
  if (!aligned(q, 16) || !aligned(Mt, 16) || !aligned(rope, 16) || !aligned(out, 16))
    return fail(GVA_ERR_INVALID_ARG, "q, Mt, rope and out must be 16-byte aligned");
  if (max_pos < 32) return fail(GVA_ERR_INVALID_ARG, "max_pos=%d must be >= 32", max_pos);
  if (max_len < 0) return fail(GVA_ERR_INVALID_ARG, "max_len=%d must be >= 0", max_len);
  if ((int64_t)max_len > (int64_t)c->max_blocks * c->block_size)
    return fail(GVA_ERR_INVALID_ARG, "max_len=%d exceeds the block table's capacity", max_len);
  if (!(scale > 0.0f) || !isfinite(scale))
    return fail(GVA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(GVA_ERR_INVALID_ARG, "num_splits=%d outside [0, %d]", num_splits, kMaxSplits);
  if (!plan_decode(&dd, B, max_len, num_splits, false, plan))
    return fail(GVA_ERR_INVALID_ARG, "cannot plan the decode split");
  if (plan->ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan->ws_bytes)
      return fail(GVA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan->ws_bytes,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(GVA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  return GVA_OK;
}

void add_latent_queue(DecodePlan *plan) {
  plan->off_queue = round_up(plan->ws_bytes, 256);
  plan->ws_bytes = plan->off_queue + 256;
}

gva_status check_latent(const gva_dims *d, const gva_cache *c, int32_t B, const int32_t *seq_len,
                        int32_t max_len, const float *q_abs, float scale, int32_t num_splits,
                        const void *workspace, size_t workspace_bytes, const float *out,
                        DecodePlan *plan) {
  if (!d) return fail(GVA_ERR_INVALID_ARG, "dims is NULL");
  if (d->G != 1) return fail(GVA_ERR_INVALID_ARG, "the latent comparator takes G=1 (one latent), got G=%d", d->G);
  if (d->H != 8 && d->H != 16 && d->H != 32)
    return fail(GVA_ERR_UNSUPPORTED, "the latent comparator supports H of 8, 16 or 32, got %d", d->H);
  if (d->d_h != 256 && d->d_h != 512)
    return fail(GVA_ERR_UNSUPPORTED, "the latent comparator supports d_c (d_h) of 256 or 512, got %d", d->d_h);
  if (d->d_r < 8 || d->d_r > 64 || d->d_r % 8 != 0)
    return fail(GVA_ERR_UNSUPPORTED, "the latent comparator needs d_r in [8, 64], a multiple of 8");
  if (!c) return fail(GVA_ERR_INVALID_ARG, "cache is NULL");
  if (c->dtype != GVA_DTYPE_BF16) return fail(GVA_ERR_UNSUPPORTED, "the latent comparator needs a bf16 cache");
  if (!c->v || !c->kr || !aligned(c->v, 16) || !aligned(c->kr, 16))
    return fail(GVA_ERR_INVALID_ARG, "cache v and kr must be 16-byte aligned pointers");
  if (!c->block_table) return fail(GVA_ERR_INVALID_ARG, "block_table is NULL");
  if (c->num_blocks < 1 || c->num_blocks > (int64_t)INT32_MAX)
    return fail(GVA_ERR_INVALID_ARG, "num_blocks must be in [1, 2^31)");
  if (!pow2(c->block_size) || c->block_size > (1 << 30))
    return fail(GVA_ERR_INVALID_ARG, "block_size=%d must be a power of two", c->block_size);
  if (c->block_size < 16)
    return fail(GVA_ERR_UNSUPPORTED, "the latent comparator needs block_size >= 16");
  if (c->max_blocks < 1) return fail(GVA_ERR_INVALID_ARG, "max_blocks must be >= 1");
  if ((int64_t)c->max_blocks * c->block_size > (int64_t)INT32_MAX)
    return fail(GVA_ERR_INVALID_ARG, "max_blocks * block_size exceeds int32 positions");
  const int64_t st[4] = {c->v_stride_block, c->v_stride_token, c->kr_stride_block, c->kr_stride_token};
  for (int i = 0; i < 4; ++i)
    if (st[i] < 0 || st[i] % 8 != 0)
      return fail(GVA_ERR_INVALID_ARG, "latent and kr strides must be >= 0 and multiples of 8 elements");
  if (c->block_size > 1 && (c->v_stride_token < d->d_h || c->kr_stride_token < d->d_r))
    return fail(GVA_ERR_INVALID_ARG, "latent or kr token rows overlap");
  if (B < 1) return fail(GVA_ERR_INVALID_ARG, "B=%d must be >= 1", B);
  if (!seq_len || !q_abs || !out) return fail(GVA_ERR_INVALID_ARG, "latent comparator argument is NULL");
  if (!aligned(q_abs, 16) || !aligned(out, 16))
    return fail(GVA_ERR_INVALID_ARG, "q_abs and out must be 16-byte aligned");
  if (max_len < 0) return fail(GVA_ERR_INVALID_ARG, "max_len=%d must be >= 0", max_len);
  if ((int64_t)max_len > (int64_t)c->max_blocks * c->block_size)
    return fail(GVA_ERR_INVALID_ARG, "max_len=%d exceeds the block table's capacity", max_len);
  if (!(scale > 0.0f) || !isfinite(scale))
    return fail(GVA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(GVA_ERR_INVALID_ARG, "num_splits=%d outside [0, %d]", num_splits, kMaxSplits);
  if (!plan_decode(d, B, max_len, num_splits, false, plan))
    return fail(GVA_ERR_INVALID_ARG, "cannot plan the decode split");
  add_latent_queue(plan);
  if (!workspace || workspace_bytes < plan->ws_bytes)
    return fail(GVA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan->ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(GVA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return GVA_OK;
}

gva_status check_prefill(const gva_dims *d, const gva_cache *c, int32_t B, const int32_t *start,
                         int32_t max_start, int32_t chunk_len, const float *q_abs,
                         const float *v_new, const float *kr_raw, float scale, const float *out) {
  gva_status st = check_dims(d);
  if (st != GVA_OK) return st;
  if ((st = check_cache(d, c)) != GVA_OK) return st;
  if (B < 1) return fail(GVA_ERR_INVALID_ARG, "B=%d must be >= 1", B);
  if (chunk_len < 0) return fail(GVA_ERR_INVALID_ARG, "chunk_len=%d must be >= 0", chunk_len);
  if (max_start < 0) return fail(GVA_ERR_INVALID_ARG, "max_start=%d must be >= 0", max_start);
  if ((int64_t)max_start + chunk_len > (int64_t)c->max_blocks * c->block_size)
    return fail(GVA_ERR_INVALID_ARG, "max_start + chunk_len exceeds the block table's capacity");
  if (chunk_len == 0) return GVA_OK;
  if (!start || !q_abs || !v_new || !kr_raw || !out)
    return fail(GVA_ERR_INVALID_ARG, "prefill argument is NULL");
  if (!aligned(q_abs, 16) || !aligned(out, 16) || !aligned(v_new, 8) || !aligned(kr_raw, 8))
    return fail(GVA_ERR_INVALID_ARG, "prefill buffers misaligned");
  if (!(scale > 0.0f) || !isfinite(scale))
    return fail(GVA_ERR_INVALID_ARG, "scale must be positive and finite");
  const char *why = nullptr;
  if (!mfma_supported(d, c, &why)) return fail(GVA_ERR_UNSUPPORTED, "%s", why);
  return GVA_OK;
}

}  // namespace gva

extern "C" {

size_t gva_rope_table_bytes(int32_t max_pos, int32_t d_r) {
  if (max_pos < 1 || d_r < 2 || d_r % 2 != 0 || d_r > gva::kMaxDn) return 0;
  return (size_t)max_pos * (size_t)(d_r / 2) * 2 * sizeof(double);
}

gva_status gva_rope_table_fill(double *host_out, int32_t max_pos, int32_t d_r, double base) {
  if (!host_out) return gva::fail(GVA_ERR_INVALID_ARG, "host_out is NULL");
  if (max_pos < 1) return gva::fail(GVA_ERR_INVALID_ARG, "max_pos=%d must be >= 1", max_pos);
  // d_r is the rotated width: the positional slice's d_r, or d_n for the comparator's keys
  if (d_r < 2 || d_r % 2 != 0 || d_r > gva::kMaxDn)
    return gva::fail(GVA_ERR_INVALID_ARG, "width=%d must be even and in [2, %d]", d_r, gva::kMaxDn);
  if (!(base > 0.0) || !isfinite(base)) return gva::fail(GVA_ERR_INVALID_ARG, "base must be > 0");
  const int half = d_r / 2;
  for (int i = 0; i < half; ++i) {
    // theta_i = base^(-2i/d_r): the exponent is the correctly rounded quotient (-2i)/d_r.
    const double theta = gva::g_libm_pow(base, (-2.0 * (double)i) / (double)d_r);
    for (int32_t p = 0; p < max_pos; ++p) {
      const double a = (double)p * theta;
      host_out[((size_t)p * half + i) * 2 + 0] = gva::g_libm_cos(a);
      host_out[((size_t)p * half + i) * 2 + 1] = gva::g_libm_sin(a);
    }
  }
  return GVA_OK;
}

size_t gva_decode_workspace_bytes(const gva_dims *dims, int32_t B, int32_t max_len,
                                  int32_t num_splits) {
  if (gva::check_dims(dims) != GVA_OK) return 0;
  // enough for either kernel's plan (the cache decides which one runs), and for the GQA
  // comparator's balanced plan
  gva::DecodePlan p, pb, pq;
  if (!gva::plan_decode(dims, B, max_len, num_splits, false, &p)) return 0;
  if (!gva::plan_decode(dims, B, max_len, num_splits, true, &pb)) return 0;
  if (!gva::plan_decode(dims, B, max_len, num_splits, true, &pq, false)) return 0;
  size_t ws = p.ws_bytes > pb.ws_bytes ? p.ws_bytes : pb.ws_bytes;
  ws = ws > pq.ws_bytes ? ws : pq.ws_bytes;
  // the one-launch decode step's partials and tickets
  gva::StepPlan sp;
  if (num_splits == 0 && gva::plan_step(dims, B, max_len, &sp) && sp.ws_bytes > ws) ws = sp.ws_bytes;
  return ws;
}

size_t gva_recon_decode_workspace_bytes(const gva_dims *dims, int32_t B, int32_t max_len,
                                        int32_t num_splits) {
  if (!dims) return 0;
  gva_dims dd = *dims;
  dd.d_r = 2;                              // not used by the comparator
  if (gva::check_dims(&dd) != GVA_OK) return 0;
  gva::DecodePlan p;
  if (!gva::plan_decode(&dd, B, max_len, num_splits, false, &p)) return 0;
  return p.ws_bytes;
}

size_t gva_mla_decode_workspace_bytes(const gva_dims *dims, int32_t B, int32_t max_len,
                                      int32_t num_splits) {
  if (!dims || dims->G != 1 || dims->H < 1) return 0;
  gva::DecodePlan p;
  if (!gva::plan_decode(dims, B, max_len, num_splits, false, &p)) return 0;
  gva::add_latent_queue(&p);
  return p.ws_bytes;
}

int32_t gva_decode_num_splits(const gva_dims *dims, int32_t B, int32_t max_len,
                              int32_t num_splits) {
  if (gva::check_dims(dims) != GVA_OK) return 0;
  gva::DecodePlan p;
  if (!gva::plan_decode(dims, B, max_len, num_splits, false, &p)) return 0;
  return p.num_splits;
}

int32_t gva_decode_step_launches(const gva_dims *dims, const gva_cache *cache, int32_t B,
                                 int32_t max_len, int32_t num_splits, int32_t kernel) {
  if (gva::check_dims(dims) != GVA_OK || gva::check_cache(dims, cache) != GVA_OK) return 0;
  if (B < 1 || max_len < 0 || num_splits < 0 || num_splits > gva::kMaxSplits) return 0;
  if (kernel < GVA_KERNEL_AUTO || kernel > GVA_KERNEL_MFMA) return 0;
  const bool can = gva::mfma_supported(dims, cache, nullptr);
  if (kernel == GVA_KERNEL_MFMA && !can) return 0;
  const bool use_mfma = kernel == GVA_KERNEL_MFMA || (kernel == GVA_KERNEL_AUTO && can);
  if (gva::step_fused_supported(dims, cache, B, max_len, num_splits, use_mfma)) return 1;
  if (gva::step_small_supported(dims, cache, B, max_len, num_splits, use_mfma)) return 1;
  gva::DecodePlan plan;
  if (!gva::plan_decode(dims, B, max_len, num_splits, use_mfma, &plan)) return 0;
  return (plan.num_splits > 1 || plan.num_ranges > 0) ? 3 : 2;  // merged: no combine
}

int32_t gva_decode_num_ranges(const gva_dims *dims, int32_t B, int32_t max_len) {
  if (gva::check_dims(dims) != GVA_OK) return 0;
  gva::DecodePlan p;
  if (!gva::plan_decode(dims, B, max_len, 0, true, &p)) return 0;
  return p.num_ranges;
}

const char *gva_status_string(gva_status status) {
  switch (status) {
    case GVA_OK: return "GVA_OK";
    case GVA_ERR_INVALID_ARG: return "GVA_ERR_INVALID_ARG";
    case GVA_ERR_UNSUPPORTED: return "GVA_ERR_UNSUPPORTED";
    case GVA_ERR_WORKSPACE: return "GVA_ERR_WORKSPACE";
    case GVA_ERR_HIP: return "GVA_ERR_HIP";
  }
  return "GVA_ERR_UNKNOWN";
}

const char *gva_last_error(void) { return gva::last_error_cstr(); }

const char *gva_version(void) { return "gva-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
