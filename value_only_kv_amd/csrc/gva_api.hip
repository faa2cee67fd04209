// gva_api.hip - the extern "C" entry points of the GVA library: validate on the host (no HIP
// call before the arguments are known good), plan, then launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>
#include <mutex>

#include "gva_internal.h"

// Scratch of the allocation-free decode (gva_decode_noalloc): its split partials. Each device
// that runs the library holds its own copy until the process ends. In host code this name is
// only a stand-in for the symbol; the device address comes from hipGetSymbolAddress (below).
static __device__ __align__(256) uint8_t scratch[GVA_NOALLOC_SCRATCH_BYTES];

namespace {

// The address of `scratch` on each device, looked up once per device on the first
// gva_decode_noalloc call made with that device current.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

gva::DecodeArgs cache_args(const gva_dims *d, const gva_cache *c) {
  gva::DecodeArgs a{};
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
  gva::group_order(d, a.head_of);
  return a;
}

gva_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return GVA_OK;
  return gva::fail(GVA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Zeroes the first n words at p (one work-group).
__global__ void k_zero_words(uint32_t *p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// Device address of this device's `scratch` (looked up on first use, then cached). The first
// lookup on a device also clears the tickets at the head of the array (zero already, as a
// static array, and left at zero by every call), in order on `stream` before the caller's
// launches.
gva_status device_scratch(void **out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return gva::fail(GVA_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table covers", dev,
                     kMaxDevices);
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
      if (!p) return gva::fail(GVA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
      hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(256), 0, stream, static_cast<uint32_t *>(p),
                         static_cast<int>(gva::kWsHeader / 4));
      e = hipGetLastError();
      if (e != hipSuccess) return hip_status(e, "scratch ticket clear launch");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return GVA_OK;
}

// Decode + combine launches for a checked call and its plan.
gva_status launch_decode(const gva_dims *dims, const gva_cache *cache, int32_t B,
                         const int32_t *seq_len, int32_t max_len, const float *q_abs, float scale,
                         const gva::DecodePlan &plan, bool use_mfma, void *workspace, float *out,
                         float *lse, hipStream_t stream) {
  gva::DecodeArgs a = cache_args(dims, cache);
  a.B = B;
  a.seq_len = seq_len;
  a.max_len = max_len;
  a.q_abs = q_abs;
  a.qscale = scale * 1.4426950408889634f;
  if (plan.merged_K > 0) {
    // small batch: decode and merge in one launch (tickets and partials in the workspace)
    gva::StepArgs sa{};
    sa.a = a;
    sa.a.out = out;
    sa.a.lse = lse;
    sa.K = plan.merged_K;
    sa.tiles_per_wave = plan.tiles_per_wave;
    if (plan.merged_K > 1) {
      char *ws = static_cast<char *>(workspace);
      sa.ticket = reinterpret_cast<int32_t *>(ws);
      sa.part_o = reinterpret_cast<float *>(ws + plan.off_o);
      sa.part_m = reinterpret_cast<float *>(ws + plan.off_m);
      sa.part_l = reinterpret_cast<float *>(ws + plan.off_l);
    }
    return hip_status(gva::launch_decode_merged(sa, stream), "merged decode launch");
  }
  a.num_splits = plan.num_splits;
  a.chunk = plan.chunk;
  a.num_ranges = plan.num_ranges;
  a.out = out;
  a.lse = lse;
  const bool partials = plan.num_splits > 1 || plan.num_ranges > 0;
  if (partials) {
    char *ws = static_cast<char *>(workspace);
    a.part_o = reinterpret_cast<float *>(ws + plan.off_o);
    a.part_m = reinterpret_cast<float *>(ws + plan.off_m);
    a.part_l = reinterpret_cast<float *>(ws + plan.off_l);
    if (plan.num_ranges > 0) a.tile_prefix = reinterpret_cast<int32_t *>(ws + plan.off_prefix);
  }
  hipError_t e = use_mfma ? gva::launch_decode_mfma(a, stream)
                          : gva::launch_decode_generic(a, cache->dtype == GVA_DTYPE_BF16, stream);
  if (e != hipSuccess) return hip_status(e, "decode launch");
  if (partials) {
    e = gva::launch_combine(a, stream);
    if (e != hipSuccess) return hip_status(e, "combine launch");
  }
  return GVA_OK;
}

}  // namespace

extern "C" {

gva_status gva_cache_append(const gva_dims *dims, const gva_cache *cache, int32_t B,
                            int32_t n_tok, const int32_t *seq, const int32_t *pos,
                            const float *v_new, const float *kr_raw, hipStream_t stream) {
  gva_status st = gva::check_append(dims, cache, B, n_tok, seq, pos, v_new, kr_raw);
  if (st != GVA_OK) return st;
  return hip_status(gva::launch_append(dims, cache, B, n_tok, seq, pos, v_new, kr_raw, stream),
                    "cache append launch");
}

gva_status gva_absorb_query(const gva_dims *dims, int32_t n_q, const float *q_nope,
                            const float *q_rope, const int32_t *q_pos, const float *M,
                            const double *rope, int32_t max_pos, float *q_abs,
                            int32_t *err_flag, hipStream_t stream) {
  gva_status st = gva::check_absorb(dims, n_q, q_nope, q_rope, q_pos, M, rope, max_pos, q_abs);
  if (st != GVA_OK) return st;
  return hip_status(gva::launch_absorb(dims, n_q, q_nope, q_rope, q_pos, M, rope, max_pos, q_abs,
                                       err_flag, stream),
                    "absorb launch");
}

gva_status gva_decode(const gva_dims *dims, const gva_cache *cache, int32_t B,
                      const int32_t *seq_len, int32_t max_len, const float *q_abs, float scale,
                      int32_t num_splits, int32_t kernel, void *workspace,
                      size_t workspace_bytes, float *out, float *lse, hipStream_t stream) {
  gva::DecodePlan plan{};
  bool use_mfma = false;
  gva_status st = gva::check_decode(dims, cache, B, seq_len, max_len, q_abs, scale, num_splits,
                                    kernel, workspace, workspace_bytes, out, &plan, &use_mfma);
  if (st != GVA_OK) return st;
  return launch_decode(dims, cache, B, seq_len, max_len, q_abs, scale, plan, use_mfma, workspace,
                       out, lse, stream);
}

gva_status gva_decode_noalloc(const gva_dims *dims, const gva_cache *cache, int32_t B,
                              const int32_t *seq_len, int32_t max_len, const float *q_abs,
                              float scale, int32_t num_splits, int32_t kernel, float *out,
                              float *lse, hipStream_t stream) {
  // Validate against a stand-in workspace of unlimited size (never dereferenced), then check
  // the plan's partials against the static scratch; both before any HIP call.
  gva::DecodePlan plan{};
  bool use_mfma = false;
  void *const stand_in = reinterpret_cast<void *>(uintptr_t{256});
  gva_status st = gva::check_decode(dims, cache, B, seq_len, max_len, q_abs, scale, num_splits,
                                    kernel, stand_in, SIZE_MAX, out, &plan, &use_mfma);
  if (st != GVA_OK) return st;
  if (plan.ws_bytes > GVA_NOALLOC_SCRATCH_BYTES)
    return gva::fail(GVA_ERR_WORKSPACE,
                     "gva_decode_noalloc: this plan needs %zu bytes of partials, above the %zu "
                     "bytes of static scratch; call gva_decode with a workspace instead",
                     plan.ws_bytes, static_cast<size_t>(GVA_NOALLOC_SCRATCH_BYTES));
  void *ws = nullptr;
  if (plan.ws_bytes > 0) {
    st = device_scratch(&ws, stream);
    if (st != GVA_OK) return st;
  }
  return launch_decode(dims, cache, B, seq_len, max_len, q_abs, scale, plan, use_mfma, ws, out,
                       lse, stream);
}

gva_status gva_decode_step(const gva_dims *dims, const gva_cache *cache, int32_t B,
                           const int32_t *pos, const float *v_new, const float *kr_raw,
                           const float *q_nope, const float *q_rope, const float *M,
                           const int32_t *seq_len, int32_t max_len, float scale,
                           int32_t num_splits, int32_t kernel, float *q_abs, void *workspace,
                           size_t workspace_bytes, float *out, float *lse, hipStream_t stream) {
  gva_status st = gva::check_step(dims, cache, B, pos, v_new, kr_raw, q_nope, q_rope, M, q_abs);
  if (st != GVA_OK) return st;
  gva::DecodePlan plan{};
  bool use_mfma = false;
  st = gva::check_decode(dims, cache, B, seq_len, max_len, q_abs, scale, num_splits, kernel,
                         workspace, workspace_bytes, out, &plan, &use_mfma);
  if (st != GVA_OK) return st;
  gva::StepPlan sp{};
  if (gva::step_fused_supported(dims, cache, B, max_len, num_splits, use_mfma) &&
      gva::plan_step(dims, B, max_len, &sp)) {
    // small batch: the whole step in one launch, K work-groups per (sequence, group)
    if (sp.ws_bytes > 0) {
      if (!workspace || workspace_bytes < sp.ws_bytes)
        return gva::fail(GVA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", sp.ws_bytes,
                         workspace ? workspace_bytes : (size_t)0);
      if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return gva::fail(GVA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }
    gva::StepArgs sa{};
    sa.a = cache_args(dims, cache);
    sa.a.B = B;
    sa.a.seq_len = seq_len;
    sa.a.max_len = max_len;
    sa.a.qscale = scale * 1.4426950408889634f;
    sa.a.out = out;
    sa.a.lse = lse;
    sa.pos = pos;
    sa.v_new = v_new;
    sa.kr_raw = kr_raw;
    sa.q_nope = q_nope;
    sa.q_rope = q_rope;
    sa.M = M;
    sa.rope = cache->rope;
    sa.max_pos = cache->max_pos;
    sa.d_n = dims->d_n;
    sa.q_abs = q_abs;
    sa.K = sp.K;
    {
      const int64_t kw = static_cast<int64_t>(sp.K) * gva::step_waves_of(dims->d_h);
      const int64_t tiles = (static_cast<int64_t>(max_len) + gva::kTilePositions - 1) / gva::kTilePositions;
      sa.tiles_per_wave = static_cast<int32_t>((tiles + kw - 1) / kw);
    }
    if (sp.K > 1) {
      char *ws = static_cast<char *>(workspace);
      sa.ticket = reinterpret_cast<int32_t *>(ws);
      sa.part_o = reinterpret_cast<float *>(ws + sp.off_po);
      sa.part_m = reinterpret_cast<float *>(ws + sp.off_pm);
      sa.part_l = reinterpret_cast<float *>(ws + sp.off_pl);
    }
    return hip_status(gva::launch_step_fused(sa, stream), "one-launch decode step");
  }
  if (gva::step_small_supported(dims, cache, B, max_len, num_splits, use_mfma)) {
    // small batch on the vector-ALU path: the whole step in one launch, one work-group per
    // (sequence, group), no workspace
    gva::StepArgs sa{};
    sa.a = cache_args(dims, cache);
    sa.a.B = B;
    sa.a.seq_len = seq_len;
    sa.a.max_len = max_len;
    sa.a.qscale = scale * 1.4426950408889634f;
    sa.a.out = out;
    sa.a.lse = lse;
    sa.pos = pos;
    sa.v_new = v_new;
    sa.kr_raw = kr_raw;
    sa.q_nope = q_nope;
    sa.q_rope = q_rope;
    sa.M = M;
    sa.rope = cache->rope;
    sa.max_pos = cache->max_pos;
    sa.d_n = dims->d_n;
    sa.q_abs = q_abs;
    sa.K = 1;
    return hip_status(gva::launch_step_small(sa, cache->dtype == GVA_DTYPE_BF16, stream),
                      "one-launch decode step (vector ALU)");
  }
  hipError_t e = gva::launch_step_prep(cache_args(dims, cache), cache->dtype == GVA_DTYPE_BF16, B,
                                       pos, v_new, kr_raw, cache->rope, cache->max_pos, dims->d_n,
                                       q_nope, q_rope, M, q_abs, stream);
  if (e != hipSuccess) return hip_status(e, "step append and absorb launch");
  return launch_decode(dims, cache, B, seq_len, max_len, q_abs, scale, plan, use_mfma, workspace,
                       out, lse, stream);
}

gva_status gva_gqa_decode(const gva_dims *dims, const gva_cache *values, const void *keys,
                          int32_t B, const int32_t *seq_len, int32_t max_len, const float *q,
                          float scale, void *workspace, size_t workspace_bytes, float *out,
                          float *lse, hipStream_t stream) {
  if (!keys || reinterpret_cast<uintptr_t>(keys) % 16 != 0)
    return gva::fail(GVA_ERR_INVALID_ARG, "keys must be a 16-byte aligned device pointer");
  gva::DecodePlan plan{};
  bool use_mfma = false;
  gva_status st = gva::check_decode(dims, values, B, seq_len, max_len, q, scale, 0,
                                    GVA_KERNEL_MFMA, workspace, workspace_bytes, out, &plan,
                                    &use_mfma, false);
  if (st != GVA_OK) return st;
  gva::DecodeArgs a = cache_args(dims, values);
  a.k = keys;
  a.d_r = 0;                          // the query rows are [q_h] (d_h wide), no positional part
  a.B = B;
  a.seq_len = seq_len;
  a.max_len = max_len;
  a.q_abs = q;
  a.qscale = scale * 1.4426950408889634f;
  a.num_splits = plan.num_splits;
  a.chunk = plan.chunk;
  a.num_ranges = plan.num_ranges;
  a.out = out;
  a.lse = lse;
  const bool partials = plan.num_splits > 1 || plan.num_ranges > 0;
  if (partials) {
    char *ws = static_cast<char *>(workspace);
    a.part_o = reinterpret_cast<float *>(ws + plan.off_o);
    a.part_m = reinterpret_cast<float *>(ws + plan.off_m);
    a.part_l = reinterpret_cast<float *>(ws + plan.off_l);
    if (plan.num_ranges > 0) a.tile_prefix = reinterpret_cast<int32_t *>(ws + plan.off_prefix);
  }
  hipError_t e = gva::launch_decode_mfma(a, stream);
  if (e != hipSuccess) return hip_status(e, "comparator decode launch");
  if (partials) {
    e = gva::launch_combine(a, stream);
    if (e != hipSuccess) return hip_status(e, "combine launch");
  }
  return GVA_OK;
}

gva_status gva_recon_decode(const gva_dims *dims, const gva_cache *values, int32_t B,
                            const int32_t *seq_len, int32_t max_len, const float *q,
                            const int32_t *q_pos, const uint16_t *Mt, const double *rope,
                            int32_t max_pos, float scale, int32_t num_splits, void *workspace,
                            size_t workspace_bytes, float *out, float *lse, hipStream_t stream) {
  gva::DecodePlan plan{};
  gva_status st = gva::check_recon(dims, values, B, seq_len, max_len, q, q_pos, Mt, rope, max_pos,
                                   scale, num_splits, workspace, workspace_bytes, out, &plan);
  if (st != GVA_OK) return st;
  gva::ReconArgs r{};
  r.kv = cache_args(dims, values);
  r.kv.kr = nullptr;
  r.kv.d_r = 0;
  r.kv.B = B;
  r.kv.seq_len = seq_len;
  r.kv.max_len = max_len;
  r.kv.qscale = scale * 1.4426950408889634f;
  r.kv.num_splits = plan.num_splits;
  r.kv.chunk = plan.chunk;
  r.kv.out = out;
  r.kv.lse = lse;
  if (plan.num_splits > 1) {
    char *ws = static_cast<char *>(workspace);
    r.kv.part_o = reinterpret_cast<float *>(ws + plan.off_o);
    r.kv.part_m = reinterpret_cast<float *>(ws + plan.off_m);
    r.kv.part_l = reinterpret_cast<float *>(ws + plan.off_l);
  }
  r.d_n = dims->d_n;
  r.q = q;
  r.q_pos = q_pos;
  r.Mt = Mt;
  r.rope = rope;
  r.max_pos = max_pos;
  hipError_t e = gva::launch_recon_decode(r, stream);
  if (e != hipSuccess) return hip_status(e, "comparator decode launch");
  if (plan.num_splits > 1) {
    e = gva::launch_combine(r.kv, stream);
    if (e != hipSuccess) return hip_status(e, "combine launch");
  }
  return GVA_OK;
}

gva_status gva_mla_decode(const gva_dims *dims, const gva_cache *latent, int32_t B,
                          const int32_t *seq_len, int32_t max_len, const float *q_abs,
                          float scale, int32_t num_splits, void *workspace,
                          size_t workspace_bytes, float *out, float *lse, hipStream_t stream) {
  gva::DecodePlan plan{};
  gva_status st = gva::check_latent(dims, latent, B, seq_len, max_len, q_abs, scale, num_splits,
                                    workspace, workspace_bytes, out, &plan);
  if (st != GVA_OK) return st;
  gva::DecodeArgs a = cache_args(dims, latent);
  a.B = B;
  a.seq_len = seq_len;
  a.max_len = max_len;
  a.q_abs = q_abs;
  a.qscale = scale * 1.4426950408889634f;
  a.num_splits = plan.num_splits;
  a.chunk = plan.chunk;
  a.out = out;
  a.lse = lse;
  char *ws = static_cast<char *>(workspace);
  if (plan.num_splits > 1) {
    a.part_o = reinterpret_cast<float *>(ws + plan.off_o);
    a.part_m = reinterpret_cast<float *>(ws + plan.off_m);
    a.part_l = reinterpret_cast<float *>(ws + plan.off_l);
  }
  a.work_next = reinterpret_cast<int32_t *>(ws + plan.off_queue);
  hipError_t e = gva::launch_latent_decode(a, stream);
  if (e != hipSuccess) return hip_status(e, "latent comparator decode launch");
  if (plan.num_splits > 1) {
    e = gva::launch_combine(a, stream);
    if (e != hipSuccess) return hip_status(e, "combine launch");
  }
  return GVA_OK;
}

gva_status gva_prefill_chunk(const gva_dims *dims, const gva_cache *cache, int32_t B,
                             const int32_t *start, int32_t max_start, int32_t chunk_len,
                             const float *q_abs, const float *v_new, const float *kr_raw,
                             float scale, float *out, float *lse, hipStream_t stream) {
  gva_status st = gva::check_prefill(dims, cache, B, start, max_start, chunk_len, q_abs, v_new,
                                     kr_raw, scale, out);
  if (st != GVA_OK) return st;
  if (chunk_len == 0) return GVA_OK;
  gva::PrefillArgs p{};
  p.kv = cache_args(dims, cache);
  p.kv.B = B;
  p.kv.qscale = scale * 1.4426950408889634f;
  p.start = start;
  p.max_start = max_start;
  p.chunk_len = chunk_len;
  p.q_abs = q_abs;
  p.out = out;
  p.lse = lse;
  p.v_new = v_new;
  p.kr_raw = kr_raw;
  p.rope = cache->rope;
  p.max_pos = cache->max_pos;
  return hip_status(gva::launch_prefill(p, stream), "prefill launch");
}

}  // extern "C"
