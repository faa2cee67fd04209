// gva_internal.h - declarations shared by the host-side validation/planning code (plain C++,
// no HIP device code) and the HIP entry points and kernel launchers.
#ifndef GVA_INTERNAL_H_
#define GVA_INTERNAL_H_

#include <stddef.h>
#include <stdint.h>

#include "gva.h"

namespace gva {

// Compute units assumed when planning a split count (MI355X: 256 CUs in 8 XCDs). A fixed
// value keeps gva_decode_workspace_bytes a pure function of its arguments.
constexpr int kPlanCUs = 256;
// Token granularity of a decode chunk: both decode kernels walk a chunk in tiles of this many
// positions, so chunk boundaries fall on tile boundaries.
constexpr int kChunkQuantum = 64;
// Balanced mode: work-groups the automatic plan fills the device with (3 resident four-wave
// work-groups on each of kPlanCUs compute units), and the fewest tiles a range should hold.
constexpr int kBalancedWorkGroups = 3 * kPlanCUs;
constexpr int kMinTilesPerRange = 32;
constexpr int kTilePositions = 32;
// Waves (value groups) per work-group of the matrix-core decode kernel: the largest divisor of
// G that is at most 4. Four lets three work-groups share a CU (one wave per SIMD each) when the
// kernel fits in 168 registers, which one 8-wave work-group per CU cannot use.
constexpr int kDecodeGroupWaves = 4;
inline int decode_waves_per_group(int G) {
  for (int w = kDecodeGroupWaves; w > 1; --w)
    if (G % w == 0) return w;
  return 1;
}
// The balanced plan of the GVA decode (not the GQA comparator) with G a multiple of 8 and
// enough tiles for ranges of kMinTilesPerRange tiles runs 8-wave work-groups, one per CU: the
// eight value groups of a range share one work-group, so its shared positional key is read from
// HBM once (by one wave, into LDS) instead of once per wave. Smaller batches (a few tiles per
// range, where the per-tile barrier costs more than the key's bytes) and other G use the
// four-wave layout above, three work-groups per CU. tiles_max = B * ceil(max_len / 32).
constexpr int kSharedKeyWaves = 8;
struct BalancedLayout {
  int waves;            // waves (value groups) per work-group
  int groups_per_cu;    // resident work-groups per CU the plan fills
};
inline BalancedLayout balanced_layout(int G, bool share_key, int64_t tiles_max) {
  if (share_key && G % kSharedKeyWaves == 0 &&
      tiles_max >= static_cast<int64_t>(kPlanCUs) * kMinTilesPerRange)
    return {kSharedKeyWaves, 1};
  return {decode_waves_per_group(G), kBalancedWorkGroups / kPlanCUs};
}
constexpr int kMaxSplits = 1024;
constexpr int kMaxH = 256;
constexpr int kMaxDh = 256;
constexpr int kMaxDn = 512;
constexpr int kMaxDr = 64;

const char *last_error_cstr();
// Records `detail` as the calling thread's last error and returns `status`.
gva_status fail(gva_status status, const char *fmt, ...);

// Argument checks. None of them touches HIP, so they run (and are tested) without a GPU.
gva_status check_dims(const gva_dims *d);
// Fills head_of[0 .. H) with the heads in group order (see DecodeArgs::head_of) for checked dims.
void group_order(const gva_dims *d, uint8_t *head_of);
gva_status check_cache(const gva_dims *d, const gva_cache *c);
gva_status check_append(const gva_dims *d, const gva_cache *c, int32_t B, int32_t n_tok,
                        const int32_t *seq, const int32_t *pos, const float *v_new,
                        const float *kr_raw);
gva_status check_absorb(const gva_dims *d, int32_t n_q, const float *q_nope, const float *q_rope,
                        const int32_t *q_pos, const float *M, const double *rope, int32_t max_pos,
                        const float *q_abs);

// Does the matrix-core decode/prefill kernel handle this shape and cache? (No HIP calls.)
bool mfma_supported(const gva_dims *d, const gva_cache *c, const char **why);

struct DecodePlan {
  int32_t num_splits;   // split grid: chunks per sequence (0 in balanced mode)
  int32_t chunk;        // split grid: positions per chunk, a multiple of kChunkQuantum
  int32_t num_ranges;   // balanced mode: equal ranges over all sequences' tiles (0: split grid)
  size_t ws_bytes;      // workspace needed (0 when num_splits == 1: output written directly)
  size_t off_m;         // byte offsets of the partial arrays inside the workspace
  size_t off_l;
  size_t off_o;
  size_t off_prefix;    // balanced mode: the per-sequence tile prefix, int32 [B + 1]
  size_t off_queue;     // latent comparator: its work queue's counter (256 bytes at the end)
  // merged mode (small batches): merged_K work-groups per (sequence, group) decode runs of
  // tiles_per_wave tiles each and merge their partials in the same launch (the one-launch
  // step's layout: tickets in the header, partials at off_o, off_m, off_l); 0 otherwise
  int32_t merged_K;
  int32_t tiles_per_wave;
};
// The latent comparator's workspace: the split plan's partials, then one 256-byte word for the
// counter of its work queue (so it is never empty).
void add_latent_queue(DecodePlan *plan);

// Plans the split of positions [0, max_len) into chunks (balanced == false), or, for the
// matrix-core kernel's automatic mode (balanced == true), the merged plan when the batch is
// small (B * G <= kPlanCUs, share_key, a shape decode_merged_supported takes) else the cut of
// all sequences' 32-position tiles into equal ranges; returns false on bad arguments.
bool plan_decode(const gva_dims *d, int32_t B, int32_t max_len, int32_t num_splits,
                 bool balanced, DecodePlan *plan, bool share_key = true);

gva_status check_decode(const gva_dims *d, const gva_cache *c, int32_t B,
                        const int32_t *seq_len, int32_t max_len, const float *q_abs,
                        float scale, int32_t num_splits, int32_t kernel, const void *workspace,
                        size_t workspace_bytes, const float *out, DecodePlan *plan,
                        bool *use_mfma, bool share_key = true);

// The append and absorption parts of a decode step: token b goes to sequence b at pos[b], and
// query b is absorbed at the same position with the cache's RoPE table.
gva_status check_step(const gva_dims *d, const gva_cache *c, int32_t B, const int32_t *pos,
                      const float *v_new, const float *kr_raw, const float *q_nope,
                      const float *q_rope, const float *M, const float *q_abs);

// The non-absorbable comparator (gva_recon_decode): shapes it implements, and its argument
// checks; the plan is the split grid of plan_decode.
bool recon_supported(const gva_dims *d, const char **why);
gva_status check_recon(const gva_dims *d, const gva_cache *c, int32_t B, const int32_t *seq_len,
                       int32_t max_len, const float *q, const int32_t *q_pos, const uint16_t *Mt,
                       const double *rope, int32_t max_pos, float scale, int32_t num_splits,
                       const void *workspace, size_t workspace_bytes, const float *out,
                       DecodePlan *plan);

// The MLA-style latent comparator (gva_mla_decode): one group (G = 1) whose value is the
// latent, d_h = d_c in {256, 512}, H in {8, 16, 32}; the plan is the split grid of plan_decode.
gva_status check_latent(const gva_dims *d, const gva_cache *c, int32_t B, const int32_t *seq_len,
                        int32_t max_len, const float *q_abs, float scale, int32_t num_splits,
                        const void *workspace, size_t workspace_bytes, const float *out,
                        DecodePlan *plan);

gva_status check_prefill(const gva_dims *d, const gva_cache *c, int32_t B, const int32_t *start,
                         int32_t max_start, int32_t chunk_len, const float *q_abs,
                         const float *v_new, const float *kr_raw, float scale, const float *out);

// ---- kernel launchers (defined in the .hip files) -------------------------------------------

struct DecodeArgs {
  // cache
  const void *v;
  const void *kr;
  const void *k;        // GQA comparator only: key pool, same layout as v (nullptr for GVA)
  int64_t v_sb, v_st, v_sg, kr_sb, kr_st;
  int64_t num_blocks;
  int32_t log2_bs;
  int32_t max_blocks;
  const int32_t *block_table;
  int32_t *err_flag;
  // shape
  int32_t H, G, d_h, d_r;
  int32_t B;
  const int32_t *seq_len;
  int32_t max_len;
  const float *q_abs;
  float qscale;         // softmax scale * log2(e): scores are kept in the base-2 domain
  int32_t num_splits;
  int32_t chunk;
  int32_t num_ranges;   // > 0: balanced mode (matrix-core kernel), see plan_decode
  int32_t *tile_prefix; // balanced mode: [B + 1], written by the decode kernel
  // outputs: partials (num_splits > 1, or balanced mode) or final rows (num_splits == 1)
  float *part_m;        // split grid [B][S][H]; balanced mode [R + B][H]
  float *part_l;        // same rows as part_m
  float *part_o;        // same rows as part_m, [d_h] each
  float *out;           // [B][H][d_h]
  float *lse;           // [B][H] or nullptr
  int32_t *work_next;   // latent comparator: the work queue's counter (zeroed before the launch)
  // Heads in group order: slot g * (H / G) + c holds the c-th head (in ascending order) of value
  // group g, so a kernel that serves group g reads the heads of slots g * (H / G) ...
  // (whole-word aligned, so a kernel can read a group's slots as aligned 32-bit words).
  alignas(4) uint8_t head_of[kMaxH];
};

hipError_t launch_append(const gva_dims *d, const gva_cache *c, int32_t B, int32_t n_tok,
                         const int32_t *seq, const int32_t *pos, const float *v_new,
                         const float *kr_raw, hipStream_t stream);
hipError_t launch_absorb(const gva_dims *d, int32_t n_q, const float *q_nope, const float *q_rope,
                         const int32_t *q_pos, const float *M, const double *rope,
                         int32_t max_pos, float *q_abs, int32_t *err_flag, hipStream_t stream);
// One launch: append token b to sequence b at pos[b] (b < B) and absorb query b at pos[b].
hipError_t launch_step_prep(const DecodeArgs &a, bool bf16, int32_t B, const int32_t *pos,
                            const float *v_new, const float *kr_raw, const double *rope,
                            int32_t max_pos, int32_t d_n, const float *q_nope, const float *q_rope,
                            const float *M, float *q_abs, hipStream_t stream);
// The decode step in one launch (small batches): one work-group per (sequence, value group)
// appends the sequence's token for its group, forms the absorbed queries of its group's heads,
// decodes with its waves splitting the positions, and merges their partials itself.
struct StepArgs {
  DecodeArgs a;           // cache, shape, seq_len, max_len, qscale, out, lse, head_of
  const int32_t *pos;     // [B]: position of the new token
  const float *v_new;     // [B][G][d_h]
  const float *kr_raw;    // [B][d_r]
  const float *q_nope;    // [B][H][d_n]
  const float *q_rope;    // [B][H][d_r]
  const float *M;         // [H][d_h][d_n]
  const double *rope;     // [max_pos][d_r / 2][2]
  int32_t max_pos;
  int32_t d_n;
  float *q_abs;           // [B][H][d_h + d_r], written
  int32_t K;              // work-groups per (sequence, group)
  int32_t tiles_per_wave; // runs of this many 32-position tiles, cut from max_len
  float *part_o;          // K > 1: per work-group partials (device scope, write-through)
  float *part_m;
  float *part_l;
  int32_t *ticket;        // K > 1: [B][G], zero between calls
};
// Whether the one-launch step serves these arguments: the matrix-core kernel's shapes with
// d_h of 32 or 64 and H / G of 1, 2, 4 or 8, at most kPlanCUs (sequence, group) pairs, at most
// 4 MiB of values per group, and the automatic split count.
bool step_fused_supported(const gva_dims *d, const gva_cache *c, int32_t B, int32_t max_len,
                          int32_t num_splits, bool use_mfma);
// Whether the one-launch step of the vector-ALU path serves these arguments: shapes the
// matrix-core kernel does not take (float32 caches among them) with H / G of 1, 2, 4 or 8, at
// most kPlanCUs (sequence, group) pairs, sequences of at most kSmallMaxLen positions, the
// automatic split count, and the group's rows of M (with q_nope) within kSmallRegionBytes.
constexpr int kSmallMaxLen = 1024;
constexpr int kSmallRegionBytes = 72 * 1024;
bool step_small_supported(const gva_dims *d, const gva_cache *c, int32_t B, int32_t max_len,
                          int32_t num_splits, bool use_mfma);
hipError_t launch_step_small(const StepArgs &s, bool bf16, hipStream_t stream);
// Waves per work-group of the one-launch step (two per SIMD, so up to 256 registers each).
inline int step_waves_of(int d_h) { (void)d_h; return 8; }
// The first kWsHeader bytes of a decode workspace hold the one-launch step's tickets, one int32
// per (sequence, group); they must be zero before a workspace's first use, each call leaves them
// at zero, and no plan writes partials there.
constexpr size_t kWsHeader = 1024;
// The one-launch step splits each (sequence, group) over K work-groups (K * B * G <= kPlanCUs,
// at least one tile per wave); with K > 1 they meet through partials at off_part and the
// tickets of the header.
struct StepPlan {
  int32_t K;
  size_t off_po, off_pm, off_pl;  // partial o [slot][NH][d_h], m and l [slot][NH]
  size_t ws_bytes;                // 0 when K == 1 (no workspace touched)
};
bool plan_step(const gva_dims *d, int32_t B, int32_t max_len, StepPlan *plan);
hipError_t launch_step_fused(const StepArgs &s, hipStream_t stream);
// The decode alone with the one-launch step's split and merge (the query rows read from q_abs,
// no token appended): one launch, no combine. Shapes: d_h of 32 or 64, H / G of 1, 2, 4 or 8,
// B * G <= kPlanCUs. (At d_h = 128 the two-launch plans measured faster: for one sequence of
// 131072 positions 69 against 61 us, for 4 of 8705 28 against 26 us.)
bool decode_merged_shape(const gva_dims *d, int32_t B);
hipError_t launch_decode_merged(const StepArgs &s, hipStream_t stream);
hipError_t launch_decode_generic(const DecodeArgs &a, bool bf16, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_combine(const DecodeArgs &a, hipStream_t stream);

struct PrefillArgs {
  DecodeArgs kv;        // cache description and shape (seq_len unused)
  const int32_t *start;
  int32_t max_start;
  int32_t chunk_len;
  const float *q_abs;   // [B][C][H][d_h + d_r]
  const float *v_new;   // [B][C][G][d_h]
  const float *kr_raw;  // [B][C][d_r]
  const double *rope;   // RoPE table used by the chunk's append
  int32_t max_pos;
  float *out;           // [B][C][H][d_h]
  float *lse;           // [B][C][H] or nullptr
};
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

struct ReconArgs {
  DecodeArgs kv;        // value cache, shape, split plan, partials and outputs (d_r unused)
  int32_t d_n;
  const float *q;       // [B][H][d_n]
  const int32_t *q_pos; // [B]
  const uint16_t *Mt;   // bf16 bits [H][d_n][d_h]
  const double *rope;   // [max_pos][d_n / 2][2]
  int32_t max_pos;
};
hipError_t launch_recon_decode(const ReconArgs &r, hipStream_t stream);
hipError_t launch_latent_decode(const DecodeArgs &a, hipStream_t stream);

}  // namespace gva

#endif  // GVA_INTERNAL_H_
