/*
 * gva.h - C ABI of a Grouped Value Attention (GVA) decode library for AMD MI355X (gfx950).
 *
 * Sources (web pages about arXiv:2609.13285, "Grouped Value Attention: Efficient KV Caching
 * via On-Demand Key Reconstruction"):
 *   [review]   shibing624.github.io review, "GVA：KV 缓存里的 Key 其实可以不存"
 *   [summary]  agihunt.info summary of the paper
 *   [kvcache]  liumengxuan04.github.io, "KV Cache 优化（一）：从 MHA 到 MQA 与 GQA"
 *
 * Notation follows the pages: T cached tokens, H query heads, G value groups, d_h value
 * width, d_n content-query width, d_r positional width, g(h) the group of head h.
 *
 * One layer's cache holds, per token, the G grouped values v_g (d_h wide) and ONE positional
 * key kr (d_r wide) shared by all heads and stored already rotated ([review] section 缓存账本;
 * section 关键技巧二). No content key is ever stored: head h's content key would be
 * K_h = V_g(h) M_h with M_h of shape d_h x d_n ([review] section 第二次尝试), and because M_h is
 * fixed it is folded into the query, q~_h = q_nope_h M_h^T ([review] section 关键技巧一). The
 * score of cached position j is q~_h . v_{j,g(h)} + rot(q_rope_h) . kr_j ([review] section
 * 关键技巧二, the two-term score), followed by a softmax and a weighted sum over the same
 * cached values ([summary]; [kvcache] section 1).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are device memory on the current HIP device; "host" is host
 *     memory. All device buffers are owned by the caller; the library allocates nothing.
 *   - Every call is asynchronous on `stream` and does no host/device synchronisation.
 *   - Inputs are read-only; outputs are fully overwritten and must not alias inputs.
 *   - Argument errors are detected on the host and returned before any launch; the detail
 *     is available from gva_last_error() on the calling thread.
 *   - Errors that only the device can see (a bad block-table entry, a position beyond the
 *     cache or the RoPE table, a length above the stated bound) set bits in *err_flag when
 *     err_flag is not NULL; the affected token is not written (append) or the affected
 *     output row is filled with NaN (decode, prefill).
 *   - Grouping: g(h) = h / (H / G) (contiguous) unless gva_dims.g_of_h names another map in
 *     which every group holds exactly H / G heads.
 *   - RoPE pairs are interleaved: (x[2i], x[2i+1]) is rotated by p * theta_i.
 */
#ifndef GVA_H_
#define GVA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gva_status {
  GVA_OK = 0,
  GVA_ERR_INVALID_ARG = 1,   /* a NULL pointer, a bad size, stride or alignment */
  GVA_ERR_UNSUPPORTED = 2,   /* valid arguments outside what the kernels implement */
  GVA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than gva_decode_workspace_bytes */
  GVA_ERR_HIP = 4            /* a HIP launch failed */
} gva_status;

typedef enum gva_dtype {
  GVA_DTYPE_F32 = 0,
  GVA_DTYPE_BF16 = 1
} gva_dtype;

/* Bits set in *err_flag by device-side checks (sticky: the library only ORs bits in). */
enum {
  GVA_DEVERR_BLOCK = 1,      /* block-table entry outside [0, num_blocks) */
  GVA_DEVERR_CAPACITY = 2,   /* position >= max_blocks * block_size */
  GVA_DEVERR_ROPE = 4,       /* position >= max_pos of the RoPE table */
  GVA_DEVERR_SEQ = 8,        /* sequence index outside [0, B) */
  GVA_DEVERR_LENGTH = 16     /* negative position or length, or length above max_len */
};

/* Which decode kernel runs. AUTO picks the MFMA kernel when the shape allows it. */
typedef enum gva_decode_kernel {
  GVA_KERNEL_AUTO = 0,
  GVA_KERNEL_GENERIC = 1,    /* vector-ALU kernel: any supported shape and dtype */
  GVA_KERNEL_MFMA = 2        /* matrix-core kernel: bf16 cache, see gva_decode */
} gva_decode_kernel;

/* Model shape in the pages' notation. Limits: 1 <= G <= H, H % G == 0, H <= 256,
 * 2 <= d_h <= 256 and even, 1 <= d_n <= 512, 2 <= d_r <= 64 and even.
 * g_of_h: host int32 [H] or NULL. g_of_h[h] is the value group g(h) that query head h reads
 * ("GVA：KV 缓存里的 Key 其实可以不存", section 第二次尝试: head h's key is built from the values of
 * its group g(h); [kvcache] section 4: query heads are partitioned into groups that share one
 * cached stream). Every entry must lie in [0, G) and every group must hold exactly H / G heads
 * (GVA_ERR_INVALID_ARG otherwise). NULL means the contiguous map g(h) = h / (H / G). The array
 * is read during the call only; the caller keeps ownership. */
typedef struct gva_dims {
  int32_t H;
  int32_t G;
  int32_t d_h;
  int32_t d_n;
  int32_t d_r;
  const int32_t *g_of_h;
} gva_dims;

/* One layer's cache, paged or contiguous, described by element strides.
 *   V(blk, tok, g, i) = v [blk * v_stride_block  + tok * v_stride_token  + g * v_stride_group + i]
 *   kr(blk, tok, i)   = kr[blk * kr_stride_block + tok * kr_stride_token + i]
 * Position p of sequence b lives in block block_table[b * max_blocks + p / block_size] at
 * token offset p % block_size. A contiguous cache is one block per sequence with
 * block_size >= its capacity. Paging only changes where entries live ([kvcache] section 7). */
typedef struct gva_cache {
  gva_dtype dtype;                 /* element type of v and kr */
  void *v;                         /* device, 16-byte aligned */
  void *kr;                        /* device, 16-byte aligned */
  int64_t v_stride_block;          /* element strides, each >= 0 */
  int64_t v_stride_token;
  int64_t v_stride_group;
  int64_t kr_stride_block;
  int64_t kr_stride_token;
  int64_t num_blocks;              /* blocks in the pool; block ids are in [0, num_blocks) */
  int32_t block_size;              /* tokens per block, a power of two */
  int32_t max_blocks;              /* columns of block_table */
  const int32_t *block_table;      /* device int32 [B][max_blocks] */
  const double *rope;              /* device float64 [max_pos][d_r / 2][2] = (cos, sin) */
  int32_t max_pos;                 /* rows of the RoPE table */
  int32_t *err_flag;               /* device, nullable: sticky GVA_DEVERR_* bits */
} gva_cache;

/* ---- RoPE table ------------------------------------------------------------------------
 * Rows p = 0 .. max_pos-1, pairs i = 0 .. d_r/2-1: (cos(p * theta_i), sin(p * theta_i)) with
 * theta_i = base^(-2i / d_r), evaluated in float64 with the C library's pow, cos and sin.
 * The positional slice is rotated by position ([review] section 关键技巧二); the frequency
 * convention is the usual RoPE one. d_r is the rotated width: the positional slice's d_r, or
 * d_n for the keys of gva_recon_decode; it must be even and in [2, 512]. */
size_t gva_rope_table_bytes(int32_t max_pos, int32_t d_r);
/* host_out: host float64 buffer of gva_rope_table_bytes(max_pos, d_r) bytes. */
gva_status gva_rope_table_fill(double *host_out, int32_t max_pos, int32_t d_r, double base);

/* ---- Cache append ([review] section 关键技巧二: the shared positional key is cached already
 * rotated; [kvcache] section 1: a new token's state is appended before the query reads the
 * history) -----------------------------------------------------------------------------------
 * Writes n_tok tokens. Token k belongs to sequence seq[k] in [0, B) at position pos[k]:
 *   V(slot, g, :) = round(v_new[k][g][:])                    for every group g
 *   kr(slot, :)   = round(rotate(kr_raw[k][:], pos[k]))      rotation in float64
 * where round() is one round-to-nearest-even to the cache type and rotate() forms each pair
 * as (x0*c - x1*s, x0*s + x1*c) with every product and sum rounded to float64 (no fused
 * multiply-add). The result is bit-exact and independent of launch configuration.
 *   seq, pos: device int32 [n_tok]. v_new: device float32 [n_tok][G][d_h].
 *   kr_raw: device float32 [n_tok][d_r]. Two tokens must not target the same slot.
 * A token with a bad index is skipped and raises its GVA_DEVERR_* bit. */
gva_status gva_cache_append(const gva_dims *dims, const gva_cache *cache, int32_t B,
                            int32_t n_tok, const int32_t *seq, const int32_t *pos,
                            const float *v_new, const float *kr_raw, hipStream_t stream);

/* ---- Query absorption ([review] section 关键技巧一: q~_h = q_nope_h M_h^T once per query
 * token; section 关键技巧二: the positional slice is rotated at the query's position) --------
 *   q_abs[k][h][0 .. d_h)         = q~_h,   q~_h[i] = sum_j M[h][i][j] * q_nope[k][h][j]
 *   q_abs[k][h][d_h .. d_h + d_r) = float32(rotate(q_rope[k][h][:], q_pos[k]))
 * The q~ part accumulates in float32 (error within d_n * 2^-24 * sum_j |M q|); the rotated
 * part is one rounding of the float64 rotation.
 *   q_nope: device float32 [n_q][H][d_n], 16-byte aligned (d_n a multiple of 4).
 *   q_rope: device float32 [n_q][H][d_r], 8-byte aligned. q_pos: device int32 [n_q].
 *   M: device float32 [H][d_h][d_n], 16-byte aligned.
 *   rope/max_pos: the device RoPE table. q_abs: device float32 [n_q][H][d_h + d_r] (output).
 * A position outside [0, max_pos) writes NaN into that token's q_abs and raises
 * GVA_DEVERR_ROPE in *err_flag (nullable). */
gva_status gva_absorb_query(const gva_dims *dims, int32_t n_q, const float *q_nope,
                            const float *q_rope, const int32_t *q_pos, const float *M,
                            const double *rope, int32_t max_pos, float *q_abs,
                            int32_t *err_flag, hipStream_t stream);

/* ---- Decode ([review] sections 关键技巧一 and 关键技巧二; [kvcache] section 1) -------------------
 * For every sequence b and head h, over the cached positions j < seq_len[b]:
 *   s_j = scale * (q~_h . V(j, g(h), :) + r_h . kr(j, :))   with [q~_h ; r_h] = q_abs[b][h]
 *   out[b][h][:] = sum_j softmax(s)_j V(j, g(h), :),   lse[b][h] = ln sum_j exp(s_j)
 * The positions are split into num_splits contiguous chunks processed in parallel and merged
 * through their log-sum-exp. With num_splits == 0 (automatic) the matrix-core kernel instead
 * cuts the 32-position tiles of all sequences, taken in sequence order, into equal ranges (see
 * gva_decode_num_ranges), so every work-group gets the same amount of cache to read whatever
 * the lengths; the chunks of one sequence are merged the same way. Small batches at d_h of 32
 * or 64 (B G <= 256 sequence-groups, H / G of 1, 2, 4 or 8; automatic split count, matrix-core
 * kernel) are decoded in ONE launch instead: K work-groups per (sequence, group) each read a
 * contiguous share of the positions cut from max_len, and the last of them to finish merges
 * the K partials (through the workspace, with a ticket per (sequence, group) in its first 1024
 * bytes); no combine follows.
 * seq_len[b] == 0 gives out = 0 and lse = -inf.
 *   seq_len: device int32 [B]. max_len: host upper bound on every seq_len[b] (it sizes the
 *   split plan; a larger length raises GVA_DEVERR_LENGTH and makes that row NaN).
 *   q_abs: device float32 [B][H][d_h + d_r], 16-byte aligned. out: device float32
 *   [B][H][d_h], 16-byte aligned. lse: device float32 [B][H] or NULL.
 *   num_splits: 0 = choose automatically, else 1 .. 1024 (rounded down so no chunk is empty
 *   for a sequence of max_len tokens).
 *   kernel: GVA_KERNEL_* ; the MFMA kernel needs a bf16 cache, d_h % 32 == 0, d_h <= 256,
 *   d_r % 8 == 0, d_r <= 32, H / G <= 16, G <= 16, block_size >= 16, every stride a multiple
 *   of 8 elements (returns GVA_ERR_UNSUPPORTED otherwise).
 *   workspace: device, 256-byte aligned, at least gva_decode_workspace_bytes(...) bytes,
 *   zero-filled before its first use (e.g. with hipMemsetAsync once after allocating it). Its
 *   first 1024 bytes hold the tickets of the one-launch plans (small batches of gva_decode and
 *   gva_decode_step); no call writes partials there and every call leaves them at zero, so one
 *   fill serves every later call of any of these entry points. Calls that overlap must not
 *   share a workspace. */
size_t gva_decode_workspace_bytes(const gva_dims *dims, int32_t B, int32_t max_len,
                                  int32_t num_splits);
/* The split count gva_decode will use for these arguments with per-sequence chunks (an
 * explicit num_splits, or the vector-ALU kernel); 0 on bad arguments. */
int32_t gva_decode_num_splits(const gva_dims *dims, int32_t B, int32_t max_len,
                              int32_t num_splits);
/* The number of equal tile ranges of the matrix-core kernel's automatic plan (num_splits == 0);
 * 0 on bad arguments, when that plan falls back to per-sequence chunks (one sequence), or when
 * the batch takes the one-launch plan (small batches at d_h of 32 or 64). */
int32_t gva_decode_num_ranges(const gva_dims *dims, int32_t B, int32_t max_len);
gva_status gva_decode(const gva_dims *dims, const gva_cache *cache, int32_t B,
                      const int32_t *seq_len, int32_t max_len, const float *q_abs, float scale,
                      int32_t num_splits, int32_t kernel, void *workspace,
                      size_t workspace_bytes, float *out, float *lse, hipStream_t stream);

/* ---- Decode without allocation --------------------------------------------------------------
 * For callers that cannot allocate device memory or hand in a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Computes exactly what
 * gva_decode computes for the same arguments (same plan, same kernels, bit-identical results),
 * with the split partials kept in a static device array of GVA_NOALLOC_SCRATCH_BYTES instead of
 * a caller workspace. That array is part of the library: each device the library runs on holds
 * one copy until the process ends; its address is looked up on the first call made with that
 * device current. The call allocates nothing (no hipMalloc, no allocating library routine).
 *   Arguments: as for gva_decode, without workspace and workspace_bytes.
 *   Returns GVA_ERR_WORKSPACE, before any launch, when the plan's partials need more than
 *   GVA_NOALLOC_SCRATCH_BYTES (gva_decode_workspace_bytes gives the need). The one-launch plan's
 *   tickets sit in the array's first 1024 bytes: they start at zero (a static array, cleared
 *   once more by a small kernel on the first call's stream when the array's address is looked
 *   up) and every call leaves them at zero.
 *   All calls on one device share its array: calls that overlap on one device (other streams,
 *   other threads) race and must be serialised by the caller. */
#define GVA_NOALLOC_SCRATCH_BYTES (32u << 20)
gva_status gva_decode_noalloc(const gva_dims *dims, const gva_cache *cache, int32_t B,
                              const int32_t *seq_len, int32_t max_len, const float *q_abs,
                              float scale, int32_t num_splits, int32_t kernel, float *out,
                              float *lse, hipStream_t stream);

/* ---- One decode step ([kvcache] section 1: each step appends the new token's state, then the
 * query reads the whole history; [review] sections 关键技巧一 and 关键技巧二) ------------------
 * For B sequences that each receive one token, does what gva_cache_append (token b to
 * sequence b at pos[b]), gva_absorb_query (query b at pos[b], with the cache's RoPE table and
 * err_flag) and gva_decode would do in that order. The cache bytes and q_abs are bit-identical
 * to those of the three calls. Small batches (the matrix-core kernel, d_h of 32 or 64,
 * H / G of 1, 2, 4 or 8, B G <= 256 sequence-groups, at most 4 MiB of values per group, the
 * automatic split count) run the whole step as ONE launch: K work-groups per (sequence, group)
 * each append the token (one of them writes it), absorb the group's queries, decode a share
 * of the positions (a wave that reads the new position takes the token it has just rounded,
 * not the cache) and merge their waves' partials; the last of the K to finish merges the K
 * partials (through the workspace and a ticket in its first 1024 bytes). Small batches of the
 * shapes the vector-ALU kernel decodes (float32 caches among them: H / G of 1, 2, 4 or 8,
 * B G <= 256, max_len <= 1024, the group's rows of M within 72 KiB of LDS, the automatic split
 * count) also run as ONE launch: one work-group per (sequence, group) appends, absorbs, decodes
 * all positions over its waves and merges them; no workspace bytes are touched. The one-launch
 * outputs equal gva_decode's to rounding (the positions are split differently), not bit for
 * bit. Other arguments take one launch for the append and the absorption, then the decode (and
 * its combine), with outputs bit-identical to the three calls. gva_decode_step_launches tells
 * which. Within one call the block that receives sequence b's token must not be read by
 * another sequence.
 *   pos: device int32 [B], the new token's position (its sequence's length before the step).
 *   v_new: device float32 [B][G][d_h]; kr_raw: device float32 [B][d_r].
 *   q_nope: device float32 [B][H][d_n]; q_rope: device float32 [B][H][d_r];
 *   M: device float32 [H][d_h][d_n].
 *   seq_len: device int32 [B], the positions the decode reads (pos[b] + 1 to include the new
 *   token); max_len, scale, num_splits, kernel, workspace, out, lse: as for gva_decode
 *   (workspace sized by gva_decode_workspace_bytes).
 *   q_abs: device float32 [B][H][d_h + d_r], written with the absorbed queries and then read
 *   by the decode (16-byte aligned).
 * Errors found on the device raise the same GVA_DEVERR_* bits as the three calls. */
gva_status gva_decode_step(const gva_dims *dims, const gva_cache *cache, int32_t B,
                           const int32_t *pos, const float *v_new, const float *kr_raw,
                           const float *q_nope, const float *q_rope, const float *M,
                           const int32_t *seq_len, int32_t max_len, float scale,
                           int32_t num_splits, int32_t kernel, float *q_abs, void *workspace,
                           size_t workspace_bytes, float *out, float *lse, hipStream_t stream);
/* How many launches gva_decode_step makes for these arguments: 1 when the whole step runs as
 * one launch (above), 2 or 3 otherwise (append and absorption, the decode, and its combine when
 * the decode splits); 0 on bad arguments. */
int32_t gva_decode_step_launches(const gva_dims *dims, const gva_cache *cache, int32_t B,
                                 int32_t max_len, int32_t num_splits, int32_t kernel);

/* ---- Chunked prefill ([summary]: prefill stays a dense, matrix-heavy pass) -----------------
 * Appends chunk_len new tokens per sequence at positions start[b] .. start[b] + chunk_len - 1
 * (exactly as gva_cache_append would), then for query i of sequence b, at position
 * start[b] + i, attends causally to positions 0 .. start[b] + i inclusive with the decode
 * score above, reading the cache-rounded values.
 *   start: device int32 [B]; max_start: host upper bound on start[b].
 *   q_abs: device float32 [B][chunk_len][H][d_h + d_r] (absorbed at positions start[b] + i).
 *   v_new: device float32 [B][chunk_len][G][d_h]; kr_raw: device float32 [B][chunk_len][d_r].
 *   out: device float32 [B][chunk_len][H][d_h]; lse: device float32 [B][chunk_len][H] or NULL.
 * Needs a bf16 cache and the MFMA kernel's shape limits (see gva_decode). */
gva_status gva_prefill_chunk(const gva_dims *dims, const gva_cache *cache, int32_t B,
                             const int32_t *start, int32_t max_start, int32_t chunk_len,
                             const float *q_abs, const float *v_new, const float *kr_raw,
                             float scale, float *out, float *lse, hipStream_t stream);

/* ---- GQA comparator ([kvcache] section 4: the query heads of a group share one key head and one
 * value head; [kvcache] section 1: the decode step) ------------------------------------------
 * Decodes the cache a matched grouped-query model would keep - G keys and G values per token,
 * 2 G d_h scalars instead of GVA's G d_h + d_r - on the same matrix-core kernel, work plan and
 * combine as gva_decode, so the two can be timed side by side:
 *   out[b][h][:] = sum_j softmax_j(scale * q[b][h] . K(j, g(h), :)) V(j, g(h), :)
 *   dims: as for gva_decode (H, G, d_h are used; the shape limits of the matrix-core kernel
 *   apply). values: a bf16 cache as for gva_decode holding the value pool; its positional-key
 *   pool and RoPE table are not read. keys: device, 16-byte aligned, the key pool, laid out
 *   exactly like values->v (same strides, block table and dtype).
 *   q: device float32 [B][H][d_h], already rotated like the cached keys.
 *   workspace: at least gva_decode_workspace_bytes(dims, B, max_len, 0) bytes.
 * Errors as for gva_decode. */
gva_status gva_gqa_decode(const gva_dims *dims, const gva_cache *values, const void *keys,
                          int32_t B, const int32_t *seq_len, int32_t max_len, const float *q,
                          float scale, void *workspace, size_t workspace_bytes, float *out,
                          float *lse, hipStream_t stream);

/* ---- Non-absorbable comparator ([summary]: the scale-matched + query RMSNorm row applies
 * ordinary RoPE to the reconstructed key and therefore cannot absorb the map; [review] section
 * 第二次尝试: K_h = V_g M_h) ---------------------------------------------------------------
 * Decodes a value-only cache whose content keys are rebuilt from the cached values at every step
 * and rotated at their own positions, so the map cannot be folded into the query:
 *   k_{h,j} = R_j (M_h^T v_{j,g(h)})      (d_n wide, M_h of shape d_h x d_n)
 *   s_j     = scale * (R_p q_h) . k_{h,j},  p = q_pos[b]
 *   out[b][h][:] = sum_{j < seq_len[b]} softmax_j(s) v_{j,g(h)},  lse as for gva_decode
 * R_x rotates interleaved pairs (x[2i], x[2i+1]) by x * theta_i with theta_i = base^(-2i / d_n):
 * the rows of a gva_rope_table_fill(max_pos, d_n, base) table.
 *   dims: H, G, d_h, d_n (d_r is not used). Supported: d_h and d_n in {64, 128}, H / G <= 4.
 *   values: a bf16 cache as for gva_decode holding the value pool; its positional-key pool and
 *   its RoPE table are not read (they may be NULL). Strides must be multiples of 8 elements.
 *   q: device float32 [B][H][d_n], 16-byte aligned (the query content vectors, normalised as
 *   the model does before attention). q_pos: device int32 [B].
 *   Mt: device, 16-byte aligned, bf16 bits [H][d_n][d_h] with Mt[h][k][i] = M_h[i][k] (the map
 *   in the model's bf16, stored transposed).
 *   rope: device float64 [max_pos][d_n / 2][2], 16-byte aligned; max_pos >= 32.
 *   num_splits: chunks per sequence (0 = automatic), merged as in gva_decode.
 *   workspace: at least gva_recon_decode_workspace_bytes(dims, B, max_len, num_splits) bytes,
 *   256-byte aligned (none when that is 0).
 *   out: device float32 [B][H][d_h], 16-byte aligned; lse: device float32 [B][H] or NULL.
 * Device-detected errors (NaN rows, err_flag bits): a bad block-table entry (BLOCK); seq_len[b]
 * negative or above max_len (LENGTH) or above the table's capacity (CAPACITY); q_pos[b] outside
 * [0, max_pos) or seq_len[b] > max_pos (ROPE). */
size_t gva_recon_decode_workspace_bytes(const gva_dims *dims, int32_t B, int32_t max_len,
                                        int32_t num_splits);
gva_status gva_recon_decode(const gva_dims *dims, const gva_cache *values, int32_t B,
                            const int32_t *seq_len, int32_t max_len, const float *q,
                            const int32_t *q_pos, const uint16_t *Mt, const double *rope,
                            int32_t max_pos, float scale, int32_t num_splits, void *workspace,
                            size_t workspace_bytes, float *out, float *lse, hipStream_t stream);

/* ---- MLA-style latent comparator ([review] section 问题: MLA caches one joint latent of width
 * d_c plus a shared RoPE channel, T (d_c + d_r) scalars, and projects keys and values back up at
 * decode) -----------------------------------------------------------------------------------
 * Decodes an MLA cache with the key up-projection folded into the query: the absorbed decode of
 * gva_decode with one group (G = 1) whose cached value is the latent (d_h = d_c):
 *   out[b][h][:] = sum_{j < seq_len[b]} softmax_j(scale * (q~_h . c_j + r_h . kr_j)) c_j
 * (width d_c); the value up-projection multiplies out afterwards, outside this call, as W_O
 * does for GVA.
 *   dims: H in {8, 16, 32}, G = 1, d_h = d_c in {256, 512}, d_r a multiple of 8 in [8, 64]
 *   (d_n is not used).
 *   latent: a bf16 cache as for gva_decode, v holding the latents (v_stride_group is not used)
 *   and kr the rotated positional keys; strides multiples of 8 elements; block_size >= 16; its
 *   RoPE table is not read. gva_cache_append fills such a pool when each latent row is described as d_c / 256
 *   groups of 256 (v_stride_group = 256).
 *   q_abs: device float32 [B][H][d_c + d_r] = [q~_h ; rotated q_rope_h], 16-byte aligned.
 *   workspace: device, at least gva_mla_decode_workspace_bytes(dims, B, max_len, num_splits)
 *   bytes (never 0: besides the split partials it holds the counter of the work queue the
 *   call's work-groups take their items from, reset by the call itself), 256-byte aligned;
 *   calls that overlap must not share one. num_splits as for gva_recon_decode.
 *   out: device float32 [B][H][d_c], 16-byte aligned; lse: device float32 [B][H] or NULL.
 * Device-detected errors: a bad block-table entry (BLOCK), seq_len[b] negative or above max_len
 * (LENGTH) or above the table's capacity (CAPACITY), each giving a NaN output row. */
size_t gva_mla_decode_workspace_bytes(const gva_dims *dims, int32_t B, int32_t max_len,
                                      int32_t num_splits);
gva_status gva_mla_decode(const gva_dims *dims, const gva_cache *latent, int32_t B,
                          const int32_t *seq_len, int32_t max_len, const float *q_abs,
                          float scale, int32_t num_splits, void *workspace,
                          size_t workspace_bytes, float *out, float *lse, hipStream_t stream);

/* ---- Diagnostics --------------------------------------------------------------------------- */
const char *gva_status_string(gva_status status);
/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char *gva_last_error(void);
/* Library version string. */
const char *gva_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GVA_H_ */
