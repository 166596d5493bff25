/*
 * bsa.h -- query-aware block-sparse attention on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbsa.so.  Every entry point takes plain pointers and sizes:
 *
 *   - Tensor data pointers are HIP DEVICE pointers.  The caller owns every
 *     buffer (inputs, outputs, workspace); the library never allocates or
 *     frees device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream).  All work is enqueued asynchronously on it; no call
 *     synchronises with the host.
 *   - Arguments are validated on the host before anything is launched.  On a
 *     non-OK status nothing has been enqueued and no output was written;
 *     bsa_last_error() returns a thread-local message with the detail.
 *   - Results are deterministic: two calls with the same inputs produce the
 *     same bytes (fixed reduction orders, no floating-point atomics).
 *
 * Sources (pages cited by title and section):
 *   LoSA   -- "LoSA: Locality Aware Sparse Attention for Block-Wise Diffusion
 *             Language Models", technical summary sec. 1-2.
 *   Prism  -- "Prism: Spectral-Aware Block-Sparse Attention", technical
 *             summary sec. 1-3.
 *   NSA    -- "Native Sparse Attention: Hardware-Aligned and Natively
 *             Trainable Sparse Attention" (news article), NSA structure
 *             section and implementation-challenges section.
 *   FASA   -- "FASA: Frequency-aware Sparse Attention", technical summary
 *             sec. 2.
 *   BLASST -- "BLASST: Dynamic BLocked Attention Sparsity via Softmax
 *             Thresholding", technical summary sec. 2.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID = 1,      /* null pointer, bad shape, misaligned or inconsistent argument */
  BSA_ERR_UNSUPPORTED = 2,  /* valid request outside what the kernels implement (dtype, D, block) */
  BSA_ERR_CAPACITY = 3,     /* index-list capacity below the bound the selection can reach */
  BSA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the *_workspace_bytes query */
  BSA_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed */
} bsa_status;

typedef enum { BSA_BF16 = 0, BSA_F32 = 1 } bsa_dtype;

/* Which head dims a RoPE frequency chunk (FC) owns.  FC i (0 <= i < D/2)
 * rotates at base^(-2i/D); a low FC index is a fast rotation.
 *   BSA_ROPE_HALF:        FC i owns dims i and i + D/2 (rotate-half layout)
 *   BSA_ROPE_INTERLEAVED: FC i owns dims 2i and 2i + 1
 * The fast (high-frequency) band is FC i < D/4; the slow band the rest. */
typedef enum { BSA_ROPE_HALF = 0, BSA_ROPE_INTERLEAVED = 1 } bsa_rope_layout;

/* A 4-D tensor [B, H, L, D] in device memory, strides in elements.  The D
 * axis must be contiguous (stride 1).  `data` must be 16-byte aligned and
 * stride_l * element size a multiple of 16 bytes.  Input tensors are never
 * written through. */
typedef struct {
  void* data;
  int32_t dtype;                 /* bsa_dtype */
  int32_t B, H, L, D;
  int64_t stride_b, stride_h, stride_l;
} bsa_tensor;

/* ------------------------------------------------------------------------ *
 * Block summaries (Prism sec. 1-2: a KV block is scored through the mean of
 * its vectors; pooling acts as a low-pass filter on RoPE'd vectors).
 *
 * For x [B, H, L, D] (bf16 or f32) and block size b, NB = ceil(L / b).  For
 * block j with tokens [j*b, min((j+1)*b, L)) writes
 *   mean[b][h][j][:]      = average of the block's vectors           (f32)
 *   energy[b][h][j][0..1] = average over tokens of ||x_t[band]||^2 for the
 *                           fast and the slow band (per `layout`)    (f32)
 * A ragged last block averages its valid tokens only.  Only blocks
 * first_block .. first_block + num_blocks - 1 are computed and written
 * (num_blocks < 0: through the last block), so a decode step can refresh just
 * the newest block.  `mean` is [B, H, NB, D] and `energy` [B, H, NB, 2], both
 * contiguous; `energy` may be NULL.
 * Supported: D in {64, 128}; b in {16, 32, 64, 128, 256}; bf16 or f32.
 * ------------------------------------------------------------------------ */
bsa_status bsa_build_block_summaries(const bsa_tensor* x, int32_t block_size, int32_t layout,
                                     int32_t first_block, int32_t num_blocks,
                                     float* mean, float* energy, void* stream);

/* ------------------------------------------------------------------------ *
 * Block selection: scoring, top-k per GQA group, union over a query block.
 *
 * Selection rows.  Raw mode (pooled_q = 0): every query row is a selection
 * row; q is [B, Hq, Lq, D] bf16/f32 and query block i holds rows
 * i*q_block .. min((i+1)*q_block, Lq) - 1.  Pooled mode (pooled_q = 1): q is
 * an f32 tensor [B, Hq, NQB, D] of mean-pooled queries (from
 * bsa_build_block_summaries) and each query block has exactly one selection
 * row; q_len gives Lq.  (Prism sec. 3: purely block-level estimation.)
 *
 * Candidates C of query block i: all NB KV blocks, or with causal = 1 the
 * blocks j whose first key j*kv_block is <= q_pos0 + (last row of block i).
 * Forced F: the first n_first and the last n_last candidates (NSA structure
 * section: block 0 and the 2 newest blocks are always among the 16; for causal
 * prefill the newest candidate is the diagonal block).  Scored picks
 * k' = topk, or ceil(topk_num * |C| / topk_den) when topk_num > 0, capped at
 * |C \ F|.
 *
 * Scores, per selection row r and KV group g (the selection is shared by the
 * query heads of a GQA group -- NSA implementation-challenges section):
 *   single band: z_h[j] = scale * q_h . kmean_g[j];  p_h = softmax over C
 *   dual band  : z_h^band[j] = scale * q_h[band] . kmean_g[j][band] / tau_h^band
 *                p_h = (softmax(z_h^fast) + softmax(z_h^slow)) / 2
 *   group score s[j] = sum over heads h of g of p_h[j]     (fp32)
 * Temperatures (dual band; Prism sec. 3, energy-based calibration):
 *   rho_X^band = sum_j ||mean_X[j][band]||^2 / sum_j energy_X[j][band]
 *   tau_h^band = max(1e-6, sqrt(rho_Q^band(h) * rho_K^band(g)))
 * with rho_Q = 1 in raw mode.  Row picks = F + the k' best of C \ F by s
 * (ties: lower block index).  The list of a query block is the union of its
 * rows' picks over rows with row_mask = 1 (LoSA sec. 1: traffic is set by the
 * union over the block; sec. 2: selecting for active rows only shrinks it).
 *
 * Outputs: idx [B, Hkv, NQB, cap] int32 -- the list, ascending and unique,
 * in the first cnt entries (the rest is left unwritten); cnt [B, Hkv, NQB].
 * Optional: row_picks [B, Hkv, R, cap] int32 (R = Lq raw or NQB pooled): each
 * selection row's own sorted picks padded with -1 (-1 everywhere for masked
 * rows); tau_out [B, Hq, 2] (dual band).
 * k_mean/k_energy: [B, Hkv, NB, D] / [B, Hkv, NB, 2] f32 contiguous with
 * Hkv = num_kv_heads dividing Hq and NB = num_kv_blocks; q_energy
 * [B, Hq, NQB, 2] (pooled + dual band), else NULL.  row_mask [B, Lq] uint8 or
 * NULL (raw mode only).  workspace: bsa_select_workspace_bytes() bytes of
 * scratch (no initial contents needed; calls that overlap on one workspace
 * race).
 * Errors: BSA_ERR_CAPACITY when cap < min(NB, R_per_block * (k'_max + n_first
 * + n_last)); BSA_ERR_UNSUPPORTED for NB > 4096, D not in {64, 128}, or more
 * than 64 query rows per block in raw mode.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t kv_block;          /* tokens per KV block (summary granularity) */
  int32_t q_block;           /* query rows per query block */
  int32_t q_pos0;            /* absolute position of query row 0 */
  int32_t q_len;             /* Lq in pooled mode (0: NQB * q_block) */
  int32_t causal;
  int32_t pooled_q;
  int32_t topk, topk_num, topk_den;
  int32_t n_first, n_last;
  int32_t dual_band;
  int32_t layout;            /* bsa_rope_layout */
  float scale;               /* logit scale, usually 1/sqrt(D) */
  int32_t cap;               /* entries per index list */
} bsa_select_params;

size_t bsa_select_workspace_bytes(const bsa_tensor* q, int32_t num_kv_heads, int32_t num_kv_blocks,
                                  const bsa_select_params* p);

bsa_status bsa_select_blocks(const bsa_tensor* q, const float* q_energy,
                             const float* k_mean, const float* k_energy,
                             int32_t num_kv_heads, int32_t num_kv_blocks,
                             const bsa_select_params* p, const uint8_t* row_mask,
                             int32_t* idx, int32_t* cnt, int32_t* row_picks, float* tau_out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * bsa_build_block_summaries for one block followed by bsa_select_blocks, in
 * the selection's launches: a decode step's newest block changes with every
 * token, and its summary (mean and, if k_energy is non-NULL, band energies;
 * Prism sec. 1-2, as the summaries entry point) is pooled from k by the
 * scoring workgroup that needs it, used, and written to k_mean / k_energy at
 * refresh_block.  k [B, Hkv, L, D] as q's dtype; num_kv_blocks must be
 * ceil(L / kv_block).  Raw query rows and one band only (pooled_q = 0,
 * dual_band = 0); with causal = 1 the block must start at or before q_pos0.
 * Other arguments and errors as bsa_select_blocks (the same workspace size).
 * ------------------------------------------------------------------------ */
bsa_status bsa_select_blocks_refresh(const bsa_tensor* k, int32_t refresh_block, const bsa_tensor* q, float* k_mean,
                                     float* k_energy, int32_t num_kv_heads, int32_t num_kv_blocks,
                                     const bsa_select_params* p, const uint8_t* row_mask, int32_t* idx, int32_t* cnt,
                                     int32_t* row_picks, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * One GQA decode step: bsa_select_blocks_refresh followed by
 * bsa_sparse_attention_fwd on the lists it selects (NSA
 * structure section: selection block 64, block 0 and the newest blocks
 * always kept; decode-speed section: the step reads only the selected
 * blocks).
 *
 * q [B, Hq, Lq, D]: decode rows, row r at position q_pos0 + r, each its own
 * query block (p->q_block must be 1; raw queries, one band: pooled_q = 0,
 * dual_band = 0); k, v [B, Hkv, L, D] of q's dtype (bf16 or f32, D 64 or
 * 128, Hq / Hkv in {1, 2, 4, 8}); NB = ceil(L / kv_block) <= 4096.
 * k_mean [B, Hkv, NB, D] f32 (and k_energy [B, Hkv, NB, 2] or NULL) hold the
 * summaries; when refresh_block >= 0 that block's summary is pooled from k
 * (the newest block, whose tokens change every step), used, and written
 * there (refresh_block = -1: none).  The scores, forced blocks, k', ties and
 * causality follow bsa_select_blocks; the attention follows
 * bsa_sparse_attention_fwd with the selection's scale, kv_block, q_pos0,
 * causal and cap.  Writes idx [B, Hkv, Lq, cap] and cnt [B, Hkv, Lq] (as
 * bsa_select_blocks), o (q's shape, q's dtype or f32) and lse [B, Hq, Lq].
 * Two launches: the block logits (with per-wavefront softmax partials),
 * then one workgroup per (slice of the list, row, KV group) that selects --
 * every workgroup of a group computes the same list -- attends to its slice
 * and publishes a split partial; the workgroup that finishes last merges the
 * slices in order.  workspace: bsa_decode_step_workspace_bytes() bytes
 * (logits, softmax partials, split-KV partials and a slice counter per row
 * that the first launch clears; no initial contents needed; calls that
 * overlap on one workspace race).  Errors: as the two entry points it
 * combines; BSA_ERR_UNSUPPORTED for q_block != 1, pooled or dual-band
 * selection, or NB > 4096.
 * ------------------------------------------------------------------------ */
size_t bsa_decode_step_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, const bsa_select_params* p);

bsa_status bsa_decode_step(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, float* k_mean,
                           float* k_energy, int32_t refresh_block, const bsa_select_params* p, int32_t* idx,
                           int32_t* cnt, const bsa_tensor* o, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ------------------------------------------------------------------------ *
 * Locality pruning (LoSA sec. 2): row r of a denoising block is active when
 * the mean over heads and dims of (q_cur - q_prev)^2 exceeds theta (taken in
 * fp32).  q_cur/q_prev [B, H, R, D] bf16/f32 of the same shape; writes
 * row_mask [B, R] (1 active / 0 stable) and, if non-NULL, mse [B, R] f32.
 * ------------------------------------------------------------------------ */
bsa_status bsa_active_rows(const bsa_tensor* q_cur, const bsa_tensor* q_prev, float theta,
                           uint8_t* row_mask, float* mse, void* stream);

/* ------------------------------------------------------------------------ *
 * Attention over the selected blocks (FASA sec. 2, focused attention: full
 * head-dim attention on the chosen tokens at their original positions).
 *
 * Each query row of block i (rows with row_mask = 1, or all rows when
 * row_mask is NULL) of head h attends to the tokens of the blocks listed in
 * idx[b][h / G][i][0 .. cnt-1]; with causal = 1 keys after the row's absolute
 * position q_pos0 + r are masked.  Exact online softmax in fp32 from bf16/f32
 * inputs:  O = sum_t softmax_t(scale * q . k_t) v_t,
 *          LSE = ln sum_t exp(scale * q . k_t)   (natural log, scale included).
 * A row that sees no key gets O = 0 and LSE = -inf.  Rows with row_mask = 0
 * are NOT written: the caller's cached O/LSE stay in place (LoSA sec. 2, stable
 * tokens reuse the previous step's output and statistics).
 * q, k, v share dtype; o has q's shape and either q's dtype or f32 (the fp32
 * result before rounding); lse is [B, Hq, Lq] f32
 * contiguous.  Supported: bf16 with D = 128 and kv_block in {64, 128}; f32
 * or D = 64 only for single-row query blocks (decode).  workspace:
 * bsa_attention_workspace_bytes() bytes: when nonzero, its first 65536
 * bytes hold arrival counters and the rest the split-KV partial results.
 * The counters must be ZERO on the first call with a workspace (clear it
 * once after allocating it); every call leaves them zero, for calls of any
 * shape, so they need no clearing after that -- unless the buffer has served
 * anything else in between.  (Single-row query blocks merge their split-KV
 * slices in the attention launch: the workgroup that finishes a row's last
 * slice, found with these counters, merges them.)  Counters that are not zero
 * give wrong outputs, not an error.  Calls that overlap on one workspace race.
 * ------------------------------------------------------------------------ */
typedef struct {
  float scale;
  int32_t kv_block;
  int32_t q_block;
  int32_t q_pos0;
  int32_t causal;
  int32_t cap;               /* entries per index list (as given to bsa_select_blocks) */
} bsa_attn_params;

size_t bsa_attention_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, const bsa_attn_params* p);

bsa_status bsa_sparse_attention_fwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                    const int32_t* idx, const int32_t* cnt, const bsa_attn_params* p,
                                    const uint8_t* row_mask, const bsa_tensor* o, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * bsa_sparse_attention_fwd without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, results and errors as
 * bsa_sparse_attention_fwd; the arrival counters and split-KV partials go
 * to a static device array of bsa_noalloc_scratch_bytes() bytes (64 MiB)
 * that each GPU the library runs on holds until the process ends (its
 * address is looked up once per device, on the first call there).  The call
 * allocates and frees nothing.  Errors besides those of
 * bsa_sparse_attention_fwd: BSA_ERR_WORKSPACE when the call needs more
 * scratch than that (the size bsa_attention_workspace_bytes reports);
 * BSA_ERR_INVALID when `stream` belongs to a device other than the current
 * one.  The array starts zeroed and keeps the last call's contents; every
 * call leaves the counters zero, so nothing needs clearing.  Calls that
 * overlap on one GPU share it and race, so keep them on one stream or order
 * them.
 * ------------------------------------------------------------------------ */
size_t bsa_noalloc_scratch_bytes(void);

bsa_status bsa_sparse_attention_fwd_noalloc(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                            const int32_t* idx, const int32_t* cnt, const bsa_attn_params* p,
                                            const uint8_t* row_mask, const bsa_tensor* o, float* lse,
                                            void* stream);

/* ------------------------------------------------------------------------ *
 * Softmax-threshold attention (BLASST sec. 2).  Per head and query tile of
 * `tile` rows, KV tiles are visited from the last one the tile can see down
 * to tile 0.  For a visited tile, S = scale * q k^T (causal-masked) and
 * tm_r = max of row r over the tile; row r votes keep when tm_r is finite and
 * either its running max m_r is still -inf or tm_r - m_r >= ln(lambda).  The
 * tile is processed (exp, V load, PV product, m_r = max(m_r, tm_r)) when any
 * row of the query tile votes keep, and skipped entirely otherwise.
 * lambda = 0 never skips (plain causal attention); lambda must lie in [0, 1].
 * O (q's shape; bf16 or f32), lse [B, Hq, Lq] f32.  Optional diagnostics:
 * kept_tiles [B, Hq, NQT] int32 (tiles processed per query tile) and keep_map
 * [B, Hq, NQT, NKT] uint8 (1 = processed; entries of tiles never visited are
 * left unwritten).  Supported: bf16, D = 128, tile = 128, Lq == L (self
 * attention from position q_pos0 = 0) or non-causal.
 * ------------------------------------------------------------------------ */
typedef struct {
  float scale;
  float lambda;
  int32_t tile;
  int32_t causal;
} bsa_thresh_params;

bsa_status bsa_threshold_attention_fwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                       const bsa_thresh_params* p, const bsa_tensor* o, float* lse,
                                       int32_t* kept_tiles, uint8_t* keep_map, void* stream);

/* ------------------------------------------------------------------------ *
 * Softmax-threshold decode (BLASST sec. 2, decode kernel: the same skip rule,
 * where the saving is the V load of a skipped block).  One query row per
 * head, q [B, Hq, 1, D], attending to all L keys of k, v [B, Hkv, L, D].  The
 * keys are cut into tiles of 64; per head, the tiles are visited from the
 * newest down with a running max m (log of the largest logit kept so far):
 * with tm the tile's largest logit scale * q . k, the newest tile is kept,
 * and an older one when tm - m >= ln(lambda); a kept tile raises m.  A
 * skipped tile never exceeds m, so m before a tile is the max over all newer
 * tiles, and the decisions do not depend on kv_split.  O (bf16 or f32, q's
 * shape) and lse [B, Hq, 1] (natural log) are the exact softmax over every
 * head's kept tiles.  kv_split (keys per slice) sets how the work is cut:
 * each slice's kept keys are summed by one workgroup and the slices are
 * merged in order.  V of a tile is loaded only when some head of its KV
 * group keeps it.  lambda in [0, 1]; lambda = 0 keeps every tile and runs a
 * variant with the skip test compiled out (dense decode over all L keys).
 * Optional: kept_tiles [B, Hq] int32 (tiles kept per head) and keep_map
 * [B, Hq, ceil(L / 64)] uint8 (1 = kept).  Supported: bf16, D = 128, group
 * size 1, 2, 4 or 8, kv_split a multiple of 64 in [64, 2048], v row stride
 * times 2 * kv_split below 2^31 bytes.  workspace:
 * bsa_threshold_decode_workspace_bytes() bytes (scores, tile maxima and
 * per-slice partial results; no initial contents needed; calls that overlap
 * on one workspace, or on one kept_tiles array, race).  Errors:
 * BSA_ERR_INVALID for bad shapes, strides, lambda or scale, a missing lse
 * or a misaligned workspace; BSA_ERR_UNSUPPORTED outside the supported set;
 * BSA_ERR_WORKSPACE when the workspace is smaller than required.
 * ------------------------------------------------------------------------ */
size_t bsa_threshold_decode_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, int32_t kv_split);

bsa_status bsa_threshold_decode_fwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, float scale,
                                    float lambda, int32_t kv_split, const bsa_tensor* o, float* lse,
                                    int32_t* kept_tiles, uint8_t* keep_map, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Selected blocks plus a sliding window in one decode pass (NSA structure
 * section: parallel branches over the selected blocks and a sliding window of
 * the newest w tokens, w = 512 on the page; the learned compression branch is
 * not here).  Arguments as bsa_sparse_attention_fwd for decode rows
 * (q_block = 1, any Lq rows, row r at position q_pos0 + r), no row mask, plus
 * window w > 0: row r's window is the w keys ending at its position (fewer
 * near the start).  Each branch is an exact softmax of its own; gates
 * [B, Hq, Lq, 2] f32 (the branch weights a model's gate would give) or NULL
 * for weights 1 and 1.  Writes o = g_sel O_sel + g_win O_win (q's dtype or
 * f32) and lse [B, Hq, Lq, 2] (natural log of each branch's softmax
 * denominator; -inf for an empty list).  K/V of the two branches stream in
 * the same launch, which also merges them.  workspace:
 * bsa_window_decode_workspace_bytes() bytes, laid out and kept as
 * bsa_sparse_attention_fwd's (arrival counters in the first 65536 bytes,
 * zero on the first call, left zero by every call).
 * Errors as bsa_sparse_attention_fwd; BSA_ERR_UNSUPPORTED for q_block > 1;
 * BSA_ERR_INVALID for w <= 0.
 * ------------------------------------------------------------------------ */
size_t bsa_window_decode_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, const bsa_attn_params* p,
                                         int32_t window);

bsa_status bsa_window_decode_fwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, const int32_t* idx,
                                 const int32_t* cnt, const bsa_attn_params* p, int32_t window, const float* gates,
                                 const bsa_tensor* o, float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* ------------------------------------------------------------------------ *
 * Token importance on a caller-given set of frequency chunks (FASA sec. 2,
 * token importance prediction; the offline calibration that finds a head's
 * dominant chunks is not here).  q [B, Hq, 1, D], k [B, Hkv, L, D], bf16,
 * D = 128, Hq / Hkv in {1, 2, 4, 8}, L <= 65536.  fc_mask [Hq, D/2] uint8
 * (device): 1 marks a chunk whose two dims (i, i + D/2 for BSA_ROPE_HALF;
 * 2i, 2i + 1 for BSA_ROPE_INTERLEAVED) count.  Each head's score of token t
 * is q . k_t over the marked dims only; idx [B, Hq, budget] int32 gets the
 * min(budget, L) best tokens in ascending order (ties: lower token first),
 * cnt [B, Hq] their number; budget at most 2048 and at most
 * 16384 / ceil(L / 4096) (1024 at 64K).  workspace:
 * bsa_token_select_workspace_bytes() bytes, no initial contents.  Errors: BSA_ERR_INVALID for shapes, layout,
 * a null mask or output, budget <= 0 or a misaligned workspace;
 * BSA_ERR_UNSUPPORTED outside the supported set; BSA_ERR_WORKSPACE.
 * ------------------------------------------------------------------------ */
size_t bsa_token_select_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, int32_t budget);

bsa_status bsa_token_select(const bsa_tensor* q, const bsa_tensor* k, const uint8_t* fc_mask, int32_t layout,
                            int32_t budget, int32_t* idx, int32_t* cnt, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------------------ *
 * Attention of every query head over its own token list (FASA sec. 2,
 * focused attention: all dims, tokens at their original positions).  q
 * [B, Hq, Lq, D], k/v [B, Hkv, L, D] (bf16 or f32, D 64 or 128), idx
 * [B, Hq, Lq, cap] int32 token indices < L (any order, no repeats) and cnt
 * [B, Hq, Lq] their number (<= cap): the layout bsa_token_select writes for
 * Lq = 1.  Writes o (q's dtype or f32) and lse [B, Hq, Lq] (natural log;
 * -inf and O = 0 for an empty list).  workspace:
 * bsa_token_attention_workspace_bytes() bytes, laid out and kept as
 * bsa_sparse_attention_fwd's: arrival counters in the first 65536 bytes,
 * zero on the first call with the workspace and left zero by every call.
 * Errors as bsa_sparse_attention_fwd.
 * ------------------------------------------------------------------------ */
size_t bsa_token_attention_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, int32_t cap);

bsa_status bsa_token_attention_fwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, const int32_t* idx,
                                   const int32_t* cnt, int32_t cap, float scale, const bsa_tensor* o, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Merge of two attention states over disjoint key sets (LoSA sec. 2: a stable
 * token of a denoising block reuses its cached prefix-attention output and
 * statistics; the full attention combines that state with the one over the
 * block's own keys).  For each (batch, head, row):
 *   lse = ln(e^lse_a + e^lse_b),  O = e^(lse_a - lse) O_a + e^(lse_b - lse) O_b.
 * o_a, o_b: [B, H, L, D], bf16 or f32 each (any strides as for every tensor);
 * lse_a, lse_b: [B, H, L] f32, natural log, -inf for an empty state (its O is
 * then ignored).  Outputs o [B, H, L, D] bf16 or f32 and lse [B, H, L] f32;
 * rows where both states are empty get O = 0 and lse = -inf.  o may be o_a or
 * o_b (the same tensor, elementwise in place) and lse may be lse_a or lse_b.
 * Errors: BSA_ERR_INVALID for null pointers, differing shapes or a misaligned
 * tensor; BSA_ERR_UNSUPPORTED for a head dim other than 64 or 128.  Nothing
 * is allocated; the call is enqueued on stream.
 * ------------------------------------------------------------------------ */
bsa_status bsa_merge_attention_states(const bsa_tensor* o_a, const float* lse_a, const bsa_tensor* o_b,
                                      const float* lse_b, const bsa_tensor* o, float* lse, void* stream);

/* ------------------------------------------------------------------------ *
 * One denoising step's attention over the block's own keys, merged with the
 * cached prefix state (LoSA sec. 2: each row's prefix attention output and
 * statistics are kept between steps; the block's own tokens are attended in
 * both directions).  q [B, Hq, R, D], kb/vb [B, Hkv, R, D] (the block's keys
 * and values; Hkv divides Hq), bf16, D = 128, 1 <= R <= 32.  o_pre [B, Hq,
 * R, D] bf16 or f32 and lse_pre [B, Hq, R] f32 (natural log; -inf for an
 * empty prefix) hold the prefix state.  Writes o [B, Hq, R, D] bf16 or f32
 * and lse [B, Hq, R]: the exact softmax of scale * q . k over the prefix
 * keys behind the cached state and the block's R keys.  o may be o_pre and
 * lse may be lse_pre (in place).  Errors: BSA_ERR_INVALID for null pointers,
 * mismatched shapes or dtypes, misaligned tensors or a bad scale;
 * BSA_ERR_UNSUPPORTED outside bf16, D = 128, R <= 32.
 * ------------------------------------------------------------------------ */
bsa_status bsa_block_attention_merge(const bsa_tensor* q, const bsa_tensor* kb, const bsa_tensor* vb, float scale,
                                     const bsa_tensor* o_pre, const float* lse_pre, const bsa_tensor* o, float* lse,
                                     void* stream);

/* Status text and the calling thread's last error detail. */
/* ------------------------------------------------------------------------ *
 * One denoising step of a block-wise diffusion LM with locality pruning, in
 * three launches (LoSA sec. 2: only the rows whose queries changed since the
 * previous step recompute their prefix attention, over the union of their
 * selected blocks; every row then attends to the block's own keys and merges
 * with its prefix state).  The results are those of, in order,
 *   bsa_active_rows(q, q_prev, theta, row_mask, mse);
 *   bsa_select_blocks(q, NULL, k_mean, NULL, Hkv, NB, p, row_mask, idx, cnt,
 *                     NULL, NULL, ...);
 *   bsa_sparse_attention_fwd(q, k, v, idx, cnt, {p->scale, p->kv_block, R,
 *                     p->q_pos0, p->causal, p->cap}, row_mask, cache_o,
 *                     cache_lse, ...);
 *   bsa_block_attention_merge(q, kb, vb, p->scale, cache_o, cache_lse, o, lse);
 * bit for bit: the same arithmetic in the same order.
 * q, q_prev [B, Hq, R, D] bf16, D = 128, 1 <= R <= 32, R * Hq / Hkv <= 128;
 * k, v [B, Hkv, L, D] bf16 (the prefix), NB = ceil(L / p->kv_block) <= 4096,
 * kv_block 64 or 128; k_mean [B, Hkv, NB, D] f32 (bsa_build_block_summaries
 * of k); kb, vb [B, Hkv, R, D] bf16 (the block's own keys and values).
 * p: one query block of raw rows (q_block = R), one band; the budget, forced
 * blocks, causality and cap as bsa_select_blocks.  cache_o [B, Hq, R, D] f32
 * and cache_lse [B, Hq, R]: the prefix state, read for stable rows and
 * rewritten for active ones.  Writes row_mask [B, R] (and mse [B, R] if not
 * NULL), idx [B, Hkv, 1, cap] / cnt [B, Hkv, 1] (the union list), o [B, Hq,
 * R, D] bf16 or f32 and lse [B, Hq, R].
 * Launches: the block logits of every row with the active-row test as extra
 * workgroups; per (slice of the list, KV group) the picks of the active rows
 * (one wavefront per row; every workgroup of a group forms the same union),
 * the slice's split partials; per (4 rows, query head) the combine of the
 * partials into the cache, the block tile and the merge.
 * workspace: bsa_denoise_step_workspace_bytes() bytes (logits, split
 * partials; no initial contents needed; calls that overlap on one workspace
 * race).  Errors: as the entry points it combines; BSA_ERR_UNSUPPORTED
 * outside the shapes above.
 * ------------------------------------------------------------------------ */
size_t bsa_denoise_step_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, const bsa_select_params* p);

bsa_status bsa_denoise_step(const bsa_tensor* q, const bsa_tensor* q_prev, float theta, const float* k_mean,
                            const bsa_tensor* k, const bsa_tensor* v, const bsa_tensor* kb, const bsa_tensor* vb,
                            const bsa_select_params* p, const bsa_tensor* cache_o, float* cache_lse,
                            uint8_t* row_mask, float* mse, int32_t* idx, int32_t* cnt, const bsa_tensor* o,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream);

const char* bsa_status_string(int32_t status);
const char* bsa_last_error(void);
int32_t bsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
