// C ABI of libbsa: host-side validation, workspace sizing and dispatch.
// Every argument is checked before anything is enqueued; a non-OK status
// leaves all outputs untouched and records a message for bsa_last_error().
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "internal.h"
#include "pick.h"
#include "split.h"

namespace bsa {

static thread_local char g_err[512] = "";

bsa_status fail(bsa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bsa_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = 0;
  return BSA_OK;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape, dtype and alignment checks common to every tensor argument.
static bsa_status check_tensor(const bsa_tensor* t, const char* name, bool allow_empty_l) {
  if (!t) return fail(BSA_ERR_INVALID, "%s: null tensor descriptor", name);
  if (t->dtype != BSA_BF16 && t->dtype != BSA_F32) return fail(BSA_ERR_INVALID, "%s: unknown dtype %d", name, t->dtype);
  if (t->B <= 0 || t->H <= 0 || t->D <= 0 || t->L < 0 || (!allow_empty_l && t->L == 0))
    return fail(BSA_ERR_INVALID, "%s: bad shape [%d,%d,%d,%d]", name, t->B, t->H, t->L, t->D);
  if (t->D != 64 && t->D != 128) return fail(BSA_ERR_UNSUPPORTED, "%s: head dim %d (supported: 64, 128)", name, t->D);
  if (!t->data) return fail(BSA_ERR_INVALID, "%s: null data pointer", name);
  const int64_t es = (int64_t)dtype_size(t->dtype);
  if (!aligned16(t->data)) return fail(BSA_ERR_INVALID, "%s: data not 16-byte aligned", name);
  if (t->stride_b < 0 || t->stride_h < 0 || t->stride_l < 0) return fail(BSA_ERR_INVALID, "%s: negative stride", name);
  if ((t->stride_b * es) % 16 || (t->stride_h * es) % 16 || (t->stride_l * es) % 16)
    return fail(BSA_ERR_INVALID, "%s: strides must be multiples of 16 bytes", name);
  if (t->L > 1 && t->stride_l < t->D) return fail(BSA_ERR_INVALID, "%s: rows overlap (stride_l < D)", name);
  return BSA_OK;
}

static bool same_dims(const bsa_tensor* a, const bsa_tensor* b) {
  return a->B == b->B && a->H == b->H && a->L == b->L && a->D == b->D;
}
static bool same_shape(const bsa_tensor* a, const bsa_tensor* b) { return same_dims(a, b) && a->dtype == b->dtype; }

}  // namespace bsa

using namespace bsa;

extern "C" {

int32_t bsa_version(void) { return 1; }

const char* bsa_status_string(int32_t s) {
  switch (s) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case BSA_ERR_CAPACITY: return "index-list capacity too small";
    case BSA_ERR_WORKSPACE: return "workspace too small";
    case BSA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* bsa_last_error(void) { return g_err; }

// --------------------------------------------------------------- summaries ---
bsa_status bsa_build_block_summaries(const bsa_tensor* x, int32_t block_size, int32_t layout, int32_t first_block,
                                     int32_t num_blocks, float* mean, float* energy, void* stream) {
  bsa_status st = check_tensor(x, "x", true);
  if (st != BSA_OK) return st;
  if (block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128 && block_size != 256)
    return fail(BSA_ERR_UNSUPPORTED, "block_size %d (supported: 16, 32, 64, 128, 256)", block_size);
  if (layout != BSA_ROPE_HALF && layout != BSA_ROPE_INTERLEAVED) return fail(BSA_ERR_INVALID, "layout %d", layout);
  if (!mean) return fail(BSA_ERR_INVALID, "mean: null pointer");
  const int NB = (int)ceil_div(x->L, block_size);
  if (first_block < 0 || first_block > NB) return fail(BSA_ERR_INVALID, "first_block %d outside [0, %d]", first_block, NB);
  const int n = num_blocks < 0 ? NB - first_block : num_blocks;
  if (first_block + n > NB) return fail(BSA_ERR_INVALID, "blocks %d..%d beyond NB = %d", first_block, first_block + n - 1, NB);
  if (n == 0) { g_err[0] = 0; return BSA_OK; }
  launch_summaries(*x, block_size, layout, first_block, n, mean, energy, static_cast<hipStream_t>(stream));
  return check_launch("block summaries");
}

// --------------------------------------------------------------- selection ---
static bsa_status validate_select(const bsa_tensor* q, int32_t Hkv, int32_t NB, const bsa_select_params* p,
                                  SelectPlan& pl) {
  if (!p) return fail(BSA_ERR_INVALID, "params: null");
  bsa_status st = check_tensor(q, "q", false);
  if (st != BSA_OK) return st;
  if (p->pooled_q && q->dtype != BSA_F32) return fail(BSA_ERR_INVALID, "pooled queries must be f32");
  if (Hkv <= 0 || q->H % Hkv) return fail(BSA_ERR_INVALID, "num_kv_heads %d must divide Hq = %d", Hkv, q->H);
  if (NB <= 0) return fail(BSA_ERR_INVALID, "num_kv_blocks %d", NB);
  if (NB > 4096) return fail(BSA_ERR_UNSUPPORTED, "num_kv_blocks %d > 4096", NB);
  if (p->kv_block <= 0 || p->q_block <= 0) return fail(BSA_ERR_INVALID, "kv_block/q_block must be positive");
  if (p->topk < 0 || p->topk_num < 0 || p->topk_den <= 0 || p->n_first < 0 || p->n_last < 0)
    return fail(BSA_ERR_INVALID, "negative budget or topk_den <= 0");
  if (p->layout != BSA_ROPE_HALF && p->layout != BSA_ROPE_INTERLEAVED) return fail(BSA_ERR_INVALID, "layout %d", p->layout);
  if (p->dual_band != 0 && p->dual_band != 1) return fail(BSA_ERR_INVALID, "dual_band %d", p->dual_band);
  if (!(p->scale > 0.f) || !std::isfinite(p->scale)) return fail(BSA_ERR_INVALID, "scale must be finite and > 0");
  if (p->q_pos0 < 0 || p->q_len < 0) return fail(BSA_ERR_INVALID, "negative q_pos0/q_len");
  if (p->pooled_q && p->q_len > 0 && ceil_div(p->q_len, p->q_block) != q->L)
    return fail(BSA_ERR_INVALID, "q_len %d does not give %d query blocks of %d", p->q_len, q->L, p->q_block);
  plan_select(*q, NB, *p, pl);
  pl.Hkv = Hkv;
  pl.G = q->H / Hkv;
  const int R = p->pooled_q ? 1 : std::min(p->q_block, pl.Lq);
  const int64_t bound = std::min<int64_t>(NB, (int64_t)R * ((int64_t)pl.kp_max + p->n_first + p->n_last));
  if (p->cap < bound) return fail(BSA_ERR_CAPACITY, "cap %d < %lld (rows per block %d x (k' %d + forced %d))", p->cap,
                                  (long long)bound, R, pl.kp_max, p->n_first + p->n_last);
  const int Rtot = p->pooled_q ? pl.NQB : pl.Lq;
  const size_t nz = (size_t)pl.B * q->H * Rtot * (p->dual_band ? 2 : 1) * (size_t)((NB + 3) & ~3);
  pl.z_bytes = align256(nz * 4);
  // tau [B][Hq][2], then the chunk sums [B][Hkv + Hq][chunks][4]
  pl.tau_bytes = p->dual_band ? align256((size_t)pl.B * q->H * 2 * 4) +
                                    align256((size_t)pl.B * (Hkv + q->H) * tau_chunks(NB, p->pooled_q ? q->L : 0) * 16)
                              : 0;
  const bool multi_row = !p->pooled_q && std::min(p->q_block, pl.Lq) > 1;
  pl.bits_bytes = multi_row ? align256((size_t)pl.B * Hkv * Rtot * 128 * 4) : 0;
  pl.cnt_bytes = 0;
  return BSA_OK;
}

size_t bsa_select_workspace_bytes(const bsa_tensor* q, int32_t num_kv_heads, int32_t num_kv_blocks,
                                  const bsa_select_params* p) {
  SelectPlan pl;
  if (validate_select(q, num_kv_heads, num_kv_blocks, p, pl) != BSA_OK) return 0;
  return pl.z_bytes + pl.tau_bytes + pl.bits_bytes + pl.cnt_bytes;
}

bsa_status bsa_select_blocks(const bsa_tensor* q, const float* q_energy, const float* k_mean, const float* k_energy,
                             int32_t num_kv_heads, int32_t num_kv_blocks, const bsa_select_params* p,
                             const uint8_t* row_mask, int32_t* idx, int32_t* cnt, int32_t* row_picks, float* tau_out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  SelectPlan pl;
  bsa_status st = validate_select(q, num_kv_heads, num_kv_blocks, p, pl);
  if (st != BSA_OK) return st;
  if (!k_mean || !idx || !cnt) return fail(BSA_ERR_INVALID, "k_mean, idx and cnt are required");
  if (!aligned16(k_mean)) return fail(BSA_ERR_INVALID, "k_mean not 16-byte aligned");
  if (p->dual_band) {
    if (!k_energy) return fail(BSA_ERR_INVALID, "dual band needs k_energy");
    if (p->pooled_q && !q_energy) return fail(BSA_ERR_INVALID, "dual band with pooled queries needs q_energy");
  }
  if (row_mask && p->pooled_q) return fail(BSA_ERR_INVALID, "row_mask applies to raw query rows only");
  const size_t need = pl.z_bytes + pl.tau_bytes + pl.bits_bytes + pl.cnt_bytes;
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(BSA_ERR_INVALID, "workspace not 16-byte aligned");
  launch_select(*q, p->pooled_q ? q_energy : nullptr, k_mean, k_energy, *p, pl, row_mask, idx, cnt, row_picks,
                tau_out, workspace, static_cast<hipStream_t>(stream));
  return check_launch("block selection");
}

bsa_status bsa_select_blocks_refresh(const bsa_tensor* k, int32_t refresh_block, const bsa_tensor* q, float* k_mean,
                                     float* k_energy, int32_t num_kv_heads, int32_t num_kv_blocks,
                                     const bsa_select_params* p, const uint8_t* row_mask, int32_t* idx, int32_t* cnt,
                                     int32_t* row_picks, void* workspace, size_t workspace_bytes, void* stream) {
  SelectPlan pl;
  bsa_status st = validate_select(q, num_kv_heads, num_kv_blocks, p, pl);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(k, "k", false)) != BSA_OK) return st;
  if (p->pooled_q || p->dual_band)
    return fail(BSA_ERR_UNSUPPORTED, "the in-selection refresh takes raw query rows and one band");
  if (k->dtype != q->dtype || k->B != q->B || k->H != num_kv_heads || k->D != q->D)
    return fail(BSA_ERR_INVALID, "k does not match q and num_kv_heads");
  if (ceil_div(k->L, p->kv_block) != num_kv_blocks)
    return fail(BSA_ERR_INVALID, "num_kv_blocks %d != ceil(L / kv_block) = %lld", num_kv_blocks,
                (long long)ceil_div(k->L, p->kv_block));
  if (refresh_block < 0 || refresh_block >= num_kv_blocks)
    return fail(BSA_ERR_INVALID, "refresh_block %d outside [0, %d)", refresh_block, num_kv_blocks);
  if (p->causal && (int64_t)refresh_block * p->kv_block > p->q_pos0)
    return fail(BSA_ERR_INVALID, "refresh_block %d is not visible to the first query row", refresh_block);
  if (!k_mean || !idx || !cnt) return fail(BSA_ERR_INVALID, "k_mean, idx and cnt are required");
  if (!aligned16(k_mean)) return fail(BSA_ERR_INVALID, "k_mean not 16-byte aligned");
  const size_t need = pl.z_bytes + pl.tau_bytes + pl.bits_bytes + pl.cnt_bytes;
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(BSA_ERR_INVALID, "workspace not 16-byte aligned");
  RefreshArgs ra;
  ra.k = static_cast<const uint8_t*>(k->data);
  ra.ksb = k->stride_b; ra.ksh = k->stride_h; ra.ksl = k->stride_l;
  ra.L = (int)k->L; ra.block = refresh_block; ra.mean = k_mean; ra.energy = k_energy;
  launch_select(*q, nullptr, k_mean, k_energy, *p, pl, row_mask, idx, cnt, row_picks, nullptr, workspace,
                static_cast<hipStream_t>(stream), ra);
  return check_launch("block selection with refresh");
}

// ------------------------------------------------------------- decode step ---
static bsa_status validate_decode_step(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                       const bsa_select_params* p, DStepPlan& pl) {
  if (!p) return fail(BSA_ERR_INVALID, "params: null");
  bsa_status st = check_tensor(q, "q", false);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(k, "k", false)) != BSA_OK) return st;
  if ((st = check_tensor(v, "v", false)) != BSA_OK) return st;
  if (!same_shape(k, v)) return fail(BSA_ERR_INVALID, "k and v differ in shape or dtype");
  if (q->dtype != k->dtype) return fail(BSA_ERR_INVALID, "q and k differ in dtype");
  if (q->B != k->B || q->D != k->D || q->H % k->H) return fail(BSA_ERR_INVALID, "q/k shapes are incompatible");
  const int G = q->H / k->H;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(BSA_ERR_UNSUPPORTED, "Hq/Hkv %d (supported: 1, 2, 4, 8)", G);
  if (p->q_block != 1 || p->pooled_q || p->dual_band)
    return fail(BSA_ERR_UNSUPPORTED, "the decode step takes decode rows (q_block 1), raw queries and one band");
  if (p->kv_block <= 0) return fail(BSA_ERR_INVALID, "kv_block must be positive");
  if (p->topk < 0 || p->topk_num < 0 || p->topk_den <= 0 || p->n_first < 0 || p->n_last < 0)
    return fail(BSA_ERR_INVALID, "negative budget or topk_den <= 0");
  if (p->layout != BSA_ROPE_HALF && p->layout != BSA_ROPE_INTERLEAVED) return fail(BSA_ERR_INVALID, "layout %d", p->layout);
  if (!(p->scale > 0.f) || !std::isfinite(p->scale)) return fail(BSA_ERR_INVALID, "scale must be finite and > 0");
  if (p->q_pos0 < 0) return fail(BSA_ERR_INVALID, "negative q_pos0");
  const int64_t NB = ceil_div(k->L, p->kv_block);
  if (NB > 4096) return fail(BSA_ERR_UNSUPPORTED, "%lld KV blocks > 4096", (long long)NB);
  const int64_t kp = p->topk_num > 0 ? ceil_div((int64_t)p->topk_num * NB, p->topk_den) : p->topk;
  const int64_t bound = std::min<int64_t>(NB, kp + p->n_first + p->n_last);
  if (p->cap < bound)
    return fail(BSA_ERR_CAPACITY, "cap %d < %lld (k' %lld + forced %d)", p->cap, (long long)bound, (long long)kp,
                p->n_first + p->n_last);
  if ((int64_t)p->cap * p->kv_block >= (int64_t(1) << 31)) return fail(BSA_ERR_UNSUPPORTED, "cap * kv_block too large");
  plan_decode_step(*q, *k, *p, pl);
  return BSA_OK;
}

size_t bsa_decode_step_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, const bsa_select_params* p) {
  DStepPlan pl;
  if (!k || validate_decode_step(q, k, k, p, pl) != BSA_OK) return 0;
  return pl.z_bytes + pl.stats_bytes + pl.part_o_bytes + pl.part_ml_bytes + pl.arrival_bytes;
}

bsa_status bsa_decode_step(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, float* k_mean,
                           float* k_energy, int32_t refresh_block, const bsa_select_params* p, int32_t* idx,
                           int32_t* cnt, const bsa_tensor* o, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  DStepPlan pl;
  bsa_status st = validate_decode_step(q, k, v, p, pl);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(o, "o", false)) != BSA_OK) return st;
  if (!same_dims(q, o) || (o->dtype != q->dtype && o->dtype != BSA_F32))
    return fail(BSA_ERR_INVALID, "o must match q in shape, with q's dtype or f32");
  if (!k_mean || !idx || !cnt || !lse) return fail(BSA_ERR_INVALID, "k_mean, idx, cnt and lse are required");
  if (!aligned16(k_mean) || (k_energy && (reinterpret_cast<uintptr_t>(k_energy) & 7u)))
    return fail(BSA_ERR_INVALID, "k_mean must be 16-byte and k_energy 8-byte aligned");
  if (refresh_block < -1 || refresh_block >= pl.NB)
    return fail(BSA_ERR_INVALID, "refresh_block %d outside [-1, %d)", refresh_block, pl.NB);
  if (refresh_block >= 0 && p->causal && (int64_t)refresh_block * p->kv_block > p->q_pos0)
    return fail(BSA_ERR_INVALID, "refresh_block %d is not visible to the first query row", refresh_block);
  const size_t need = pl.z_bytes + pl.stats_bytes + pl.part_o_bytes + pl.part_ml_bytes + pl.arrival_bytes;
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(BSA_ERR_INVALID, "workspace not 16-byte aligned");
  launch_decode_step(*q, *k, *v, k_mean, k_energy, refresh_block, *p, pl, idx, cnt, *o, lse, workspace,
                     static_cast<hipStream_t>(stream));
  return check_launch("decode step");
}

// ------------------------------------------------------------- active rows ---
bsa_status bsa_active_rows(const bsa_tensor* q_cur, const bsa_tensor* q_prev, float theta, uint8_t* row_mask,
                           float* mse, void* stream) {
  bsa_status st = check_tensor(q_cur, "q_cur", false);
  if (st != BSA_OK) return st;
  st = check_tensor(q_prev, "q_prev", false);
  if (st != BSA_OK) return st;
  if (!same_shape(q_cur, q_prev)) return fail(BSA_ERR_INVALID, "q_cur and q_prev differ in shape or dtype");
  if (!row_mask) return fail(BSA_ERR_INVALID, "row_mask: null pointer");
  if (!std::isfinite(theta)) return fail(BSA_ERR_INVALID, "theta must be finite");
  launch_active_rows(*q_cur, *q_prev, theta, row_mask, mse, static_cast<hipStream_t>(stream));
  return check_launch("active rows");
}

// --------------------------------------------------------------- attention ---
static bsa_status validate_attention(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                     const bsa_attn_params* p, AttnPlan& pl) {
  if (!p) return fail(BSA_ERR_INVALID, "params: null");
  bsa_status st = check_tensor(q, "q", true);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(k, "k", false)) != BSA_OK) return st;
  if ((st = check_tensor(v, "v", false)) != BSA_OK) return st;
  if (!same_shape(k, v)) return fail(BSA_ERR_INVALID, "k and v differ in shape or dtype");
  if (q->dtype != k->dtype) return fail(BSA_ERR_INVALID, "q and k differ in dtype");
  if (q->B != k->B || q->D != k->D || q->H % k->H) return fail(BSA_ERR_INVALID, "q/k shapes are incompatible");
  if (p->kv_block <= 0 || p->q_block <= 0 || p->cap <= 0) return fail(BSA_ERR_INVALID, "kv_block, q_block, cap > 0");
  if (!(p->scale > 0.f) || !std::isfinite(p->scale)) return fail(BSA_ERR_INVALID, "scale must be finite and > 0");
  if (p->q_pos0 < 0) return fail(BSA_ERR_INVALID, "negative q_pos0");
  if ((int64_t)p->cap * p->kv_block >= (int64_t(1) << 30))
    return fail(BSA_ERR_UNSUPPORTED, "cap * kv_block too large");
  plan_attention(*q, *k, *p, pl);
  plan_attention_counters(pl);
  if (pl.kind == 0) {
    if (pl.G != 1 && pl.G != 2 && pl.G != 4 && pl.G != 8)
      return fail(BSA_ERR_UNSUPPORTED, "decode path needs Hq/Hkv in {1, 2, 4, 8}, got %d", pl.G);
  } else {
    if (q->dtype != BSA_BF16 || q->D != 128)
      return fail(BSA_ERR_UNSUPPORTED, "multi-row query blocks need bf16 and D = 128");
    if (p->kv_block != 64 && p->kv_block != 128)
      return fail(BSA_ERR_UNSUPPORTED, "multi-row query blocks need kv_block 64 or 128");
    if (pl.kind == 1 && p->q_block > 128) return fail(BSA_ERR_UNSUPPORTED, "q_block %d > 128", p->q_block);
    if (pl.kind == 1 && p->cap > kMaxListMfma)
      return fail(BSA_ERR_UNSUPPORTED, "cap %d > %d for query blocks over 64 rows", p->cap, kMaxListMfma);
    // the tile copies address a row of a K/V tile with a 32-bit byte offset
    if ((int64_t)p->kv_block * 2 * std::max(k->stride_l, v->stride_l) >= (int64_t(1) << 31))
      return fail(BSA_ERR_UNSUPPORTED, "K/V row stride too large for kv_block %d", p->kv_block);
  }
  return BSA_OK;
}

size_t bsa_attention_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, const bsa_attn_params* p) {
  AttnPlan pl;
  if (!k || validate_attention(q, k, k, p, pl) != BSA_OK) return 0;
  return pl.arrival_bytes + pl.part_bytes;
}

bsa_status bsa_sparse_attention_fwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, const int32_t* idx,
                                    const int32_t* cnt, const bsa_attn_params* p, const uint8_t* row_mask,
                                    const bsa_tensor* o, float* lse, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  AttnPlan pl;
  bsa_status st = validate_attention(q, k, v, p, pl);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(o, "o", true)) != BSA_OK) return st;
  if (!same_dims(q, o) || (o->dtype != q->dtype && o->dtype != BSA_F32))
    return fail(BSA_ERR_INVALID, "o must match q in shape, with q's dtype or f32");
  if (!idx || !cnt || !lse) return fail(BSA_ERR_INVALID, "idx, cnt and lse are required");
  const size_t need = pl.arrival_bytes + pl.part_bytes;
  if (need && (!workspace || workspace_bytes < need))
    return fail(BSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (need && !aligned16(workspace)) return fail(BSA_ERR_INVALID, "workspace not 16-byte aligned");
  if (q->L == 0) { g_err[0] = 0; return BSA_OK; }
  launch_attention(*q, *k, *v, idx, cnt, *p, pl, row_mask, *o, lse, workspace, static_cast<hipStream_t>(stream));
  return check_launch("sparse attention");
}

// ------------------------------------------ attention without a workspace ---
// bsa_sparse_attention_fwd_noalloc keeps its arrival counters and split-KV
// partials in this array instead of a caller's workspace.  Each GPU the library
// runs on holds its own copy until the process ends; it starts zeroed, and
// every call leaves the counters zero.  Host code never passes the array's name to a
// kernel: it asks for the device address once per device and uses that.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_dev[kScratchDevices];

// Device address of `scratch` on the device that runs `stream` (which must be
// the current device); looked up on the first call for that device.
static bsa_status scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(BSA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (sdev != dev) return fail(BSA_ERR_INVALID, "stream belongs to device %d, the current device is %d", sdev, dev);
  }
  if (dev < 0 || dev >= kScratchDevices) return fail(BSA_ERR_UNSUPPORTED, "device ordinal %d >= %d", dev, kScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(BSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return BSA_OK;
}

size_t bsa_noalloc_scratch_bytes(void) { return kScratchBytes; }

bsa_status bsa_sparse_attention_fwd_noalloc(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                            const int32_t* idx, const int32_t* cnt, const bsa_attn_params* p,
                                            const uint8_t* row_mask, const bsa_tensor* o, float* lse, void* stream) {
  AttnPlan pl;
  bsa_status st = validate_attention(q, k, v, p, pl);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(o, "o", true)) != BSA_OK) return st;
  if (!same_dims(q, o) || (o->dtype != q->dtype && o->dtype != BSA_F32))
    return fail(BSA_ERR_INVALID, "o must match q in shape, with q's dtype or f32");
  if (!idx || !cnt || !lse) return fail(BSA_ERR_INVALID, "idx, cnt and lse are required");
  const size_t need = pl.arrival_bytes + pl.part_bytes;
  if (need > kScratchBytes)
    return fail(BSA_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the static scratch holds %zu", need,
                kScratchBytes);
  if (q->L == 0) { g_err[0] = 0; return BSA_OK; }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need && (st = scratch_for_stream(s, &ws)) != BSA_OK) return st;
  launch_attention(*q, *k, *v, idx, cnt, *p, pl, row_mask, *o, lse, ws, s);
  return check_launch("sparse attention (static scratch)");
}

// ------------------------------------------------ selection + sliding window ---
static bsa_status validate_window_decode(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                         const bsa_attn_params* p, int32_t window, AttnPlan& pl) {
  bsa_status st = validate_attention(q, k, v, p, pl);
  if (st != BSA_OK) return st;
  if (pl.kind != 0) return fail(BSA_ERR_UNSUPPORTED, "the sliding window joins decode rows only (q_block = 1)");
  if (window <= 0) return fail(BSA_ERR_INVALID, "window %d must be positive", window);
  plan_attention(*q, *k, *p, pl, window);
  plan_attention_counters(pl);
  return BSA_OK;
}

size_t bsa_window_decode_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, const bsa_attn_params* p,
                                         int32_t window) {
  AttnPlan pl;
  if (!k || validate_window_decode(q, k, k, p, window, pl) != BSA_OK) return 0;
  return pl.arrival_bytes + pl.part_bytes;
}

bsa_status bsa_window_decode_fwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, const int32_t* idx,
                                 const int32_t* cnt, const bsa_attn_params* p, int32_t window, const float* gates,
                                 const bsa_tensor* o, float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  AttnPlan pl;
  bsa_status st = validate_window_decode(q, k, v, p, window, pl);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(o, "o", true)) != BSA_OK) return st;
  if (!same_dims(q, o) || (o->dtype != q->dtype && o->dtype != BSA_F32))
    return fail(BSA_ERR_INVALID, "o must match q in shape, with q's dtype or f32");
  if (!idx || !cnt || !lse) return fail(BSA_ERR_INVALID, "idx, cnt and lse are required");
  const size_t need = pl.arrival_bytes + pl.part_bytes;
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(BSA_ERR_INVALID, "workspace not 16-byte aligned");
  if (q->L == 0) { g_err[0] = 0; return BSA_OK; }
  launch_attention(*q, *k, *v, idx, cnt, *p, pl, nullptr, *o, lse, workspace, static_cast<hipStream_t>(stream),
                   window, gates);
  return check_launch("selection + window decode");
}

// ------------------------------------------------ token-level importance ---
static bsa_status validate_token_select(const bsa_tensor* q, const bsa_tensor* k, const uint8_t* fc_mask,
                                        int32_t layout, int32_t budget) {
  bsa_status st = check_tensor(q, "q", false);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(k, "k", false)) != BSA_OK) return st;
  if (q->dtype != k->dtype || q->B != k->B || q->D != k->D || q->H % k->H)
    return fail(BSA_ERR_INVALID, "q/k shapes are incompatible");
  if (q->L != 1) return fail(BSA_ERR_INVALID, "token selection takes one query row (q.L = %d)", q->L);
  if (q->dtype != BSA_BF16 || q->D != 128) return fail(BSA_ERR_UNSUPPORTED, "token selection needs bf16, D = 128");
  const int64_t G = q->H / k->H;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(BSA_ERR_UNSUPPORTED, "group size %d (supported: 1, 2, 4, 8)", (int)G);
  if (k->L > 65536) return fail(BSA_ERR_UNSUPPORTED, "L = %d > 65536 keys", (int)k->L);
  if (layout != BSA_ROPE_HALF && layout != BSA_ROPE_INTERLEAVED) return fail(BSA_ERR_INVALID, "layout %d", layout);
  if (!fc_mask) return fail(BSA_ERR_INVALID, "fc_mask is required");
  if (budget <= 0) return fail(BSA_ERR_INVALID, "budget %d must be positive", budget);
  if (!token_select_supported(*k, budget))
    return fail(BSA_ERR_UNSUPPORTED, "budget %d with L = %d: at most 2048 and at most 16384 / ceil(L / 4096)", budget,
                (int)k->L);
  return BSA_OK;
}

size_t bsa_token_select_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, int32_t budget) {
  if (!q || !k || q->H <= 0 || k->H <= 0 || k->L <= 0 || budget <= 0) return 0;
  return token_select_workspace(*q, *k, budget);
}

bsa_status bsa_token_select(const bsa_tensor* q, const bsa_tensor* k, const uint8_t* fc_mask, int32_t layout,
                            int32_t budget, int32_t* idx, int32_t* cnt, void* workspace, size_t workspace_bytes,
                            void* stream) {
  bsa_status st = validate_token_select(q, k, fc_mask, layout, budget);
  if (st != BSA_OK) return st;
  if (!idx || !cnt) return fail(BSA_ERR_INVALID, "idx and cnt are required");
  const size_t need = token_select_workspace(*q, *k, budget);
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(BSA_ERR_INVALID, "workspace not 16-byte aligned");
  launch_token_select(*q, *k, fc_mask, layout, budget, idx, cnt, nullptr, workspace, static_cast<hipStream_t>(stream));
  return check_launch("token selection");
}

static bsa_status validate_token_attention(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, int32_t cap,
                                           float scale) {
  bsa_status st = check_tensor(q, "q", false);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(k, "k", false)) != BSA_OK) return st;
  if ((st = check_tensor(v, "v", false)) != BSA_OK) return st;
  if (!same_shape(k, v)) return fail(BSA_ERR_INVALID, "k and v differ in shape or dtype");
  if (q->dtype != k->dtype || q->B != k->B || q->D != k->D || q->H % k->H)
    return fail(BSA_ERR_INVALID, "q/k shapes are incompatible");
  if (cap <= 0) return fail(BSA_ERR_INVALID, "cap %d must be positive", cap);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(BSA_ERR_INVALID, "scale must be finite and > 0");
  return BSA_OK;
}

size_t bsa_token_attention_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, int32_t cap) {
  if (!q || !k || q->H <= 0 || k->H <= 0 || cap <= 0) return 0;
  AttnPlan pl;
  plan_token_attention(*q, *k, cap, pl);
  return pl.arrival_bytes + pl.part_bytes;
}

bsa_status bsa_token_attention_fwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, const int32_t* idx,
                                   const int32_t* cnt, int32_t cap, float scale, const bsa_tensor* o, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  bsa_status st = validate_token_attention(q, k, v, cap, scale);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(o, "o", false)) != BSA_OK) return st;
  if (!same_dims(q, o) || (o->dtype != q->dtype && o->dtype != BSA_F32))
    return fail(BSA_ERR_INVALID, "o must match q in shape, with q's dtype or f32");
  if (!idx || !cnt || !lse) return fail(BSA_ERR_INVALID, "idx, cnt and lse are required");
  AttnPlan pl;
  plan_token_attention(*q, *k, cap, pl);
  const size_t need = pl.arrival_bytes + pl.part_bytes;
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(BSA_ERR_INVALID, "workspace not 16-byte aligned");
  launch_token_attention(*q, *k, *v, idx, cnt, cap, scale, pl, *o, lse, workspace, static_cast<hipStream_t>(stream));
  return check_launch("token attention");
}

// ----------------------------------------------------- threshold attention ---
bsa_status bsa_threshold_attention_fwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                       const bsa_thresh_params* p, const bsa_tensor* o, float* lse,
                                       int32_t* kept_tiles, uint8_t* keep_map, void* stream) {
  if (!p) return fail(BSA_ERR_INVALID, "params: null");
  bsa_status st = check_tensor(q, "q", true);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(k, "k", false)) != BSA_OK) return st;
  if ((st = check_tensor(v, "v", false)) != BSA_OK) return st;
  if ((st = check_tensor(o, "o", true)) != BSA_OK) return st;
  if (!same_shape(k, v) || !same_dims(q, o) || (o->dtype != q->dtype && o->dtype != BSA_F32))
    return fail(BSA_ERR_INVALID, "k/v shapes differ, or o does not match q in shape (dtype: q's or f32)");
  if (q->dtype != k->dtype || q->B != k->B || q->D != k->D || q->H % k->H)
    return fail(BSA_ERR_INVALID, "q/k shapes are incompatible");
  if (q->dtype != BSA_BF16 || q->D != 128) return fail(BSA_ERR_UNSUPPORTED, "threshold attention needs bf16, D = 128");
  if (p->tile != 128) return fail(BSA_ERR_UNSUPPORTED, "tile %d (supported: 128)", p->tile);
  if (!(p->lambda >= 0.f && p->lambda <= 1.f)) return fail(BSA_ERR_INVALID, "lambda %g outside [0, 1]", p->lambda);
  if (!(p->scale > 0.f) || !std::isfinite(p->scale)) return fail(BSA_ERR_INVALID, "scale must be finite and > 0");
  if (p->causal && q->L != k->L) return fail(BSA_ERR_UNSUPPORTED, "causal threshold attention needs Lq == L");
  if (!lse) return fail(BSA_ERR_INVALID, "lse is required");
  if (q->L == 0) { g_err[0] = 0; return BSA_OK; }
  launch_threshold(*q, *k, *v, *p, *o, lse, kept_tiles, keep_map, static_cast<hipStream_t>(stream));
  return check_launch("threshold attention");
}

// ------------------------------------------------------ threshold decode ---
static bsa_status validate_threshold_decode(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, float scale,
                                            float lambda, int32_t kv_split) {
  bsa_status st = check_tensor(q, "q", false);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(k, "k", false)) != BSA_OK) return st;
  if ((st = check_tensor(v, "v", false)) != BSA_OK) return st;
  if (!same_shape(k, v)) return fail(BSA_ERR_INVALID, "k and v differ in shape or dtype");
  if (q->dtype != k->dtype || q->B != k->B || q->D != k->D || q->H % k->H)
    return fail(BSA_ERR_INVALID, "q/k shapes are incompatible");
  if (q->L != 1) return fail(BSA_ERR_INVALID, "threshold decode takes one query row (q.L = %d)", q->L);
  if (q->dtype != BSA_BF16 || q->D != 128) return fail(BSA_ERR_UNSUPPORTED, "threshold decode needs bf16, D = 128");
  const int64_t G = q->H / k->H;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(BSA_ERR_UNSUPPORTED, "group size %d (supported: 1, 2, 4, 8)", (int)G);
  if (kv_split < 64 || kv_split > 2048 || kv_split % 64)
    return fail(BSA_ERR_UNSUPPORTED, "kv_split %d (a multiple of 64 in [64, 2048])", kv_split);
  if (v->stride_l * 2 * (int64_t)kv_split >= (int64_t)1 << 31)
    return fail(BSA_ERR_UNSUPPORTED, "v row stride %lld too large for a slice of %d keys", (long long)v->stride_l, kv_split);
  if (!(lambda >= 0.f && lambda <= 1.f)) return fail(BSA_ERR_INVALID, "lambda %g outside [0, 1]", lambda);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(BSA_ERR_INVALID, "scale must be finite and > 0");
  return BSA_OK;
}

bsa_status bsa_merge_attention_states(const bsa_tensor* o_a, const float* lse_a, const bsa_tensor* o_b,
                                      const float* lse_b, const bsa_tensor* o, float* lse, void* stream) {
  bsa_status st = check_tensor(o_a, "o_a", true);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(o_b, "o_b", true)) != BSA_OK) return st;
  if ((st = check_tensor(o, "o", true)) != BSA_OK) return st;
  if (!same_dims(o_a, o_b) || !same_dims(o_a, o)) return fail(BSA_ERR_INVALID, "o_a, o_b and o differ in shape");
  if (!lse_a || !lse_b || !lse) return fail(BSA_ERR_INVALID, "lse_a, lse_b and lse are required");
  const int64_t rows = o_a->B * o_a->H * o_a->L;
  if (rows == 0 || o_a->D == 0) return BSA_OK;
  MergeArgs a;
  a.o_a = o_a->data; a.o_b = o_b->data; a.lse_a = lse_a; a.lse_b = lse_b; a.o = o->data; a.lse = lse;
  a.asb = o_a->stride_b; a.ash = o_a->stride_h; a.asl = o_a->stride_l;
  a.bsb = o_b->stride_b; a.bsh = o_b->stride_h; a.bsl = o_b->stride_l;
  a.osb = o->stride_b; a.osh = o->stride_h; a.osl = o->stride_l;
  a.rows = rows; a.H = (int)o_a->H; a.L = (int)o_a->L; a.D = (int)o_a->D;
  launch_merge_states(a, o_a->dtype, o_b->dtype, o->dtype, static_cast<hipStream_t>(stream));
  return check_launch("merge attention states");
}

bsa_status bsa_block_attention_merge(const bsa_tensor* q, const bsa_tensor* kb, const bsa_tensor* vb, float scale,
                                     const bsa_tensor* o_pre, const float* lse_pre, const bsa_tensor* o, float* lse,
                                     void* stream) {
  bsa_status st = check_tensor(q, "q", false);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(kb, "kb", false)) != BSA_OK) return st;
  if ((st = check_tensor(vb, "vb", false)) != BSA_OK) return st;
  if ((st = check_tensor(o_pre, "o_pre", false)) != BSA_OK) return st;
  if ((st = check_tensor(o, "o", false)) != BSA_OK) return st;
  if (!same_shape(kb, vb)) return fail(BSA_ERR_INVALID, "kb and vb differ in shape or dtype");
  if (q->B != kb->B || q->L != kb->L || q->D != kb->D || q->H % kb->H || q->dtype != kb->dtype)
    return fail(BSA_ERR_INVALID, "q and kb/vb are incompatible");
  if (!same_dims(q, o_pre) || !same_dims(q, o)) return fail(BSA_ERR_INVALID, "o_pre and o must have q's shape");
  if (q->dtype != BSA_BF16 || q->D != 128 || q->L > 32)
    return fail(BSA_ERR_UNSUPPORTED, "block attention needs bf16, D = 128 and at most 32 rows (got %d)", (int)q->L);
  if (!lse_pre || !lse) return fail(BSA_ERR_INVALID, "lse_pre and lse are required");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(BSA_ERR_INVALID, "scale must be finite and > 0");
  BlockMergeArgs a;
  a.q = static_cast<const uint8_t*>(q->data);
  a.kb = static_cast<const uint8_t*>(kb->data);
  a.vb = static_cast<const uint8_t*>(vb->data);
  a.o_pre = o_pre->data; a.lse_pre = lse_pre; a.o = o->data; a.lse = lse;
  a.qsb = q->stride_b; a.qsh = q->stride_h; a.qsl = q->stride_l;
  a.ksb = kb->stride_b; a.ksh = kb->stride_h; a.ksl = kb->stride_l;
  a.vsb = vb->stride_b; a.vsh = vb->stride_h; a.vsl = vb->stride_l;
  a.psb = o_pre->stride_b; a.psh = o_pre->stride_h; a.psl = o_pre->stride_l;
  a.osb = o->stride_b; a.osh = o->stride_h; a.osl = o->stride_l;
  a.B = (int)q->B; a.Hq = (int)q->H; a.G = (int)(q->H / kb->H); a.R = (int)q->L;
  a.pre_f32 = o_pre->dtype == BSA_F32;
  a.scale = scale;
  launch_block_attn_merge(a, o->dtype, static_cast<hipStream_t>(stream));
  return check_launch("block attention merge");
}

// ----------------------------------------------------------- denoise step ---
static bsa_status validate_denoise_step(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v,
                                        const bsa_select_params* p, SelectPlan& sp, bsa_attn_params& ap,
                                        AttnPlan& pl) {
  if (!p) return fail(BSA_ERR_INVALID, "params: null");
  bsa_status st = check_tensor(q, "q", false);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(k, "k", false)) != BSA_OK) return st;
  if ((st = check_tensor(v, "v", false)) != BSA_OK) return st;
  if (!same_shape(k, v)) return fail(BSA_ERR_INVALID, "k and v differ in shape or dtype");
  if (q->dtype != BSA_BF16 || k->dtype != BSA_BF16 || q->D != 128)
    return fail(BSA_ERR_UNSUPPORTED, "the denoising step takes bf16 with D = 128");
  if (q->B != k->B || q->D != k->D || q->H % k->H) return fail(BSA_ERR_INVALID, "q/k shapes are incompatible");
  if (q->L > 32) return fail(BSA_ERR_UNSUPPORTED, "the denoising block has %d rows (at most 32)", (int)q->L);
  if (p->q_block != q->L || p->pooled_q || p->dual_band)
    return fail(BSA_ERR_UNSUPPORTED, "the denoising step takes one query block of raw rows (q_block = %d) and one band",
                (int)q->L);
  if (p->kv_block != 64 && p->kv_block != 128) return fail(BSA_ERR_UNSUPPORTED, "kv_block must be 64 or 128");
  if ((int64_t)q->L * (q->H / k->H) > 128)
    return fail(BSA_ERR_UNSUPPORTED, "rows x group size %d > 128", (int)(q->L * (q->H / k->H)));
  const int64_t NB = ceil_div(k->L, p->kv_block);
  if (NB > 4096) return fail(BSA_ERR_UNSUPPORTED, "%lld KV blocks > 4096", (long long)NB);
  if ((st = validate_select(q, k->H, (int32_t)NB, p, sp)) != BSA_OK) return st;
  ap.scale = p->scale;
  ap.kv_block = p->kv_block;
  ap.q_block = p->q_block;
  ap.q_pos0 = p->q_pos0;
  ap.causal = p->causal;
  ap.cap = p->cap;
  if ((st = validate_attention(q, k, v, &ap, pl)) != BSA_OK) return st;
  if (pl.kind != 2) return fail(BSA_ERR_UNSUPPORTED, "the denoising block does not fit the split gather");
  return BSA_OK;
}

size_t bsa_denoise_step_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, const bsa_select_params* p) {
  SelectPlan sp;
  bsa_attn_params ap;
  AttnPlan pl;
  if (!k || validate_denoise_step(q, k, k, p, sp, ap, pl) != BSA_OK) return 0;
  return sp.z_bytes + pl.part_bytes;
}

bsa_status bsa_denoise_step(const bsa_tensor* q, const bsa_tensor* q_prev, float theta, const float* k_mean,
                            const bsa_tensor* k, const bsa_tensor* v, const bsa_tensor* kb, const bsa_tensor* vb,
                            const bsa_select_params* p, const bsa_tensor* cache_o, float* cache_lse,
                            uint8_t* row_mask, float* mse, int32_t* idx, int32_t* cnt, const bsa_tensor* o, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  SelectPlan sp;
  bsa_attn_params ap;
  AttnPlan pl;
  bsa_status st = validate_denoise_step(q, k, v, p, sp, ap, pl);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(q_prev, "q_prev", false)) != BSA_OK) return st;
  if (!same_shape(q, q_prev)) return fail(BSA_ERR_INVALID, "q and q_prev differ in shape or dtype");
  if (!std::isfinite(theta)) return fail(BSA_ERR_INVALID, "theta must be finite");
  if ((st = check_tensor(kb, "kb", false)) != BSA_OK) return st;
  if ((st = check_tensor(vb, "vb", false)) != BSA_OK) return st;
  if (!same_shape(kb, vb) || kb->dtype != BSA_BF16 || kb->B != q->B || kb->H != k->H || kb->L != q->L ||
      kb->D != q->D)
    return fail(BSA_ERR_INVALID, "kb and vb must be bf16 [B, Hkv, R, D]");
  if ((st = check_tensor(cache_o, "cache_o", false)) != BSA_OK) return st;
  if (!same_dims(q, cache_o) || cache_o->dtype != BSA_F32)
    return fail(BSA_ERR_INVALID, "cache_o must be f32 with q's shape");
  if ((st = check_tensor(o, "o", false)) != BSA_OK) return st;
  if (!same_dims(q, o)) return fail(BSA_ERR_INVALID, "o must have q's shape");
  if (!k_mean || !cache_lse || !row_mask || !idx || !cnt || !lse)
    return fail(BSA_ERR_INVALID, "k_mean, cache_lse, row_mask, idx, cnt and lse are required");
  if (!aligned16(k_mean)) return fail(BSA_ERR_INVALID, "k_mean not 16-byte aligned");
  const size_t need = sp.z_bytes + pl.part_bytes;
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(BSA_ERR_INVALID, "workspace not 16-byte aligned");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // 1: the block logits of every row, with the active-row test of every row in the same launch
  launch_select_logits(*q, k_mean, *p, sp, workspace, s, active_rows_args(*q, *q_prev, theta, row_mask, mse));
  // 2: per (slice, KV group): the active rows' picks, their union and the slice's split partials
  void* part = static_cast<uint8_t*>(workspace) + sp.z_bytes;
  const PickArgs pk = make_pick_args(*p, sp, workspace, row_mask, idx, cnt, nullptr);
  launch_denoise_gather(*q, *k, *v, ap, pl, pk, row_mask, idx, cnt, part, s);
  // 3: per (rows, head): combine of the active rows into the cache, block attention and merge
  DenMergeArgs dm;
  BlockMergeArgs& a = dm.m;
  a.q = static_cast<const uint8_t*>(q->data);
  a.kb = static_cast<const uint8_t*>(kb->data);
  a.vb = static_cast<const uint8_t*>(vb->data);
  a.o_pre = cache_o->data; a.lse_pre = cache_lse; a.o = o->data; a.lse = lse;
  a.qsb = q->stride_b; a.qsh = q->stride_h; a.qsl = q->stride_l;
  a.ksb = kb->stride_b; a.ksh = kb->stride_h; a.ksl = kb->stride_l;
  a.vsb = vb->stride_b; a.vsh = vb->stride_h; a.vsl = vb->stride_l;
  a.psb = cache_o->stride_b; a.psh = cache_o->stride_h; a.psl = cache_o->stride_l;
  a.osb = o->stride_b; a.osh = o->stride_h; a.osl = o->stride_l;
  a.B = (int)q->B; a.Hq = (int)q->H; a.G = (int)(q->H / k->H); a.R = (int)q->L;
  a.pre_f32 = 1;
  a.scale = p->scale;
  const size_t n = (size_t)pl.B * pl.Hkv * pl.NQB * pl.items * pl.qv;
  dm.part_o = static_cast<const float*>(part);
  dm.part_ml = reinterpret_cast<const float*>(static_cast<uint8_t*>(part) + align256(n * pl.D * 4));
  dm.cnt = cnt;
  dm.row_mask = row_mask;
  dm.cache_o = static_cast<float*>(cache_o->data);
  dm.cache_lse = cache_lse;
  dm.Hkv = (int)k->H;
  dm.items = pl.items;
  launch_den_merge(dm, o->dtype, s);
  return check_launch("denoising step");
}

size_t bsa_threshold_decode_workspace_bytes(const bsa_tensor* q, const bsa_tensor* k, int32_t kv_split) {
  if (!q || !k || q->H <= 0 || k->H <= 0 || k->L <= 0 || kv_split < 64 || kv_split % 64) return 0;
  size_t bytes = 0;
  plan_threshold_decode(*q, *k, kv_split, bytes);
  return bytes;
}

bsa_status bsa_threshold_decode_fwd(const bsa_tensor* q, const bsa_tensor* k, const bsa_tensor* v, float scale,
                                    float lambda, int32_t kv_split, const bsa_tensor* o, float* lse,
                                    int32_t* kept_tiles, uint8_t* keep_map, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  bsa_status st = validate_threshold_decode(q, k, v, scale, lambda, kv_split);
  if (st != BSA_OK) return st;
  if ((st = check_tensor(o, "o", false)) != BSA_OK) return st;
  if (!same_dims(q, o) || (o->dtype != q->dtype && o->dtype != BSA_F32))
    return fail(BSA_ERR_INVALID, "o must match q in shape, with q's dtype or f32");
  if (!lse) return fail(BSA_ERR_INVALID, "lse is required");
  size_t need = 0;
  if (!plan_threshold_decode(*q, *k, kv_split, need))
    return fail(BSA_ERR_UNSUPPORTED, "L = %lld: more than 4096 decision chunks per head", (long long)k->L);
  if (!workspace || workspace_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace %zu bytes < %zu required", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(BSA_ERR_INVALID, "workspace not 16-byte aligned");
  launch_threshold_decode(*q, *k, *v, scale, lambda, kv_split, *o, lse, kept_tiles, keep_map, workspace,
                          static_cast<hipStream_t>(stream));
  return check_launch("threshold decode");
}

}  // extern "C"
