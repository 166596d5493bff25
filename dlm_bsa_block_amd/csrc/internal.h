// Host-side declarations shared by the translation units of libbsa.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/bsa.h"

namespace bsa {

bsa_status fail(bsa_status s, const char* fmt, ...);
bsa_status check_launch(const char* what);

constexpr int kMaxListMfma = 4096;   // list entries a multi-row MFMA workgroup stages in LDS

inline size_t dtype_size(int dt) { return dt == BSA_BF16 ? 2 : 4; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// ---- launchers (arguments already validated) ----
void launch_summaries(const bsa_tensor& x, int block, int layout, int first, int nblk,
                      float* mean, float* energy, hipStream_t s);

// Band-temperature sums are taken over chunks of this many pooled vectors.
constexpr int kTauChunk = 16;
inline int tau_chunks(int nb_k, int nb_q) { return (int)ceil_div(nb_k > nb_q ? nb_k : nb_q, kTauChunk); }

struct SelectPlan {
  int B, Hq, Hkv, G, D, NB, NQB, Lq, R;   // R = selection rows per query block (1 when pooled)
  int kp_max, cap;
  size_t z_bytes, tau_bytes, bits_bytes, cnt_bytes;   // workspace regions, in this order
};
bool plan_select(const bsa_tensor& q, int NB, const bsa_select_params& p, SelectPlan& pl);
// Optional refresh of one block's summary inside the selection (the newest decode block): the logits
// workgroup that holds the block pools it from K, uses it and writes it out.  block < 0: none.
struct RefreshArgs {
  const uint8_t* k = nullptr;        // [B, Hkv, L, D], the selection's dtype
  int64_t ksb = 0, ksh = 0, ksl = 0;
  int L = 0, block = -1;
  float* mean = nullptr;             // the k_mean array (written at `block`)
  float* energy = nullptr;           // the k_energy array, or null
};
void launch_select(const bsa_tensor& q, const float* q_energy, const float* k_mean, const float* k_energy,
                   const bsa_select_params& p, const SelectPlan& pl, const uint8_t* row_mask,
                   int32_t* idx, int32_t* cnt, int32_t* row_picks, float* tau_out, void* ws, hipStream_t s,
                   const RefreshArgs& ra = RefreshArgs());

void launch_active_rows(const bsa_tensor& a, const bsa_tensor& b, float theta, uint8_t* mask, float* mse,
                        hipStream_t s);

// The active-row test of a denoising block (row mean of (q_cur - q_prev)^2 over heads and dims
// against theta); also run as extra workgroups of the denoising step's logits launch.
struct ActiveRowsArgs {
  const uint8_t* a = nullptr;        // q_cur [B, H, R, D]; null: no row jobs in the launch
  const uint8_t* c = nullptr;        // q_prev, same shape and dtype
  int64_t asb = 0, ash = 0, asl = 0, csb = 0, csh = 0, csl = 0;
  int H = 0, R = 0, D = 0;
  float theta = 0.f;
  uint8_t* mask = nullptr;           // [B, R]
  float* mse = nullptr;              // [B, R] or null
  int z0 = 0, slices = 0;            // in a logits launch: first z index of the row jobs, z-slices per batch
};
ActiveRowsArgs active_rows_args(const bsa_tensor& x, const bsa_tensor& y, float theta, uint8_t* mask, float* mse);
// The block logits of bsa_select_blocks alone (one band, no refresh) into the workspace's logit
// region, with the active-row jobs `act` (if act.a is set) in the same launch.
void launch_select_logits(const bsa_tensor& q, const float* k_mean, const bsa_select_params& p,
                          const SelectPlan& pl, void* ws, hipStream_t s, const ActiveRowsArgs& act);

// Merge of two attention states (o_x [B, H, L, D] any of bf16/f32, lse_x [B, H, L] natural log).
struct MergeArgs {
  const void* o_a;
  const void* o_b;
  const float* lse_a;
  const float* lse_b;
  void* o;
  float* lse;
  int64_t asb, ash, asl, bsb, bsh, bsl, osb, osh, osl;
  int64_t rows;                      // B * H * L
  int H, L, D;
};
void launch_merge_states(const MergeArgs& a, int da, int db, int dout, hipStream_t s);

// A denoising block's attention over its own keys merged with the cached prefix state.
struct BlockMergeArgs {
  const uint8_t* q;                  // [B, Hq, R, D] bf16
  const uint8_t* kb;                 // [B, Hkv, R, D] bf16
  const uint8_t* vb;
  const void* o_pre;                 // [B, Hq, R, D] bf16 or f32
  const float* lse_pre;              // [B, Hq, R]
  void* o;                           // [B, Hq, R, D] bf16 or f32
  float* lse;                        // [B, Hq, R]
  int64_t qsb, qsh, qsl, ksb, ksh, ksl, vsb, vsh, vsl, psb, psh, psl, osb, osh, osl;
  int B, Hq, G, R, pre_f32;
  float scale;
};
void launch_block_attn_merge(const BlockMergeArgs& a, int dout, hipStream_t s);

// The fused denoising step's last launch: combine of the split partials of the active rows into the
// prefix cache (f32), then the block attention and merge of every row.
constexpr int kDenRows = 4;          // rows per workgroup
struct DenMergeArgs {
  BlockMergeArgs m;                  // o_pre = the prefix cache (f32, pre_f32 = 1), lse_pre = its lse
  const float* part_o;               // [B][Hkv][items][R * G][D] split partials (query block 0)
  const float* part_ml;              // [B][Hkv][items][R * G][2]
  const int32_t* cnt;                // [B][Hkv] list lengths
  const uint8_t* row_mask;           // [B][R]
  float* cache_o;                    // the prefix cache again, written for active rows
  float* cache_lse;
  int Hkv, items;
};
void launch_den_merge(const DenMergeArgs& a, int dout, hipStream_t s);

struct AttnPlan {
  int kind;                 // 0 = VALU decode split, 1 = MFMA gather (direct), 2 = MFMA gather split
  int B, Hq, Hkv, G, D, Lq, L, NQB;
  int items;                // split-KV items per (b, g, q-block)
  int tok_per_item;         // decode: list tokens per item
  int qv;                   // query vectors per (b, g, q-block) in split mode
  size_t part_bytes;
  // bsa_sparse_attention_fwd's workspace: arrival counters at the front (kArrivalBytes, or 0 for
  // a call without partials), then the partials; merge_in_launch: the decode split merges its
  // slices in its own launch (counters there) instead of a combine launch
  size_t arrival_bytes = 0;
  bool merge_in_launch = false;
};
// Sets the entry point's counter region and whether the decode split merges in its launch.
void plan_attention_counters(AttnPlan& pl);
// win > 0 (decode only): a sliding window of win keys per row joins the list
// (NSA sliding-window branch); gates [B][Hq][Lq][2] or null; lse then [B][Hq][Lq][2].
bool plan_attention(const bsa_tensor& q, const bsa_tensor& k, const bsa_attn_params& p, AttnPlan& pl, int win = 0);
void launch_attention(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, const int32_t* idx,
                      const int32_t* cnt, const bsa_attn_params& p, const AttnPlan& pl, const uint8_t* row_mask,
                      const bsa_tensor& o, float* lse, void* ws, hipStream_t s, int win = 0,
                      const float* gates = nullptr);

// Token importance on a subset of frequency chunks, top-N tokens per query head, and the
// attention of each head over its own token list.
size_t token_select_workspace(const bsa_tensor& q, const bsa_tensor& k, int budget);
bool token_select_supported(const bsa_tensor& k, int budget);
void launch_token_select(const bsa_tensor& q, const bsa_tensor& k, const uint8_t* fc_mask, int layout, int budget,
                         int32_t* idx, int32_t* cnt, float* scores_out, void* ws, hipStream_t s);
void plan_token_attention(const bsa_tensor& q, const bsa_tensor& k, int cap, AttnPlan& pl);
void launch_token_attention(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, const int32_t* idx,
                            const int32_t* cnt, int cap, float scale, const AttnPlan& pl, const bsa_tensor& o,
                            float* lse, void* ws, hipStream_t s);


// One decode step (selection with an optional summary refresh, then attention over the lists) in
// two launches: logits + softmax partials, then selection + split attention per workgroup with the
// merge done by the workgroup that finishes last.
struct DStepPlan {
  int B, Hq, Hkv, G, D, Lq, L, NB, NBp, KPL, P, items, tok_per_item;
  size_t z_bytes, stats_bytes, part_o_bytes, part_ml_bytes, arrival_bytes;   // workspace regions, in this order
};
bool plan_decode_step(const bsa_tensor& q, const bsa_tensor& k, const bsa_select_params& p, DStepPlan& pl);
void launch_decode_step(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, float* k_mean,
                        float* k_energy, int refresh, const bsa_select_params& p, const DStepPlan& pl, int32_t* idx,
                        int32_t* cnt, const bsa_tensor& o, float* lse, void* ws, hipStream_t s);

bool plan_threshold_decode(const bsa_tensor& q, const bsa_tensor& k, int kv_split, size_t& bytes);
void launch_threshold_decode(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, float scale,
                             float lambda, int kv_split, const bsa_tensor& o, float* lse, int32_t* kept,
                             uint8_t* keep_map, void* ws, hipStream_t s);

void launch_threshold(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, const bsa_thresh_params& p,
                      const bsa_tensor& o, float* lse, int32_t* kept, uint8_t* keep_map, hipStream_t s);

}  // namespace bsa
