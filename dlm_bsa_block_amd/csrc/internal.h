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
void launch_select(const bsa_tensor& q, const float* q_energy, const float* k_mean, const float* k_energy,
                   const bsa_select_params& p, const SelectPlan& pl, const uint8_t* row_mask,
                   int32_t* idx, int32_t* cnt, int32_t* row_picks, float* tau_out, void* ws, hipStream_t s);

void launch_active_rows(const bsa_tensor& a, const bsa_tensor& b, float theta, uint8_t* mask, float* mse,
                        hipStream_t s);

struct AttnPlan {
  int kind;                 // 0 = VALU decode split, 1 = MFMA gather (direct), 2 = MFMA gather split
  int B, Hq, Hkv, G, D, Lq, L, NQB;
  int items;                // split-KV items per (b, g, q-block)
  int tok_per_item;         // decode: list tokens per item
  int qv;                   // query vectors per (b, g, q-block) in split mode
  size_t part_bytes;
};
bool plan_attention(const bsa_tensor& q, const bsa_tensor& k, const bsa_attn_params& p, AttnPlan& pl);
void launch_attention(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, const int32_t* idx,
                      const int32_t* cnt, const bsa_attn_params& p, const AttnPlan& pl, const uint8_t* row_mask,
                      const bsa_tensor& o, float* lse, void* ws, hipStream_t s);

bool plan_threshold_decode(const bsa_tensor& q, const bsa_tensor& k, int kv_split, size_t& bytes);
void launch_threshold_decode(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, float scale,
                             float lambda, int kv_split, const bsa_tensor& o, float* lse, int32_t* kept,
                             uint8_t* keep_map, void* ws, hipStream_t s);

void launch_threshold(const bsa_tensor& q, const bsa_tensor& k, const bsa_tensor& v, const bsa_thresh_params& p,
                      const bsa_tensor& o, float* lse, int32_t* kept, uint8_t* keep_map, hipStream_t s);

}  // namespace bsa
