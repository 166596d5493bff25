// Argument blocks of the split-KV attention kernels and their combine.
//
// Partial results live in the caller's workspace:
//   part_o [B][Hkv][NQB][items][QV][D]  unnormalised sum of p * v
//   part_ml[B][Hkv][NQB][items][QV][2]  (running max in log2 units, sum of p)
// with QV = q_block * G query vectors per query block (qv = row * G + head).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace bsa {

constexpr int kDecTok = 32;         // list tokens per decode chunk (4 waves x 8 tokens)
constexpr int kDecMaxItems = 512;   // decode slices per (row, group)
constexpr int kDecMinSlice = 32;    // list tokens per decode slice, at least
constexpr int kDecMinSliceMfma = 64;  // ... for the matrix-core form of the attention entry point
constexpr int kDecLaunchWG = 512;   // decode workgroups per launch beyond which slices lengthen
constexpr int kDecWideSub = 4;      // sub-chunks per chunk of a lengthened slice
constexpr int kSplitBlocks = 16;    // list entries per MFMA split workgroup, at most
constexpr int kCombMaxItems = 512;  // split slices the combine can merge
constexpr int kSplitMinBlocks = 1;  // list entries per MFMA split workgroup, at least

// List entries per slice of the MFMA split over `items` launched workgroups:
// an even share of the n entries, at least kSplitMinBlocks (at most
// kSplitBlocks, since items = ceil(cap / kSplitBlocks)).  Every kernel that
// walks or merges the slices uses this one rule.
__host__ __device__ __forceinline__ int split_per(int n, int items) {
  return max(kSplitMinBlocks, (n + items - 1) / items);
}

// List tokens per decode slice for `lists` lists of `toks` list tokens each:
// whole chunks of kDecTok, at least kDecMinSlice, at most kDecMaxItems slices
// per list.  A workgroup's time is mostly fixed round trips (list, K/V,
// partial store, arrival count), so one launch with many lists (a batch of
// decode rows) gives each workgroup more chunks, keeping the launch near
// kDecLaunchWG workgroups; a single decode row keeps 32-token slices, which
// spread its few lists over the most CUs (64 tokens for the matrix-core form of
// the attention entry point, half the partials).  A lengthened slice is a whole
// number of kDecWideSub-sub-chunk chunks, whose K/V rows a workgroup requests
// at once.
inline int64_t dec_slice_tokens(int64_t toks, int64_t lists, int min_slice = kDecMinSlice) {
  const int64_t chunks = (toks + kDecTok - 1) / kDecTok;
  int64_t per = std::max<int64_t>(min_slice / kDecTok, (chunks + kDecMaxItems - 1) / kDecMaxItems);
  const int64_t share = std::max<int64_t>(1, kDecLaunchWG / std::max<int64_t>(1, lists));
  const int64_t want = (chunks + share - 1) / share;
  if (want > 1) per = std::max<int64_t>(per, (want + kDecWideSub - 1) / kDecWideSub * kDecWideSub);
  return per * kDecTok;
}

struct DecArgs {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  int64_t qsb, qsh, qsl, ksb, ksh, ksl, vsb, vsh, vsl;
  const int32_t* idx;
  const int32_t* cnt;
  int cap, NQB, Hkv, L, kv_block, causal, q_pos0, Lq, items, tok_per_item;
  float c2;                       // scale * log2(e)
  const uint8_t* row_mask;
  float* part_o;
  float* part_ml;
  int win = 0;                    // > 0: items past the list's walk the win keys ending at the row
  int kv_div = 1;                 // lists per K/V head (per-query-head token lists: the group size)
  // Non-null: the slices are merged in the same launch by the last workgroup of each (row, group)
  // to finish, counted on arrivals[li * kArrivalStride] (zero on entry, left zero), and O / LSE
  // are written here; null: the partials wait for combine_kernel.
  uint32_t* arrivals = nullptr;
  void* o = nullptr;
  int o_f32 = 0;
  int64_t osb = 0, osh = 0, osl = 0;
  float* lse = nullptr;           // [B][Hq][Lq], or [B][Hq][Lq][2] (list, window) when win > 0
  const float* gates = nullptr;   // win > 0: [B][Hq][Lq][2] branch gates, or null for 1 and 1
};

struct CombArgs {
  const float* part_o;
  const float* part_ml;
  const int32_t* cnt;             // null: every one of the items slices is valid
  int items, unit_num, unit_den;  // valid slices = ceil(cnt * unit_num / unit_den)
  int Hkv, G, NQB, q_block, Lq, D, QV;
  int qvc;                        // query vectors per combine workgroup (256 / D)
  const uint8_t* row_mask;
  void* o;
  int64_t osb, osh, osl;
  float* lse;                     // [B][Hq][Lq], or [B][Hq][Lq][2] (list, window) when win > 0
  int win = 0;                    // sliding window: its items follow the list's (decode only)
  int q_pos0 = 0, L = 0;
  const float* gates = nullptr;   // [B][Hq][Lq][2] branch gates, or null for 1 and 1
  int per_item_from_count = 0;    // 1: each slice took split_per(cnt, items) list entries
};

void launch_decode(const DecArgs& a, int dt, int D, int G, int B, hipStream_t s);
void launch_combine(const CombArgs& a, int odt, int B, hipStream_t s);

}  // namespace bsa
