// dkv_launch.hpp -- host-side launch wrappers of the libdiffkv kernels
// (internal to the library; the exported C-ABI lives in api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dkv_common.hpp"

namespace dkv {

struct Cfg {
  int d, H, G, L, W, lo_en, S_max;
  float ah, al;
  // per-KV-head thresholds (device arrays of H, or null: ah, al for every head)
  const float* ah_head;
  const float* al_head;
  int prompt_rule;  // 0: prompt tokens against alpha/N; 1: against alpha/i (i = position + 1)
  bool plain;       // a tier codec variant: the plain layout (else the default K8V4 / K4V2 layout)
  Codec codec;      // its widths (the default pair when !plain)
  int page_bytes;   // bytes of one unified page under this codec
  // precision levels: K = 2 (the two tiers) or 3, 4 (level 0 high .. K-1
  // low, plain layout); table rows R = ceil(K/2) of L entries (row r: level
  // 2r from the left, 2r+1 from the right); tier state 2K words per unit
  int K, R, LT;     // LT = R * L entries per unit
  float amid[2];    // thresholds of levels 1 .. K-2
  Seg lv[4];        // page layout of each level
};

// The levels as the general kernels see them (passed by value).
struct Levels {
  int K, R, L;      // levels, table rows, row length
  Seg s[4];
  __host__ __device__ int entry(int l, int j) const { return (l >> 1) * L + ((l & 1) ? L - 1 - j : j); }
  __host__ __device__ int T(int l) const { return l == 0 ? kHiTokens : kLoTokens; }
};

inline Levels levels_of(const Cfg& c) {
  Levels v;
  v.K = c.K;
  v.R = c.R;
  v.L = c.L;
  for (int l = 0; l < 4; l++) v.s[l] = c.lv[l];
  return v;
}

struct Pool {
  uint8_t* pages;
  int32_t* list;
  uint64_t* ptr;
  uint32_t* status;
  int64_t P;
  int page_bytes;
};

// classify / init
hipError_t launch_pool_init(const Pool& p, hipStream_t s);
hipError_t launch_state_init(const Cfg& c, int batch, int32_t* table, int32_t* state, hipStream_t s);
hipError_t launch_classify(const Cfg& c, int batch, int64_t total, const int64_t* cu,
                           const float* scores, uint8_t* tiers, int32_t* counts, hipStream_t s);

// prompt compaction
size_t prompt_workspace(const Cfg& c, int batch, int64_t total);
hipError_t launch_prompt(const Cfg& c, const Pool& p, int batch, int64_t total, const int64_t* cu,
                         const uint16_t* k, const uint16_t* v, const float* scores,
                         const uint8_t* tiers, int32_t* table, int32_t* state, void* ws,
                         hipStream_t s);

// generation step and release
size_t step_workspace(const Cfg& c, int batch);
hipError_t launch_step(const Cfg& c, const Pool& p, int batch, const int32_t* seq_len,
                       const uint16_t* k, const uint16_t* v, int32_t* table, int32_t* state,
                       void* ws, hipStream_t s);
// the two halves of launch_step
hipError_t launch_step_plan(const Cfg& c, const Pool& p, int batch, const int32_t* seq_len,
                            const int32_t* table, const int32_t* state, void* ws, hipStream_t s);
// prefix sum of page demand in one workgroup (past the direct-commit size)
hipError_t launch_step_coord(const Cfg& c, const Pool& p, int batch, void* ws, hipStream_t s);
hipError_t launch_step_commit(const Cfg& c, const Pool& p, int batch, const int32_t* seq_len,
                              const uint16_t* k, const uint16_t* v, int32_t* table, int32_t* state,
                              void* ws, hipStream_t s);
size_t release_workspace(const Cfg& c, int batch);
hipError_t launch_release(const Cfg& c, const Pool& p, int batch, const uint8_t* mask,
                          int32_t* table, int32_t* state, void* ws, hipStream_t s);

// decode attention
int attn_splits(const Cfg& c, int batch);
// pages per split: a unit with TPg pages takes them in chunks of
// max(ceil(TPg / S), kSplitMinPages)
constexpr int kSplitMinPages = 16;
__host__ __device__ inline int split_pages(int TPg, int S) {
  if (S <= 1) return TPg;
  const int q = (TPg + S - 1) / S;
  return q > kSplitMinPages ? q : kSplitMinPages;
}
size_t attn_workspace(const Cfg& c, int batch, bool scores);
// mode 0: attention; 1: attention + score update; 2: attention keeping logits.
// reuse_order: the dispatch order a previous call left in ws stands (it
// changes timing only)
hipError_t launch_attn(const Cfg& c, const Pool& p, int batch, const uint16_t* q,
                       const int32_t* table, const int32_t* state, const int32_t* seq_len,
                       float* out, int mode, void* ws, hipStream_t s, bool reuse_order = false);
hipError_t launch_scores(const Cfg& c, const Pool& p, int batch, const int32_t* table,
                         const int32_t* state, const int32_t* seq_len, void* ws, hipStream_t s);
hipError_t launch_scores_merge(const Cfg& c, const Pool& p, int batch, const int32_t* table,
                               const int32_t* state, const int32_t* seq_len, void* ws, hipStream_t s,
                               int merge_S, float* out);
// the split merge: partials [U][S][G][d + 2] -> out; (max, sum) to ml when save
hipError_t launch_attn_merge(const Cfg& c, int batch, int S, const int32_t* seq_len, const float* part,
                             float* out, float* ml, bool save, hipStream_t s);
// tier codec variants (plain layout): attention, score update, workspace
size_t plain_attn_workspace(const Cfg& c, int batch, bool scores);
hipError_t launch_attn_plain(const Cfg& c, const Pool& p, int batch, const uint16_t* q,
                             const int32_t* table, const int32_t* state, const int32_t* seq_len,
                             float* out, int mode, void* ws, hipStream_t s);
hipError_t launch_scores_plain(const Cfg& c, const Pool& p, int batch, const int32_t* table,
                               const int32_t* state, const int32_t* seq_len, void* ws, hipStream_t s);
// generation step then attention for the same step; ws_step and ws_next are
// the two step slots (chain: consecutive chained calls before this one)
hipError_t launch_decode_step(const Cfg& c, const Pool& p, int batch, const int32_t* seq_len,
                              const uint16_t* k, const uint16_t* v, const uint16_t* q, int32_t* table,
                              int32_t* state, float* out, int mode, int chain, void* ws_step, void* ws_attn,
                              void* ws_next, hipStream_t s);

// prompt-phase importance (nqtot: queries in all: total tokens, or batch * nq probes)
size_t importance_workspace(const Cfg& c, int64_t nqtot);
hipError_t launch_importance(const Cfg& c, int batch, int64_t total, const int64_t* cu, int probe, int nq,
                             const uint16_t* q, const uint16_t* k, float* scores, void* ws, hipStream_t s);

// query-free importance from the keys (anchor cosine); raw: anchor of raw keys
size_t keydiff_workspace(const Cfg& c, int batch, int64_t total);
hipError_t launch_keydiff(const Cfg& c, int batch, int64_t total, const int64_t* cu, const uint16_t* k, int raw,
                          float* scores, void* ws, hipStream_t s);

// per-page key bounds [P][2][d] and page scores [batch][H][L]
hipError_t launch_page_bounds(const Cfg& c, const Pool& p, int batch, const int32_t* table, const int32_t* state,
                              float* bounds, hipStream_t s);
hipError_t launch_page_scores(const Cfg& c, int64_t P, int batch, const uint16_t* q, const int32_t* table,
                              const int32_t* state, const int32_t* seq_len, const float* bounds, float* scores,
                              hipStream_t s);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace dkv
