// api.hip -- the exported C-ABI of libdiffkv.so (declared in include/diffkv.h):
// host-side validation, workspace sizing and kernel launches.
#include <hip/hip_runtime.h>

#include "diffkv.h"
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

using namespace dkv;

namespace {

// workspaces hold 8- and 16-byte words at 256-byte offsets
bool ws_ok(const void* ws) { return ws && ((uintptr_t)ws & 255) == 0; }

bool cfg_ok(const diffkv_config* c) {
  if (!c) return false;
  if (c->head_dim != 64 && c->head_dim != 128) return false;
  if (c->num_kv_heads < 1 || c->gqa_group < 1 || c->gqa_group > 16) return false;
  if (c->hi_page_tokens != kHiTokens || c->lo_page_tokens != kLoTokens) return false;
  // max_seq_len < 2^29: a fp32 score sum times a token count is exact in fp64
  if (c->max_seq_len < 1 || c->max_seq_len >= (1 << 29) || c->window < 0) return false;
  if (!(c->alpha_l >= 0.0f) || !(c->alpha_h >= 0.0f)) return false;
  if (c->lo_enabled && c->alpha_l > c->alpha_h) return false;
  if (c->prompt_rule != DIFFKV_RULE_ALPHA_N && c->prompt_rule != DIFFKV_RULE_ALPHA_I) return false;
  if ((c->alpha_h_head == nullptr) != (c->alpha_l_head == nullptr)) return false;
  const bool plain = c->hi_k_bits || c->hi_v_bits || c->lo_k_bits || c->lo_v_bits;
  auto bits_ok = [](int32_t b) { return b == 1 || b == 2 || b == 4 || b == 8; };
  if (plain && !(bits_ok(c->hi_k_bits) && bits_ok(c->hi_v_bits) && bits_ok(c->lo_k_bits) && bits_ok(c->lo_v_bits)))
    return false;
  if (c->num_levels != 0 && c->num_levels != 2) {
    // K = 3 or 4 levels: every width given, the low level on, thresholds
    // descending (the per-head arrays live on the device: the caller keeps
    // alpha_h_head[h] >= alpha_mid[0] and alpha_mid[K-3] >= alpha_l_head[h])
    const int K = c->num_levels;
    if (K != 3 && K != 4) return false;
    if (!plain || !c->lo_enabled) return false;
    float prev = c->alpha_h;
    for (int m = 0; m < K - 2; m++) {
      if (!bits_ok(c->mid_k_bits[m]) || !bits_ok(c->mid_v_bits[m])) return false;
      if (!(c->alpha_mid[m] >= 0.0f)) return false;
      if (c->alpha_h_head == nullptr && c->alpha_mid[m] > prev) return false;
      prev = c->alpha_mid[m];
    }
    if (c->alpha_h_head == nullptr && c->alpha_l > prev) return false;
  }
  return true;
}

Cfg to_cfg(const diffkv_config* c) {
  Cfg r;
  r.d = c->head_dim;
  r.H = c->num_kv_heads;
  r.G = c->gqa_group;
  r.L = (c->max_seq_len + kHiTokens - 1) / kHiTokens + 1;
  r.W = c->window;
  r.lo_en = c->lo_enabled ? 1 : 0;
  r.S_max = c->max_seq_len;
  r.ah = c->alpha_h;
  r.al = c->alpha_l;
  r.ah_head = c->alpha_h_head;
  r.al_head = c->alpha_l_head;
  r.prompt_rule = c->prompt_rule;
  r.plain = c->hi_k_bits || c->hi_v_bits || c->lo_k_bits || c->lo_v_bits;
  r.codec = r.plain ? Codec{c->hi_k_bits, c->hi_v_bits, c->lo_k_bits, c->lo_v_bits} : Codec{8, 4, 4, 2};
  r.page_bytes = r.plain ? plain_page_bytes(r.d, r.codec) : page_bytes_for(r.d);
  r.K = c->num_levels >= 3 ? c->num_levels : 2;
  r.R = (r.K + 1) / 2;
  r.LT = r.R * r.L;
  r.amid[0] = c->alpha_mid[0];
  r.amid[1] = c->alpha_mid[1];
  if (r.K == 2) {
    r.lv[0] = r.plain ? plain_seg(r.d, true, r.codec) : tier_seg(r.d, true);
    r.lv[1] = r.plain ? plain_seg(r.d, false, r.codec) : tier_seg(r.d, false);
    r.lv[2] = r.lv[3] = r.lv[1];
  } else {
    r.page_bytes = 0;
    for (int l = 0; l < 4; l++) {
      const int ll = l < r.K ? l : r.K - 1;
      const int kb = ll == 0 ? c->hi_k_bits : (ll == r.K - 1 ? c->lo_k_bits : c->mid_k_bits[ll - 1]);
      const int vb = ll == 0 ? c->hi_v_bits : (ll == r.K - 1 ? c->lo_v_bits : c->mid_v_bits[ll - 1]);
      r.lv[l] = level_seg(r.d, ll == 0 ? kHiTokens : kLoTokens, kb, vb);
      if (r.lv[l].bytes > r.page_bytes) r.page_bytes = r.lv[l].bytes;
    }
  }
  return r;
}

bool pool_ok(const diffkv_config* c, const diffkv_pool* p) {
  return p && p->pages && p->free_list && p->ptr && p->status && p->num_pages >= 1 &&
         p->num_pages < (int64_t(1) << 31) && p->page_bytes == to_cfg(c).page_bytes;
}

Pool to_pool(const diffkv_pool* p) {
  return Pool{(uint8_t*)p->pages, p->free_list, p->ptr, p->status, p->num_pages, p->page_bytes};
}

int rc(hipError_t e) { return e == hipSuccess ? DIFFKV_OK : DIFFKV_E_HIP; }

}  // namespace

extern "C" {

int32_t diffkv_page_bytes(const diffkv_config* cfg) {
  if (!cfg_ok(cfg)) return -1;
  return to_cfg(cfg).page_bytes;
}

int32_t diffkv_table_len(const diffkv_config* cfg) {
  if (!cfg_ok(cfg)) return -1;
  return to_cfg(cfg).LT;
}

int32_t diffkv_state_words(const diffkv_config* cfg) {
  if (!cfg_ok(cfg)) return -1;
  return 2 * to_cfg(cfg).K;
}

int32_t diffkv_attn_splits(const diffkv_config* cfg, int32_t batch) {
  if (!cfg_ok(cfg) || batch < 0) return -1;
  return attn_splits(to_cfg(cfg), batch);
}

size_t diffkv_workspace_bytes(const diffkv_config* cfg, int32_t op, int32_t batch, int64_t total_tokens) {
  if (!cfg_ok(cfg) || batch < 0 || total_tokens < 0) return 0;
  const Cfg c = to_cfg(cfg);
  switch (op) {
    case DIFFKV_PROMPT: return prompt_workspace(c, batch, total_tokens);
    case DIFFKV_STEP: return step_workspace(c, batch);
    case DIFFKV_RELEASE: return release_workspace(c, batch);
    case DIFFKV_ATTN: return attn_workspace(c, batch, false);
    case DIFFKV_ATTN_SCORES: return attn_workspace(c, batch, true);
    case DIFFKV_DECODE_STEP:
      return align_up(step_workspace(c, batch), 256) + align_up(attn_workspace(c, batch, false), 256) +
             step_workspace(c, batch);
    case DIFFKV_DECODE_STEP_SCORES:
      return align_up(step_workspace(c, batch), 256) + align_up(attn_workspace(c, batch, true), 256) +
             step_workspace(c, batch);
    case DIFFKV_IMPORTANCE: return importance_workspace(c, total_tokens);
    case DIFFKV_KEYDIFF: return keydiff_workspace(c, batch, total_tokens);
    default: return 0;
  }
}

int diffkv_pool_init(const diffkv_config* cfg, const diffkv_pool* pool, void* stream) {
  if (!cfg_ok(cfg) || !pool_ok(cfg, pool)) return DIFFKV_E_INVALID;
  return rc(launch_pool_init(to_pool(pool), (hipStream_t)stream));
}

int diffkv_state_init(const diffkv_config* cfg, int32_t batch, int32_t* page_table, int32_t* tier_state,
                      void* stream) {
  if (!cfg_ok(cfg) || batch < 0 || (batch > 0 && (!page_table || !tier_state))) return DIFFKV_E_INVALID;
  return rc(launch_state_init(to_cfg(cfg), batch, page_table, tier_state, (hipStream_t)stream));
}

int diffkv_classify(const diffkv_config* cfg, int32_t batch, int64_t total_tokens, const int64_t* cu_seqlens,
                    const float* scores, uint8_t* tiers, int32_t* tier_counts, void* stream) {
  if (!cfg_ok(cfg) || batch < 0 || total_tokens < 0) return DIFFKV_E_INVALID;
  if (batch > 0 && (!cu_seqlens || !tier_counts)) return DIFFKV_E_INVALID;
  if (total_tokens > 0 && (!scores || !tiers)) return DIFFKV_E_INVALID;
  if (batch > 65535) return DIFFKV_E_INVALID;
  return rc(launch_classify(to_cfg(cfg), batch, total_tokens, cu_seqlens, scores, tiers, tier_counts,
                            (hipStream_t)stream));
}

int diffkv_compact(const diffkv_config* cfg, const diffkv_pool* pool, int32_t mode, int32_t batch,
                   int64_t total_tokens, const int64_t* cu_seqlens, const int32_t* seq_len, const uint16_t* k,
                   const uint16_t* v, const float* scores, const uint8_t* tiers, const uint8_t* release_mask,
                   int32_t* page_table, int32_t* tier_state, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (!cfg_ok(cfg) || !pool_ok(cfg, pool) || batch < 0 || total_tokens < 0) return DIFFKV_E_INVALID;
  if (batch > 0 && (!page_table || !tier_state)) return DIFFKV_E_INVALID;
  if ((int64_t)batch * cfg->num_kv_heads > 65535) return DIFFKV_E_INVALID;
  const Cfg c = to_cfg(cfg);
  const Pool p = to_pool(pool);
  hipStream_t s = (hipStream_t)stream;
  size_t need = 0;
  switch (mode) {
    case DIFFKV_PROMPT:
      if (batch > 0 && !cu_seqlens) return DIFFKV_E_INVALID;
      if (total_tokens > 0 && (!k || !v || !scores || !tiers)) return DIFFKV_E_INVALID;
      // token rows are read with 16-byte loads
      if (((uintptr_t)k | (uintptr_t)v) & 15u) return DIFFKV_E_INVALID;
      need = prompt_workspace(c, batch, total_tokens);
      if (!ws_ok(workspace) || workspace_bytes < need) return DIFFKV_E_WORKSPACE;
      return rc(launch_prompt(c, p, batch, total_tokens, cu_seqlens, k, v, scores, tiers, page_table, tier_state,
                              workspace, s));
    case DIFFKV_STEP:
      if (c.W < 2) return DIFFKV_E_INVALID;
      if (batch > 0 && (!seq_len || !k || !v)) return DIFFKV_E_INVALID;
      need = step_workspace(c, batch);
      if (!ws_ok(workspace) || workspace_bytes < need) return DIFFKV_E_WORKSPACE;
      return rc(launch_step(c, p, batch, seq_len, k, v, page_table, tier_state, workspace, s));
    case DIFFKV_RELEASE:
      if (batch > 0 && !release_mask) return DIFFKV_E_INVALID;
      need = release_workspace(c, batch);
      if (!ws_ok(workspace) || workspace_bytes < need) return DIFFKV_E_WORKSPACE;
      return rc(launch_release(c, p, batch, release_mask, page_table, tier_state, workspace, s));
    default:
      return DIFFKV_E_INVALID;
  }
}

int diffkv_decode_attn(const diffkv_config* cfg, const diffkv_pool* pool, int32_t batch, const uint16_t* q,
                       const int32_t* page_table, const int32_t* tier_state, const int32_t* seq_len, float* out,
                       int32_t update_scores, void* workspace, size_t workspace_bytes, void* stream) {
  if (!cfg_ok(cfg) || !pool_ok(cfg, pool) || batch < 0) return DIFFKV_E_INVALID;
  if (batch > 0 && (!q || !page_table || !tier_state || !seq_len || !out)) return DIFFKV_E_INVALID;
  if ((int64_t)batch * cfg->num_kv_heads > 65535) return DIFFKV_E_INVALID;
  if (update_scores < 0 || update_scores > 2) return DIFFKV_E_INVALID;
  const Cfg c = to_cfg(cfg);
  const size_t need = attn_workspace(c, batch, update_scores != 0);
  if (!ws_ok(workspace) || workspace_bytes < need) return DIFFKV_E_WORKSPACE;
  return rc(launch_attn(c, to_pool(pool), batch, q, page_table, tier_state, seq_len, out, update_scores,
                        workspace, (hipStream_t)stream));
}

int diffkv_decode_step(const diffkv_config* cfg, const diffkv_pool* pool, int32_t batch, const int32_t* seq_len,
                       const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q, int32_t* page_table,
                       int32_t* tier_state, float* out, int32_t update_scores, int32_t chain, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!cfg_ok(cfg) || !pool_ok(cfg, pool) || batch < 0) return DIFFKV_E_INVALID;
  if (batch > 0 && (!seq_len || !k_new || !v_new || !q || !page_table || !tier_state || !out))
    return DIFFKV_E_INVALID;
  if ((int64_t)batch * cfg->num_kv_heads > 65535) return DIFFKV_E_INVALID;
  if (update_scores < 0 || update_scores > 2 || chain < 0) return DIFFKV_E_INVALID;
  const Cfg c = to_cfg(cfg);
  if (c.W < 2) return DIFFKV_E_INVALID;
  const size_t ws_step = align_up(step_workspace(c, batch), 256);
  const size_t ws_attn = align_up(attn_workspace(c, batch, update_scores != 0), 256);
  const size_t need = ws_step + ws_attn + step_workspace(c, batch);
  if (!ws_ok(workspace) || workspace_bytes < need) return DIFFKV_E_WORKSPACE;
  uint8_t* w = (uint8_t*)workspace;
  return rc(launch_decode_step(c, to_pool(pool), batch, seq_len, k_new, v_new, q, page_table, tier_state, out,
                               update_scores, chain, w, w + ws_step, w + ws_step + ws_attn, (hipStream_t)stream));
}

int diffkv_importance(const diffkv_config* cfg, int32_t mode, int32_t batch, int64_t total_tokens,
                      const int64_t* cu_seqlens, int32_t nq, const uint16_t* q, const uint16_t* k, float* scores,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!cfg_ok(cfg) || batch < 0 || batch > 65535 || total_tokens < 0) return DIFFKV_E_INVALID;
  if (mode != DIFFKV_IMP_CAUSAL && mode != DIFFKV_IMP_PROBE) return DIFFKV_E_INVALID;
  if ((int64_t)cfg->num_kv_heads * cfg->gqa_group > 65535) return DIFFKV_E_INVALID;
  if (batch > 0 && !cu_seqlens) return DIFFKV_E_INVALID;
  if (mode == DIFFKV_IMP_PROBE && (nq < 1 || nq > 65536)) return DIFFKV_E_INVALID;
  if (total_tokens > 0 && (!q || !k || !scores)) return DIFFKV_E_INVALID;
  // rows are read with 16-byte loads
  if (((uintptr_t)q | (uintptr_t)k) & 15u) return DIFFKV_E_INVALID;
  const Cfg c = to_cfg(cfg);
  const int64_t nqtot = mode == DIFFKV_IMP_PROBE ? (int64_t)batch * nq : total_tokens;
  if (!ws_ok(workspace) || workspace_bytes < importance_workspace(c, nqtot)) return DIFFKV_E_WORKSPACE;
  return rc(launch_importance(c, batch, total_tokens, cu_seqlens, mode == DIFFKV_IMP_PROBE ? 1 : 0, nq, q, k,
                              scores, workspace, (hipStream_t)stream));
}

int diffkv_keydiff_scores(const diffkv_config* cfg, int32_t batch, int64_t total_tokens, const int64_t* cu_seqlens,
                          const uint16_t* k, int32_t anchor_raw, float* scores, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!cfg_ok(cfg) || batch < 0 || batch > 65535 || total_tokens < 0) return DIFFKV_E_INVALID;
  if (cfg->num_kv_heads > 65535 || (anchor_raw != 0 && anchor_raw != 1)) return DIFFKV_E_INVALID;
  if (batch > 0 && !cu_seqlens) return DIFFKV_E_INVALID;
  if (total_tokens > 0 && (!k || !scores)) return DIFFKV_E_INVALID;
  if ((uintptr_t)k & 15u) return DIFFKV_E_INVALID;  // rows are read with 16-byte loads
  const Cfg c = to_cfg(cfg);
  if (!ws_ok(workspace) || workspace_bytes < keydiff_workspace(c, batch, total_tokens)) return DIFFKV_E_WORKSPACE;
  return rc(launch_keydiff(c, batch, total_tokens, cu_seqlens, k, anchor_raw, scores, workspace,
                           (hipStream_t)stream));
}

int diffkv_page_bounds(const diffkv_config* cfg, const diffkv_pool* pool, int32_t batch, const int32_t* page_table,
                       const int32_t* tier_state, float* bounds, void* stream) {
  if (!cfg_ok(cfg) || !pool_ok(cfg, pool) || batch < 0) return DIFFKV_E_INVALID;
  if (batch > 0 && (!page_table || !tier_state || !bounds)) return DIFFKV_E_INVALID;
  if ((int64_t)batch * cfg->num_kv_heads > 65535) return DIFFKV_E_INVALID;
  return rc(launch_page_bounds(to_cfg(cfg), to_pool(pool), batch, page_table, tier_state, bounds,
                               (hipStream_t)stream));
}

int diffkv_page_scores(const diffkv_config* cfg, const diffkv_pool* pool, int32_t batch, const uint16_t* q,
                       const int32_t* page_table, const int32_t* tier_state, const int32_t* seq_len,
                       const float* bounds, float* scores, void* stream) {
  if (!cfg_ok(cfg) || !pool_ok(cfg, pool) || batch < 0) return DIFFKV_E_INVALID;
  if (batch > 0 && (!q || !page_table || !tier_state || !seq_len || !bounds || !scores)) return DIFFKV_E_INVALID;
  if ((int64_t)batch * cfg->num_kv_heads > 65535) return DIFFKV_E_INVALID;
  // pairs of dimensions per lane: 4-byte query words, 8-byte bound pairs
  if (((uintptr_t)q & 3) != 0 || ((uintptr_t)bounds & 7) != 0) return DIFFKV_E_INVALID;
  return rc(launch_page_scores(to_cfg(cfg), pool->num_pages, batch, q, page_table, tier_state, seq_len, bounds,
                               scores, (hipStream_t)stream));
}

int diffkv_update_scores(const diffkv_config* cfg, const diffkv_pool* pool, int32_t batch, const int32_t* page_table,
                         const int32_t* tier_state, const int32_t* seq_len, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!cfg_ok(cfg) || !pool_ok(cfg, pool) || batch < 0) return DIFFKV_E_INVALID;
  if (batch > 0 && (!page_table || !tier_state || !seq_len)) return DIFFKV_E_INVALID;
  if ((int64_t)batch * cfg->num_kv_heads > 65535) return DIFFKV_E_INVALID;
  const Cfg c = to_cfg(cfg);
  if (!ws_ok(workspace) || workspace_bytes < attn_workspace(c, batch, true)) return DIFFKV_E_WORKSPACE;
  return rc(launch_scores(c, to_pool(pool), batch, page_table, tier_state, seq_len, workspace,
                          (hipStream_t)stream));
}

}  // extern "C"
