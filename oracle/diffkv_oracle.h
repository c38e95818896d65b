/*
 * diffkv_oracle.h -- plain, slow, serial CPU oracle for the DiffKV hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link
 * or call this.  Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library; the two agree only through the written specification of
 * the page layout and the policy readings.
 *
 * Source of what is computed: the notes page "DiffKV: Differentiated Memory
 * Management for Large Language Models with Parallel KV Compaction"
 * (SOSP'25, arXiv 2412.03131), sections "Background" (attention formula and
 * asymmetric quantization), "KV compression policy" (prompt- and
 * generation-phase logic), "Memory management" (unified pages, circular free
 * page list, bidirectional page table, Fig 6 prompt workflow, generation
 * workflow) and "Implementation" (compactor before attention).
 *
 * All buffers are host memory owned by the caller.  Layouts match the HIP
 * library's C-ABI so parity tests can compare them byte for byte.
 */
#ifndef DIFFKV_ORACLE_H
#define DIFFKV_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t head_dim;       /* d: 64 or 128 */
  int32_t num_kv_heads;   /* H */
  int32_t gqa_group;      /* G: q head j reads KV head j / G */
  int32_t hi_page_tokens; /* T_h (16) */
  int32_t lo_page_tokens; /* T_l = 2 T_h */
  int32_t max_seq_len;    /* S_max; table row length L_max = ceil(S_max/T_h)+1 */
  int32_t window;         /* W: most recent tokens always high precision */
  int32_t lo_enabled;     /* 0: high / prune only */
  float alpha_h, alpha_l; /* thresholds are alpha/N */
  int32_t prompt_rule;    /* ORC_RULE_ALPHA_N: prompt tokens against alpha/N;
                             ORC_RULE_ALPHA_I: the i-th prompt token against alpha/i */
  const float* alpha_h_head; /* host arrays of H per-KV-head thresholds, or both NULL */
  const float* alpha_l_head;
  /* tier codecs: bits of K and V codes per tier, each in {1, 2, 4, 8};
   * all four 0 = the default K8V4 (high) / K4V2 (low) */
  int32_t hi_k_bits, hi_v_bits, lo_k_bits, lo_v_bits;
  /* More than two precision levels: num_levels K = 0 or 2 keeps the two
   * tiers above; K = 3 or 4 gives levels 0 (high: alpha_h, hi bits, T_h
   * tokens per page) .. K-1 (low: alpha_l, lo bits, T_l tokens), the middle
   * levels l = 1..K-2 with alpha_mid[l-1] and mid_k_bits / mid_v_bits[l-1]
   * (T_l tokens).  Codecs must be given (plain layout); table rows: level
   * 2r from the left and level 2r+1 from the right of row r. */
  int32_t num_levels;
  float alpha_mid[2];
  int32_t mid_k_bits[2], mid_v_bits[2];
} orc_cfg;

enum { ORC_RULE_ALPHA_N = 0, ORC_RULE_ALPHA_I = 1 };

typedef struct {
  uint8_t* pages;     /* [num_pages * page_bytes] */
  int32_t* free_list; /* [num_pages] circular list of page ids */
  uint64_t* ptr;      /* [2]: allocation counter (start), reclaim counter (end) */
  uint32_t* status;   /* [1] sticky status bits */
  int64_t num_pages;
  int32_t page_bytes;
} orc_pool;

enum { ORC_OK = 0, ORC_E_INVALID = 1 };
enum { ORC_ST_POOL_EXHAUSTED = 1u, ORC_ST_TABLE_OVERFLOW = 2u, ORC_ST_BAD_STATE = 4u };
enum { ORC_PRUNE = 0, ORC_LO = 1, ORC_HI = 2 };

/* ---- layout ---------------------------------------------------------- */
int32_t orc_page_bytes(const orc_cfg* c);
int32_t orc_table_len(const orc_cfg* c);
/* seg[0..5] = byte offsets of K codes, K meta, V codes, V meta, score, pos;
 * seg[6] = bytes used by the tier; returns tokens per page of the tier. */
int32_t orc_tier_layout(const orc_cfg* c, int32_t tier, int32_t seg[7]);
/* Byte offset and bit shift of one K or V code inside a page of `tier`. */
void orc_k_code_addr(const orc_cfg* c, int32_t tier, int32_t tok, int32_t j,
                     int32_t* byte, int32_t* shift);
void orc_v_code_addr(const orc_cfg* c, int32_t tier, int32_t tok, int32_t j,
                     int32_t* byte, int32_t* shift);
/* Unpack one slot of a page: codes one per byte, metadata, score, pos. */
void orc_read_slot(const orc_cfg* c, const uint8_t* page, int32_t tier, int32_t slot,
                   uint8_t* kc, uint8_t* vc, uint16_t* kmeta /*[2]*/,
                   uint16_t* vmeta /*[2]*/, float* score, int32_t* pos);

/* Levels (K >= 3, or K = 2 as the two tiers: level 0 = high, 1 = low):
 * number of levels, int32 words of tier state per unit (n_0..n_{K-1},
 * p_0..p_{K-1}), and the layout of one level's pages (as orc_tier_layout). */
int32_t orc_num_levels(const orc_cfg* c);
int32_t orc_state_words(const orc_cfg* c);
int32_t orc_level_layout(const orc_cfg* c, int32_t level, int32_t seg[7]);
/* Unpack one slot of a level's page (as orc_read_slot). */
void orc_read_level_slot(const orc_cfg* c, const uint8_t* page, int32_t level, int32_t slot,
                         uint8_t* kc, uint8_t* vc, uint16_t* kmeta, uint16_t* vmeta,
                         float* score, int32_t* pos);
/* The generation step over K levels (any K, also 2), recording per unit:
 * bits 0-3 the class of t_c (level, 14 = pruned, 15 = no t_c), bits 4-7 the
 * class of the victim (level, 14 = pruned, 15 = no victim considered),
 * bits 8-11 the level of the new page + 1 (0: none); -1 inactive. */
int orc_levels_compact_step(const orc_cfg* c, orc_pool* p, int32_t batch,
                            const int32_t* seq_len, const uint16_t* k_new,
                            const uint16_t* v_new, int32_t* page_table,
                            int32_t* tier_state, int32_t* branch);
/* Level versions of classify, prompt compaction, release and attention
 * (any K; the two-tier entry points call them when K >= 3). */
int orc_levels_classify(const orc_cfg* c, int32_t batch, const int64_t* cu_seqlens,
                        const float* scores, uint8_t* tiers, int32_t* tier_counts);
int orc_levels_compact_prompt(const orc_cfg* c, orc_pool* p, int32_t batch,
                              const int64_t* cu_seqlens, const uint16_t* k,
                              const uint16_t* v, const float* scores,
                              const uint8_t* tiers, int32_t* page_table,
                              int32_t* tier_state);
int orc_levels_release(const orc_cfg* c, orc_pool* p, int32_t batch,
                       const uint8_t* release_mask, int32_t* page_table,
                       int32_t* tier_state);
int orc_levels_decode_attn(const orc_cfg* c, orc_pool* p, int32_t batch,
                           const uint16_t* q, const int32_t* page_table,
                           const int32_t* tier_state, const int32_t* seq_len,
                           float* out, int32_t update_scores);

/* ---- fp16 and codec ---------------------------------------------------- */
uint16_t orc_f32_to_f16(float f);
float orc_f16_to_f32(uint16_t h);
void orc_f32_to_f16_n(const float* x, uint16_t* h, int64_t n);
void orc_f16_to_f32_n(const uint16_t* h, float* x, int64_t n);
/* Per-vector asymmetric min/max quantization to `bits` (8, 4 or 2). */
void orc_quantize(const float* x, int32_t n, int32_t bits, uint16_t* s16,
                  uint16_t* z16, uint8_t* codes);
float orc_dequant(uint16_t s16, uint16_t z16, int32_t code);

/* ---- policy ------------------------------------------------------------ */
int orc_classify(const orc_cfg* c, int32_t batch, const int64_t* cu_seqlens,
                 const float* scores, uint8_t* tiers, int32_t* tier_counts);

/* Plan + allocation part of prompt compaction on page counts only (used by
 * the worked-example test with small pages).  n_hi/n_lo: [batch*H]; seqlens
 * [batch]; writes tables and state; returns ORC_OK or ORC_E_INVALID. */
int orc_prompt_allocate(int32_t H, int32_t T_h, int32_t T_l, int32_t L_max,
                        int32_t batch, const int64_t* seqlens,
                        const int32_t* n_hi, const int32_t* n_lo,
                        int32_t* free_list, uint64_t* ptr, uint32_t* status,
                        int64_t num_pages, int32_t* page_table,
                        int32_t* tier_state);

int orc_pool_init(orc_pool* p);
int orc_compact_prompt(const orc_cfg* c, orc_pool* p, int32_t batch,
                       const int64_t* cu_seqlens, const uint16_t* k,
                       const uint16_t* v, const float* scores,
                       const uint8_t* tiers, int32_t* page_table,
                       int32_t* tier_state);
int orc_compact_step(const orc_cfg* c, orc_pool* p, int32_t batch,
                     const int32_t* seq_len, const uint16_t* k_new,
                     const uint16_t* v_new, int32_t* page_table,
                     int32_t* tier_state);
/* The same step, also recording per unit which case of the generation-phase
 * policy the plan took (bookkeeping for tests): bits 0-3 one of ORC_BR_*,
 * bits 4-5 the tier of the unit's new page (0: none). */
enum {
  ORC_BR_INACTIVE = 0,  /* seq_len <= 0, or the unit was rejected */
  ORC_BR_NO_TC = 1,     /* no token leaves the window yet (N < W) */
  ORC_BR_HI_KEEP = 2,   /* t_c high, the least important high token stays */
  ORC_BR_HI_DEMOTE = 3, /* t_c high, the least important high token moves to low */
  ORC_BR_HI_PRUNE = 4,  /* t_c high, the least important high token is pruned */
  ORC_BR_LO_KEEP = 5,   /* t_c low, no low token is pruned */
  ORC_BR_LO_PRUNE = 6,  /* t_c low, the least important low token is pruned */
  ORC_BR_PRUNE = 7      /* t_c pruned */
};
int orc_compact_step_branches(const orc_cfg* c, orc_pool* p, int32_t batch,
                              const int32_t* seq_len, const uint16_t* k_new,
                              const uint16_t* v_new, int32_t* page_table,
                              int32_t* tier_state, int32_t* branch);
int orc_release(const orc_cfg* c, orc_pool* p, int32_t batch,
                const uint8_t* release_mask, int32_t* page_table,
                int32_t* tier_state);

/* ---- attention ----------------------------------------------------------- */
int orc_decode_attn(const orc_cfg* c, orc_pool* p, int32_t batch,
                    const uint16_t* q, const int32_t* page_table,
                    const int32_t* tier_state, const int32_t* seq_len,
                    float* out, int32_t update_scores);
/* Full-precision textbook attention of one query over n keys (fp64). */
void orc_attention_dense(const double* q, const double* k, const double* v,
                         int32_t n, int32_t d, double* out);
/* Same output through the coefficient x unit-vector decomposition. */
void orc_attention_unit_vectors(const double* q, const double* k,
                                const double* v, int32_t n, int32_t d,
                                double* out);
/* Prompt importance from nq probe queries: per token, mean over queries of
 * the max over the G q heads of a KV head of the softmax weight. */
/* Prompt importance from the prompt's own queries under causal attention:
 * per token the mean over the later tokens' queries of the max over the
 * KV head's q heads of the weight it receives.  q [total, H*G, d], k
 * [total, H, d] fp16; scores [H, total] fp32. */
int orc_importance_causal(const orc_cfg* c, int32_t batch, const int64_t* cu_seqlens,
                          const uint16_t* q, const uint16_t* k, float* scores);
/* The same for the last `tail` tokens of each request only (the others'
 * scores are left as they are): sampled outputs of long prompts. */
int orc_importance_causal_tail(const orc_cfg* c, int32_t batch, const int64_t* cu_seqlens,
                               const uint16_t* q, const uint16_t* k, int64_t tail, float* scores);
/* Per-page key bounds: bounds [num_pages][2][d] fp32 (min row, max row)
 * over the dequantized keys of each live page's retained slots. */
int orc_page_bounds(const orc_cfg* c, orc_pool* p, int32_t batch, const int32_t* page_table,
                    const int32_t* tier_state, float* bounds);
/* Page scores in table order [batch, H, L]: max over the group's q heads of
 * sum_i max(q_i kmin_i, q_i kmax_i); -inf at empty entries. */
int orc_page_scores(const orc_cfg* c, int32_t batch, const uint16_t* q, const int32_t* page_table,
                    const int32_t* tier_state, const int32_t* seq_len, const float* bounds,
                    int64_t num_pages, float* scores);
/* Query-free importance (KeyDiff anchor cosine): w_i = 1 - cos(anchor, k_i),
 * the anchor the mean of the unit's normalized keys (anchor_raw = 0) or raw
 * keys (1); scores = w normalized over the unit's tokens. */
int orc_keydiff_scores(const orc_cfg* c, int32_t batch, const int64_t* cu_seqlens,
                       const uint16_t* k, int32_t anchor_raw, float* scores);
int orc_importance_from_queries(const orc_cfg* c, int32_t batch,
                                const int64_t* cu_seqlens, const uint16_t* k,
                                int32_t nq, const uint16_t* qprobe,
                                float* scores);

#ifdef __cplusplus
}
#endif
#endif
