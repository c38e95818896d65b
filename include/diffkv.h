/*
 * diffkv.h -- C-ABI of libdiffkv.so, the MI355X (gfx950) DiffKV hot path:
 * differentiated KV compaction and paged decode attention over the
 * compacted cache.
 *
 * What is computed follows the notes page "DiffKV: Differentiated Memory
 * Management for Large Language Models with Parallel KV Compaction"
 * (SOSP'25, arXiv 2412.03131).  Each entry point names the section it
 * implements.
 *
 * Conventions (all entry points)
 *  - Every pointer argument is DEVICE memory unless marked "host".  The
 *    caller allocates and owns every buffer; the library allocates nothing.
 *    Its only global state is a per-device cache of the compute-unit count
 *    (read once with hipDeviceGetAttribute) and, for
 *    diffkv_decode_attn_noalloc, one fixed device array per GPU; distinct
 *    pools can be used concurrently.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    kernels on it and return without synchronizing.
 *  - fp16 tensors travel as raw IEEE binary16 bits (uint16_t).
 *  - Tensors are row-major and contiguous in the shapes given below.
 *  - Return codes report host-detectable problems only: DIFFKV_E_INVALID
 *    (null pointer, bad config or sizes), DIFFKV_E_WORKSPACE (workspace
 *    smaller than diffkv_workspace_bytes, or not 256-byte aligned as
 *    hipMalloc returns it), DIFFKV_E_HIP (launch error).  On
 *    a non-zero return nothing was enqueued.
 *  - Conditions found on the device (pool exhausted, table row overflow,
 *    inconsistent state) set sticky bits in pool->status; a compaction call
 *    that sets one commits nothing (all or nothing over the whole call).
 *    The caller reads status after synchronizing and clears it itself.
 *  - Determinism: identical inputs give byte-identical outputs; no result
 *    depends on the order of atomic operations.
 *
 * Units: one (request b, KV head h) pair, u = b*H + h.  Tiers: 2 = high
 * (K 8 bit, V 4 bit, 16 tokens per page), 1 = low (K 4 bit, V 2 bit, 32
 * tokens per page), 0 = pruned.
 */
#ifndef DIFFKV_H
#define DIFFKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Host struct.  Thresholds: high if mean score > alpha_h/N, low if in
 * [alpha_l/N, alpha_h/N], pruned below alpha_l/N ("Approach"; "KV
 * compression policy").  With lo_enabled = 0: high iff >= alpha_l/N.
 * Policy variants ("KV compression policy"):
 *  - prompt_rule = DIFFKV_RULE_ALPHA_I compares the i-th prompt token
 *    (i = position + 1) against alpha/i, as the prompt-phase paragraph
 *    states; the generation step always uses alpha/N (N = the new length).
 *  - alpha_h_head / alpha_l_head (DEVICE arrays of num_kv_heads floats, both
 *    or neither) give each KV head its own pair, the extensibility
 *    paragraph's option; NULL = the shared pair for every head.  The library
 *    cannot read them on the host: the caller guarantees
 *    0 <= alpha_l_head[h] <= alpha_h_head[h] when lo_enabled (other values
 *    are used as given in the same comparisons).
 * Valid: head_dim in {64,128}; 1 <= gqa_group <= 16; hi_page_tokens = 16;
 * 1 <= max_seq_len < 2^29 (score sums times token counts stay exact in fp64);
 * lo_page_tokens = 32; window >= 0 (>= 2 for STEP);
 * 0 <= alpha_l <= alpha_h when lo_enabled; prompt_rule in {0, 1}. */
typedef struct {
  int32_t head_dim;       /* d */
  int32_t num_kv_heads;   /* H */
  int32_t gqa_group;      /* G: q head j reads KV head j / G */
  int32_t hi_page_tokens; /* T_h = 16 */
  int32_t lo_page_tokens; /* T_l = 32 */
  int32_t max_seq_len;    /* S_max; table row length L = ceil(S_max/16) + 1 */
  int32_t window;         /* W: the most recent W tokens stay high precision */
  int32_t lo_enabled;     /* 0: high / prune only */
  float alpha_h, alpha_l;
  int32_t prompt_rule;        /* DIFFKV_RULE_ALPHA_N (0) or DIFFKV_RULE_ALPHA_I (1) */
  const float* alpha_h_head;  /* [num_kv_heads] device, or NULL */
  const float* alpha_l_head;  /* [num_kv_heads] device, or NULL */
  /* Tier codecs ("Results": the bit-split ablation, e.g. K4V8, K2V4, K8V2,
   * K4V1 against K8V4 / K4V2): code widths of K and V in the high and the
   * low tier, each in {1, 2, 4, 8}; all four 0 = the default K8V4 / K4V2.
   * A variant (or the default pair given explicitly) uses the plain page
   * layout: the same six segments and 16 / 32 tokens per page, codes
   * token-major and packed from bit 0 (code (t, j) at bit (t d + j) b of its
   * segment); diffkv_page_bytes gives its page size.  Every entry point
   * takes variants, with the same results and status rules; they run on
   * general kernels (codes dequantized in fp32 on the vector units): a
   * decode step is the STEP followed by the attention (chain is ignored) and
   * no next-step plan records are kept (a STEP always scans the unit). */
  int32_t hi_k_bits, hi_v_bits, lo_k_bits, lo_v_bits;
  /* More than two precision levels ("KV compression policy", extensibility
   * paragraph; "Memory management", generation workflow: extra levels by
   * combining unidirectional or bidirectional page tables).  num_levels K:
   * 0 or 2 = the two tiers above; 3 or 4 = levels 0 (most precise) .. K-1:
   *   level 0: alpha_h, hi bits, 16 tokens per page;
   *   levels 1 .. K-2: alpha_mid[l-1], mid_k_bits / mid_v_bits[l-1], 32 tokens;
   *   level K-1: alpha_l, lo bits, 32 tokens.
   * All of the used widths must be given (plain layout), lo_enabled = 1, and
   * alpha_h >= alpha_mid[0] (>= alpha_mid[1]) >= alpha_l (per-head arrays
   * replace alpha_h and alpha_l per head and must keep that order; the
   * middle thresholds are shared).  A token is in the first level l < K-1
   * with mean * N > alpha_l, else in level K-1 if mean * N >= alpha_{K-1},
   * else pruned; the window is level 0.  The page table has R = ceil(K/2)
   * rows per unit (row r: level 2r from the left, level 2r+1 from the
   * right); the tier state has 2K words per unit (token counts n_0..n_{K-1},
   * then page counts); the prompt's block feeds levels 0, 2, 3 from its left
   * end and level 1 from its right end; a generation step moves at most t_c
   * and one victim down (see diffkv_compact).  Per-page key bounds and page
   * scores cover every level (scores over all R rows of the table). */
  int32_t num_levels;
  float alpha_mid[2];
  int32_t mid_k_bits[2], mid_v_bits[2];
} diffkv_config;

enum { DIFFKV_RULE_ALPHA_N = 0, DIFFKV_RULE_ALPHA_I = 1 };

/* Host struct describing caller-owned device buffers of one page pool
 * ("Memory management": unified pages, circular free page list). */
typedef struct {
  void* pages;        /* [num_pages * page_bytes] unified pages */
  int32_t* free_list; /* [num_pages] circular list of page ids */
  uint64_t* ptr;      /* [2]: allocation counter, reclamation counter; list
                         index = counter mod num_pages, free = ptr[1]-ptr[0] */
  uint32_t* status;   /* [1] sticky DIFFKV_ST_* bits */
  int64_t num_pages;  /* 1 <= num_pages < 2^31 */
  int32_t page_bytes; /* must equal diffkv_page_bytes(cfg) */
} diffkv_pool;

enum { DIFFKV_OK = 0, DIFFKV_E_INVALID = 1, DIFFKV_E_WORKSPACE = 2, DIFFKV_E_HIP = 3 };
enum {
  DIFFKV_ST_POOL_EXHAUSTED = 1u,
  DIFFKV_ST_TABLE_OVERFLOW = 2u,
  DIFFKV_ST_BAD_STATE = 4u,
  DIFFKV_ST_STALE_CHAIN = 8u /* diffkv_decode_step: chain > 0 on a cache changed since its plans,
                                or one whose previous step left no plan (a state the plan
                                kernel rejects, e.g. after aborted steps) */
};
enum {
  DIFFKV_PROMPT = 0,
  DIFFKV_STEP = 1,
  DIFFKV_RELEASE = 2,
  DIFFKV_ATTN = 3,
  DIFFKV_ATTN_SCORES = 4,
  DIFFKV_DECODE_STEP = 5,        /* diffkv_decode_step, update_scores = 0 */
  DIFFKV_DECODE_STEP_SCORES = 6, /* diffkv_decode_step, update_scores = 1 or 2 */
  DIFFKV_IMPORTANCE = 7,         /* diffkv_importance; total_tokens = queries in all (see there) */
  DIFFKV_KEYDIFF = 8             /* diffkv_keydiff_scores */
};
enum { DIFFKV_IMP_CAUSAL = 0, DIFFKV_IMP_PROBE = 1 };

/* Bytes of one unified page (six segments, "Memory management"): 3584 at
 * d = 128, 2048 at d = 64; -1 for an invalid config. */
int32_t diffkv_page_bytes(const diffkv_config* cfg);

/* Page-table entries per unit: R rows of ceil(max_seq_len / 16) + 1 (R = 1
 * for the two tiers, ceil(K / 2) with K precision levels); -1 if invalid. */
int32_t diffkv_table_len(const diffkv_config* cfg);

/* int32 words of tier state per unit: 2K (4 for the two tiers); -1 if
 * invalid. */
int32_t diffkv_state_words(const diffkv_config* cfg);

/* Device scratch needed by one call of `op` (DIFFKV_PROMPT / STEP / RELEASE
 * for diffkv_compact, DIFFKV_ATTN or DIFFKV_ATTN_SCORES for
 * diffkv_decode_attn without / with update_scores) on `batch` requests with
 * `total_tokens` = sum of prompt lengths (PROMPT only).  0 on invalid input.
 * Workspaces need no initialization.  A DIFFKV_ATTN_SCORES workspace carries
 * the logits from diffkv_decode_attn(update_scores = 2) to
 * diffkv_update_scores, so nothing else may use it in between.  Calls that
 * share one workspace must not overlap. */
size_t diffkv_workspace_bytes(const diffkv_config* cfg, int32_t op, int32_t batch,
                              int64_t total_tokens);

/* Fills free_list with 0..num_pages-1, ptr = {0, num_pages}, status = 0. */
int diffkv_pool_init(const diffkv_config* cfg, const diffkv_pool* pool, void* stream);

/* Resets `batch` requests to empty: page_table [batch, H, table_len] = -1,
 * tier_state [batch, H, state_words] = 0. */
int diffkv_state_init(const diffkv_config* cfg, int32_t batch, int32_t* page_table,
                      int32_t* tier_state, void* stream);

/* Prompt-phase token importance, the input of diffkv_classify ("KV
 * compression policy", prompt phase: a token's importance is the mean of the
 * attention weights it receives from the tokens after it; the weights of the
 * q heads sharing a KV head are combined with max).
 *  mode DIFFKV_IMP_CAUSAL: q fp16 [total_tokens, H*G, d] holds the prompt's
 *    own queries (token-major, as a prefill produces them).  Query j of a
 *    request attends causally to its keys 0..j (softmax of q.k/sqrt(d));
 *    token i's importance is the mean over the N-1-i later queries j > i of
 *    max over the group of its weight; the last token gets 0.
 *  mode DIFFKV_IMP_PROBE: q fp16 [batch, nq, H*G, d] holds nq probe queries
 *    per request that attend to all N tokens; importance = the mean over the
 *    nq probes of max over the group of the weight.
 *  cu_seqlens int64 [batch+1] (device), k fp16 [total_tokens, H, d]; q and k
 *    16-byte aligned, else DIFFKV_E_INVALID.
 *  scores fp32 [H, total_tokens] out: the mean per token, as diffkv_classify
 *    and diffkv_compact(PROMPT) take it.
 *  workspace: diffkv_workspace_bytes(cfg, DIFFKV_IMPORTANCE, batch, n) with
 *    n = total_tokens (causal) or batch * nq (probe): one fp32 softmax
 *    reference per query and q head.
 * Work is quadratic in the prompt length (causal); computed in fp32 on the
 * matrix units from the fp16 inputs (within 1e-4 relative of the fp64
 * definition on the tested inputs). */
int diffkv_importance(const diffkv_config* cfg, int32_t mode, int32_t batch, int64_t total_tokens,
                      const int64_t* cu_seqlens, int32_t nq, const uint16_t* q, const uint16_t* k,
                      float* scores, void* workspace, size_t workspace_bytes, void* stream);

/* Query-free token importance from the keys alone, an alternative input of
 * diffkv_classify (KeyDiff page, method details: the anchor is the mean of
 * the unit's normalized keys -- anchor_raw = 1: of the raw keys, the page's
 * simplification -- and a key's eviction score is its cosine to the anchor,
 * the least similar keys being kept).  Per unit, importance
 * w_i = 1 - cos(anchor, k_i) normalized over the unit's tokens
 * (scores[h][token] sum to 1 per unit, like the mean attention; 1/N each
 * when every key is parallel to the anchor; a zero key or anchor has
 * cosine 0), so the alpha/N thresholds apply unchanged.
 *  cu_seqlens int64 [batch+1] (device), k fp16 [total_tokens, H, d]
 *  (16-byte aligned), scores fp32 [H, total_tokens] out.
 *  workspace: diffkv_workspace_bytes(cfg, DIFFKV_KEYDIFF, batch, total_tokens).
 * Every sum runs in a fixed order: the scores are deterministic. */
int diffkv_keydiff_scores(const diffkv_config* cfg, int32_t batch, int64_t total_tokens,
                          const int64_t* cu_seqlens, const uint16_t* k, int32_t anchor_raw, float* scores,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Per-page key bounds (FlexiCache page, "3.2 KV page scoring", after
 * Quest: each KV page keeps the per-dimension minimum and maximum of its
 * keys).  For every live page of the batch's units (table entries in the
 * unit's high prefix / low suffix; with K levels the p_l pages of every
 * level, each with its own codec and page size), over the dequantized keys
 * of its retained slots (the keys the attention reads):
 *  bounds fp32 [pool->num_pages][2][d] out: row 0 the minima, row 1 the
 *  maxima (exact fp32 values); other pages' rows untouched.  Kept apart from
 *  the pages, as the page keeps its min-max vectors in a cache of their own;
 *  call again after compaction to refresh them.  Units with an inconsistent
 *  tier state and page ids outside the pool are skipped. */
int diffkv_page_bounds(const diffkv_config* cfg, const diffkv_pool* pool, int32_t batch,
                       const int32_t* page_table, const int32_t* tier_state, float* bounds, void* stream);

/* Page scores from the bounds: for a query, the largest dot product it
 * could have with any key of the page, sum_i max(q_i kmin_i, q_i kmax_i),
 * combined over the KV head's q heads with max (the aggregation used for
 * token scores); a decode step can skip the pages whose score is low.
 *  q fp16 [batch, H*G, d] (4-byte aligned); seq_len int32 [batch] (<= 0:
 *  inactive); bounds as diffkv_page_bounds wrote them (8-byte aligned);
 *  scores fp32 [batch, H, table_len] out in table order (diffkv_table_len
 *  entries per unit), -inf at empty entries and for inactive requests.  fp32 with fixed-order sums.  DIFFKV_E_INVALID on
 *  a misaligned q or bounds. */
int diffkv_page_scores(const diffkv_config* cfg, const diffkv_pool* pool, int32_t batch, const uint16_t* q,
                       const int32_t* page_table, const int32_t* tier_state, const int32_t* seq_len,
                       const float* bounds, float* scores, void* stream);

/* Token classification ("Approach"; "KV compression policy", prompt phase).
 *  cu_seqlens  int64 [batch+1], cu[0] = 0, non-decreasing; N_r = cu[r+1]-cu[r]
 *  scores      fp32 [H, cu[batch]]: per token its mean received attention
 *  tiers       uint8 [H, cu[batch]] out: 2 high, 1 low, 0 pruned (K levels:
 *              K - level, 0 pruned).  The last
 *              W tokens of each request are high; otherwise s*N_r (with
 *              prompt_rule = DIFFKV_RULE_ALPHA_I: s*(p+1) for position p) is
 *              compared with the KV head's alpha_h and alpha_l exactly (fp64,
 *              no division).
 *  tier_counts int32 [batch, H, 2] out: (high count, low count) (K levels:
 *              [batch, H, K], one count per level). */
int diffkv_classify(const diffkv_config* cfg, int32_t batch, int64_t total_tokens,
                    const int64_t* cu_seqlens, const float* scores, uint8_t* tiers,
                    int32_t* tier_counts, void* stream);

/* KV compaction ("Memory management": parallel KV compaction, planning per
 * head plus a prefix sum over the circular free page list; bidirectional
 * page table; Fig 6 prompt workflow; generation workflow; "Implementation":
 * called after K/V are computed, before attention).
 *
 * page_table int32 [batch, H, L]: high page ids from the left (index 0 up),
 *            low page ids from the right (index L-1 down), -1 elsewhere.
 * tier_state int32 [batch, H, 4]: (high tokens, low tokens, high pages,
 *            low pages) per unit.
 * Inside a tier, slot s of a unit lives in page table[s/16] (high) or
 * table[L-1-s/32] (low) at in-page index s mod 16 (32).
 *
 * mode DIFFKV_PROMPT: admits requests with N_r > 0 (others untouched; their
 *   rows must be empty).  Uses cu_seqlens, k/v fp16 [cu[batch], H, d]
 *   (token-major; both 16-byte aligned, else DIFFKV_E_INVALID), scores (mean per token, [H, total]) and tiers from
 *   diffkv_classify.  Per unit: a conservative block of ceil(N/16) pages
 *   from the allocation pointer (units in order); high pages take the block
 *   from the left, low pages from the right; the middle is reclaimed at the
 *   reclamation pointer (units in order, ascending block index); a unit
 *   that needs one page more than its block takes it after the frees as its
 *   innermost low page.  Tokens are quantized per vector (min/max
 *   asymmetric, fp16 scale/zero; "Background") and packed in position
 *   order; the stored score is mean * (N - 1 - pos) (a running sum).
 * mode DIFFKV_STEP: one generation step for every request with
 *   seq_len[b] > 0 (seq_len = length before this step's token).  Uses
 *   k/v fp16 [batch, H, d] (the new token per unit).  The new token enters
 *   the high tier; the token that leaves the window is classified against
 *   alpha/(N+1); a least-important token of the receiving tier may be
 *   requantized to low or pruned ("KV compression policy", generation
 *   phase).  At most one new page per unit, no reclamation.
 * mode DIFFKV_RELEASE: for requests with release_mask[b] != 0, appends the
 *   unit's high pages (left to right) then low pages (right to left) at the
 *   reclamation pointer, units in order, and resets the rows.  A released
 *   unit with an inconsistent page count, or whose used table entries hold
 *   a page id outside [0, num_pages), sets DIFFKV_ST_BAD_STATE and the call
 *   commits nothing.
 * K precision levels (num_levels 3 or 4): page_table [batch, H, R * L] (row
 *   r = level 2r from the left, level 2r+1 from the right), tier_state
 *   [batch, H, 2K] (n_0..n_{K-1}, p_0..p_{K-1}); level l's slot s lives in
 *   page s / T_l of that level (T_0 = 16, else 32).  PROMPT: the block of
 *   ceil(N/16) pages feeds levels 0, 2, 3 (in that order) from its left end
 *   and level 1 from its right end, the middle is reclaimed, pages the block
 *   lacks are taken after the frees (levels 0, 2, 3, then level 1 innermost
 *   first).  STEP: t_c's level l_c; l_c = 0: the least important non-window
 *   level-0 token (t_c included) moves to its class's level or is pruned;
 *   l_c >= 1: t_c moves to level l_c and the least important token of level
 *   l_c (t_c included) moves down to its class's level or is pruned when
 *   its class is below l_c; a removal and an insertion in one level share
 *   the slot, otherwise the insertion appends.  RELEASE: row by row, the
 *   left level's pages left to right, then the right level's right to left.
 * Unused pointer arguments of a mode may be NULL. */
int diffkv_compact(const diffkv_config* cfg, const diffkv_pool* pool, int32_t mode,
                   int32_t batch, int64_t total_tokens, const int64_t* cu_seqlens,
                   const int32_t* seq_len, const uint16_t* k, const uint16_t* v,
                   const float* scores, const uint8_t* tiers, const uint8_t* release_mask,
                   int32_t* page_table, int32_t* tier_state, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Paged decode attention over the compacted cache ("Background": softmax of
 * q.k/sqrt(d) weighting v; "Implementation": custom attention kernel, high
 * pages before low pages, sequence split with a merge).
 *  q       fp16 [batch, H*G, d]; q head j uses KV head j / G
 *  seq_len int32 [batch]: position of the query token (its K/V was appended
 *          by the preceding STEP); <= 0 marks an inactive request (output 0)
 *  out     fp32 [batch, H*G, d]
 * Keys and values are dequantized on the fly (x = s*code + z per token);
 * softmax is fp32 online with a split-sequence merge; only retained tokens
 * take part.
 * update_scores: 0 = attention only; 1 = attention, then the score update
 * (each retained token with position < seq_len[b] adds the max over the
 * group's q heads of its softmax weight to its stored score sum; pages are
 * written; the next generation step's plan for length seq_len[b] + 1 is
 * left in spare bytes of the unit's first high page, where a STEP with that
 * length and tier state uses it instead of scanning the unit); 2 = attention
 * that keeps its logits in `workspace` for a later diffkv_update_scores call
 * (needs the DIFFKV_ATTN_SCORES workspace size).
 * A unit whose tier_state is inconsistent, or whose table row holds a page
 * id outside [0, num_pages), gets output 0, no score update, and sets
 * DIFFKV_ST_BAD_STATE; no load leaves the pool.
 * With more workgroups (units times splits) than the device has compute
 * units, a small kernel first sorts the units by page count into the
 * workspace so that the longest start first; results do not depend on that
 * order. */
int diffkv_decode_attn(const diffkv_config* cfg, const diffkv_pool* pool, int32_t batch,
                       const uint16_t* q, const int32_t* page_table,
                       const int32_t* tier_state, const int32_t* seq_len, float* out,
                       int32_t update_scores, void* workspace, size_t workspace_bytes,
                       void* stream);

/* One decode step: diffkv_compact(DIFFKV_STEP) followed by
 * diffkv_decode_attn on the updated cache with the same seq_len, as one call
 * ("Implementation": the compactor runs after K/V are computed and before the
 * attention kernel).  Results, status bits and all-or-nothing behaviour are
 * those of the two calls in sequence (an aborted step leaves the cache as it
 * was and the attention runs on it).  When every unit is one split
 * (diffkv_attn_splits == 1) and update_scores != 2, the commit runs inside
 * the attention kernel; one difference remains there: a free-list entry
 * outside the pool (a corrupt pool) leaves that unit uncommitted, sets
 * BAD_STATE and zeroes its output, where the two calls would attend to the
 * uncommitted unit.
 *  seq_len  int32 [batch]: length before this step's token (= position of
 *           the query token); <= 0 marks an inactive request
 *  k_new, v_new fp16 [batch, H, d]; q fp16 [batch, H*G, d]; out fp32
 *  chain    0, or the number of diffkv_decode_step(update_scores = 1) calls
 *           made just before this one on the same pool, page_table,
 *           tier_state and workspace, with nothing else writing them in
 *           between (seq_len one higher at each call).  The attention of
 *           such a step updates every score sum of a unit and, from them,
 *           plans the unit's next step (the generation-phase decision at
 *           length seq_len + 1) into the workspace; a chained call
 *           (chain > 0, update_scores = 1, one split per unit,
 *           batch * H <= 2048) takes those plans and runs no plan kernel.
 *           Each plan carries a tag of the length and tier state it was
 *           made for, and the pool's start pointer is checked against the
 *           previous step's: on any mismatch the whole step is aborted
 *           (nothing committed, DIFFKV_ST_STALE_CHAIN set; repeat it with
 *           chain = 0).  Ignored where a chained call does not apply.
 *           With more units (or unit splits) than compute units any call
 *           with chain > 0 also reuses the dispatch order (units by page
 *           count) the chain's first call left in the workspace,
 *           recomputing it every 16 calls; the order changes timing only,
 *           never results.
 *  workspace: diffkv_workspace_bytes(DIFFKV_DECODE_STEP[_SCORES]); it
 *           carries the plans from one chained call to the next; with
 *           update_scores = 2 it carries the logits to diffkv_update_scores
 *           at byte offset diffkv_workspace_bytes(DIFFKV_STEP) rounded up to
 *           256 (pass that sub-buffer). */
int diffkv_decode_step(const diffkv_config* cfg, const diffkv_pool* pool, int32_t batch,
                       const int32_t* seq_len, const uint16_t* k_new, const uint16_t* v_new,
                       const uint16_t* q, int32_t* page_table, int32_t* tier_state, float* out,
                       int32_t update_scores, int32_t chain, void* workspace, size_t workspace_bytes,
                       void* stream);

/* The score update of a preceding diffkv_decode_attn(update_scores = 2) call
 * with the same arguments and workspace (policy reading of the notes' stored
 * token scores: a running sum of received attention, max over the group's q
 * heads).  Writes the score segment of pool->pages and, like update_scores
 * = 1, the next step's plan record. */
int diffkv_update_scores(const diffkv_config* cfg, const diffkv_pool* pool, int32_t batch,
                         const int32_t* page_table, const int32_t* tier_state,
                         const int32_t* seq_len, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Decode attention without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, results and errors are those of
 * diffkv_decode_attn with update_scores 0 or 1; the scratch the call needs
 * is a fixed array of DIFFKV_NOALLOC_SCRATCH_BYTES inside the library (one
 * per GPU, held until the process ends; its device address is looked up
 * once per device, on the first call with that device current).
 *  - update_scores = 2 (logits kept for a later call) -> DIFFKV_E_INVALID.
 *  - A call whose workspace (diffkv_workspace_bytes(DIFFKV_ATTN or
 *    DIFFKV_ATTN_SCORES, batch)) exceeds the array -> DIFFKV_E_WORKSPACE,
 *    nothing enqueued.
 *  - Calls the library makes: no hipMalloc, hipFree or other allocation.
 *  - Every call on one GPU uses the same array and leaves its contents
 *    there: calls that overlap on one GPU (other streams, other threads)
 *    race and must be serialized by the caller. */
#define DIFFKV_NOALLOC_SCRATCH_BYTES (64u << 20)
int diffkv_decode_attn_noalloc(const diffkv_config* cfg, const diffkv_pool* pool, int32_t batch,
                               const uint16_t* q, const int32_t* page_table, const int32_t* tier_state,
                               const int32_t* seq_len, float* out, int32_t update_scores, void* stream);

/* Number of sequence splits (workgroups per unit) diffkv_decode_attn uses
 * for this config and batch; the workspace size depends on it.  1 when
 * batch * H >= 256; otherwise max(ceil(256 / (batch * H)), ceil(L / 256)),
 * at most L / 16 and 128 (L = one table row: ceil(max_seq_len / 16) + 1).
 * A unit then takes its
 * pages in chunks of max(ceil(pages / splits), 16), so units with many
 * retained pages use all splits and small ones few. */
int32_t diffkv_attn_splits(const diffkv_config* cfg, int32_t batch);

#ifdef __cplusplus
}
#endif
#endif
