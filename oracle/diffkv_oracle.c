/*
 * diffkv_oracle.c -- plain serial CPU oracle for the DiffKV hot path.
 *
 * TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code
 * with the HIP library under compressed_paged_attention_amd/.
 *
 * Every function follows a passage of the notes page "DiffKV: Differentiated
 * Memory Management for Large Language Models with Parallel KV Compaction"
 * (SOSP'25, arXiv 2412.03131); the passage is named at each function.  Where
 * the page leaves a step open, the reading taken is stated at the function.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC.
 * Floating point: fp32 steps use IEEE single arithmetic with round to
 * nearest even (x86-64 SSE, FLT_EVAL_METHOD 0, no contraction); attention
 * and softmax are computed in fp64.
 *
 * Parity status: every function here is pinned by a -m "not gpu" test
 * (closed forms, the Fig 6 worked example, invariants, brute force on tiny
 * inputs, numpy's IEEE fp16 conversion) except the fp32 rounding of the score
 * sums after a score update, which is compared within a tolerance only.
 */
#include "diffkv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* small helpers                                                             */
/* ------------------------------------------------------------------------ */

static int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int32_t round16(int32_t x) { return (x + 15) / 16 * 16; }

/* Tier codecs ("Results": the bit-split ablation compares K and V code
 * widths such as K8V4, K4V8, K4V2, K2V4, K8V2, K4V1).  All four widths 0
 * select the default pair, high K8V4 and low K4V2, with the page layout
 * below; any other choice uses the plain layout (codec_plain). */
static void tier_bits(const orc_cfg* c, int32_t tier, int32_t* kb, int32_t* vb) {
  int dflt = c->hi_k_bits == 0 && c->hi_v_bits == 0 && c->lo_k_bits == 0 && c->lo_v_bits == 0;
  if (tier == ORC_HI) {
    *kb = dflt ? 8 : c->hi_k_bits;
    *vb = dflt ? 4 : c->hi_v_bits;
  } else {
    *kb = dflt ? 4 : c->lo_k_bits;
    *vb = dflt ? 2 : c->lo_v_bits;
  }
}

/* The plain layout: any widths other than the default pair, or the default
 * pair given explicitly (it is not the default layout then).  Codes are
 * token-major and packed from bit 0: code (t, j) at bit (t d + j) b of its
 * segment. */
static int codec_plain(const orc_cfg* c) {
  return c->hi_k_bits != 0 || c->hi_v_bits != 0 || c->lo_k_bits != 0 || c->lo_v_bits != 0;
}

static int bits_ok(int32_t b) { return b == 1 || b == 2 || b == 4 || b == 8; }

static int levels_valid(const orc_cfg* c);

static int cfg_valid(const orc_cfg* c) {
  if (!c) return 0;
  if (!levels_valid(c)) return 0;
  if (codec_plain(c) && !(bits_ok(c->hi_k_bits) && bits_ok(c->hi_v_bits) && bits_ok(c->lo_k_bits) &&
                          bits_ok(c->lo_v_bits)))
    return 0;
  if (c->head_dim != 64 && c->head_dim != 128) return 0;
  if (c->num_kv_heads < 1 || c->gqa_group < 1 || c->gqa_group > 16) return 0;
  if (c->hi_page_tokens != 16 || c->lo_page_tokens != 2 * c->hi_page_tokens) return 0;
  /* N < 2^29 keeps fp32 score sums times counts exact in fp64 (exact threshold compares) */
  if (c->max_seq_len < 1 || c->max_seq_len >= (1 << 29) || c->window < 0) return 0;
  if (!(c->alpha_l >= 0.0f) || !(c->alpha_h >= 0.0f)) return 0;
  if (c->lo_enabled && c->alpha_l > c->alpha_h) return 0;
  if (c->prompt_rule != ORC_RULE_ALPHA_N && c->prompt_rule != ORC_RULE_ALPHA_I) return 0;
  if ((c->alpha_h_head == NULL) != (c->alpha_l_head == NULL)) return 0;
  if (c->alpha_h_head) {
    for (int32_t h = 0; h < c->num_kv_heads; h++) {
      float ah = c->alpha_h_head[h], al = c->alpha_l_head[h];
      if (!(al >= 0.0f) || !(ah >= 0.0f)) return 0;
      if (c->lo_enabled && al > ah) return 0;
    }
  }
  return 1;
}

/* Thresholds of KV head h: the head's own pair when the config carries
 * per-head arrays ("KV compression policy", the extensibility paragraph: one
 * shared pair by default, tuned per head as an option), else the shared pair. */
static double alpha_hi(const orc_cfg* c, int32_t h) {
  return (double)(c->alpha_h_head ? c->alpha_h_head[h] : c->alpha_h);
}
static double alpha_lo(const orc_cfg* c, int32_t h) {
  return (double)(c->alpha_l_head ? c->alpha_l_head[h] : c->alpha_l);
}

/* Entries of one table row ("Memory management": the row length is the
 * maximum sequence length over the high tier's tokens per page). */
static int32_t row_len(const orc_cfg* c) {
  /* The page says a row of S_max / T_h entries cannot overflow; one more is
   * needed (hi and lo pages together can exceed ceil(N/T_h) by one). */
  return (int32_t)cdiv64(c->max_seq_len, c->hi_page_tokens) + 1;
}

static int32_t num_levels(const orc_cfg* c) { return c->num_levels >= 3 ? c->num_levels : 2; }

int32_t orc_table_len(const orc_cfg* c) {
  /* one row per pair of levels (two tiers: one row) */
  return (num_levels(c) + 1) / 2 * row_len(c);
}

/* ------------------------------------------------------------------------ */
/* Unified page layout ("Memory management": unified pages have six segments:
 * quantized K, K metadata, quantized V, V metadata, token score, position;
 * tokens per page depend on the precision).  Segment order follows the page;
 * each segment starts on a 16-byte boundary.                                 */
/* ------------------------------------------------------------------------ */

int32_t orc_tier_layout(const orc_cfg* c, int32_t tier, int32_t seg[7]) {
  int32_t d = c->head_dim;
  int32_t T = (tier == ORC_HI) ? c->hi_page_tokens : c->lo_page_tokens;
  int32_t kbits, vbits;
  tier_bits(c, tier, &kbits, &vbits);
  int32_t size[6];
  size[0] = T * d * kbits / 8; /* K codes */
  size[1] = 4 * T;             /* K scale + zero, fp16 each */
  size[2] = T * d * vbits / 8; /* V codes */
  size[3] = 4 * T;             /* V scale + zero */
  size[4] = 4 * T;             /* score (fp32) */
  size[5] = 4 * T;             /* position (int32) */
  int32_t off = 0;
  for (int i = 0; i < 6; i++) {
    seg[i] = off;
    off += round16(size[i]);
  }
  seg[6] = off;
  return T;
}

int32_t orc_page_bytes(const orc_cfg* c) {
  if (!cfg_valid(c)) return -1;
  if (num_levels(c) >= 3) {
    int32_t best = 0, seg[7];
    for (int32_t l = 0; l < num_levels(c); l++) {
      orc_level_layout(c, l, seg);
      if (seg[6] > best) best = seg[6];
    }
    return best;
  }
  int32_t a[7], b[7];
  orc_tier_layout(c, ORC_HI, a);
  orc_tier_layout(c, ORC_LO, b);
  return a[6] > b[6] ? a[6] : b[6];
}

/* K codes are token-major: token t's d codes are contiguous.  8-bit codes
 * take one byte each.  4-bit codes: dims 8w..8w+7 of a token share 32-bit
 * word w; dim 8w+e sits in nibble n(e) = e/2 + 4 (e mod 2) (bits 4n..4n+3),
 * so even dims fill the low half-word and odd dims the high half-word. */
void orc_k_code_addr(const orc_cfg* c, int32_t tier, int32_t tok, int32_t j,
                     int32_t* byte, int32_t* shift) {
  int32_t seg[7];
  orc_tier_layout(c, tier, seg);
  int32_t d = c->head_dim;
  if (codec_plain(c)) {
    int32_t kb, vb;
    tier_bits(c, tier, &kb, &vb);
    int64_t bit = ((int64_t)tok * d + j) * kb;
    *byte = seg[0] + (int32_t)(bit / 8);
    *shift = (int32_t)(bit % 8);
    return;
  }
  if (tier == ORC_HI) {
    *byte = seg[0] + tok * d + j;
    *shift = 0;
  } else {
    int32_t e = j % 8;
    int32_t n = e / 2 + 4 * (e % 2);
    *byte = seg[0] + tok * (d / 2) + 4 * (j / 8) + n / 2;
    *shift = 4 * (n % 2);
  }
}

/* V codes use a token-vectorized layout (the page's value-layout idea:
 * vectorize along tokens, not features) cut into 64 equal lane chunks of
 * d/8 bytes.  For dim j put i = j mod 16, nb = j div 16, r = t mod 4.
 *   hi (16 tokens, 4 bits): q = t div 4, M = nb;
 *   lo (32 tokens, 2 bits): q = (t mod 16) div 4, M = 2 nb + (t div 16).
 * Chunk L = i + 16 q.  Inside the chunk the code is field h = r mod 2 of pair
 * P = 2 M + r div 2, where pair P sits in 32-bit word w with its two fields
 * 16 bits apart:
 *   hi: w = P div 4, bit = 4 (P mod 4) + 16 h
 *   lo: w = P div 8, bit = 2 (P mod 8) + 16 h
 * (little-endian words).  Every (t, j) gets a distinct field. */
void orc_v_code_addr(const orc_cfg* c, int32_t tier, int32_t tok, int32_t j,
                     int32_t* byte, int32_t* shift) {
  int32_t seg[7];
  orc_tier_layout(c, tier, seg);
  if (codec_plain(c)) {
    int32_t kb, vb;
    tier_bits(c, tier, &kb, &vb);
    int64_t bit = ((int64_t)tok * c->head_dim + j) * vb;
    *byte = seg[2] + (int32_t)(bit / 8);
    *shift = (int32_t)(bit % 8);
    return;
  }
  int32_t chunk = c->head_dim / 8;
  int32_t i = j % 16, nb = j / 16, r = tok % 4;
  int32_t q, M, w, bit;
  int32_t h = r % 2;
  if (tier == ORC_HI) {
    q = tok / 4;
    M = nb;
    int32_t P = 2 * M + r / 2;
    w = P / 4;
    bit = 4 * (P % 4) + 16 * h;
  } else {
    q = (tok % 16) / 4;
    M = 2 * nb + tok / 16;
    int32_t P = 2 * M + r / 2;
    w = P / 8;
    bit = 2 * (P % 8) + 16 * h;
  }
  int32_t L = i + 16 * q;
  *byte = seg[2] + L * chunk + 4 * w + bit / 8;
  *shift = bit % 8;
}

static void put_field(uint8_t* page, int32_t byte, int32_t shift, int32_t bits,
                      uint32_t val) {
  uint8_t mask = (uint8_t)(((1u << bits) - 1u) << shift);
  page[byte] = (uint8_t)((page[byte] & ~mask) | ((val << shift) & mask));
}

static uint32_t get_field(const uint8_t* page, int32_t byte, int32_t shift, int32_t bits) {
  return (page[byte] >> shift) & ((1u << bits) - 1u);
}

static void put_u16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void put_u32(uint8_t* p, uint32_t v) {
  for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static uint32_t get_u32(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static void write_slot(const orc_cfg* c, uint8_t* page, int32_t tier, int32_t slot,
                       const uint8_t* kc, const uint8_t* vc, const uint16_t km[2],
                       const uint16_t vm[2], float score, int32_t pos) {
  int32_t seg[7];
  orc_tier_layout(c, tier, seg);
  int32_t kbits, vbits;
  tier_bits(c, tier, &kbits, &vbits);
  for (int32_t j = 0; j < c->head_dim; j++) {
    int32_t byte, shift;
    orc_k_code_addr(c, tier, slot, j, &byte, &shift);
    put_field(page, byte, shift, kbits, kc[j]);
    orc_v_code_addr(c, tier, slot, j, &byte, &shift);
    put_field(page, byte, shift, vbits, vc[j]);
  }
  put_u16(page + seg[1] + 4 * slot, km[0]);
  put_u16(page + seg[1] + 4 * slot + 2, km[1]);
  put_u16(page + seg[3] + 4 * slot, vm[0]);
  put_u16(page + seg[3] + 4 * slot + 2, vm[1]);
  put_u32(page + seg[4] + 4 * slot, f32_bits(score));
  put_u32(page + seg[5] + 4 * slot, (uint32_t)pos);
}

void orc_read_slot(const orc_cfg* c, const uint8_t* page, int32_t tier, int32_t slot,
                   uint8_t* kc, uint8_t* vc, uint16_t* km, uint16_t* vm,
                   float* score, int32_t* pos) {
  int32_t seg[7];
  orc_tier_layout(c, tier, seg);
  int32_t kbits, vbits;
  tier_bits(c, tier, &kbits, &vbits);
  for (int32_t j = 0; j < c->head_dim; j++) {
    int32_t byte, shift;
    if (kc) {
      orc_k_code_addr(c, tier, slot, j, &byte, &shift);
      kc[j] = (uint8_t)get_field(page, byte, shift, kbits);
    }
    if (vc) {
      orc_v_code_addr(c, tier, slot, j, &byte, &shift);
      vc[j] = (uint8_t)get_field(page, byte, shift, vbits);
    }
  }
  if (km) { km[0] = get_u16(page + seg[1] + 4 * slot); km[1] = get_u16(page + seg[1] + 4 * slot + 2); }
  if (vm) { vm[0] = get_u16(page + seg[3] + 4 * slot); vm[1] = get_u16(page + seg[3] + 4 * slot + 2); }
  if (score) *score = bits_f32(get_u32(page + seg[4] + 4 * slot));
  if (pos) *pos = (int32_t)get_u32(page + seg[5] + 4 * slot);
}

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 conversion, written from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; subnormals below
 * 2^-14 with quantum 2^-24; rounding to nearest, ties to even.             */
/* ------------------------------------------------------------------------ */

uint16_t orc_f32_to_f16(float f) {
  uint32_t u = f32_bits(f);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
  double a = fabs((double)f);
  if (isinf(f)) return (uint16_t)(sign | 0x7c00u);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1) -> floor(log2 a) = e - 1 */
  int ex = e - 1;
  if (ex < -14) ex = -14; /* subnormal range shares the quantum 2^-24 */
  double quantum = ldexp(1.0, ex - 10);
  double n = nearbyint(a / quantum); /* exact division (power of two), RNE */
  if (n >= 2048.0) {      /* rounding carried into the next binade */
    n /= 2.0;
    ex += 1;
  }
  if (ex > 15) return (uint16_t)(sign | 0x7c00u); /* overflow to infinity */
  if (n < 1024.0) return (uint16_t)(sign | (uint16_t)n); /* subnormal (ex == -14) */
  uint16_t bexp = (uint16_t)(ex + 15);
  uint16_t frac = (uint16_t)(n - 1024.0);
  return (uint16_t)(sign | (bexp << 10) | frac);
}

float orc_f16_to_f32(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return (float)(s ? -v : v);
}

void orc_f32_to_f16_n(const float* x, uint16_t* h, int64_t n) {
  for (int64_t i = 0; i < n; i++) h[i] = orc_f32_to_f16(x[i]);
}
void orc_f16_to_f32_n(const uint16_t* h, float* x, int64_t n) {
  for (int64_t i = 0; i < n; i++) x[i] = orc_f16_to_f32(h[i]);
}

/* ------------------------------------------------------------------------ */
/* Asymmetric quantization ("Background", KV cache optimization: scale s and
 * zero z, Q = round((X - z) / s), X^ = s Q + z, applied to each K and each V
 * vector on its own).  Reading: z = min, s = (max - min)/(2^b - 1), both
 * stored as fp16 (rounded to nearest even); the code uses the stored fp16
 * values, fp32 IEEE division and rint (ties to even), clamped to
 * [0, 2^b - 1]; a zero scale gives code 0.                                 */
/* ------------------------------------------------------------------------ */

void orc_quantize(const float* x, int32_t n, int32_t bits, uint16_t* s16,
                  uint16_t* z16, uint8_t* codes) {
  float mn = x[0], mx = x[0];
  for (int32_t i = 1; i < n; i++) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  int32_t qmax = (1 << bits) - 1;
  float range = mx - mn;
  float scale = range / (float)qmax;
  *s16 = orc_f32_to_f16(scale);
  *z16 = orc_f32_to_f16(mn);
  float s = orc_f16_to_f32(*s16), z = orc_f16_to_f32(*z16);
  for (int32_t i = 0; i < n; i++) {
    if (s == 0.0f) {
      codes[i] = 0;
      continue;
    }
    float t = (x[i] - z) / s;
    float r = rintf(t);
    if (r < 0.0f) r = 0.0f;
    if (r > (float)qmax) r = (float)qmax;
    codes[i] = (uint8_t)r;
  }
}

float orc_dequant(uint16_t s16, uint16_t z16, int32_t code) {
  /* The product of an fp16 scale and a code of at most 8 bits is exact in
   * fp32, so this is one rounding (the add). */
  float s = orc_f16_to_f32(s16), z = orc_f16_to_f32(z16);
  float prod = s * (float)code;
  return prod + z;
}

/* ------------------------------------------------------------------------ */
/* Classification ("Approach" and "KV compression policy", prompt phase):
 * the last W tokens are always high precision; otherwise a token whose mean
 * score exceeds alpha_h/N is high, one in [alpha_l/N, alpha_h/N] is low, and
 * one below alpha_l/N is pruned.  N is the request's length (the approach
 * summary and the generation-phase algorithm use N).  The prompt passage
 * compares the i-th token against alpha/i instead, a threshold that adapts
 * along the sequence; prompt_rule = ORC_RULE_ALPHA_I takes that reading,
 * with i = position + 1 (tokens counted from 1).  Comparisons are made
 * without division, as s*N (or s*i) against alpha in fp64, which is exact
 * for N < 2^29.  With the low tier closed, a token is high iff
 * s*N >= alpha_l and pruned otherwise.                                     */
/* ------------------------------------------------------------------------ */

static int32_t classify_prompt(const orc_cfg* c, int32_t h, float s, int64_t N, int64_t p) {
  if (c->window > 0 && p >= N - c->window) return ORC_HI;
  int64_t denom = c->prompt_rule == ORC_RULE_ALPHA_I ? p + 1 : N;
  double x = (double)s * (double)denom;
  if (c->lo_enabled) {
    if (x > alpha_hi(c, h)) return ORC_HI;
    if (x >= alpha_lo(c, h)) return ORC_LO;
    return ORC_PRUNE;
  }
  return x >= alpha_lo(c, h) ? ORC_HI : ORC_PRUNE;
}

static int cu_valid(int32_t batch, const int64_t* cu) {
  if (batch < 0 || !cu || cu[0] != 0) return 0;
  for (int32_t r = 0; r < batch; r++)
    if (cu[r + 1] < cu[r]) return 0;
  return 1;
}

int orc_classify(const orc_cfg* c, int32_t batch, const int64_t* cu,
                 const float* scores, uint8_t* tiers, int32_t* counts) {
  if (!cfg_valid(c) || !cu_valid(batch, cu)) return ORC_E_INVALID;
  if (num_levels(c) >= 3) return orc_levels_classify(c, batch, cu, scores, tiers, counts);
  int32_t H = c->num_kv_heads;
  int64_t total = cu[batch];
  for (int32_t r = 0; r < batch; r++) {
    int64_t N = cu[r + 1] - cu[r];
    for (int32_t h = 0; h < H; h++) {
      int32_t nh = 0, nl = 0;
      for (int64_t p = 0; p < N; p++) {
        int64_t idx = (int64_t)h * total + cu[r] + p;
        int32_t t = classify_prompt(c, h, scores[idx], N, p);
        tiers[idx] = (uint8_t)t;
        if (t == ORC_HI) nh++;
        if (t == ORC_LO) nl++;
      }
      counts[((int64_t)r * H + h) * 2 + 0] = nh;
      counts[((int64_t)r * H + h) * 2 + 1] = nl;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Circular free page list ("Memory management": one contiguous list of all
 * page ids with an allocation pointer (start) and a reclamation pointer
 * (end), both wrapping; allocating advances start, freeing advances end; a
 * prefix sum over per-head counts gives each head its own region).
 * Reading: the two pointers are monotonically increasing 64-bit counters,
 * the list index is counter mod P and the free count is end - start.       */
/* ------------------------------------------------------------------------ */

int orc_pool_init(orc_pool* p) {
  if (!p || p->num_pages < 1) return ORC_E_INVALID;
  for (int64_t i = 0; i < p->num_pages; i++) p->free_list[i] = (int32_t)i;
  p->ptr[0] = 0;
  p->ptr[1] = (uint64_t)p->num_pages;
  p->status[0] = 0;
  return ORC_OK;
}

/* Plan + coordination of prompt compaction (Fig 6 workflow).  Per unit
 * (request r, KV head h; units in r-major, h-minor order):
 *   1. conservatively take k = ceil(N/T_h) pages (all assumed high), as one
 *      block from the allocation pointer, block ids in list order;
 *   2. plan n_hp = ceil(n_hi/T_h) high pages and n_lp = ceil(n_lo/T_l) low
 *      pages; high pages are block[0..n_hp) placed left to right in the
 *      table row, low pages are block[k-1], block[k-2], ... placed right to
 *      left;
 *   3. the unused middle of the block is appended at the reclamation pointer
 *      (units in order, each unit's pages in ascending block index);
 *   4. reading for the case the page misses: when n_hp + n_lp = k + 1 the
 *      block is one page short; that unit takes one more page from the
 *      allocation pointer after the frees, and it becomes the innermost low
 *      page (table index L_max - n_lp).
 * All or nothing: if the pool cannot supply the pages, or any unit is not
 * empty, nothing is written except the sticky status bit. */
static int prompt_allocate_core(int32_t H, int32_t T_h, int32_t T_l, int32_t L_max,
                                int32_t batch, const int64_t* seqlens,
                                const int32_t* n_hi, const int32_t* n_lo,
                                int32_t* free_list, uint64_t* ptr, uint32_t* status,
                                int64_t P, int32_t* table, int32_t* state,
                                int64_t S_max) {
  int64_t U = (int64_t)batch * H;
  int64_t K = 0, F = 0, E = 0;
  uint32_t st = 0;
  for (int64_t u = 0; u < U; u++) {
    int64_t N = seqlens[u / H];
    if (N <= 0) continue;
    const int32_t* s = state + 4 * u;
    if (s[0] || s[1] || s[2] || s[3]) st |= ORC_ST_BAD_STATE;
    if (n_hi[u] < 0 || n_lo[u] < 0 || n_hi[u] + n_lo[u] > N) st |= ORC_ST_BAD_STATE;
    if (S_max > 0 && N > S_max) st |= ORC_ST_TABLE_OVERFLOW;
    int64_t k = cdiv64(N, T_h), hp = cdiv64(n_hi[u], T_h), lp = cdiv64(n_lo[u], T_l);
    if (k > L_max || hp + lp > L_max) st |= ORC_ST_TABLE_OVERFLOW;
    K += k;
    if (k > hp + lp) F += k - hp - lp;
    if (hp + lp > k) E += hp + lp - k;
  }
  int64_t free0 = (int64_t)(ptr[1] - ptr[0]);
  if (!st && (K > free0 || K - F + E > free0)) st |= ORC_ST_POOL_EXHAUSTED;
  if (st) {
    *status |= st;
    return 0;
  }
  uint64_t start = ptr[0], end = ptr[1];
  int32_t* freed = (int32_t*)malloc(sizeof(int32_t) * (size_t)(F > 0 ? F : 1));
  int64_t nf = 0;
  /* 1-3: conservative block per unit, table placement, middle collected */
  for (int64_t u = 0; u < U; u++) {
    int64_t N = seqlens[u / H];
    if (N <= 0) continue;
    int64_t k = cdiv64(N, T_h), hp = cdiv64(n_hi[u], T_h), lp = cdiv64(n_lo[u], T_l);
    int32_t* row = table + u * L_max;
    for (int64_t i = 0; i < k; i++) {
      int32_t id = free_list[(start + (uint64_t)i) % (uint64_t)P];
      if (i < hp) row[i] = id;                      /* high: left to right */
      else if (i >= k - lp) row[L_max - 1 - (k - 1 - i)] = id; /* low: right to left */
      else freed[nf++] = id;                        /* unused middle */
    }
    start += (uint64_t)k;
  }
  /* 3: reclaim at the end pointer */
  for (int64_t i = 0; i < nf; i++) free_list[(end + (uint64_t)i) % (uint64_t)P] = freed[i];
  end += (uint64_t)nf;
  /* 4: extra page for units whose block was one short */
  for (int64_t u = 0; u < U; u++) {
    int64_t N = seqlens[u / H];
    if (N <= 0) continue;
    int64_t k = cdiv64(N, T_h), hp = cdiv64(n_hi[u], T_h), lp = cdiv64(n_lo[u], T_l);
    if (hp + lp > k) {
      table[u * L_max + (L_max - lp)] = free_list[start % (uint64_t)P];
      start += 1;
    }
    state[4 * u + 0] = n_hi[u];
    state[4 * u + 1] = n_lo[u];
    state[4 * u + 2] = (int32_t)hp;
    state[4 * u + 3] = (int32_t)lp;
  }
  ptr[0] = start;
  ptr[1] = end;
  free(freed);
  return 1;
}

int orc_prompt_allocate(int32_t H, int32_t T_h, int32_t T_l, int32_t L_max,
                        int32_t batch, const int64_t* seqlens,
                        const int32_t* n_hi, const int32_t* n_lo,
                        int32_t* free_list, uint64_t* ptr, uint32_t* status,
                        int64_t num_pages, int32_t* page_table,
                        int32_t* tier_state) {
  if (H < 1 || T_h < 1 || T_l < 1 || L_max < 1 || batch < 0 || num_pages < 1) return ORC_E_INVALID;
  prompt_allocate_core(H, T_h, T_l, L_max, batch, seqlens, n_hi, n_lo, free_list, ptr,
                       status, num_pages, page_table, tier_state, 0);
  return ORC_OK;
}

static uint8_t* page_at(orc_pool* p, int32_t id) {
  return p->pages + (int64_t)id * p->page_bytes;
}

/* Quantize one token (fp32 K and V vectors) for a tier and write its slot. */
static void store_token(const orc_cfg* c, uint8_t* page, int32_t tier, int32_t slot,
                        const float* xk, const float* xv, float score, int32_t pos) {
  int32_t d = c->head_dim;
  uint8_t kc[128], vc[128];
  uint16_t km[2], vm[2];
  int32_t kb, vb;
  tier_bits(c, tier, &kb, &vb);
  orc_quantize(xk, d, kb, &km[0], &km[1], kc);
  orc_quantize(xv, d, vb, &vm[0], &vm[1], vc);
  write_slot(c, page, tier, slot, kc, vc, km, vm, score, pos);
}

/* Prompt compaction: classify counts, the Fig 6 plan/coordination above,
 * then packing.  Packing reading: inside a tier, tokens take slots in
 * position order; high slot s lives in the page at table index s div T_h,
 * low slot s in the page at L_max - 1 - (s div T_l); every page handed to a
 * unit is zero-filled before its tokens are written.  The stored score is
 * the running sum of received attention, mean * count with
 * count = N - 1 - p queries so far (one fp32 multiply), so a later mean is
 * sum / count. */
int orc_compact_prompt(const orc_cfg* c, orc_pool* p, int32_t batch,
                       const int64_t* cu, const uint16_t* k, const uint16_t* v,
                       const float* scores, const uint8_t* tiers,
                       int32_t* table, int32_t* state) {
  if (!cfg_valid(c) || !p || !cu_valid(batch, cu)) return ORC_E_INVALID;
  if (p->page_bytes != orc_page_bytes(c)) return ORC_E_INVALID;
  if (num_levels(c) >= 3) return orc_levels_compact_prompt(c, p, batch, cu, k, v, scores, tiers, table, state);
  int32_t H = c->num_kv_heads, d = c->head_dim, L = orc_table_len(c);
  int32_t Th = c->hi_page_tokens, Tl = c->lo_page_tokens;
  int64_t total = cu[batch];
  int64_t U = (int64_t)batch * H;
  int64_t* seqlens = (int64_t*)malloc(sizeof(int64_t) * (size_t)(batch > 0 ? batch : 1));
  int32_t* nh = (int32_t*)calloc((size_t)(U > 0 ? U : 1), sizeof(int32_t));
  int32_t* nl = (int32_t*)calloc((size_t)(U > 0 ? U : 1), sizeof(int32_t));
  for (int32_t r = 0; r < batch; r++) seqlens[r] = cu[r + 1] - cu[r];
  for (int64_t u = 0; u < U; u++) {
    int32_t r = (int32_t)(u / H), h = (int32_t)(u % H);
    for (int64_t t = 0; t < seqlens[r]; t++) {
      uint8_t ti = tiers[(int64_t)h * total + cu[r] + t];
      if (ti == ORC_HI) nh[u]++;
      else if (ti == ORC_LO) nl[u]++;
    }
  }
  int ok = prompt_allocate_core(H, Th, Tl, L, batch, seqlens, nh, nl, p->free_list, p->ptr,
                                p->status, p->num_pages, table, state, c->max_seq_len);
  if (ok) {
    float xk[128], xv[128];
    for (int64_t u = 0; u < U; u++) {
      int32_t r = (int32_t)(u / H), h = (int32_t)(u % H);
      int64_t N = seqlens[r];
      if (N <= 0) continue;
      int32_t* row = table + u * L;
      for (int32_t j = 0; j < state[4 * u + 2]; j++) memset(page_at(p, row[j]), 0, (size_t)p->page_bytes);
      for (int32_t j = 0; j < state[4 * u + 3]; j++) memset(page_at(p, row[L - 1 - j]), 0, (size_t)p->page_bytes);
      int32_t sh = 0, sl = 0;
      for (int64_t t = 0; t < N; t++) {
        int64_t idx = (int64_t)h * total + cu[r] + t;
        uint8_t ti = tiers[idx];
        if (ti != ORC_HI && ti != ORC_LO) continue;
        const uint16_t* kr = k + ((cu[r] + t) * H + h) * d;
        const uint16_t* vr = v + ((cu[r] + t) * H + h) * d;
        for (int32_t j = 0; j < d; j++) {
          xk[j] = orc_f16_to_f32(kr[j]);
          xv[j] = orc_f16_to_f32(vr[j]);
        }
        float sum = scores[idx] * (float)(N - 1 - t);
        if (ti == ORC_HI) {
          int32_t s = sh++;
          store_token(c, page_at(p, row[s / Th]), ORC_HI, s % Th, xk, xv, sum, (int32_t)t);
        } else {
          int32_t s = sl++;
          store_token(c, page_at(p, row[L - 1 - s / Tl]), ORC_LO, s % Tl, xk, xv, sum, (int32_t)t);
        }
      }
    }
  }
  free(seqlens);
  free(nh);
  free(nl);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Generation-phase step ("KV compression policy", generation phase and the
 * algorithm flow; "Memory management", generation workflow; "Implementation":
 * the compactor runs before the attention kernel).
 *
 * Per active unit with current length N (the new token gets position N and
 * N' = N + 1 is the length the thresholds use):
 *   - the new token enters the window, i.e. the high tier (8/4 bits);
 *   - t_c, the token at position N - W, just left the window; its mean is
 *     sum / (W - 1) and it is classified against alpha/N';
 *   - t_c high: the least important non-window high token t_v (position
 *     <= N - W, t_c included) stays if its mean still exceeds alpha_h/N', is
 *     requantized to the low tier if it lies in [alpha_l/N', alpha_h/N'], and
 *     is pruned otherwise;
 *   - t_c low: t_c is requantized into the low tier; the least important low
 *     token (t_c included) is pruned if its mean is below alpha_l/N';
 *   - t_c pruned: it is removed.
 * Readings: means are compared without division (sum_a cnt_b vs
 * sum_b cnt_a in fp64; ties go to the smaller position); count of a token at
 * position p is N - 1 - p; requantization starts from the fp32 values
 * dequantized from the high codes; a removal and an insertion in the same
 * tier share the slot, otherwise the insertion appends.  Neither tier ever
 * shrinks, so a unit needs at most one new page per step and never frees
 * one (pages return only on release).  All or nothing over the call. */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t active;
  int32_t new_hi_slot, hi_append;
  int32_t lo_src_hi_slot; /* hi slot of the token moving to the low tier, -1 */
  int32_t lo_slot, lo_append;
  int32_t need_page;      /* 0 none, ORC_HI or ORC_LO */
  int32_t page_id;
} step_plan;

static int32_t classify_mean(const orc_cfg* c, int32_t h, float sum, int64_t cnt, int64_t Np) {
  double x = (double)sum * (double)Np;
  double ch = alpha_hi(c, h) * (double)cnt, cl = alpha_lo(c, h) * (double)cnt;
  if (c->lo_enabled) {
    if (x > ch) return ORC_HI;
    if (x >= cl) return ORC_LO;
    return ORC_PRUNE;
  }
  return x >= cl ? ORC_HI : ORC_PRUNE;
}

/* a strictly less important than b */
static int less_important(float sa, int64_t ca, int32_t pa, float sb, int64_t cb, int32_t pb) {
  double l = (double)sa * (double)cb, r = (double)sb * (double)ca;
  if (l != r) return l < r;
  return pa < pb;
}

static uint8_t* slot_page(orc_pool* p, const int32_t* row, int32_t L, int32_t tier,
                          int32_t slot, const orc_cfg* c) {
  if (tier == ORC_HI) return page_at(p, row[slot / c->hi_page_tokens]);
  return page_at(p, row[L - 1 - slot / c->lo_page_tokens]);
}

/* branch (optional, test bookkeeping): per unit the case the plan took,
 * ORC_BR_* in bits 0-3 and the tier of a new page (0 none) in bits 4-5. */
static int compact_step_impl(const orc_cfg* c, orc_pool* p, int32_t batch,
                             const int32_t* seq_len, const uint16_t* k_new,
                             const uint16_t* v_new, int32_t* table, int32_t* state,
                             int32_t* branch) {
  if (!cfg_valid(c) || !p || batch < 0 || c->window < 2) return ORC_E_INVALID;
  if (p->page_bytes != orc_page_bytes(c)) return ORC_E_INVALID;
  int32_t H = c->num_kv_heads, d = c->head_dim, L = orc_table_len(c), W = c->window;
  int32_t Th = c->hi_page_tokens, Tl = c->lo_page_tokens;
  int64_t U = (int64_t)batch * H;
  step_plan* pl = (step_plan*)calloc((size_t)(U > 0 ? U : 1), sizeof(step_plan));
  uint32_t st = 0;
  int64_t demand = 0;
  for (int64_t u = 0; u < U; u++) {
    step_plan* P = &pl[u];
    P->lo_src_hi_slot = -1;
    int64_t N = seq_len[u / H];
    if (N <= 0) continue;
    P->active = 1;
    int32_t n_hi = state[4 * u], n_lo = state[4 * u + 1], ph = state[4 * u + 2], plo = state[4 * u + 3];
    if (N + 1 > c->max_seq_len) { st |= ORC_ST_TABLE_OVERFLOW; continue; }
    if (n_hi < 0 || n_lo < 0 || ph != cdiv64(n_hi, Th) || plo != cdiv64(n_lo, Tl) ||
        n_hi + n_lo > N || ph + plo > L) {
      st |= ORC_ST_BAD_STATE;
      continue;
    }
    const int32_t* row = table + u * L;
    int bad_id = 0;
    for (int32_t j = 0; j < ph; j++) if (row[j] < 0 || row[j] >= p->num_pages) bad_id = 1;
    for (int32_t j = 0; j < plo; j++) if (row[L - 1 - j] < 0 || row[L - 1 - j] >= p->num_pages) bad_id = 1;
    if (bad_id) { st |= ORC_ST_BAD_STATE; continue; }
    int64_t Np = N + 1;
    int64_t tc_pos = N - W;
    int32_t hh = (int32_t)(u % H);
    P->new_hi_slot = n_hi;
    P->hi_append = 1;
    if (branch) branch[u] = ORC_BR_NO_TC;
    if (tc_pos >= 0) {
      int32_t tc = -1;
      float tc_sum = 0;
      for (int32_t s = 0; s < n_hi; s++) {
        float sc; int32_t pos;
        orc_read_slot(c, slot_page(p, row, L, ORC_HI, s, c), ORC_HI, s % Th, 0, 0, 0, 0, &sc, &pos);
        if (pos == tc_pos) { tc = s; tc_sum = sc; }
      }
      if (tc < 0) { st |= ORC_ST_BAD_STATE; continue; }
      int32_t cls = classify_mean(c, hh, tc_sum, W - 1, Np);
      if (cls == ORC_HI) {
        int32_t v = -1; float vs = 0; int32_t vp = 0; int64_t vc = 0;
        for (int32_t s = 0; s < n_hi; s++) {
          float sc; int32_t pos;
          orc_read_slot(c, slot_page(p, row, L, ORC_HI, s, c), ORC_HI, s % Th, 0, 0, 0, 0, &sc, &pos);
          if (pos > tc_pos) continue; /* window */
          int64_t cnt = N - 1 - pos;
          if (v < 0 || less_important(sc, cnt, pos, vs, vc, vp)) { v = s; vs = sc; vp = pos; vc = cnt; }
        }
        int32_t vcls = classify_mean(c, hh, vs, vc, Np);
        if (branch) branch[u] = vcls == ORC_HI ? ORC_BR_HI_KEEP : (vcls == ORC_LO ? ORC_BR_HI_DEMOTE : ORC_BR_HI_PRUNE);
        if (vcls == ORC_LO) {
          P->lo_src_hi_slot = v;
          P->lo_slot = n_lo;
          P->lo_append = 1;
          P->new_hi_slot = v;
          P->hi_append = 0;
        } else if (vcls == ORC_PRUNE) {
          P->new_hi_slot = v;
          P->hi_append = 0;
        }
      } else if (cls == ORC_LO) {
        P->lo_src_hi_slot = tc;
        P->new_hi_slot = tc;
        P->hi_append = 0;
        /* least important among low tokens and t_c */
        int32_t v = -1; float vs = tc_sum; int32_t vp = (int32_t)tc_pos; int64_t vc = W - 1;
        for (int32_t s = 0; s < n_lo; s++) {
          float sc; int32_t pos;
          orc_read_slot(c, slot_page(p, row, L, ORC_LO, s, c), ORC_LO, s % Tl, 0, 0, 0, 0, &sc, &pos);
          int64_t cnt = N - 1 - pos;
          if (less_important(sc, cnt, pos, vs, vc, vp)) { v = s; vs = sc; vp = pos; vc = cnt; }
        }
        if (v >= 0 && classify_mean(c, hh, vs, vc, Np) == ORC_PRUNE) {
          P->lo_slot = v;
          P->lo_append = 0;
          if (branch) branch[u] = ORC_BR_LO_PRUNE;
        } else {
          if (branch) branch[u] = ORC_BR_LO_KEEP;
          P->lo_slot = n_lo;
          P->lo_append = 1;
        }
      } else {
        P->new_hi_slot = tc;
        P->hi_append = 0;
        if (branch) branch[u] = ORC_BR_PRUNE;
      }
    }
    if (P->hi_append && n_hi % Th == 0) P->need_page = ORC_HI;
    if (P->lo_append && n_lo % Tl == 0) P->need_page = ORC_LO;
    if (branch) branch[u] |= P->need_page << 4;
    if (P->need_page && ph + plo + 1 > L) { st |= ORC_ST_TABLE_OVERFLOW; continue; }
    if (P->need_page) demand++;
  }
  if (!st && demand > (int64_t)(p->ptr[1] - p->ptr[0])) st |= ORC_ST_POOL_EXHAUSTED;
  if (st) {
    p->status[0] |= st;
    free(pl);
    return ORC_OK;
  }
  /* coordination: pages in unit order from the allocation pointer */
  uint64_t start = p->ptr[0];
  for (int64_t u = 0; u < U; u++) {
    if (!pl[u].active || !pl[u].need_page) continue;
    pl[u].page_id = p->free_list[start % (uint64_t)p->num_pages];
    start++;
  }
  p->ptr[0] = start;
  /* commit */
  float xk[128], xv[128];
  for (int64_t u = 0; u < U; u++) {
    step_plan* P = &pl[u];
    if (!P->active) continue;
    int32_t b = (int32_t)(u / H);
    int32_t* row = table + u * L;
    int32_t* s4 = state + 4 * u;
    if (P->need_page == ORC_HI) {
      row[s4[2]] = P->page_id;
      s4[2]++;
      memset(page_at(p, P->page_id), 0, (size_t)p->page_bytes);
    } else if (P->need_page == ORC_LO) {
      row[L - 1 - s4[3]] = P->page_id;
      s4[3]++;
      memset(page_at(p, P->page_id), 0, (size_t)p->page_bytes);
    }
    if (P->lo_src_hi_slot >= 0) {
      uint8_t kc[128], vc[128];
      uint16_t km[2], vm[2];
      float sc; int32_t pos;
      orc_read_slot(c, slot_page(p, row, L, ORC_HI, P->lo_src_hi_slot, c), ORC_HI,
                    P->lo_src_hi_slot % Th, kc, vc, km, vm, &sc, &pos);
      for (int32_t j = 0; j < d; j++) {
        xk[j] = orc_dequant(km[0], km[1], kc[j]);
        xv[j] = orc_dequant(vm[0], vm[1], vc[j]);
      }
      store_token(c, slot_page(p, row, L, ORC_LO, P->lo_slot, c), ORC_LO, P->lo_slot % Tl,
                  xk, xv, sc, pos);
      if (P->lo_append) s4[1]++;
    }
    const uint16_t* kr = k_new + ((int64_t)b * H + (u % H)) * d;
    const uint16_t* vr = v_new + ((int64_t)b * H + (u % H)) * d;
    for (int32_t j = 0; j < d; j++) {
      xk[j] = orc_f16_to_f32(kr[j]);
      xv[j] = orc_f16_to_f32(vr[j]);
    }
    store_token(c, slot_page(p, row, L, ORC_HI, P->new_hi_slot, c), ORC_HI, P->new_hi_slot % Th,
                xk, xv, 0.0f, seq_len[b]);
    if (P->hi_append) s4[0]++;
  }
  free(pl);
  return ORC_OK;
}

int orc_compact_step(const orc_cfg* c, orc_pool* p, int32_t batch,
                     const int32_t* seq_len, const uint16_t* k_new,
                     const uint16_t* v_new, int32_t* table, int32_t* state) {
  if (c && num_levels(c) >= 3) return orc_levels_compact_step(c, p, batch, seq_len, k_new, v_new, table, state, NULL);
  return compact_step_impl(c, p, batch, seq_len, k_new, v_new, table, state, NULL);
}

int orc_compact_step_branches(const orc_cfg* c, orc_pool* p, int32_t batch,
                              const int32_t* seq_len, const uint16_t* k_new,
                              const uint16_t* v_new, int32_t* table, int32_t* state,
                              int32_t* branch) {
  if (c && num_levels(c) >= 3) return orc_levels_compact_step(c, p, batch, seq_len, k_new, v_new, table, state, branch);
  if (branch)
    for (int64_t u = 0; u < (int64_t)batch * (c ? c->num_kv_heads : 0); u++) branch[u] = ORC_BR_INACTIVE;
  return compact_step_impl(c, p, batch, seq_len, k_new, v_new, table, state, branch);
}

/* Release ("Memory management", generation workflow: when a request
 * completes, all its pages are reclaimed).  Units of released requests in
 * order; each unit's high pages (table left to right) then low pages (table
 * right to left) are appended at the reclamation pointer; the rows are reset
 * to -1 and the unit state to zero. */
int orc_release(const orc_cfg* c, orc_pool* p, int32_t batch, const uint8_t* mask,
                int32_t* table, int32_t* state) {
  if (!cfg_valid(c) || !p || batch < 0) return ORC_E_INVALID;
  if (num_levels(c) >= 3) return orc_levels_release(c, p, batch, mask, table, state);
  int32_t H = c->num_kv_heads, L = orc_table_len(c);
  int64_t U = (int64_t)batch * H, total = 0;
  uint32_t st = 0;
  for (int64_t u = 0; u < U; u++) {
    if (!mask[u / H]) continue;
    int32_t ph = state[4 * u + 2], plo = state[4 * u + 3];
    if (ph < 0 || plo < 0 || ph + plo > L) { st |= ORC_ST_BAD_STATE; continue; }
    /* a page id outside the pool would enter the free list: refuse the call */
    const int32_t* row = table + u * L;
    for (int32_t j = 0; j < ph; j++) if (row[j] < 0 || row[j] >= p->num_pages) st |= ORC_ST_BAD_STATE;
    for (int32_t j = 0; j < plo; j++) if (row[L - 1 - j] < 0 || row[L - 1 - j] >= p->num_pages) st |= ORC_ST_BAD_STATE;
    total += ph + plo;
  }
  if (!st && (int64_t)(p->ptr[1] - p->ptr[0]) + total > p->num_pages) st |= ORC_ST_BAD_STATE;
  if (st) {
    p->status[0] |= st;
    return ORC_OK;
  }
  uint64_t end = p->ptr[1];
  for (int64_t u = 0; u < U; u++) {
    if (!mask[u / H]) continue;
    int32_t* row = table + u * L;
    int32_t ph = state[4 * u + 2], plo = state[4 * u + 3];
    for (int32_t j = 0; j < ph; j++) p->free_list[(end++) % (uint64_t)p->num_pages] = row[j];
    for (int32_t j = 0; j < plo; j++) p->free_list[(end++) % (uint64_t)p->num_pages] = row[L - 1 - j];
    for (int32_t j = 0; j < L; j++) row[j] = -1;
    for (int32_t j = 0; j < 4; j++) state[4 * u + j] = 0;
  }
  p->ptr[1] = end;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Attention ("Background", the attention formula: softmax of q.k/sqrt(d)
 * over the cached tokens weighting the values; GQA: the q heads of a group
 * share one KV head).  Over the compressed cache the keys and values are the
 * dequantized ones and only retained tokens take part.  fp64 throughout.   */
/* ------------------------------------------------------------------------ */

void orc_attention_dense(const double* q, const double* k, const double* v, int32_t n,
                         int32_t d, double* out) {
  double* x = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double scale = 1.0 / sqrt((double)d), m = -INFINITY, z = 0.0;
  for (int32_t t = 0; t < n; t++) {
    double acc = 0.0;
    for (int32_t i = 0; i < d; i++) acc += q[i] * k[(int64_t)t * d + i];
    x[t] = acc * scale;
    if (x[t] > m) m = x[t];
  }
  for (int32_t t = 0; t < n; t++) z += exp(x[t] - m);
  for (int32_t i = 0; i < d; i++) out[i] = 0.0;
  for (int32_t t = 0; t < n; t++) {
    double pr = exp(x[t] - m) / z;
    for (int32_t i = 0; i < d; i++) out[i] += pr * v[(int64_t)t * d + i];
  }
  free(x);
}

/* The page's decomposition: each token adds coefficient (softmax weight
 * times |v|) times the unit vector v/|v|; a zero value vector adds nothing. */
void orc_attention_unit_vectors(const double* q, const double* k, const double* v,
                                int32_t n, int32_t d, double* out) {
  double* x = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double scale = 1.0 / sqrt((double)d), m = -INFINITY, z = 0.0;
  for (int32_t t = 0; t < n; t++) {
    double acc = 0.0;
    for (int32_t i = 0; i < d; i++) acc += q[i] * k[(int64_t)t * d + i];
    x[t] = acc * scale;
    if (x[t] > m) m = x[t];
  }
  for (int32_t t = 0; t < n; t++) z += exp(x[t] - m);
  for (int32_t i = 0; i < d; i++) out[i] = 0.0;
  for (int32_t t = 0; t < n; t++) {
    double norm = 0.0;
    for (int32_t i = 0; i < d; i++) norm += v[(int64_t)t * d + i] * v[(int64_t)t * d + i];
    norm = sqrt(norm);
    if (norm == 0.0) continue;
    double coef = exp(x[t] - m) / z * norm;
    for (int32_t i = 0; i < d; i++) out[i] += coef * (v[(int64_t)t * d + i] / norm);
  }
  free(x);
}

/* Decode attention over the compressed cache of each active request: one
 * query per q head, keys/values dequantized from every retained slot (high
 * pages then low pages; the order does not change the result), softmax in
 * fp64, output rounded to fp32.  An inactive request (seq_len <= 0) or a unit
 * without tokens gives zeros.
 * Score update (reading of the stored token scores, policy section): with
 * update_scores set, each retained token other than the query's own
 * (position < seq_len) adds the max over the group's q heads of its softmax
 * weight to its stored sum (fp32 add of the fp64 value rounded once). */
int orc_decode_attn(const orc_cfg* c, orc_pool* p, int32_t batch, const uint16_t* q,
                    const int32_t* table, const int32_t* state, const int32_t* seq_len,
                    float* out, int32_t update_scores) {
  if (!cfg_valid(c) || !p || batch < 0) return ORC_E_INVALID;
  if (p->page_bytes != orc_page_bytes(c)) return ORC_E_INVALID;
  if (num_levels(c) >= 3) return orc_levels_decode_attn(c, p, batch, q, table, state, seq_len, out, update_scores);
  int32_t H = c->num_kv_heads, G = c->gqa_group, d = c->head_dim, L = orc_table_len(c);
  int32_t Th = c->hi_page_tokens, Tl = c->lo_page_tokens;
  memset(out, 0, sizeof(float) * (size_t)batch * H * G * d);
  uint32_t st = 0;
  for (int64_t u = 0; u < (int64_t)batch * H; u++) {
    int32_t b = (int32_t)(u / H), h = (int32_t)(u % H);
    if (seq_len[b] <= 0) continue;
    const int32_t* s4 = state + 4 * u;
    const int32_t* row = table + u * L;
    int32_t n_hi = s4[0], n_lo = s4[1];
    int bad = (n_hi < 0 || n_lo < 0 || s4[2] != cdiv64(n_hi, Th) || s4[3] != cdiv64(n_lo, Tl) ||
               s4[2] + s4[3] > L);
    if (!bad) {
      for (int32_t j = 0; j < s4[2]; j++) if (row[j] < 0 || row[j] >= p->num_pages) bad = 1;
      for (int32_t j = 0; j < s4[3]; j++) if (row[L - 1 - j] < 0 || row[L - 1 - j] >= p->num_pages) bad = 1;
    }
    if (bad) { st |= ORC_ST_BAD_STATE; continue; }
    int32_t n = n_hi + n_lo;
    if (n == 0) continue;
    double* kh = (double*)malloc(sizeof(double) * (size_t)n * d);
    double* vh = (double*)malloc(sizeof(double) * (size_t)n * d);
    int32_t* tier = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t* slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    double* pmax = (double*)calloc((size_t)n, sizeof(double));
    double* x = (double*)malloc(sizeof(double) * (size_t)n);
    for (int32_t t = 0; t < n; t++) {
      int32_t tr = t < n_hi ? ORC_HI : ORC_LO;
      int32_t s = t < n_hi ? t : t - n_hi;
      uint8_t kc[128], vc[128];
      uint16_t km[2], vm[2];
      float sc;
      const uint8_t* pg = slot_page(p, row, L, tr, s, c);
      orc_read_slot(c, pg, tr, s % (tr == ORC_HI ? Th : Tl), kc, vc, km, vm, &sc, &pos[t]);
      tier[t] = tr;
      slot[t] = s;
      for (int32_t i = 0; i < d; i++) {
        kh[(int64_t)t * d + i] = (double)orc_dequant(km[0], km[1], kc[i]);
        vh[(int64_t)t * d + i] = (double)orc_dequant(vm[0], vm[1], vc[i]);
      }
    }
    double scale = 1.0 / sqrt((double)d);
    for (int32_t g = 0; g < G; g++) {
      int32_t jh = h * G + g;
      const uint16_t* qr = q + ((int64_t)b * H * G + jh) * d;
      double qd[128];
      for (int32_t i = 0; i < d; i++) qd[i] = (double)orc_f16_to_f32(qr[i]);
      double m = -INFINITY, z = 0.0;
      for (int32_t t = 0; t < n; t++) {
        double acc = 0.0;
        for (int32_t i = 0; i < d; i++) acc += qd[i] * kh[(int64_t)t * d + i];
        x[t] = acc * scale;
        if (x[t] > m) m = x[t];
      }
      for (int32_t t = 0; t < n; t++) z += exp(x[t] - m);
      float* o = out + ((int64_t)b * H * G + jh) * d;
      for (int32_t i = 0; i < d; i++) {
        double acc = 0.0;
        for (int32_t t = 0; t < n; t++) acc += exp(x[t] - m) / z * vh[(int64_t)t * d + i];
        o[i] = (float)acc;
      }
      for (int32_t t = 0; t < n; t++) {
        double pr = exp(x[t] - m) / z;
        if (pr > pmax[t]) pmax[t] = pr;
      }
    }
    if (update_scores) {
      for (int32_t t = 0; t < n; t++) {
        if (pos[t] >= seq_len[b]) continue;
        int32_t tr = tier[t], s = slot[t];
        uint8_t* pg = slot_page(p, row, L, tr, s, c);
        int32_t seg[7];
        orc_tier_layout(c, tr, seg);
        uint8_t* sp = pg + seg[4] + 4 * (s % (tr == ORC_HI ? Th : Tl));
        float old = bits_f32(get_u32(sp));
        float nw = (float)((double)old + pmax[t]);
        put_u32(sp, f32_bits(nw));
      }
    }
    free(kh); free(vh); free(tier); free(slot); free(pos); free(pmax); free(x);
  }
  p->status[0] |= st;
  return ORC_OK;
}

/* Prompt importance ("KV compression policy", prompt phase: a token's
 * importance is the mean of the attention it receives; for GQA the group's
 * q heads are combined with max).  Here the receiving attention comes from
 * nq probe queries per request that attend to every token of the request;
 * per probe query the max over the group's q heads is taken, then the mean
 * over probes (fp64, rounded to fp32 once). */
int orc_importance_from_queries(const orc_cfg* c, int32_t batch, const int64_t* cu,
                                const uint16_t* k, int32_t nq, const uint16_t* qp,
                                float* scores) {
  if (!cfg_valid(c) || !cu_valid(batch, cu) || nq < 1) return ORC_E_INVALID;
  int32_t H = c->num_kv_heads, G = c->gqa_group, d = c->head_dim;
  int64_t total = cu[batch];
  double scale = 1.0 / sqrt((double)d);
  for (int32_t r = 0; r < batch; r++) {
    int64_t N = cu[r + 1] - cu[r];
    if (N <= 0) continue;
    double* acc = (double*)malloc(sizeof(double) * (size_t)N);
    double* mx = (double*)malloc(sizeof(double) * (size_t)N);
    double* x = (double*)malloc(sizeof(double) * (size_t)N);
    for (int32_t h = 0; h < H; h++) {
      for (int64_t t = 0; t < N; t++) acc[t] = 0.0;
      for (int32_t qi = 0; qi < nq; qi++) {
        for (int64_t t = 0; t < N; t++) mx[t] = 0.0;
        for (int32_t g = 0; g < G; g++) {
          const uint16_t* qr = qp + (((int64_t)r * nq + qi) * H * G + (h * G + g)) * d;
          double m = -INFINITY, z = 0.0;
          for (int64_t t = 0; t < N; t++) {
            const uint16_t* kr = k + ((cu[r] + t) * H + h) * d;
            double a = 0.0;
            for (int32_t i = 0; i < d; i++)
              a += (double)orc_f16_to_f32(qr[i]) * (double)orc_f16_to_f32(kr[i]);
            x[t] = a * scale;
            if (x[t] > m) m = x[t];
          }
          for (int64_t t = 0; t < N; t++) z += exp(x[t] - m);
          for (int64_t t = 0; t < N; t++) {
            double pr = exp(x[t] - m) / z;
            if (pr > mx[t]) mx[t] = pr;
          }
        }
        for (int64_t t = 0; t < N; t++) acc[t] += mx[t];
      }
      for (int64_t t = 0; t < N; t++) scores[(int64_t)h * total + cu[r] + t] = (float)(acc[t] / nq);
    }
    free(acc); free(mx); free(x);
  }
  return ORC_OK;
}

/* Prompt importance from the prompt's own queries ("KV compression policy",
 * prompt phase: the importance of token i is the average of the attention
 * scores it receives from the tokens after it; for GQA the scores of the q
 * heads sharing the KV head are combined with max).  Causal attention: query
 * j attends to keys 0..j, softmax over them (fp64, scale 1/sqrt(d)).  For
 * every later query j > i the group's weight of key i is the max over the G
 * heads of a_{j,i}; the importance is the mean over those N-1-i queries
 * (the query's own weight a_{i,i} is excluded: the count of token i is the
 * number of tokens after it), rounded to fp32 once; the last token (no later
 * query) gets 0.  q: [total, H*G, d] fp16, k: [total, H, d] fp16, scores:
 * [H, total] fp32. */
/* tail > 0: only the last `tail` tokens of each request get a value (the
 * sampled outputs of a long prompt: they need only the queries after them);
 * the other scores are left as they are. */
static int importance_causal_impl(const orc_cfg* c, int32_t batch, const int64_t* cu,
                                  const uint16_t* q, const uint16_t* k, int64_t tail, float* scores) {
  if (!cfg_valid(c) || !cu_valid(batch, cu) || tail < 0) return ORC_E_INVALID;
  int32_t H = c->num_kv_heads, G = c->gqa_group, d = c->head_dim;
  int64_t total = cu[batch];
  double scale = 1.0 / sqrt((double)d);
  double qd[128];
  for (int32_t r = 0; r < batch; r++) {
    int64_t N = cu[r + 1] - cu[r];
    if (N <= 0) continue;
    int64_t first = (tail > 0 && tail < N) ? N - tail : 0; /* tokens first..N-1 get a value */
    double* acc = (double*)malloc(sizeof(double) * (size_t)N);
    double* mx = (double*)malloc(sizeof(double) * (size_t)N);
    double* x = (double*)malloc(sizeof(double) * (size_t)N);
    double* kd = (double*)malloc(sizeof(double) * (size_t)N * d);
    for (int32_t h = 0; h < H; h++) {
      for (int64_t i = 0; i < N; i++) {
        acc[i] = 0.0;
        const uint16_t* kr = k + ((cu[r] + i) * H + h) * d;
        for (int32_t e = 0; e < d; e++) kd[i * d + e] = (double)orc_f16_to_f32(kr[e]);
      }
      /* only the queries after a token count for it */
      for (int64_t j = first + 1; j < N; j++) {
        for (int64_t i = first; i < j; i++) mx[i] = 0.0;
        for (int32_t g = 0; g < G; g++) {
          const uint16_t* qr = q + ((cu[r] + j) * H * G + (int64_t)h * G + g) * d;
          for (int32_t e = 0; e < d; e++) qd[e] = (double)orc_f16_to_f32(qr[e]);
          double m = -INFINITY, z = 0.0;
          for (int64_t i = 0; i <= j; i++) {
            double a = 0.0;
            for (int32_t e = 0; e < d; e++) a += qd[e] * kd[i * d + e];
            x[i] = a * scale;
            if (x[i] > m) m = x[i];
          }
          for (int64_t i = 0; i <= j; i++) z += exp(x[i] - m);
          for (int64_t i = first; i < j; i++) {
            double p = exp(x[i] - m) / z;
            if (p > mx[i]) mx[i] = p;
          }
        }
        for (int64_t i = first; i < j; i++) acc[i] += mx[i];
      }
      for (int64_t i = first; i < N; i++) {
        int64_t cnt = N - 1 - i;
        scores[(int64_t)h * total + cu[r] + i] = cnt > 0 ? (float)(acc[i] / (double)cnt) : 0.0f;
      }
    }
    free(acc); free(mx); free(x); free(kd);
  }
  return ORC_OK;
}

int orc_importance_causal(const orc_cfg* c, int32_t batch, const int64_t* cu,
                          const uint16_t* q, const uint16_t* k, float* scores) {
  return importance_causal_impl(c, batch, cu, q, k, 0, scores);
}

int orc_importance_causal_tail(const orc_cfg* c, int32_t batch, const int64_t* cu,
                               const uint16_t* q, const uint16_t* k, int64_t tail, float* scores) {
  return importance_causal_impl(c, batch, cu, q, k, tail, scores);
}

/* Query-free importance, KeyDiff page ("方法细节", efficient variant): the
 * anchor is the mean of the unit's keys, normalized to unit length
 * (anchor_raw = 0, the method's anchor) or as they are (anchor_raw = 1, the
 * page's reported simplification); a key's eviction score is its cosine
 * similarity to the anchor, the least similar keys being the ones to keep.
 * Reading taken to feed the alpha/N classification: importance
 * w_i = 1 - cos(anchor, k_i) normalized over the unit's tokens,
 * s_i = w_i / sum_j w_j (a distribution over the tokens like the mean
 * attention, uniform 1/N when every key is parallel to the anchor); a zero
 * key or a zero anchor has cosine 0.  fp64, rounded to fp32 once.
 * k [total, H, d] fp16; scores [H, total] fp32. */
int orc_keydiff_scores(const orc_cfg* c, int32_t batch, const int64_t* cu, const uint16_t* k,
                       int32_t anchor_raw, float* scores) {
  if (!cfg_valid(c) || !cu_valid(batch, cu)) return ORC_E_INVALID;
  int32_t H = c->num_kv_heads, d = c->head_dim;
  int64_t total = cu[batch];
  double mu[128], x[128];
  for (int32_t r = 0; r < batch; r++) {
    int64_t N = cu[r + 1] - cu[r];
    if (N <= 0) continue;
    double* w = (double*)malloc(sizeof(double) * (size_t)N);
    for (int32_t h = 0; h < H; h++) {
      for (int32_t e = 0; e < d; e++) mu[e] = 0.0;
      for (int64_t i = 0; i < N; i++) {
        const uint16_t* kr = k + ((cu[r] + i) * H + h) * d;
        double nn = 0.0;
        for (int32_t e = 0; e < d; e++) {
          x[e] = (double)orc_f16_to_f32(kr[e]);
          nn += x[e] * x[e];
        }
        double inv = anchor_raw ? 1.0 : (nn > 0.0 ? 1.0 / sqrt(nn) : 0.0);
        for (int32_t e = 0; e < d; e++) mu[e] += x[e] * inv;
      }
      double mn = 0.0;
      for (int32_t e = 0; e < d; e++) {
        mu[e] /= (double)N;
        mn += mu[e] * mu[e];
      }
      mn = sqrt(mn);
      double sw = 0.0;
      for (int64_t i = 0; i < N; i++) {
        const uint16_t* kr = k + ((cu[r] + i) * H + h) * d;
        double dot = 0.0, nn = 0.0;
        for (int32_t e = 0; e < d; e++) {
          double v = (double)orc_f16_to_f32(kr[e]);
          dot += v * mu[e];
          nn += v * v;
        }
        double cs = (nn > 0.0 && mn > 0.0) ? dot / (sqrt(nn) * mn) : 0.0;
        w[i] = 1.0 - cs;
        sw += w[i];
      }
      for (int64_t i = 0; i < N; i++)
        scores[(int64_t)h * total + cu[r] + i] = (float)(sw > 0.0 ? w[i] / sw : 1.0 / (double)N);
    }
    free(w);
  }
  return ORC_OK;
}

/* Per-page key bounds (FlexiCache page, "3.2 KV页评分机制", after Quest: each
 * KV page keeps the per-dimension minimum and maximum of its keys; the
 * page's importance for a query q is the largest dot product q could have
 * with any key of the page, sum_i max(q_i kmin_i, q_i kmax_i)).
 * Here a page's keys are the dequantized keys of its retained slots (what
 * the attention reads).  bounds [num_pages][2][d] fp32: row 0 the minima,
 * row 1 the maxima, written for every live page of the batch's units
 * (other pages untouched).  With K precision levels every level's pages
 * count (level l: p_l pages of the unit's rows, its own codec and page
 * size); two levels are the high and low tiers. */
static int32_t level_tokens(const orc_cfg* c, int32_t l);
static int64_t level_entry(const orc_cfg* c, int32_t l, int32_t j);
int orc_page_bounds(const orc_cfg* c, orc_pool* p, int32_t batch, const int32_t* table,
                    const int32_t* state, float* bounds) {
  if (!cfg_valid(c) || !p || batch < 0) return ORC_E_INVALID;
  int32_t H = c->num_kv_heads, d = c->head_dim, LT = orc_table_len(c), K = num_levels(c);
  for (int64_t u = 0; u < (int64_t)batch * H; u++) {
    const int32_t* s = state + (int64_t)2 * K * u;
    const int32_t* row = table + u * LT;
    for (int32_t l = 0; l < K; l++) {
      int32_t n = s[l], np = s[K + l], T = level_tokens(c, l);
      for (int32_t j = 0; j < np; j++) {
        int32_t id = row[level_entry(c, l, j)];
        if (id < 0 || id >= p->num_pages) continue;
        float* mn = bounds + (int64_t)id * 2 * d;
        float* mx = mn + d;
        for (int32_t e = 0; e < d; e++) { mn[e] = INFINITY; mx[e] = -INFINITY; }
        int32_t nv = n - T * j < T ? n - T * j : T;
        for (int32_t t = 0; t < nv; t++) {
          uint8_t kc[128];
          uint16_t km[2];
          orc_read_level_slot(c, page_at(p, id), l, t, kc, NULL, km, NULL, NULL, NULL);
          for (int32_t e = 0; e < d; e++) {
            float x = orc_dequant(km[0], km[1], kc[e]);
            if (x < mn[e]) mn[e] = x;
            if (x > mx[e]) mx[e] = x;
          }
        }
      }
    }
  }
  return ORC_OK;
}

/* Page scores from the bounds: for every page of every unit, in table order,
 * the max over the KV head's q heads (the group's combination, as for the
 * token scores) of sum_i max(q_i kmin_i, q_i kmax_i), fp64 rounded to fp32;
 * q [batch, H*G, d] fp16; scores [batch, H, table_len] fp32, -inf at empty
 * entries and for inactive requests (seq_len <= 0). */
int orc_page_scores(const orc_cfg* c, int32_t batch, const uint16_t* q, const int32_t* table,
                    const int32_t* state, const int32_t* seq_len, const float* bounds,
                    int64_t num_pages, float* scores) {
  if (!cfg_valid(c) || batch < 0) return ORC_E_INVALID;
  int32_t H = c->num_kv_heads, G = c->gqa_group, d = c->head_dim, LT = orc_table_len(c), K = num_levels(c);
  for (int64_t u = 0; u < (int64_t)batch * H; u++) {
    int32_t b = (int32_t)(u / H), h = (int32_t)(u % H);
    const int32_t* s = state + (int64_t)2 * K * u;
    const int32_t* row = table + u * LT;
    float* out = scores + u * LT;
    for (int32_t t = 0; t < LT; t++) out[t] = -INFINITY;
    if (seq_len[b] <= 0) continue;
    for (int32_t l = 0; l < K; l++) {
      for (int32_t j = 0; j < s[K + l]; j++) {
        int64_t t = level_entry(c, l, j);
        int32_t id = row[t];
        if (id < 0 || id >= num_pages) continue;
        const float* mn = bounds + (int64_t)id * 2 * d;
        const float* mx = mn + d;
        double best = -INFINITY;
        for (int32_t g = 0; g < G; g++) {
          const uint16_t* qr = q + ((int64_t)b * H * G + (int64_t)h * G + g) * d;
          double sum = 0.0;
          for (int32_t e = 0; e < d; e++) {
            double qe = (double)orc_f16_to_f32(qr[e]);
            double x0 = qe * mn[e], x1 = qe * mx[e];
            sum += x0 > x1 ? x0 : x1;
          }
          if (sum > best) best = sum;
        }
        out[t] = (float)best;
      }
    }
  }
  return ORC_OK;
}

/* ======================================================================== */
/* More than two precision levels ("KV compression policy", extensibility
 * paragraph: the policy allows more than two quantization levels; "Memory
 * management", generation workflow: extra levels are supported by combining
 * unidirectional or bidirectional page tables).                           */
/*                                                                          */
/* Readings (the pages name the extension but do not spell it out):         */
/*  - K levels 0 (most precise) .. K-1; thresholds alpha_0 = alpha_h >=     */
/*    alpha_1 >= .. >= alpha_{K-1} = alpha_l; a token is in the first level */
/*    l < K-1 with mean * N > alpha_l, else in level K-1 if mean * N >=     */
/*    alpha_{K-1}, else pruned (K = 2: the two-tier rule).  The window is   */
/*    level 0.                                                               */
/*  - level 0 holds T_h tokens per page, the others T_l;                     */
/*  - table row r holds level 2r from the left and level 2r+1 from the       */
/*    right (a bidirectional row; with K = 3 row 1 holds level 2 alone, a   */
/*    unidirectional row); every row has the two-tier row length;            */
/*  - prompt allocation generalizes Fig 6: the conservative block of         */
/*    ceil(N/T_h) pages feeds levels 0, 2, 3 (in that order) from its left  */
/*    end and level 1 from its right end; the middle returns to the list;   */
/*    pages the block lacks come after the frees, in the order levels 0, 2, */
/*    3, then level 1 innermost first (two tiers: the extra low page);      */
/*  - generation step: t_c's level l_c; l_c = 0: the least important        */
/*    non-window level-0 token (t_c included) moves to its own class's      */
/*    level or is pruned; l_c >= 1: t_c moves to level l_c and the least    */
/*    important token of level l_c (t_c included) moves down to its class's */
/*    level or is pruned when its class is below l_c; a removal and an      */
/*    insertion in one level share the slot, otherwise the insertion        */
/*    appends (one new page at most, never a free);                        */
/*  - release: row by row, the left level's pages left to right, then the   */
/*    right level's pages right to left.                                    */
/* ======================================================================== */

static int levels_valid(const orc_cfg* c) {
  if (c->num_levels == 0 || c->num_levels == 2) return 1;
  if (c->num_levels != 3 && c->num_levels != 4) return 0;
  int32_t K = c->num_levels;
  if (!c->lo_enabled) return 0;
  if (!(bits_ok(c->hi_k_bits) && bits_ok(c->hi_v_bits) && bits_ok(c->lo_k_bits) && bits_ok(c->lo_v_bits)))
    return 0;
  for (int32_t m = 0; m < K - 2; m++) {
    if (!bits_ok(c->mid_k_bits[m]) || !bits_ok(c->mid_v_bits[m])) return 0;
    if (!(c->alpha_mid[m] >= 0.0f)) return 0;
  }
  /* thresholds descend with the level, for the shared pair and every head */
  for (int32_t h = -1; h < (c->alpha_h_head ? c->num_kv_heads : 0); h++) {
    float prev = h < 0 ? c->alpha_h : c->alpha_h_head[h];
    for (int32_t m = 0; m < K - 2; m++) {
      if (c->alpha_mid[m] > prev) return 0;
      prev = c->alpha_mid[m];
    }
    if ((h < 0 ? c->alpha_l : c->alpha_l_head[h]) > prev) return 0;
  }
  return 1;
}

int32_t orc_num_levels(const orc_cfg* c) { return cfg_valid(c) ? num_levels(c) : -1; }
int32_t orc_state_words(const orc_cfg* c) { return cfg_valid(c) ? 2 * num_levels(c) : -1; }

static int32_t level_tokens(const orc_cfg* c, int32_t l) { return l == 0 ? c->hi_page_tokens : c->lo_page_tokens; }

static void level_bits(const orc_cfg* c, int32_t l, int32_t* kb, int32_t* vb) {
  int32_t K = num_levels(c);
  if (K == 2) {
    tier_bits(c, l == 0 ? ORC_HI : ORC_LO, kb, vb);
  } else if (l == 0) {
    *kb = c->hi_k_bits;
    *vb = c->hi_v_bits;
  } else if (l == K - 1) {
    *kb = c->lo_k_bits;
    *vb = c->lo_v_bits;
  } else {
    *kb = c->mid_k_bits[l - 1];
    *vb = c->mid_v_bits[l - 1];
  }
}

static double level_alpha(const orc_cfg* c, int32_t h, int32_t l) {
  int32_t K = num_levels(c);
  if (l == 0) return alpha_hi(c, h);
  if (l == K - 1) return alpha_lo(c, h);
  return (double)c->alpha_mid[l - 1];
}

int32_t orc_level_layout(const orc_cfg* c, int32_t l, int32_t seg[7]) {
  if (num_levels(c) == 2) return orc_tier_layout(c, l == 0 ? ORC_HI : ORC_LO, seg);
  int32_t d = c->head_dim, T = level_tokens(c, l), kb, vb;
  level_bits(c, l, &kb, &vb);
  int32_t size[6] = {T * d * kb / 8, 4 * T, T * d * vb / 8, 4 * T, 4 * T, 4 * T};
  int32_t off = 0;
  for (int i = 0; i < 6; i++) {
    seg[i] = off;
    off += round16(size[i]);
  }
  seg[6] = off;
  return T;
}

/* code (tok, j) of level l: the two tiers' own layouts, else plain */
static void level_code_addr(const orc_cfg* c, int32_t l, int is_v, int32_t tok, int32_t j, int32_t* byte,
                            int32_t* shift) {
  if (num_levels(c) == 2) {
    if (is_v) orc_v_code_addr(c, l == 0 ? ORC_HI : ORC_LO, tok, j, byte, shift);
    else orc_k_code_addr(c, l == 0 ? ORC_HI : ORC_LO, tok, j, byte, shift);
    return;
  }
  int32_t seg[7], kb, vb;
  orc_level_layout(c, l, seg);
  level_bits(c, l, &kb, &vb);
  int64_t bit = ((int64_t)tok * c->head_dim + j) * (is_v ? vb : kb);
  *byte = seg[is_v ? 2 : 0] + (int32_t)(bit / 8);
  *shift = (int32_t)(bit % 8);
}

void orc_read_level_slot(const orc_cfg* c, const uint8_t* page, int32_t l, int32_t slot, uint8_t* kc,
                         uint8_t* vc, uint16_t* km, uint16_t* vm, float* score, int32_t* pos) {
  int32_t seg[7], kb, vb;
  orc_level_layout(c, l, seg);
  level_bits(c, l, &kb, &vb);
  for (int32_t j = 0; j < c->head_dim; j++) {
    int32_t byte, shift;
    if (kc) {
      level_code_addr(c, l, 0, slot, j, &byte, &shift);
      kc[j] = (uint8_t)get_field(page, byte, shift, kb);
    }
    if (vc) {
      level_code_addr(c, l, 1, slot, j, &byte, &shift);
      vc[j] = (uint8_t)get_field(page, byte, shift, vb);
    }
  }
  if (km) { km[0] = get_u16(page + seg[1] + 4 * slot); km[1] = get_u16(page + seg[1] + 4 * slot + 2); }
  if (vm) { vm[0] = get_u16(page + seg[3] + 4 * slot); vm[1] = get_u16(page + seg[3] + 4 * slot + 2); }
  if (score) *score = bits_f32(get_u32(page + seg[4] + 4 * slot));
  if (pos) *pos = (int32_t)get_u32(page + seg[5] + 4 * slot);
}

/* Quantize one token (fp32 K and V) with level l's codec into its slot. */
static void store_level_token(const orc_cfg* c, uint8_t* page, int32_t l, int32_t slot, const float* xk,
                              const float* xv, float score, int32_t pos) {
  int32_t seg[7], kb, vb;
  orc_level_layout(c, l, seg);
  level_bits(c, l, &kb, &vb);
  uint8_t kc[128], vc[128];
  uint16_t km[2], vm[2];
  orc_quantize(xk, c->head_dim, kb, &km[0], &km[1], kc);
  orc_quantize(xv, c->head_dim, vb, &vm[0], &vm[1], vc);
  for (int32_t j = 0; j < c->head_dim; j++) {
    int32_t byte, shift;
    level_code_addr(c, l, 0, slot, j, &byte, &shift);
    put_field(page, byte, shift, kb, kc[j]);
    level_code_addr(c, l, 1, slot, j, &byte, &shift);
    put_field(page, byte, shift, vb, vc[j]);
  }
  put_u16(page + seg[1] + 4 * slot, km[0]);
  put_u16(page + seg[1] + 4 * slot + 2, km[1]);
  put_u16(page + seg[3] + 4 * slot, vm[0]);
  put_u16(page + seg[3] + 4 * slot + 2, vm[1]);
  put_u32(page + seg[4] + 4 * slot, f32_bits(score));
  put_u32(page + seg[5] + 4 * slot, (uint32_t)pos);
}

/* Table entry (index within the unit's R rows) of page j of level l. */
static int64_t level_entry(const orc_cfg* c, int32_t l, int32_t j) {
  int32_t Lr = row_len(c);
  return (int64_t)(l / 2) * Lr + (l % 2 == 0 ? j : Lr - 1 - j);
}

static uint8_t* level_slot_page(orc_pool* p, const int32_t* row, const orc_cfg* c, int32_t l, int32_t slot) {
  return page_at(p, row[level_entry(c, l, slot / level_tokens(c, l))]);
}

/* Class of a value x = mean * N (or mean * i) against the levels'
 * thresholds times `scale` (1, or a count): level, or -1 pruned. */
static int32_t level_class(const orc_cfg* c, int32_t h, double x, double scale) {
  int32_t K = num_levels(c);
  if (K == 2 && !c->lo_enabled) return x >= alpha_lo(c, h) * scale ? 0 : -1; /* two tiers, low tier closed */
  for (int32_t l = 0; l < K - 1; l++)
    if (x > level_alpha(c, h, l) * scale) return l;
  return x >= level_alpha(c, h, K - 1) * scale ? K - 1 : -1;
}

/* Prompt classification: tier code K - l for level l, 0 pruned; counts
 * [batch][H][K] per level. */
int orc_levels_classify(const orc_cfg* c, int32_t batch, const int64_t* cu, const float* scores, uint8_t* tiers,
                        int32_t* counts) {
  if (!cfg_valid(c) || !cu_valid(batch, cu)) return ORC_E_INVALID;
  int32_t H = c->num_kv_heads, K = num_levels(c);
  int64_t total = cu[batch];
  for (int32_t r = 0; r < batch; r++) {
    int64_t N = cu[r + 1] - cu[r];
    for (int32_t h = 0; h < H; h++) {
      int32_t* cnt = counts + ((int64_t)r * H + h) * K;
      for (int32_t l = 0; l < K; l++) cnt[l] = 0;
      for (int64_t p = 0; p < N; p++) {
        int64_t idx = (int64_t)h * total + cu[r] + p;
        int32_t l;
        if (c->window > 0 && p >= N - c->window) {
          l = 0;
        } else {
          int64_t denom = c->prompt_rule == ORC_RULE_ALPHA_I ? p + 1 : N;
          l = level_class(c, h, (double)scores[idx] * (double)denom, 1.0);
        }
        tiers[idx] = (uint8_t)(l < 0 ? 0 : K - l);
        if (l >= 0) cnt[l]++;
      }
    }
  }
  return ORC_OK;
}

/* Which block page or extra page each of a unit's pages takes (readings
 * above).  Q order: levels 0, 2, 3 (index order), then level 1 innermost
 * first.  For every Q position: block index >= 0, or -1 - (extra number). */
static void level_block_map(const orc_cfg* c, int64_t k, const int64_t* np, int64_t* map, int64_t* freed_lo,
                            int64_t* freed_hi, int64_t* extras) {
  int32_t K = num_levels(c);
  int64_t A = 0;
  for (int32_t l = 0; l < K; l++)
    if (l != 1) A += np[l];
  int64_t p1 = np[1];
  int64_t Ain = A < k ? A : k;
  int64_t Rin = p1 < k - Ain ? p1 : k - Ain;
  int64_t e = 0;
  for (int64_t i = 0; i < A; i++) map[i] = i < Ain ? i : -1 - (e++);
  for (int64_t m = 0; m < p1; m++) map[A + m] = m < p1 - Rin ? -1 - (e++) : k - p1 + m;
  *freed_lo = Ain;
  *freed_hi = k - Rin; /* freed block pages [Ain, k - Rin) */
  *extras = e;
}

/* (level, page index) of Q position i */
static void level_q_page(const orc_cfg* c, const int64_t* np, int64_t i, int32_t* l, int64_t* j) {
  int32_t K = num_levels(c);
  for (int32_t x = 0; x < K; x++) {
    if (x == 1) continue;
    if (i < np[x]) {
      *l = x;
      *j = i;
      return;
    }
    i -= np[x];
  }
  *l = 1;
  *j = np[1] - 1 - i; /* level 1 innermost first */
}

int orc_levels_compact_prompt(const orc_cfg* c, orc_pool* p, int32_t batch, const int64_t* cu, const uint16_t* k,
                              const uint16_t* v, const float* scores, const uint8_t* tiers, int32_t* table,
                              int32_t* state) {
  if (!cfg_valid(c) || !p || !cu_valid(batch, cu)) return ORC_E_INVALID;
  if (p->page_bytes != orc_page_bytes(c)) return ORC_E_INVALID;
  int32_t H = c->num_kv_heads, d = c->head_dim, K = num_levels(c), Lr = row_len(c), LT = orc_table_len(c);
  int32_t SW = 2 * K;
  int64_t total = cu[batch], U = (int64_t)batch * H;
  int64_t* cnt = (int64_t*)calloc((size_t)(U > 0 ? U : 1) * K, sizeof(int64_t));
  for (int64_t u = 0; u < U; u++) {
    int32_t r = (int32_t)(u / H), h = (int32_t)(u % H);
    for (int64_t t = 0; t < cu[r + 1] - cu[r]; t++) {
      uint8_t ti = tiers[(int64_t)h * total + cu[r] + t];
      if (ti >= 1 && ti <= K) cnt[u * K + (K - ti)]++;
    }
  }
  /* plan: per-unit block, pages, frees, extras; validity and capacity */
  uint32_t st = 0;
  int64_t Ktot = 0, F = 0, E = 0;
  for (int64_t u = 0; u < U; u++) {
    int64_t N = cu[u / H + 1] - cu[u / H];
    if (N <= 0) continue;
    for (int32_t w = 0; w < SW; w++)
      if (state[u * SW + w]) st |= ORC_ST_BAD_STATE;
    if (N > c->max_seq_len) st |= ORC_ST_TABLE_OVERFLOW;
    int64_t np[4] = {0, 0, 0, 0}, sum_n = 0;
    for (int32_t l = 0; l < K; l++) {
      np[l] = cdiv64(cnt[u * K + l], level_tokens(c, l));
      sum_n += cnt[u * K + l];
    }
    if (sum_n > N) st |= ORC_ST_BAD_STATE;
    int64_t kk = cdiv64(N, c->hi_page_tokens);
    if (kk > Lr) st |= ORC_ST_TABLE_OVERFLOW;
    for (int32_t r = 0; r < (K + 1) / 2; r++)
      if (np[2 * r] + (2 * r + 1 < K ? np[2 * r + 1] : 0) > Lr) st |= ORC_ST_TABLE_OVERFLOW;
    int64_t flo, fhi, e;
    int64_t* map = (int64_t*)malloc(sizeof(int64_t) * (size_t)(np[0] + np[1] + np[2] + np[3] + 1));
    level_block_map(c, kk, np, map, &flo, &fhi, &e);
    free(map);
    Ktot += kk;
    F += fhi - flo;
    E += e;
  }
  int64_t free0 = (int64_t)(p->ptr[1] - p->ptr[0]);
  if (!st && (Ktot > free0 || Ktot - F + E > free0)) st |= ORC_ST_POOL_EXHAUSTED;
  if (st) {
    p->status[0] |= st;
    free(cnt);
    return ORC_OK;
  }
  /* coordination (as in the two-tier Fig 6 workflow): every unit's block in
   * unit order from the allocation pointer, placed into the table; the
   * unused block pages appended at the reclamation pointer (units in order);
   * then the extra pages, units in order, each unit's in Q order. */
  uint64_t start = p->ptr[0], end = p->ptr[1];
  int32_t* freed = (int32_t*)malloc(sizeof(int32_t) * (size_t)(F > 0 ? F : 1));
  int64_t nf = 0;
  for (int64_t u = 0; u < U; u++) {
    int64_t N = cu[u / H + 1] - cu[u / H];
    if (N <= 0) continue;
    int64_t kk = cdiv64(N, c->hi_page_tokens);
    int64_t np[4] = {0, 0, 0, 0}, flo, fhi, e;
    for (int32_t l = 0; l < K; l++) np[l] = cdiv64(cnt[u * K + l], level_tokens(c, l));
    int64_t nq = np[0] + np[1] + np[2] + np[3];
    int64_t* map = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nq + 1));
    level_block_map(c, kk, np, map, &flo, &fhi, &e);
    int32_t* row = table + u * LT;
    for (int64_t i = 0; i < nq; i++) {
      if (map[i] < 0) continue;
      int32_t l;
      int64_t j;
      level_q_page(c, np, i, &l, &j);
      row[level_entry(c, l, (int32_t)j)] = p->free_list[(start + (uint64_t)map[i]) % (uint64_t)p->num_pages];
    }
    for (int64_t i = flo; i < fhi; i++) freed[nf++] = p->free_list[(start + (uint64_t)i) % (uint64_t)p->num_pages];
    start += (uint64_t)kk;
    free(map);
  }
  for (int64_t i = 0; i < nf; i++) p->free_list[(end + (uint64_t)i) % (uint64_t)p->num_pages] = freed[i];
  end += (uint64_t)nf;
  for (int64_t u = 0; u < U; u++) {
    int64_t N = cu[u / H + 1] - cu[u / H];
    if (N <= 0) continue;
    int64_t np[4] = {0, 0, 0, 0}, flo, fhi, e;
    for (int32_t l = 0; l < K; l++) np[l] = cdiv64(cnt[u * K + l], level_tokens(c, l));
    int64_t nq = np[0] + np[1] + np[2] + np[3];
    int64_t* map = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nq + 1));
    level_block_map(c, cdiv64(N, c->hi_page_tokens), np, map, &flo, &fhi, &e);
    int32_t* row = table + u * LT;
    for (int64_t i = 0; i < nq; i++) {
      if (map[i] >= 0) continue;
      int32_t l;
      int64_t j;
      level_q_page(c, np, i, &l, &j);
      row[level_entry(c, l, (int32_t)j)] = p->free_list[(start + (uint64_t)(-1 - map[i])) % (uint64_t)p->num_pages];
    }
    start += (uint64_t)e;
    free(map);
    for (int32_t l = 0; l < K; l++) {
      state[u * SW + l] = (int32_t)cnt[u * K + l];
      state[u * SW + K + l] = (int32_t)np[l];
    }
  }
  p->ptr[0] = start;
  p->ptr[1] = end;
  free(freed);
  /* packing: zeroed pages, tokens in position order into their level */
  float xk[128], xv[128];
  for (int64_t u = 0; u < U; u++) {
    int32_t r = (int32_t)(u / H), h = (int32_t)(u % H);
    int64_t N = cu[r + 1] - cu[r];
    if (N <= 0) continue;
    int32_t* row = table + u * LT;
    for (int32_t l = 0; l < K; l++)
      for (int32_t j = 0; j < state[u * SW + K + l]; j++)
        memset(page_at(p, row[level_entry(c, l, j)]), 0, (size_t)p->page_bytes);
    int32_t next[4] = {0, 0, 0, 0};
    for (int64_t t = 0; t < N; t++) {
      int64_t idx = (int64_t)h * total + cu[r] + t;
      uint8_t ti = tiers[idx];
      if (ti < 1 || ti > K) continue;
      int32_t l = K - ti, s = next[l]++;
      const uint16_t* kr = k + ((cu[r] + t) * H + h) * d;
      const uint16_t* vr = v + ((cu[r] + t) * H + h) * d;
      for (int32_t j = 0; j < d; j++) {
        xk[j] = orc_f16_to_f32(kr[j]);
        xv[j] = orc_f16_to_f32(vr[j]);
      }
      float sum = scores[idx] * (float)(N - 1 - t);
      store_level_token(c, level_slot_page(p, row, c, l, s), l, s % level_tokens(c, l), xk, xv, sum, (int32_t)t);
    }
  }
  free(cnt);
  return ORC_OK;
}

/* One token move of a step: from (level, slot) to (level, slot). */
typedef struct {
  int32_t on, src_l, src_s, dst_l, dst_s;
} lv_move;

typedef struct {
  int32_t active;
  int32_t new_slot;         /* level-0 slot of the new token */
  lv_move mv[2];            /* mv[0] leaves level 0 (t_c or the level-0 victim); mv[1] the level-l_c victim */
  int32_t append[4];        /* tokens each level gains */
  int32_t need_level;       /* level of the new page, -1 none */
  int32_t page_id;
} lv_plan;

int orc_levels_compact_step(const orc_cfg* c, orc_pool* p, int32_t batch, const int32_t* seq_len,
                            const uint16_t* k_new, const uint16_t* v_new, int32_t* table, int32_t* state,
                            int32_t* branch) {
  if (!cfg_valid(c) || !p || batch < 0 || c->window < 2) return ORC_E_INVALID;
  if (p->page_bytes != orc_page_bytes(c)) return ORC_E_INVALID;
  int32_t H = c->num_kv_heads, d = c->head_dim, K = num_levels(c), W = c->window, LT = orc_table_len(c);
  int32_t SW = 2 * K, Lr = row_len(c);
  int64_t U = (int64_t)batch * H;
  lv_plan* pl = (lv_plan*)calloc((size_t)(U > 0 ? U : 1), sizeof(lv_plan));
  if (branch)
    for (int64_t u = 0; u < U; u++) branch[u] = -1;
  uint32_t st = 0;
  int64_t demand = 0;
  for (int64_t u = 0; u < U; u++) {
    lv_plan* P = &pl[u];
    P->need_level = -1;
    int64_t N = seq_len[u / H];
    if (N <= 0) continue;
    P->active = 1;
    const int32_t* s = state + u * SW;
    const int32_t* row = table + u * LT;
    if (N + 1 > c->max_seq_len) { st |= ORC_ST_TABLE_OVERFLOW; continue; }
    int bad = 0;
    int64_t sum_n = 0;
    for (int32_t l = 0; l < K; l++) {
      if (s[l] < 0 || s[K + l] != cdiv64(s[l], level_tokens(c, l))) bad = 1;
      sum_n += s[l];
    }
    for (int32_t r = 0; r < (K + 1) / 2; r++)
      if (s[K + 2 * r] + (2 * r + 1 < K ? s[K + 2 * r + 1] : 0) > Lr) bad = 1;
    if (sum_n > N) bad = 1;
    if (!bad)
      for (int32_t l = 0; l < K; l++)
        for (int32_t j = 0; j < s[K + l]; j++) {
          int32_t id = row[level_entry(c, l, j)];
          if (id < 0 || id >= p->num_pages) bad = 1;
        }
    if (bad) { st |= ORC_ST_BAD_STATE; continue; }
    int64_t Np = N + 1, tc_pos = N - W;
    int32_t hh = (int32_t)(u % H);
    P->new_slot = s[0];
    P->append[0] = 1;
    int32_t br_tc = 15, br_v = 15;
    if (tc_pos >= 0) {
      int32_t tc = -1;
      float tc_sum = 0;
      for (int32_t x = 0; x < s[0]; x++) {
        float sc; int32_t pos;
        orc_read_level_slot(c, level_slot_page(p, row, c, 0, x), 0, x % level_tokens(c, 0), 0, 0, 0, 0, &sc, &pos);
        if (pos == tc_pos) { tc = x; tc_sum = sc; }
      }
      if (tc < 0) { st |= ORC_ST_BAD_STATE; continue; }
      int32_t lc = level_class(c, hh, (double)tc_sum * (double)Np, (double)(W - 1));
      br_tc = lc < 0 ? 14 : lc;
      if (lc == 0) {
        /* the least important non-window level-0 token (t_c included) */
        int32_t v = -1; float vs = 0; int32_t vp = 0; int64_t vcn = 0;
        for (int32_t x = 0; x < s[0]; x++) {
          float sc; int32_t pos;
          orc_read_level_slot(c, level_slot_page(p, row, c, 0, x), 0, x % level_tokens(c, 0), 0, 0, 0, 0, &sc, &pos);
          if (pos > tc_pos) continue;
          int64_t cn = N - 1 - pos;
          if (v < 0 || less_important(sc, cn, pos, vs, vcn, vp)) { v = x; vs = sc; vp = pos; vcn = cn; }
        }
        int32_t lv = level_class(c, hh, (double)vs * (double)Np, (double)vcn);
        br_v = lv < 0 ? 14 : lv;
        if (lv != 0) {
          P->new_slot = v;
          P->append[0] = 0;
          if (lv > 0) {
            P->mv[0] = (lv_move){1, 0, v, lv, s[lv]};
            P->append[lv] = 1;
          }
        }
      } else if (lc > 0) {
        /* t_c leaves level 0; the least important of level l_c and t_c */
        P->new_slot = tc;
        P->append[0] = 0;
        int32_t v = -1; float vs = tc_sum; int32_t vp = (int32_t)tc_pos; int64_t vcn = W - 1;
        for (int32_t x = 0; x < s[lc]; x++) {
          float sc; int32_t pos;
          orc_read_level_slot(c, level_slot_page(p, row, c, lc, x), lc, x % level_tokens(c, lc), 0, 0, 0, 0, &sc,
                              &pos);
          int64_t cn = N - 1 - pos;
          if (less_important(sc, cn, pos, vs, vcn, vp)) { v = x; vs = sc; vp = pos; vcn = cn; }
        }
        int32_t lv = v >= 0 ? level_class(c, hh, (double)vs * (double)Np, (double)vcn) : lc;
        br_v = v < 0 ? 15 : (lv < 0 ? 14 : lv);
        if (v >= 0 && lv != lc) {
          /* the victim moves down (or is pruned); t_c takes its slot */
          P->mv[0] = (lv_move){1, 0, tc, lc, v};
          if (lv > 0) {
            P->mv[1] = (lv_move){1, lc, v, lv, s[lv]};
            P->append[lv] = 1;
          }
        } else {
          P->mv[0] = (lv_move){1, 0, tc, lc, s[lc]};
          P->append[lc] = 1;
        }
      } else {
        P->new_slot = tc;
        P->append[0] = 0;
      }
    }
    for (int32_t l = 0; l < K; l++)
      if (P->append[l] && s[l] % level_tokens(c, l) == 0) P->need_level = l;
    if (branch) branch[u] = br_tc | (br_v << 4) | ((P->need_level + 1) << 8);
    if (P->need_level >= 0) {
      int32_t l = P->need_level, r = l / 2;
      if (s[K + 2 * r] + (2 * r + 1 < K ? s[K + 2 * r + 1] : 0) + 1 > Lr) { st |= ORC_ST_TABLE_OVERFLOW; continue; }
      demand++;
    }
  }
  if (!st && demand > (int64_t)(p->ptr[1] - p->ptr[0])) st |= ORC_ST_POOL_EXHAUSTED;
  if (st) {
    p->status[0] |= st;
    free(pl);
    return ORC_OK;
  }
  uint64_t start = p->ptr[0];
  for (int64_t u = 0; u < U; u++)
    if (pl[u].active && pl[u].need_level >= 0) pl[u].page_id = p->free_list[(start++) % (uint64_t)p->num_pages];
  p->ptr[0] = start;
  /* commit: the new page, the moves (sources read before any write), the new token */
  float xk[128], xv[128];
  for (int64_t u = 0; u < U; u++) {
    lv_plan* P = &pl[u];
    if (!P->active) continue;
    int32_t b = (int32_t)(u / H);
    int32_t* row = table + u * LT;
    int32_t* s = state + u * SW;
    if (P->need_level >= 0) {
      int32_t l = P->need_level;
      row[level_entry(c, l, s[K + l])] = P->page_id;
      s[K + l]++;
      memset(page_at(p, P->page_id), 0, (size_t)p->page_bytes);
    }
    float mk[2][128], mvv[2][128], msc[2];
    int32_t mpos[2];
    for (int m = 0; m < 2; m++) {
      if (!P->mv[m].on) continue;
      uint8_t kc[128], vc[128];
      uint16_t km[2], vm[2];
      int32_t l = P->mv[m].src_l, x = P->mv[m].src_s;
      orc_read_level_slot(c, level_slot_page(p, row, c, l, x), l, x % level_tokens(c, l), kc, vc, km, vm, &msc[m],
                          &mpos[m]);
      for (int32_t j = 0; j < d; j++) {
        mk[m][j] = orc_dequant(km[0], km[1], kc[j]);
        mvv[m][j] = orc_dequant(vm[0], vm[1], vc[j]);
      }
    }
    for (int m = 0; m < 2; m++) {
      if (!P->mv[m].on) continue;
      int32_t l = P->mv[m].dst_l, x = P->mv[m].dst_s;
      store_level_token(c, level_slot_page(p, row, c, l, x), l, x % level_tokens(c, l), mk[m], mvv[m], msc[m],
                        mpos[m]);
    }
    for (int32_t l = 1; l < K; l++) s[l] += P->append[l];
    const uint16_t* kr = k_new + ((int64_t)b * H + (u % H)) * d;
    const uint16_t* vr = v_new + ((int64_t)b * H + (u % H)) * d;
    for (int32_t j = 0; j < d; j++) {
      xk[j] = orc_f16_to_f32(kr[j]);
      xv[j] = orc_f16_to_f32(vr[j]);
    }
    store_level_token(c, level_slot_page(p, row, c, 0, P->new_slot), 0, P->new_slot % level_tokens(c, 0), xk, xv,
                      0.0f, seq_len[b]);
    s[0] += P->append[0];
  }
  free(pl);
  return ORC_OK;
}

int orc_levels_release(const orc_cfg* c, orc_pool* p, int32_t batch, const uint8_t* mask, int32_t* table,
                       int32_t* state) {
  if (!cfg_valid(c) || !p || batch < 0) return ORC_E_INVALID;
  int32_t H = c->num_kv_heads, K = num_levels(c), SW = 2 * K, Lr = row_len(c), LT = orc_table_len(c);
  int64_t U = (int64_t)batch * H, total = 0;
  uint32_t st = 0;
  for (int64_t u = 0; u < U; u++) {
    if (!mask[u / H]) continue;
    const int32_t* s = state + u * SW;
    const int32_t* row = table + u * LT;
    for (int32_t r = 0; r < (K + 1) / 2; r++) {
      int32_t a = s[K + 2 * r], bb = 2 * r + 1 < K ? s[K + 2 * r + 1] : 0;
      if (a < 0 || bb < 0 || a + bb > Lr) { st |= ORC_ST_BAD_STATE; break; }
    }
    if (st) continue;
    for (int32_t l = 0; l < K; l++)
      for (int32_t j = 0; j < s[K + l]; j++) {
        int32_t id = row[level_entry(c, l, j)];
        if (id < 0 || id >= p->num_pages) st |= ORC_ST_BAD_STATE;
      }
    for (int32_t l = 0; l < K; l++) total += s[K + l];
  }
  if (!st && (int64_t)(p->ptr[1] - p->ptr[0]) + total > p->num_pages) st |= ORC_ST_BAD_STATE;
  if (st) {
    p->status[0] |= st;
    return ORC_OK;
  }
  uint64_t end = p->ptr[1];
  for (int64_t u = 0; u < U; u++) {
    if (!mask[u / H]) continue;
    int32_t* row = table + u * LT;
    int32_t* s = state + u * SW;
    for (int32_t l = 0; l < K; l++) /* levels in order: left levels left to right, right levels right to left */
      for (int32_t j = 0; j < s[K + l]; j++) p->free_list[(end++) % (uint64_t)p->num_pages] = row[level_entry(c, l, j)];
    for (int32_t j = 0; j < LT; j++) row[j] = -1;
    for (int32_t w = 0; w < SW; w++) s[w] = 0;
  }
  p->ptr[1] = end;
  return ORC_OK;
}

int orc_levels_decode_attn(const orc_cfg* c, orc_pool* p, int32_t batch, const uint16_t* q, const int32_t* table,
                           const int32_t* state, const int32_t* seq_len, float* out, int32_t update_scores) {
  if (!cfg_valid(c) || !p || batch < 0) return ORC_E_INVALID;
  if (p->page_bytes != orc_page_bytes(c)) return ORC_E_INVALID;
  int32_t H = c->num_kv_heads, G = c->gqa_group, d = c->head_dim, K = num_levels(c), SW = 2 * K;
  int32_t Lr = row_len(c), LT = orc_table_len(c);
  memset(out, 0, sizeof(float) * (size_t)batch * H * G * d);
  uint32_t st = 0;
  for (int64_t u = 0; u < (int64_t)batch * H; u++) {
    int32_t b = (int32_t)(u / H), h = (int32_t)(u % H);
    if (seq_len[b] <= 0) continue;
    const int32_t* s = state + u * SW;
    const int32_t* row = table + u * LT;
    int bad = 0;
    int32_t n = 0;
    for (int32_t l = 0; l < K; l++) {
      if (s[l] < 0 || s[K + l] != cdiv64(s[l], level_tokens(c, l))) bad = 1;
      n += s[l];
    }
    for (int32_t r = 0; r < (K + 1) / 2; r++)
      if (s[K + 2 * r] + (2 * r + 1 < K ? s[K + 2 * r + 1] : 0) > Lr) bad = 1;
    if (!bad)
      for (int32_t l = 0; l < K; l++)
        for (int32_t j = 0; j < s[K + l]; j++) {
          int32_t id = row[level_entry(c, l, j)];
          if (id < 0 || id >= p->num_pages) bad = 1;
        }
    if (bad) { st |= ORC_ST_BAD_STATE; continue; }
    if (n == 0) continue;
    double* kh = (double*)malloc(sizeof(double) * (size_t)n * d);
    double* vh = (double*)malloc(sizeof(double) * (size_t)n * d);
    int32_t* lev = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t* slot = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    double* pmax = (double*)calloc((size_t)n, sizeof(double));
    double* x = (double*)malloc(sizeof(double) * (size_t)n);
    int32_t t = 0;
    for (int32_t l = 0; l < K; l++)
      for (int32_t sl = 0; sl < s[l]; sl++, t++) {
        uint8_t kc[128], vc[128];
        uint16_t km[2], vm[2];
        float sc;
        orc_read_level_slot(c, level_slot_page(p, row, c, l, sl), l, sl % level_tokens(c, l), kc, vc, km, vm, &sc,
                            &pos[t]);
        lev[t] = l;
        slot[t] = sl;
        for (int32_t i = 0; i < d; i++) {
          kh[(int64_t)t * d + i] = (double)orc_dequant(km[0], km[1], kc[i]);
          vh[(int64_t)t * d + i] = (double)orc_dequant(vm[0], vm[1], vc[i]);
        }
      }
    double scale = 1.0 / sqrt((double)d);
    for (int32_t g = 0; g < G; g++) {
      int32_t jh = h * G + g;
      const uint16_t* qr = q + ((int64_t)b * H * G + jh) * d;
      double qd[128];
      for (int32_t i = 0; i < d; i++) qd[i] = (double)orc_f16_to_f32(qr[i]);
      double m = -INFINITY, z = 0.0;
      for (int32_t a = 0; a < n; a++) {
        double acc = 0.0;
        for (int32_t i = 0; i < d; i++) acc += qd[i] * kh[(int64_t)a * d + i];
        x[a] = acc * scale;
        if (x[a] > m) m = x[a];
      }
      for (int32_t a = 0; a < n; a++) z += exp(x[a] - m);
      float* o = out + ((int64_t)b * H * G + jh) * d;
      for (int32_t i = 0; i < d; i++) {
        double acc = 0.0;
        for (int32_t a = 0; a < n; a++) acc += exp(x[a] - m) / z * vh[(int64_t)a * d + i];
        o[i] = (float)acc;
      }
      for (int32_t a = 0; a < n; a++) {
        double pr = exp(x[a] - m) / z;
        if (pr > pmax[a]) pmax[a] = pr;
      }
    }
    if (update_scores) {
      for (int32_t a = 0; a < n; a++) {
        if (pos[a] >= seq_len[b]) continue;
        int32_t seg[7];
        orc_level_layout(c, lev[a], seg);
        uint8_t* sp = level_slot_page(p, row, c, lev[a], slot[a]) + seg[4] + 4 * (slot[a] % level_tokens(c, lev[a]));
        put_u32(sp, f32_bits((float)((double)bits_f32(get_u32(sp)) + pmax[a])));
      }
    }
    free(kh); free(vh); free(lev); free(slot); free(pos); free(pmax); free(x);
  }
  p->status[0] |= st;
  return ORC_OK;
}
