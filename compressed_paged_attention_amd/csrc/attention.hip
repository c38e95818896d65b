// attention.hip -- paged decode attention over the compacted cache, and the
// score update that feeds the next generation step.
//
// What is computed (DiffKV notes, "Background": softmax(q.k/sqrt(d))
// weighting v; GQA: the q heads of a group share a KV head; "Implementation":
// a custom kernel over the compressed cache walks high-precision pages before
// low-precision ones and splits long sequences into segments merged at the
// end): for every request and q head j, the softmax over the unit's retained
// tokens of q_j . k^ / sqrt(d) weighting v^, with k^ = s_k c + z_k and
// v^ = s_v c + z_v dequantized per token on the fly.
//
// MI355X mapping.  One workgroup = (unit, split) with 8 waves; wave w takes
// the split's pages w, w+8, ... and keeps the next page's loads in flight
// while it computes the current one.  The first page's loads are issued
// before anything else; page ids are checked as they are used (a load never
// leaves the pool; a bad id zeroes the unit's output).  Per page a wave uses 16x16x16 fp16
// matrix instructions:
//   S (16 tokens x 16 heads)   = codes_K (16 x d) * Q^T (d x 16)
//   O^T (16 dims x 16 heads)  += codes_V^T (16 x 16 tokens) * P'^T (16 x 16)
// with P' = softmax weight * s_v.  The dequantization is algebraic:
//   q . k^ = s_k (q . c_k) + z_k sum(q)
//   sum_t p_t v^_t = sum_t (p_t s_v,t) c_t + (sum_t p_t z_v,t) * 1
// so only codes enter the matrix units, as exact fp16 values (8-bit codes as
// subnormals c 2^-24, 4- and 2-bit codes as 1 + c/2^b; the offsets are
// removed in fp32 with sum(q) and sum(p s_v), see block_logits/block_pv).  P' is
// split into an fp16 head and an fp16 tail (with 2G <= 16 the tail rides in
// columns G..2G-1 of the same instruction) so the PV product keeps ~22 bits.
// The S accumulator layout equals the
// P'^T operand layout, so softmax needs no data movement between the two
// products.  K codes are
// read token-major (lane: token l%16, a quarter of d); V codes are stored in
// 64 lane chunks so each lane issues one 16-byte load per page.  The online
// softmax is fp32 in base 2.  The waves are merged in LDS by a fixed-order
// tree (deterministic).  With one split per unit the same workgroup then runs
// the score update over the unit's saved logits; with several splits the
// partials go through a merge kernel.  No device-scope fence is used: on a
// multi-XCD part those write back and invalidate whole L2 caches.
#include <atomic>
#include <type_traits>

#include "dkv_common.hpp"
#include "dkv_launch.hpp"
#include "dkv_step.hpp"

namespace dkv {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;              // waves per attention workgroup
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float4_t mfma16(half4_t a, half4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ inline float4_t mfma32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline half4_t cat(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(half4_t, (uint64_t)a | ((uint64_t)b << 32));
}
// 8-bit codes enter as fp16 subnormals: the 16-bit pattern c is the value
// c 2^-24 (exact; measured on the matrix unit to keep fp32-level accuracy for
// codes of this size), so unpacking 4 codes of a dword is two byte permutes
// with zero bytes (selector 0x0C gives 0x00); the 2^24 is folded into the
// logit scale.
__device__ inline half4_t u8x4(uint32_t w) {
  return cat(__builtin_amdgcn_perm(0u, w, 0x0C010C00u), __builtin_amdgcn_perm(0u, w, 0x0C030C02u));
}
// two fp32 values to a packed fp16 pair, rounded toward zero (one instruction)
__device__ inline half2_t pkrtz(float a, float b) {
  return __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ inline half8_t cat8(half4_t a, half4_t b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
constexpr float kTwo24 = 16777216.0f;
// 4- and 2-bit codes enter as the normal fp16 values 1 + c/16 and 1 + c/4:
// the code goes to the top of the mantissa under the exponent of 1.0 (as
// subnormals these small codes lose precision in the matrix unit).  The
// fields at bits s and s+16 of a dword give a packed fp16 pair: one shift
// and one v_and_or_b32.  (The mask and the exponent bits are kept in a
// scalar and a vector register: with both as literals the compiler emits an
// and and an or, since a three-operand instruction takes no literal here.)
template <uint32_t V>
__device__ inline uint32_t sreg_const() {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(V));
  return r;
}
template <uint32_t V>
__device__ inline uint32_t vreg_const() {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(V));
  return r;
}
__device__ inline uint32_t nib2(uint32_t w, int s) {
  const uint32_t t = s >= 6 ? w >> (s - 6) : w << (6 - s);
  return (t & sreg_const<0x03C003C0u>()) | vreg_const<0x3C003C00u>();
}
__device__ inline uint32_t crumb2(uint32_t w, int s) {
  const uint32_t t = s >= 8 ? w >> (s - 8) : w << (8 - s);
  return (t & sreg_const<0x03000300u>()) | vreg_const<0x3C003C00u>();
}

// Splits per unit (grid width) when there are fewer units than compute
// units: at least one 8-wave workgroup per compute unit, and enough that a
// unit holding a whole row of pages spreads over workgroups of about
// kSplitPages pages.  A unit takes pages in chunks of
// max(ceil(pages / S), kSplitMinPages), so small units use few of the S
// workgroups and large ones all of them (retention differs widely between
// heads); the rest exit at once.
constexpr int kSplitPages = 256;
constexpr int kMaxSplits = 128;  // the merge kernel holds one weight per split and head in LDS

int attn_splits(const Cfg& c, int batch) {
  const int64_t U = (int64_t)batch * c.H;
  if (U <= 0 || U >= 256) return 1;
  int64_t S = (256 + U - 1) / U;
  const int64_t byrow = (c.L + kSplitPages - 1) / kSplitPages;
  if (S < byrow) S = byrow;
  int64_t cap = c.L / 16;
  if (cap < 1) cap = 1;
  if (S > cap) S = cap;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  return (int)S;
}


// Score-update chunks (several splits, or a deferred update): 64 pages each.
constexpr int kScorePages = 64;
constexpr int kCandWords = 8;  // per chunk: least important high / low candidate, t_c

struct AttnWs {
  float* part;    // [U][S][G][D + 2] split partials (unnormalized O, max, sum)
  float* ml;      // [U][G][2] final (max, sum) in base 2, for the score update
  float* logits;  // [U][L][32][logit_stride(G)] base-2 logits of every retained slot
  int32_t* cand;  // [U][ceil(L/kScorePages)][8] score-update candidates per chunk, for the next step's plan
  int32_t* order; // [U] dispatch order: units by descending page count (more units than compute units)
};

// Logits of one slot in the workspace: G of them, padded to a power of two
// (4, 8 or 16 floats: one slot is one or more aligned 16-byte loads).
__host__ __device__ constexpr int logit_stride(int G) { return G <= 4 ? 4 : (G <= 8 ? 8 : 16); }

static AttnWs attn_carve(const Cfg& c, int batch, bool scores, void* ws, size_t* bytes) {
  const int64_t U = (int64_t)batch * c.H;
  const int S = attn_splits(c, batch);
  uint8_t* b = (uint8_t*)ws;
  size_t off = 0;
  AttnWs w;
  w.part = (float*)(b + off);
  if (S > 1) off = align_up(off + (size_t)U * S * c.G * (c.d + 2) * sizeof(float), 256);
  w.ml = (float*)(b + off);
  off = align_up(off + (size_t)U * c.G * 2 * sizeof(float), 256);
  w.logits = (float*)(b + off);
  if (scores) off = align_up(off + (size_t)U * c.L * 32 * logit_stride(c.G) * sizeof(float), 256);
  w.cand = (int32_t*)(b + off);
  if (scores)
    off = align_up(off + (size_t)U * ((c.L + kScorePages - 1) / kScorePages) * kCandWords * sizeof(int32_t), 256);
  w.order = (int32_t*)(b + off);
  off = align_up(off + (size_t)U * sizeof(int32_t), 256);
  if (bytes) *bytes = off < 256 ? 256 : off;
  return w;
}

size_t attn_workspace(const Cfg& c, int batch, bool scores) {
  if (c.plain) return plain_attn_workspace(c, batch, scores);
  size_t n = 0;
  attn_carve(c, batch, scores, nullptr, &n);
  return n;
}

__device__ inline bool state_ok(int nh, int nl, int ph, int pl, int L) {
  return nh >= 0 && nl >= 0 && ph == (int)cdiv(nh, kHiTokens) && pl == (int)cdiv(nl, kLoTokens) && ph + pl <= L;
}

// Validates every page id of the unit (same answer in every workgroup of the
// unit; the row is then cache-resident for the page loop's scalar loads).
__device__ inline bool unit_ids(int ph, int pl, int L, int64_t P, const int32_t* row) {
  int bad = 0;
  for (int j = threadIdx.x; j < ph + pl; j += blockDim.x) {
    const int32_t id = j < ph ? row[j] : row[L - 1 - (j - ph)];
    bad |= (id < 0 || id >= P);
  }
  return __syncthreads_or(bad) == 0;
}

// Registers of one page for one lane.  A page is read with the same loads
// whatever its tier (tier offsets are scalar selects, not branches), so the
// compiler keeps the following pages' loads in flight during a compute.
// E = the lane's tokens per 16-token block in the softmax layout (below).
template <int D, int E>
struct PageRegs {
  static constexpr int KW = D / 32;  // dwords per K load
  uint32_t k[2 * KW];  // high: 2*KW dwords of token i; low: KW of token i, KW of i+16
  uint32_t km[2 * E];  // K (scale, zero) words of the lane's softmax tokens (low: both blocks)
  uint32_t vm[2 * E];  // V (scale, zero) words
  uint32_t v[KW];      // the lane's V chunk
  uint32_t sp;         // fused score update: lane < 32 score slot lane, else position slot lane - 32
  int32_t id;          // page id (wave-uniform)
};

// Page words are read once per launch: non-temporal loads (measured: the
// plain attention 4 % faster; they keep the caches for the rest)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <int N>
__device__ inline void ldw(uint32_t* r, const uint8_t* p) {
  if constexpr (N == 4) {
    const u32x4_t a = __builtin_nontemporal_load((const u32x4_t*)p);
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  } else if constexpr (N == 2) {
    const u32x2_t a = __builtin_nontemporal_load((const u32x2_t*)p);
    r[0] = a[0]; r[1] = a[1];
  } else {
    r[0] = __builtin_nontemporal_load((const uint32_t*)p);
  }
}

// kb: lane K offset of the high tier (token i, dims qg*D/4); the low tier's
// is kb/2 (token i) and kb/2 + 16*D/2 (token i + 16).  mt = 4 x the lane's
// first softmax token, vl = lane chunk offset.  Metadata segments start at
// the same offset in both tiers.
template <int D, int E>
__device__ inline void load_page(PageRegs<D, E>& R, const uint8_t* pg, bool lo, int kb, int mt, int vl) {
  constexpr int KW = PageRegs<D, E>::KW;
  constexpr Seg sh = tier_seg(D, true), sl = tier_seg(D, false);
  static_assert(sh.km == sl.km, "K metadata offsets differ between tiers");
  const int k0 = lo ? (kb >> 1) : kb;
  const int k1 = lo ? (kb >> 1) + 16 * (D / 2) : kb + 4 * KW;
  ldw<KW>(R.k, pg + k0);
  ldw<KW>(R.k + KW, pg + k1);
  ldw<E>(R.km, pg + sh.km + mt);
  ldw<E>(R.km + E, pg + sh.km + mt + (lo ? 64 : 0));
  const int vm = lo ? sl.vm : sh.vm;
  ldw<E>(R.vm, pg + vm + mt);
  ldw<E>(R.vm + E, pg + vm + mt + (lo ? 64 : 0));
  ldw<KW>(R.v, pg + (lo ? sl.vc : sh.vc) + vl);
}

// Score and position words of the page's 32 slots (high pages: slots 16..31
// are other in-page bytes, never used).
template <int D, int E>
__device__ inline void load_page_sp(PageRegs<D, E>& R, const uint8_t* pg, bool lo, int lane) {
  constexpr Seg sh = tier_seg(D, true), sl = tier_seg(D, false);
  const int off = lane < 32 ? (lo ? sl.sc : sh.sc) + 4 * lane : (lo ? sl.ps : sh.ps) + 4 * (lane - 32);
  R.sp = __builtin_nontemporal_load((const uint32_t*)(pg + off));
}

struct Softmax {
  float m, lsum, zsum;  // reference (base 2), sum of weights, sum of weight * z_v
};

// max over the lanes i, i+16, i+32, i+48 (the four token rows of a head):
// two lane swaps (rows 0<->1, 2<->3, then halves), no LDS round trip
__device__ inline float rows_max(float v) {
  uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  u = __float_as_uint(v);
  auto c = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ inline float rows_sum(float v) {
  uint32_t u = __float_as_uint(v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  u = __float_as_uint(v);
  auto c = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// The softmax layout.  The QK product leaves lane (i, qg) the logits of
// tokens 4qg .. 4qg+3 of column i; with G <= 8 most of the 16 columns repeat
// or carry nothing, so the per-element work (logit, weight, sums) would run
// on 4 values per lane of which G/16 matter.  With GP = G rounded up to a
// power of two (4, 8 or 16) and E = GP / 4, lane (i, qg) instead takes E
// elements: head i & (GP-1), tokens 4qg + E (i / GP) + e.  The moves are DPP
// row shifts restricted to the banks (groups of 4 lanes of a row) that
// receive (`bank` mask); the weights go back to the matrix operand layout
// (head columns 0..GP-1, their fp16 tails in columns GP..2GP-1) the same way.
// E = 4 is the identity.
constexpr int kRowShl = 0x100, kRowShr = 0x110;
template <int CTRL, int BANK>
__device__ inline float dpp_mov(float old, float src) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, 0xF, BANK, false));
}
// lane i of a row takes element e from register E (i / GP) + e of lane i & (GP-1)
template <int E>
__device__ inline void spread(const float4_t& s, float* v) {
  if constexpr (E == 4) {
#pragma unroll
    for (int r = 0; r < 4; r++) v[r] = s[r];
  } else if constexpr (E == 2) {
    v[0] = dpp_mov<kRowShr + 8, 0xC>(s[0], s[2]);
    v[1] = dpp_mov<kRowShr + 8, 0xC>(s[1], s[3]);
  } else {
    float t = dpp_mov<kRowShr + 4, 0x2>(s[0], s[1]);
    t = dpp_mov<kRowShr + 8, 0x4>(t, s[2]);
    v[0] = dpp_mov<kRowShr + 12, 0x8>(t, s[3]);
  }
}
// back to the operand layout: lane i (head column i < GP, or the tail column
// of head i - GP) takes token r of its head from lane (i & (GP-1)) + GP (r / E),
// element r % E (lanes of columns >= 2GP keep finite values of their own)
template <int E>
__device__ inline void gather(const float* pp, float* g) {
  if constexpr (E == 4) {
#pragma unroll
    for (int r = 0; r < 4; r++) g[r] = pp[r];
  } else if constexpr (E == 2) {
    g[0] = dpp_mov<kRowShr + 8, 0xC>(pp[0], pp[0]);
    g[1] = dpp_mov<kRowShr + 8, 0xC>(pp[1], pp[1]);
    g[2] = dpp_mov<kRowShl + 8, 0x3>(pp[0], pp[0]);
    g[3] = dpp_mov<kRowShl + 8, 0x3>(pp[1], pp[1]);
  } else {
    g[0] = dpp_mov<kRowShr + 4, 0x2>(pp[0], pp[0]);
    g[1] = dpp_mov<kRowShl + 4, 0x1>(pp[0], pp[0]);
    g[2] = dpp_mov<kRowShl + 4, 0x2>(dpp_mov<kRowShl + 8, 0x1>(pp[0], pp[0]), pp[0]);
    g[3] = dpp_mov<kRowShl + 8, 0x2>(dpp_mov<kRowShl + 12, 0x1>(pp[0], pp[0]), pp[0]);
  }
}
// a per-head value over the lanes of one row that hold the same head
template <int E>
__device__ inline float heads_max(float v) {
  if constexpr (E <= 2) v = fmaxf(v, __shfl_xor(v, 8, 64));
  if constexpr (E == 1) v = fmaxf(v, __shfl_xor(v, 4, 64));
  return v;
}
template <int E>
__device__ inline float heads_sum(float v) {
  if constexpr (E <= 2) v += __shfl_xor(v, 8, 64);
  if constexpr (E == 1) v += __shfl_xor(v, 4, 64);
  return v;
}

// Reference of the online softmax.  Weights are p = 2^(x - m) for a
// reference m the wave chooses; every sum (weights, the z term, the PV
// accumulator) carries the same 2^-m, which the normalization removes, so m
// is free.  It is kept at least kHead above the largest logit seen, so
// p <= 1/4 and the fp16 operand p s_v kv stays below 4 s_v (high, kv = 16)
// or s_v (low, kv = 4): finite for the scale of any vector of fp16 values
// (range <= 131008, so s_v <= 8734 high, 43670 low).  It moves (to the page's
// head max + kHead + kLazy) only when a page breaks that bound, so the
// accumulators are rescaled rarely.  Every lane of a head holds its reference.
constexpr float kHead = 2.0f;
constexpr float kLazy = 4.0f;

// One 16-token block.  block_logits: the lane's E logits of the block
// (masked on a partial page).  `v` holds q.c'' for in-page tokens
// first..first+E-1 of the lane's head; `kmw` the K metadata words of those
// tokens.  sq2 = sum(q) scale_log2 (of that head).  K: c'' = c 2^-24 (high)
// or 1 + c/16 (low), so q.c = 2^24 s or 16 (s - sum q) and
//   x = ks (s kmul - cq2) + kz sq2,  kmul = 2^24 sl or 16 sl, cq2 = 0 or 16 sq2.
template <int E>
__device__ inline void block_logits(const float* v, const uint32_t* kmw, int first, int nval, bool partial,
                                    float sq2, float kmul, float cq2, float* x) {
#pragma unroll
  for (int e = 0; e < E; e++) {
    // log2e/sqrt(d) (s_k q.c + z_k sum(q)); both fp16 factors enter
    // mixed-precision fmas straight from the metadata word (z_k sq2 as an
    // fma with a zero addend: one instruction, no conversion)
    const _Float16 ks = __builtin_bit_cast(_Float16, (uint16_t)kmw[e]);
    const _Float16 kz = __builtin_bit_cast(_Float16, (uint16_t)(kmw[e] >> 16));
    x[e] = __builtin_fmaf((float)ks, __builtin_fmaf(v[e], kmul, -cq2), __builtin_fmaf((float)kz, sq2, 0.0f));
  }
  if (partial) {
#pragma unroll
    for (int e = 0; e < E; e++)
      if (first + e >= nval) x[e] = -INFINITY;
  }
}

// The reference check, once per page: lm is the lane's largest logit of the
// page.  A head's maximum breaks the bound exactly when one of its lanes'
// does, so the common case needs no cross-lane step (ref_breaks); when some
// head breaks it (rare), every head's reference moves to its maximum +
// kHead + kLazy if that is higher, and the sums are rescaled (ref_move).
// The accumulator columns of lane i belong to head i & (GP-1), the lane's
// own softmax head, so its reference scales them.
__device__ inline bool ref_breaks(float lm, const Softmax& sm) { return __any(lm + kHead > sm.m); }
template <int D, int E>
__device__ inline void ref_move(float lm, Softmax& sm, float4_t* acc) {
  constexpr int NB = D / 16;
  const float pm = heads_max<E>(rows_max(lm)) + kHead;
  const float mn = pm > sm.m ? pm + kLazy : sm.m;
  const float alpha = __builtin_amdgcn_exp2f(sm.m - mn);
  sm.lsum *= alpha;
  sm.zsum *= alpha;
#pragma unroll
  for (int nb = 0; nb < NB; nb++) acc[nb] *= alpha;
  sm.m = mn;
}

// block_pv: weights of the lane's E logits under the reference, their sums,
// and the PV products.  `vmw` the V metadata words of those tokens;
// `vpair(nb)` the fp16 V operand of 16-dim block nb.
// V: codes c'' = 1 + c/kv (kv = 16 high, 4 low) with operand p s_v kv, so
//   sum p s_v kv c'' = sum p s_v c + sum p s_v kv, and the z term collects
//   p (z_v - kv s_v).  The weights come as pk = p kv = 2^(x - mk) with
//   mk = m - log2 kv, so pk s_v is the operand, the sums take pk / kv and
//   the z term pk (z_v / kv - s_v).
// PACK: column GP + h carries the fp16 tail of head h's weights (one matrix
// instruction per block instead of two); tm is 1 on those lanes, else 0.
template <int D, int E, bool PACK, typename VOp>
__device__ inline void block_pv(const float* x, const uint32_t* vmw, float mk, float ikv, float tm, Softmax& sm,
                                float4_t* acc, VOp vpair) {
  constexpr int NB = D / 16;
  float pe[E];
#pragma unroll
  for (int e = 0; e < E; e++) {
    const float pk = __builtin_amdgcn_exp2f(x[e] - mk);
    const _Float16 vs = __builtin_bit_cast(_Float16, (uint16_t)vmw[e]);
    const _Float16 vz = __builtin_bit_cast(_Float16, (uint16_t)(vmw[e] >> 16));
    sm.lsum = __builtin_fmaf(pk, ikv, sm.lsum);
    sm.zsum = __builtin_fmaf(pk, __builtin_fmaf((float)vz, ikv, -(float)vs), sm.zsum);
    pe[e] = __builtin_fmaf(pk, (float)vs, 0.0f);  // a mixed-precision fma: no conversion of s_v
    asm("" : "+v"(pe[e]));
  }
  float pp[4];
  gather<E>(pe, pp);
#pragma unroll
  for (int r = 0; r < 4; r++) asm("" : "+v"(pp[r]));
  // Head and tail of each weight: the head is one conversion of the fp32
  // value (toward zero), the tail the exact remainder pp - head, converted
  // again, so head + tail = pp within 2^-21.  The head must be a single
  // value: when the compiler was free to round the exact product pk vs to
  // fp16 in one use (a mixed-precision fma) and the fp32 product in another,
  // the two heads differed by one ulp wherever the product lay within fp32
  // rounding of an fp16 midpoint, and head + tail missed the weight by that
  // ulp (measured: 7.5e-4 relative on a token holding 8 % of a sharp
  // softmax).  The empty asm keeps pp an fp32 value the conversions share.
  const half2_t h01 = pkrtz(pp[0], pp[1]);
  const half2_t h23 = pkrtz(pp[2], pp[3]);
  // PACK: the head on head lanes (tm = 0: pp itself, whose conversion is the
  // head), the tail on tail lanes (tm = 1), without a select
  const float tmv = PACK ? tm : 1.0f;
  const half2_t t01 = pkrtz(__builtin_fmaf((float)h01[0], -tmv, pp[0]), __builtin_fmaf((float)h01[1], -tmv, pp[1]));
  const half2_t t23 = pkrtz(__builtin_fmaf((float)h23[0], -tmv, pp[2]), __builtin_fmaf((float)h23[1], -tmv, pp[3]));
  const _Float16 ph16[4] = {h01[0], h01[1], h23[0], h23[1]};
  const _Float16 pl16[4] = {t01[0], t01[1], t23[0], t23[1]};
  if constexpr (PACK) {
    const half4_t bt = {pl16[0], pl16[1], pl16[2], pl16[3]};
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[nb] = mfma16(vpair(nb), bt, acc[nb]);
  } else {
    const half4_t bh = {ph16[0], ph16[1], ph16[2], ph16[3]};
    const half4_t bl = {pl16[0], pl16[1], pl16[2], pl16[3]};
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
      const half4_t a = vpair(nb);
      acc[nb] = mfma16(a, bh, acc[nb]);
      acc[nb] = mfma16(a, bl, acc[nb]);
    }
  }
}

template <int E>
__device__ inline float maxe(const float* x) {
  float m = x[0];
#pragma unroll
  for (int e = 1; e < E; e++) m = fmaxf(m, x[e]);
  return m;
}

// keep(mb, x): stores the lane's E logits of 16-token block mb of the page.
// The q.c products use the K = 32 instruction: lane (i, qg) holds 8 dims of
// token i per step, the same 8 dims of q as its Q operand.  One reference
// check per page (a low page's two blocks share it, so nothing branches
// between their weights).  ts = the lane's first softmax token in a block.
template <int D, int E, bool PACK, typename Keep>
__device__ inline void compute_page(const PageRegs<D, E>& R, bool hi, int nval, const half8_t* qop, float sq2,
                                    float sl, float tm, int ts, Softmax& sm, float4_t* acc, Keep keep) {
  constexpr int NS = D / 32, KW = PageRegs<D, E>::KW;
  if (hi) {
    // one accumulator: dependent matrix instructions of one shape issue
    // back to back (the chain costs no vector instructions)
    float4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < NS; ks++) s0 = mfma32(cat8(u8x4(R.k[2 * ks]), u8x4(R.k[2 * ks + 1])), qop[ks], s0);
    float v[E], x[E];
    spread<E>(s0, v);
    block_logits<E>(v, R.km, ts, nval, nval < kHiTokens, sq2, kTwo24 * sl, 0.0f, x);
    keep(0, x);
    auto pv = [&]() {
      block_pv<D, E, PACK>(x, R.vm, sm.m - 4.0f, 1.0f / 16.0f, tm, sm, acc, [&](int nb) {
        // block nb: pairs 2nb (tokens 0, 1) and 2nb + 1 (tokens 2, 3)
        const uint32_t w = R.v[nb >> 1];
        const int sft = 8 * (nb & 1);
        return cat(nib2(w, sft), nib2(w, sft + 4));
      });
    };
    // each outcome of the reference check has its own products, so the
    // accumulators are not copied to join the two paths
    const float lm = maxe<E>(x);
    if (ref_breaks(lm, sm)) {
      ref_move<D, E>(lm, sm, acc);
      pv();
    } else {
      pv();
    }
  } else {
    // both blocks' q.c products and logits first, then one reference check
    float x[2][E];
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
      float4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < NS; ks++) {
        // word w: dims 8w .. 8w + 7 as nibble pairs (0, 4), (1, 5), (2, 6), (3, 7)
        const uint32_t w0 = R.k[KW * mb + ks];
        s0 = mfma32(cat8(cat(nib2(w0, 0), nib2(w0, 4)), cat(nib2(w0, 8), nib2(w0, 12))), qop[ks], s0);
      }
      float v[E];
      spread<E>(s0, v);
      block_logits<E>(v, R.km + E * mb, 16 * mb + ts, nval, nval < 16 * (mb + 1), sq2, 16.0f * sl, 16.0f * sq2,
                      x[mb]);
      keep(mb, x[mb]);
    }
    auto pv = [&]() {
#pragma unroll
      for (int mb = 0; mb < 2; mb++) {
        block_pv<D, E, PACK>(x[mb], R.vm + E * mb, sm.m - 2.0f, 0.25f, tm, sm, acc, [&](int nb) {
          // block (nb, mb): pairs P = 2M, 2M + 1 with M = 2nb + mb, in word P / 8
          const int M = 2 * nb + mb;
          const int P0 = 2 * M, P1 = 2 * M + 1;
          return cat(crumb2(R.v[P0 >> 3], 2 * (P0 & 7)), crumb2(R.v[P1 >> 3], 2 * (P1 & 7)));
        });
      }
    };
    const float lm = fmaxf(maxe<E>(x[0]), maxe<E>(x[1]));
    if (ref_breaks(lm, sm)) {
      ref_move<D, E>(lm, sm, acc);
      pv();
    } else {
      pv();
    }
  }
}

// fused score update: a unit's logits, old scores, positions and page ids
// are kept in LDS when they fit in this many 32-bit words
constexpr int kLdsWords = 16384;

// MODE 0: attention; 1: attention + score update in the same workgroup (one
// split only); 2: attention keeping logits (score update later).
// Policy parameters for the next step's plan (made by the fused score update).
struct PolicyArgs {
  int W, S_max, lo_en;
  float ah, al;
  const float* ah_head;  // per-KV-head thresholds (null: ah, al)
  const float* al_head;
};
__device__ inline double pa_ah(const PolicyArgs& pa, int h) { return (double)(pa.ah_head ? pa.ah_head[h] : pa.ah); }
__device__ inline double pa_al(const PolicyArgs& pa, int h) { return (double)(pa.al_head ? pa.al_head[h] : pa.al); }

// The generation step's commit, run in front of the attention (STEP): the
// step workspace made by the plan kernel, the new tokens and the pool lists.
// The kernel reads the table and tier state through its read-only (and
// restrict) parameters and writes them only through these: the one table
// entry a step writes (a new page's) is never read back in the kernel, whose
// page loop and score pass take that id from LDS, and the tier state is read
// before the commit.
struct StepArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int64_t* hdr;
  const int32_t* rec;
  const int32_t* nf;
  const int32_t* list;
  int32_t* table;
  int32_t* state;
  uint64_t* ptr;
  int64_t U;
  int direct;  // every workgroup redoes the demand prefix sum (no coordination kernel)
  // chained: hdr/rec/nf are the slot the previous step's attention left
  // (its chain words checked by every workgroup, pointer start from it),
  // not the plan kernel's
  int chained;
  const int32_t* cw;
  // the other slot, for the next step (written with the score update; null: none)
  int64_t* hdr_n;
  int32_t* rec_n;
  int32_t* nf_n;
  int32_t* cw_n;
};

template <int D, int MODE, int GP, bool STEP>
__global__ __launch_bounds__(kThreads) void attn_kernel(int H, int G, int L, int S, int64_t P, int page_bytes,
                                                        PolicyArgs pa, float scale_log2, const uint16_t* __restrict__ q,
                                                        const int32_t* __restrict__ table,
                                                        const int32_t* __restrict__ state,
                                                        const int32_t* __restrict__ seq_len, uint8_t* pages,
                                                        float* __restrict__ out, float* __restrict__ part,
                                                        float* __restrict__ ml, float* logits, uint32_t* status,
                                                        StepArgs sa, const int32_t* __restrict__ order) {
  constexpr bool SAVE = MODE != 0;
  // GP: G rounded up to 4, 8 or 16; with GP <= 8 the heads' fp16 tails ride
  // in columns GP .. 2GP-1 of the PV product (PACK), and the softmax runs on
  // E = GP / 4 elements per lane
  constexpr bool PACK = GP <= 8;
  constexpr int E = GP / 4;
  constexpr int NB = D / 16;  // 16-dim blocks (N-blocks of PV)
  constexpr int NS = D / 32;  // 32-dim K-steps of QK
  constexpr int QD = D / 4;   // dims per lane group
  const int split = blockIdx.x;
  // a permutation of the units (clamped: a workspace overwritten between
  // chained calls cannot send a load outside the tables)
  const int64_t u = order ? min(max(order[blockIdx.y], 0), (int32_t)gridDim.y - 1) : blockIdx.y;
  const int b = (int)u / H, h = (int)u % H;  // u < 2^31: 32-bit division
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loop control
  const int i = lane & 15, qg = lane >> 4;
  const int32_t* row = table + u * L;
  // the query and the table entry of this wave's first page (a guess that
  // holds when the unit has more than wid high pages) go out first: neither
  // waits for the unit's state
  const int hs = i & (GP - 1);  // the lane's softmax head (and its columns' head)
  const int qhead = (i < 2 * GP && hs < G && (PACK || i < GP)) ? hs : -1;
  uint4 qraw[QD / 8];
  {
    const uint4* src =
        (const uint4*)(q + ((int64_t)b * H * G + (int64_t)h * G + max(qhead, 0)) * D + qg * QD);
#pragma unroll
    for (int c = 0; c < QD / 8; c++) qraw[c] = src[c];
  }
  const int32_t id_guess = row[min(wid, L - 1)];
  const int32_t* s4 = state + 4 * u;
  int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  const int N = seq_len[b];

  __shared__ float wm[kWaves][16], wl[kWaves][16], sM[16], sL[16], sI[16];
  // every wave's O columns, for the merge; before that (STEP) the commit's
  // scratch, whose two page images the page loop reads
  __shared__ float4_t buf[kWaves][16 * D / 4];
  static_assert(sizeof(buf) >= 4 * commit_lds_words<D>(), "commit scratch");
  // fused score update: [TPg*32*G] logits, [TPg*32] old scores, [TPg*32]
  // positions, [TPg] page ids
  __shared__ uint32_t lds_w[MODE == 1 ? kLdsWords : 1];

  // ---- generation step fused in front (STEP; one split per unit) ----
  // Every wave learns the step's decision for the unit (the verdict over all
  // units' demand words, the unit's plan words), hence the tier state after
  // the step.  The last wave commits, building the written pages whole in
  // LDS (over the merge buffer), while the others attend to the pages the
  // step leaves alone; it then takes a smaller share of those, and the
  // written pages from their images.
  constexpr int kCW = kWaves - 1;     // the committing wave
  static_assert(sizeof(buf) >= 2 * page_bytes_for(D), "two page images in the merge buffer");
  __shared__ int s_vd[3 * kWaves];
  __shared__ int32_t s_idt[2];        // ids of the written high and low pages
  const uint32_t* img_h = (const uint32_t*)&buf[0][0];
  const uint32_t* img_l = img_h + page_bytes_for(D) / 4;
  bool go = false;
  int jh = -1, jl = -1;               // written pages: page-loop index
  int tix_h = -1, tix_l = -1;         // ... and table index
  const int nh0 = nh, nl0 = nl, ph0 = ph, pl0 = pl;  // before the step
  int need = 0, new_hi = 0, hi_app = 0, lo_src = -1, lo_slot = 0, lo_app = 0, rank = 0;
  int32_t id_hrow = 0, id_lrow = 0, id_src = 0, id_first = 0;
  int64_t start = 0;
  // ts: the lane's first softmax token of a 16-token block (4 x it: its
  // metadata words' offset)
  const int ts = 4 * qg + E * (i / GP);
  const int kbase = i * D + qg * (D / 4), mt = 4 * ts, vl = lane * (D / 8);
  uint32_t badid = 0;
  // page ids are checked where they are used (check: the id names a page of
  // the unit); a bad id is clamped into the pool (the load stays in bounds)
  // and zeroes the unit's result
  auto fetch_id = [&](PageRegs<D, E>& R, int jj, int32_t id, bool check) {
    badid |= (uint32_t)(check && (id < 0 || id >= P));
    id = min(max(id, 0), (int32_t)(P - 1));
    R.id = id;
    const uint8_t* pg = pages + (int64_t)id * page_bytes;
    load_page<D, E>(R, pg, jj >= ph, kbase, mt, vl);
    if (MODE == 1) load_page_sp<D, E>(R, pg, jj >= ph, lane);
  };
  PageRegs<D, E> A, B;
  WaveCommit<D> wc;
  if constexpr (STEP) {
    // with at most kWaveVerdictUnits units the committing wave takes the
    // verdict alone, its loads (and the pool pointers) issued before
    // anything else; the other waves' first page loads do not wait for them
    const bool wv = sa.direct && sa.U <= kWaveVerdictUnits;
    WaveVerdict vd;
    int64_t h_start = 0, h_end = 0, p_live = 0;
    if (sa.direct) {
      h_start = sa.hdr[SH_START];
      // chained: the pool's end pointer moves only between steps; its start
      // is read live as a check (workgroup 0 may already have advanced it)
      h_end = sa.chained ? (int64_t)sa.ptr[1] : sa.hdr[SH_END];
      p_live = (int64_t)sa.ptr[0];
    }
    if (wv && wid == kCW) vd.load(sa.chained, sa.U, H, sa.nf, sa.cw, seq_len, state);
    const int32_t wu = sa.nf[u];
    const int32_t* R = sa.rec + u * kSRec;
    new_hi = R[S_NEWHI];
    hi_app = R[S_HIAPP];
    lo_src = R[S_LOSRC];
    lo_slot = R[S_LOSLOT];
    lo_app = R[S_LOAPP];
    id_hrow = R[S_IDH];
    id_lrow = R[S_IDL];
    id_src = R[S_IDS];
    id_first = R[S_IDF];
    need = wu & 3;
    // (no page load goes out before the verdict: issuing the first pages of
    // waves 0-3 speculatively made the verdict's own loads wait behind them,
    // 2 % slower steps)
    // the committing wave's loads, before the verdict (its unit asks for a
    // commit; the verdict may still refuse it)
    if (wid == kCW && (wu & kActive) && ((uint32_t)wu >> 8) == 0)
      wc.begin(u, page_bytes, P, sa.k_new, sa.v_new, need, lo_src, id_hrow, id_lrow, id_src, pages,
               (uint32_t*)img_h, (uint32_t*)img_l);
    if (sa.direct) {
      start = h_start;
      const int64_t end = h_end;
      uint32_t fl;
      int total;
      if (wv) {
        if (wid == kCW) {
          vd.eval(sa.chained, u, sa.U, fl, total, rank);
          if (sa.chained && p_live != start && p_live != start + total) fl |= kStStale;
          if (lane == 0) {
            s_vd[0] = total;
            s_vd[1] = rank;
            s_vd[2] = (int)fl;
          }
        }
        __syncthreads();
        total = s_vd[0];
        rank = s_vd[1];
        fl = (uint32_t)s_vd[2];
      } else if (sa.chained) {
        step_verdict_chain(u, sa.U, H, sa.cw, seq_len, state, s_vd, fl, total, rank);
        if (p_live != start && p_live != start + total) fl |= kStStale;
      } else {
        step_verdict(u, sa.U, sa.nf, s_vd, fl, total, rank);
      }
      const uint32_t st = fl ? fl : (total > end - start ? (uint32_t)kStExhausted : 0u);
      if (u == 0 && tid == 64 * kCW) {
        if (st) atomicOr(status, st);
        else sa.ptr[0] = (uint64_t)(start + total);
        if (sa.hdr_n) sa.hdr_n[SH_START] = st ? start : start + total;
      }
      go = st == 0 && (wu & kActive) != 0;
    } else {
      go = sa.hdr[SH_COMMIT] != 0 && (wu & kActive) != 0;
    }
    if (go) {
      nh += hi_app;
      nl += lo_app;
      ph += need == kTierHi;
      pl += need == kTierLo;
      tix_h = new_hi >> 4;
      tix_l = lo_src >= 0 ? L - 1 - (lo_slot >> 5) : -1;
      jh = tix_h;
      jl = lo_src >= 0 ? ph + (lo_slot >> 5) : -1;
    }
  }
  auto table_idx = [&](int j) { return j < ph ? j : L - 1 - (j - ph); };
  // page id by table index, the written pages' from LDS (read only after
  // the commit wave has published them); values, not pointers, are selected
  auto id_tix = [&](int tix) -> int32_t {
    const int32_t g = row[tix];
    if (!STEP) return g;
    const int32_t a = s_idt[0], c = s_idt[1];
    return tix == tix_h ? a : (tix == tix_l ? c : g);
  };
  auto valid = [&](int j) {
    return j < ph ? min(kHiTokens, nh - kHiTokens * j) : min(kLoTokens, nl - kLoTokens * (j - ph));
  };
  const bool sok = state_ok(nh, nl, ph, pl, L);
  const int TPg = sok ? ph + pl : 0;
  const int pps = split_pages(TPg, S);
  const int p0 = split * pps;
  const int p1 = min(TPg, p0 + pps);

  float* orow = out + ((int64_t)b * H * G + (int64_t)h * G) * D;
  if (N <= 0 || !sok || nh + nl == 0) {  // (a committing unit never ends here)
    if (S == 1 || split == 0) {
      for (int x = tid; x < G * D; x += blockDim.x) orow[x] = 0.0f;
      if (SAVE)
        for (int x = tid; x < G; x += blockDim.x) {
          ml[(u * G + x) * 2 + 0] = -INFINITY;
          ml[(u * G + x) * 2 + 1] = 0.0f;
        }
      if (N > 0 && !sok && tid == 0) atomicOr(status, kStBadState);
    }
    if constexpr (STEP)
      if (sa.cw_n && tid == 0) sa.cw_n[kChainWords * u] = -1;  // no plan for the next step
    if (S > 1) {
      float* mp = part + (((int64_t)u * S + split) * G) * (D + 2);
      for (int x = tid; x < G; x += blockDim.x) {
        mp[x * (D + 2) + D] = -INFINITY;
        mp[x * (D + 2) + D + 1] = 0.0f;
      }
    }
    return;
  }
  if (S > 1 && p0 >= p1) {  // a split past the unit's pages: an empty partial
    float* mp = part + (((int64_t)u * S + split) * G) * (D + 2);
    for (int x = tid; x < G; x += blockDim.x) {
      mp[x * (D + 2) + D] = -INFINITY;
      mp[x * (D + 2) + D + 1] = 0.0f;
    }
    return;
  }

  // ---- page order (wave-uniform).  The two waves that share a SIMD (w and
  // w + 4) do not progress alike: the hardware prefers the older one, whose
  // pages take 1.2-2x less time, by how much depending on the softmax layout
  // and the mode.  So the pages are cut in two ranges, each taken
  // round-robin: waves 0-3 the first kShare/256 of them, the others the
  // rest.  With a step, the commit wave takes the n_cw pages from `cut` up
  // (a linear fit in the page count: its share of the unit less its commit)
  // and then the written pages, which everyone else skips; waves 0-3 and 4-6
  // share the pages below `cut`.  The shares were measured (per-workgroup
  // timestamps) to end the waves together: G <= 4 on the Llama3-8B layer,
  // 4 < G <= 8 on the 200 GB stress workload.  The order is static: results
  // do not depend on timing.
  constexpr int kShare0 = E == 1 ? 171 : (E == 2 ? 165 : 170);  // attention alone
  constexpr int kShare1 = E == 1 ? 158 : (E == 2 ? 142 : 150);  // with the score update
  constexpr int kShareS = E == 1 ? 176 : (E == 2 ? 161 : 170);  // with a step: 4 waves against 3
  constexpr int kCwMul = E == 1 ? 24 : (E == 2 ? 28 : 32);       // n_cw = (TPg kCwMul - kCwSub) / 256
  constexpr int kCwSub = E == 1 ? 1137 : (E == 2 ? 640 : 2240);
  const int n_cw = go ? max(0, (TPg * kCwMul - kCwSub) >> 8) : 0;
  const int cut = TPg - n_cw;
  int lo, hi, stride, off;  // this wave's pages: lo + off, lo + off + stride, ... below hi
  if (!go) {
    const int nA = ((p1 - p0) * (MODE == 1 ? kShare1 : kShare0)) >> 8;
    lo = wid < 4 ? p0 : p0 + nA;
    hi = wid < 4 ? p0 + nA : p1;
    stride = 4;
    off = wid & 3;
  } else if (wid < kCW) {
    const int nA = (cut * kShareS) >> 8;  // 4 waves against 3
    lo = wid < 4 ? 0 : nA;
    hi = wid < 4 ? nA : cut;
    stride = wid < 4 ? 4 : kCW - 4;
    off = wid < 4 ? wid : wid - 4;
  } else {
    lo = cut;
    hi = TPg;
    stride = 1;
    off = 0;
  }
  auto nextj = [&](int j) -> int {
    j = j < 0 ? lo + off : j + stride;
    if (go)
      while (j < hi && (j == jh || j == jl)) j += stride;
    return j < hi ? j : -1;
  };
  auto fetch = [&](PageRegs<D, E>& R, int jj) {
    fetch_id(R, jj, row[table_idx(max(jj, 0))], true);  // uniform index: scalar load
  };
  const int ja0 = nextj(-1);
  const bool committer = STEP && go && wid == kCW;
  // this wave's page count (then, for the commit wave, the written pages from LDS)
  auto in_seq = [&](int x) { return x >= lo + off && x < hi && (x - lo - off) % stride == 0; };
  int n_w = lo + off < hi ? (hi - 1 - lo - off) / stride + 1 : 0;
  if (go) n_w -= (int)in_seq(jh) + (int)(jl >= 0 && in_seq(jl));
  if (ja0 >= 0 && !committer)
    fetch_id(A, ja0, (ja0 == wid && ja0 < ph0) ? id_guess : row[table_idx(ja0)], true);
  if constexpr (STEP) {
    if (committer) {
      int32_t page = -1;
      if (need) page = sa.direct ? sa.list[(uint64_t)(start + rank) % (uint64_t)P] : sa.rec[u * kSRec + S_PAGE];
      if (need && (page < 0 || page >= P)) {
        // a corrupt free list: nothing is committed and the unit's result is zeroed
        if (lane == 0) {
          atomicOr(status, kStBadState);
          s_idt[0] = 0;
          s_idt[1] = 0;
        }
        badid = 1;
      } else {
        int32_t idh, idl;
        wc.finish(L, page_bytes, P, N, nh0, nl0, ph0, pl0, need, page, new_hi, hi_app, lo_src, lo_slot, lo_app,
                  id_hrow, id_lrow, id_first, sa.table + u * L, sa.state + 4 * u, pages, (uint32_t*)img_h,
                  (uint32_t*)img_l, idh, idl);
        if (lane == 0) {
          s_idt[0] = min(max(idh, 0), (int32_t)(P - 1));
          s_idt[1] = min(max(idl, 0), (int32_t)(P - 1));
        }
      }
      if (ja0 >= 0) fetch(A, ja0);
    }
  }

  // ---- Q operand: lane (i, qg) holds column i's head, dims qg*QD .. +QD-1;
  // with PACK, columns GP .. GP+G-1 repeat heads 0 .. G-1 (their tails) ----
  const bool tail = PACK && i >= GP;
  half8_t qop[NS];
  float sumq = 0.0f;
  {
    uint16_t qv[QD];
#pragma unroll
    for (int c = 0; c < QD / 8; c++) {
      const uint4 w = qraw[c];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        qv[8 * c + 2 * e] = qhead >= 0 ? (uint16_t)(ws[e] & 0xFFFFu) : (uint16_t)0;
        qv[8 * c + 2 * e + 1] = qhead >= 0 ? (uint16_t)(ws[e] >> 16) : (uint16_t)0;
      }
    }
#pragma unroll
    for (int e = 0; e < QD; e++) sumq += h2f(qv[e]);
    auto H16 = [&](int e) { return __builtin_bit_cast(_Float16, qv[e]); };
#pragma unroll
    for (int ks = 0; ks < NS; ks++)
      qop[ks] = half8_t{H16(8 * ks), H16(8 * ks + 1), H16(8 * ks + 2), H16(8 * ks + 3),
                        H16(8 * ks + 4), H16(8 * ks + 5), H16(8 * ks + 6), H16(8 * ks + 7)};
    sumq += __shfl_xor(sumq, 16, 64);
    sumq += __shfl_xor(sumq, 32, 64);
  }
  // sum(q) of the lane's softmax head (lanes of columns >= 2GP hold no q)
  const float sq2c = sumq * scale_log2;
  const float sq2 = PACK ? __shfl(sq2c, (lane & 48) | hs, 64) : sq2c;
  const float tm = tail ? 1.0f : 0.0f;

  Softmax sm{-INFINITY, 0.0f, 0.0f};
  float4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++) acc[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // logits go to LDS when the whole unit's fit (fused score update), else to
  // the workspace (indexed by table slot)
  const bool lg_lds = MODE == 1 && TPg * 32 * (G + 2) + TPg <= kLdsWords;
  const bool ids_lds = MODE == 1 && !lg_lds && TPg <= kLdsWords;  // workspace logits, page ids in LDS
  const int GS = logit_stride(G);
  float* lg_s = (float*)lds_w;
  float* osc_s = (float*)lds_w + TPg * 32 * G;
  int32_t* pos_s = (int32_t*)lds_w + TPg * 32 * (G + 1);
  int32_t* id_s = (int32_t*)lds_w + TPg * 32 * (G + 2);

  // ---- page loop: the next page's loads in flight during each compute ----
  // Instantiated once per logits destination (LDS or workspace) so that the
  // per-block stores need no branch.
  auto page_loop = [&](auto lds_tag) {
    constexpr bool kLds = decltype(lds_tag)::value;
    auto run = [&](PageRegs<D, E>& R, int j) {
      if (kLds) {
        if (lane < 32) osc_s[j * 32 + lane] = __uint_as_float(R.sp);
        else pos_s[j * 32 + lane - 32] = (int32_t)R.sp;
      }
      // the page ids the score pass visits (workspace logits: the LDS area
      // holds only the ids)
      if (MODE == 1 && lane == 0 && (kLds || ids_lds)) (kLds ? id_s : (int32_t*)lds_w)[j] = R.id;
      // logits: LDS g-major [G][TPg * 32]; workspace by table slot in the
      // lanes' own order, [L][32/4][GS][4] (GS = GP): the E consecutive
      // tokens a lane holds for its head are one store, every lane storing
      // (heads G..GS-1 hold finite values the score pass masks)
      float* lgp = kLds ? lg_s + hs * (TPg * 32) + j * 32 : logits + ((int64_t)u * L + table_idx(j)) * 32 * GS;
      compute_page<D, E, PACK>(R, j < ph, valid(j), qop, sq2, scale_log2, tm, ts, sm, acc, [&](int mb, const float* x) {
        if (!SAVE || hs >= (kLds ? G : GS)) return;
        const int t0 = 16 * mb + ts;
        if (kLds) {
#pragma unroll
          for (int e = 0; e < E; e++) lgp[t0 + e] = x[e];
        } else {
          float* dst = lgp + ((t0 >> 2) * GS + hs) * 4 + (t0 & 3);
          if constexpr (E == 4) *(float4_t*)dst = float4_t{x[0], x[1], x[2], x[3]};
          else if constexpr (E == 2) *(float2_t*)dst = float2_t{x[0], x[1]};
          else *dst = x[0];
        }
      });
    };
    // A and B alternate over the wave's n_w pages; the last one is peeled
    // so that no load is in flight when the wave reaches the merge (the
    // loads of each iteration are unconditional: nothing for the compiler
    // to wait on at a join)
    int ja = ja0;
    int k = 1;
    if (n_w > 0) {
    for (; k + 2 <= n_w; k += 2) {
      const int jb = nextj(ja);
      fetch(B, jb);
      run(A, ja);
      ja = nextj(jb);
      fetch(A, ja);
      run(B, jb);
    }
    if (k < n_w) {
      const int jb = nextj(ja);
      fetch(B, jb);
      run(A, ja);
      run(B, jb);
    } else {
      run(A, ja);
    }
    }
    if constexpr (STEP) {
      // the commit wave: the pages the step wrote, from their LDS images
      // (after the regular loop, so that no join in it mixes LDS and memory
      // loads of a page)
      if (committer) {
        for (int t = 0; t < 2; t++) {
          const int j = t == 0 ? jh : jl;
          if (j < 0) continue;
          const uint8_t* img = (const uint8_t*)(t == 0 ? img_h : img_l);
          load_page<D, E>(A, img, j >= ph, kbase, mt, vl);
          if (MODE == 1) load_page_sp<D, E>(A, img, j >= ph, lane);
          A.id = s_idt[t];
          run(A, j);
        }
      }
    }
  };
  if (n_w > 0 || committer) {
    if constexpr (MODE == 1) {
      if (lg_lds) page_loop(std::true_type{});
      else page_loop(std::false_type{});
    } else {
      page_loop(std::false_type{});
    }
  }

  // ---- merge the waves: maxima, rescale, fixed-order sums in LDS ----
  // Two barriers: after the first every lane derives its column's maximum
  // and sum from the waves' values itself (same order in every lane).
  sm.lsum = heads_sum<E>(rows_sum(sm.lsum));
  sm.zsum = heads_sum<E>(rows_sum(sm.zsum));
  __shared__ uint32_t wbad[kWaves];
  __shared__ int s_tc;
  __shared__ float s_tcsum;
  if (qg == 0) {
    wm[wid][i] = sm.m;
    wl[wid][i] = sm.lsum;
  }
  if (lane == 0) wbad[wid] = 0;
  if (badid) wbad[wid] = 1;
  if (MODE == 1 && tid == 0) s_tc = -1;
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (int w = 0; w < kWaves; w++) bad |= wbad[w] != 0;
  {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; w++) M = fmaxf(M, wm[w][i]);
    float l = 0.0f;
    if (M != -INFINITY)
#pragma unroll
      for (int w = 0; w < kWaves; w++) l += wl[w][i] * __builtin_amdgcn_exp2f(wm[w][i] - M);
    if (wid == 0 && qg == 0) {
      sM[i] = M;
      sL[i] = l;
      sI[i] = l > 0.0f ? 1.0f / l : 0.0f;
    }
    const int ncol = PACK ? 2 * GP : G;  // columns that carry data
    if (i < ncol) {
      // O = acc + sum p (z_v - kv s_v) (the z term once per head: not in tail columns)
      const float f = (M == -INFINITY || sm.m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sm.m - M);
      const float z = tail ? 0.0f : sm.zsum;
      // lane (i, qg), block nb: dims 16nb + 4qg .. +3 of column i; the 16-byte
      // slot index is xor-swizzled with the column so that the 16 columns of
      // one store land in different banks
#pragma unroll
      for (int nb = 0; nb < NB; nb++) buf[wid][i * (D / 4) + ((4 * nb + qg) ^ (i & 15))] = (acc[nb] + z) * f;
    }
  }
  __syncthreads();
  const float* ob = (const float*)&buf[0][0];
  auto ocol = [&](int g, int dim) {  // sum over waves (fixed order) of column g (+ its tail)
    const int o0 = (g * (D / 4) + ((dim >> 2) ^ (g & 15))) * 4 + (dim & 3);
    const int o1 = ((g + GP) * (D / 4) + ((dim >> 2) ^ ((g + GP) & 15))) * 4 + (dim & 3);
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
      o += ob[w * 16 * D + o0];
      if (PACK) o += ob[w * 16 * D + o1];
    }
    return o;
  };

  if (bad && tid == 0) atomicOr(status, kStBadState);
  if (S == 1) {
    if (bad) {
      for (int x = tid; x < G * D; x += blockDim.x) orow[x] = 0.0f;
      if (SAVE && tid < G) {
        ml[(u * G + tid) * 2 + 0] = -INFINITY;
        ml[(u * G + tid) * 2 + 1] = 0.0f;
      }
      if constexpr (STEP)
        if (sa.cw_n && tid == 0) sa.cw_n[kChainWords * u] = -1;
      return;
    }
    for (int x = tid; x < G * D; x += blockDim.x) orow[x] = ocol(x / D, x % D) * sI[x / D];
    if (SAVE && tid < G) {
      ml[(u * G + tid) * 2 + 0] = sM[tid];
      ml[(u * G + tid) * 2 + 1] = sL[tid];
    }
    if (MODE == 1) {
      // score update: every retained token other than the query's own
      // (position seq_len) adds max over the group of its softmax weight.
      // With every score sum of the unit in hand, the pass also plans the
      // next generation step (length N + 1) and leaves the plan in the
      // unit's first high page, so that step needs no scan.
      const Seg sh = tier_seg(D, true), sl = tier_seg(D, false);
      const int64_t N1 = (int64_t)N + 1, tc1 = N1 - pa.W;
      __shared__ Cand cw[2][kWaves];
      Cand bh{0.0f, kNoPos, 0}, bl{0.0f, kNoPos, 0};
      const int NSL = TPg * 32;  // slot rows in LDS, 32 per page (high pages use 16)
      const int NE = 16 * ph + 32 * pl;  // slots the pass visits: 16 per high page
      // pass index -> (page, in-page slot): high pages first, then low pages
      auto slot_of = [&](int xe, int& j, int& t) {
        if (xe < 16 * ph) {
          j = xe >> 4;
          t = xe & 15;
        } else {
          const int y = xe - 16 * ph;
          j = ph + (y >> 5);
          t = y & 31;
        }
      };
      // c_g with max_g 2^(x_g - M_g) / L_g = 2^(max_g (x_g + c_g)),
      // c_g = -M_g - log2 L_g: one exponential per slot.  GB >= G heads per
      // slot (LDS: indices clamped to G - 1, repeats do not change a maximum;
      // workspace: GB = GS, heads G..GB-1 masked by c = -inf)
      auto cvec = [&](float* cg, int GB, bool lds) {
        for (int g = 0; g < GB; g++) {
          const float M = sM[min(g, G - 1)], I = sI[min(g, G - 1)];
          cg[g] = (M == -INFINITY || I == 0.0f || (!lds && g >= G)) ? -INFINITY : __builtin_amdgcn_logf(I) - M;
        }
      };
      // one slot's new sum: t_c's sum published, the tier's running
      // candidate updated with one comparison
      auto visit = [&](bool ok, bool hi, int j, int t, float ns, int32_t pos) {
        const int ls = hi ? 16 * j + t : 32 * (j - ph) + t;
        if (ok && hi && pos == tc1) {  // positions are unique: one writer
          s_tc = ls;
          s_tcsum = ns;
        }
        const Cand c{ns, (ok && (!hi || pos <= tc1)) ? pos : kNoPos, ls};
        const Cand a{hi ? bh.sum : bl.sum, hi ? bh.pos : bl.pos, hi ? bh.slot : bl.slot};
        const bool win = less_imp(c, a, N1);
        if (win && hi) bh = c;
        if (win && !hi) bl = c;
      };
      // logits in LDS: one slot per thread and round
      auto pass_lds = [&](auto gb_tag) {
        constexpr int GB = decltype(gb_tag)::value;
        float cg[GB];
#pragma unroll
        for (int g = 0; g < GB; g++) cg[g] = 0.0f;
        cvec(cg, GB, true);
        // wave-uniform trip count: a wave runs while its first slot is in range
        for (int xe = tid; xe - lane < NE; xe += kThreads) {
          int j, t;
          slot_of(min(xe, NE - 1), j, t);
          const int x = 32 * j + t;
          const bool hi = j < ph;
          float xm = -INFINITY;
#pragma unroll
          for (int g = 0; g < GB; g++) xm = fmaxf(xm, lg_s[min(g, G - 1) * NSL + x] + cg[g]);
          const int32_t pos = pos_s[x];
          const bool ok = xe < NE && t < valid(j) && pos < N;
          const float ns = osc_s[x] + __builtin_amdgcn_exp2f(xm);
          uint8_t* pg = pages + (int64_t)id_s[j] * page_bytes;
          // non-temporal: these words are read again only by a later
          // step, and the launch then ends with fewer dirty lines to write back
          if (ok) __builtin_nontemporal_store(ns, (float*)(pg + (hi ? sh.sc : sl.sc) + 4 * t));
          visit(ok, hi, j, t, ns, pos);
        }
      };
      // logits in the workspace, [L][32/4][GB][4] per unit: four consecutive
      // slots of a page per thread (pages hold 16 or 32 slots, so a group
      // never straddles two), kUG groups per round with every load issued
      // before any use; a group's sums are stored as one 16-byte word (slots
      // that do not change are stored back unchanged)
      auto pass_ws = [&](auto gb_tag) {
        constexpr int GB = decltype(gb_tag)::value;
        constexpr int kUG = 2;
        float cg[GB];
#pragma unroll
        for (int g = 0; g < GB; g++) cg[g] = 0.0f;
        cvec(cg, GB, false);
        const float* lgg = logits + (int64_t)u * L * 32 * GB;
        const int NG = NE >> 2;  // NE is a multiple of 16
        for (int x0 = tid; x0 - lane < NG; x0 += kUG * kThreads) {
          float lv[kUG][GB][4];
          float4_t osv[kUG];
          int4 psv[kUG];
          uint8_t* pgv[kUG];
#pragma unroll
          for (int e = 0; e < kUG; e++) {
            int j, t;
            slot_of(4 * min(x0 + e * kThreads, NG - 1), j, t);
            const bool hi = j < ph;
            const int tx = table_idx(j);
            const float4_t* src = (const float4_t*)(lgg + ((int64_t)tx * 32 + t) * GB);
#pragma unroll
            for (int g = 0; g < GB; g++) {
              const float4_t v4 = src[g];
#pragma unroll
              for (int r = 0; r < 4; r++) lv[e][g][r] = v4[r];
            }
            pgv[e] = pages + (int64_t)(ids_lds ? ((const int32_t*)lds_w)[j] : id_tix(tx)) * page_bytes;
            osv[e] = *(const float4_t*)(pgv[e] + (hi ? sh.sc : sl.sc) + 4 * t);
            psv[e] = *(const int4*)(pgv[e] + (hi ? sh.ps : sl.ps) + 4 * t);
          }
#pragma unroll
          for (int e = 0; e < kUG; e++) {
            const int xg = x0 + e * kThreads;
            int j, t;
            slot_of(4 * min(xg, NG - 1), j, t);
            const bool hi = j < ph;
            const int nv = valid(j);
            const int32_t pv[4] = {psv[e].x, psv[e].y, psv[e].z, psv[e].w};
            float4_t nsv;
#pragma unroll
            for (int r = 0; r < 4; r++) {
              const bool ok = xg < NG && t + r < nv && pv[r] < N;
              float xm = -INFINITY;
#pragma unroll
              for (int g = 0; g < GB; g++) xm = fmaxf(xm, lv[e][g][r] + cg[g]);
              const float ns = osv[e][r] + __builtin_amdgcn_exp2f(xm);
              nsv[r] = ok ? ns : osv[e][r];
              visit(ok, hi, j, t + r, ns, pv[r]);
            }
            if (xg < NG) __builtin_nontemporal_store(nsv, (float4_t*)(pgv[e] + (hi ? sh.sc : sl.sc) + 4 * t));
          }
        }
      };
      using I4 = std::integral_constant<int, 4>;
      using I8 = std::integral_constant<int, 8>;
      using I16 = std::integral_constant<int, 16>;
      if (lg_lds) {
        if (G <= 4) pass_lds(I4{});
        else if (G <= 8) pass_lds(I8{});
        else pass_lds(I16{});
      } else {
        if (G <= 4) pass_ws(I4{});
        else if (G <= 8) pass_ws(I8{});
        else pass_ws(I16{});
      }
      // The next step's plan needs at most one of the two candidates: the
      // class of the token leaving the window decides (high: the least
      // important high token; low: the least important low token; pruned:
      // neither), and it is known once the pass has published t_c.
      __syncthreads();
      const int tcs = s_tc;
      const float tcsum = s_tcsum;
      int cls = -1;
      if (tc1 >= 0 && tcs >= 0)
        cls = classify_mean(tcsum, pa.W - 1, N1 + 1, pa.lo_en, pa_ah(pa, h), pa_al(pa, h));
      const bool needH = cls == kTierHi, needL = cls == kTierLo;
      // the needed candidate: wave butterflies, then the waves' results in
      // lanes 0..7 of wave 0
      if (needH) bh = wave_argmin(bh, N1);
      if (needL) bl = wave_argmin(bl, N1);
      if (lane == 0) {
        cw[0][wid] = bh;
        cw[1][wid] = bl;
      }
      __syncthreads();
      static_assert(kWaves == 8, "eight wave candidates");
      if (wid == 0) {
        if (needH) {
          bh = cw[0][lane & 7];
          argmin_step<0>(bh, N1);
          argmin_step<1>(bh, N1);
          argmin_step<2>(bh, N1);
        }
        if (needL) {
          bl = cw[1][lane & 7];
          argmin_step<0>(bl, N1);
          argmin_step<1>(bl, N1);
          argmin_step<2>(bl, N1);
        }
        // a record only where the next step's plan kernel would accept the
        // state.  Every lane holds the candidates and takes the decision;
        // lane k writes word k of each record (one store instruction per
        // record, one round of id lookups).
        const bool rec_ok = ph >= 1 && nh + nl <= N1 && !(tc1 >= 0 && tcs < 0);
        if (rec_ok) {
          const Plan pn = plan_decide(N1, pa.W, pa.S_max, pa.lo_en, pa_ah(pa, h), pa_al(pa, h), nh, nl, ph, pl,
                                      L, tcs, tcsum, bh, bl);
          uint32_t rw[kRecWords];
          plan_rec_fill(rw, N1, nh, nl, ph, pl, pn);
          uint32_t wv = rw[0];
#pragma unroll
          for (int k = 1; k < kRecWords; k++) wv = lane == k ? rw[k] : wv;
          // the unit's first high page (page-loop index 0: its id in LDS when the ids are there)
          const int32_t id0 = lg_lds ? id_s[0] : (ids_lds ? ((const int32_t*)lds_w)[0] : id_tix(0));
          uint32_t* dst = (uint32_t*)(pages + (int64_t)id0 * page_bytes + plan_rec_off<D>());
          if (lane < kRecWords) dst[lane] = wv;
          if constexpr (STEP) {
            if (sa.cw_n) {
              // the same plan in the next step's slot: the step record
              // (plan fields, then the ids of the pages the commit reads,
              // from the table after this step: the page list in LDS when it
              // is there; entries past the unit's pages are -1), the chain
              // words and the demand word
              auto cl = [&](int t) { return min(max(t, 0), L - 1); };
              const int tix = lane == S_IDH   ? cl(pn.new_hi >> 4)
                              : lane == S_IDL ? cl(L - 1 - (pn.lo_slot >> 5))
                              : lane == S_IDS ? cl(pn.lo_src >> 4)
                                              : 0;
              int32_t id;
              if (lg_lds || ids_lds) {
                const int32_t* ids = lg_lds ? id_s : (const int32_t*)lds_w;
                const int j = tix < ph ? tix : ph + (L - 1 - tix);
                id = ids[min(j, TPg - 1)];
                id = j < TPg ? id : -1;
              } else {
                id = id_tix(tix);
              }
              const int32_t rv = lane == S_NEWHI   ? pn.new_hi
                                 : lane == S_HIAPP  ? pn.hi_app
                                 : lane == S_LOSRC  ? pn.lo_src
                                 : lane == S_LOSLOT ? pn.lo_slot
                                 : lane == S_LOAPP  ? pn.lo_app
                                 : lane == S_PAGE   ? -1
                                                    : id;
              if (lane <= S_IDF) sa.rec_n[u * kSRec + lane] = rv;
              const int32_t c4[kChainWords] = {(int32_t)N1, nh, nl, ph, pl, pn.nfw, pn.hi_app, pn.lo_app};
              int32_t cv = c4[0];
#pragma unroll
              for (int k = 1; k < kChainWords; k++) cv = lane == k ? c4[k] : cv;
              if (lane < kChainWords) sa.cw_n[kChainWords * u + lane] = cv;
              if (lane == 0) sa.nf_n[u] = pn.nfw;
            }
          }
        } else if (STEP && lane == 0 && sa.cw_n) {
          sa.cw_n[kChainWords * u] = -1;
        }
      }
    }
  } else {
    float* mp = part + (((int64_t)u * S + split) * G) * (D + 2);
    for (int x = tid; x < G * D; x += blockDim.x) mp[(x / D) * (D + 2) + x % D] = ocol(x / D, x % D);
    if (tid < G) {
      mp[tid * (D + 2) + D] = bad ? NAN : sM[tid];  // NaN marks a bad unit for the merge
      mp[tid * (D + 2) + D + 1] = sL[tid];
    }
  }
}

// Split merge (several workgroups per unit): out = sum_s O_s 2^(m_s - M) /
// sum_s l_s 2^(m_s - M); also the final (M, L) for the score update.  One
// workgroup per (head, unit): the splits' maxima and sums come in one pass,
// every thread derives M and the sum from LDS (same order everywhere), and an
// output dim is summed by 256 / D threads over interleaved attending splits
// (loads eight at a time), then added in LDS.
// A NaN maximum marks a unit with a bad page id: output 0, (M, L) = (-inf, 0).

template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(int H, int G, int S, const int32_t* __restrict__ seq_len,
                                                         const float* __restrict__ part, float* __restrict__ out,
                                                         float* __restrict__ ml, int save) {
  constexpr int T = 256 / D;  // threads per output dim
  const int g = blockIdx.x;
  const int64_t u = blockIdx.y;
  const int b = (int)u / H, h = (int)u % H;  // u < 2^31: 32-bit division
  if (seq_len[b] <= 0) return;  // the attention kernel already wrote zeros
  const int64_t stride = (int64_t)G * (D + 2);  // from one split's head g to the next split's
  const float* up = part + (u * S * G + g) * (D + 2);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  __shared__ float sm[kMaxSplits], sl[kMaxSplits], sw[kMaxSplits];  // maxima, sums, weights
  __shared__ float so[256];
  __shared__ int s_act[kMaxSplits], s_cnt[2];
  if (tid < S) {
    sm[tid] = up[tid * stride + D];
    sl[tid] = up[tid * stride + D + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  bool bad = false;
  for (int sp = 0; sp < S; sp++) {
    const float m = sm[sp];
    bad |= m != m;
    M = fmaxf(M, m);
  }
  if (bad) M = -INFINITY;
  bool act = false;
  if (tid < S) {
    const float m = sm[tid];
    const float w = (M == -INFINITY || m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    sw[tid] = w;
    act = w != 0.0f;
  }
  // the splits with a nonzero weight, in order
  const uint64_t mask = __ballot(act);
  if (wid < 2 && lane == 0) s_cnt[wid] = __popcll(mask);
  __syncthreads();
  if (wid < 2 && act) {
    const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    s_act[(wid == 1 ? s_cnt[0] : 0) + below] = tid;
  }
  float l = 0.0f;
  for (int sp = 0; sp < S; sp++) {
    const float w = sw[sp];
    if (w != 0.0f) l += sl[sp] * w;
  }
  if (save && tid == 0) {
    ml[(u * G + g) * 2 + 0] = M;
    ml[(u * G + g) * 2 + 1] = l;
  }
  __syncthreads();
  const int na = s_cnt[0] + (S > 64 ? s_cnt[1] : 0);
  const int dd = tid % D;
  float o = 0.0f;
  int k = tid / D;
  for (; k + 7 * T < na; k += 8 * T) {
    float v[8], w[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int sp = s_act[k + e * T];
      v[e] = up[sp * stride + dd];
      w[e] = sw[sp];
    }
#pragma unroll
    for (int e = 0; e < 8; e++) o += v[e] * w[e];
  }
  for (; k < na; k += T) {
    const int sp = s_act[k];
    o += up[sp * stride + dd] * sw[sp];
  }
  so[tid] = o;
  __syncthreads();
  if (tid < D) {
    float t = so[tid];
#pragma unroll
    for (int p = 1; p < T; p++) t += so[p * D + tid];
    out[(((int64_t)b * H + h) * G + g) * D + tid] = l > 0.0f ? t / l : 0.0f;
  }
}

// Score update from saved logits (several splits, or a deferred update):
// 64 pages per workgroup, their slots enumerated as the fused pass does (16
// per high page, 32 per low page: at most 2048, in groups of four
// consecutive slots, two groups per thread); every load of a thread's groups
// (table entries, the group's logits as GB 16-byte loads, then positions and
// old sums) is issued before any is used, each slot takes one exponential:
// max_g p_g = 2^(max_g (x_g + c_g)), c_g = -M_g - log2 L_g, and a group's new
// sums are stored as one 16-byte word.
// A unit whose merge found a bad page id has (M, L) = (-inf, 0) and is left
// alone; ids are checked where they are used.  Each chunk also leaves the
// candidates the next generation step (length N + 1) needs: the least
// important non-window high token, the least important low token and the
// token leaving the window, from the updated sums (the rules of the fused
// update); score_finish_kernel turns them into the unit's plan record.
// MERGE (the update in the same call as the attention): every workgroup takes
// its unit's (M, L) from the S split partials itself, and the unit's first
// chunk also writes the merged output and (M, L) -- the split merge as
// attn_merge_kernel does it, one kernel launch fewer.

template <int D, int GB, bool MERGE>
__global__ __launch_bounds__(256) void score_kernel(int H, int G, int L, int64_t P, int page_bytes, int W,
                                                    const int32_t* __restrict__ table,
                                                    const int32_t* __restrict__ state,
                                                    const int32_t* __restrict__ seq_len,
                                                    float* __restrict__ ml,
                                                    const float* __restrict__ logits, uint8_t* pages,
                                                    int32_t* __restrict__ cand, int S,
                                                    const float* __restrict__ part, float* __restrict__ out) {
  const int split = blockIdx.x;
  const int64_t u = blockIdx.y;
  const int b = (int)u / H;
  const int tid = threadIdx.x;
  const int32_t* row = table + u * L;
  const int32_t* s4 = state + 4 * u;
  const int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  const int N = seq_len[b];
  if (N <= 0 || nh + nl == 0 || !state_ok(nh, nl, ph, pl, L)) return;
  const int TPg = ph + pl;
  const int p0 = split * kScorePages, p1 = min(TPg, p0 + kScorePages);
  if (p0 >= p1) return;
  __shared__ float sC[16];  // c_g = -M_g - log2 L_g (-inf: no weight)
  if constexpr (MERGE) {
    // every split's (m, l) per head into LDS in one round of loads; per head
    // M = max over the splits (a NaN marks a bad unit: M = -inf), the splits'
    // weights 2^(m_s - M) and L, in split order
    __shared__ float sW[16][kMaxSplits];
    __shared__ float sMS[kMaxSplits * 16], sLS[kMaxSplits * 16];
    __shared__ float sML[16][2];
    const float* up = part + (u * S) * G * (D + 2);
    for (int x = tid; x < S * G; x += 256) {
      sMS[x] = up[x * (D + 2) + D];
      sLS[x] = up[x * (D + 2) + D + 1];
    }
    __syncthreads();
    if (tid < G) {
      float M = -INFINITY;
      bool badp = false;
      for (int sp = 0; sp < S; sp++) {
        const float m = sMS[sp * G + tid];
        badp |= m != m;
        M = fmaxf(M, m);
      }
      if (badp) M = -INFINITY;
      float l = 0.0f;
      for (int sp = 0; sp < S; sp++) {
        const float m = sMS[sp * G + tid];
        const float w = (M == -INFINITY || m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
        sW[tid][sp] = w;
        if (w != 0.0f) l += sLS[sp * G + tid] * w;
      }
      sML[tid][0] = M;
      sML[tid][1] = l;
    }
    __syncthreads();
    if (split == 0) {
      // the merged output: eight splits' values of an output loaded at once
      const int hh = (int)(u % H);
      for (int x = tid; x < G * D; x += 256) {
        const int g = x / D, dd = x % D;
        float o = 0.0f;
        for (int sp0 = 0; sp0 < S; sp0 += 8) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; e++) v[e] = sp0 + e < S ? up[((sp0 + e) * G + g) * (D + 2) + dd] : 0.0f;
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const float w = sp0 + e < S ? sW[g][sp0 + e] : 0.0f;
            if (w != 0.0f) o += v[e] * w;
          }
        }
        const float l = sML[g][1];
        out[(((int64_t)b * H + hh) * G + g) * D + dd] = l > 0.0f ? o / l : 0.0f;
      }
      if (tid < G) {
        ml[(u * G + tid) * 2 + 0] = sML[tid][0];
        ml[(u * G + tid) * 2 + 1] = sML[tid][1];
      }
    }
    if (!(sML[0][1] > 0.0f)) return;  // bad unit (or nothing attended)
    if (tid < GB) {
      const float M = tid < G ? sML[tid][0] : -INFINITY;
      const float l = tid < G ? sML[tid][1] : 0.0f;
      sC[tid] = (M == -INFINITY || !(l > 0.0f)) ? -INFINITY : __builtin_amdgcn_logf(1.0f / l) - M;
    }
  } else {
    if (ml[u * G * 2 + 1] <= 0.0f) return;  // bad unit (or nothing attended)
    if (tid < GB) {
      const float M = tid < G ? ml[(u * G + tid) * 2 + 0] : -INFINITY;
      const float l = tid < G ? ml[(u * G + tid) * 2 + 1] : 0.0f;
      sC[tid] = (M == -INFINITY || !(l > 0.0f)) ? -INFINITY : __builtin_amdgcn_logf(1.0f / l) - M;
    }
  }
  // the unit's scores change here: a plan record no longer applies
  if (split == 0 && tid == 0 && ph >= 1) {
    const int32_t id0 = row[0];
    if (id0 >= 0 && id0 < P) *(uint32_t*)(pages + (int64_t)id0 * page_bytes + plan_rec_off<D>()) = 0u;
  }
  __shared__ int s_tc;      // slot of the token leaving the window at length N + 1
  __shared__ float s_tcsum;
  if (tid == 0) s_tc = -1;
  // the chunk's slots: high pages (16 slots) first, then low pages (32)
  const int nhp = max(0, min(ph, p1) - p0);
  const int NE = 16 * nhp + 32 * (p1 - p0 - nhp);
  auto slot_of = [&](int xe, int& j, int& t) {
    if (xe < 16 * nhp) {
      j = p0 + (xe >> 4);
      t = xe & 15;
    } else {
      const int y = xe - 16 * nhp;
      j = p0 + nhp + (y >> 5);
      t = y & 31;
    }
  };
  const Seg sh = tier_seg(D, true), sl = tier_seg(D, false);
  // groups of four consecutive slots of a page (logits [L][32/4][GB][4] per
  // unit, as the attention stores them)
  constexpr int GPT = kScorePages * 32 / 4 / 256;  // groups per thread
  const int NG = NE >> 2;
  int32_t id[GPT], jx[GPT], tt[GPT];
  float lv[GPT][GB][4];
#pragma unroll
  for (int e = 0; e < GPT; e++) {
    const int xg = tid + 256 * e;
    int j, t;
    slot_of(4 * min(xg, NG - 1), j, t);
    const bool is_hi = j < ph;
    const int jt = is_hi ? j : j - ph;
    const int tx = is_hi ? jt : L - 1 - jt;
    jx[e] = j;
    tt[e] = t;
    id[e] = row[tx];
    const float4_t* src = (const float4_t*)(logits + (((int64_t)u * L + tx) * 32 + t) * GB);
#pragma unroll
    for (int g = 0; g < GB; g++) {
      const float4_t v4 = src[g];
#pragma unroll
      for (int r = 0; r < 4; r++) lv[e][g][r] = v4[r];
    }
  }
  int4 pos[GPT];
  float4_t old[GPT];
  uint8_t* pgs[GPT];
  bool okp[GPT];
#pragma unroll
  for (int e = 0; e < GPT; e++) {
    const bool is_hi = jx[e] < ph;
    okp[e] = tid + 256 * e < NG && id[e] >= 0 && id[e] < P;
    const uint8_t* pg = pages + (int64_t)(okp[e] ? id[e] : 0) * page_bytes;
    pgs[e] = (uint8_t*)pg + (is_hi ? sh.sc : sl.sc) + 4 * tt[e];
    pos[e] = *(const int4*)(pg + (is_hi ? sh.ps : sl.ps) + 4 * tt[e]);
    old[e] = *(const float4_t*)pgs[e];
  }
  __syncthreads();  // sC, s_tc
  float cg[GB];
#pragma unroll
  for (int g = 0; g < GB; g++) cg[g] = sC[g];
  const int64_t N1 = (int64_t)N + 1, tc1 = N1 - W;
  __shared__ Cand cw[2][4];
  Cand bh{0.0f, kNoPos, 0}, bl{0.0f, kNoPos, 0};
#pragma unroll
  for (int e = 0; e < GPT; e++) {
    const int j = jx[e];
    const bool is_hi = j < ph;
    const int jt = is_hi ? j : j - ph;
    const int nval = is_hi ? min(kHiTokens, nh - kHiTokens * jt) : min(kLoTokens, nl - kLoTokens * jt);
    const int32_t pv[4] = {pos[e].x, pos[e].y, pos[e].z, pos[e].w};
    float4_t nsv;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int t = tt[e] + r;
      const bool upd = okp[e] && t < nval && pv[r] < N;
      float xm = -INFINITY;
#pragma unroll
      for (int g = 0; g < GB; g++) xm = fmaxf(xm, lv[e][g][r] + cg[g]);
      const float ns = old[e][r] + __builtin_amdgcn_exp2f(xm);
      nsv[r] = upd ? ns : old[e][r];
      const int ls = is_hi ? 16 * j + t : 32 * (j - ph) + t;
      if (upd && is_hi && pv[r] == tc1) {  // positions are unique: one writer
        s_tc = ls;
        s_tcsum = ns;
      }
      const Cand c{ns, (upd && (!is_hi || pv[r] <= tc1)) ? pv[r] : kNoPos, ls};
      if (is_hi) bh = min_imp(bh, c, N1);
      else bl = min_imp(bl, c, N1);
    }
    // the group's sums as one word (unchanged slots stored back as they were)
    if (okp[e]) *(float4_t*)pgs[e] = nsv;
  }
  bh = wave_argmin(bh, N1);
  bl = wave_argmin(bl, N1);
  const int lane = tid & 63, wid = tid >> 6;
  if (lane == 0) {
    cw[0][wid] = bh;
    cw[1][wid] = bl;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; w++) {
      bh = min_imp(bh, cw[0][w], N1);
      bl = min_imp(bl, cw[1][w], N1);
    }
    int32_t* cp = cand + ((int64_t)u * gridDim.x + split) * kCandWords;
    cp[0] = __float_as_int(bh.sum);
    cp[1] = bh.pos;
    cp[2] = bh.slot;
    cp[3] = __float_as_int(bl.sum);
    cp[4] = bl.pos;
    cp[5] = bl.slot;
    cp[6] = s_tc;
    cp[7] = __float_as_int(s_tcsum);
  }
}

// One wave per unit: the chunks' candidates reduced (the order does not
// matter: the comparison is a strict total order), then the next step's
// decision written as the unit's plan record, as the fused update does.  The
// conditions under which score_kernel leaves a unit alone are re-checked
// here, so candidates of an earlier call are never used.
template <int D>
__global__ __launch_bounds__(64) void score_finish_kernel(int H, int G, int L, int64_t P, int page_bytes,
                                                          PolicyArgs pa, const int32_t* __restrict__ table,
                                                          const int32_t* __restrict__ state,
                                                          const int32_t* __restrict__ seq_len,
                                                          const float* __restrict__ ml,
                                                          const int32_t* __restrict__ cand, uint8_t* pages) {
  const int64_t u = blockIdx.x;
  const int b = (int)u / H;
  const int lane = threadIdx.x;
  const int32_t* row = table + u * L;
  const int32_t* s4 = state + 4 * u;
  const int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  const int N = seq_len[b];
  if (N <= 0 || nh + nl == 0 || !state_ok(nh, nl, ph, pl, L) || ph < 1) return;
  if (ml[u * G * 2 + 1] <= 0.0f) return;
  const int64_t N1 = (int64_t)N + 1, tc1 = N1 - pa.W;
  if (nh + nl > N1) return;
  const int nck = (ph + pl + kScorePages - 1) / kScorePages, ncs = (L + kScorePages - 1) / kScorePages;
  Cand bh{0.0f, kNoPos, 0}, bl{0.0f, kNoPos, 0};
  int tcs = -1;
  float tcsum = 0.0f;
  for (int k = lane; k < nck; k += 64) {
    const int32_t* cp = cand + (u * ncs + k) * kCandWords;
    bh = min_imp(bh, Cand{__int_as_float(cp[0]), cp[1], cp[2]}, N1);
    bl = min_imp(bl, Cand{__int_as_float(cp[3]), cp[4], cp[5]}, N1);
    if (cp[6] >= 0) {
      tcs = cp[6];
      tcsum = __int_as_float(cp[7]);
    }
  }
  bh = wave_argmin(bh, N1);
  bl = wave_argmin(bl, N1);
  const uint64_t has = __ballot(tcs >= 0);
  if (has) {
    const int src = (int)__builtin_ctzll(has);
    tcs = __shfl(tcs, src, 64);
    tcsum = __shfl(tcsum, src, 64);
  }
  if (tc1 >= 0 && tcs < 0) return;  // the plan kernel would not accept the state
  const int32_t id0 = row[0];
  if (id0 < 0 || id0 >= P) return;
  const Plan pn = plan_decide(N1, pa.W, pa.S_max, pa.lo_en, pa_ah(pa, (int)(u % H)), pa_al(pa, (int)(u % H)), nh, nl,
                              ph, pl, L, tcs,
                              tcsum, bh, bl);
  uint32_t rw[kRecWords];
  plan_rec_fill(rw, N1, nh, nl, ph, pl, pn);
  uint32_t wv = rw[0];
#pragma unroll
  for (int k = 1; k < kRecWords; k++) wv = lane == k ? rw[k] : wv;
  uint32_t* dst = (uint32_t*)(pages + (int64_t)id0 * page_bytes + plan_rec_off<D>());
  if (lane < kRecWords) dst[lane] = wv;
}

hipError_t launch_scores(const Cfg& c, const Pool& p, int batch, const int32_t* table, const int32_t* state,
                         const int32_t* seq_len, void* ws, hipStream_t s) {
  return launch_scores_merge(c, p, batch, table, state, seq_len, ws, s, 0, nullptr);
}

// merge_S > 0: the split partials of the attention just run (S = merge_S)
// are merged into out by the score kernel itself
hipError_t launch_scores_merge(const Cfg& c, const Pool& p, int batch, const int32_t* table, const int32_t* state,
                               const int32_t* seq_len, void* ws, hipStream_t s, int merge_S, float* out) {
  if (c.plain) return launch_scores_plain(c, p, batch, table, state, seq_len, ws, s);
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  AttnWs w = attn_carve(c, batch, true, ws, nullptr);
  const dim3 grid((unsigned)((c.L + kScorePages - 1) / kScorePages), (unsigned)U), block(256);
  const PolicyArgs pa{c.W, c.S_max, c.lo_en, c.ah, c.al, c.ah_head, c.al_head};
  const int GS = logit_stride(c.G);
  const bool merge = merge_S > 0;
#define DKV_SCORE(D, GB)                                                                                          \
  if (merge)                                                                                                      \
    score_kernel<D, GB, true><<<grid, block, 0, s>>>(c.H, c.G, c.L, p.P, p.page_bytes, c.W, table, state, seq_len, \
                                                     w.ml, w.logits, p.pages, w.cand, merge_S, w.part, out);     \
  else                                                                                                            \
    score_kernel<D, GB, false><<<grid, block, 0, s>>>(c.H, c.G, c.L, p.P, p.page_bytes, c.W, table, state,        \
                                                      seq_len, w.ml, w.logits, p.pages, w.cand, 0, nullptr,     \
                                                      nullptr)
#define DKV_SCORE_D(D)                  \
  if (GS == 4) DKV_SCORE(D, 4);         \
  else if (GS == 8) DKV_SCORE(D, 8);    \
  else DKV_SCORE(D, 16);
  if (c.d == 128) {
    DKV_SCORE_D(128)
    score_finish_kernel<128><<<dim3((unsigned)U), dim3(64), 0, s>>>(c.H, c.G, c.L, p.P, p.page_bytes, pa, table,
                                                                    state, seq_len, w.ml, w.cand, p.pages);
  } else {
    DKV_SCORE_D(64)
    score_finish_kernel<64><<<dim3((unsigned)U), dim3(64), 0, s>>>(c.H, c.G, c.L, p.P, p.page_bytes, pa, table,
                                                                   state, seq_len, w.ml, w.cand, p.pages);
  }
#undef DKV_SCORE_D
#undef DKV_SCORE
  return hipGetLastError();
}

// Dispatch order when there are more workgroups than compute units (one
// resident attention workgroup per compute unit): the
// hardware starts workgroups in index order as compute units free up, so
// handing out the units with the most pages first keeps a long unit from
// starting last (list scheduling, longest first).  A counting sort of the
// units on ph + pl (capped); the order among equal keys is whatever the LDS
// atomics give, which changes timing only: every unit still runs in exactly
// one workgroup and computes the same result.
constexpr int kOrderKeys = 4096;
constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads) void unit_order_kernel(int64_t U, const int32_t* __restrict__ state,
                                                                 int32_t* __restrict__ order) {
  __shared__ int32_t cnt[kOrderKeys];
  __shared__ int32_t wsum[kOrderThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // bucket kOrderKeys - 1 - pages: the largest page counts first
  auto bucket = [&](int64_t u) -> int {
    const int64_t n = (int64_t)state[4 * u + 2] + state[4 * u + 3];
    return kOrderKeys - 1 - (int)(n < 0 ? 0 : (n >= kOrderKeys ? kOrderKeys - 1 : n));
  };
  for (int k = tid; k < kOrderKeys; k += kOrderThreads) cnt[k] = 0;
  __syncthreads();
  for (int64_t u = tid; u < U; u += kOrderThreads) atomicAdd(&cnt[bucket(u)], 1);
  __syncthreads();
  // exclusive prefix sum over the buckets, kOrderKeys / kOrderThreads per thread
  constexpr int KPT = kOrderKeys / kOrderThreads;
  int v[KPT], sum = 0;
#pragma unroll
  for (int e = 0; e < KPT; e++) {
    v[e] = cnt[KPT * tid + e];
    sum += v[e];
  }
  int x = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  int ex = x - sum;
  for (int w = 0; w < wid; w++) ex += wsum[w];
#pragma unroll
  for (int e = 0; e < KPT; e++) {
    cnt[KPT * tid + e] = ex;
    ex += v[e];
  }
  __syncthreads();
  for (int64_t u = tid; u < U; u += kOrderThreads) order[atomicAdd(&cnt[bucket(u)], 1)] = (int32_t)u;
}

static int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

// the order array to pass (and its kernel launched) or null: with more
// workgroups than compute units; with several splits the units' workgroups
// stay adjacent (split index fastest), a long unit's all early.  reuse: the
// workspace already holds an order for these units (a chained decode step:
// the previous call of the chain wrote it; page counts move by at most one
// page per unit and step, and the order only affects timing).
static const int32_t* launch_order(int S, int64_t U, const int32_t* state, const AttnWs& w, hipStream_t s,
                                   bool reuse = false) {
  const int cus = device_cus();
  if (cus <= 0 || U * S <= cus) return nullptr;
  if (!reuse) unit_order_kernel<<<dim3(1), dim3(kOrderThreads), 0, s>>>(U, state, w.order);
  return w.order;
}

// a chain recomputes the dispatch order at its start and every this many steps
constexpr int kOrderRefresh = 16;

hipError_t launch_attn(const Cfg& c, const Pool& p, int batch, const uint16_t* q, const int32_t* table,
                       const int32_t* state, const int32_t* seq_len, float* out, int mode, void* ws,
                       hipStream_t s, bool reuse_order) {
  if (c.plain) return launch_attn_plain(c, p, batch, q, table, state, seq_len, out, mode, ws, s);
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const int S = attn_splits(c, batch);
  AttnWs w = attn_carve(c, batch, mode != 0, ws, nullptr);
  const float scale_log2 = (1.0f / sqrtf((float)c.d)) * kLog2e;
  const dim3 grid(S, (unsigned)U), block(kThreads);
  // a single split runs the score update inside the attention workgroup
  const int kmode = mode == 1 && S > 1 ? 2 : mode;
  // G rounded up to 4, 8 or 16 (the kernel's softmax layout)
  const int gp = c.G <= 4 ? 4 : (c.G <= 8 ? 8 : 16);
  const PolicyArgs pa{c.W, c.S_max, c.lo_en, c.ah, c.al, c.ah_head, c.al_head};
  const StepArgs none{};
  const int32_t* order = launch_order(S, U, state, w, s, reuse_order);
#define DKV_ATTN(D, M, GPV)                                                                                \
  attn_kernel<D, M, GPV, false><<<grid, block, 0, s>>>(c.H, c.G, c.L, S, p.P, p.page_bytes, pa, scale_log2, q, \
                                                      table, state, seq_len, p.pages, out, w.part, w.ml,      \
                                                      w.logits, p.status, none, order)
#define DKV_ATTN_G(D, GPV)                     \
  if (kmode == 0) DKV_ATTN(D, 0, GPV);         \
  else if (kmode == 1) DKV_ATTN(D, 1, GPV);    \
  else DKV_ATTN(D, 2, GPV);
#define DKV_ATTN_D(D)                          \
  if (gp == 4) {                               \
    DKV_ATTN_G(D, 4)                           \
  } else if (gp == 8) {                        \
    DKV_ATTN_G(D, 8)                           \
  } else {                                     \
    DKV_ATTN_G(D, 16)                          \
  }
  if (c.d == 128) {
    DKV_ATTN_D(128)
  } else {
    DKV_ATTN_D(64)
  }
#undef DKV_ATTN_D
#undef DKV_ATTN_G
#undef DKV_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (S > 1) {
    // with the score update the score kernel merges the splits itself
    if (mode == 1) return launch_scores_merge(c, p, batch, table, state, seq_len, ws, s, S, out);
    return launch_attn_merge(c, batch, S, seq_len, w.part, out, w.ml, mode != 0, s);
  }
  return hipSuccess;
}

hipError_t launch_attn_merge(const Cfg& c, int batch, int S, const int32_t* seq_len, const float* part, float* out,
                             float* ml, bool save, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const dim3 grid((unsigned)c.G, (unsigned)U), block(256);
  if (c.d == 128)
    attn_merge_kernel<128><<<grid, block, 0, s>>>(c.H, c.G, S, seq_len, part, out, ml, save ? 1 : 0);
  else
    attn_merge_kernel<64><<<grid, block, 0, s>>>(c.H, c.G, S, seq_len, part, out, ml, save ? 1 : 0);
  return hipGetLastError();
}

// With one split per unit the step's commit runs inside the attention
// workgroup (plan kernel, then one kernel); otherwise, and when the score
// update is deferred (mode 2: the logits go to the workspace for a later
// diffkv_update_scores), plan, commit and attention kernels in turn.
hipError_t launch_decode_step(const Cfg& c, const Pool& p, int batch, const int32_t* seq_len, const uint16_t* k,
                              const uint16_t* v, const uint16_t* q, int32_t* table, int32_t* state, float* out,
                              int mode, int chain, void* ws_step, void* ws_attn, void* ws_next, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const int S = attn_splits(c, batch);
  if (S != 1 || mode == 2 || c.plain) {
    hipError_t e = launch_step(c, p, batch, seq_len, k, v, table, state, ws_step, s);
    if (e != hipSuccess) return e;
    // a chained call (same workspace, nothing else writing it) keeps the
    // chain's dispatch order, recomputed every kOrderRefresh calls
    return launch_attn(c, p, batch, q, table, state, seq_len, out, mode, ws_attn, s,
                       !c.plain && chain > 0 && chain % kOrderRefresh != 0);
  }
  const bool direct = U <= kDirectUnits;
  // chained steps: the attention with the score update plans the next step
  // into the other slot; a chained call reads slot (chain & 1) and runs no
  // plan kernel
  const bool can_chain = direct && mode == 1;
  const bool chained = can_chain && chain > 0;
  void* cur = chained && (chain & 1) ? ws_next : ws_step;
  void* nxt = cur == ws_step ? ws_next : ws_step;
  hipError_t e;
  if (!chained) {
    e = launch_step_plan(c, p, batch, seq_len, table, state, ws_step, s);
    if (e != hipSuccess) return e;
    if (!direct) {
      e = launch_step_coord(c, p, batch, ws_step, s);
      if (e != hipSuccess) return e;
    }
  }
  const StepWs sw = step_carve(c, batch, cur), sn = step_carve(c, batch, nxt);
  AttnWs w = attn_carve(c, batch, mode != 0, ws_attn, nullptr);
  const float scale_log2 = (1.0f / sqrtf((float)c.d)) * kLog2e;
  const dim3 grid(1, (unsigned)U), block(kThreads);
  const int gp = c.G <= 4 ? 4 : (c.G <= 8 ? 8 : 16);
  const PolicyArgs pa{c.W, c.S_max, c.lo_en, c.ah, c.al, c.ah_head, c.al_head};
  const StepArgs sa{k,
                    v,
                    sw.hdr,
                    sw.rec,
                    sw.nf,
                    p.list,
                    table,
                    state,
                    p.ptr,
                    U,
                    direct ? 1 : 0,
                    chained ? 1 : 0,
                    sw.cw,
                    can_chain ? sn.hdr : nullptr,
                    can_chain ? sn.rec : nullptr,
                    can_chain ? sn.nf : nullptr,
                    can_chain ? sn.cw : nullptr};
  const int32_t* order = launch_order(1, U, state, w, s, chained && chain % kOrderRefresh != 0);
#define DKV_STEP(D, M, GPV)                                                                               \
  attn_kernel<D, M, GPV, true><<<grid, block, 0, s>>>(c.H, c.G, c.L, 1, p.P, p.page_bytes, pa, scale_log2, q, \
                                                     table, state, seq_len, p.pages, out, w.part, w.ml,      \
                                                     w.logits, p.status, sa, order)
#define DKV_STEP_G(D, GPV)                      \
  if (mode == 0) DKV_STEP(D, 0, GPV);           \
  else DKV_STEP(D, 1, GPV);
#define DKV_STEP_D(D)                           \
  if (gp == 4) {                                \
    DKV_STEP_G(D, 4)                            \
  } else if (gp == 8) {                         \
    DKV_STEP_G(D, 8)                            \
  } else {                                      \
    DKV_STEP_G(D, 16)                           \
  }
  if (c.d == 128) {
    DKV_STEP_D(128)
  } else {
    DKV_STEP_D(64)
  }
#undef DKV_STEP_D
#undef DKV_STEP_G
#undef DKV_STEP
  return hipGetLastError();
}

}  // namespace dkv
