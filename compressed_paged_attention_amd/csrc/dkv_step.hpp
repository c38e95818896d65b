// dkv_step.hpp -- generation-step commit of one unit: by a workgroup (the
// step commit kernel) or by one wave of the attention workgroup (the decode
// step), with the plan and plan-record helpers both use.
//
// Step workspace: a header (pointer snapshot, commit flag), per-unit plan
// records and one demand word per unit (see step.hip for the plan).
#pragma once

#include "dkv_common.hpp"
#include "dkv_launch.hpp"

namespace dkv {

// Per-unit plan record and a compact demand word per unit:
//   nf[u] = need tier (bits 0-1: 0 none, 1 low, 2 high) | kActive | status flags << 8
// The record also carries the ids of the pages the commit reads (the high
// page of slot new_hi, the low page of slot lo_slot, the high page of
// lo_src, the first high page), so the commit needs no table lookup.
constexpr int kSRec = 12;
enum { S_NEWHI = 0, S_HIAPP, S_LOSRC, S_LOSLOT, S_LOAPP, S_PAGE, S_IDH, S_IDL, S_IDS, S_IDF };
// K precision levels: the level-0 slot of the new token, the appends per
// level (bit l), the level of a new page (-1 none), the page (S_PAGE, as in
// the two-tier record) and two token moves {on, source level, slot,
// destination level, slot}: t_c or a level-0 victim leaving level 0, and a
// victim of t_c's level moving further down.
constexpr int kLRec = 16;
enum { LS_NEW = 0, LS_APP, LS_NEED, LS_MV0 = 6, LS_MV1 = 11 };
static_assert(S_PAGE == 5, "the level record keeps the page where the coordination kernel writes it");
inline int rec_words(const Cfg& c) { return c.K >= 3 ? kLRec : kSRec; }
enum { SH_COMMIT = 0, SH_START, SH_END, SH_D };
constexpr int32_t kActive = 4;
// Up to this many units every commit workgroup redoes the unit-order prefix
// sum over the demand words itself (no coordination kernel in between).
constexpr int64_t kDirectUnits = 2048;

// One step workspace (slot): pointer snapshot, per-unit records and demand
// words, and per-unit chain words (see kChainWords).
struct StepWs {
  int64_t* hdr;
  int32_t* rec;
  int32_t* nf;
  int32_t* cw;
};

inline StepWs step_carve(const Cfg& c, int batch, void* ws) {
  const size_t U = (size_t)batch * c.H;
  uint8_t* p = (uint8_t*)ws;
  StepWs w;
  w.hdr = (int64_t*)p;
  p += align_up(16 * sizeof(int64_t), 256);
  w.rec = (int32_t*)p;
  p += align_up(U * rec_words(c) * sizeof(int32_t), 256);
  w.nf = (int32_t*)p;
  p += align_up(U * sizeof(int32_t), 256);
  w.cw = (int32_t*)p;
  return w;
}

// Chained decode steps: a step whose attention updates every score sum of a
// unit also plans the unit's next step (length N + 1, the tier state after
// this step's commit) and leaves record, demand word and these chain words
// in the other workspace slot, so the next step needs no plan kernel:
//   {N the plan is for (-1: no plan), nh, nl, ph, pl, demand word, hi_app, lo_app}
// The consumer checks every active unit's words against its length and tier
// state (a tier state word may also read as its value after the unit's own
// commit in the same launch).
constexpr int kChainWords = 8;

// ---------------------------------------------------------------------------
// commit: phase 1 loads everything the unit needs, phase 2 quantizes and
// edits LDS images of the destination pages, phase 3 stores.  No barrier
// waits on an outstanding global store.
// ---------------------------------------------------------------------------

// LDS field update (other fields of the word may be edited concurrently)
__device__ inline void lds_put(uint32_t* img, int byte, int shift, int bits, uint32_t val) {
  const int sh = 8 * (byte & 3) + shift;
  const uint32_t mask = ((1u << bits) - 1u) << sh;
  atomicAnd(&img[byte >> 2], ~mask);
  atomicOr(&img[byte >> 2], (val << sh) & mask);
}

// One token written into one page through an LDS image of that page.
struct TokWrite {
  bool on;     // this token is written
  bool hi;     // destination tier
  bool fresh;  // the page is new: the whole page is written (zeros elsewhere)
  int idx;     // slot inside the page
  int32_t id;  // page id
};

// Phase 1: a fresh page's image is zeroed; an existing page's image gets the
// V segment (the only one shared between tokens at byte level) and a zeroed
// K range for the token.
template <int D>
__device__ void img_load(uint32_t* img, const TokWrite& t, const uint8_t* pages, int page_bytes) {
  if (!t.on) return;
  const Seg sg = tier_seg(D, t.hi);
  if (t.fresh) {
    for (int w = threadIdx.x; w < page_bytes / 4; w += blockDim.x) img[w] = 0u;
  } else {
    const uint4* src = (const uint4*)(pages + (int64_t)t.id * page_bytes + sg.vc);
    uint4* dst = (uint4*)(img + sg.vc / 4);
    for (int c = threadIdx.x; c < (sg.vm - sg.vc) / 16; c += blockDim.x) dst[c] = src[c];
    const int kb = t.idx * D * sg.kbits / 8;
    for (int w = threadIdx.x; w < D * sg.kbits / 32; w += blockDim.x) img[kb / 4 + w] = 0u;
  }
}

// Phase 2: the token's codes (dim threadIdx.x < D), metadata, score, position.
template <int D>
__device__ void img_token(uint32_t* img, const TokWrite& t, uint32_t ck, uint32_t cv, uint32_t kmeta,
                          uint32_t vmeta, float score, int32_t pos) {
  if (!t.on) return;
  const Seg sg = tier_seg(D, t.hi);
  if (threadIdx.x < D) {
    int byte, shift;
    k_field(D, t.hi, t.idx, threadIdx.x, byte, shift);
    lds_put(img, byte, shift, sg.kbits, ck);
    v_field(D, t.hi, t.idx, threadIdx.x, byte, shift);
    lds_put(img, byte, shift, sg.vbits, cv);
  }
  if (threadIdx.x == 0) {
    img[sg.km / 4 + t.idx] = kmeta;
    img[sg.vm / 4 + t.idx] = vmeta;
    img[sg.sc / 4 + t.idx] = __float_as_uint(score);
    img[sg.ps / 4 + t.idx] = (uint32_t)pos;
  }
}

// Phase 3: a fresh page is written whole; otherwise the token's K range, the
// V segment and the token's four words.
template <int D>
__device__ void img_store(const uint32_t* img, const TokWrite& t, uint8_t* pages, int page_bytes) {
  if (!t.on) return;
  const Seg sg = tier_seg(D, t.hi);
  uint8_t* pg = pages + (int64_t)t.id * page_bytes;
  if (t.fresh) {
    for (int c = threadIdx.x; c < page_bytes / 16; c += blockDim.x) ((uint4*)pg)[c] = ((const uint4*)img)[c];
    return;
  }
  const int kb = t.idx * D * sg.kbits / 8, kn = D * sg.kbits / 128;  // 16-byte chunks
  const int vn = (sg.vm - sg.vc) / 16;
  for (int c = threadIdx.x; c < kn + vn + 4; c += blockDim.x) {
    if (c < kn) {
      ((uint4*)(pg + kb))[c] = ((const uint4*)(img + kb / 4))[c];
    } else if (c < kn + vn) {
      ((uint4*)(pg + sg.vc))[c - kn] = ((const uint4*)(img + sg.vc / 4))[c - kn];
    } else {
      const int seg = c - kn - vn;
      const int off = (seg == 0 ? sg.km : seg == 1 ? sg.vm : seg == 2 ? sg.sc : sg.ps) + 4 * t.idx;
      *(uint32_t*)(pg + off) = img[off / 4];
    }
  }
}

// The same three phases for the plain layout of a tier codec variant: a
// token's K and V codes are whole, 8-byte aligned byte ranges of their own
// (t d b / 8 bytes in, d b / 8 long), so an existing page needs no load:
// the token's ranges are zeroed in the image, edited and stored with its
// four words.
__device__ inline void img_load_plain(uint32_t* img, const TokWrite& t, const Lay& lay, int page_bytes) {
  if (!t.on) return;
  const Seg& sg = lay.seg(t.hi);
  if (t.fresh) {
    for (int w = threadIdx.x; w < page_bytes / 4; w += blockDim.x) img[w] = 0u;
  } else {
    const int kw = lay.d * sg.kbits / 32, vw = lay.d * sg.vbits / 32;  // words per token
    for (int w = threadIdx.x; w < kw + vw; w += blockDim.x)
      img[w < kw ? (sg.kc / 4 + t.idx * kw + w) : (sg.vc / 4 + t.idx * vw + (w - kw))] = 0u;
  }
}

__device__ inline void img_token_plain(uint32_t* img, const TokWrite& t, const Lay& lay, uint32_t ck, uint32_t cv,
                                       uint32_t kmeta, uint32_t vmeta, float score, int32_t pos) {
  if (!t.on) return;
  const Seg& sg = lay.seg(t.hi);
  if (threadIdx.x < lay.d) {
    int byte, shift;
    lay.kf(t.hi, t.idx, threadIdx.x, byte, shift);
    lds_put(img, byte, shift, sg.kbits, ck);
    lay.vf(t.hi, t.idx, threadIdx.x, byte, shift);
    lds_put(img, byte, shift, sg.vbits, cv);
  }
  if (threadIdx.x == 0) {
    img[sg.km / 4 + t.idx] = kmeta;
    img[sg.vm / 4 + t.idx] = vmeta;
    img[sg.sc / 4 + t.idx] = __float_as_uint(score);
    img[sg.ps / 4 + t.idx] = (uint32_t)pos;
  }
}

__device__ inline void img_store_plain(const uint32_t* img, const TokWrite& t, const Lay& lay, uint8_t* pages,
                                       int page_bytes) {
  if (!t.on) return;
  const Seg& sg = lay.seg(t.hi);
  uint8_t* pg = pages + (int64_t)t.id * page_bytes;
  if (t.fresh) {
    for (int c = threadIdx.x; c < page_bytes / 16; c += blockDim.x) ((uint4*)pg)[c] = ((const uint4*)img)[c];
    return;
  }
  const int kw = lay.d * sg.kbits / 32, vw = lay.d * sg.vbits / 32;
  for (int w = threadIdx.x; w < kw + vw + 4; w += blockDim.x) {
    int off;  // word index
    if (w < kw) off = sg.kc / 4 + t.idx * kw + w;
    else if (w < kw + vw) off = sg.vc / 4 + t.idx * vw + (w - kw);
    else {
      const int seg = w - kw - vw;
      off = (seg == 0 ? sg.km : seg == 1 ? sg.vm : seg == 2 ? sg.sc : sg.ps) / 4 + t.idx;
    }
    ((uint32_t*)pg)[off] = img[off];
  }
}

// min and max of the D values held by threads 0..D-1, for n vectors at once
template <int D, int NV>
__device__ void block_minmax(float (&mn)[NV], float (&mx)[NV], float* red) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  constexpr int nw = (D + 63) / 64;
#pragma unroll
  for (int v = 0; v < NV; v++) {
    if (tid >= D) {
      mn[v] = INFINITY;
      mx[v] = -INFINITY;
    }
    mn[v] = wave_min(mn[v]);
    mx[v] = wave_max(mx[v]);
  }
  if (lane == 0 && wid < nw) {
#pragma unroll
    for (int v = 0; v < NV; v++) {
      red[(2 * v) * nw + wid] = mn[v];
      red[(2 * v + 1) * nw + wid] = mx[v];
    }
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < NV; v++) {
    mn[v] = red[(2 * v) * nw];
    mx[v] = red[(2 * v + 1) * nw];
    for (int w = 1; w < nw; w++) {
      mn[v] = fminf(mn[v], red[(2 * v) * nw + w]);
      mx[v] = fmaxf(mx[v], red[(2 * v + 1) * nw + w]);
    }
  }
}

// A candidate token: running score sum, position, slot; pos == kNoPos: none.
// Its observation count is N - 1 - pos.
constexpr int32_t kNoPos = 0x7FFFFFFF;
struct Cand {
  float sum;
  int32_t pos, slot;
};

// Strictly less important: sum_a * cnt_b < sum_b * cnt_a (exact in fp64),
// ties to the smaller position.
// Counts are below 2^29 (max_seq_len), so both products are exact.  Written
// without branches: it sits on the critical path of every reduction.
__device__ inline bool less_imp(const Cand& a, const Cand& b, int64_t N) {
  const int32_t n1 = (int32_t)(N - 1);
  const double l = (double)a.sum * (double)(n1 - b.pos), r = (double)b.sum * (double)(n1 - a.pos);
  const bool lt = (l < r) | ((l == r) & (a.pos < b.pos));
  return (a.pos != kNoPos) & ((b.pos == kNoPos) | lt);
}

__device__ inline Cand min_imp(const Cand& a, const Cand& b, int64_t N) { return less_imp(b, a, N) ? b : a; }

template <int LVL>
__device__ inline void argmin_step(Cand& c, int64_t N) {
  const Cand t{lane_xchg_t<LVL>(c.sum), lane_xchg_t<LVL>(c.pos), lane_xchg_t<LVL>(c.slot)};
  c = min_imp(c, t, N);
}

__device__ inline Cand wave_argmin(Cand c, int64_t N) {
  argmin_step<0>(c, N);
  argmin_step<1>(c, N);
  argmin_step<2>(c, N);
  argmin_step<3>(c, N);
  argmin_step<4>(c, N);
  argmin_step<5>(c, N);
  return c;
}

__device__ inline int classify_mean(float sum, int64_t cnt, int64_t Np, int lo_en, double ah, double al) {
  const double x = (double)sum * (double)Np;
  const double ch = ah * (double)cnt, cl = al * (double)cnt;
  if (lo_en) {
    if (x > ch) return kTierHi;
    return x >= cl ? kTierLo : kTierPrune;
  }
  return x >= cl ? kTierHi : kTierPrune;
}

// The step's decision for one unit (DiffKV notes, "KV compression policy",
// generation phase), from t_c (slot tcs, sum tcsum; tcs < 0: none, N < W),
// the least important non-window high token bh and low token bl, at length N
// (the new token's position; thresholds use N + 1).
struct Plan {
  int32_t new_hi, hi_app, lo_src, lo_slot, lo_app;
  int32_t nfw;  // demand word: need tier | kActive | status flags << 8
};

__device__ inline Plan plan_decide(int64_t N, int W, int S_max, int lo_en, double dah, double dal, int nh, int nl,
                                   int ph, int pl, int L, int tcs, float tcsum, const Cand& bh, const Cand& bl) {
  Plan r{nh, 1, -1, 0, 0, kActive};
  if (N + 1 > S_max) {
    r.nfw = kActive | (int32_t)(kStOverflow << 8);
    return r;
  }
  const int64_t Np = N + 1, tc_pos = N - W;
  if (tc_pos >= 0) {
    const int cls = classify_mean(tcsum, W - 1, Np, lo_en, dah, dal);
    if (cls == kTierHi) {
      const int vcls = classify_mean(bh.sum, N - 1 - bh.pos, Np, lo_en, dah, dal);
      if (vcls == kTierLo) {
        r.lo_src = bh.slot;
        r.lo_slot = nl;
        r.lo_app = 1;
        r.new_hi = bh.slot;
        r.hi_app = 0;
      } else if (vcls == kTierPrune) {
        r.new_hi = bh.slot;
        r.hi_app = 0;
      }
    } else if (cls == kTierLo) {
      // t_c moves to the low tier; the least important low token, t_c
      // included, is pruned below alpha_l / N'
      r.lo_src = tcs;
      r.new_hi = tcs;
      r.hi_app = 0;
      const Cand tcc{tcsum, (int32_t)tc_pos, -1};
      const Cand lv = less_imp(tcc, bl, N) ? tcc : bl;
      if (lv.slot >= 0 && classify_mean(lv.sum, N - 1 - lv.pos, Np, lo_en, dah, dal) == kTierPrune) {
        r.lo_slot = lv.slot;
        r.lo_app = 0;
      } else {
        r.lo_slot = nl;
        r.lo_app = 1;
      }
    } else {
      r.new_hi = tcs;
      r.hi_app = 0;
    }
  }
  int need = 0;
  if (r.hi_app && nh % kHiTokens == 0) need = kTierHi;
  if (r.lo_app && nl % kLoTokens == 0) need = kTierLo;
  const uint32_t fl = (need && ph + pl + 1 > L) ? kStOverflow : 0u;
  r.nfw = kActive | (fl ? 0 : need) | (int32_t)(fl << 8);
  return r;
}

// The step workspace's record of unit u: the plan and the page ids it
// names (row: the unit's table row, any readable copy; indices clamped into
// it, as a unit without a commit reads but does not use some entry).
template <typename RowAt>
__device__ inline void step_rec_put(int32_t* R, int32_t* nfu, const Plan& x, int L, RowAt row_at) {
  auto cl = [&](int t) { return min(max(t, 0), L - 1); };
  R[S_NEWHI] = x.new_hi;
  R[S_HIAPP] = x.hi_app;
  R[S_LOSRC] = x.lo_src;
  R[S_LOSLOT] = x.lo_slot;
  R[S_LOAPP] = x.lo_app;
  R[S_PAGE] = -1;
  R[S_IDH] = row_at(cl(x.new_hi >> 4));
  R[S_IDL] = row_at(cl(L - 1 - (x.lo_slot >> 5)));
  R[S_IDS] = row_at(cl(x.lo_src >> 4));
  R[S_IDF] = row_at(0);
  *nfu = x.nfw;
}

// Plan record of the next step, kept in the spare bytes after the last
// segment of a unit's first high page (table entry 0): written by a
// workgroup that has just updated all of the unit's score sums, read by the
// next step's plan kernel instead of a scan, and invalidated by every other
// write to the unit's slots or scores (zeroed magic).  Prompt pages start
// with these bytes zero.
constexpr uint32_t kPlanMagic = 0x4E414C50u;
constexpr int kRecWords = 13;  // magic, seq, nh, nl, ph, pl, 5 plan fields, demand word, check
template <int D>
constexpr int plan_rec_off() {
  return tier_seg(D, true).bytes;
}
static_assert(page_bytes_for(64) - tier_seg(64, true).bytes >= 4 * kRecWords, "plan record space");
static_assert(page_bytes_for(128) - tier_seg(128, true).bytes >= 4 * kRecWords, "plan record space");

// integrity word over the first 12 words (rotate-xor: no multiplies on the
// single-lane tail that writes a record)
__device__ inline uint32_t plan_rec_hash(const uint32_t* w) {
  uint32_t x = 0x9E3779B9u;
#pragma unroll
  for (int k = 0; k < 12; k++) x = __builtin_rotateleft32(x, 7) ^ (w[k] + (uint32_t)k);
  return ~x;
}

__device__ inline void plan_rec_fill(uint32_t* w, int64_t seq, int nh, int nl, int ph, int pl, const Plan& p) {
  w[0] = kPlanMagic;
  w[1] = (uint32_t)seq;
  w[2] = (uint32_t)nh;
  w[3] = (uint32_t)nl;
  w[4] = (uint32_t)ph;
  w[5] = (uint32_t)pl;
  w[6] = (uint32_t)p.new_hi;
  w[7] = (uint32_t)p.hi_app;
  w[8] = (uint32_t)p.lo_src;
  w[9] = (uint32_t)p.lo_slot;
  w[10] = (uint32_t)p.lo_app;
  w[11] = (uint32_t)p.nfw;
  w[12] = plan_rec_hash(w);
}

// true when the record is intact and was made for this length and state
__device__ inline bool plan_rec_check(const uint32_t* w, int64_t seq, int nh, int nl, int ph, int pl, Plan& p) {
  if (w[0] != kPlanMagic || plan_rec_hash(w) != w[12] || w[1] != (uint32_t)seq || w[2] != (uint32_t)nh ||
      w[3] != (uint32_t)nl || w[4] != (uint32_t)ph || w[5] != (uint32_t)pl)
    return false;
  p = Plan{(int32_t)w[6], (int32_t)w[7], (int32_t)w[8], (int32_t)w[9], (int32_t)w[10], (int32_t)w[11]};
  return true;
}

// LDS scratch of commit_unit, in 32-bit words: two page images plus misc.
template <int D, bool PLAIN = false>
constexpr int commit_lds_words() {
  return 2 * ((PLAIN ? plain_page_max(D) : page_bytes_for(D)) / 4) + 64;
}

// Result of commit_unit: whether this unit's step was committed, and its
// tier state afterwards (as written to tier_state).
struct UnitState {
  bool committed;
  int nh, nl, ph, pl;
  int new_tix;   // table index of a page this step added (-1: none)
  int new_page;  // its id
};

// The commit of unit u (one workgroup, any size >= D threads).  DIRECT: the
// workgroup recomputes the unit-order prefix sum of page demand from the
// demand words (all-or-nothing check included) and workgroup 0 advances the
// allocation pointer; otherwise the coordination kernel's result is read.
// `sm` is LDS scratch of commit_lds_words<D>() words, 16-byte aligned.
// PLAIN: the plain layout of a tier codec variant, described by `lay`
// (ignored otherwise); `sm` then holds commit_lds_words<D, true>() words.
template <int D, bool DIRECT, bool PLAIN = false>
__device__ UnitState commit_unit(int64_t u, int H, int L, int64_t U, int64_t P, int page_bytes,
                                 const int32_t* __restrict__ seq_len, const uint16_t* __restrict__ k_new,
                                 const uint16_t* __restrict__ v_new, const int64_t* __restrict__ hdr,
                                 const int32_t* __restrict__ rec, const int32_t* __restrict__ nf,
                                 const int32_t* __restrict__ list, int32_t* __restrict__ table,
                                 int32_t* __restrict__ state, uint8_t* pages, uint64_t* ptr, uint32_t* status,
                                 uint32_t* sm, const Lay& lay = Lay(D, false, Codec{8, 4, 4, 2})) {
  const Seg sh = PLAIN ? lay.seg(true) : tier_seg(D, true);
  constexpr int kPageWords = (PLAIN ? plain_page_max(D) : page_bytes_for(D)) / 4;
  const int tid = threadIdx.x;
  const int b = (int)u / H, h = (int)u % H;  // u < 2^31: 32-bit division
  const int32_t* s4c = state + 4 * u;
  UnitState res{false, s4c[0], s4c[1], s4c[2], s4c[3], -1, -1};
  // ---- phase 1: loads ----
  const int32_t wu = nf[u];
  const int32_t* R = rec + u * kSRec;
  int32_t* row = table + u * L;
  int32_t* s4 = state + 4 * u;
  const int64_t rowi = ((int64_t)b * H + h) * D + tid;
  float xk_new = tid < D ? h2f(k_new[rowi]) : 0.0f;
  float xv_new = tid < D ? h2f(v_new[rowi]) : 0.0f;
  // the plan record and the page ids it names, read before any barrier
  // (indices clamped into the row: a unit without a record reads, but does
  // not use, some entry)
  const int nh = res.nh, nl = res.nl, ph = res.ph, pl = res.pl;
  const int new_hi = R[S_NEWHI], lo_src = R[S_LOSRC], lo_slot = R[S_LOSLOT];
  const int hi_app = R[S_HIAPP], lo_app = R[S_LOAPP];
  const int32_t id_hrow = R[S_IDH], id_lrow = R[S_IDL], id_src = R[S_IDS], id_first = R[S_IDF];
  int64_t start = 0, end = 0;
  if constexpr (DIRECT) {
    start = hdr[SH_START];
    end = hdr[SH_END];
  }
  int32_t page = -1;
  if constexpr (DIRECT) {
    int* lds = (int*)(sm + 2 * kPageWords);  // 16 ints
    int64_t& s_off = *(int64_t*)(lds + 16);
    uint32_t& s_fl = *(uint32_t*)(lds + 18);
    if (tid == 0) s_fl = 0;
    int64_t total = 0;
    uint32_t fl = 0;
    for (int64_t base = 0; base < U; base += blockDim.x) {
      const int64_t x = base + tid;
      const int32_t w = x < U ? nf[x] : 0;
      fl |= (uint32_t)w >> 8;
      int t;
      const int excl = block_excl_count((w & 3) != 0, lds, t);
      if (x == u) s_off = total + excl;
      total += t;
    }
    if (fl) atomicOr(&s_fl, fl);
    __syncthreads();
    uint32_t st = s_fl;
    if (!st && total > end - start) st = kStExhausted;
    if (u == 0 && tid == 0) {
      if (st) atomicOr(status, st);
      else ptr[0] = (uint64_t)(start + total);
    }
    if (st || !(wu & kActive)) return res;
    if (wu & 3) page = list[(uint64_t)(start + s_off) % (uint64_t)P];
  } else {
    if (!hdr[SH_COMMIT] || !(wu & kActive)) return res;
    page = R[S_PAGE];
  }
  const int need = wu & 3;
  if (need && (page < 0 || page >= P)) {
    if (tid == 0) atomicOr(status, kStBadState);
    return res;
  }
  // destinations: the new token's high slot; the requantized token's low slot
  TokWrite th{true, true, need == kTierHi, new_hi & 15, need == kTierHi ? page : id_hrow};
  TokWrite tl{lo_src >= 0, false, need == kTierLo, lo_slot & 31,
              lo_src < 0 ? 0 : (need == kTierLo ? page : id_lrow)};
  uint32_t* img_h = sm;
  uint32_t* img_l = sm + kPageWords;
  float* red = (float*)(sm + 2 * kPageWords + 20);  // 16 floats
  if constexpr (PLAIN) {
    img_load_plain(img_h, th, lay, page_bytes);
    img_load_plain(img_l, tl, lay, page_bytes);
  } else {
    img_load<D>(img_h, th, pages, page_bytes);
    img_load<D>(img_l, tl, pages, page_bytes);
  }
  // the requantized token's dequantized values (read before anything is
  // written: its high slot may be the new token's)
  float xk_rq = 0.0f, xv_rq = 0.0f, sc_rq = 0.0f;
  int32_t pos_rq = 0;
  if (tl.on) {
    const uint8_t* src = pages + (int64_t)id_src * page_bytes;
    const int si = lo_src & 15;
    const uint32_t km = *(const uint32_t*)(src + sh.km + 4 * si);
    const uint32_t vm = *(const uint32_t*)(src + sh.vm + 4 * si);
    sc_rq = *(const float*)(src + sh.sc + 4 * si);
    pos_rq = *(const int32_t*)(src + sh.ps + 4 * si);
    if (tid < D) {
      int byte, shift;
      if constexpr (PLAIN) {
        lay.kf(true, si, tid, byte, shift);
        xk_rq = dequant(h2f((uint16_t)km), h2f((uint16_t)(km >> 16)),
                        ((uint32_t)src[byte] >> shift) & ((1u << sh.kbits) - 1u));
        lay.vf(true, si, tid, byte, shift);
        xv_rq = dequant(h2f((uint16_t)vm), h2f((uint16_t)(vm >> 16)),
                        ((uint32_t)src[byte] >> shift) & ((1u << sh.vbits) - 1u));
      } else {
        k_field(D, true, si, tid, byte, shift);
        xk_rq = dequant(h2f((uint16_t)km), h2f((uint16_t)(km >> 16)), ((uint32_t)src[byte] >> shift) & 0xFFu);
        v_field(D, true, si, tid, byte, shift);
        xv_rq = dequant(h2f((uint16_t)vm), h2f((uint16_t)(vm >> 16)), ((uint32_t)src[byte] >> shift) & 0xFu);
      }
    }
  }
  const int32_t N = seq_len[b];
  __syncthreads();  // LDS images loaded (no global store is outstanding)
  // ---- phase 2: quantize, edit the images ----
  float mn[4] = {xk_new, xv_new, xk_rq, xv_rq}, mx[4] = {xk_new, xv_new, xk_rq, xv_rq};
  block_minmax<D, 4>(mn, mx, red);
  auto token = [&](uint32_t* img, const TokWrite& t, float xk, float xv, int v, float score, int32_t pos) {
    const Seg sg = PLAIN ? lay.seg(t.hi) : tier_seg(D, t.hi);
    uint16_t ks16, kz16, vs16, vz16;
    float ks, kz, vs, vz;
    codec_params(mn[v], mx[v], sg.kbits, ks16, kz16, ks, kz);
    codec_params(mn[v + 1], mx[v + 1], sg.vbits, vs16, vz16, vs, vz);
    const uint32_t ck = codec_code(xk, ks, kz, sg.kbits), cv = codec_code(xv, vs, vz, sg.vbits);
    const uint32_t kmeta = (uint32_t)ks16 | ((uint32_t)kz16 << 16), vmeta = (uint32_t)vs16 | ((uint32_t)vz16 << 16);
    if constexpr (PLAIN) img_token_plain(img, t, lay, ck, cv, kmeta, vmeta, score, pos);
    else img_token<D>(img, t, ck, cv, kmeta, vmeta, score, pos);
  };
  token(img_h, th, xk_new, xv_new, 0, 0.0f, N);
  if (tl.on) token(img_l, tl, xk_rq, xv_rq, 2, sc_rq, pos_rq);
  __syncthreads();
  // ---- phase 3: stores ----
  if constexpr (PLAIN) {
    img_store_plain(img_h, th, lay, pages, page_bytes);
    img_store_plain(img_l, tl, lay, pages, page_bytes);
  } else {
    img_store<D>(img_h, th, pages, page_bytes);
    img_store<D>(img_l, tl, pages, page_bytes);
    // the unit changed: its plan record (first high page) no longer applies
    if (tid == 0 && ph >= 1 && id_first >= 0 && id_first < P)
      *(uint32_t*)(pages + (int64_t)id_first * page_bytes + plan_rec_off<D>()) = 0u;
  }
  res = UnitState{true, nh + hi_app, nl + lo_app, ph + (need == kTierHi), pl + (need == kTierLo),
                  need == kTierHi ? ph : (need == kTierLo ? L - 1 - pl : -1), page};
  if (tid == 0) {
    if (need == kTierHi) row[ph] = page;
    if (need == kTierLo) row[L - 1 - pl] = page;
    s4[0] = res.nh;
    s4[1] = res.nl;
    s4[2] = res.ph;
    s4[3] = res.pl;
  }
  return res;
}

// ---------------------------------------------------------------------------
// The step's commit inside the attention workgroup: every thread takes part
// in the verdict; one wave then commits while the others attend.
// ---------------------------------------------------------------------------

// All threads of the workgroup: status flags of any unit, the total page
// demand and the number of units before u that need a page, from the demand
// words in one pass (no barrier inside it); lds holds 3 ints per wave.
__device__ inline void step_verdict(int64_t u, int64_t U, const int32_t* nf, int* lds, uint32_t& flags, int& total,
                                    int& rank) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int tot = 0, rk = 0;
  uint32_t fl = 0;
#pragma unroll 4
  for (int64_t base = 0; base < U; base += blockDim.x) {
    const int64_t x = base + threadIdx.x;
    const int32_t w = x < U ? nf[x] : 0;
    fl |= (uint32_t)w >> 8;
    const bool need = (w & 3) != 0;
    tot += __popcll(__ballot(need));
    rk += __popcll(__ballot(need && x < u));
  }
  fl = wave_reduce(fl, [](uint32_t a, uint32_t b) { return a | b; });
  if (lane == 0) {
    lds[wid] = tot;
    lds[nw + wid] = rk;
    lds[2 * nw + wid] = (int)fl;
  }
  __syncthreads();
  total = 0;
  rank = 0;
  flags = 0;
  for (int w = 0; w < nw; w++) {
    total += lds[w];
    rank += lds[nw + w];
    flags |= (uint32_t)lds[2 * nw + w];
  }
}

// step_verdict over a chained slot: a unit whose batch slot is inactive
// (seq_len <= 0) demands nothing; an active unit whose chain words were not
// made for its length and tier state (the caller broke the chain) sets
// kStStale.  Other workgroups may commit while this one reads: each tier
// state word passes as its value before the step or after the unit's commit
// (a word may be read before its store and its neighbour after).
__device__ inline void step_verdict_chain(int64_t u, int64_t U, int H, const int32_t* cw, const int32_t* seq_len,
                                          const int32_t* state, int* lds, uint32_t& flags, int& total, int& rank) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int tot = 0, rk = 0;
  uint32_t fl = 0;
#pragma unroll 2
  for (int64_t base = 0; base < U; base += blockDim.x) {
    const int64_t x = base + threadIdx.x;
    const bool in = x < U;
    const int64_t xc = in ? x : 0;
    const int32_t N = seq_len[(int)xc / H];
    const int4 c0 = ((const int4*)cw)[2 * xc], c1 = ((const int4*)cw)[2 * xc + 1];
    const int32_t* s4 = state + 4 * xc;
    const int32_t snh = s4[0], snl = s4[1], sph = s4[2], spl = s4[3];
    int32_t w = c1.y;
    if (!in || N <= 0) {
      w = 0;
    } else {
      const int need = w & 3;
      const bool ok = c0.x == N && (snh == c0.y || snh == c0.y + c1.z) && (snl == c0.z || snl == c0.z + c1.w) &&
                      (sph == c0.w || sph == c0.w + (need == kTierHi)) &&
                      (spl == c1.x || spl == c1.x + (need == kTierLo));
      // a unit that fails the check contributes only the stale bit (its
      // words may be anything)
      if (!ok) {
        fl |= kStStale;
        w = 0;
      }
    }
    fl |= ((uint32_t)w >> 8) & kStAll;
    const bool need = (w & 3) != 0;
    tot += __popcll(__ballot(need));
    rk += __popcll(__ballot(need && x < u));
  }
  fl = wave_reduce(fl, [](uint32_t a, uint32_t b) { return a | b; });
  if (lane == 0) {
    lds[wid] = tot;
    lds[nw + wid] = rk;
    lds[2 * nw + wid] = (int)fl;
  }
  __syncthreads();
  total = 0;
  rank = 0;
  flags = 0;
  for (int w = 0; w < nw; w++) {
    total += lds[w];
    rank += lds[nw + w];
    flags |= (uint32_t)lds[2 * nw + w];
  }
}

// One unit's inputs to a chained verdict: its chain words, batch length and
// tier state (loads clamped into the arrays; chain_eval decides as
// step_verdict_chain does).
struct ChainIn {
  int4 c0, c1;
  int32_t N, snh, snl, sph, spl;
};

__device__ __forceinline__ ChainIn chain_load(int64_t x, int64_t U, int H, const int32_t* cw,
                                              const int32_t* seq_len, const int32_t* state) {
  const int64_t xc = x < U ? x : 0;
  ChainIn c;
  c.N = seq_len[(int)xc / H];
  c.c0 = ((const int4*)cw)[2 * xc];
  c.c1 = ((const int4*)cw)[2 * xc + 1];
  const int32_t* s4 = state + 4 * xc;
  c.snh = s4[0];
  c.snl = s4[1];
  c.sph = s4[2];
  c.spl = s4[3];
  return c;
}

// The unit's demand word (0 when out of range or inactive); when its chain
// words were not made for its length and tier state, kStStale into fl and 0
// (the words may be anything).
__device__ __forceinline__ int32_t chain_eval(const ChainIn& c, bool in, uint32_t& fl) {
  if (!in || c.N <= 0) return 0;
  const int32_t w = c.c1.y;
  const int need = w & 3;
  const bool ok = c.c0.x == c.N && (c.snh == c.c0.y || c.snh == c.c0.y + c.c1.z) &&
                  (c.snl == c.c0.z || c.snl == c.c0.z + c.c1.w) &&
                  (c.sph == c.c0.w || c.sph == c.c0.w + (need == kTierHi)) &&
                  (c.spl == c.c1.x || c.spl == c.c1.x + (need == kTierLo));
  if (!ok) {
    fl |= kStStale;
    return 0;
  }
  return w;
}

// The step verdict taken by one wave, for up to kWaveVerdictUnits units:
// load issues every unit's inputs at once (first thing in the kernel, so
// they do not queue behind the wave's page loads); eval reduces them with
// ballots to the status flags, the total page demand and the number of units
// before u that need a page.
constexpr int kWaveVerdictUnits = 256;
struct WaveVerdict {
  static constexpr int NC = kWaveVerdictUnits / 64;
  ChainIn c[NC];
  int32_t w[NC];

  __device__ __forceinline__ void load(bool chained, int64_t U, int H, const int32_t* nf, const int32_t* cw,
                                       const int32_t* seq_len, const int32_t* state) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < NC; k++) {
      const int64_t x = lane + 64 * k;
      if (chained) c[k] = chain_load(x, U, H, cw, seq_len, state);
      else w[k] = nf[x < U ? x : 0];
    }
  }

  __device__ __forceinline__ void eval(bool chained, int64_t u, int64_t U, uint32_t& flags, int& total,
                                       int& rank) const {
    const int lane = threadIdx.x & 63;
    uint32_t fl = 0;
    int tot = 0, rk = 0;
#pragma unroll
    for (int k = 0; k < NC; k++) {
      const int64_t x = lane + 64 * k;
      const bool in = x < U;
      const int32_t wk = chained ? chain_eval(c[k], in, fl) : (in ? w[k] : 0);
      fl |= ((uint32_t)wk >> 8) & kStAll;
      const bool need = (wk & 3) != 0;
      tot += __popcll(__ballot(need));
      rk += __popcll(__ballot(need && x < u));
    }
    flags = wave_reduce(fl, [](uint32_t a, uint32_t b) { return a | b; });
    total = tot;
    rank = rk;
  }
};

// The commit of unit u by one wave, in two phases around the verdict.
// begin (before it; loads only): the new token, the existing pages the step
// writes (straight into their LDS images img_h, img_l: the high page of the
// new token, the low page of the requantized token) and the token it
// requantizes; ids are clamped into the pool, since a unit that will not
// commit may carry a stale plan.  finish (committing units, page: the new
// page when need): fresh images zeroed, fields edited, changed bytes stored,
// then the table entry and the tier state.  The wave's LDS operations
// complete in program order, so no barrier is needed between the phases.
template <int D>
struct WaveCommit {
  static constexpr int PD = D / 64;  // dims per lane
  static constexpr int kPB = page_bytes_for(D);
  float xk[PD], xv[PD];
  uint32_t km_rq = 0, vm_rq = 0, kc_rq[PD], vc_rq[PD];
  float sc_rq = 0.0f;
  int32_t pos_rq = 0;

  __device__ __forceinline__ void begin(int64_t u, int page_bytes, int64_t P, const uint16_t* k_new,
                                        const uint16_t* v_new, int need, int lo_src, int32_t id_hrow,
                                        int32_t id_lrow, int32_t id_src, const uint8_t* pages, uint32_t* img_h,
                                        uint32_t* img_l) {
    constexpr Seg sh = tier_seg(D, true);
    const int lane = threadIdx.x & 63;
    auto clampP = [&](int32_t id) { return min(max(id, 0), (int32_t)(P - 1)); };
#pragma unroll
    for (int e = 0; e < PD; e++) {
      xk[e] = h2f(k_new[u * D + lane + 64 * e]);
      xv[e] = h2f(v_new[u * D + lane + 64 * e]);
      kc_rq[e] = vc_rq[e] = 0u;
    }
    // an existing page goes straight from memory into its image (16 bytes
    // per lane and instruction, every chunk in flight at once)
    auto img_load = [&](uint32_t* img, int32_t id) {
      const uint8_t* src = pages + (int64_t)clampP(id) * page_bytes;
#pragma unroll
      for (int c = 0; c < (kPB + 1023) / 1024; c++)
        if (c * 1024 + lane * 16 < kPB)
          __builtin_amdgcn_global_load_lds((const void*)(src + c * 1024 + lane * 16),
                                           (__attribute__((address_space(3))) void*)((uint8_t*)img + c * 1024),
                                           16, 0, 0);
    };
    if (need != kTierHi) img_load(img_h, id_hrow);
    if (lo_src >= 0 && need != kTierLo) img_load(img_l, id_lrow);
    if (lo_src >= 0) {
      const uint8_t* src = pages + (int64_t)clampP(id_src) * page_bytes;
      const int si = lo_src & 15;
      km_rq = *(const uint32_t*)(src + sh.km + 4 * si);
      vm_rq = *(const uint32_t*)(src + sh.vm + 4 * si);
      sc_rq = *(const float*)(src + sh.sc + 4 * si);
      pos_rq = *(const int32_t*)(src + sh.ps + 4 * si);
#pragma unroll
      for (int e = 0; e < PD; e++) {
        int byte, shift;
        k_field(D, true, si, lane + 64 * e, byte, shift);
        kc_rq[e] = ((uint32_t)src[byte] >> shift) & 0xFFu;
        v_field(D, true, si, lane + 64 * e, byte, shift);
        vc_rq[e] = ((uint32_t)src[byte] >> shift) & 0xFu;
      }
    }
  }

  __device__ __forceinline__ void finish(int L, int page_bytes, int64_t P, int N, int nh, int nl, int ph, int pl,
                                         int need, int32_t page, int new_hi, int hi_app, int lo_src, int lo_slot,
                                         int lo_app, int32_t id_hrow, int32_t id_lrow, int32_t id_first,
                                         int32_t* row, int32_t* s4, uint8_t* pages, uint32_t* img_h,
                                         uint32_t* img_l, int32_t& id_h, int32_t& id_l) {
    const int lane = threadIdx.x & 63;
    const TokWrite th{true, true, need == kTierHi, new_hi & 15, need == kTierHi ? page : id_hrow};
    const TokWrite tl{lo_src >= 0, false, need == kTierLo, lo_slot & 31,
                      lo_src < 0 ? 0 : (need == kTierLo ? page : id_lrow)};
    id_h = th.id;
    id_l = tl.id;
    // a fresh page's image starts zeroed
    if (th.fresh)
      for (int c = lane; c < kPB / 16; c += 64) ((uint4*)img_h)[c] = make_uint4(0u, 0u, 0u, 0u);
    if (tl.on && tl.fresh)
      for (int c = lane; c < kPB / 16; c += 64) ((uint4*)img_l)[c] = make_uint4(0u, 0u, 0u, 0u);
    // the requantized token's dequantized values (its high slot may be the
    // new token's: read in begin, before anything is written)
    float xk_rq[PD], xv_rq[PD];
#pragma unroll
    for (int e = 0; e < PD; e++) {
      xk_rq[e] = tl.on ? dequant(h2f((uint16_t)km_rq), h2f((uint16_t)(km_rq >> 16)), kc_rq[e]) : 0.0f;
      xv_rq[e] = tl.on ? dequant(h2f((uint16_t)vm_rq), h2f((uint16_t)(vm_rq >> 16)), vc_rq[e]) : 0.0f;
    }
    float mn[4], mx[4];
    mn[0] = mx[0] = xk[0];
    mn[1] = mx[1] = xv[0];
    mn[2] = mx[2] = xk_rq[0];
    mn[3] = mx[3] = xv_rq[0];
#pragma unroll
    for (int e = 1; e < PD; e++) {
      mn[0] = fminf(mn[0], xk[e]);
      mx[0] = fmaxf(mx[0], xk[e]);
      mn[1] = fminf(mn[1], xv[e]);
      mx[1] = fmaxf(mx[1], xv[e]);
      mn[2] = fminf(mn[2], xk_rq[e]);
      mx[2] = fmaxf(mx[2], xk_rq[e]);
      mn[3] = fminf(mn[3], xv_rq[e]);
      mx[3] = fmaxf(mx[3], xv_rq[e]);
    }
#pragma unroll
    for (int v = 0; v < 4; v++) {
      mn[v] = wave_min(mn[v]);
      mx[v] = wave_max(mx[v]);
    }
    // the images have landed (their loads count as vector memory reads)
    // before any field edit: s_waitcnt vmcnt(0)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");
    auto put = [&](uint32_t* img, const TokWrite& t, const float* xkv, const float* xvv, float kmn, float kmx,
                   float vmn, float vmx, float score, int32_t pos) {
      const Seg sg = tier_seg(D, t.hi);
      uint16_t ks16, kz16, vs16, vz16;
      float ks, kz, vs, vz;
      codec_params(kmn, kmx, sg.kbits, ks16, kz16, ks, kz);
      codec_params(vmn, vmx, sg.vbits, vs16, vz16, vs, vz);
#pragma unroll
      for (int e = 0; e < PD; e++) {
        int byte, shift;
        k_field(D, t.hi, t.idx, lane + 64 * e, byte, shift);
        lds_put(img, byte, shift, sg.kbits, codec_code(xkv[e], ks, kz, sg.kbits));
        v_field(D, t.hi, t.idx, lane + 64 * e, byte, shift);
        lds_put(img, byte, shift, sg.vbits, codec_code(xvv[e], vs, vz, sg.vbits));
      }
      if (lane == 0) {
        img[sg.km / 4 + t.idx] = (uint32_t)ks16 | ((uint32_t)kz16 << 16);
        img[sg.vm / 4 + t.idx] = (uint32_t)vs16 | ((uint32_t)vz16 << 16);
        img[sg.sc / 4 + t.idx] = __float_as_uint(score);
        img[sg.ps / 4 + t.idx] = (uint32_t)pos;
      }
    };
    put(img_h, th, xk, xv, mn[0], mx[0], mn[1], mx[1], 0.0f, N);
    if (tl.on) put(img_l, tl, xk_rq, xv_rq, mn[2], mx[2], mn[3], mx[3], sc_rq, pos_rq);
    asm volatile("" ::: "memory");  // every field is written before the stores read the images
    auto store = [&](const uint32_t* img, const TokWrite& t) {
      if (!t.on) return;
      const Seg sg = tier_seg(D, t.hi);
      uint8_t* pg = pages + (int64_t)t.id * page_bytes;
      if (t.fresh) {
        for (int c = lane; c < page_bytes / 16; c += 64) ((uint4*)pg)[c] = ((const uint4*)img)[c];
        return;
      }
      const int kb = t.idx * D * sg.kbits / 8, kn = D * sg.kbits / 128;  // 16-byte chunks
      const int vn = (sg.vm - sg.vc) / 16;
      for (int c = lane; c < kn + vn + 4; c += 64) {
        if (c < kn) {
          ((uint4*)(pg + kb))[c] = ((const uint4*)(img + kb / 4))[c];
        } else if (c < kn + vn) {
          ((uint4*)(pg + sg.vc))[c - kn] = ((const uint4*)(img + sg.vc / 4))[c - kn];
        } else {
          const int seg = c - kn - vn;
          const int off = (seg == 0 ? sg.km : seg == 1 ? sg.vm : seg == 2 ? sg.sc : sg.ps) + 4 * t.idx;
          *(uint32_t*)(pg + off) = img[off / 4];
        }
      }
    };
    store(img_h, th);
    store(img_l, tl);
    if (lane == 0) {
      // the unit changed: its plan record (first high page) no longer applies
      if (ph >= 1 && id_first >= 0 && id_first < P)
        *(uint32_t*)(pages + (int64_t)id_first * page_bytes + plan_rec_off<D>()) = 0u;
      if (need == kTierHi) row[ph] = page;
      if (need == kTierLo) row[L - 1 - pl] = page;
      s4[0] = nh + hi_app;
      s4[1] = nl + lo_app;
      s4[2] = ph + (need == kTierHi);
      s4[3] = pl + (need == kTierLo);
    }
  }
};

}  // namespace dkv
