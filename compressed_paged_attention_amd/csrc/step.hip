// step.hip -- generation-phase compaction and request release.
//
// Generation step (DiffKV notes, "KV compression policy", generation phase
// and algorithm flow; "Memory management", generation workflow;
// "Implementation": the compactor runs before the attention kernel).  Per
// active unit with length N (new token at position N, thresholds use
// N' = N + 1):
//   * the new token enters the window, i.e. the high tier (K8 V4);
//   * t_c, the token at position N - W, leaves the window; its mean
//     sum/(W - 1) is classified against alpha/N';
//   * t_c high: the least important non-window high token (t_c included)
//     stays above alpha_h/N', is requantized to low inside
//     [alpha_l/N', alpha_h/N'], or is pruned below;
//   * t_c low: t_c is requantized to low; the least important low token
//     (t_c included) is pruned below alpha_l/N';
//   * t_c pruned: removed.
// Means compare as sum_a*cnt_b vs sum_b*cnt_a in fp64 (cnt = N - 1 - pos,
// exact), ties to the smaller position.  A removal and an insertion in one
// tier share a slot, otherwise the insertion appends: no tier shrinks, so a
// unit needs at most one new page and never frees one.
//
// Kernels: plan (one block per unit: one scan over both tiers' score and
// position words), commit (one block per unit: the unit-order prefix sum over
// page demand with the capacity check, redone by every block; new page
// zero-filled, requantization, new token).  Past kDirectUnits units a
// single-block coordination kernel computes the prefix sum once instead.
//
// Release ("Memory management": a finished request's pages are reclaimed):
// plan (one block: prefix sum over released page counts) and write (one block
// per unit: high pages left to right, then low pages right to left, appended
// at the reclamation pointer; rows reset).
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

namespace dkv {

// Per-unit plan record and a compact demand word per unit:
//   nf[u] = need tier (bits 0-1: 0 none, 1 low, 2 high) | kActive | status flags << 8
constexpr int kSRec = 8;
enum { S_NEWHI = 0, S_HIAPP, S_LOSRC, S_LOSLOT, S_LOAPP, S_PAGE };
enum { SH_COMMIT = 0, SH_START, SH_END, SH_D };
constexpr int32_t kActive = 4;
// Up to this many units every commit workgroup redoes the unit-order prefix
// sum over the demand words itself (no coordination kernel in between).
constexpr int64_t kDirectUnits = 2048;

size_t step_workspace(const Cfg& c, int batch) {
  const size_t U = (size_t)batch * c.H;
  return align_up(16 * sizeof(int64_t), 256) + align_up(U * kSRec * sizeof(int32_t), 256) +
         align_up(U * sizeof(int32_t), 256);
}

struct StepWs {
  int64_t* hdr;
  int32_t* rec;
  int32_t* nf;
};

static StepWs step_carve(const Cfg& c, int batch, void* ws) {
  const size_t U = (size_t)batch * c.H;
  uint8_t* p = (uint8_t*)ws;
  StepWs w;
  w.hdr = (int64_t*)p;
  p += align_up(16 * sizeof(int64_t), 256);
  w.rec = (int32_t*)p;
  p += align_up(U * kSRec * sizeof(int32_t), 256);
  w.nf = (int32_t*)p;
  return w;
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
// Counts are below 2^31 (N <= max_seq_len), so both products are exact.
__device__ inline bool less_imp(const Cand& a, const Cand& b, int64_t N) {
  if (a.pos == kNoPos) return false;
  if (b.pos == kNoPos) return true;
  const int32_t n1 = (int32_t)(N - 1);
  const double l = (double)a.sum * (double)(n1 - b.pos), r = (double)b.sum * (double)(n1 - a.pos);
  return l < r || (l == r && a.pos < b.pos);
}

template <int LVL>
__device__ inline void argmin_step(Cand& c, int64_t N) {
  const Cand t{lane_xchg_t<LVL>(c.sum), lane_xchg_t<LVL>(c.pos), lane_xchg_t<LVL>(c.slot)};
  if (less_imp(t, c, N)) c = t;
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

constexpr int kPlanThreads = 512;

__device__ inline int classify_mean(float sum, int64_t cnt, int64_t Np, int lo_en, double ah, double al) {
  const double x = (double)sum * (double)Np;
  const double ch = ah * (double)cnt, cl = al * (double)cnt;
  if (lo_en) {
    if (x > ch) return kTierHi;
    return x >= cl ? kTierLo : kTierPrune;
  }
  return x >= cl ? kTierHi : kTierPrune;
}

// One block per unit.  A single pass over both tiers' score and position
// words finds t_c, the least important non-window high token and the least
// important low token; the decision needs no second pass.
template <int D>
__global__ __launch_bounds__(kPlanThreads) void step_plan_kernel(int H, int L, int W, int S_max, int lo_en, float ah,
                                                        float al, int64_t P, int page_bytes,
                                                        const int32_t* __restrict__ seq_len,
                                                        const int32_t* __restrict__ table,
                                                        const int32_t* __restrict__ state,
                                                        const uint8_t* __restrict__ pages,
                                                        const uint64_t* __restrict__ ptr, int64_t* __restrict__ hdr,
                                                        int32_t* __restrict__ rec, int32_t* __restrict__ nf) {
  const int64_t u = blockIdx.x;
  const int b = (int)u / H;
  const int tid = threadIdx.x;
  if (u == 0 && tid == 0) {  // pointer snapshot for the commit kernel
    hdr[SH_START] = (int64_t)ptr[0];
    hdr[SH_END] = (int64_t)ptr[1];
  }
  const int64_t N = seq_len[b];
  if (N <= 0) {
    if (tid == 0) nf[u] = 0;
    return;
  }
  int32_t* R = rec + u * kSRec;
  const int32_t* s4 = state + 4 * u;
  const int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  const int32_t* row = table + u * L;
  uint32_t flags = 0;
  if (N + 1 > S_max) flags = kStOverflow;
  else if (nh < 0 || nl < 0 || ph != cdiv(nh, kHiTokens) || pl != cdiv(nl, kLoTokens) || nh + nl > N ||
           ph + pl > L)
    flags = kStBadState;
  if (flags) {
    if (tid == 0) nf[u] = kActive | (int32_t)(flags << 8);
    return;
  }
  const Seg sh = tier_seg(D, true), sl = tier_seg(D, false);
  const int64_t Np = N + 1, tc_pos = N - W;
  const double dah = (double)ah, dal = (double)al;
  __shared__ int s_tc;
  __shared__ float s_tcsum;
  __shared__ uint32_t s_bad;
  __shared__ Cand lds[2][kPlanThreads / 64];
  const Cand none{0.0f, kNoPos, 0};
  if (tid == 0) {
    s_tc = -1;
    s_bad = 0;
  }
  __syncthreads();
  Cand bh = none, bl = none;
  if (tc_pos >= 0) {
    // every slot of both tiers (this also checks every page id of the row);
    // kPer slots per thread per round, their loads issued together
    constexpr int kPer = 4;
    const int n = nh + nl;
    for (int base = 0; base < n; base += kPer * kPlanThreads) {
      // branch-free loads (indices clamped into the unit) so that each
      // round costs two dependent trips to memory
      int32_t id[kPer];
#pragma unroll
      for (int e = 0; e < kPer; e++) {
        const int s = min(base + e * kPlanThreads + tid, n - 1);
        const bool hi = s < nh;
        const int ls = hi ? s : s - nh;
        id[e] = row[hi ? (ls >> 4) : L - 1 - (ls >> 5)];
      }
      int32_t pos[kPer];
      float sum[kPer];
#pragma unroll
      for (int e = 0; e < kPer; e++) {
        const int s = min(base + e * kPlanThreads + tid, n - 1);
        const bool hi = s < nh;
        const int ls = hi ? s : s - nh;
        const uint8_t* pg = pages + (int64_t)min(max(id[e], 0), (int32_t)(P - 1)) * page_bytes;
        const int idx = hi ? (ls & 15) : (ls & 31);
        pos[e] = *(const int32_t*)(pg + (hi ? sh.ps : sl.ps) + 4 * idx);
        sum[e] = *(const float*)(pg + (hi ? sh.sc : sl.sc) + 4 * idx);
      }
#pragma unroll
      for (int e = 0; e < kPer; e++) {
        const int s = base + e * kPlanThreads + tid;
        if (s >= n) continue;
        if (id[e] < 0 || id[e] >= P) s_bad = 1;
        const bool hi = s < nh;
        const int ls = hi ? s : s - nh;
        const Cand c{sum[e], pos[e], ls};
        if (hi) {
          if (pos[e] == tc_pos) {  // positions are unique: one writer
            s_tc = ls;
            s_tcsum = sum[e];
          }
          if (pos[e] <= tc_pos && less_imp(c, bh, N)) bh = c;
        } else if (less_imp(c, bl, N)) {
          bl = c;
        }
      }
    }
  } else {
    for (int j = tid; j < ph + pl; j += blockDim.x) {
      const int32_t id = j < ph ? row[j] : row[L - 1 - (j - ph)];
      if (id < 0 || id >= P) s_bad = 1;
    }
  }
  bh = wave_argmin(bh, N);
  bl = wave_argmin(bl, N);
  if ((tid & 63) == 0) {
    lds[0][tid >> 6] = bh;
    lds[1][tid >> 6] = bl;
  }
  __syncthreads();  // also publishes s_tc and s_bad
  if (tid == 0) {
    for (int w = 1; w < kPlanThreads / 64; w++) {
      if (less_imp(lds[0][w], bh, N)) bh = lds[0][w];
      if (less_imp(lds[1][w], bl, N)) bl = lds[1][w];
    }
  }
  const int tcs = s_tc;
  const float tcsum = s_tcsum;
  // t_c is in the high tier by construction; a missing t_c is bad state
  if (s_bad || (tc_pos >= 0 && tcs < 0)) {
    if (tid == 0) nf[u] = kActive | (int32_t)(kStBadState << 8);
    return;
  }
  if (tid != 0) return;
  int new_hi = nh, hi_app = 1, lo_src = -1, lo_slot = 0, lo_app = 0;
  if (tc_pos >= 0) {
    const int cls = classify_mean(tcsum, W - 1, Np, lo_en, dah, dal);
    if (cls == kTierHi) {
      const int vcls = classify_mean(bh.sum, N - 1 - bh.pos, Np, lo_en, dah, dal);
      if (vcls == kTierLo) {
        lo_src = bh.slot;
        lo_slot = nl;
        lo_app = 1;
        new_hi = bh.slot;
        hi_app = 0;
      } else if (vcls == kTierPrune) {
        new_hi = bh.slot;
        hi_app = 0;
      }
    } else if (cls == kTierLo) {
      // t_c moves to the low tier; the least important low token, t_c
      // included, is pruned below alpha_l / N'
      lo_src = tcs;
      new_hi = tcs;
      hi_app = 0;
      const Cand tcc{tcsum, (int32_t)tc_pos, -1};
      const Cand lv = less_imp(tcc, bl, N) ? tcc : bl;
      if (lv.slot >= 0 && classify_mean(lv.sum, N - 1 - lv.pos, Np, lo_en, dah, dal) == kTierPrune) {
        lo_slot = lv.slot;
        lo_app = 0;
      } else {
        lo_slot = nl;
        lo_app = 1;
      }
    } else {
      new_hi = tcs;
      hi_app = 0;
    }
  }
  int need = 0;
  if (hi_app && nh % kHiTokens == 0) need = kTierHi;
  if (lo_app && nl % kLoTokens == 0) need = kTierLo;
  uint32_t fl = 0;
  if (need && ph + pl + 1 > L) fl = kStOverflow;
  R[S_NEWHI] = new_hi;
  R[S_HIAPP] = hi_app;
  R[S_LOSRC] = lo_src;
  R[S_LOSLOT] = lo_slot;
  R[S_LOAPP] = lo_app;
  R[S_PAGE] = -1;
  nf[u] = kActive | (fl ? 0 : need) | (int32_t)(fl << 8);
}

// Coordination for large batches: prefix sum over the demand words, capacity
// check, page ids, pointer.
__global__ __launch_bounds__(1024) void step_coord_kernel(int64_t U, int64_t P, const int32_t* __restrict__ nf,
                                                          int32_t* __restrict__ rec, const int32_t* list,
                                                          int64_t* __restrict__ hdr, uint64_t* ptr,
                                                          uint32_t* status) {
  __shared__ int64_t lds[20];
  __shared__ uint32_t sflags;
  __shared__ int scommit;
  if (threadIdx.x == 0) sflags = 0;
  __syncthreads();
  int64_t total = 0;
  uint32_t fl = 0;
  for (int64_t base = 0; base < U; base += blockDim.x) {
    const int64_t u = base + threadIdx.x;
    const int32_t w = u < U ? nf[u] : 0;
    fl |= (uint32_t)w >> 8;
    int64_t t;
    block_excl_scan((int64_t)((w & 3) != 0), lds, t);
    total += t;
  }
  if (fl) atomicOr(&sflags, fl);
  __syncthreads();
  const uint64_t start = ptr[0], end = ptr[1];
  if (threadIdx.x == 0) {
    uint32_t st = sflags;
    if (!st && total > (int64_t)(end - start)) st |= kStExhausted;
    scommit = st == 0;
    if (st) atomicOr(status, st);
  }
  __syncthreads();
  const int commit = scommit;
  if (commit) {
    int64_t carry = 0;
    for (int64_t base = 0; base < U; base += blockDim.x) {
      const int64_t u = base + threadIdx.x;
      const int need = u < U ? (nf[u] & 3) != 0 : 0;
      int64_t t;
      const int64_t off = block_excl_scan((int64_t)need, lds, t);
      if (need) rec[u * kSRec + S_PAGE] = list[(start + (uint64_t)(carry + off)) % (uint64_t)P];
      carry += t;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    hdr[SH_COMMIT] = commit;
    if (commit) ptr[0] = start + (uint64_t)total;
  }
}

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

// One block per unit.  DIRECT: the block recomputes the unit-order prefix sum
// of page demand from the demand words (all-or-nothing check included) and
// block 0 advances the allocation pointer; otherwise the coordination
// kernel's result is read.
template <int D, bool DIRECT>
__global__ __launch_bounds__(256) void step_commit_kernel(int H, int L, int64_t U, int64_t P, int page_bytes,
                                                          const int32_t* __restrict__ seq_len,
                                                          const uint16_t* __restrict__ k_new,
                                                          const uint16_t* __restrict__ v_new,
                                                          const int64_t* __restrict__ hdr,
                                                          const int32_t* __restrict__ rec,
                                                          const int32_t* __restrict__ nf,
                                                          const int32_t* __restrict__ list,
                                                          int32_t* __restrict__ table,
                                                          int32_t* __restrict__ state, uint8_t* pages,
                                                          uint64_t* ptr, uint32_t* status) {
  constexpr Seg sh = tier_seg(D, true);
  constexpr int kPageWords = page_bytes_for(D) / 4;
  const int64_t u = blockIdx.x;
  const int tid = threadIdx.x;
  const int b = (int)u / H, h = (int)u % H;  // u < 2^31: 32-bit division
  // ---- phase 1: loads ----
  const int32_t wu = nf[u];
  const int32_t* R = rec + u * kSRec;
  int32_t* row = table + u * L;
  int32_t* s4 = state + 4 * u;
  const int64_t rowi = ((int64_t)b * H + h) * D + tid;
  float xk_new = tid < D ? h2f(k_new[rowi]) : 0.0f;
  float xv_new = tid < D ? h2f(v_new[rowi]) : 0.0f;
  int32_t page = -1;
  if constexpr (DIRECT) {
    __shared__ int lds[16];
    __shared__ int64_t s_off;
    __shared__ uint32_t s_fl;
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
    const int64_t start = hdr[SH_START], end = hdr[SH_END];
    uint32_t st = s_fl;
    if (!st && total > end - start) st = kStExhausted;
    if (u == 0 && tid == 0) {
      if (st) atomicOr(status, st);
      else ptr[0] = (uint64_t)(start + total);
    }
    if (st || !(wu & kActive)) return;
    if (wu & 3) page = list[(uint64_t)(start + s_off) % (uint64_t)P];
  } else {
    if (!hdr[SH_COMMIT] || !(wu & kActive)) return;
    page = R[S_PAGE];
  }
  const int need = wu & 3;
  const int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  const int new_hi = R[S_NEWHI], lo_src = R[S_LOSRC], lo_slot = R[S_LOSLOT];
  const int hi_app = R[S_HIAPP], lo_app = R[S_LOAPP];
  if (need && (page < 0 || page >= P)) {
    if (tid == 0) atomicOr(status, kStBadState);
    return;
  }
  // destinations: the new token's high slot; the requantized token's low slot
  TokWrite th{true, true, need == kTierHi, new_hi & 15,
              need == kTierHi ? page : row[new_hi >> 4]};
  TokWrite tl{lo_src >= 0, false, need == kTierLo, lo_slot & 31,
              lo_src < 0 ? 0 : (need == kTierLo ? page : row[L - 1 - (lo_slot >> 5)])};
  __shared__ uint32_t img_h[kPageWords], img_l[kPageWords];
  __shared__ float red[16];
  img_load<D>(img_h, th, pages, page_bytes);
  img_load<D>(img_l, tl, pages, page_bytes);
  // the requantized token's dequantized values (read before anything is
  // written: its high slot may be the new token's)
  float xk_rq = 0.0f, xv_rq = 0.0f, sc_rq = 0.0f;
  int32_t pos_rq = 0;
  if (tl.on) {
    const uint8_t* src = pages + (int64_t)row[lo_src >> 4] * page_bytes;
    const int si = lo_src & 15;
    const uint32_t km = *(const uint32_t*)(src + sh.km + 4 * si);
    const uint32_t vm = *(const uint32_t*)(src + sh.vm + 4 * si);
    sc_rq = *(const float*)(src + sh.sc + 4 * si);
    pos_rq = *(const int32_t*)(src + sh.ps + 4 * si);
    if (tid < D) {
      int byte, shift;
      k_field(D, true, si, tid, byte, shift);
      xk_rq = dequant(h2f((uint16_t)km), h2f((uint16_t)(km >> 16)), ((uint32_t)src[byte] >> shift) & 0xFFu);
      v_field(D, true, si, tid, byte, shift);
      xv_rq = dequant(h2f((uint16_t)vm), h2f((uint16_t)(vm >> 16)), ((uint32_t)src[byte] >> shift) & 0xFu);
    }
  }
  const int32_t N = seq_len[b];
  __syncthreads();  // LDS images loaded (no global store is outstanding)
  // ---- phase 2: quantize, edit the images ----
  float mn[4] = {xk_new, xv_new, xk_rq, xv_rq}, mx[4] = {xk_new, xv_new, xk_rq, xv_rq};
  block_minmax<D, 4>(mn, mx, red);
  {
    const Seg sg = tier_seg(D, true);
    uint16_t ks16, kz16, vs16, vz16;
    float ks, kz, vs, vz;
    codec_params(mn[0], mx[0], sg.kbits, ks16, kz16, ks, kz);
    codec_params(mn[1], mx[1], sg.vbits, vs16, vz16, vs, vz);
    img_token<D>(img_h, th, codec_code(xk_new, ks, kz, sg.kbits), codec_code(xv_new, vs, vz, sg.vbits),
                 (uint32_t)ks16 | ((uint32_t)kz16 << 16), (uint32_t)vs16 | ((uint32_t)vz16 << 16), 0.0f, N);
  }
  if (tl.on) {
    const Seg sg = tier_seg(D, false);
    uint16_t ks16, kz16, vs16, vz16;
    float ks, kz, vs, vz;
    codec_params(mn[2], mx[2], sg.kbits, ks16, kz16, ks, kz);
    codec_params(mn[3], mx[3], sg.vbits, vs16, vz16, vs, vz);
    img_token<D>(img_l, tl, codec_code(xk_rq, ks, kz, sg.kbits), codec_code(xv_rq, vs, vz, sg.vbits),
                 (uint32_t)ks16 | ((uint32_t)kz16 << 16), (uint32_t)vs16 | ((uint32_t)vz16 << 16), sc_rq,
                 pos_rq);
  }
  __syncthreads();
  // ---- phase 3: stores ----
  img_store<D>(img_h, th, pages, page_bytes);
  img_store<D>(img_l, tl, pages, page_bytes);
  if (tid == 0) {
    if (need == kTierHi) row[ph] = page;
    if (need == kTierLo) row[L - 1 - pl] = page;
    s4[0] = nh + hi_app;
    s4[1] = nl + lo_app;
    s4[2] = ph + (need == kTierHi);
    s4[3] = pl + (need == kTierLo);
  }
}

hipError_t launch_step(const Cfg& c, const Pool& p, int batch, const int32_t* seq_len, const uint16_t* k,
                       const uint16_t* v, int32_t* table, int32_t* state, void* ws, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const StepWs w = step_carve(c, batch, ws);
  const dim3 grid((unsigned)U), block(256);
#define DKV_PLAN(D)                                                                                   \
  step_plan_kernel<D><<<grid, dim3(kPlanThreads), 0, s>>>(c.H, c.L, c.W, c.S_max, c.lo_en, c.ah, c.al, p.P,       \
                                             p.page_bytes, seq_len, table, state, p.pages, p.ptr, w.hdr, \
                                             w.rec, w.nf)
#define DKV_COMMIT(D, DIR)                                                                             \
  step_commit_kernel<D, DIR><<<grid, block, 0, s>>>(c.H, c.L, U, p.P, p.page_bytes, seq_len, k, v, w.hdr, \
                                                    w.rec, w.nf, p.list, table, state, p.pages, p.ptr,  \
                                                    p.status)
  if (c.d == 128) DKV_PLAN(128);
  else DKV_PLAN(64);
  if (U <= kDirectUnits) {
    if (c.d == 128) DKV_COMMIT(128, true);
    else DKV_COMMIT(64, true);
  } else {
    step_coord_kernel<<<dim3(1), dim3(1024), 0, s>>>(U, p.P, w.nf, w.rec, p.list, w.hdr, p.ptr, p.status);
    if (c.d == 128) DKV_COMMIT(128, false);
    else DKV_COMMIT(64, false);
  }
#undef DKV_PLAN
#undef DKV_COMMIT
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// release
// ---------------------------------------------------------------------------
size_t release_workspace(const Cfg& c, int batch) {
  return align_up(16 * sizeof(int64_t), 256) + align_up((size_t)batch * c.H * sizeof(int64_t), 256);
}

__global__ __launch_bounds__(1024) void release_plan_kernel(int H, int L, int64_t U, int64_t P,
                                                            const uint8_t* __restrict__ mask,
                                                            const int32_t* __restrict__ state,
                                                            int64_t* __restrict__ off, int64_t* hdr,
                                                            uint64_t* ptr, uint32_t* status) {
  __shared__ int64_t lds[20];
  __shared__ uint32_t sflags;
  if (threadIdx.x == 0) sflags = 0;
  __syncthreads();
  int64_t carry = 0;
  for (int64_t base = 0; base < U; base += blockDim.x) {
    const int64_t u = base + threadIdx.x;
    int64_t n = 0;
    if (u < U && mask[u / H]) {
      const int32_t ph = state[4 * u + 2], pl = state[4 * u + 3];
      if (ph < 0 || pl < 0 || ph + pl > L) atomicOr(&sflags, kStBadState);
      else n = ph + pl;
    }
    int64_t t;
    const int64_t o = block_excl_scan(n, lds, t);
    if (u < U) off[u] = carry + o;
    carry += t;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t start = ptr[0], end = ptr[1];
    uint32_t st = sflags;
    if (!st && (int64_t)(end - start) + carry > P) st |= kStBadState;
    hdr[0] = st == 0;
    hdr[1] = (int64_t)end;
    if (st) atomicOr(status, st);
    else ptr[1] = end + (uint64_t)carry;
  }
}

__global__ __launch_bounds__(256) void release_write_kernel(int H, int L, int64_t P,
                                                            const uint8_t* __restrict__ mask,
                                                            const int64_t* __restrict__ off,
                                                            const int64_t* __restrict__ hdr,
                                                            int32_t* __restrict__ list,
                                                            int32_t* __restrict__ table,
                                                            int32_t* __restrict__ state) {
  if (!hdr[0]) return;
  const int64_t u = blockIdx.x;
  if (!mask[u / H]) return;
  int32_t* row = table + u * L;
  int32_t* s4 = state + 4 * u;
  const int ph = s4[2], pl = s4[3];
  const uint64_t e0 = (uint64_t)hdr[1] + (uint64_t)off[u];
  for (int j = threadIdx.x; j < ph + pl; j += blockDim.x) {
    const int32_t id = j < ph ? row[j] : row[L - 1 - (j - ph)];
    list[(e0 + (uint64_t)j) % (uint64_t)P] = id;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < L; j += blockDim.x) row[j] = -1;
  if (threadIdx.x < 4) s4[threadIdx.x] = 0;
}

hipError_t launch_release(const Cfg& c, const Pool& p, int batch, const uint8_t* mask, int32_t* table,
                          int32_t* state, void* ws, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  int64_t* hdr = (int64_t*)ws;
  int64_t* off = (int64_t*)((uint8_t*)ws + align_up(16 * sizeof(int64_t), 256));
  release_plan_kernel<<<dim3(1), dim3(1024), 0, s>>>(c.H, c.L, U, p.P, mask, state, off, hdr, p.ptr, p.status);
  release_write_kernel<<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.L, p.P, mask, off, hdr, p.list, table,
                                                               state);
  return hipGetLastError();
}

}  // namespace dkv
