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
#include "dkv_step.hpp"

namespace dkv {

size_t step_workspace(const Cfg& c, int batch) {
  const size_t U = (size_t)batch * c.H;
  return align_up(16 * sizeof(int64_t), 256) + align_up(U * rec_words(c) * sizeof(int32_t), 256) +
         align_up(U * sizeof(int32_t), 256) + align_up(U * kChainWords * sizeof(int32_t), 256);
}

constexpr int kPlanThreads = 256;
constexpr int kPlanPer = 8;       // slots per thread per round, loads issued together
constexpr int kRowCache = 4096;   // table rows up to this long are read once into LDS


// One block per unit.  The unit's length, tier state and table row are read
// in one round; then one pass over both tiers' score and position words finds
// t_c, the least important non-window high token and the least important low
// token (wave butterflies, then the four waves' candidates in one quad).
// PLAIN (a tier codec variant): score and position words at the offsets of
// sh / sl, and no plan records (their spare bytes are not reserved there).
template <int D, bool PLAIN>
__global__ __launch_bounds__(kPlanThreads) void step_plan_kernel(int H, int L, int W, int S_max, int lo_en, float ah,
                                                                 float al, const float* __restrict__ ah_head,
                                                                 const float* __restrict__ al_head, int64_t P,
                                                                 int page_bytes, Seg shp, Seg slp,
                                                                 const int32_t* __restrict__ seq_len,
                                                                 const int32_t* __restrict__ table,
                                                                 const int32_t* __restrict__ state,
                                                                 const uint8_t* __restrict__ pages,
                                                                 const uint64_t* __restrict__ ptr,
                                                                 int64_t* __restrict__ hdr, int32_t* __restrict__ rec,
                                                                 int32_t* __restrict__ nf) {
  const int u = blockIdx.x;
  const int b = u / H;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int32_t* row = table + (int64_t)u * L;
  __shared__ int32_t row_s[kRowCache];
  __shared__ int s_tc;
  __shared__ float s_tcsum;
  __shared__ uint32_t s_bad;
  __shared__ Cand lds[2][kPlanThreads / 64];
  __shared__ int s_rec;
  // ---- first round trip: length, tier state, the table row (every load of a
  // thread issued before any is used: one round trip) ----
  const bool cached = L <= kRowCache;
  if (cached) {
    constexpr int kPer = kRowCache / kPlanThreads;
    int32_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
      const int j = tid + k * kPlanThreads;
      v[k] = j < L ? row[j] : 0;
    }
#pragma unroll
    for (int k = 0; k < kPer; k++) {
      const int j = tid + k * kPlanThreads;
      if (j < L) row_s[j] = v[k];
    }
  }
  // the plan record in the unit's first page: its loads go out before the
  // barrier (the id is clamped into the pool; used only if it is the
  // unit's first high page)
  const int32_t first_id = row[0];
  uint32_t rw[kRecWords];
  if (!PLAIN && tid == 0) {
    const uint32_t* w = (const uint32_t*)(pages + (int64_t)min(max(first_id, 0), (int32_t)(P - 1)) * page_bytes +
                                          plan_rec_off<D>());
#pragma unroll
    for (int k = 0; k < kRecWords; k++) rw[k] = w[k];
  }
  if (u == 0 && tid == 0) {  // pointer snapshot for the commit kernel
    hdr[SH_START] = (int64_t)ptr[0];
    hdr[SH_END] = (int64_t)ptr[1];
  }
  const int64_t N = seq_len[b];
  const int32_t* s4 = state + 4 * (int64_t)u;
  const int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  if (tid == 0) {
    s_tc = -1;
    s_bad = 0;
  }
  __syncthreads();
  if (N <= 0) {
    if (tid == 0) nf[u] = 0;
    return;
  }
  int32_t* R = rec + (int64_t)u * kSRec;
  uint32_t flags = 0;
  if (N + 1 > S_max) flags = kStOverflow;
  else if (nh < 0 || nl < 0 || ph != cdiv(nh, kHiTokens) || pl != cdiv(nl, kLoTokens) || nh + nl > N ||
           ph + pl > L)
    flags = kStBadState;
  if (flags) {
    if (tid == 0) nf[u] = kActive | (int32_t)(flags << 8);
    return;
  }
  auto page_of = [&](int tix) { return cached ? row_s[tix] : row[tix]; };
  // ---- a plan record left by the previous attention: no scan needed ----
  if (!PLAIN && tid == 0) {
    s_rec = 0;
    const int32_t p0 = ph >= 1 ? first_id : -1;
    if (p0 >= 0 && p0 < P) {
      Plan pr;
      if (plan_rec_check(rw, N, nh, nl, ph, pl, pr)) {
        s_rec = 1;
        step_rec_put(R, nf + u, pr, L, page_of);
      }
    }
  }
  if (PLAIN && tid == 0) s_rec = 0;
  __syncthreads();
  if (s_rec) return;
  const Seg sh = PLAIN ? shp : tier_seg(D, true), sl = PLAIN ? slp : tier_seg(D, false);
  const int64_t tc_pos = N - W;
  const double dah = (double)(ah_head ? ah_head[u % H] : ah), dal = (double)(al_head ? al_head[u % H] : al);
  const Cand none{0.0f, kNoPos, 0};
  Cand bh = none, bl = none;
  if (tc_pos >= 0) {
    // every slot of both tiers (this also checks every page id of the row)
    const int n = nh + nl;
    for (int base = 0; base < n; base += kPlanPer * kPlanThreads) {
      int32_t pos[kPlanPer];
      float sum[kPlanPer];
      int32_t id[kPlanPer];
#pragma unroll
      for (int e = 0; e < kPlanPer; e++) {
        // branch-free loads (indices clamped into the unit)
        const int s = min(base + e * kPlanThreads + tid, n - 1);
        const bool hi = s < nh;
        const int ls = hi ? s : s - nh;
        id[e] = page_of(hi ? (ls >> 4) : L - 1 - (ls >> 5));
        const uint8_t* pg = pages + (int64_t)min(max(id[e], 0), (int32_t)(P - 1)) * page_bytes;
        const int idx = hi ? (ls & 15) : (ls & 31);
        pos[e] = __builtin_nontemporal_load((const int32_t*)(pg + (hi ? sh.ps : sl.ps) + 4 * idx));
        sum[e] = __builtin_nontemporal_load((const float*)(pg + (hi ? sh.sc : sl.sc) + 4 * idx));
      }
      // this round's candidates, then a pairwise tree (short dependent chain)
      Cand ch[kPlanPer], cl[kPlanPer];
#pragma unroll
      for (int e = 0; e < kPlanPer; e++) {
        const int s = base + e * kPlanThreads + tid;
        const bool in = s < n, hi = s < nh;
        const int ls = hi ? s : s - nh;
        if (in && (id[e] < 0 || id[e] >= P)) s_bad = 1;
        if (in && hi && pos[e] == tc_pos) {  // positions are unique: one writer
          s_tc = ls;
          s_tcsum = sum[e];
        }
        ch[e] = Cand{sum[e], (in && hi && pos[e] <= tc_pos) ? pos[e] : kNoPos, ls};
        cl[e] = Cand{sum[e], (in && !hi) ? pos[e] : kNoPos, ls};
      }
#pragma unroll
      for (int w = kPlanPer / 2; w >= 1; w >>= 1)
#pragma unroll
        for (int e = 0; e < w; e++) {
          ch[e] = min_imp(ch[e], ch[e + w], N);
          cl[e] = min_imp(cl[e], cl[e + w], N);
        }
      bh = min_imp(bh, ch[0], N);
      bl = min_imp(bl, cl[0], N);
    }
  } else {
    for (int j = tid; j < ph + pl; j += kPlanThreads) {
      const int32_t id = page_of(j < ph ? j : L - 1 - (j - ph));
      if (id < 0 || id >= P) s_bad = 1;
    }
  }
  bh = wave_argmin(bh, N);
  bl = wave_argmin(bl, N);
  if (lane == 0) {
    lds[0][wid] = bh;
    lds[1][wid] = bl;
  }
  __syncthreads();  // also publishes s_tc and s_bad
  if (wid != 0) return;
  // the waves' candidates: lane q of each quad holds wave q's, two butterfly levels
  static_assert(kPlanThreads / 64 == 4, "one quad of candidates");
  bh = lds[0][lane & 3];
  bl = lds[1][lane & 3];
  argmin_step<0>(bh, N);
  argmin_step<1>(bh, N);
  argmin_step<0>(bl, N);
  argmin_step<1>(bl, N);
  if (lane != 0) return;
  const int tcs = s_tc;
  const float tcsum = s_tcsum;
  // t_c is in the high tier by construction; a missing t_c is bad state
  if (s_bad || (tc_pos >= 0 && tcs < 0)) {
    nf[u] = kActive | (int32_t)(kStBadState << 8);
    return;
  }
  const Plan pl_ = plan_decide(N, W, S_max, lo_en, dah, dal, nh, nl, ph, pl, L, tcs, tcsum, bh, bl);
  step_rec_put(R, nf + u, pl_, L, page_of);
}

// Coordination for large batches: prefix sum over the demand words, capacity
// check, page ids, pointer.
__global__ __launch_bounds__(1024) void step_coord_kernel(int64_t U, int64_t P, int rs, const int32_t* __restrict__ nf,
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
      if (need) rec[u * rs + S_PAGE] = list[(start + (uint64_t)(carry + off)) % (uint64_t)P];
      carry += t;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    hdr[SH_COMMIT] = commit;
    if (commit) ptr[0] = start + (uint64_t)total;
  }
}

// One block per unit: the commit of its unit.
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
  __shared__ __align__(16) uint32_t sm[commit_lds_words<D>()];
  commit_unit<D, DIRECT>(blockIdx.x, H, L, U, P, page_bytes, seq_len, k_new, v_new, hdr, rec, nf, list, table,
                         state, pages, ptr, status, sm);
}

// The same for the plain layout of a tier codec variant.
template <int D, bool DIRECT>
__global__ __launch_bounds__(256) void step_commit_plain_kernel(int H, int L, int64_t U, int64_t P, int page_bytes,
                                                                Lay lay, const int32_t* __restrict__ seq_len,
                                                                const uint16_t* __restrict__ k_new,
                                                                const uint16_t* __restrict__ v_new,
                                                                const int64_t* __restrict__ hdr,
                                                                const int32_t* __restrict__ rec,
                                                                const int32_t* __restrict__ nf,
                                                                const int32_t* __restrict__ list,
                                                                int32_t* __restrict__ table,
                                                                int32_t* __restrict__ state, uint8_t* pages,
                                                                uint64_t* ptr, uint32_t* status) {
  __shared__ __align__(16) uint32_t sm[commit_lds_words<D, true>()];
  commit_unit<D, DIRECT, true>(blockIdx.x, H, L, U, P, page_bytes, seq_len, k_new, v_new, hdr, rec, nf, list,
                               table, state, pages, ptr, status, sm, lay);
}


// ---------------------------------------------------------------------------
// K precision levels (DiffKV notes, "KV compression policy", extensibility;
// "Memory management", generation workflow).  Plan (one block per unit: one
// scan over every level's score and position words: t_c, the least
// important non-window level-0 token and the least important token of each
// other level), the coordination kernel (always), commit (one block per
// unit: up to two token moves and the new token through LDS images of the
// written code ranges).  The decision, at length N with N' = N + 1:
//   l_c = level of t_c (mean over W - 1 observations);
//   l_c = 0: the least important non-window level-0 token v (t_c included)
//            moves to its level or is pruned unless it stays in level 0;
//   l_c > 0: t_c moves to level l_c; the least important token v of level
//            l_c and t_c, if it is not t_c and its level is below l_c,
//            gives t_c its slot and moves down (or is pruned);
//   pruned:  t_c is removed.
// The new token takes a freed level-0 slot or appends.
// ---------------------------------------------------------------------------

// level of a mean sum / cnt at N' (x = sum N' against alpha cnt), -1 pruned
__device__ inline int level_of_mean(float sum, int64_t cnt, int64_t Np, int K, double a0, double a1, double a2,
                                    double aL) {
  const double x = (double)sum * (double)Np, c = (double)cnt;
  if (x > a0 * c) return 0;
  if (x > a1 * c) return 1;
  if (K == 4 && x > a2 * c) return 2;
  return x >= aL * c ? K - 1 : -1;
}

__global__ __launch_bounds__(kPlanThreads) void step_plan_levels_kernel(int H, int L, int LT, int W, int S_max,
                                                                        float ah, float am0, float am1, float al,
                                                                        const float* __restrict__ ah_head,
                                                                        const float* __restrict__ al_head,
                                                                        int64_t P, int page_bytes, Levels lv,
                                                                        const int32_t* __restrict__ seq_len,
                                                                        const int32_t* __restrict__ table,
                                                                        const int32_t* __restrict__ state,
                                                                        const uint8_t* __restrict__ pages,
                                                                        const uint64_t* __restrict__ ptr,
                                                                        int64_t* __restrict__ hdr,
                                                                        int32_t* __restrict__ rec,
                                                                        int32_t* __restrict__ nf) {
  const int u = blockIdx.x;
  const int b = u / H;
  const int K = lv.K;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  __shared__ int s_tc;
  __shared__ float s_tcsum;
  __shared__ uint32_t s_bad;
  __shared__ Cand lds[4][kPlanThreads / 64];
  if (u == 0 && tid == 0) {  // pointer snapshot for the commit
    hdr[SH_START] = (int64_t)ptr[0];
    hdr[SH_END] = (int64_t)ptr[1];
  }
  if (tid == 0) {
    s_tc = -1;
    s_bad = 0;
  }
  const int64_t N = seq_len[b];
  const int32_t* s = state + (int64_t)u * 2 * K;
  int n[4] = {0, 0, 0, 0}, np[4] = {0, 0, 0, 0};
  for (int l = 0; l < K; l++) {
    n[l] = s[l];
    np[l] = s[K + l];
  }
  __syncthreads();
  if (N <= 0) {
    if (tid == 0) nf[u] = 0;
    return;
  }
  uint32_t flags = 0;
  if (N + 1 > S_max) flags = kStOverflow;
  int64_t ntot = 0;
  for (int l = 0; l < K; l++) {
    if (n[l] < 0 || np[l] != cdiv(n[l], lv.T(l))) flags |= kStBadState;
    ntot += n[l];
  }
  if (np[0] + np[1] > L || np[2] + np[3] > L || ntot > N) flags |= kStBadState;
  if (flags) {
    if (tid == 0) nf[u] = kActive | (int32_t)(flags << 8);
    return;
  }
  const int32_t* row = table + (int64_t)u * LT;
  const int64_t tc_pos = N - W;
  const Cand none{0.0f, kNoPos, 0};
  Cand best[4] = {none, none, none, none};
  for (int x = tid; x < ntot; x += kPlanThreads) {
    int l = 0, ls = x;
    while (ls >= n[l]) {  // (at most K - 1 steps)
      ls -= n[l];
      l++;
    }
    const int T = lv.T(l);
    const int32_t id = row[lv.entry(l, ls / T)];
    if (id < 0 || id >= P) {
      s_bad = 1;
      continue;
    }
    const uint8_t* pg = pages + (int64_t)id * page_bytes;
    const int32_t pos = *(const int32_t*)(pg + lv.s[l].ps + 4 * (ls % T));
    const float sum = *(const float*)(pg + lv.s[l].sc + 4 * (ls % T));
    if (l == 0 && pos == tc_pos) {  // positions are unique: one writer
      s_tc = ls;
      s_tcsum = sum;
    }
    const Cand c{sum, (l > 0 || pos <= tc_pos) ? pos : kNoPos, ls};
    if (l == 0) best[0] = min_imp(best[0], c, N);
    else if (l == 1) best[1] = min_imp(best[1], c, N);
    else if (l == 2) best[2] = min_imp(best[2], c, N);
    else best[3] = min_imp(best[3], c, N);
  }
#pragma unroll
  for (int l = 0; l < 4; l++) {
    best[l] = wave_argmin(best[l], N);
    if (lane == 0) lds[l][wid] = best[l];
  }
  __syncthreads();
  if (tid != 0) return;
#pragma unroll
  for (int l = 0; l < 4; l++) {
    best[l] = lds[l][0];
    for (int w2 = 1; w2 < kPlanThreads / 64; w2++) best[l] = min_imp(best[l], lds[l][w2], N);
  }
  int32_t* R = rec + (int64_t)u * kLRec;
  const int tcs = s_tc;
  if (s_bad || (tc_pos >= 0 && tcs < 0)) {
    nf[u] = kActive | (int32_t)(kStBadState << 8);
    return;
  }
  const double a0 = (double)(ah_head ? ah_head[u % H] : ah), aL = (double)(al_head ? al_head[u % H] : al);
  const int64_t Np = N + 1;
  auto level_of = [&](const Cand& c) { return level_of_mean(c.sum, N - 1 - c.pos, Np, K, a0, am0, am1, aL); };
  int new_slot = n[0], app = 1;
  int mv0[5] = {0, 0, 0, 0, 0}, mv1[5] = {0, 0, 0, 0, 0};
  if (tc_pos >= 0) {
    const Cand tcc{s_tcsum, (int32_t)tc_pos, tcs};
    const int lc = level_of(tcc);
    if (lc == 0) {
      const Cand v = best[0];  // t_c is a candidate: never none
      const int lvv = level_of(v);
      if (lvv != 0) {
        new_slot = v.slot;
        app = 0;
        if (lvv > 0) {
          mv0[0] = 1; mv0[1] = 0; mv0[2] = v.slot; mv0[3] = lvv; mv0[4] = n[lvv];
          app |= 1 << lvv;
        }
      }
    } else if (lc > 0) {
      new_slot = tcs;
      app = 0;
      const Cand v = min_imp(tcc, best[lc], N);
      const int lvv = v.pos == tcc.pos ? lc : level_of(v);
      if (lvv != lc) {
        mv0[0] = 1; mv0[1] = 0; mv0[2] = tcs; mv0[3] = lc; mv0[4] = v.slot;
        if (lvv > 0) {
          mv1[0] = 1; mv1[1] = lc; mv1[2] = v.slot; mv1[3] = lvv; mv1[4] = n[lvv];
          app |= 1 << lvv;
        }
      } else {
        mv0[0] = 1; mv0[1] = 0; mv0[2] = tcs; mv0[3] = lc; mv0[4] = n[lc];
        app |= 1 << lc;
      }
    } else {
      new_slot = tcs;
      app = 0;
    }
  }
  int need = -1;
  for (int l = 0; l < K; l++)
    if (((app >> l) & 1) && n[l] % lv.T(l) == 0) need = l;
  uint32_t fl = 0;
  if (need >= 0) {
    const int r = need >> 1;
    if (np[2 * r] + (2 * r + 1 < K ? np[2 * r + 1] : 0) + 1 > L) fl = kStOverflow;
  }
  R[LS_NEW] = new_slot;
  R[LS_APP] = app;
  R[LS_NEED] = need;
  for (int i = 0; i < 5; i++) {
    R[LS_MV0 + i] = mv0[i];
    R[LS_MV1 + i] = mv1[i];
  }
  nf[u] = (need >= 0 && !fl ? 1 : 0) | kActive | (int32_t)(fl << 8);
}

// One block per unit (>= D threads).  Reads first (the new token, the moved
// tokens' dequantized values: a move's source slot may be another write's
// destination), then per written token its codec over the block and its
// code ranges edited in LDS, then the stores.  A new page is zeroed first.
template <int D>
__global__ __launch_bounds__(256) void step_commit_levels_kernel(int H, int L, int LT, int64_t P, int page_bytes,
                                                                 Levels lv, const int32_t* __restrict__ seq_len,
                                                                 const uint16_t* __restrict__ k_new,
                                                                 const uint16_t* __restrict__ v_new,
                                                                 const int64_t* __restrict__ hdr,
                                                                 const int32_t* __restrict__ rec,
                                                                 const int32_t* __restrict__ nf,
                                                                 int32_t* __restrict__ table,
                                                                 int32_t* __restrict__ state, uint8_t* pages,
                                                                 uint32_t* status) {
  const int64_t u = blockIdx.x;
  const int K = lv.K;
  const int tid = threadIdx.x;
  const int b = (int)(u / H);
  __shared__ __align__(16) uint32_t img[3][64];  // per written token: K code words, then V code words
  __shared__ float red[2 * 6 * 4];
  if (!hdr[SH_COMMIT]) return;
  const int32_t w = nf[u];
  if (!(w & kActive)) return;
  const int32_t* R = rec + u * kLRec;
  int32_t* row = table + u * LT;
  int32_t* s = state + u * 2 * K;
  const int need = R[LS_NEED];
  const int32_t page = need >= 0 ? R[S_PAGE] : -1;
  if (need >= 0 && (page < 0 || page >= P)) {
    if (tid == 0) atomicOr(status, kStBadState);
    return;
  }
  // the written tokens: 0 the new token (level 0), 1 and 2 the moves
  int dl[3], ds[3], on[3];
  on[0] = 1;
  dl[0] = 0;
  ds[0] = R[LS_NEW];
  for (int m = 0; m < 2; m++) {
    on[1 + m] = R[(m ? LS_MV1 : LS_MV0) + 0];
    dl[1 + m] = R[(m ? LS_MV1 : LS_MV0) + 3];
    ds[1 + m] = R[(m ? LS_MV1 : LS_MV0) + 4];
  }
  // page id of each written token (the new page when it is its level's next
  // page), taken before anything is written: the tier state and the row
  // change at the end
  int32_t pid[3];
  for (int i = 0; i < 3; i++) {
    const int j = ds[i] / lv.T(dl[i]);
    pid[i] = (dl[i] == need && j == s[K + dl[i]]) ? page : row[lv.entry(dl[i], j)];
    if (on[i] && (pid[i] < 0 || pid[i] >= P)) {
      if (tid == 0) atomicOr(status, kStBadState);
      return;
    }
  }
  // ---- reads ----
  float x[3][2];  // [token][K, V] value of dim tid
  float msc[3] = {0.0f, 0.0f, 0.0f};
  int32_t mpos[3] = {seq_len[b], 0, 0};
  x[0][0] = tid < D ? h2f(k_new[u * D + tid]) : 0.0f;
  x[0][1] = tid < D ? h2f(v_new[u * D + tid]) : 0.0f;
  for (int m = 0; m < 2; m++) {
    x[1 + m][0] = x[1 + m][1] = 0.0f;
    if (!on[1 + m]) continue;
    const int* M = R + (m ? LS_MV1 : LS_MV0);
    const int l = M[1], sl = M[2], T = lv.T(l);
    const int32_t id = row[lv.entry(l, sl / T)];
    const uint8_t* pg = pages + (int64_t)min(max(id, 0), (int32_t)(P - 1)) * page_bytes;
    const Seg& sg = lv.s[l];
    const int t = sl % T;
    const uint32_t km = *(const uint32_t*)(pg + sg.km + 4 * t), vm = *(const uint32_t*)(pg + sg.vm + 4 * t);
    msc[1 + m] = *(const float*)(pg + sg.sc + 4 * t);
    mpos[1 + m] = *(const int32_t*)(pg + sg.ps + 4 * t);
    if (tid < D) {
      int byte, shift;
      plain_field(sg.kc, D, sg.kbits, t, tid, byte, shift);
      x[1 + m][0] = dequant(h2f((uint16_t)km), h2f((uint16_t)(km >> 16)),
                            ((uint32_t)pg[byte] >> shift) & ((1u << sg.kbits) - 1u));
      plain_field(sg.vc, D, sg.vbits, t, tid, byte, shift);
      x[1 + m][1] = dequant(h2f((uint16_t)vm), h2f((uint16_t)(vm >> 16)),
                            ((uint32_t)pg[byte] >> shift) & ((1u << sg.vbits) - 1u));
    }
  }
  for (int i = tid; i < 3 * 64; i += blockDim.x) (&img[0][0])[i] = 0u;
  __syncthreads();  // every read done before any write
  // ---- a new page starts zeroed ----
  if (need >= 0)
    for (int c = tid; c < page_bytes / 16; c += blockDim.x)
      ((uint4*)(pages + (int64_t)page * page_bytes))[c] = make_uint4(0u, 0u, 0u, 0u);
  // ---- codecs ----
  float mn[6], mx[6];
#pragma unroll
  for (int i = 0; i < 3; i++)
#pragma unroll
    for (int e = 0; e < 2; e++) mn[2 * i + e] = mx[2 * i + e] = x[i][e];
  block_minmax<D, 6>(mn, mx, red);
  uint32_t meta[3][2];
#pragma unroll
  for (int i = 0; i < 3; i++) {
    if (!on[i]) continue;
    const Seg& sg = lv.s[dl[i]];
    const int t = ds[i] % lv.T(dl[i]);
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const int bits = e ? sg.vbits : sg.kbits;
      uint16_t s16, z16;
      float sc, zc;
      codec_params(mn[2 * i + e], mx[2 * i + e], bits, s16, z16, sc, zc);
      meta[i][e] = (uint32_t)s16 | ((uint32_t)z16 << 16);
      if (tid < D) {
        // code of dim tid inside the token's own range (8-byte aligned runs)
        const int bit = tid * bits;
        lds_put(img[i] + (e ? 32 : 0), bit >> 3, bit & 7, bits, codec_code(x[i][e], sc, zc, bits));
      }
    }
    (void)t;
  }
  __syncthreads();  // the page is zeroed and every code range assembled
  // ---- stores ----
#pragma unroll
  for (int i = 0; i < 3; i++) {
    if (!on[i]) continue;
    const int l = dl[i], T = lv.T(l), t = ds[i] % T;
    const Seg& sg = lv.s[l];
    uint8_t* pg = pages + (int64_t)pid[i] * page_bytes;
    const int kw = D * sg.kbits / 32, vw = D * sg.vbits / 32;  // words per token range
    for (int c = tid; c < kw + vw; c += blockDim.x) {
      if (c < kw) ((uint32_t*)(pg + sg.kc))[t * kw + c] = img[i][c];
      else ((uint32_t*)(pg + sg.vc))[t * vw + (c - kw)] = img[i][32 + (c - kw)];
    }
    if (tid == 0) {
      *(uint32_t*)(pg + sg.km + 4 * t) = meta[i][0];
      *(uint32_t*)(pg + sg.vm + 4 * t) = meta[i][1];
      *(float*)(pg + sg.sc + 4 * t) = i == 0 ? 0.0f : msc[i];
      *(int32_t*)(pg + sg.ps + 4 * t) = mpos[i];
    }
  }
  if (tid == 0) {
    if (need >= 0) {
      row[lv.entry(need, s[K + need])] = page;
      s[K + need] += 1;
    }
    const int app = R[LS_APP];
    for (int l = 0; l < K; l++) s[l] += (app >> l) & 1;
  }
}

static hipError_t launch_step_levels(const Cfg& c, const Pool& p, int batch, const int32_t* seq_len,
                                     const uint16_t* k, const uint16_t* v, int32_t* table, int32_t* state, void* ws,
                                     hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  const StepWs w = step_carve(c, batch, ws);
  const Levels lv = levels_of(c);
  step_plan_levels_kernel<<<dim3((unsigned)U), dim3(kPlanThreads), 0, s>>>(
      c.H, c.L, c.LT, c.W, c.S_max, c.ah, c.amid[0], c.amid[1], c.al, c.ah_head, c.al_head, p.P, p.page_bytes, lv,
      seq_len, table, state, p.pages, p.ptr, w.hdr, w.rec, w.nf);
  step_coord_kernel<<<dim3(1), dim3(1024), 0, s>>>(U, p.P, kLRec, w.nf, w.rec, p.list, w.hdr, p.ptr, p.status);
  if (c.d == 128)
    step_commit_levels_kernel<128><<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.L, c.LT, p.P, p.page_bytes, lv,
                                                                           seq_len, k, v, w.hdr, w.rec, w.nf,
                                                                           table, state, p.pages, p.status);
  else
    step_commit_levels_kernel<64><<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.L, c.LT, p.P, p.page_bytes, lv,
                                                                          seq_len, k, v, w.hdr, w.rec, w.nf, table,
                                                                          state, p.pages, p.status);
  return hipGetLastError();
}

// Release with K levels: per unit the pages of level 0, 1, 2, 3 in turn
// (each level's pages in index order: left levels left to right, right
// levels right to left), appended at the reclamation pointer, units in
// order; rows reset.  One block (a release is rare): check, count, then
// write only if every released unit is consistent and the list has room.
__global__ __launch_bounds__(256) void release_levels_kernel(int H, int L, int LT, int K, int64_t P, int64_t U,
                                                             const uint8_t* __restrict__ mask,
                                                             int32_t* __restrict__ table,
                                                             int32_t* __restrict__ state, int32_t* list,
                                                             uint64_t* ptr, uint32_t* status) {
  __shared__ int64_t lds[20];
  __shared__ uint32_t sflags;
  __shared__ int s_go;
  if (threadIdx.x == 0) sflags = 0;
  __syncthreads();
  int64_t total = 0;
  for (int64_t u0 = 0; u0 < U; u0 += blockDim.x) {
    const int64_t u = u0 + threadIdx.x;
    int64_t n = 0;
    if (u < U && mask[u / H]) {
      const int32_t* s = state + u * 2 * K;
      const int32_t* row = table + u * LT;
      int np[4] = {0, 0, 0, 0};
      for (int l = 0; l < K; l++) np[l] = s[K + l];
      bool bad = np[0] < 0 || np[1] < 0 || np[2] < 0 || np[3] < 0 || np[0] + np[1] > L || np[2] + np[3] > L;
      for (int l = 0; l < K && !bad; l++)
        for (int j = 0; j < np[l]; j++) {
          const int32_t id = row[(l >> 1) * L + ((l & 1) ? L - 1 - j : j)];
          bad |= id < 0 || id >= P;
        }
      if (bad) atomicOr(&sflags, kStBadState);
      else n = np[0] + np[1] + np[2] + np[3];
    }
    int64_t t;
    block_excl_scan(n, lds, t);
    total += t;
  }
  const uint64_t start = ptr[0], end = ptr[1];
  if (threadIdx.x == 0) {
    uint32_t st = sflags;
    if (!st && (int64_t)(end - start) + total > P) st |= kStBadState;
    if (st) atomicOr(status, st);
    s_go = st == 0;
  }
  __syncthreads();
  if (!s_go) return;
  int64_t carry = 0;
  for (int64_t u0 = 0; u0 < U; u0 += blockDim.x) {
    const int64_t u = u0 + threadIdx.x;
    const bool rel = u < U && mask[u / H];
    int64_t n = 0;
    if (rel)
      for (int l = 0; l < K; l++) n += state[u * 2 * K + K + l];
    int64_t t;
    const int64_t o = block_excl_scan(n, lds, t);
    if (rel) {
      int32_t* s = state + u * 2 * K;
      int32_t* row = table + u * LT;
      uint64_t e = end + (uint64_t)(carry + o);
      for (int l = 0; l < K; l++)
        for (int j = 0; j < s[K + l]; j++) list[(e++) % (uint64_t)P] = row[(l >> 1) * L + ((l & 1) ? L - 1 - j : j)];
      for (int j = 0; j < LT; j++) row[j] = -1;
      for (int w = 0; w < 2 * K; w++) s[w] = 0;
    }
    carry += t;
  }
  if (threadIdx.x == 0) ptr[1] = end + (uint64_t)carry;
}

hipError_t launch_step_plan(const Cfg& c, const Pool& p, int batch, const int32_t* seq_len, const int32_t* table,
                            const int32_t* state, void* ws, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const StepWs w = step_carve(c, batch, ws);
  const Lay lay(c.d, c.plain, c.codec);
#define DKV_PLAN(D, PL)                                                                                    \
  step_plan_kernel<D, PL><<<dim3((unsigned)U), dim3(kPlanThreads), 0, s>>>(                                 \
      c.H, c.L, c.W, c.S_max, c.lo_en, c.ah, c.al, c.ah_head, c.al_head, p.P, p.page_bytes, lay.seg(true),  \
      lay.seg(false), seq_len, table, state, p.pages, p.ptr, w.hdr, w.rec, w.nf)
  if (c.d == 128) {
    if (c.plain) DKV_PLAN(128, true);
    else DKV_PLAN(128, false);
  } else {
    if (c.plain) DKV_PLAN(64, true);
    else DKV_PLAN(64, false);
  }
#undef DKV_PLAN
  return hipGetLastError();
}

hipError_t launch_step_coord(const Cfg& c, const Pool& p, int batch, void* ws, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const StepWs w = step_carve(c, batch, ws);
  step_coord_kernel<<<dim3(1), dim3(1024), 0, s>>>(U, p.P, kSRec, w.nf, w.rec, p.list, w.hdr, p.ptr, p.status);
  return hipGetLastError();
}

hipError_t launch_step_commit(const Cfg& c, const Pool& p, int batch, const int32_t* seq_len, const uint16_t* k,
                              const uint16_t* v, int32_t* table, int32_t* state, void* ws, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const StepWs w = step_carve(c, batch, ws);
  const dim3 grid((unsigned)U), block(256);
#define DKV_COMMIT(D, DIR)                                                                             \
  step_commit_kernel<D, DIR><<<grid, block, 0, s>>>(c.H, c.L, U, p.P, p.page_bytes, seq_len, k, v, w.hdr, \
                                                    w.rec, w.nf, p.list, table, state, p.pages, p.ptr,  \
                                                    p.status)
#define DKV_COMMIT_PLAIN(D, DIR)                                                                         \
  step_commit_plain_kernel<D, DIR><<<grid, block, 0, s>>>(c.H, c.L, U, p.P, p.page_bytes,                 \
                                                          Lay(c.d, true, c.codec), seq_len, k, v, w.hdr,  \
                                                          w.rec, w.nf, p.list, table, state, p.pages,     \
                                                          p.ptr, p.status)
  const bool direct = U <= kDirectUnits;
  if (!direct)
    step_coord_kernel<<<dim3(1), dim3(1024), 0, s>>>(U, p.P, kSRec, w.nf, w.rec, p.list, w.hdr, p.ptr, p.status);
  if (c.plain) {
    if (c.d == 128) {
      if (direct) DKV_COMMIT_PLAIN(128, true);
      else DKV_COMMIT_PLAIN(128, false);
    } else {
      if (direct) DKV_COMMIT_PLAIN(64, true);
      else DKV_COMMIT_PLAIN(64, false);
    }
  } else if (direct) {
    if (c.d == 128) DKV_COMMIT(128, true);
    else DKV_COMMIT(64, true);
  } else {
    if (c.d == 128) DKV_COMMIT(128, false);
    else DKV_COMMIT(64, false);
  }
#undef DKV_COMMIT_PLAIN
#undef DKV_COMMIT
  return hipGetLastError();
}

hipError_t launch_step(const Cfg& c, const Pool& p, int batch, const int32_t* seq_len, const uint16_t* k,
                       const uint16_t* v, int32_t* table, int32_t* state, void* ws, hipStream_t s) {
  if (c.K >= 3) {
    if ((int64_t)batch * c.H == 0) return hipSuccess;
    return launch_step_levels(c, p, batch, seq_len, k, v, table, state, ws, s);
  }
  hipError_t e = launch_step_plan(c, p, batch, seq_len, table, state, ws, s);
  if (e != hipSuccess) return e;
  return launch_step_commit(c, p, batch, seq_len, k, v, table, state, ws, s);
}

// ---------------------------------------------------------------------------
// release
// ---------------------------------------------------------------------------
size_t release_workspace(const Cfg& c, int batch) {
  return align_up(16 * sizeof(int64_t), 256) + align_up((size_t)batch * c.H * sizeof(int64_t), 256);
}

// One workgroup per unit: off[u] = 1 when a released unit's row holds a page
// id outside the pool in its used entries (such an id would enter the free
// list), else 0.  The plan kernel reads the flag before it overwrites off[u].
__global__ __launch_bounds__(256) void release_check_kernel(int H, int L, int64_t P,
                                                            const uint8_t* __restrict__ mask,
                                                            const int32_t* __restrict__ table,
                                                            const int32_t* __restrict__ state,
                                                            int64_t* __restrict__ off) {
  const int64_t u = blockIdx.x;
  int bad = 0;
  if (mask[u / H]) {
    const int32_t ph = state[4 * u + 2], pl = state[4 * u + 3];
    if (ph >= 0 && pl >= 0 && ph + pl <= L) {
      const int32_t* row = table + u * L;
      for (int j = threadIdx.x; j < ph + pl; j += blockDim.x) {
        const int32_t id = j < ph ? row[j] : row[L - 1 - (j - ph)];
        bad |= id < 0 || id >= P;
      }
    }
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) off[u] = bad ? 1 : 0;
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
      if (ph < 0 || pl < 0 || ph + pl > L || off[u] != 0) atomicOr(&sflags, kStBadState);
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
  if (c.K >= 3) {
    release_levels_kernel<<<dim3(1), dim3(256), 0, s>>>(c.H, c.L, c.LT, c.K, p.P, U, mask, table, state, p.list,
                                                        p.ptr, p.status);
    return hipGetLastError();
  }
  int64_t* hdr = (int64_t*)ws;
  int64_t* off = (int64_t*)((uint8_t*)ws + align_up(16 * sizeof(int64_t), 256));
  release_check_kernel<<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.L, p.P, mask, table, state, off);
  release_plan_kernel<<<dim3(1), dim3(1024), 0, s>>>(c.H, c.L, U, p.P, mask, state, off, hdr, p.ptr, p.status);
  release_write_kernel<<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.L, p.P, mask, off, hdr, p.list, table,
                                                               state);
  return hipGetLastError();
}

}  // namespace dkv
