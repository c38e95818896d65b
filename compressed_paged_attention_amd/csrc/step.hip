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
  return align_up(16 * sizeof(int64_t), 256) + align_up(U * kSRec * sizeof(int32_t), 256) +
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
  step_coord_kernel<<<dim3(1), dim3(1024), 0, s>>>(U, p.P, w.nf, w.rec, p.list, w.hdr, p.ptr, p.status);
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
    step_coord_kernel<<<dim3(1), dim3(1024), 0, s>>>(U, p.P, w.nf, w.rec, p.list, w.hdr, p.ptr, p.status);
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
  int64_t* hdr = (int64_t*)ws;
  int64_t* off = (int64_t*)((uint8_t*)ws + align_up(16 * sizeof(int64_t), 256));
  release_check_kernel<<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.L, p.P, mask, table, state, off);
  release_plan_kernel<<<dim3(1), dim3(1024), 0, s>>>(c.H, c.L, U, p.P, mask, state, off, hdr, p.ptr, p.status);
  release_write_kernel<<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.L, p.P, mask, off, hdr, p.list, table,
                                                               state);
  return hipGetLastError();
}

}  // namespace dkv
