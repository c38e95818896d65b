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
         align_up(U * sizeof(int32_t), 256);
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

hipError_t launch_step_plan(const Cfg& c, const Pool& p, int batch, const int32_t* seq_len, const int32_t* table,
                            const int32_t* state, void* ws, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const StepWs w = step_carve(c, batch, ws);
#define DKV_PLAN(D)                                                                                       \
  step_plan_kernel<D><<<dim3((unsigned)U), dim3(kPlanThreads), 0, s>>>(c.H, c.L, c.W, c.S_max, c.lo_en, c.ah, \
                                                                       c.al, p.P, p.page_bytes, seq_len, table, \
                                                                       state, p.pages, p.ptr, w.hdr, w.rec, w.nf)
  if (c.d == 128) DKV_PLAN(128);
  else DKV_PLAN(64);
#undef DKV_PLAN
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
  if (U <= kDirectUnits) {
    if (c.d == 128) DKV_COMMIT(128, true);
    else DKV_COMMIT(64, true);
  } else {
    step_coord_kernel<<<dim3(1), dim3(1024), 0, s>>>(U, p.P, w.nf, w.rec, p.list, w.hdr, p.ptr, p.status);
    if (c.d == 128) DKV_COMMIT(128, false);
    else DKV_COMMIT(64, false);
  }
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
