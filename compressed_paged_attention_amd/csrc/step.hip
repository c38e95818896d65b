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
// Kernels: plan (one block per unit: slot scans), coord (one block: prefix
// sum over page demand, capacity check, page ids, pointer), commit (one block
// per unit: new page zero-filled, requantization, new token).
//
// Release ("Memory management": a finished request's pages are reclaimed):
// plan (one block: prefix sum over released page counts) and write (one block
// per unit: high pages left to right, then low pages right to left, appended
// at the reclamation pointer; rows reset).
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

namespace dkv {

constexpr int kSRec = 12;
enum { S_ACTIVE = 0, S_NEWHI, S_HIAPP, S_LOSRC, S_LOSLOT, S_LOAPP, S_NEED, S_PAGE, S_FLAGS };
enum { SH_COMMIT = 0, SH_START, SH_D };

size_t step_workspace(const Cfg& c, int batch) {
  return align_up(16 * sizeof(int64_t), 256) + align_up((size_t)batch * c.H * kSRec * sizeof(int32_t), 256);
}

struct Cand {
  float sum;
  int cnt, pos, slot;  // slot < 0 with pos >= 0: the t_c candidate of the low scan
  bool has;
};

__device__ inline bool less_imp(const Cand& a, const Cand& b) {
  if (!a.has) return false;
  if (!b.has) return true;
  const double l = (double)a.sum * (double)b.cnt, r = (double)b.sum * (double)a.cnt;
  if (l != r) return l < r;
  return a.pos < b.pos;
}

__device__ inline Cand shfl_cand(const Cand& c, int o) {
  Cand r;
  r.sum = __shfl_xor(c.sum, o, 64);
  r.cnt = __shfl_xor(c.cnt, o, 64);
  r.pos = __shfl_xor(c.pos, o, 64);
  r.slot = __shfl_xor(c.slot, o, 64);
  r.has = __shfl_xor((int)c.has, o, 64) != 0;
  return r;
}

__device__ Cand block_argmin(Cand c, Cand* lds) {
  for (int o = 32; o >= 1; o >>= 1) {
    Cand t = shfl_cand(c, o);
    if (less_imp(t, c)) c = t;
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (lane == 0) lds[wid] = c;
  __syncthreads();
  Cand best = lds[0];
  for (int w = 1; w < nw; w++)
    if (less_imp(lds[w], best)) best = lds[w];
  __syncthreads();
  return best;
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

template <int D>
__global__ __launch_bounds__(256) void step_plan_kernel(int H, int L, int W, int S_max, int lo_en, float ah,
                                                        float al, int64_t P, int page_bytes,
                                                        const int32_t* __restrict__ seq_len,
                                                        const int32_t* __restrict__ table,
                                                        const int32_t* __restrict__ state,
                                                        const uint8_t* __restrict__ pages,
                                                        int32_t* __restrict__ rec) {
  const int64_t u = blockIdx.x;
  const int b = (int)(u / H);
  const int tid = threadIdx.x;
  int32_t* R = rec + u * kSRec;
  const int64_t N = seq_len[b];
  if (N <= 0) {
    if (tid == 0) {
      R[S_ACTIVE] = 0;
      R[S_FLAGS] = 0;
      R[S_NEED] = 0;
    }
    return;
  }
  const int32_t* s4 = state + 4 * u;
  const int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  const int32_t* row = table + u * L;
  __shared__ uint32_t sflags;
  __shared__ Cand lds[4];
  if (tid == 0) sflags = 0;
  __syncthreads();
  uint32_t flags = 0;
  if (N + 1 > S_max) flags = kStOverflow;
  else if (nh < 0 || nl < 0 || ph != cdiv(nh, kHiTokens) || pl != cdiv(nl, kLoTokens) || nh + nl > N ||
           ph + pl > L)
    flags = kStBadState;
  if (!flags) {
    for (int j = tid; j < ph + pl; j += blockDim.x) {
      const int32_t id = j < ph ? row[j] : row[L - 1 - (j - ph)];
      if (id < 0 || id >= P) atomicOr(&sflags, kStBadState);
    }
  }
  __syncthreads();
  flags |= sflags;
  if (flags) {
    if (tid == 0) {
      R[S_ACTIVE] = 1;
      R[S_FLAGS] = (int32_t)flags;
      R[S_NEED] = 0;
    }
    return;
  }
  const Seg sh = tier_seg(D, true), sl = tier_seg(D, false);
  const int64_t Np = N + 1, tc_pos = N - W;
  const double dah = (double)ah, dal = (double)al;
  int new_hi = nh, hi_app = 1, lo_src = -1, lo_slot = 0, lo_app = 0;
  if (tc_pos >= 0) {
    // one pass over the high tier: t_c's slot and the least important
    // non-window token (position <= N - W)
    __shared__ int s_tc;
    __shared__ float s_tcsum;
    if (tid == 0) s_tc = -1;
    __syncthreads();
    Cand best{0.0f, 0, 0, 0, false};
    for (int s = tid; s < nh; s += blockDim.x) {
      const uint8_t* pg = pages + (int64_t)row[s >> 4] * page_bytes;
      const int idx = s & 15;
      const int32_t pos = *(const int32_t*)(pg + sh.ps + 4 * idx);
      const float sum = *(const float*)(pg + sh.sc + 4 * idx);
      if (pos == tc_pos) {  // positions are unique: one writer
        s_tc = s;
        s_tcsum = sum;
      }
      if (pos <= tc_pos) {
        Cand c{sum, (int)(N - 1 - pos), pos, s, true};
        if (less_imp(c, best)) best = c;
      }
    }
    const Cand v = block_argmin(best, lds);  // its barriers publish s_tc
    const int tcs = s_tc;
    const float tcsum = s_tcsum;
    // t_c is in the high tier by construction; a missing t_c is bad state
    if (tcs < 0) {
      if (tid == 0) {
        R[S_ACTIVE] = 1;
        R[S_FLAGS] = kStBadState;
        R[S_NEED] = 0;
      }
      return;
    }
    const int cls = classify_mean(tcsum, W - 1, Np, lo_en, dah, dal);
    if (cls == kTierHi) {
      const int vcls = classify_mean(v.sum, v.cnt, Np, lo_en, dah, dal);
      if (vcls == kTierLo) {
        lo_src = v.slot;
        lo_slot = nl;
        lo_app = 1;
        new_hi = v.slot;
        hi_app = 0;
      } else if (vcls == kTierPrune) {
        new_hi = v.slot;
        hi_app = 0;
      }
    } else if (cls == kTierLo) {
      lo_src = tcs;
      new_hi = tcs;
      hi_app = 0;
      Cand bl{0.0f, 0, 0, 0, false};
      if (tid == 0) bl = Cand{tcsum, W - 1, (int)tc_pos, -1, true};
      for (int s = tid; s < nl; s += blockDim.x) {
        const uint8_t* pg = pages + (int64_t)row[L - 1 - (s >> 5)] * page_bytes;
        const int idx = s & 31;
        const int32_t pos = *(const int32_t*)(pg + sl.ps + 4 * idx);
        const float sum = *(const float*)(pg + sl.sc + 4 * idx);
        Cand c{sum, (int)(N - 1 - pos), pos, s, true};
        if (less_imp(c, bl)) bl = c;
      }
      Cand lv = block_argmin(bl, lds);
      if (lv.slot >= 0 && classify_mean(lv.sum, lv.cnt, Np, lo_en, dah, dal) == kTierPrune) {
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
  if (tid == 0) {
    int need = 0;
    if (hi_app && nh % kHiTokens == 0) need = kTierHi;
    if (lo_app && nl % kLoTokens == 0) need = kTierLo;
    uint32_t fl = 0;
    if (need && ph + pl + 1 > L) fl = kStOverflow;
    R[S_ACTIVE] = 1;
    R[S_NEWHI] = new_hi;
    R[S_HIAPP] = hi_app;
    R[S_LOSRC] = lo_src;
    R[S_LOSLOT] = lo_slot;
    R[S_LOAPP] = lo_app;
    R[S_NEED] = fl ? 0 : need;
    R[S_PAGE] = -1;
    R[S_FLAGS] = (int32_t)fl;
  }
}

__global__ __launch_bounds__(1024) void step_coord_kernel(int64_t U, int64_t P, int32_t* __restrict__ rec,
                                                          const int32_t* list, int64_t* __restrict__ hdr,
                                                          uint64_t* ptr, uint32_t* status) {
  __shared__ int64_t lds[20];
  __shared__ uint32_t sflags;
  __shared__ int scommit;
  if (threadIdx.x == 0) sflags = 0;
  __syncthreads();
  int64_t total = 0;
  for (int64_t base = 0; base < U; base += blockDim.x) {
    const int64_t u = base + threadIdx.x;
    int64_t need = 0;
    if (u < U) {
      const int32_t* R = rec + u * kSRec;
      if (R[S_ACTIVE]) {
        if (R[S_FLAGS]) atomicOr(&sflags, (uint32_t)R[S_FLAGS]);
        need = R[S_NEED] != 0;
      }
    }
    int64_t t;
    block_excl_scan(need, lds, t);
    total += t;
  }
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
      int64_t need = 0;
      if (u < U) {
        const int32_t* R = rec + u * kSRec;
        need = R[S_ACTIVE] && R[S_NEED] != 0;
      }
      int64_t t;
      const int64_t off = block_excl_scan(need, lds, t);
      if (need) rec[u * kSRec + S_PAGE] = list[(start + (uint64_t)(carry + off)) % (uint64_t)P];
      carry += t;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    hdr[SH_COMMIT] = commit;
    hdr[SH_START] = (int64_t)start;
    hdr[SH_D] = total;
    if (commit) ptr[0] = start + (uint64_t)total;
  }
}

// Clears and sets a `bits`-wide field of a page through 32-bit atomics (other
// fields of the same word may be written concurrently by other threads).
__device__ inline void put_field(uint8_t* page, int byte, int shift, int bits, uint32_t val) {
  uint32_t* w = (uint32_t*)(page + (byte & ~3));
  const int sh = 8 * (byte & 3) + shift;
  const uint32_t mask = ((1u << bits) - 1u) << sh;
  atomicAnd(w, ~mask);
  atomicOr(w, (val << sh) & mask);
}

__device__ inline uint32_t get_field(const uint8_t* page, int byte, int shift, int bits) {
  return ((uint32_t)page[byte] >> shift) & ((1u << bits) - 1u);
}

template <int D>
__device__ void store_token(uint8_t* pg, bool hi, int idx, float x_k, float x_v, float* red,
                            float score, int32_t pos) {
  // min/max over the D values held by threads 0..D-1
  const int tid = threadIdx.x;
  const bool act = tid < D;
  float kmn = act ? x_k : INFINITY, kmx = act ? x_k : -INFINITY;
  float vmn = act ? x_v : INFINITY, vmx = act ? x_v : -INFINITY;
  kmn = wave_min(kmn);
  kmx = wave_max(kmx);
  vmn = wave_min(vmn);
  vmx = wave_max(vmx);
  const int lane = tid & 63, wid = tid >> 6;
  if (lane == 0) {
    red[4 * wid + 0] = kmn;
    red[4 * wid + 1] = kmx;
    red[4 * wid + 2] = vmn;
    red[4 * wid + 3] = vmx;
  }
  __syncthreads();
  kmn = red[0];
  kmx = red[1];
  vmn = red[2];
  vmx = red[3];
  for (int w = 1; w < (D + 63) / 64; w++) {
    kmn = fminf(kmn, red[4 * w + 0]);
    kmx = fmaxf(kmx, red[4 * w + 1]);
    vmn = fminf(vmn, red[4 * w + 2]);
    vmx = fmaxf(vmx, red[4 * w + 3]);
  }
  __syncthreads();
  const Seg sg = tier_seg(D, hi);
  uint16_t ks16, kz16, vs16, vz16;
  float ks, kz, vs, vz;
  codec_params(kmn, kmx, sg.kbits, ks16, kz16, ks, kz);
  codec_params(vmn, vmx, sg.vbits, vs16, vz16, vs, vz);
  if (act) {
    int byte, shift;
    k_field(D, hi, idx, tid, byte, shift);
    put_field(pg, byte, shift, sg.kbits, codec_code(x_k, ks, kz, sg.kbits));
    v_field(D, hi, idx, tid, byte, shift);
    put_field(pg, byte, shift, sg.vbits, codec_code(x_v, vs, vz, sg.vbits));
  }
  if (tid == 0) {
    *(uint32_t*)(pg + sg.km + 4 * idx) = (uint32_t)ks16 | ((uint32_t)kz16 << 16);
    *(uint32_t*)(pg + sg.vm + 4 * idx) = (uint32_t)vs16 | ((uint32_t)vz16 << 16);
    *(float*)(pg + sg.sc + 4 * idx) = score;
    *(int32_t*)(pg + sg.ps + 4 * idx) = pos;
  }
}

template <int D>
__global__ __launch_bounds__(256) void step_commit_kernel(int H, int L, int64_t P, int page_bytes,
                                                          const int32_t* __restrict__ seq_len,
                                                          const uint16_t* __restrict__ k_new,
                                                          const uint16_t* __restrict__ v_new,
                                                          const int64_t* __restrict__ hdr,
                                                          const int32_t* __restrict__ rec,
                                                          int32_t* __restrict__ table,
                                                          int32_t* __restrict__ state, uint8_t* pages,
                                                          uint32_t* status) {
  if (!hdr[SH_COMMIT]) return;
  const int64_t u = blockIdx.x;
  const int32_t* R = rec + u * kSRec;
  if (!R[S_ACTIVE]) return;
  const int b = (int)(u / H), h = (int)(u % H);
  const int tid = threadIdx.x;
  int32_t* row = table + u * L;
  int32_t* s4 = state + 4 * u;
  const int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  const int need = R[S_NEED];
  __shared__ float red[16];
  if (need) {
    const int32_t id = R[S_PAGE];
    if (id < 0 || id >= P) {
      if (tid == 0) atomicOr(status, kStBadState);
      return;
    }
    uint4* dst = (uint4*)(pages + (int64_t)id * page_bytes);
    for (int c = tid; c < page_bytes / 16; c += blockDim.x) dst[c] = make_uint4(0, 0, 0, 0);
    if (tid == 0) {
      if (need == kTierHi) row[ph] = id;
      else row[L - 1 - pl] = id;
    }
  }
  __syncthreads();  // workgroup scope suffices: no device-scope fence (it flushes L2)
  const Seg sh = tier_seg(D, true);
  const int lo_src = R[S_LOSRC];
  if (lo_src >= 0) {
    // requantize a high token to the low tier, from its dequantized values
    const uint8_t* src = pages + (int64_t)row[lo_src >> 4] * page_bytes;
    const int si = lo_src & 15;
    const uint32_t km = *(const uint32_t*)(src + sh.km + 4 * si);
    const uint32_t vm = *(const uint32_t*)(src + sh.vm + 4 * si);
    const float sc = *(const float*)(src + sh.sc + 4 * si);
    const int32_t pos = *(const int32_t*)(src + sh.ps + 4 * si);
    float xk = 0.0f, xv = 0.0f;
    if (tid < D) {
      int byte, shift;
      k_field(D, true, si, tid, byte, shift);
      xk = dequant(h2f((uint16_t)km), h2f((uint16_t)(km >> 16)), get_field(src, byte, shift, 8));
      v_field(D, true, si, tid, byte, shift);
      xv = dequant(h2f((uint16_t)vm), h2f((uint16_t)(vm >> 16)), get_field(src, byte, shift, 4));
    }
    const int lo_slot = R[S_LOSLOT];
    uint8_t* dstp = pages + (int64_t)row[L - 1 - (lo_slot >> 5)] * page_bytes;
    store_token<D>(dstp, false, lo_slot & 31, xk, xv, red, sc, pos);
  }
  __syncthreads();  // workgroup scope suffices: no device-scope fence (it flushes L2)
  {
    const int64_t rowi = ((int64_t)b * H + h) * D + tid;
    const float xk = tid < D ? h2f(k_new[rowi]) : 0.0f;
    const float xv = tid < D ? h2f(v_new[rowi]) : 0.0f;
    const int slot = R[S_NEWHI];
    uint8_t* dstp = pages + (int64_t)row[slot >> 4] * page_bytes;
    store_token<D>(dstp, true, slot & 15, xk, xv, red, 0.0f, seq_len[b]);
  }
  if (tid == 0) {
    s4[0] = nh + R[S_HIAPP];
    s4[1] = nl + R[S_LOAPP];
    s4[2] = ph + (need == kTierHi);
    s4[3] = pl + (need == kTierLo);
  }
}

hipError_t launch_step(const Cfg& c, const Pool& p, int batch, const int32_t* seq_len, const uint16_t* k,
                       const uint16_t* v, int32_t* table, int32_t* state, void* ws, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  int64_t* hdr = (int64_t*)ws;
  int32_t* rec = (int32_t*)((uint8_t*)ws + align_up(16 * sizeof(int64_t), 256));
  if (c.d == 128)
    step_plan_kernel<128><<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.L, c.W, c.S_max, c.lo_en, c.ah, c.al,
                                                                  p.P, p.page_bytes, seq_len, table, state,
                                                                  p.pages, rec);
  else
    step_plan_kernel<64><<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.L, c.W, c.S_max, c.lo_en, c.ah, c.al,
                                                                 p.P, p.page_bytes, seq_len, table, state,
                                                                 p.pages, rec);
  step_coord_kernel<<<dim3(1), dim3(1024), 0, s>>>(U, p.P, rec, p.list, hdr, p.ptr, p.status);
  if (c.d == 128)
    step_commit_kernel<128><<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.L, p.P, p.page_bytes, seq_len, k, v,
                                                                    hdr, rec, table, state, p.pages, p.status);
  else
    step_commit_kernel<64><<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.L, p.P, p.page_bytes, seq_len, k, v,
                                                                   hdr, rec, table, state, p.pages, p.status);
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
