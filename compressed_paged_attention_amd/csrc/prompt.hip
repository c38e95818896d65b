// prompt.hip -- prompt-phase KV compaction (DiffKV notes, "Memory
// management": parallel KV compaction = per-head planning + a prefix sum that
// maps the heads' page needs onto the circular free page list; Fig 6 prompt
// workflow; bidirectional page table; unified pages).
//
// Per unit u = (request r, KV head h), units in r-major order:
//   1. a conservative block of k = ceil(N/16) pages (all tokens assumed
//      high precision) from the allocation pointer;
//   2. the plan: n_hp = ceil(n_hi/16) high pages, n_lp = ceil(n_lo/32) low
//      pages; high pages take the block from the left, low pages from the
//      right (table row filled left->right / right->left);
//   3. the unused middle of the block goes back at the reclamation pointer;
//   4. when n_hp + n_lp = k + 1 (possible: 17 high + 15 low tokens in 32)
//      the unit takes one more page after the frees as its innermost low page.
// All or nothing: the plan kernel checks every unit and the pool first and
// commits only if everything fits.
//
// Kernels (one stream, in order):
//   count   (chunks x units)  per-chunk high/low counts
//   plan    (1 block)         per-unit plan, exclusive scans, capacity check,
//                             pointer update (later kernels use a snapshot)
//   scatter (chunks x units)  slot -> position lists (stable per tier) and the
//                             table rows from the conservative block
//   list    (units)           frees appended at the old end pointer, extra pages
//   pack    (persistent)      one page per iteration: quantize its tokens into
//                             an LDS image of the page, write the whole page
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

namespace dkv {

constexpr int kChunk = 2048;  // tokens per count/scatter block
constexpr int kRec = 12;      // int64 fields per unit record
enum { R_K = 0, R_HP, R_LP, R_KOFF, R_FOFF, R_EOFF, R_POFF, R_NH, R_NL, R_N, R_BASE, R_FLAGS };
enum { H_K = 0, H_F, H_E, H_COMMIT, H_START, H_END, H_PAGES };

struct PromptWs {
  int64_t* hdr;
  int64_t* rec;
  int32_t* chunks;
  int32_t* pos;
  int32_t* freed;
};

static inline int num_chunks(const Cfg& c) { return (c.S_max + kChunk - 1) / kChunk; }

static PromptWs carve(const Cfg& c, int batch, int64_t total, void* ws, size_t* bytes) {
  const int64_t U = (int64_t)batch * c.H;
  const int C = num_chunks(c);
  size_t off = 0;
  PromptWs w;
  uint8_t* b = (uint8_t*)ws;
  w.hdr = (int64_t*)(b + off);
  off = align_up(off + 16 * sizeof(int64_t), 256);
  w.rec = (int64_t*)(b + off);
  off = align_up(off + (size_t)U * kRec * sizeof(int64_t), 256);
  w.chunks = (int32_t*)(b + off);
  off = align_up(off + (size_t)U * C * 2 * sizeof(int32_t), 256);
  w.pos = (int32_t*)(b + off);
  off = align_up(off + (size_t)c.H * total * sizeof(int32_t), 256);
  w.freed = (int32_t*)(b + off);
  off = align_up(off + (size_t)U * c.L * sizeof(int32_t), 256);
  if (bytes) *bytes = off;
  return w;
}

size_t prompt_workspace(const Cfg& c, int batch, int64_t total) {
  size_t n = 0;
  carve(c, batch, total, nullptr, &n);
  return n;
}

__device__ inline void block_sum2(int& a, int& b, int* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (lane == 0) {
    red[2 * wid] = a;
    red[2 * wid + 1] = b;
  }
  __syncthreads();
  a = 0;
  b = 0;
  for (int w = 0; w < nw; w++) {
    a += red[2 * w];
    b += red[2 * w + 1];
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void prompt_count_kernel(int H, int64_t total, int C,
                                                           const int64_t* __restrict__ cu,
                                                           const uint8_t* __restrict__ tiers,
                                                           int32_t* __restrict__ chunks) {
  const int c = blockIdx.x;
  const int64_t u = blockIdx.y;
  const int r = (int)(u / H), h = (int)(u % H);
  const int64_t b0 = cu[r], N = cu[r + 1] - b0;
  const int64_t t0 = (int64_t)c * kChunk;
  const int64_t t1 = N < t0 + kChunk ? N : t0 + kChunk;
  int nh = 0, nl = 0;
  if (b0 >= 0 && N > 0 && cu[r + 1] <= total) {
    const uint8_t* t = tiers + (int64_t)h * total + b0;
    for (int64_t p = t0 + threadIdx.x; p < t1; p += blockDim.x) {
      const uint8_t v = t[p];
      nh += v == kTierHi;
      nl += v == kTierLo;
    }
  }
  __shared__ int red[8];
  block_sum2(nh, nl, red);
  if (threadIdx.x == 0) {
    chunks[(u * C + c) * 2 + 0] = nh;
    chunks[(u * C + c) * 2 + 1] = nl;
  }
}

__global__ __launch_bounds__(1024) void prompt_plan_kernel(int H, int L, int S_max, int batch, int C,
                                                           int64_t total, const int64_t* __restrict__ cu,
                                                           const int32_t* __restrict__ state,
                                                           int32_t* __restrict__ chunks,
                                                           int64_t* __restrict__ rec,
                                                           int64_t* __restrict__ hdr, uint64_t* ptr,
                                                           uint32_t* status) {
  __shared__ int64_t lds[20];
  __shared__ uint32_t sflags;
  if (threadIdx.x == 0) sflags = 0;
  __syncthreads();
  const int64_t U = (int64_t)batch * H;
  int64_t carry[4] = {0, 0, 0, 0};  // K, F, E, pages
  for (int64_t base = 0; base < U; base += blockDim.x) {
    const int64_t u = base + threadIdx.x;
    int64_t k = 0, hp = 0, lp = 0, f = 0, e = 0, nh = 0, nl = 0, N = 0, b0 = 0;
    uint32_t flags = 0;
    if (u < U) {
      const int r = (int)(u / H);
      b0 = cu[r];
      const int64_t b1 = cu[r + 1];
      N = b1 - b0;
      if (b0 < 0 || N < 0 || b1 > total || (r == 0 && b0 != 0)) {
        flags |= kStBadState;
        N = 0;
      } else if (N > 0) {
        const int32_t* s = state + 4 * u;
        if (s[0] | s[1] | s[2] | s[3]) flags |= kStBadState;
        if (N > S_max) {
          flags |= kStOverflow;
        } else {
          int64_t ah = 0, al = 0;
          for (int c = 0; c < C; c++) {
            int32_t* ch = chunks + (u * C + c) * 2;
            const int32_t a = ch[0], b = ch[1];
            ch[0] = (int32_t)ah;
            ch[1] = (int32_t)al;
            ah += a;
            al += b;
          }
          nh = ah;
          nl = al;
          k = cdiv(N, kHiTokens);
          hp = cdiv(nh, kHiTokens);
          lp = cdiv(nl, kLoTokens);
          if (k > L || hp + lp > L) flags |= kStOverflow;
          if (nh + nl > N) flags |= kStBadState;
          f = k > hp + lp ? k - hp - lp : 0;
          e = hp + lp > k ? hp + lp - k : 0;
        }
      }
    }
    if (flags) atomicOr(&sflags, flags);
    int64_t tot[4];
    const int64_t ok = block_excl_scan(k, lds, tot[0]);
    const int64_t of = block_excl_scan(f, lds, tot[1]);
    const int64_t oe = block_excl_scan(e, lds, tot[2]);
    const int64_t op = block_excl_scan(hp + lp, lds, tot[3]);
    if (u < U) {
      int64_t* R = rec + u * kRec;
      R[R_K] = k;
      R[R_HP] = hp;
      R[R_LP] = lp;
      R[R_KOFF] = carry[0] + ok;
      R[R_FOFF] = carry[1] + of;
      R[R_EOFF] = carry[2] + oe;
      R[R_POFF] = carry[3] + op;
      R[R_NH] = nh;
      R[R_NL] = nl;
      R[R_N] = N;
      R[R_BASE] = b0;
      R[R_FLAGS] = flags;
    }
    for (int i = 0; i < 4; i++) carry[i] += tot[i];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t start = ptr[0], end = ptr[1];
    const int64_t free0 = (int64_t)(end - start);
    uint32_t st = sflags;
    const int64_t K = carry[0], F = carry[1], E = carry[2];
    if (!st && (K > free0 || K - F + E > free0)) st |= kStExhausted;
    hdr[H_K] = K;
    hdr[H_F] = F;
    hdr[H_E] = E;
    hdr[H_START] = (int64_t)start;
    hdr[H_END] = (int64_t)end;
    hdr[H_PAGES] = carry[3];
    hdr[H_COMMIT] = st == 0;
    if (st) {
      atomicOr(status, st);
    } else {
      ptr[0] = start + (uint64_t)(K + E);
      ptr[1] = end + (uint64_t)F;
    }
  }
}

// Slot -> position lists (high slots from the left of the unit's token range,
// low slots from the right), plus the table rows from the conservative block.
__global__ __launch_bounds__(256) void prompt_scatter_kernel(int H, int L, int C, int64_t total, int64_t P,
                                                             const uint8_t* __restrict__ tiers,
                                                             const int64_t* __restrict__ hdr,
                                                             const int64_t* __restrict__ rec,
                                                             const int32_t* __restrict__ chunks,
                                                             const int32_t* __restrict__ list,
                                                             int32_t* __restrict__ pos_list,
                                                             int32_t* __restrict__ freed,
                                                             int32_t* __restrict__ table,
                                                             int32_t* __restrict__ state) {
  if (!hdr[H_COMMIT]) return;
  const int c = blockIdx.x;
  const int64_t u = blockIdx.y;
  const int h = (int)(u % H);
  const int64_t* R = rec + u * kRec;
  const int64_t N = R[R_N], b0 = R[R_BASE];
  if (N <= 0) return;
  const int64_t t0 = (int64_t)c * kChunk;
  if (t0 < N) {
    const uint8_t* t = tiers + (int64_t)h * total + b0;
    constexpr int kPer = kChunk / 256;
    const int64_t p0 = t0 + (int64_t)threadIdx.x * kPer;
    uint8_t v[kPer];
    int lh = 0, ll = 0;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int64_t p = p0 + i;
      v[i] = p < N ? t[p] : (uint8_t)kTierPrune;
      lh += v[i] == kTierHi;
      ll += v[i] == kTierLo;
    }
    __shared__ int lds[20];
    int th, tl;
    int bh = block_excl_scan(lh, lds, th);
    int bl = block_excl_scan(ll, lds, tl);
    bh += chunks[(u * C + c) * 2 + 0];
    bl += chunks[(u * C + c) * 2 + 1];
    int32_t* pl = pos_list + (int64_t)h * total + b0;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int64_t p = p0 + i;
      if (v[i] == kTierHi) pl[bh++] = (int32_t)p;
      else if (v[i] == kTierLo) pl[N - 1 - (bl++)] = (int32_t)p;
    }
  }
  if (c == 0) {
    const int64_t k = R[R_K], hp = R[R_HP], lp = R[R_LP];
    const uint64_t start = (uint64_t)hdr[H_START] + (uint64_t)R[R_KOFF];
    int32_t* row = table + u * L;
    for (int64_t i = threadIdx.x; i < k; i += blockDim.x) {
      const int32_t id = list[(start + (uint64_t)i) % (uint64_t)P];
      if (i < hp) row[i] = id;
      else if (i >= k - lp) row[L - 1 - (k - 1 - i)] = id;
      else freed[R[R_FOFF] + (i - hp)] = id;
    }
    if (threadIdx.x == 0) {
      int32_t* s = state + 4 * u;
      s[0] = (int32_t)R[R_NH];
      s[1] = (int32_t)R[R_NL];
      s[2] = (int32_t)hp;
      s[3] = (int32_t)lp;
    }
  }
}

// Frees appended at the old reclamation pointer; extra pages taken after
// them.  A list slot read here (logical index below the old end) is never
// one of the slots written here: the written logical indices sit exactly P
// above indices this call already consumed.
__global__ __launch_bounds__(256) void prompt_list_kernel(int L, int64_t P, const int64_t* __restrict__ hdr,
                                                          const int64_t* __restrict__ rec,
                                                          const int32_t* __restrict__ freed,
                                                          int32_t* list, int32_t* __restrict__ table) {
  if (!hdr[H_COMMIT]) return;
  const int64_t u = blockIdx.x;
  const int64_t* R = rec + u * kRec;
  if (R[R_N] <= 0) return;
  const int64_t k = R[R_K], hp = R[R_HP], lp = R[R_LP];
  const int64_t f = k > hp + lp ? k - hp - lp : 0;
  const uint64_t end0 = (uint64_t)hdr[H_END];
  for (int64_t i = threadIdx.x; i < f; i += blockDim.x)
    list[(end0 + (uint64_t)(R[R_FOFF] + i)) % (uint64_t)P] = freed[R[R_FOFF] + i];
  if (hp + lp > k && threadIdx.x == 0) {
    const uint64_t x = (uint64_t)hdr[H_START] + (uint64_t)hdr[H_K] + (uint64_t)R[R_EOFF];
    const int32_t id = x < end0 ? list[x % (uint64_t)P] : freed[x - end0];
    table[u * L + (L - lp)] = id;
  }
}

template <int D>
__global__ __launch_bounds__(256) void prompt_pack_kernel(int H, int L, int64_t total, int64_t U, int64_t P,
                                                          int page_bytes, const int64_t* __restrict__ hdr,
                                                          const int64_t* __restrict__ rec,
                                                          const int32_t* __restrict__ pos_list,
                                                          const int32_t* __restrict__ table,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const float* __restrict__ scores,
                                                          uint8_t* __restrict__ pages, uint32_t* status) {
  if (!hdr[H_COMMIT]) return;
  const int64_t TP = hdr[H_PAGES];
  __shared__ uint32_t img[page_bytes_for(D) / 4];
  const int tid = threadIdx.x;
  for (int64_t item = blockIdx.x; item < TP; item += gridDim.x) {
    // the unit owning this page: the largest u with Poff[u] <= item
    int64_t lo = 0, hi = U - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (rec[mid * kRec + R_POFF] <= item) lo = mid;
      else hi = mid - 1;
    }
    const int64_t u = lo;
    const int64_t* R = rec + u * kRec;
    const int h = (int)(u % H);
    const int64_t j = item - R[R_POFF];
    const bool is_hi = j < R[R_HP];
    const int64_t jt = is_hi ? j : j - R[R_HP];
    const int32_t id = is_hi ? table[u * L + jt] : table[u * L + L - 1 - jt];
    const int T = is_hi ? kHiTokens : kLoTokens;
    const int64_t n_tier = is_hi ? R[R_NH] : R[R_NL];
    const int64_t slot0 = jt * T;
    const int valid = (int)(n_tier - slot0 < T ? n_tier - slot0 : T);
    const int64_t N = R[R_N], b0 = R[R_BASE];
    for (int w = tid; w < page_bytes / 4; w += blockDim.x) img[w] = 0u;
    __syncthreads();
    const Seg sg = tier_seg(D, is_hi);
    const int TPT = 256 / T;          // threads per token
    const int DPT = D / TPT;          // dims per thread
    const int t = tid / TPT, sub = tid % TPT;
    if (t < valid) {
      const int64_t slot = slot0 + t;
      const int32_t* pl = pos_list + (int64_t)h * total + b0;
      const int64_t pos = is_hi ? pl[slot] : pl[N - 1 - slot];
      const int64_t rowi = ((b0 + pos) * H + h) * D + (int64_t)sub * DPT;
      float xk[16], xv[16];
      float kmn = INFINITY, kmx = -INFINITY, vmn = INFINITY, vmx = -INFINITY;
      for (int i = 0; i < DPT; i++) {
        xk[i] = h2f(k[rowi + i]);
        xv[i] = h2f(v[rowi + i]);
        kmn = fminf(kmn, xk[i]);
        kmx = fmaxf(kmx, xk[i]);
        vmn = fminf(vmn, xv[i]);
        vmx = fmaxf(vmx, xv[i]);
      }
      auto fmn = [](float a, float b) { return fminf(a, b); };
      auto fmx = [](float a, float b) { return fmaxf(a, b); };
      kmn = group_reduce(kmn, TPT, fmn);
      kmx = group_reduce(kmx, TPT, fmx);
      vmn = group_reduce(vmn, TPT, fmn);
      vmx = group_reduce(vmx, TPT, fmx);
      uint16_t ks16, kz16, vs16, vz16;
      float ks, kz, vs, vz;
      codec_params(kmn, kmx, sg.kbits, ks16, kz16, ks, kz);
      codec_params(vmn, vmx, sg.vbits, vs16, vz16, vs, vz);
      for (int i = 0; i < DPT; i++) {
        const int jd = sub * DPT + i;
        int byte, shift;
        k_field(D, is_hi, t, jd, byte, shift);
        const uint32_t kc = codec_code(xk[i], ks, kz, sg.kbits);
        atomicOr(&img[byte >> 2], kc << (8 * (byte & 3) + shift));
        v_field(D, is_hi, t, jd, byte, shift);
        const uint32_t vc = codec_code(xv[i], vs, vz, sg.vbits);
        atomicOr(&img[byte >> 2], vc << (8 * (byte & 3) + shift));
      }
      if (sub == 0) {
        img[(sg.km >> 2) + t] = (uint32_t)ks16 | ((uint32_t)kz16 << 16);
        img[(sg.vm >> 2) + t] = (uint32_t)vs16 | ((uint32_t)vz16 << 16);
        const float mean = scores[(int64_t)h * total + b0 + pos];
        img[(sg.sc >> 2) + t] = __float_as_uint(__fmul_rn(mean, (float)(N - 1 - pos)));
        img[(sg.ps >> 2) + t] = (uint32_t)pos;
      }
    }
    __syncthreads();
    if (id >= 0 && id < P) {
      uint4* dst = (uint4*)(pages + (int64_t)id * page_bytes);
      const uint4* src = (const uint4*)img;
      for (int c = tid; c < page_bytes / 16; c += blockDim.x) dst[c] = src[c];
    } else if (tid == 0) {
      atomicOr(status, kStBadState);
    }
    __syncthreads();
  }
}

hipError_t launch_prompt(const Cfg& c, const Pool& p, int batch, int64_t total, const int64_t* cu,
                         const uint16_t* k, const uint16_t* v, const float* scores,
                         const uint8_t* tiers, int32_t* table, int32_t* state, void* ws,
                         hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  PromptWs w = carve(c, batch, total, ws, nullptr);
  const int C = num_chunks(c);
  prompt_count_kernel<<<dim3(C, (unsigned)U), dim3(256), 0, s>>>(c.H, total, C, cu, tiers, w.chunks);
  prompt_plan_kernel<<<dim3(1), dim3(1024), 0, s>>>(c.H, c.L, c.S_max, batch, C, total, cu, state,
                                                    w.chunks, w.rec, w.hdr, p.ptr, p.status);
  prompt_scatter_kernel<<<dim3(C, (unsigned)U), dim3(256), 0, s>>>(c.H, c.L, C, total, p.P, tiers, w.hdr,
                                                                   w.rec, w.chunks, p.list, w.pos,
                                                                   w.freed, table, state);
  prompt_list_kernel<<<dim3((unsigned)U), dim3(256), 0, s>>>(c.L, p.P, w.hdr, w.rec, w.freed, p.list,
                                                             table);
  int64_t grid = U * c.L;
  if (grid > 4096) grid = 4096;
  if (c.d == 128)
    prompt_pack_kernel<128><<<dim3((unsigned)grid), dim3(256), 0, s>>>(
        c.H, c.L, total, U, p.P, p.page_bytes, w.hdr, w.rec, w.pos, table, k, v, scores, p.pages, p.status);
  else
    prompt_pack_kernel<64><<<dim3((unsigned)grid), dim3(256), 0, s>>>(
        c.H, c.L, total, U, p.P, p.page_bytes, w.hdr, w.rec, w.pos, table, k, v, scores, p.pages, p.status);
  return hipGetLastError();
}

}  // namespace dkv
