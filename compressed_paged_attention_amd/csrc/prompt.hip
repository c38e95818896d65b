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
  int32_t* pmap;  // [U*L] owning unit of each page of the call, in page order
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
  w.pmap = (int32_t*)(b + off);
  off = align_up(off + (size_t)U * c.L * sizeof(int32_t), 256);
  if (bytes) *bytes = off;
  return w;
}

constexpr int kLRecP = 24;  // int64 fields per unit record (levels)
enum { LP_K = 0, LP_KOFF, LP_FOFF, LP_EOFF, LP_POFF, LP_N, LP_BASE, LP_FLAGS, LP_A, LP_AIN, LP_RIN, LP_E,
       LP_NL0, LP_NP0 = LP_NL0 + 4, LP_OFF0 = LP_NP0 + 4 };  // + per-level counts, pages, token offsets

struct PromptLvWs {
  int64_t* hdr;
  int64_t* rec;
  int32_t* chunks;  // [U][C][4] counts, then chunk offsets
  int32_t* pos;     // [H][total]
  int32_t* freed;   // [U * L]
  int32_t* pmap;    // [U * LT]
};

static PromptLvWs carve_levels(const Cfg& c, int batch, int64_t total, void* ws, size_t* bytes) {
  const int64_t U = (int64_t)batch * c.H;
  const int C = num_chunks(c);
  size_t off = 0;
  PromptLvWs w;
  uint8_t* b = (uint8_t*)ws;
  w.hdr = (int64_t*)(b + off);
  off = align_up(off + 16 * sizeof(int64_t), 256);
  w.rec = (int64_t*)(b + off);
  off = align_up(off + (size_t)U * kLRecP * sizeof(int64_t), 256);
  w.chunks = (int32_t*)(b + off);
  off = align_up(off + (size_t)U * C * 4 * sizeof(int32_t), 256);
  w.pos = (int32_t*)(b + off);
  off = align_up(off + (size_t)c.H * total * sizeof(int32_t), 256);
  w.freed = (int32_t*)(b + off);
  off = align_up(off + (size_t)U * c.L * sizeof(int32_t), 256);
  w.pmap = (int32_t*)(b + off);
  off = align_up(off + (size_t)U * c.LT * sizeof(int32_t), 256);
  if (bytes) *bytes = off;
  return w;
}

size_t prompt_workspace(const Cfg& c, int batch, int64_t total) {
  size_t n = 0;
  if (c.K >= 3) carve_levels(c, batch, total, nullptr, &n);
  else carve(c, batch, total, nullptr, &n);
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
// them; the page map (owner of each page the pack kernel writes).  A list slot read here (logical index below the old end) is never
// one of the slots written here: the written logical indices sit exactly P
// above indices this call already consumed.
__global__ __launch_bounds__(256) void prompt_list_kernel(int L, int64_t P, const int64_t* __restrict__ hdr,
                                                          const int64_t* __restrict__ rec,
                                                          const int32_t* __restrict__ freed,
                                                          int32_t* list, int32_t* __restrict__ table,
                                                          int32_t* __restrict__ pmap) {
  if (!hdr[H_COMMIT]) return;
  const int64_t u = blockIdx.x;
  const int64_t* R = rec + u * kRec;
  if (R[R_N] <= 0) return;
  const int64_t k = R[R_K], hp = R[R_HP], lp = R[R_LP];
  for (int64_t i = threadIdx.x; i < hp + lp; i += blockDim.x) pmap[R[R_POFF] + i] = (int32_t)u;
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // K/V rows: 16-byte non-temporal loads

// Codes of the per-vector codec without a division: t = fl(x - z) * (1/s)
// with the hardware reciprocal (1 ulp; 2 ulp still suffice) is within 8e-5
// of the quotient q wherever |q| <= 257, so rounding t gives the code unless
// t lies within 2^-13 of a half-integer; then the codes are redone with the
// IEEE division.  Quotients beyond the code range clamp the same either
// way; a zero scale comes in as rs = 0 and gives code 0.  (K and V are
// finite fp16 values.)
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

__device__ inline float lo_h(uint32_t w) { return h2f((uint16_t)(w & 0xFFFFu)); }
__device__ inline float hi_h(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

// fp16 pairs: elementwise min / max (exact; the 3-input packed forms)
__device__ inline uint32_t pmin(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_minimum(__builtin_bit_cast(h2v, a), __builtin_bit_cast(h2v, b)));
}
__device__ inline uint32_t pmax(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_maximum(__builtin_bit_cast(h2v, a), __builtin_bit_cast(h2v, b)));
}

// fl(x - z) for the fp16 half SEL of w: one mixed-precision fma (x * 1 - z,
// a single rounding, the same value as converting x and subtracting)
template <int SEL>
__device__ inline float sub_h(uint32_t w, float z) {
  float r;
  if constexpr (SEL == 0)
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(z));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(z));
  return r;
}

// The 8 codes of a lane's dims 8a..8a+7 of one token (element e in half
// e&1 of word e>>1), as integers.
template <int BITS>
__device__ inline void codes8(const uint32_t* w, float s, float z, uint32_t* c) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  const float rs = s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s);
  float dmax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const float d = (e & 1) ? sub_h<1>(w[e >> 1], z) : sub_h<0>(w[e >> 1], z);
    const float t = __fmul_rn(d, rs);
    const float rt = __builtin_rintf(t);
    dmax = fmaxf(dmax, __builtin_fabsf(t - rt));
    c[e] = (uint32_t)__builtin_amdgcn_fmed3f(rt, 0.0f, qmax);
  }
  if (!(dmax < 0.5f - 0x1p-13f)) {
#pragma unroll
    for (int e = 0; e < 8; e++) c[e] = codec_code((e & 1) ? hi_h(w[e >> 1]) : lo_h(w[e >> 1]), s, z, BITS);
  }
}

// The codec's scale and zero (fp16 of range / (2^b - 1), fp16 of the
// minimum) with the division by the constant 2^b - 1 done as a product with
// its correctly rounded reciprocal and one fma correction: for every fp32
// range in [0, 2^17] (ranges of fp16 vectors are at most 131008) the result
// equals the IEEE quotient bit for bit (checked exhaustively on the CPU for
// 1, 3, 15 and 255: none of 4 x 1.2e9 differ).
template <int BITS>
__device__ inline void codec_params_c(float mn, float mx, uint16_t& s16, uint16_t& z16, float& s, float& z) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  constexpr float rq = 1.0f / qmax;
  const float range = __fsub_rn(mx, mn);
  const float q0 = __fmul_rn(range, rq);
  const float scale = __builtin_fmaf(__builtin_fmaf(-q0, qmax, range), rq, q0);
  s16 = f2h_bits(scale);
  z16 = f2h_bits(mn);
  s = h2f(s16);
  z = h2f(z16);
}

// Where a page comes from (wave-uniform).
struct PackMeta {
  int32_t id;
  int hi, valid, h;
  int64_t slot0, N, b0;
};

__device__ inline PackMeta pack_meta(int64_t item, int H, int L, const int64_t* __restrict__ rec,
                                     const int32_t* __restrict__ pmap, const int32_t* __restrict__ table) {
  PackMeta m;
  const int u = __builtin_amdgcn_readfirstlane(pmap[item]);
  const int64_t* R = rec + (int64_t)u * kRec;
  m.h = u % H;
  const int64_t j = item - R[R_POFF], hp = R[R_HP];
  m.hi = j < hp;
  const int64_t jt = m.hi ? j : j - hp;
  m.id = table[(int64_t)u * L + (m.hi ? jt : L - 1 - jt)];
  const int T = m.hi ? kHiTokens : kLoTokens;
  const int64_t n_tier = m.hi ? R[R_NH] : R[R_NL];
  m.slot0 = jt * T;
  m.valid = (int)(n_tier - m.slot0 < T ? n_tier - m.slot0 : T);
  m.N = R[R_N];
  m.b0 = R[R_BASE];
  return m;
}

// Positions of the lane's tokens 16 th + 4 g + r (high pages: th = 0 only);
// slots past the tier's count read the page's first slot.
__device__ inline void pack_pos(const PackMeta& m, int g, bool act, const int32_t* __restrict__ pos_list,
                                int64_t total, int32_t (&pos)[2][4]) {
  const int32_t* pl = pos_list + (int64_t)m.h * total + m.b0;
#pragma unroll
  for (int th = 0; th < 2; th++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int t = 16 * th + 4 * g + r;
      const int64_t slot = m.slot0 + ((act && t < m.valid) ? t : 0);
      pos[th][r] = m.hi ? pl[slot] : pl[m.N - 1 - slot];
    }
}

// Per token: the (K, V) minima and maxima over the group's NA lanes as fp16
// pairs (K in the low half, V in the high half) from the lane's 8 K and 8 V
// values (per-lane pair minima / maxima, then a reduction over the group).
template <int NA>
__device__ inline void tok_minmax(const uint32_t (&kw)[4], const uint32_t (&vw)[4], uint32_t& mn, uint32_t& mx) {
  const uint32_t kn = pmin(pmin(kw[0], kw[1]), pmin(kw[2], kw[3]));
  const uint32_t kx = pmax(pmax(kw[0], kw[1]), pmax(kw[2], kw[3]));
  const uint32_t vn = pmin(pmin(vw[0], vw[1]), pmin(vw[2], vw[3]));
  const uint32_t vx = pmax(pmax(vw[0], vw[1]), pmax(vw[2], vw[3]));
  mn = pmin(__builtin_amdgcn_perm(vn, kn, 0x05040100u), __builtin_amdgcn_perm(vn, kn, 0x07060302u));
  mx = pmax(__builtin_amdgcn_perm(vx, kx, 0x05040100u), __builtin_amdgcn_perm(vx, kx, 0x07060302u));
  mn = pmin(mn, lane_xchg<0>(mn));
  mx = pmax(mx, lane_xchg<0>(mx));
  mn = pmin(mn, lane_xchg<1>(mn));
  mx = pmax(mx, lane_xchg<1>(mx));
  mn = pmin(mn, lane_xchg<2>(mn));
  mx = pmax(mx, lane_xchg<2>(mx));
  if constexpr (NA > 8) {
    mn = pmin(mn, lane_xchg<3>(mn));
    mx = pmax(mx, lane_xchg<3>(mx));
  }
}

// Page packing ("Memory management": a unified page holds its tokens'
// quantized K and V with their metadata, score and position).  One wave per
// page, no LDS: lane (g, a), a = lane mod d/8, holds dims 8a..8a+7 of the
// tokens 4g..4g+3 (and, in a low page, 16+4g..16+4g+3), one 16-byte row
// load each for K and V.  Per token the min/max come from a reduction over
// the d/8 lanes of the group (fp16 pairs: K and V minima in one word, maxima
// in another); K codes leave as whole words, V codes are assembled into the
// lane-chunk layout: a V word holds the 4 (low: 8) tokens of a group at one
// in-chunk dim and two 16-dim blocks, the second block from lane a^2.  Lanes
// a = 0..3 store the metadata, score and position words.  Slots past the
// tier's count are written as zeros, as is the page's tail after the last
// segment.
template <int D, bool HI>
__device__ inline void pack_compute(uint8_t* pg, int lane, int valid, int64_t N, const int32_t (&pos)[2][4],
                                    u32x4 (&kr)[2][4], u32x4 (&vr)[2][4], const float (&mean)[2][4]) {
  constexpr int NA = D / 8;             // lanes per token group
  constexpr int NT = HI ? 1 : 2;        // token quads per lane
  constexpr Seg sg = tier_seg(D, HI);
  const int a = lane % NA, g = lane / NA;
  const bool act = g < 4;
#pragma unroll
  for (int th = 0; th < NT; th++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int t = 16 * th + 4 * g + r;
      const bool ok = act && t < valid;
      if (!ok) {
        kr[th][r] = u32x4{0u, 0u, 0u, 0u};
        vr[th][r] = u32x4{0u, 0u, 0u, 0u};
      }
      // score (mean * (N - 1 - pos), a running sum over the tokens after
      // pos) and position words, by lanes a == 2 and a == 3
      if (act && (a == 2 || a == 3)) {
        uint32_t wd = 0u;
        if (ok)
          wd = a == 3 ? (uint32_t)pos[th][r] : __float_as_uint(__fmul_rn(mean[th][r], (float)(N - 1 - pos[th][r])));
        *(uint32_t*)(pg + (a == 2 ? sg.sc : sg.ps) + 4 * t) = wd;
      }
    }
  const int nbp = (a >> 1) & 1;  // parity of the lane's 16-dim block
  uint32_t vw[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};  // V word per in-chunk dim 8(a&1)+e
  uint8_t* kc = pg + sg.kc;
#pragma unroll
  for (int th = 0; th < NT; th++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int t = 16 * th + 4 * g + r;
      const uint32_t kw[4] = {kr[th][r][0], kr[th][r][1], kr[th][r][2], kr[th][r][3]};
      const uint32_t vwr[4] = {vr[th][r][0], vr[th][r][1], vr[th][r][2], vr[th][r][3]};
      uint32_t mn, mx;
      tok_minmax<NA>(kw, vwr, mn, mx);
      uint16_t ks16, kz16, vs16, vz16;
      float ks, kz, vs, vz;
      codec_params_c<sg.kbits>(lo_h(mn), lo_h(mx), ks16, kz16, ks, kz);
      codec_params_c<sg.vbits>(hi_h(mn), hi_h(mx), vs16, vz16, vs, vz);
      uint32_t c[8];
      codes8<sg.kbits>(kw, ks, kz, c);
      if (act) {
        if (HI) {
          // 8-bit K, token-major: bytes t*D + 8a .. +7
          const uint32_t w0 = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
          const uint32_t w1 = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
          *(uint2*)(kc + t * D + 8 * a) = make_uint2(w0, w1);
        } else {
          // 4-bit K: dim 8a+e in nibble e/2 + 4(e&1) of word a
          uint32_t w = 0;
#pragma unroll
          for (int e = 0; e < 8; e++) w |= c[e] << (4 * ((e >> 1) + 4 * (e & 1)));
          *(uint32_t*)(kc + t * (D / 2) + 4 * a) = w;
        }
        if (a < 2)
          *(uint32_t*)(pg + (a == 0 ? sg.km : sg.vm) + 4 * t) =
              a == 0 ? ((uint32_t)ks16 | ((uint32_t)kz16 << 16)) : ((uint32_t)vs16 | ((uint32_t)vz16 << 16));
      }
      codes8<sg.vbits>(vwr, vs, vz, c);
      // V field of (token t, dim 8a+e): bit 8 nbp + 4(r>>1) + 16(r&1)
      // (high), 8 nbp + 4 th + 2(r>>1) + 16(r&1) (low)
      const int sh = HI ? 8 * nbp + 4 * (r >> 1) + 16 * (r & 1) : 8 * nbp + 4 * th + 2 * (r >> 1) + 16 * (r & 1);
#pragma unroll
      for (int e = 0; e < 8; e++) vw[e] |= c[e] << sh;
    }
  // the other 16-dim block of each word comes from lane a^2
#pragma unroll
  for (int e = 0; e < 8; e++) vw[e] |= lane_xchg<1>(vw[e]);
  if (act) {
    // lane keeps in-chunk dims 8(a&1) + 4 nbp .. +3: chunk L = i + 16 g, word a>>2
    // (a bitwise select: an index that depends on the lane would move the
    // array out of registers)
    uint8_t* vc = pg + sg.vc;
    const uint32_t msk = 0u - (uint32_t)nbp;
#pragma unroll
    for (int e4 = 0; e4 < 4; e4++) {
      const int L = 8 * (a & 1) + 4 * nbp + e4 + 16 * g;
      *(uint32_t*)(vc + L * (D / 8) + 4 * (a >> 2)) = vw[e4] ^ ((vw[e4] ^ vw[4 + e4]) & msk);
    }
  }
  // bytes after the last segment (high pages are shorter than the page)
  for (int off = sg.bytes + 16 * lane; off < page_bytes_for(D); off += 16 * 64)
    *(uint4*)(pg + off) = make_uint4(0u, 0u, 0u, 0u);
}

// codes8 and codec_params_c for a width known at run time (wave-uniform):
// the same operations with 2^b - 1 and its correctly rounded reciprocal
// (an IEEE division, as the constant one is) in registers, so the results are
// those of the constant-width helpers.
__device__ inline void codes8_var(int bits, const uint32_t* w, float s, float z, uint32_t* c) {
  const float qmax = (float)((1 << bits) - 1);
  const float rs = s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s);
  float dmax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const float d = (e & 1) ? sub_h<1>(w[e >> 1], z) : sub_h<0>(w[e >> 1], z);
    const float t = __fmul_rn(d, rs);
    const float rt = __builtin_rintf(t);
    dmax = fmaxf(dmax, __builtin_fabsf(t - rt));
    c[e] = (uint32_t)__builtin_amdgcn_fmed3f(rt, 0.0f, qmax);
  }
  if (!(dmax < 0.5f - 0x1p-13f)) {
#pragma unroll
    for (int e = 0; e < 8; e++) c[e] = codec_code((e & 1) ? hi_h(w[e >> 1]) : lo_h(w[e >> 1]), s, z, bits);
  }
}

__device__ inline void codec_params_var(int bits, float mn, float mx, uint16_t& s16, uint16_t& z16, float& s,
                                        float& z) {
  const float qmax = (float)((1 << bits) - 1);
  const float rq = __fdiv_rn(1.0f, qmax);
  const float range = __fsub_rn(mx, mn);
  const float q0 = __fmul_rn(range, rq);
  const float scale = __builtin_fmaf(__builtin_fmaf(-q0, qmax, range), rq, q0);
  s16 = f2h_bits(scale);
  z16 = f2h_bits(mn);
  s = h2f(s16);
  z = h2f(z16);
}

// The 8 codes of dims 8a..8a+7 of token t in the plain layout: 8b bits at
// bit (t d + 8a) b of the segment, i.e. b whole bytes at byte (t d/8 + a) b,
// code e at bit e b (little-endian).
template <int D>
__device__ inline void put_codes8(uint8_t* seg, int bits, int t, int a, const uint32_t* c) {
  uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const int bit = e * bits;  // < 64
    if (bit < 32) w0 |= c[e] << bit;
    else w1 |= c[e] << (bit - 32);
  }
  uint8_t* dst = seg + (t * (D / 8) + a) * bits;
  if (bits == 8) *(uint2*)dst = make_uint2(w0, w1);
  else if (bits == 4) *(uint32_t*)dst = w0;
  else if (bits == 2) *(uint16_t*)dst = (uint16_t)w0;
  else *dst = (uint8_t)w0;
}

// Page packing for a tier codec variant (plain layout, widths in sg): the
// lane and token mapping, minima / maxima and the score and position words
// of pack_compute; the codes of a lane's 8 dims leave as whole bytes.
template <int D, bool HI>
__device__ inline void pack_compute_plain(uint8_t* pg, int lane, int valid, int64_t N, const int32_t (&pos)[2][4],
                                          u32x4 (&kr)[2][4], u32x4 (&vr)[2][4], const float (&mean)[2][4],
                                          const Seg& sg, int page_bytes) {
  constexpr int NA = D / 8;
  constexpr int NT = HI ? 1 : 2;
  const int a = lane % NA, g = lane / NA;
  const bool act = g < 4;
#pragma unroll
  for (int th = 0; th < NT; th++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int t = 16 * th + 4 * g + r;
      const bool ok = act && t < valid;
      if (!ok) {
        kr[th][r] = u32x4{0u, 0u, 0u, 0u};
        vr[th][r] = u32x4{0u, 0u, 0u, 0u};
      }
      if (act && (a == 2 || a == 3)) {
        uint32_t wd = 0u;
        if (ok)
          wd = a == 3 ? (uint32_t)pos[th][r] : __float_as_uint(__fmul_rn(mean[th][r], (float)(N - 1 - pos[th][r])));
        *(uint32_t*)(pg + (a == 2 ? sg.sc : sg.ps) + 4 * t) = wd;
      }
    }
#pragma unroll
  for (int th = 0; th < NT; th++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int t = 16 * th + 4 * g + r;
      const uint32_t kw[4] = {kr[th][r][0], kr[th][r][1], kr[th][r][2], kr[th][r][3]};
      const uint32_t vwr[4] = {vr[th][r][0], vr[th][r][1], vr[th][r][2], vr[th][r][3]};
      uint32_t mn, mx;
      tok_minmax<NA>(kw, vwr, mn, mx);
      uint16_t ks16, kz16, vs16, vz16;
      float ks, kz, vs, vz;
      codec_params_var(sg.kbits, lo_h(mn), lo_h(mx), ks16, kz16, ks, kz);
      codec_params_var(sg.vbits, hi_h(mn), hi_h(mx), vs16, vz16, vs, vz);
      uint32_t c[8];
      codes8_var(sg.kbits, kw, ks, kz, c);
      if (act) put_codes8<D>(pg + sg.kc, sg.kbits, t, a, c);
      codes8_var(sg.vbits, vwr, vs, vz, c);
      if (act) {
        put_codes8<D>(pg + sg.vc, sg.vbits, t, a, c);
        if (a < 2)
          *(uint32_t*)(pg + (a == 0 ? sg.km : sg.vm) + 4 * t) =
              a == 0 ? ((uint32_t)ks16 | ((uint32_t)kz16 << 16)) : ((uint32_t)vs16 | ((uint32_t)vz16 << 16));
      }
    }
  for (int off = sg.bytes + 16 * lane; off < page_bytes; off += 16 * 64)
    *(uint4*)(pg + off) = make_uint4(0u, 0u, 0u, 0u);
}

// Persistent: each wave packs a contiguous range of the call's TP pages
// (items in unit order, each unit's high pages then its low pages; the
// owner of an item comes from the page map the list kernel wrote).  While a
// page's rows are in flight the wave looks up the next page and loads its
// positions, so a page waits for one round trip.
template <int D, bool PLAIN>
__global__ __launch_bounds__(256) void prompt_pack_kernel(int H, int L, int64_t total, int64_t P, int page_bytes,
                                                          Seg sgh, Seg sgl,
                                                          const int64_t* __restrict__ hdr,
                                                          const int64_t* __restrict__ rec,
                                                          const int32_t* __restrict__ pmap,
                                                          const int32_t* __restrict__ pos_list,
                                                          const int32_t* __restrict__ table,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const float* __restrict__ scores,
                                                          uint8_t* __restrict__ pages, uint32_t* status) {
  if (!hdr[H_COMMIT]) return;
  const int64_t TP = hdr[H_PAGES];
  constexpr int NA = D / 8;
  const int lane = threadIdx.x & 63;
  const int a = lane % NA, g = lane / NA;
  const bool act = g < 4;
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t per = (TP + nw - 1) / nw;
  const int64_t i0 = w * per, i1 = TP < i0 + per ? TP : i0 + per;
  if (i0 >= i1) return;
  PackMeta m = pack_meta(i0, H, L, rec, pmap, table);
  int32_t pos[2][4];
  pack_pos(m, g, act, pos_list, total, pos);
  for (int64_t item = i0; item < i1; item++) {
    // this page's rows and mean scores
    u32x4 kr[2][4], vr[2][4];
    float mean[2][4];
    const float* sc = scores + (int64_t)m.h * total + m.b0;
#pragma unroll
    for (int th = 0; th < 2; th++) {
      if (th == 1 && m.hi) break;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int64_t row = ((m.b0 + pos[th][r]) * H + m.h) * D + 8 * a;
        kr[th][r] = __builtin_nontemporal_load((const u32x4*)(k + row));
        vr[th][r] = __builtin_nontemporal_load((const u32x4*)(v + row));
        mean[th][r] = sc[pos[th][r]];
      }
    }
    // the next page's metadata and positions meanwhile
    PackMeta mn = m;
    int32_t posn[2][4];
    if (item + 1 < i1) {
      mn = pack_meta(item + 1, H, L, rec, pmap, table);
      pack_pos(mn, g, act, pos_list, total, posn);
    }
    if (m.id < 0 || m.id >= P) {
      if (lane == 0) atomicOr(status, kStBadState);
    } else {
      uint8_t* pg = pages + (int64_t)m.id * page_bytes;
      if constexpr (PLAIN) {
        if (m.hi) pack_compute_plain<D, true>(pg, lane, m.valid, m.N, pos, kr, vr, mean, sgh, page_bytes);
        else pack_compute_plain<D, false>(pg, lane, m.valid, m.N, pos, kr, vr, mean, sgl, page_bytes);
      } else {
        if (m.hi) pack_compute<D, true>(pg, lane, m.valid, m.N, pos, kr, vr, mean);
        else pack_compute<D, false>(pg, lane, m.valid, m.N, pos, kr, vr, mean);
      }
    }
    m = mn;
#pragma unroll
    for (int th = 0; th < 2; th++)
#pragma unroll
      for (int r = 0; r < 4; r++) pos[th][r] = posn[th][r];
  }
}


// ===========================================================================
// K precision levels (DiffKV notes, "KV compression policy", extensibility;
// "Memory management", generation workflow: extra levels by combining
// unidirectional or bidirectional page tables).  The same five phases over
// K = 3 or 4 levels:
//   count   per-chunk counts of every level;
//   plan    per unit: pages per level, the conservative block of ceil(N/16)
//           pages, its use (levels 0, 2, 3 from the left end in that order,
//           level 1 from the right end, the middle freed) and the pages it
//           lacks (extras); scans over units; capacity; pointers;
//   scatter slot -> position lists (levels contiguous in the unit's token
//           range, each in position order) and the block's table entries;
//   list    frees at the old reclamation pointer, extras after them, the
//           page map;
//   pack    one wave per page (persistent), as the plain packer.
// A unit's pages in "Q order": level 0, 2, 3 pages (index order), then
// level 1's innermost first; block page i serves Q position i (i < A'),
// the right end serves level 1, positions between take extras.
// ===========================================================================
__global__ __launch_bounds__(256) void prompt_count_levels_kernel(int H, int K, int64_t total, int C,
                                                                  const int64_t* __restrict__ cu,
                                                                  const uint8_t* __restrict__ tiers,
                                                                  int32_t* __restrict__ chunks) {
  const int c = blockIdx.x;
  const int64_t u = blockIdx.y;
  const int r = (int)(u / H), h = (int)(u % H);
  const int64_t b0 = cu[r], N = cu[r + 1] - b0;
  const int64_t t0 = (int64_t)c * kChunk;
  const int64_t t1 = N < t0 + kChunk ? N : t0 + kChunk;
  int n[4] = {0, 0, 0, 0};
  if (b0 >= 0 && N > 0 && cu[r + 1] <= total) {
    const uint8_t* t = tiers + (int64_t)h * total + b0;
    for (int64_t p = t0 + threadIdx.x; p < t1; p += blockDim.x) {
      const int code = t[p];
#pragma unroll
      for (int l = 0; l < 4; l++) n[l] += l < K && code == K - l;  // (code 0: pruned)
    }
  }
  __shared__ int red[4][4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int l = 0; l < 4; l++) {
    n[l] = wave_sum(n[l]);
    if (lane == 0) red[l][wid] = n[l];
  }
  __syncthreads();
  if (threadIdx.x < 4) chunks[(u * C + c) * 4 + threadIdx.x] = red[threadIdx.x][0] + red[threadIdx.x][1] +
                                                                 red[threadIdx.x][2] + red[threadIdx.x][3];
}

__global__ __launch_bounds__(1024) void prompt_plan_levels_kernel(int H, int K, int L, int S_max, int batch, int C,
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
    int64_t k = 0, f = 0, e = 0, nq = 0, N = 0, b0 = 0, A = 0, Ain = 0, Rin = 0;
    int64_t n[4] = {0, 0, 0, 0}, np[4] = {0, 0, 0, 0};
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
        for (int w = 0; w < 2 * K; w++)
          if (state[u * 2 * K + w]) flags |= kStBadState;
        if (N > S_max) {
          flags |= kStOverflow;
        } else {
          for (int c = 0; c < C; c++) {
            int32_t* ch = chunks + (u * C + c) * 4;
#pragma unroll
            for (int l = 0; l < 4; l++) {
              const int32_t a = ch[l];
              ch[l] = (int32_t)n[l];
              n[l] += a;
            }
          }
          int64_t sum = 0;
#pragma unroll
          for (int l = 0; l < 4; l++) {
            np[l] = cdiv(n[l], l == 0 ? kHiTokens : kLoTokens);
            sum += n[l];
          }
          k = cdiv(N, kHiTokens);
          if (sum > N) flags |= kStBadState;
          if (k > L || np[0] + np[1] > L || np[2] + np[3] > L) flags |= kStOverflow;
          A = np[0] + np[2] + np[3];
          Ain = A < k ? A : k;
          Rin = np[1] < k - Ain ? np[1] : k - Ain;
          f = k - Ain - Rin;
          e = (A - Ain) + (np[1] - Rin);
          nq = A + np[1];
        }
      }
    }
    if (flags) atomicOr(&sflags, flags);
    int64_t tot[4];
    const int64_t ok = block_excl_scan(k, lds, tot[0]);
    const int64_t of = block_excl_scan(f, lds, tot[1]);
    const int64_t oe = block_excl_scan(e, lds, tot[2]);
    const int64_t op = block_excl_scan(nq, lds, tot[3]);
    if (u < U) {
      int64_t* R = rec + u * kLRecP;
      R[LP_K] = k;
      R[LP_KOFF] = carry[0] + ok;
      R[LP_FOFF] = carry[1] + of;
      R[LP_EOFF] = carry[2] + oe;
      R[LP_POFF] = carry[3] + op;
      R[LP_N] = N;
      R[LP_BASE] = b0;
      R[LP_FLAGS] = flags;
      R[LP_A] = A;
      R[LP_AIN] = Ain;
      R[LP_RIN] = Rin;
      R[LP_E] = e;
      int64_t o = 0;
      for (int l = 0; l < 4; l++) {
        R[LP_NL0 + l] = n[l];
        R[LP_NP0 + l] = np[l];
        R[LP_OFF0 + l] = o;
        o += n[l];
      }
    }
    for (int i = 0; i < 4; i++) carry[i] += tot[i];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t start = ptr[0], end = ptr[1];
    const int64_t free0 = (int64_t)(end - start);
    uint32_t st = sflags;
    const int64_t Kt = carry[0], F = carry[1], E = carry[2];
    if (!st && (Kt > free0 || Kt - F + E > free0)) st |= kStExhausted;
    hdr[H_K] = Kt;
    hdr[H_F] = F;
    hdr[H_E] = E;
    hdr[H_START] = (int64_t)start;
    hdr[H_END] = (int64_t)end;
    hdr[H_PAGES] = carry[3];
    hdr[H_COMMIT] = st == 0;
    if (st) {
      atomicOr(status, st);
    } else {
      ptr[0] = start + (uint64_t)(Kt + E);
      ptr[1] = end + (uint64_t)F;
    }
  }
}

// (level, page index) of Q position i of a unit (record R)
__device__ inline void lv_q_page(const int64_t* R, int64_t i, int& l, int64_t& j) {
  const int64_t p0 = R[LP_NP0], p1 = R[LP_NP0 + 1], p2 = R[LP_NP0 + 2], p3 = R[LP_NP0 + 3];
  if (i < p0) { l = 0; j = i; return; }
  i -= p0;
  if (i < p2) { l = 2; j = i; return; }
  i -= p2;
  if (i < p3) { l = 3; j = i; return; }
  i -= p3;
  l = 1;
  j = p1 - 1 - i;  // level 1 innermost first
}

__global__ __launch_bounds__(256) void prompt_scatter_levels_kernel(int H, int K, int L, int LT, int C,
                                                                    int64_t total, int64_t P,
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
  const int64_t* R = rec + u * kLRecP;
  const int64_t N = R[LP_N], b0 = R[LP_BASE];
  if (N <= 0) return;
  const int64_t t0 = (int64_t)c * kChunk;
  if (t0 < N) {
    const uint8_t* t = tiers + (int64_t)h * total + b0;
    constexpr int kPer = kChunk / 256;
    const int64_t p0 = t0 + (int64_t)threadIdx.x * kPer;
    uint8_t v[kPer];
    int cnt[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int64_t p = p0 + i;
      v[i] = p < N ? t[p] : (uint8_t)0;
#pragma unroll
      for (int l = 0; l < 4; l++) cnt[l] += l < K && v[i] == K - l;  // (code 0: pruned)
    }
    __shared__ int lds[20];
    int base[4];
#pragma unroll
    for (int l = 0; l < 4; l++) {
      int tl;
      base[l] = block_excl_scan(cnt[l], lds, tl) + chunks[(u * C + c) * 4 + l] + (int)R[LP_OFF0 + l];
    }
    int32_t* pl = pos_list + (int64_t)h * total + b0;
#pragma unroll
    for (int i = 0; i < kPer; i++) {
      const int code = v[i];
      if (code >= 1 && code <= K) {
        // (a bitwise select keeps base[] in registers)
        const int l = K - code;
        const int s = l == 0 ? base[0]++ : l == 1 ? base[1]++ : l == 2 ? base[2]++ : base[3]++;
        pl[s] = (int32_t)(p0 + i);
      }
    }
  }
  if (c == 0) {
    const int64_t k = R[LP_K], Ain = R[LP_AIN], Rin = R[LP_RIN], A = R[LP_A], p1 = R[LP_NP0 + 1];
    const uint64_t start = (uint64_t)hdr[H_START] + (uint64_t)R[LP_KOFF];
    int32_t* row = table + u * LT;
    for (int64_t i = threadIdx.x; i < k; i += blockDim.x) {
      const int32_t id = list[(start + (uint64_t)i) % (uint64_t)P];
      int64_t q = -1;
      if (i < Ain) q = i;                              // left end
      else if (i >= k - Rin) q = A + (i - (k - p1));   // right end: level 1
      if (q >= 0) {
        int l;
        int64_t j;
        lv_q_page(R, q, l, j);
        row[(l >> 1) * L + ((l & 1) ? L - 1 - j : j)] = id;
      } else {
        freed[R[LP_FOFF] + (i - Ain)] = id;
      }
    }
    if (threadIdx.x < 2 * K) {
      const int w = threadIdx.x;
      state[u * 2 * K + w] = (int32_t)(w < K ? R[LP_NL0 + w] : R[LP_NP0 + (w - K)]);
    }
  }
}

__global__ __launch_bounds__(256) void prompt_list_levels_kernel(int L, int LT, int64_t P,
                                                                 const int64_t* __restrict__ hdr,
                                                                 const int64_t* __restrict__ rec,
                                                                 const int32_t* __restrict__ freed, int32_t* list,
                                                                 int32_t* __restrict__ table,
                                                                 int32_t* __restrict__ pmap) {
  if (!hdr[H_COMMIT]) return;
  const int64_t u = blockIdx.x;
  const int64_t* R = rec + u * kLRecP;
  if (R[LP_N] <= 0) return;
  const int64_t k = R[LP_K], Ain = R[LP_AIN], Rin = R[LP_RIN], A = R[LP_A], e = R[LP_E];
  const int64_t nq = A + R[LP_NP0 + 1];
  for (int64_t i = threadIdx.x; i < nq; i += blockDim.x) pmap[R[LP_POFF] + i] = (int32_t)u;
  const int64_t f = k - Ain - Rin;
  const uint64_t end0 = (uint64_t)hdr[H_END];
  for (int64_t i = threadIdx.x; i < f; i += blockDim.x)
    list[(end0 + (uint64_t)(R[LP_FOFF] + i)) % (uint64_t)P] = freed[R[LP_FOFF] + i];
  // extras after the frees: the left part's first, then level 1's (the
  // frees being appended now are read from their own array)
  for (int64_t x = threadIdx.x; x < e; x += blockDim.x) {
    const uint64_t li = (uint64_t)hdr[H_START] + (uint64_t)hdr[H_K] + (uint64_t)(R[LP_EOFF] + x);
    const int32_t id = li < end0 ? list[li % (uint64_t)P] : freed[li - end0];
    const int64_t q = x < A - Ain ? Ain + x : A + (x - (A - Ain));
    int l;
    int64_t j;
    lv_q_page(R, q, l, j);
    table[u * LT + (l >> 1) * L + ((l & 1) ? L - 1 - j : j)] = id;
  }
}

// Persistent: each wave packs pages item = w, w + nw, ... (the call's TP
// pages in unit order, each unit's in Q order).
template <int D>
__global__ __launch_bounds__(256) void prompt_pack_levels_kernel(int H, int L, int LT, int64_t total, int64_t P,
                                                                 int page_bytes, Levels lv,
                                                                 const int64_t* __restrict__ hdr,
                                                                 const int64_t* __restrict__ rec,
                                                                 const int32_t* __restrict__ pmap,
                                                                 const int32_t* __restrict__ pos_list,
                                                                 const int32_t* __restrict__ table,
                                                                 const uint16_t* __restrict__ k,
                                                                 const uint16_t* __restrict__ v,
                                                                 const float* __restrict__ scores,
                                                                 uint8_t* __restrict__ pages, uint32_t* status) {
  if (!hdr[H_COMMIT]) return;
  const int64_t TP = hdr[H_PAGES];
  constexpr int NA = D / 8;
  const int lane = threadIdx.x & 63;
  const int a = lane % NA, g = lane / NA;
  const bool act = g < 4;
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int64_t item = w; item < TP; item += nw) {
    const int u = __builtin_amdgcn_readfirstlane(pmap[item]);
    const int64_t* R = rec + (int64_t)u * kLRecP;
    const int h = u % H;
    int l;
    int64_t j;
    lv_q_page(R, item - R[LP_POFF], l, j);
    const int T = l == 0 ? kHiTokens : kLoTokens;
    const int64_t n_l = R[LP_NL0 + l], slot0 = j * T;
    const int valid = (int)(n_l - slot0 < T ? n_l - slot0 : T);
    const int64_t N = R[LP_N], b0 = R[LP_BASE];
    const int32_t id = table[(int64_t)u * LT + (l >> 1) * L + ((l & 1) ? L - 1 - j : j)];
    const int32_t* pl = pos_list + (int64_t)h * total + b0 + R[LP_OFF0 + l];
    int32_t pos[2][4];
#pragma unroll
    for (int th = 0; th < 2; th++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int t = 16 * th + 4 * g + r;
        pos[th][r] = pl[slot0 + ((act && t < valid) ? t : 0)];
      }
    u32x4 kr[2][4], vr[2][4];
    float mean[2][4];
    const float* sc = scores + (int64_t)h * total + b0;
#pragma unroll
    for (int th = 0; th < 2; th++) {
      if (th == 1 && l == 0) break;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int64_t row = ((b0 + pos[th][r]) * H + h) * D + 8 * a;
        kr[th][r] = __builtin_nontemporal_load((const u32x4*)(k + row));
        vr[th][r] = __builtin_nontemporal_load((const u32x4*)(v + row));
        mean[th][r] = sc[pos[th][r]];
      }
    }
    if (id < 0 || id >= P) {
      if (lane == 0) atomicOr(status, kStBadState);
      continue;
    }
    uint8_t* pg = pages + (int64_t)id * page_bytes;
    if (l == 0) pack_compute_plain<D, true>(pg, lane, valid, N, pos, kr, vr, mean, lv.s[0], page_bytes);
    else pack_compute_plain<D, false>(pg, lane, valid, N, pos, kr, vr, mean, lv.s[l], page_bytes);
  }
}

static hipError_t launch_prompt_levels(const Cfg& c, const Pool& p, int batch, int64_t total, const int64_t* cu,
                                       const uint16_t* k, const uint16_t* v, const float* scores,
                                       const uint8_t* tiers, int32_t* table, int32_t* state, void* ws,
                                       hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  PromptLvWs w = carve_levels(c, batch, total, ws, nullptr);
  const int C = num_chunks(c);
  prompt_count_levels_kernel<<<dim3(C, (unsigned)U), dim3(256), 0, s>>>(c.H, c.K, total, C, cu, tiers, w.chunks);
  prompt_plan_levels_kernel<<<dim3(1), dim3(1024), 0, s>>>(c.H, c.K, c.L, c.S_max, batch, C, total, cu, state,
                                                           w.chunks, w.rec, w.hdr, p.ptr, p.status);
  prompt_scatter_levels_kernel<<<dim3(C, (unsigned)U), dim3(256), 0, s>>>(c.H, c.K, c.L, c.LT, C, total, p.P,
                                                                          tiers, w.hdr, w.rec, w.chunks, p.list,
                                                                          w.pos, w.freed, table, state);
  prompt_list_levels_kernel<<<dim3((unsigned)U), dim3(256), 0, s>>>(c.L, c.LT, p.P, w.hdr, w.rec, w.freed, p.list,
                                                                    table, w.pmap);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(4 * (cus > 0 ? cus : 1)));
  const Levels lv = levels_of(c);
  if (c.d == 128)
    prompt_pack_levels_kernel<128><<<grid, dim3(256), 0, s>>>(c.H, c.L, c.LT, total, p.P, p.page_bytes, lv, w.hdr,
                                                              w.rec, w.pmap, w.pos, table, k, v, scores, p.pages,
                                                              p.status);
  else
    prompt_pack_levels_kernel<64><<<grid, dim3(256), 0, s>>>(c.H, c.L, c.LT, total, p.P, p.page_bytes, lv, w.hdr,
                                                             w.rec, w.pmap, w.pos, table, k, v, scores, p.pages,
                                                             p.status);
  return hipGetLastError();
}

hipError_t launch_prompt(const Cfg& c, const Pool& p, int batch, int64_t total, const int64_t* cu,
                         const uint16_t* k, const uint16_t* v, const float* scores,
                         const uint8_t* tiers, int32_t* table, int32_t* state, void* ws,
                         hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  if (c.K >= 3) return launch_prompt_levels(c, p, batch, total, cu, k, v, scores, tiers, table, state, ws, s);
  PromptWs w = carve(c, batch, total, ws, nullptr);
  const int C = num_chunks(c);
  prompt_count_kernel<<<dim3(C, (unsigned)U), dim3(256), 0, s>>>(c.H, total, C, cu, tiers, w.chunks);
  prompt_plan_kernel<<<dim3(1), dim3(1024), 0, s>>>(c.H, c.L, c.S_max, batch, C, total, cu, state,
                                                    w.chunks, w.rec, w.hdr, p.ptr, p.status);
  prompt_scatter_kernel<<<dim3(C, (unsigned)U), dim3(256), 0, s>>>(c.H, c.L, C, total, p.P, tiers, w.hdr,
                                                                   w.rec, w.chunks, p.list, w.pos,
                                                                   w.freed, table, state);
  prompt_list_kernel<<<dim3((unsigned)U), dim3(256), 0, s>>>(c.L, p.P, w.hdr, w.rec, w.freed, p.list,
                                                             table, w.pmap);
  // persistent: as many 4-wave workgroups as fit on the device at once
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const Lay lay(c.d, c.plain, c.codec);
#define DKV_PACK(D, PL)                                                                                            \
  do {                                                                                                             \
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prompt_pack_kernel<D, PL>, 256, 0); \
    if (e != hipSuccess) return e;                                                                                 \
    const int64_t grid = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);                                 \
    prompt_pack_kernel<D, PL><<<dim3((unsigned)grid), dim3(256), 0, s>>>(                                          \
        c.H, c.L, total, p.P, p.page_bytes, lay.seg(true), lay.seg(false), w.hdr, w.rec, w.pmap, w.pos, table, k,  \
        v, scores, p.pages, p.status);                                                                             \
  } while (0)
  if (c.d == 128) {
    if (c.plain) DKV_PACK(128, true);
    else DKV_PACK(128, false);
  } else {
    if (c.plain) DKV_PACK(64, true);
    else DKV_PACK(64, false);
  }
#undef DKV_PACK
  return hipGetLastError();
}

}  // namespace dkv
