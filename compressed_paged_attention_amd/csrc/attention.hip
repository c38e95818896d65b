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
// so only integer codes (exact fp16 subnormals) enter the matrix units.  P' is split
// into an fp16 head and an fp16 tail (two instructions) so the PV product
// keeps ~22 bits.  The online softmax rescales lazily (reference max moves
// by more than 2^4 at a time).  The S accumulator layout equals the P'^T operand layout,
// so softmax needs no data movement between the two products.  K codes are
// read token-major (lane: token l%16, a quarter of d); V codes are stored in
// 64 lane chunks so each lane issues one 16-byte load per page.  The online
// softmax is fp32 in base 2.  The waves are merged in LDS by a fixed-order
// tree (deterministic).  With one split per unit the same workgroup then runs
// the score update over the unit's saved logits; with several splits the
// partials go through a merge kernel.  No device-scope fence is used: on a
// multi-XCD part those write back and invalidate whole L2 caches.
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

namespace dkv {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;              // waves per attention workgroup
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float4_t mfma16(half4_t a, half4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Codes enter the matrix units as fp16 subnormals: the 16-bit pattern c is
// the fp16 value c * 2^-24 (exact), so unpacking is a mask or a byte permute
// and the 2^24 is restored in fp32 (K: folded into the scale; V: at the
// merge).  The matrix instruction keeps fp16 subnormal inputs exactly.
__device__ inline half4_t cat(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(half4_t, (uint64_t)a | ((uint64_t)b << 32));
}
// 4 u8 codes of one dword -> 4 subnormal fp16 codes in order (byte permutes
// with zero bytes: selector 0x0C gives 0x00)
__device__ inline half4_t u8x4(uint32_t w) {
  return cat(__builtin_amdgcn_perm(0u, w, 0x0C010C00u), __builtin_amdgcn_perm(0u, w, 0x0C030C02u));
}
// the fields at bits s and s+16 of a dword -> subnormal fp16 pair
__device__ inline uint32_t nib2(uint32_t w, int s) { return (w >> s) & 0x000F000Fu; }
__device__ inline uint32_t crumb2(uint32_t w, int s) { return (w >> s) & 0x00030003u; }
constexpr float kTwo24 = 16777216.0f;

int attn_splits(const Cfg& c, int batch) {
  const int64_t U = (int64_t)batch * c.H;
  if (U <= 0) return 1;
  int64_t S = (256 + U - 1) / U;  // about one 8-wave workgroup per compute unit
  int64_t cap = c.L / 16;
  if (cap < 1) cap = 1;
  if (S > cap) S = cap;
  if (S > 64) S = 64;
  if (S < 1) S = 1;
  return (int)S;
}

struct AttnWs {
  float* part;    // [U][S][G][D + 2] split partials (unnormalized O, max, sum)
  float* ml;      // [U][G][2] final (max, sum) in base 2, for the score update
  float* logits;  // [U][L][32][G] base-2 logits of every retained slot
};

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
  if (scores) off = align_up(off + (size_t)U * c.L * 32 * c.G * sizeof(float), 256);
  if (bytes) *bytes = off < 256 ? 256 : off;
  return w;
}

size_t attn_workspace(const Cfg& c, int batch, bool scores) {
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
template <int D>
struct PageRegs {
  static constexpr int KW = D / 32;  // dwords per K load
  uint32_t k[2 * KW];  // high: 2*KW dwords of token i; low: KW of token i, KW of i+16
  uint32_t km[8];      // K (scale, zero) words: tokens 4qg.. (low: and 16+4qg..)
  uint32_t vm[8];      // V (scale, zero) words
  uint32_t v[KW];      // the lane's V chunk
};

template <int N>
__device__ inline void ldw(uint32_t* r, const uint8_t* p) {
  if constexpr (N == 4) {
    const uint4 a = *(const uint4*)p;
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  } else {
    const uint2 a = *(const uint2*)p;
    r[0] = a.x; r[1] = a.y;
  }
}

// kb: lane K offset of the high tier (token i, dims qg*D/4); the low tier's
// is kb/2 (token i) and kb/2 + 16*D/2 (token i + 16).  mq = 16 qg, vl = lane
// chunk offset.  Metadata segments start at the same offset in both tiers.
template <int D>
__device__ inline void load_page(PageRegs<D>& R, const uint8_t* pg, bool lo, int kb, int mq, int vl) {
  constexpr int KW = PageRegs<D>::KW;
  constexpr Seg sh = tier_seg(D, true), sl = tier_seg(D, false);
  static_assert(sh.km == sl.km, "K metadata offsets differ between tiers");
  const int k0 = lo ? (kb >> 1) : kb;
  const int k1 = lo ? (kb >> 1) + 16 * (D / 2) : kb + 4 * KW;
  ldw<KW>(R.k, pg + k0);
  ldw<KW>(R.k + KW, pg + k1);
  ldw<4>(R.km, pg + sh.km + mq);
  ldw<4>(R.km + 4, pg + sh.km + mq + (lo ? 64 : 0));
  const int vm = lo ? sl.vm : sh.vm;
  ldw<4>(R.vm, pg + vm + mq);
  ldw<4>(R.vm + 4, pg + vm + mq + (lo ? 64 : 0));
  ldw<KW>(R.v, pg + (lo ? sl.vc : sh.vc) + vl);
}

struct Softmax {
  float m, lsum, zsum;  // reference max (base 2), sum of weights, sum of weight * z_v
};

// The reference max moves only when a block's max exceeds it by more than
// kLazy (base 2), so weights stay <= 2^kLazy and the accumulators are
// rescaled rarely.  P' = p s_v is carried at 2^-kLazy so its fp16 head can
// never overflow (|P'| 2^-kLazy <= s_v); the scale is restored at the merge.
constexpr float kLazy = 4.0f;
constexpr float kPScale = 1.0f / 16.0f;  // 2^-kLazy

// One 16-token block: logits (masked), online-softmax update, PV products.
// `s` holds q.c * 2^-24 for tokens first..first+3 of the page; `kmw`/`vmw`
// the metadata words of those tokens; `vpair(nb)` the fp16 V operand of
// 16-dim block nb; `keep(x)` stores the block's logits.
template <int D, typename VOp, typename Keep>
__device__ inline void block_update(const float4_t& s, const uint32_t* kmw, const uint32_t* vmw, int first,
                                    int nval, float sumq, float scale_log2, Softmax& sm, float4_t* acc,
                                    VOp vpair, Keep keep) {
  constexpr int NB = D / 16;
  float x[4];
  float pm = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    // q.k^ = s_k q.c + z_k sum(q); s holds q.c * 2^-24
    const float ks = h2f((uint16_t)kmw[r]) * kTwo24, kz = h2f((uint16_t)(kmw[r] >> 16));
    x[r] = (ks * s[r] + kz * sumq) * scale_log2;
    if (first + r >= nval) x[r] = -INFINITY;
    pm = fmaxf(pm, x[r]);
  }
  keep(x);
  pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
  pm = fmaxf(pm, __shfl_xor(pm, 32, 64));
  if (__any(pm > sm.m + kLazy)) {
    const float mn = pm > sm.m + kLazy ? pm : sm.m;
    const float alpha = __builtin_amdgcn_exp2f(sm.m - mn);
    sm.lsum *= alpha;
    sm.zsum *= alpha;
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[nb] *= alpha;
    sm.m = mn;
  }
  float p[4];
  _Float16 ph16[4], pl16[4];
#pragma unroll
  for (int r = 0; r < 4; r++) {
    p[r] = __builtin_amdgcn_exp2f(x[r] - sm.m);
    sm.lsum += p[r];
    sm.zsum += p[r] * h2f((uint16_t)(vmw[r] >> 16));
    const float pp = p[r] * h2f((uint16_t)vmw[r]) * kPScale;
    ph16[r] = (_Float16)pp;
    pl16[r] = (_Float16)(pp - (float)ph16[r]);
  }
  const half4_t bh = {ph16[0], ph16[1], ph16[2], ph16[3]};
  const half4_t bl = {pl16[0], pl16[1], pl16[2], pl16[3]};
#pragma unroll
  for (int nb = 0; nb < NB; nb++) {
    const half4_t a = vpair(nb);
    acc[nb] = mfma16(a, bh, acc[nb]);
    acc[nb] = mfma16(a, bl, acc[nb]);
  }
}

// keep(mb, x): stores the 4 logits of 16-token block mb of the page
template <int D, typename Keep>
__device__ inline void compute_page(const PageRegs<D>& R, bool hi, int nval, const half4_t* qop, float sumq,
                                    float scale_log2, int qg, Softmax& sm, float4_t* acc, Keep keep) {
  constexpr int NB = D / 16, KW = PageRegs<D>::KW;
  if (hi) {
    // two accumulators halve the dependent chain of the q.c products
    float4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
#pragma unroll
    for (int kb = 0; kb < NB; kb += 2) {
      s0 = mfma16(u8x4(R.k[kb]), qop[kb], s0);
      s1 = mfma16(u8x4(R.k[kb + 1]), qop[kb + 1], s1);
    }
    block_update<D>(
        s0 + s1, R.km, R.vm, 4 * qg, nval, sumq, scale_log2, sm, acc,
        [&](int nb) {
          // block nb: pairs 2nb (tokens 0, 1) and 2nb + 1 (tokens 2, 3)
          const uint32_t w = R.v[nb >> 1];
          const int sft = 8 * (nb & 1);
          return cat(nib2(w, sft), nib2(w, sft + 4));
        },
        [&](const float* x) { keep(0, x); });
  } else {
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
      float4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
#pragma unroll
      for (int kb = 0; kb < NB; kb += 2) {
        const uint32_t w = R.k[KW * mb + (kb >> 1)];
        s0 = mfma16(cat(nib2(w, 0), nib2(w, 4)), qop[kb], s0);
        s1 = mfma16(cat(nib2(w, 8), nib2(w, 12)), qop[kb + 1], s1);
      }
      block_update<D>(
          s0 + s1, R.km + 4 * mb, R.vm + 4 * mb, 16 * mb + 4 * qg, nval, sumq, scale_log2, sm, acc,
          [&](int nb) {
            // block (nb, mb): pairs P = 2M, 2M + 1 with M = 2nb + mb, in word P / 8
            const int M = 2 * nb + mb;
            const int P0 = 2 * M, P1 = 2 * M + 1;
            return cat(crumb2(R.v[P0 >> 3], 2 * (P0 & 7)), crumb2(R.v[P1 >> 3], 2 * (P1 & 7)));
          },
          [&](const float* x) { keep(mb, x); });
    }
  }
}

constexpr int kLgCap = 16384;  // logits kept in LDS when a unit needs at most this many

// MODE 0: attention; 1: attention + score update in the same workgroup (one
// split only); 2: attention keeping logits (score update later).
template <int D, int MODE>
__global__ __launch_bounds__(kThreads) void attn_kernel(int H, int G, int L, int S, int64_t P, int page_bytes,
                                                        float scale_log2, const uint16_t* __restrict__ q,
                                                        const int32_t* __restrict__ table,
                                                        const int32_t* __restrict__ state,
                                                        const int32_t* __restrict__ seq_len, uint8_t* pages,
                                                        float* __restrict__ out, float* __restrict__ part,
                                                        float* __restrict__ ml, float* logits, uint32_t* status) {
  constexpr bool SAVE = MODE != 0;
  constexpr int NB = D / 16;  // 16-dim blocks (K-steps of QK, N-blocks of PV)
  constexpr int QD = D / 4;   // dims per lane group
  const int split = blockIdx.x;
  const int64_t u = blockIdx.y;
  const int b = (int)(u / H), h = (int)(u % H);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loop control
  const int i = lane & 15, qg = lane >> 4;
  const int32_t* row = table + u * L;
  const int32_t* s4 = state + 4 * u;
  const int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  const int N = seq_len[b];
  const bool sok = state_ok(nh, nl, ph, pl, L);
  const int TPg = sok ? ph + pl : 0;
  const int pps = (TPg + S - 1) / S;
  const int p0 = split * pps;
  const int p1 = min(TPg, p0 + pps);

  __shared__ float wm[kWaves][16], wl[kWaves][16], sM[16], sL[16];
  __shared__ float4_t buf[kWaves / 2][16 * D / 4];  // kWaves even
  __shared__ float lg_s[MODE == 1 ? kLgCap : 1];

  float* orow = out + ((int64_t)b * H * G + (int64_t)h * G) * D;
  if (N <= 0 || !sok || nh + nl == 0) {
    if (S == 1 || split == 0) {
      for (int x = tid; x < G * D; x += blockDim.x) orow[x] = 0.0f;
      if (SAVE)
        for (int x = tid; x < G; x += blockDim.x) {
          ml[(u * G + x) * 2 + 0] = -INFINITY;
          ml[(u * G + x) * 2 + 1] = 0.0f;
        }
      if (N > 0 && !sok && tid == 0) atomicOr(status, kStBadState);
    }
    if (S > 1) {
      float* mp = part + (((int64_t)u * S + split) * G) * (D + 2);
      for (int x = tid; x < G; x += blockDim.x) {
        mp[x * (D + 2) + D] = -INFINITY;
        mp[x * (D + 2) + D + 1] = 0.0f;
      }
    }
    return;
  }

  auto table_idx = [&](int j) { return j < ph ? j : L - 1 - (j - ph); };
  auto valid = [&](int j) {
    return j < ph ? min(kHiTokens, nh - kHiTokens * j) : min(kLoTokens, nl - kLoTokens * (j - ph));
  };
  const int kbase = i * D + qg * (D / 4), mq = 16 * qg, vl = lane * (D / 8);
  uint32_t badid = 0;
  // page ids are checked where they are used; a bad id is clamped into the
  // pool (the load stays in bounds) and zeroes the unit's result
  auto fetch = [&](PageRegs<D>& R, int jj) {
    jj = min(jj, p1 - 1);  // past the end: reload the last page (unused)
    int32_t id = row[table_idx(jj)];  // uniform index: scalar load
    badid |= (uint32_t)(id < 0 || id >= P);
    id = min(max(id, 0), (int32_t)(P - 1));
    load_page<D>(R, pages + (int64_t)id * page_bytes, jj >= ph, kbase, mq, vl);
  };
  PageRegs<D> A, B;
  const bool busy = p0 + wid < p1;
  if (busy) fetch(A, p0 + wid);

  // ---- Q operand: lane (i, qg) holds head i, dims qg*QD .. qg*QD+QD-1 ----
  half4_t qop[NB];
  float sumq = 0.0f;
  {
    uint16_t qv[QD];
    if (i < G) {
      const uint4* src = (const uint4*)(q + ((int64_t)b * H * G + (int64_t)h * G + i) * D + qg * QD);
#pragma unroll
      for (int c = 0; c < QD / 8; c++) {
        const uint4 w = src[c];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          qv[8 * c + 2 * e] = (uint16_t)(ws[e] & 0xFFFFu);
          qv[8 * c + 2 * e + 1] = (uint16_t)(ws[e] >> 16);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < QD; e++) qv[e] = 0;
    }
#pragma unroll
    for (int e = 0; e < QD; e++) sumq += h2f(qv[e]);
    auto H16 = [&](int e) { return __builtin_bit_cast(_Float16, qv[e]); };
#pragma unroll
    for (int kb = 0; kb < NB; kb++)
      qop[kb] = half4_t{H16(4 * kb), H16(4 * kb + 1), H16(4 * kb + 2), H16(4 * kb + 3)};
    sumq += __shfl_xor(sumq, 16, 64);
    sumq += __shfl_xor(sumq, 32, 64);
  }

  Softmax sm{-INFINITY, 0.0f, 0.0f};
  float4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++) acc[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // logits go to LDS when the whole unit's fit (fused score update), else to
  // the workspace (indexed by table slot)
  const bool lg_lds = MODE == 1 && TPg * 32 * G <= kLgCap;

  // ---- page loop: the next page's loads in flight during each compute ----
  if (busy) {
    auto run = [&](const PageRegs<D>& R, int j) {
      const int lgl = j * 32 * G, lgg = table_idx(j) * 32 * G;
      compute_page<D>(R, j < ph, valid(j), qop, sumq, scale_log2, qg, sm, acc, [&](int mb, const float* x) {
        if (!SAVE || i >= G) return;
        const int t0 = 16 * mb + 4 * qg;
        if (MODE == 1 && lg_lds) {
#pragma unroll
          for (int r = 0; r < 4; r++) lg_s[lgl + (t0 + r) * G + i] = x[r];
        } else {
#pragma unroll
          for (int r = 0; r < 4; r++) logits[(int64_t)u * L * 32 * G + lgg + (t0 + r) * G + i] = x[r];
        }
      });
    };
    int j = p0 + wid;
    while (true) {
      fetch(B, j + kWaves);
      run(A, j);
      j += kWaves;
      if (j >= p1) break;
      fetch(A, j + kWaves);
      run(B, j);
      j += kWaves;
      if (j >= p1) break;
    }
  }

  // ---- merge the waves: maxima, rescale, fixed-order tree in LDS ----
  sm.lsum += __shfl_xor(sm.lsum, 16, 64);
  sm.lsum += __shfl_xor(sm.lsum, 32, 64);
  sm.zsum += __shfl_xor(sm.zsum, 16, 64);
  sm.zsum += __shfl_xor(sm.zsum, 32, 64);
  __shared__ uint32_t s_bad;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (badid) s_bad = 1;
  if (qg == 0) {
    wm[wid][i] = sm.m;
    wl[wid][i] = sm.lsum;
  }
  __syncthreads();
  const bool bad = s_bad != 0;
  if (tid < 16) {
    float M = -INFINITY;
    for (int w = 0; w < kWaves; w++) M = fmaxf(M, wm[w][tid]);
    float l = 0.0f;
    if (M != -INFINITY)
      for (int w = 0; w < kWaves; w++) l += wl[w][tid] * __builtin_amdgcn_exp2f(wm[w][tid] - M);
    sM[tid] = M;
    sL[tid] = l;
  }
  __syncthreads();
  {
    const float M = sM[i];
    const float f = (M == -INFINITY || sm.m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sm.m - M);
#pragma unroll
    for (int nb = 0; nb < NB; nb++) acc[nb] = (acc[nb] * (kTwo24 / kPScale) + sm.zsum) * f;
  }
  // lane (i, qg), block nb holds dims 16nb + 4qg .. +3 of head i -> float4
  // slot; waves [half, active) fold into [0, active - half), fixed order
#pragma unroll
  for (int active = kWaves; active > 1; active = (active + 1) >> 1) {
    const int half = (active + 1) >> 1;
    if (wid >= half && wid < active) {
#pragma unroll
      for (int nb = 0; nb < NB; nb++) buf[wid - half][i * (D / 4) + 4 * nb + qg] = acc[nb];
    }
    __syncthreads();
    if (wid < active - half) {
#pragma unroll
      for (int nb = 0; nb < NB; nb++) acc[nb] += buf[wid][i * (D / 4) + 4 * nb + qg];
    }
    __syncthreads();
  }

  if (bad && tid == 0) atomicOr(status, kStBadState);
  if (S == 1) {
    if (bad) {
      for (int x = tid; x < G * D; x += blockDim.x) orow[x] = 0.0f;
      if (SAVE && tid < G) {
        ml[(u * G + tid) * 2 + 0] = -INFINITY;
        ml[(u * G + tid) * 2 + 1] = 0.0f;
      }
      return;
    }
    if (wid == 0 && i < G) {
      const float inv = sL[i] > 0.0f ? 1.0f / sL[i] : 0.0f;
#pragma unroll
      for (int nb = 0; nb < NB; nb++) *(float4_t*)(orow + i * D + 16 * nb + 4 * qg) = acc[nb] * inv;
    }
    if (SAVE && tid < G) {
      ml[(u * G + tid) * 2 + 0] = sM[tid];
      ml[(u * G + tid) * 2 + 1] = sL[tid];
    }
    if (MODE == 1) {
      // score update: every retained token other than the query's own
      // (position seq_len) adds max over the group of its softmax weight
      if (tid < 16) sL[tid] = sL[tid] > 0.0f ? 1.0f / sL[tid] : 0.0f;
      __syncthreads();
      const Seg sh = tier_seg(D, true), sl = tier_seg(D, false);
      const float* lgg = logits + (int64_t)u * L * 32 * G;
      constexpr int kU = 4;
      for (int x0 = tid; x0 < TPg * 32; x0 += kU * blockDim.x) {
        float* sc[kU];
        const int32_t* pp[kU];
        float old[kU], add[kU];
#pragma unroll
        for (int e = 0; e < kU; e++) {
          const int x = x0 + e * blockDim.x;
          const int j = x >> 5, t = x & 31;
          sc[e] = nullptr;
          add[e] = 0.0f;
          if (x < TPg * 32 && t < valid(j)) {
            const float* lg = lg_lds ? lg_s + (j * 32 + t) * G : lgg + (table_idx(j) * 32 + t) * G;
            float mx = 0.0f;
            for (int g = 0; g < G; g++) mx = fmaxf(mx, __builtin_amdgcn_exp2f(lg[g] - sM[g]) * sL[g]);
            add[e] = mx;
            const uint8_t* pg = pages + (int64_t)row[table_idx(j)] * page_bytes;
            sc[e] = (float*)(pg + (j < ph ? sh.sc : sl.sc) + 4 * t);
            pp[e] = (const int32_t*)(pg + (j < ph ? sh.ps : sl.ps) + 4 * t);
          }
        }
        int32_t pos[kU];
#pragma unroll
        for (int e = 0; e < kU; e++) {
          old[e] = sc[e] ? *sc[e] : 0.0f;
          pos[e] = sc[e] ? *pp[e] : N;
        }
#pragma unroll
        for (int e = 0; e < kU; e++)
          if (sc[e] && pos[e] < N) *sc[e] = old[e] + add[e];
      }
    }
  } else {
    float* mp = part + (((int64_t)u * S + split) * G) * (D + 2);
    if (wid == 0 && i < G) {
#pragma unroll
      for (int nb = 0; nb < NB; nb++)
#pragma unroll
        for (int r = 0; r < 4; r++) mp[i * (D + 2) + 16 * nb + 4 * qg + r] = acc[nb][r];
    }
    if (tid < G) {
      mp[tid * (D + 2) + D] = bad ? NAN : sM[tid];  // NaN marks a bad unit for the merge
      mp[tid * (D + 2) + D + 1] = sL[tid];
    }
  }
}

// Split merge (several workgroups per unit): out = sum_s O_s 2^(m_s - M) /
// sum_s l_s 2^(m_s - M); also the final (M, L) for the score update.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(int H, int G, int S, const int32_t* __restrict__ seq_len,
                                                         const float* __restrict__ part, float* __restrict__ out,
                                                         float* __restrict__ ml, int save) {
  const int64_t u = blockIdx.x;
  const int b = (int)(u / H), h = (int)(u % H);
  if (seq_len[b] <= 0) return;  // the attention kernel already wrote zeros
  const float* up = part + (u * S * G) * (D + 2);
  float* orow = out + ((int64_t)b * H * G + (int64_t)h * G) * D;
  for (int x = threadIdx.x; x < G * D; x += blockDim.x) {
    const int g = x / D, dd = x % D;
    float M = -INFINITY;
    bool bad = false;
    for (int sp = 0; sp < S; sp++) {
      const float ms = up[(sp * G + g) * (D + 2) + D];
      bad |= ms != ms;
      M = fmaxf(M, ms);
    }
    float o = 0.0f, l = 0.0f;
    if (bad) M = -INFINITY;
    else if (M != -INFINITY)
      for (int sp = 0; sp < S; sp++) {
        const float* pp = up + (sp * G + g) * (D + 2);
        if (pp[D] == -INFINITY) continue;
        const float f = __builtin_amdgcn_exp2f(pp[D] - M);
        o += pp[dd] * f;
        l += pp[D + 1] * f;
      }
    orow[x] = l > 0.0f ? o / l : 0.0f;
    if (save && dd == 0) {
      ml[(u * G + g) * 2 + 0] = M;
      ml[(u * G + g) * 2 + 1] = l;
    }
  }
}

// Score update from saved logits (several splits, or a deferred update).
template <int D>
__global__ __launch_bounds__(256) void score_kernel(int H, int G, int L, int S, int64_t P, int page_bytes,
                                                    const int32_t* __restrict__ table,
                                                    const int32_t* __restrict__ state,
                                                    const int32_t* __restrict__ seq_len,
                                                    const float* __restrict__ ml,
                                                    const float* __restrict__ logits, uint8_t* pages) {
  const int split = blockIdx.x;
  const int64_t u = blockIdx.y;
  const int b = (int)(u / H);
  const int tid = threadIdx.x;
  const int32_t* row = table + u * L;
  const int32_t* s4 = state + 4 * u;
  const int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  const int N = seq_len[b];
  if (N <= 0 || nh + nl == 0 || !state_ok(nh, nl, ph, pl, L)) return;
  if (!unit_ids(ph, pl, L, P, row)) return;
  __shared__ float sM[16], sI[16];
  if (tid < G) {
    sM[tid] = ml[(u * G + tid) * 2 + 0];
    const float l = ml[(u * G + tid) * 2 + 1];
    sI[tid] = l > 0.0f ? 1.0f / l : 0.0f;
  }
  __syncthreads();
  const int TPg = ph + pl;
  const int pps = (TPg + S - 1) / S;
  const int p0 = split * pps;
  const int p1 = min(TPg, p0 + pps);
  const Seg sh = tier_seg(D, true), sl = tier_seg(D, false);
  for (int x = tid; x < (p1 - p0) * 32; x += blockDim.x) {
    const int j = p0 + x / 32, t = x % 32;
    const bool is_hi = j < ph;
    const int jt = is_hi ? j : j - ph;
    const int nval = is_hi ? min(kHiTokens, nh - kHiTokens * jt) : min(kLoTokens, nl - kLoTokens * jt);
    if (t >= nval) continue;
    const int tidx = is_hi ? jt : L - 1 - jt;
    const uint8_t* pg = pages + (int64_t)row[tidx] * page_bytes;
    if (*(const int32_t*)(pg + (is_hi ? sh.ps : sl.ps) + 4 * t) >= N) continue;
    const float* lg = logits + (((int64_t)u * L + tidx) * 32 + t) * G;
    float mx = 0.0f;
    for (int g = 0; g < G; g++) mx = fmaxf(mx, __builtin_amdgcn_exp2f(lg[g] - sM[g]) * sI[g]);
    float* sc = (float*)(pg + (is_hi ? sh.sc : sl.sc) + 4 * t);
    *sc = *sc + mx;
  }
}

hipError_t launch_scores(const Cfg& c, const Pool& p, int batch, const int32_t* table, const int32_t* state,
                         const int32_t* seq_len, void* ws, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const int S = attn_splits(c, batch);
  AttnWs w = attn_carve(c, batch, true, ws, nullptr);
  const dim3 grid(S, (unsigned)U), block(256);
  if (c.d == 128)
    score_kernel<128><<<grid, block, 0, s>>>(c.H, c.G, c.L, S, p.P, p.page_bytes, table, state, seq_len, w.ml,
                                             w.logits, p.pages);
  else
    score_kernel<64><<<grid, block, 0, s>>>(c.H, c.G, c.L, S, p.P, p.page_bytes, table, state, seq_len, w.ml,
                                            w.logits, p.pages);
  return hipGetLastError();
}

hipError_t launch_attn(const Cfg& c, const Pool& p, int batch, const uint16_t* q, const int32_t* table,
                       const int32_t* state, const int32_t* seq_len, float* out, int mode, void* ws,
                       hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const int S = attn_splits(c, batch);
  AttnWs w = attn_carve(c, batch, mode != 0, ws, nullptr);
  const float scale_log2 = (1.0f / sqrtf((float)c.d)) * kLog2e;
  const dim3 grid(S, (unsigned)U), block(kThreads);
  // a single split runs the score update inside the attention workgroup
  const int kmode = mode == 1 && S > 1 ? 2 : mode;
#define DKV_ATTN(D, M)                                                                                     \
  attn_kernel<D, M><<<grid, block, 0, s>>>(c.H, c.G, c.L, S, p.P, p.page_bytes, scale_log2, q, table,   \
                                           state, seq_len, p.pages, out, w.part, w.ml, w.logits, p.status)
  if (c.d == 128) {
    if (kmode == 0) DKV_ATTN(128, 0);
    else if (kmode == 1) DKV_ATTN(128, 1);
    else DKV_ATTN(128, 2);
  } else {
    if (kmode == 0) DKV_ATTN(64, 0);
    else if (kmode == 1) DKV_ATTN(64, 1);
    else DKV_ATTN(64, 2);
  }
#undef DKV_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (S > 1) {
    if (c.d == 128)
      attn_merge_kernel<128><<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.G, S, seq_len, w.part, out, w.ml,
                                                                     mode != 0);
    else
      attn_merge_kernel<64><<<dim3((unsigned)U), dim3(256), 0, s>>>(c.H, c.G, S, seq_len, w.part, out, w.ml,
                                                                    mode != 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mode == 1) return launch_scores(c, p, batch, table, state, seq_len, ws, s);
  }
  return hipSuccess;
}

}  // namespace dkv
