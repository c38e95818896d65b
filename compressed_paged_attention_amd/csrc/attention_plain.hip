// attention_plain.hip -- decode attention and score update over pages of a
// tier codec variant (DiffKV notes, "Results": the bit-split ablation of K
// and V code widths; plain page layout, widths in {1, 2, 4, 8}).
//
// What is computed is that of the default kernels ("Background": the softmax
// of q.k/sqrt(d) weighting v over the unit's retained tokens, K and V
// dequantized per token as s*c + z; "Implementation": high pages before low
// pages, sequence splits merged at the end), for any pair of widths per tier:
//
//   plain_attn_kernel   (split, unit) workgroups of 8 waves; wave w takes the
//                       split's pages w, w+8, ...  Per page (every load of
//                       the page issued first):
//     QK: lane = (token t, part of d): the token's codes of that part in
//         16-code blocks (2b bytes each), dequantized in fp32 and dotted with
//         the group's q heads (fp32 in LDS, padded with zero rows to GB);
//         the parts are summed with two (high page) or one (low page) lane
//         exchanges in a fixed order;
//     online softmax per head in base 2 (fp32);
//     PV: lane = d/64 consecutive dims; per token the lane's codes (one byte,
//         or two for 8-bit codes at d = 128), dequantized, times the token's
//         weights (broadcast LDS reads);
//   then the waves are merged in LDS in a fixed order into one partial
//   (unnormalized O, max, sum) per split and head, and the split merge of the
//   default path normalizes them (it also keeps (max, sum) for the score
//   update).
//   plain_score_kernel  the score update from the logits the attention kept:
//     each retained token with position < seq_len adds max_g of its softmax
//     weight to its score word.
//
// A bad page id makes its split's partial NaN: the merge then writes zeros
// for the unit and (max, sum) = (-inf, 0), so the score update skips it.
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

namespace dkv {

namespace {

constexpr int kPWaves = 8;
constexpr int kPThreads = 64 * kPWaves;
constexpr float kLog2eP = 1.4426950408889634f;

struct PlainWs {
  float* part;    // [U][S][G][D + 2]
  float* ml;      // [U][G][2] base-2 (max, sum) after the merge
  float* logits;  // [U][G][32 L] base-2 logits by slot (high slots, then low)
};

PlainWs plain_carve(const Cfg& c, int batch, bool scores, void* ws, size_t* bytes) {
  const int64_t U = (int64_t)batch * c.H;
  const int S = attn_splits(c, batch);
  uint8_t* b = (uint8_t*)ws;
  size_t off = 0;
  PlainWs w;
  w.part = (float*)(b + off);
  off = align_up(off + (size_t)U * S * c.G * (c.d + 2) * sizeof(float), 256);
  w.ml = (float*)(b + off);
  off = align_up(off + (size_t)U * c.G * 2 * sizeof(float), 256);
  w.logits = (float*)(b + off);
  if (scores) off = align_up(off + (size_t)U * c.G * 32 * c.LT * sizeof(float), 256);
  if (bytes) *bytes = off < 256 ? 256 : off;
  return w;
}

// A unit's levels: token counts n_l, page counts p_l (state words l and
// K + l), and the prefix sums pp_l (pages) and np_l (slots) of the levels
// before l, as scalars: looked up by a run-time level through selects (an
// array indexed at run time would live in scratch memory).
struct UnitLv {
  int n0, n1, n2, n3, pp1, pp2, pp3, pp4, np1, np2, np3, np4;
  bool ok;
  __device__ int n(int l) const { return l == 0 ? n0 : l == 1 ? n1 : l == 2 ? n2 : n3; }
  __device__ int pp(int l) const { return l == 0 ? 0 : l == 1 ? pp1 : l == 2 ? pp2 : l == 3 ? pp3 : pp4; }
  __device__ int np(int l) const { return l == 0 ? 0 : l == 1 ? np1 : l == 2 ? np2 : l == 3 ? np3 : np4; }
};

__device__ inline UnitLv unit_levels(const int32_t* s, const Levels& lv) {
  const int K = lv.K;
  const int n0 = s[0], n1 = s[1], n2 = K > 2 ? s[2] : 0, n3 = K > 3 ? s[3] : 0;
  const int p0 = s[K], p1 = s[K + 1], p2 = K > 2 ? s[K + 2] : 0, p3 = K > 3 ? s[K + 3] : 0;
  UnitLv x;
  x.n0 = n0;
  x.n1 = n1;
  x.n2 = n2;
  x.n3 = n3;
  x.pp1 = p0;
  x.pp2 = p0 + p1;
  x.pp3 = p0 + p1 + p2;
  x.pp4 = p0 + p1 + p2 + p3;
  x.np1 = n0;
  x.np2 = n0 + n1;
  x.np3 = n0 + n1 + n2;
  x.np4 = n0 + n1 + n2 + n3;
  x.ok = n0 >= 0 && n1 >= 0 && n2 >= 0 && n3 >= 0 && p0 == (int)cdiv(n0, kHiTokens) &&
         p1 == (int)cdiv(n1, kLoTokens) && p2 == (int)cdiv(n2, kLoTokens) && p3 == (int)cdiv(n3, kLoTokens) &&
         p0 + p1 <= lv.L && p2 + p3 <= lv.L;
  return x;
}

// level of the unit's page j (pages in level order)
__device__ inline int level_of_page(const UnitLv& x, int j) {
  return j < x.pp1 ? 0 : j < x.pp2 ? 1 : j < x.pp3 ? 2 : 3;
}
// level of the unit's slot s (slots in level order)
__device__ inline int level_of_slot(const UnitLv& x, int s) {
  return s < x.np1 ? 0 : s < x.np2 ? 1 : s < x.np3 ? 2 : 3;
}

// 16 codes of width B from a 2B-byte block (aligned to 2B bytes); code e at
// bit e B, little-endian.
template <int B>
__device__ inline void load16(const uint8_t* p, uint32_t (&w)[4]) {
  w[1] = w[2] = w[3] = 0u;
  if constexpr (B == 8) {
    const uint4 x = *(const uint4*)p;
    w[0] = x.x;
    w[1] = x.y;
    w[2] = x.z;
    w[3] = x.w;
  } else if constexpr (B == 4) {
    const uint2 x = *(const uint2*)p;
    w[0] = x.x;
    w[1] = x.y;
  } else if constexpr (B == 2) {
    w[0] = *(const uint32_t*)p;
  } else {
    w[0] = *(const uint16_t*)p;
  }
}

template <int B>
__device__ inline uint32_t code_at(const uint32_t (&w)[4], int e) {
  return (w[(e * B) >> 5] >> ((e * B) & 31)) & ((1u << B) - 1u);
}

// Everything one lane loads for one page: the K code blocks of its token and
// part of d (QK mapping), its token's K scale/zero word, the V scale/zero
// word of slot `lane`, and the bytes holding its V codes of every slot (d/64
// consecutive dims: one byte, or two for 8-bit codes at d = 128).  High
// pages use the first half of kw and cw.
template <int D>
struct PageLd {
  uint32_t kw[D / 32][4];
  uint32_t cw[kLoTokens];
  uint32_t kmw, vmw;
};

template <int D, int T, int KB>
__device__ inline void plain_load_k(const uint8_t* pg, const Seg& sg, int lane, int nv, PageLd<D>& r) {
  constexpr int PARTS = 64 / T, DP = D / PARTS, DL = D / 64;
  const int t = lane % T, part = lane / T;
  r.kmw = *(const uint32_t*)(pg + sg.km + 4 * t);
  r.vmw = lane < T ? *(const uint32_t*)(pg + sg.vm + 4 * lane) : 0u;
#pragma unroll
  for (int blk = 0; blk < DP / 16; blk++) load16<KB>(pg + sg.kc + (t * D + part * DP + 16 * blk) * KB / 8, r.kw[blk]);
  // V: slot k's codes of the lane's dims start at bit (k d + jd) b; k d b is
  // a whole number of bytes, so the shift (jd b mod 8) is the lane's own and
  // is applied where the codes are used.  Slots past nv are read too (they
  // are inside the page) and never used.
  const int vb = sg.vbits;
  const uint8_t* vbase = pg + sg.vc + ((lane * DL * vb) >> 3);
  const int stride = D * vb / 8;
  if (DL * vb <= 8) {
#pragma unroll
    for (int k = 0; k < T; k++) r.cw[k] = vbase[k * stride];
  } else {  // two 8-bit codes, 2-byte aligned
#pragma unroll
    for (int k = 0; k < T; k++) r.cw[k] = *(const uint16_t*)(vbase + k * stride);
  }
  (void)nv;
}

template <int D, int T>
__device__ inline void plain_load(const uint8_t* pg, const Seg& sg, int lane, int nv, PageLd<D>& r) {
  if (sg.kbits == 8) plain_load_k<D, T, 8>(pg, sg, lane, nv, r);
  else if (sg.kbits == 4) plain_load_k<D, T, 4>(pg, sg, lane, nv, r);
  else if (sg.kbits == 2) plain_load_k<D, T, 2>(pg, sg, lane, nv, r);
  else plain_load_k<D, T, 1>(pg, sg, lane, nv, r);
}

// q . k^ for the lane's token and part of d, every head of the padded group,
// from the codes: q . k^ = s (q . c) + z sum(q) (the parts of d summed
// first).  qs holds q as [d][GB] (one 16-byte read gives four heads of a
// dim), qsum the heads' sums.
template <int D, int T, int KB, int GB>
__device__ inline void plain_qk(const uint32_t (&w)[D / 32][4], uint32_t mw, int lane, const float* qs,
                                const float* qsum, float (&x)[GB]) {
  constexpr int PARTS = 64 / T, DP = D / PARTS;
  const int part = lane / T;
  float acc[GB];
#pragma unroll
  for (int g = 0; g < GB; g++) acc[g] = 0.0f;
#pragma unroll
  for (int blk = 0; blk < DP / 16; blk++) {
    const int j0 = part * DP + 16 * blk;
#pragma unroll
    for (int e = 0; e < 16; e++) {
      const float c = (float)code_at<KB>(w[blk], e);
      const float4* qv = (const float4*)(qs + (j0 + e) * GB);
#pragma unroll
      for (int g4 = 0; g4 < GB / 4; g4++) {
        const float4 q4 = qv[g4];
        acc[4 * g4 + 0] = __builtin_fmaf(q4.x, c, acc[4 * g4 + 0]);
        acc[4 * g4 + 1] = __builtin_fmaf(q4.y, c, acc[4 * g4 + 1]);
        acc[4 * g4 + 2] = __builtin_fmaf(q4.z, c, acc[4 * g4 + 2]);
        acc[4 * g4 + 3] = __builtin_fmaf(q4.w, c, acc[4 * g4 + 3]);
      }
    }
  }
  // the parts of d (lanes t + T k), summed in the same order in every lane
#pragma unroll
  for (int g = 0; g < GB; g++) {
    if constexpr (PARTS == 4) acc[g] += __shfl_xor(acc[g], 16, 64);
    acc[g] += __shfl_xor(acc[g], 32, 64);
  }
  const float s = h2f((uint16_t)(mw & 0xFFFFu)), z = h2f((uint16_t)(mw >> 16));
#pragma unroll
  for (int g = 0; g < GB; g++) x[g] = __builtin_fmaf(s, acc[g], z * qsum[g]);
}

template <int D, int T, int GB>
__device__ inline void plain_qk_any(int kb, const PageLd<D>& r, int lane, const float* qs, const float* qsum,
                                    float (&x)[GB]) {
  if (kb == 8) plain_qk<D, T, 8, GB>(r.kw, r.kmw, lane, qs, qsum, x);
  else if (kb == 4) plain_qk<D, T, 4, GB>(r.kw, r.kmw, lane, qs, qsum, x);
  else if (kb == 2) plain_qk<D, T, 2, GB>(r.kw, r.kmw, lane, qs, qsum, x);
  else plain_qk<D, T, 1, GB>(r.kw, r.kmw, lane, qs, qsum, x);
}

// o[g][e] += p'[t][g] c[t][lane dims] over the page's nv slots, pw holding
// this wave's p' = p s_v as [32][16] (the z_v part is summed separately:
// sum_t p v^ = sum_t (p s_v) c + sum_t p z_v).
template <int D, int T, int GB>
__device__ inline void plain_pv(int vb, const uint32_t (&cw)[kLoTokens], int nv, int lane, const float* pw,
                                float (&o)[GB][D / 64]) {
  constexpr int DL = D / 64;
  const uint32_t mask = (1u << vb) - 1u;
  const int sh = (lane * DL * vb) & 7;  // the lane's first code within its byte
#pragma unroll
  for (int t = 0; t < T; t++) {
    if (t < nv) {  // uniform
      float c[DL];
#pragma unroll
      for (int e = 0; e < DL; e++) c[e] = (float)((cw[t] >> (sh + e * vb)) & mask);
      const float4* pv = (const float4*)(pw + t * 16);
#pragma unroll
      for (int g4 = 0; g4 < GB / 4; g4++) {
        const float4 p4 = pv[g4];
#pragma unroll
        for (int e = 0; e < DL; e++) {
          o[4 * g4 + 0][e] = __builtin_fmaf(p4.x, c[e], o[4 * g4 + 0][e]);
          o[4 * g4 + 1][e] = __builtin_fmaf(p4.y, c[e], o[4 * g4 + 1][e]);
          o[4 * g4 + 2][e] = __builtin_fmaf(p4.z, c[e], o[4 * g4 + 2][e]);
          o[4 * g4 + 3][e] = __builtin_fmaf(p4.w, c[e], o[4 * g4 + 3][e]);
        }
      }
    }
  }
}

// LDS operations of one wave complete in program order; this keeps the
// compiler from moving them across the point
__device__ inline void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

}  // namespace

// One page of one wave from its loaded words: QK, the online softmax update
// of (m, l, o, zs) and PV.  lg: where the page's logits go (slot t of head g
// at lg[g LS + t]), or null.  zs: this lane's share of sum_t p z_v per head
// (lanes below T).
template <int D, int T, int GB>
__device__ inline void plain_page(const PageLd<D>& r, const Seg& sg, int lane, int nv, int G, int64_t LS, float* lg,
                                  const float* qs, const float* qsum, float scale_log2, float* pw, float (&m)[GB],
                                  float (&l)[GB], float (&o)[GB][D / 64], float (&zs)[GB]) {
  constexpr int DL = D / 64;
  float x[GB];
  plain_qk_any<D, T, GB>(sg.kbits, r, lane, qs, qsum, x);
  const int t = lane % T;
  const bool first = lane < T, live = t < nv;
  const float sv = h2f((uint16_t)(r.vmw & 0xFFFFu)), zv = h2f((uint16_t)(r.vmw >> 16));
#pragma unroll
  for (int g = 0; g < GB; g++) x[g] = live ? x[g] * scale_log2 : -INFINITY;
  if (lg && first && live)
    for (int g = 0; g < G; g++) lg[g * LS + t] = x[g];
  wave_lds_order();  // the previous page's weights have been read
#pragma unroll
  for (int g = 0; g < GB; g++) {
    const float mn = fmaxf(m[g], wave_max(x[g]));  // finite: nv >= 1
    const float al = __builtin_amdgcn_exp2f(m[g] - mn);
    const float p = (first && live) ? __builtin_amdgcn_exp2f(x[g] - mn) : 0.0f;
    l[g] = l[g] * al + wave_sum(p);
#pragma unroll
    for (int e = 0; e < DL; e++) o[g][e] *= al;
    zs[g] = __builtin_fmaf(p, zv, zs[g] * al);
    m[g] = mn;
    if (first) pw[t * 16 + g] = p * sv;
  }
  wave_lds_order();
  plain_pv<D, T, GB>(sg.vbits, r.cw, nv, lane, pw, o);
}

template <int D, int GB>
__global__ __launch_bounds__(kPThreads) void plain_attn_kernel(int H, int G, int L, int S, int64_t P, int page_bytes,
                                                               int LT, Levels lv, float scale_log2,
                                                               int keep_logits,
                                                               const uint16_t* __restrict__ q,
                                                               const int32_t* __restrict__ table,
                                                               const int32_t* __restrict__ state,
                                                               const int32_t* __restrict__ seq_len,
                                                               const uint8_t* __restrict__ pages,
                                                               float* __restrict__ out, float* __restrict__ part,
                                                               float* __restrict__ logits, uint32_t* status) {
  constexpr int DL = D / 64;
  const int split = blockIdx.x;
  const int64_t u = blockIdx.y;
  const int b = (int)u / H, h = (int)u % H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: page choice and loads in scalar registers
  __shared__ __align__(16) float qs[D * GB];  // [d][GB]
  __shared__ float qsum[GB];
  __shared__ __align__(16) float ps[kPWaves][32 * 16];
  __shared__ float sml[kPWaves][GB][2];
  __shared__ float ob[kPWaves][GB * D];
  const int N = seq_len[b];
  if (N <= 0) {
    if (split == 0)
      for (int x = tid; x < G * D; x += kPThreads) out[((int64_t)b * H * G + (int64_t)h * G) * D + x] = 0.0f;
    return;
  }
  const UnitLv ux = unit_levels(state + 2 * lv.K * u, lv);
  const bool sok = ux.ok;
  if (!sok && split == 0 && tid == 0) atomicOr(status, kStBadState);
  const int TPg = sok ? ux.pp4 : 0;
  const int pps = split_pages(TPg, S);
  const int p0 = split * pps, p1 = min(TPg, p0 + pps);
  // the group's q heads (fp32, [d][GB]; heads G..GB-1 zero) and their sums
  const uint16_t* qb = q + ((int64_t)b * H * G + (int64_t)h * G) * D;
  for (int x = tid; x < GB * D; x += kPThreads) {
    const int g = x / D, j = x % D;
    qs[j * GB + g] = g < G ? h2f(qb[x]) : 0.0f;
  }
  __syncthreads();
  if (tid < GB) {
    float a = 0.0f;
    for (int j = 0; j < D; j++) a += qs[j * GB + tid];
    qsum[tid] = a;
  }
  __syncthreads();
  float m[GB], l[GB], o[GB][DL], zs[GB];
#pragma unroll
  for (int g = 0; g < GB; g++) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
    zs[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < DL; e++) o[g][e] = 0.0f;
  }
  bool bad = false;
  float* pw = ps[wid];
  const int64_t LS = (int64_t)32 * LT;
  // The wave's pages j = p0 + wid + 8k.  Software pipeline: the table id two
  // pages ahead and every load of the next page are issued before the
  // current page is computed.
  auto id_of = [&](int jj) {
    const int l = level_of_page(ux, jj);
    return table[u * LT + lv.entry(l, jj - ux.pp(l))];
  };
  auto ok_id = [&](int32_t id) { return id >= 0 && id < P; };
  auto nv_of = [&](int l, int jt) { return min(lv.T(l), ux.n(l) - lv.T(l) * jt); };
  auto load = [&](int jj, int32_t id, PageLd<D>& r) {
    const int l = level_of_page(ux, jj);
    const int jt = jj - ux.pp(l);
    const uint8_t* pg = pages + (int64_t)id * page_bytes;
    if (l == 0) plain_load<D, kHiTokens>(pg, lv.s[0], lane, nv_of(0, jt), r);
    else plain_load<D, kLoTokens>(pg, lv.s[l], lane, nv_of(l, jt), r);
  };
  int j = p0 + wid;
  int32_t id_cur = j < p1 ? id_of(j) : -1;
  int32_t id_nx = j + kPWaves < p1 ? id_of(j + kPWaves) : -1;
  PageLd<D> cur;
  if (j < p1 && ok_id(id_cur)) load(j, id_cur, cur);
  for (; j < p1; j += kPWaves) {
    const int jn = j + kPWaves;
    const int32_t id_n = id_nx;
    id_nx = jn + kPWaves < p1 ? id_of(jn + kPWaves) : -1;
    PageLd<D> nxt;
    if (jn < p1 && ok_id(id_n)) load(jn, id_n, nxt);
    if (!ok_id(id_cur)) {
      bad = true;
    } else {
      const int lev = level_of_page(ux, j);
      const int jt = j - ux.pp(lev);
      const int nv = nv_of(lev, jt);
      const int slot0 = ux.np(lev) + lv.T(lev) * jt;
      float* lg = keep_logits ? logits + u * G * LS + slot0 : nullptr;
      if (lev == 0) plain_page<D, kHiTokens, GB>(cur, lv.s[0], lane, nv, G, LS, lg, qs, qsum, scale_log2, pw, m, l, o, zs);
      else plain_page<D, kLoTokens, GB>(cur, lv.s[lev], lane, nv, G, LS, lg, qs, qsum, scale_log2, pw, m, l, o, zs);
    }
    cur = nxt;
    id_cur = id_n;
  }
  // the z_v part of every dim: the wave's sum of p z_v
#pragma unroll
  for (int g = 0; g < GB; g++) {
    const float zt = wave_sum(zs[g]);
#pragma unroll
    for (int e = 0; e < DL; e++) o[g][e] += zt;
  }
  // the waves' partials, merged in a fixed order
  if (lane == 0)
#pragma unroll
    for (int g = 0; g < GB; g++) {
      sml[wid][g][0] = m[g];
      sml[wid][g][1] = l[g];
    }
#pragma unroll
  for (int g = 0; g < GB; g++)
#pragma unroll
    for (int e = 0; e < DL; e++) ob[wid][g * D + lane * DL + e] = o[g][e];
  bad = __syncthreads_or(bad);
  if (bad && tid == 0) atomicOr(status, kStBadState);
  float* up = part + ((u * S + split) * G) * (D + 2);
  for (int x = tid; x < G * D; x += kPThreads) {
    const int g = x / D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kPWaves; w++) M = fmaxf(M, sml[w][g][0]);
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kPWaves; w++) {
      const float mw = sml[w][g][0];
      const float wt = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      acc += ob[w][x] * wt;
    }
    up[g * (D + 2) + (x % D)] = acc;
  }
  if (tid < G) {
    const int g = tid;
    float M = -INFINITY, Lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kPWaves; w++) M = fmaxf(M, sml[w][g][0]);
#pragma unroll
    for (int w = 0; w < kPWaves; w++) {
      const float mw = sml[w][g][0];
      if (mw != -INFINITY) Lsum += sml[w][g][1] * __builtin_amdgcn_exp2f(mw - M);
    }
    up[g * (D + 2) + D] = bad ? __builtin_nanf("") : M;
    up[g * (D + 2) + D + 1] = Lsum;
  }
}

// One thread per retained slot of the unit (grid x: blocks of 256 slots).
__global__ __launch_bounds__(256) void plain_score_kernel(int H, int G, int LT, int64_t P, int page_bytes, Levels lv,
                                                          const int32_t* __restrict__ table,
                                                          const int32_t* __restrict__ state,
                                                          const int32_t* __restrict__ seq_len,
                                                          const float* __restrict__ ml,
                                                          const float* __restrict__ logits, uint8_t* pages) {
  const int64_t u = blockIdx.y;
  const int b = (int)u / H;
  const int N = seq_len[b];
  if (N <= 0) return;
  const UnitLv ux = unit_levels(state + 2 * lv.K * u, lv);
  if (!ux.ok) return;
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= ux.np4) return;
  if (!(ml[u * G * 2 + 1] > 0.0f)) return;  // bad unit
  const int lev = level_of_slot(ux, s);
  const int ls = s - ux.np(lev), T = lv.T(lev);
  const int jt = ls / T, idx = ls % T;
  const int32_t id = table[u * LT + lv.entry(lev, jt)];
  if (id < 0 || id >= P) return;
  const int64_t LS = (int64_t)32 * LT;
  float pmax = 0.0f;
  for (int g = 0; g < G; g++) {
    const float M = ml[(u * G + g) * 2 + 0], Ls = ml[(u * G + g) * 2 + 1];
    const float p = __builtin_amdgcn_exp2f(logits[(u * G + g) * LS + s] - M) / Ls;
    pmax = fmaxf(pmax, p);
  }
  const Seg& sg = lv.s[lev];
  uint8_t* pg = pages + (int64_t)id * page_bytes;
  const int32_t pos = *(const int32_t*)(pg + sg.ps + 4 * idx);
  if (pos >= N) return;
  float* sc = (float*)(pg + sg.sc + 4 * idx);
  *sc = *sc + pmax;
}

size_t plain_attn_workspace(const Cfg& c, int batch, bool scores) {
  size_t n = 0;
  plain_carve(c, batch, scores, nullptr, &n);
  return n;
}

hipError_t launch_scores_plain(const Cfg& c, const Pool& p, int batch, const int32_t* table, const int32_t* state,
                               const int32_t* seq_len, void* ws, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const PlainWs w = plain_carve(c, batch, true, ws, nullptr);
  const dim3 grid((unsigned)((32 * (int64_t)c.LT + 255) / 256), (unsigned)U), block(256);
  plain_score_kernel<<<grid, block, 0, s>>>(c.H, c.G, c.LT, p.P, p.page_bytes, levels_of(c), table, state, seq_len,
                                            w.ml, w.logits, p.pages);
  return hipGetLastError();
}

hipError_t launch_attn_plain(const Cfg& c, const Pool& p, int batch, const uint16_t* q, const int32_t* table,
                             const int32_t* state, const int32_t* seq_len, float* out, int mode, void* ws,
                             hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const int S = attn_splits(c, batch);
  const PlainWs w = plain_carve(c, batch, mode != 0, ws, nullptr);
  const float scale_log2 = (1.0f / sqrtf((float)c.d)) * kLog2eP;
  const dim3 grid((unsigned)S, (unsigned)U), block(kPThreads);
  const Levels lv = levels_of(c);
  const int GB = c.G <= 4 ? 4 : (c.G <= 8 ? 8 : 16);
#define DKV_PATTN(D, GB_)                                                                                      \
  plain_attn_kernel<D, GB_><<<grid, block, 0, s>>>(c.H, c.G, c.L, S, p.P, p.page_bytes, c.LT, lv, scale_log2,  \
                                                   mode != 0, q, table, state, seq_len, p.pages, out, w.part,  \
                                                   w.logits, p.status)
#define DKV_PATTN_D(D)              \
  if (GB == 4) DKV_PATTN(D, 4);     \
  else if (GB == 8) DKV_PATTN(D, 8); \
  else DKV_PATTN(D, 16);
  if (c.d == 128) {
    DKV_PATTN_D(128)
  } else {
    DKV_PATTN_D(64)
  }
#undef DKV_PATTN_D
#undef DKV_PATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_attn_merge(c, batch, S, seq_len, w.part, out, w.ml, mode != 0, s);
  if (e != hipSuccess) return e;
  if (mode == 1) return launch_scores_plain(c, p, batch, table, state, seq_len, ws, s);
  return hipSuccess;
}

}  // namespace dkv
