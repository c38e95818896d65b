// bounds.hip -- per-page key bounds and page scores (FlexiCache page, "3.2
// KV页评分机制", after Quest: each KV page keeps the per-dimension minimum and
// maximum of its keys; a query's page score is the largest dot product it
// could have with any key of the page, sum_i max(q_i kmin_i, q_i kmax_i);
// here the KV head's q heads are combined with max, as for token scores).
//
// The bounds live in a table of their own indexed by page id (as FlexiCache
// keeps its min-max vectors apart from the KV pages), fp32, over the
// dequantized keys of each page's retained slots -- the keys the attention
// reads -- so they are exact.  One thread per (page, dimension):
//   page_bounds_kernel: walks the page's valid slots (codes and scale/zero),
//     min and max per dimension;
//   page_scores_kernel: per q head of the group the block sum of
//     max(q kmin, q kmax) in a fixed order, max over the group, written in
//     table order (-inf at empty entries).
// HBM-bound: a refresh reads the K codes and metadata of every live page
// (~2.1 KB per page at d = 128) and writes 2d fp32; scoring reads the bounds.
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

namespace dkv {

namespace {

constexpr int kBThreads = 256;

__device__ inline bool state_valid(int nh, int nl, int ph, int pl, int L) {
  return nh >= 0 && nl >= 0 && ph == (int)cdiv(nh, kHiTokens) && pl == (int)cdiv(nl, kLoTokens) && ph + pl <= L;
}

}  // namespace

// bounds [P][2][D]: row 0 minima, row 1 maxima
template <int D>
__global__ __launch_bounds__(kBThreads) void page_bounds_kernel(int L, int64_t P, int page_bytes,
                                                               const int32_t* __restrict__ table,
                                                               const int32_t* __restrict__ state,
                                                               const uint8_t* __restrict__ pages,
                                                               float* __restrict__ bounds) {
  constexpr int PPB = kBThreads / D;  // pages per workgroup
  const int64_t u = blockIdx.y;
  const int pj = blockIdx.x * PPB + threadIdx.x / D, dim = threadIdx.x % D;
  const int32_t* s4 = state + 4 * u;
  const int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  if (!state_valid(nh, nl, ph, pl, L) || pj >= ph + pl) return;
  const bool hi = pj < ph;
  const int jt = hi ? pj : pj - ph;
  const int32_t id = table[u * L + (hi ? jt : L - 1 - jt)];
  if (id < 0 || id >= P) return;
  const int nv = hi ? min(kHiTokens, nh - kHiTokens * jt) : min(kLoTokens, nl - kLoTokens * jt);
  const Seg sg = tier_seg(D, hi);
  const uint8_t* pg = pages + (int64_t)id * page_bytes;
  float mn = INFINITY, mx = -INFINITY;
  for (int t = 0; t < nv; t++) {
    int byte, shift;
    k_field(D, hi, t, dim, byte, shift);
    const uint32_t code = (uint32_t)(pg[sg.kc + byte] >> shift) & (hi ? 0xFFu : 0xFu);
    const uint32_t m = *(const uint32_t*)(pg + sg.km + 4 * t);
    const float x = dequant(h2f((uint16_t)m), h2f((uint16_t)(m >> 16)), code);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  float* b = bounds + (int64_t)id * 2 * D;
  b[dim] = mn;
  b[D + dim] = mx;
}

// scores [U][L] in table order
template <int D>
__global__ __launch_bounds__(kBThreads) void page_scores_kernel(int H, int G, int L, int64_t P,
                                                               const uint16_t* __restrict__ q,
                                                               const int32_t* __restrict__ table,
                                                               const int32_t* __restrict__ state,
                                                               const int32_t* __restrict__ seq_len,
                                                               const float* __restrict__ bounds,
                                                               float* __restrict__ scores) {
  constexpr int PPB = kBThreads / D;
  constexpr int WPP = D / 64;  // waves per page
  const int64_t u = blockIdx.y;
  const int b = (int)(u / H), h = (int)(u % H);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int pp = tid / D, dim = tid % D;
  const int tix = blockIdx.x * PPB + pp;  // table index of this thread's page
  const int32_t* s4 = state + 4 * u;
  const int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  const bool live = seq_len[b] > 0 && state_valid(nh, nl, ph, pl, L) && tix < L && (tix < ph || tix >= L - pl);
  const int32_t id = live ? table[u * L + tix] : -1;
  const bool ok = live && id >= 0 && id < P;
  const float* bp = bounds + (int64_t)(ok ? id : 0) * 2 * D;
  const float mn = ok ? bp[dim] : 0.0f, mx = ok ? bp[D + dim] : 0.0f;
  __shared__ float part[kBThreads / 64];
  float best = -INFINITY;
  for (int g = 0; g < G; g++) {
    const float qe = h2f(q[((int64_t)b * H * G + (int64_t)h * G + g) * D + dim]);
    float v = fmaxf(qe * mn, qe * mx);
    v = wave_sum(v);  // the 64 dims of this wave, fixed butterfly order
    __syncthreads();
    if (lane == 0) part[wid] = v;
    __syncthreads();
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < WPP; w++) s += part[pp * WPP + w];
    best = fmaxf(best, s);
  }
  if (dim == 0 && tix < L) scores[u * L + tix] = ok ? best : -INFINITY;
}

hipError_t launch_page_bounds(const Cfg& c, const Pool& p, int batch, const int32_t* table, const int32_t* state,
                              float* bounds, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const int ppb = kBThreads / c.d;
  const dim3 grid((unsigned)((c.L + ppb - 1) / ppb), (unsigned)U), block(kBThreads);
  if (c.d == 128)
    page_bounds_kernel<128><<<grid, block, 0, s>>>(c.L, p.P, p.page_bytes, table, state, p.pages, bounds);
  else
    page_bounds_kernel<64><<<grid, block, 0, s>>>(c.L, p.P, p.page_bytes, table, state, p.pages, bounds);
  return hipGetLastError();
}

hipError_t launch_page_scores(const Cfg& c, int64_t P, int batch, const uint16_t* q, const int32_t* table,
                              const int32_t* state, const int32_t* seq_len, const float* bounds, float* scores,
                              hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const int ppb = kBThreads / c.d;
  const dim3 grid((unsigned)((c.L + ppb - 1) / ppb), (unsigned)U), block(kBThreads);
  if (c.d == 128)
    page_scores_kernel<128><<<grid, block, 0, s>>>(c.H, c.G, c.L, P, q, table, state, seq_len, bounds, scores);
  else
    page_scores_kernel<64><<<grid, block, 0, s>>>(c.H, c.G, c.L, P, q, table, state, seq_len, bounds, scores);
  return hipGetLastError();
}

}  // namespace dkv
