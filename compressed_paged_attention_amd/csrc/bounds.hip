// bounds.hip -- per-page key bounds and page scores (FlexiCache page, "3.2
// KV页评分机制", after Quest: each KV page keeps the per-dimension minimum and
// maximum of its keys; a query's page score is the largest dot product it
// could have with any key of the page, sum_i max(q_i kmin_i, q_i kmax_i);
// here the KV head's q heads are combined with max, as for token scores).
//
// The bounds live in a table of their own indexed by page id (as FlexiCache
// keeps its min-max vectors apart from the KV pages), fp32, over the
// dequantized keys of each page's retained slots -- the keys the attention
// reads -- so they are exact.
//   page_bounds_kernel: one thread per (page, dimension); every slot's code
//     byte and scale/zero word of the page are loaded before any is used (one
//     round trip per page, not one per slot), then min and max per dimension;
//     with K precision levels (DiffKV notes, "KV compression policy",
//     extensibility paragraph) every level's pages, each with its own codec
//     and page size;
//   page_scores_kernel: a wave per table entry, each lane D/64 dimensions,
//     the live entries enumerated densely, eight per wave and round (their
//     table ids, then their bounds, loaded before any is used); per q head
//     of the group the lane's max(q kmin, q kmax) terms, a wave sum in a
//     fixed butterfly order, then the max over the group, written in table
//     order (-inf at empty entries, filled in one coalesced pass).
// Both grids give each unit a fixed number of workgroups that stride over its
// live pages.
// HBM-bound: a refresh reads the K codes and metadata of every live page
// (~2.1 KB per page at d = 128) and writes 2d fp32; scoring reads the bounds.
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

namespace dkv {

namespace {


// A unit's level state is consistent: n_l >= 0 tokens in p_l = ceil(n_l / T_l)
// pages per level, and the two levels that share a table row fit in it.
__device__ inline bool levels_valid(const int32_t* s, const Levels& lv) {
  bool ok = true;
#pragma unroll
  for (int l = 0; l < 4; l++) {
    if (l < lv.K) ok = ok && s[l] >= 0 && s[lv.K + l] == (int)cdiv(s[l], lv.T(l));
  }
#pragma unroll
  for (int r = 0; r < 2; r++) {
    if (r < lv.R) ok = ok && s[lv.K + 2 * r] + (2 * r + 1 < lv.K ? s[lv.K + 2 * r + 1] : 0) <= lv.L;
  }
  return ok;
}

}  // namespace

// min and max over the first nv of a page's T slots for dimension dim:
// every slot's code and metadata loaded first (all in the page), then used
template <int D, bool HI>
__device__ inline void page_dim_bounds(const uint8_t* pg, int nv, int dim, float& mn, float& mx) {
  constexpr int T = HI ? kHiTokens : kLoTokens;
  constexpr Seg sg = tier_seg(D, HI);
  uint32_t cb[T], m[T];
#pragma unroll
  for (int t = 0; t < T; t++) {
    int byte, shift;
    k_field(D, HI, t, dim, byte, shift);
    cb[t] = (uint32_t)pg[sg.kc + byte] >> shift;
    m[t] = *(const uint32_t*)(pg + sg.km + 4 * t);
  }
  mn = INFINITY;
  mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < T; t++) {
    if (t >= nv) continue;
    const float x = dequant(h2f((uint16_t)m[t]), h2f((uint16_t)(m[t] >> 16)), cb[t] & (HI ? 0xFFu : 0xFu));
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
}

// The same for the plain layout of a tier codec variant (segment offsets and
// K width from sg; a code never spans two bytes).
template <int D, bool HI>
__device__ inline void page_dim_bounds_plain(const uint8_t* pg, int nv, int dim, const Seg& sg, float& mn,
                                             float& mx) {
  constexpr int T = HI ? kHiTokens : kLoTokens;
  const uint32_t mask = (1u << sg.kbits) - 1u;
  uint32_t cb[T], m[T];
#pragma unroll
  for (int t = 0; t < T; t++) {
    int byte, shift;
    plain_field(sg.kc, D, sg.kbits, t, dim, byte, shift);
    cb[t] = (uint32_t)pg[byte] >> shift;
    m[t] = *(const uint32_t*)(pg + sg.km + 4 * t);
  }
  mn = INFINITY;
  mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < T; t++) {
    if (t >= nv) continue;
    const float x = dequant(h2f((uint16_t)m[t]), h2f((uint16_t)(m[t] >> 16)), cb[t] & mask);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
}

// bounds: threads per workgroup (the plain layouts' kernels hold more
// registers per thread), and one workgroup per this many entries of a
// unit's table row
template <bool PLAIN>
constexpr int bnd_threads() { return PLAIN ? 512 : 1024; }
constexpr int kBndRowEntries = 512;
// page scores: workgroups of 16 waves, at most 8 per unit, each wave kNB
// live table entries per round
constexpr int kSThreads = 1024;
constexpr int kScoreWgPerUnit = 8;
constexpr int kNB = 8;

// bounds [P][2][D]: row 0 minima, row 1 maxima.  Levels in turn (the level
// is uniform over the grid, so the page size and codec are too); within a
// level the unit's workgroups stride over its pages.
template <int D, bool PLAIN>
__global__ __launch_bounds__(bnd_threads<PLAIN>()) void page_bounds_kernel(Levels lv, int64_t P, int page_bytes,
                                                               const int32_t* __restrict__ table,
                                                               const int32_t* __restrict__ state,
                                                               const uint8_t* __restrict__ pages,
                                                               float* __restrict__ bounds) {
  constexpr int PPB = bnd_threads<PLAIN>() / D;  // pages per workgroup and round
  const int64_t u = blockIdx.y;
  const int dim = threadIdx.x % D;
  const int K = lv.K;
  const int64_t LT = (int64_t)lv.R * lv.L;
  const int32_t* s = state + 2 * K * u;
  if (!levels_valid(s, lv)) return;
  for (int l = 0; l < K; l++) {
    const int n = s[l], np = s[K + l];
    // the level's layout by selects (a run-time index into the argument
    // would go through scratch memory)
    const Seg sg = l == 0 ? lv.s[0] : l == 1 ? lv.s[1] : l == 2 ? lv.s[2] : lv.s[3];
    for (int j = blockIdx.x * PPB + threadIdx.x / D; j < np; j += gridDim.x * PPB) {
      const int32_t id = table[u * LT + lv.entry(l, j)];
      if (id < 0 || id >= P) continue;
      const uint8_t* pg = pages + (int64_t)id * page_bytes;
      float mn, mx;
      if (l == 0) {
        const int nv = min(kHiTokens, n - kHiTokens * j);
        if constexpr (PLAIN) page_dim_bounds_plain<D, true>(pg, nv, dim, sg, mn, mx);
        else page_dim_bounds<D, true>(pg, nv, dim, mn, mx);
      } else {
        const int nv = min(kLoTokens, n - kLoTokens * j);
        if constexpr (PLAIN) page_dim_bounds_plain<D, false>(pg, nv, dim, sg, mn, mx);
        else page_dim_bounds<D, false>(pg, nv, dim, mn, mx);
      }
      float* bo = bounds + (int64_t)id * 2 * D;
      bo[dim] = mn;
      bo[D + dim] = mx;
    }
  }
}

// scores [U][R L] in table order (row r: level 2r from the left, 2r + 1
// from the right).  The empty entries get -inf in one coalesced pass; the
// live ones are enumerated densely (level by level) over the unit's waves.
template <int D>
__global__ __launch_bounds__(kSThreads) void page_scores_kernel(int H, int G, Levels lv, int64_t P,
                                                               const uint16_t* __restrict__ q,
                                                               const int32_t* __restrict__ table,
                                                               const int32_t* __restrict__ state,
                                                               const int32_t* __restrict__ seq_len,
                                                               const float* __restrict__ bounds,
                                                               float* __restrict__ scores) {
  constexpr int WPB = kSThreads / 64;  // waves per workgroup
  constexpr int DPL = D / 64;          // dimensions per lane: 2l, 2l + 1 (d = 128) or l (d = 64)
  const int64_t u = blockIdx.y;
  const int b = (int)(u / H), h = (int)(u % H);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int K = lv.K, L = lv.L, LT = lv.R * lv.L;
  const int32_t* s = state + 2 * K * u;
  const bool unit_ok = seq_len[b] > 0 && levels_valid(s, lv);
  const int p0 = unit_ok ? s[K] : 0, p1 = unit_ok ? s[K + 1] : 0;
  const int p2 = unit_ok && K > 2 ? s[K + 2] : 0, p3 = unit_ok && K > 3 ? s[K + 3] : 0;
  float* out = scores + u * LT;
  for (int tix = blockIdx.x * kSThreads + threadIdx.x; tix < LT; tix += gridDim.x * kSThreads) {
    const bool r1 = tix >= L;
    const int col = r1 ? tix - L : tix, pa = r1 ? p2 : p0, pb = r1 ? p3 : p1;
    if (!(col < pa || col >= L - pb)) out[tix] = -INFINITY;
  }
  const int nlive = p0 + p1 + p2 + p3;
  if (nlive == 0) return;
  // the group's query elements of this lane's dimensions (fp16 bits)
  uint32_t qw[16];
  const uint16_t* qb = q + ((int64_t)b * H * G + (int64_t)h * G) * D;
#pragma unroll
  for (int g = 0; g < 16; g++) {
    if (g >= G) {
      qw[g] = 0u;
    } else if constexpr (DPL == 2) {
      qw[g] = *(const uint32_t*)(qb + (int64_t)g * D + 2 * lane);
    } else {
      qw[g] = qb[(int64_t)g * D + lane];
    }
  }
  // live entry v -> table entry: level 0 from the left of row 0, level 1
  // from its right, levels 2 and 3 likewise in row 1
  auto entry_of = [&](int v) {
    return v < p0 ? v
                  : v < p0 + p1 ? L - 1 - (v - p0)
                                : v < p0 + p1 + p2 ? L + (v - p0 - p1) : 2 * L - 1 - (v - p0 - p1 - p2);
  };
  const int nw = gridDim.x * WPB;
  for (int v0 = blockIdx.x * WPB + wid; v0 < nlive; v0 += kNB * nw) {
    // kNB entries: their table ids, then their bounds, loaded before any is used
    int32_t id[kNB];
#pragma unroll
    for (int k = 0; k < kNB; k++) {
      const int v = v0 + k * nw;
      id[k] = v < nlive ? table[u * LT + entry_of(v)] : -1;
    }
    float mn[kNB][DPL], mx[kNB][DPL];
#pragma unroll
    for (int k = 0; k < kNB; k++) {
      const bool ok = id[k] >= 0 && id[k] < P;  // uniform over the wave
      const float* bp = bounds + (int64_t)(ok ? id[k] : 0) * 2 * D;
      if constexpr (DPL == 2) {
        float2 x0 = {0.0f, 0.0f}, x1 = {0.0f, 0.0f};
        if (ok) {
          x0 = *(const float2*)(bp + 2 * lane);
          x1 = *(const float2*)(bp + D + 2 * lane);
        }
        mn[k][0] = x0.x;
        mn[k][1] = x0.y;
        mx[k][0] = x1.x;
        mx[k][1] = x1.y;
      } else {
        mn[k][0] = ok ? bp[lane] : 0.0f;
        mx[k][0] = ok ? bp[D + lane] : 0.0f;
      }
    }
#pragma unroll
    for (int k = 0; k < kNB; k++) {
      const int v = v0 + k * nw;
      if (v >= nlive) continue;  // (uniform)
      float best = -INFINITY;
      if (id[k] >= 0 && id[k] < P) {
#pragma unroll
        for (int g = 0; g < 16; g++) {
          if (g < G) {  // (G is uniform)
            float x = 0.0f;
#pragma unroll
            for (int e = 0; e < DPL; e++) {
              const float qe = h2f((uint16_t)(qw[g] >> (16 * e)));
              x += fmaxf(qe * mn[k][e], qe * mx[k][e]);
            }
            best = fmaxf(best, wave_sum(x));  // fixed butterfly order
          }
        }
      }
      if (lane == 0) out[entry_of(v)] = best;
    }
  }
}

hipError_t launch_page_bounds(const Cfg& c, const Pool& p, int batch, const int32_t* table, const int32_t* state,
                              float* bounds, hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const int gx = (c.L + kBndRowEntries - 1) / kBndRowEntries;
  const dim3 grid((unsigned)gx, (unsigned)U), block(c.plain ? bnd_threads<true>() : bnd_threads<false>());
  const Levels lv = levels_of(c);
#define DKV_BOUNDS(D, PL) \
  page_bounds_kernel<D, PL><<<grid, block, 0, s>>>(lv, p.P, p.page_bytes, table, state, p.pages, bounds)
  if (c.d == 128) {
    if (c.plain) DKV_BOUNDS(128, true);
    else DKV_BOUNDS(128, false);
  } else {
    if (c.plain) DKV_BOUNDS(64, true);
    else DKV_BOUNDS(64, false);
  }
#undef DKV_BOUNDS
  return hipGetLastError();
}

hipError_t launch_page_scores(const Cfg& c, int64_t P, int batch, const uint16_t* q, const int32_t* table,
                              const int32_t* state, const int32_t* seq_len, const float* bounds, float* scores,
                              hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const int gx = min((c.LT + 511) / 512, kScoreWgPerUnit);
  const dim3 grid((unsigned)gx, (unsigned)U), block(kSThreads);
  const Levels lv = levels_of(c);
  if (c.d == 128)
    page_scores_kernel<128><<<grid, block, 0, s>>>(c.H, c.G, lv, P, q, table, state, seq_len, bounds, scores);
  else
    page_scores_kernel<64><<<grid, block, 0, s>>>(c.H, c.G, lv, P, q, table, state, seq_len, bounds, scores);
  return hipGetLastError();
}

}  // namespace dkv
