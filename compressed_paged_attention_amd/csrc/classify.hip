// classify.hip -- pool/state initialisation and token classification.
//
// Classification follows the "Approach" summary and the prompt-phase logic
// of "KV compression policy" in the DiffKV notes: the most recent W tokens
// are high precision; any other token is high if its mean score exceeds
// alpha_h/N, low if it lies in [alpha_l/N, alpha_h/N], pruned below
// alpha_l/N (N = the request's length).  The comparison is s*N against alpha
// in fp64, exact for N < 2^29, so no division rounding decides a tier.
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

namespace dkv {

__global__ void pool_init_kernel(int32_t* list, uint64_t* ptr, uint32_t* status, int64_t P) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < P) list[i] = (int32_t)i;
  if (i == 0) {
    ptr[0] = 0;
    ptr[1] = (uint64_t)P;
    status[0] = 0;
  }
}

__global__ void state_init_kernel(int32_t* table, int64_t n_table, int32_t* state, int64_t n_state) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_table) table[i] = -1;
  if (i < n_state) state[i] = 0;
}

hipError_t launch_pool_init(const Pool& p, hipStream_t s) {
  const int64_t blocks = (p.P + 255) / 256;
  pool_init_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p.list, p.ptr, p.status, p.P);
  return hipGetLastError();
}

hipError_t launch_state_init(const Cfg& c, int batch, int32_t* table, int32_t* state, hipStream_t s) {
  const int64_t nt = (int64_t)batch * c.H * c.LT, ns = (int64_t)batch * c.H * 2 * c.K;
  const int64_t n = nt > ns ? nt : ns;
  if (n == 0) return hipSuccess;
  state_init_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(table, nt, state, ns);
  return hipGetLastError();
}

// rule 0: s N against alpha (threshold alpha/N); rule 1: s (p + 1) against
// alpha (threshold alpha/i for the i-th token, i = p + 1)
__device__ inline int tier_of(float s, int64_t N, int64_t p, int W, int lo_en, double ah, double al, int rule) {
  if (W > 0 && p >= N - W) return kTierHi;
  const double x = (double)s * (double)(rule ? p + 1 : N);
  if (lo_en) {
    if (x > ah) return kTierHi;
    return x >= al ? kTierLo : kTierPrune;
  }
  return x >= al ? kTierHi : kTierPrune;
}

// grid (H, batch); one workgroup per unit walks its tokens and reduces the
// two counts.
__global__ __launch_bounds__(1024) void classify_kernel(int H, int W, int lo_en, float ah, float al,
                                                        const float* __restrict__ ah_head,
                                                        const float* __restrict__ al_head, int rule,
                                                        int64_t total, const int64_t* __restrict__ cu,
                                                        const float* __restrict__ scores,
                                                        uint8_t* __restrict__ tiers,
                                                        int32_t* __restrict__ counts) {
  const int h = blockIdx.x, r = blockIdx.y;
  const int64_t b0 = cu[r], N = cu[r + 1] - b0;
  if (b0 < 0 || N < 0 || cu[r + 1] > total) {  // inconsistent offsets: nothing is read
    if (threadIdx.x == 0) {
      counts[((int64_t)r * H + h) * 2 + 0] = 0;
      counts[((int64_t)r * H + h) * 2 + 1] = 0;
    }
    return;
  }
  const float* s = scores + (int64_t)h * total + b0;
  uint8_t* t = tiers + (int64_t)h * total + b0;
  const double dah = (double)(ah_head ? ah_head[h] : ah), dal = (double)(al_head ? al_head[h] : al);
  int nh = 0, nl = 0;
  for (int64_t p = threadIdx.x; p < N; p += blockDim.x) {
    const int ti = tier_of(s[p], N, p, W, lo_en, dah, dal, rule);
    t[p] = (uint8_t)ti;
    nh += ti == kTierHi;
    nl += ti == kTierLo;
  }
  __shared__ int red[2][16];
  nh = wave_sum(nh);
  nl = wave_sum(nl);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wid] = nh;
    red[1][wid] = nl;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0, b = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); w++) {
      a += red[0][w];
      b += red[1][w];
    }
    counts[((int64_t)r * H + h) * 2 + 0] = a;
    counts[((int64_t)r * H + h) * 2 + 1] = b;
  }
}

// K precision levels: the first level l < K-1 with x > alpha_l, else level
// K-1 if x >= alpha_{K-1}, else pruned; code K - l (0 pruned).
// (a0: level 0's threshold, a1 and a2 the middle levels', aL the last's)
__device__ inline int level_code(float s, int64_t N, int64_t p, int W, int K, double a0, double a1, double a2,
                                 double aL, int rule) {
  if (W > 0 && p >= N - W) return K;
  const double x = (double)s * (double)(rule ? p + 1 : N);
  if (x > a0) return K;
  if (x > a1) return K - 1;
  if (K == 4 && x > a2) return 2;
  return x >= aL ? 1 : 0;
}

// grid (H, batch); one workgroup per unit, K counts per unit
__global__ __launch_bounds__(1024) void classify_levels_kernel(int H, int W, int K, float ah, float al, float am0,
                                                               float am1, const float* __restrict__ ah_head,
                                                               const float* __restrict__ al_head, int rule,
                                                               int64_t total, const int64_t* __restrict__ cu,
                                                               const float* __restrict__ scores,
                                                               uint8_t* __restrict__ tiers,
                                                               int32_t* __restrict__ counts) {
  const int h = blockIdx.x, r = blockIdx.y;
  const int64_t b0 = cu[r], N = cu[r + 1] - b0;
  int32_t* cnt = counts + ((int64_t)r * H + h) * K;
  const bool ok = !(b0 < 0 || N < 0 || cu[r + 1] > total);  // inconsistent offsets: nothing is read
  const double a0 = (double)(ah_head ? ah_head[h] : ah), aL = (double)(al_head ? al_head[h] : al);
  int n[4] = {0, 0, 0, 0};
  if (ok) {
    const float* s = scores + (int64_t)h * total + b0;
    uint8_t* t = tiers + (int64_t)h * total + b0;
    for (int64_t p = threadIdx.x; p < N; p += blockDim.x) {
      const int code = level_code(s[p], N, p, W, K, a0, (double)am0, (double)am1, aL, rule);
      t[p] = (uint8_t)code;
#pragma unroll
      for (int l = 0; l < 4; l++) n[l] += l < K && code == K - l;
    }
  }
  __shared__ int red[4][16];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int l = 0; l < 4; l++) {
    n[l] = wave_sum(n[l]);
    if (lane == 0) red[l][wid] = n[l];
  }
  __syncthreads();
  if (threadIdx.x < K) {
    int x = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); w++) x += red[threadIdx.x][w];
    cnt[threadIdx.x] = x;
  }
}

hipError_t launch_classify(const Cfg& c, int batch, int64_t total, const int64_t* cu,
                           const float* scores, uint8_t* tiers, int32_t* counts, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  if (c.K >= 3) {
    classify_levels_kernel<<<dim3(c.H, batch), dim3(1024), 0, s>>>(c.H, c.W, c.K, c.ah, c.al, c.amid[0], c.amid[1],
                                                                   c.ah_head, c.al_head, c.prompt_rule, total, cu,
                                                                   scores, tiers, counts);
    return hipGetLastError();
  }
  classify_kernel<<<dim3(c.H, batch), dim3(1024), 0, s>>>(c.H, c.W, c.lo_en, c.ah, c.al, c.ah_head, c.al_head,
                                                          c.prompt_rule, total, cu,
                                                          scores, tiers, counts);
  return hipGetLastError();
}

}  // namespace dkv
