// keydiff.hip -- query-free token importance from the keys alone, an
// alternative input of classification (KeyDiff page, "方法细节": the anchor is
// the mean of the unit's normalized keys, or of the raw keys, and a key's
// eviction score is its cosine to the anchor; the least similar keys are the
// ones to keep).  Importance w_i = 1 - cos(anchor, k_i), normalized over the
// unit's tokens (uniform when every key is parallel to the anchor; a zero
// key or anchor has cosine 0), so the alpha/N thresholds apply as to the
// mean attention.
//
// HBM-bound (the keys are read twice); every sum runs in a fixed order, so
// the scores are deterministic:
//   kd_partial_kernel  per 256-token chunk: sum of the chunk's (normalized)
//                      keys, d floats;
//   kd_anchor_kernel   per unit: the chunks' sums in order -> anchor and norm;
//   kd_score_kernel    per chunk: w_i = 1 - cos, written to scores, and the
//                      chunk's sum of w;
//   kd_norm_kernel     per chunk: the unit's sum of w in order, scores /= it.
// A unit's chunks sit at workspace row floor(cu[r] / 256) + r onward, which
// keeps the units' rows apart whatever the lengths.
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

namespace dkv {

namespace {

constexpr int kChunk = 256;       // tokens per chunk (and threads per workgroup)

struct KdWs {
  float* part;  // [rows][H][D] chunk sums of keys
  float* mu;    // [B][H][D + 1] anchor and its norm
  float* wsum;  // [rows][H] chunk sums of w
};

inline int64_t kd_rows(int batch, int64_t total) { return total / kChunk + batch + 1; }

KdWs kd_carve(const Cfg& c, int batch, int64_t total, void* ws, size_t* bytes) {
  uint8_t* b = (uint8_t*)ws;
  const int64_t rows = kd_rows(batch, total);
  size_t off = 0;
  KdWs w;
  w.part = (float*)(b + off);
  off = align_up(off + (size_t)rows * c.H * c.d * sizeof(float), 256);
  w.mu = (float*)(b + off);
  off = align_up(off + (size_t)batch * c.H * (c.d + 1) * sizeof(float), 256);
  w.wsum = (float*)(b + off);
  off = align_up(off + (size_t)rows * c.H * sizeof(float), 256);
  if (bytes) *bytes = off;
  return w;
}

__device__ inline bool unit_range(const int64_t* cu, int r, int64_t total, int64_t& c0, int& N) {
  c0 = cu[r];
  const int64_t c1 = cu[r + 1];
  N = (int)(c1 - c0);
  return N > 0 && c0 >= 0 && c1 <= total;  // (a malformed entry: nothing read)
}

// one token row per group of D/8 lanes (8 dims each, one 16-byte load)
template <int D>
__device__ inline void load_row(const uint16_t* p, float* x) {
  const uint4 w = *(const uint4*)p;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; e++) {
    x[2 * e] = h2f((uint16_t)(ws[e] & 0xFFFFu));
    x[2 * e + 1] = h2f((uint16_t)(ws[e] >> 16));
  }
}

}  // namespace

// part[row][h][:] = sum over the chunk's tokens of k / |k| (raw: k)
template <int D>
__global__ __launch_bounds__(kChunk) void kd_partial_kernel(int H, int raw, const int64_t* __restrict__ cu,
                                                           int64_t total, const uint16_t* __restrict__ k,
                                                           float* __restrict__ part) {
  constexpr int LPT = D / 8;          // lanes per token
  constexpr int TPW = 64 / LPT;       // tokens per wave and round
  const int r = blockIdx.z, h = blockIdx.y;
  int64_t c0;
  int N;
  if (!unit_range(cu, r, total, c0, N)) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int sl = lane % LPT, tw = lane / LPT;  // dim slice, token within the round
  const int64_t base = c0 / kChunk + r;
  __shared__ float red[kChunk / 64][TPW][D];
  for (int ch = blockIdx.x; ch * kChunk < N; ch += gridDim.x) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // wave wid takes the chunk's tokens wid*64 .. wid*64+63, TPW at a time
    for (int t0 = wid * 64; t0 < wid * 64 + 64; t0 += TPW) {
      const int i = ch * kChunk + t0 + tw;
      if (i >= N) continue;  // (lanes of one token share the condition)
      float x[8];
      load_row<D>(k + ((c0 + i) * H + h) * D + 8 * sl, x);
      float nn = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; e++) nn = __builtin_fmaf(x[e], x[e], nn);
      nn = group_reduce<LPT>(nn, [](float a, float b) { return a + b; });
      const float inv = raw ? 1.0f : (nn > 0.0f ? 1.0f / sqrtf(nn) : 0.0f);
#pragma unroll
      for (int e = 0; e < 8; e++) acc[e] = __builtin_fmaf(x[e], inv, acc[e]);
    }
    // fixed-order sum over the token groups of each wave, then the waves
#pragma unroll
    for (int e = 0; e < 8; e++) red[wid][tw][8 * sl + e] = acc[e];
    __syncthreads();
    for (int j = tid; j < D; j += kChunk) {
      float s = 0.0f;
      for (int w = 0; w < kChunk / 64; w++)
        for (int g = 0; g < TPW; g++) s += red[w][g][j];
      part[((base + ch) * H + h) * D + j] = s;
    }
    __syncthreads();
  }
}

// mu[r][h][:] = sum of the unit's chunk sums / N; mu[r][h][D] = |mu|
template <int D>
__global__ __launch_bounds__(D) void kd_anchor_kernel(int H, const int64_t* __restrict__ cu, int64_t total,
                                                     const float* __restrict__ part, float* __restrict__ mu) {
  const int r = blockIdx.y, h = blockIdx.x, j = threadIdx.x;
  int64_t c0;
  int N;
  if (!unit_range(cu, r, total, c0, N)) return;
  const int64_t base = c0 / kChunk + r;
  const int nch = (N + kChunk - 1) / kChunk;
  float s = 0.0f;
  for (int ch = 0; ch < nch; ch++) s += part[((base + ch) * H + h) * D + j];
  s /= (float)N;
  __shared__ float sq[D];
  sq[j] = s * s;
  __syncthreads();
  float* m = mu + ((int64_t)r * H + h) * (D + 1);
  m[j] = s;
  if (j == 0) {
    float t = 0.0f;
    for (int e = 0; e < D; e++) t += sq[e];
    m[D] = sqrtf(t);
  }
}

// scores[h][c0 + i] = w_i = 1 - cos(mu, k_i); wsum[row][h] = the chunk's sum of w
template <int D>
__global__ __launch_bounds__(kChunk) void kd_score_kernel(int H, const int64_t* __restrict__ cu, int64_t total,
                                                         const uint16_t* __restrict__ k, const float* __restrict__ mu,
                                                         float* __restrict__ scores, float* __restrict__ wsum) {
  constexpr int LPT = D / 8;
  constexpr int TPW = 64 / LPT;
  // the blocks take the chunks in the reverse of kd_partial_kernel's order,
  // so the keys read last there are read first here, while the memory-side
  // cache may still hold them
  const int r = gridDim.z - 1 - blockIdx.z, h = gridDim.y - 1 - blockIdx.y;
  int64_t c0;
  int N;
  if (!unit_range(cu, r, total, c0, N)) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int sl = lane % LPT, tw = lane / LPT;
  const int64_t base = c0 / kChunk + r;
  const int nch = (N + kChunk - 1) / kChunk;
  const float* m = mu + ((int64_t)r * H + h) * (D + 1);
  float mv[8];
#pragma unroll
  for (int e = 0; e < 8; e++) mv[e] = m[8 * sl + e];
  const float mn = m[D];
  __shared__ float wl[kChunk];
  for (int cx = blockIdx.x; cx < nch; cx += gridDim.x) {
    const int ch = nch - 1 - cx;
    for (int t0 = wid * 64; t0 < wid * 64 + 64; t0 += TPW) {
      const int tt = t0 + tw, i = ch * kChunk + tt;
      if (i >= N) {
        if (sl == 0) wl[tt] = 0.0f;
        continue;
      }
      float x[8];
      load_row<D>(k + ((c0 + i) * H + h) * D + 8 * sl, x);
      float dot = 0.0f, nn = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        dot = __builtin_fmaf(x[e], mv[e], dot);
        nn = __builtin_fmaf(x[e], x[e], nn);
      }
      dot = group_reduce<LPT>(dot, [](float a, float b) { return a + b; });
      nn = group_reduce<LPT>(nn, [](float a, float b) { return a + b; });
      const float cs = (nn > 0.0f && mn > 0.0f) ? dot / (sqrtf(nn) * mn) : 0.0f;
      const float w = 1.0f - cs;
      if (sl == 0) {
        scores[(int64_t)h * total + c0 + i] = w;
        wl[tt] = w;
      }
    }
    __syncthreads();
    if (tid == 0) {
      float s = 0.0f;
      for (int t = 0; t < kChunk; t++) s += wl[t];
      wsum[(base + ch) * H + h] = s;
    }
    __syncthreads();
  }
}

// scores /= the unit's sum of w (chunk sums in order); 1/N when it is 0
__global__ __launch_bounds__(kChunk) void kd_norm_kernel(int H, const int64_t* __restrict__ cu, int64_t total,
                                                        const float* __restrict__ wsum, float* __restrict__ scores) {
  const int r = blockIdx.z, h = blockIdx.y;
  int64_t c0;
  int N;
  if (!unit_range(cu, r, total, c0, N)) return;
  const int64_t base = c0 / kChunk + r;
  const int nch = (N + kChunk - 1) / kChunk;
  __shared__ float s_tot;
  if (threadIdx.x == 0) {
    float s = 0.0f;
    for (int ch = 0; ch < nch; ch++) s += wsum[(base + ch) * H + h];
    s_tot = s;
  }
  __syncthreads();
  const float tot = s_tot;
  for (int ch = blockIdx.x; ch * kChunk < N; ch += gridDim.x) {
    const int i = ch * kChunk + threadIdx.x;
    if (i >= N) continue;
    float* p = scores + (int64_t)h * total + c0 + i;
    *p = tot > 0.0f ? *p / tot : 1.0f / (float)N;
  }
}

size_t keydiff_workspace(const Cfg& c, int batch, int64_t total) {
  size_t n = 0;
  kd_carve(c, batch, total, nullptr, &n);
  return n < 256 ? 256 : n;
}

hipError_t launch_keydiff(const Cfg& c, int batch, int64_t total, const int64_t* cu, const uint16_t* k, int raw,
                          float* scores, void* ws, hipStream_t s) {
  if (batch == 0 || total == 0) return hipSuccess;
  const KdWs w = kd_carve(c, batch, total, ws, nullptr);
  const int64_t maxlen = c.S_max < total ? c.S_max : total;
  const unsigned gx = (unsigned)((maxlen + kChunk - 1) / kChunk);
  const dim3 grid(gx, c.H, batch), block(kChunk);
  if (c.d == 128) {
    kd_partial_kernel<128><<<grid, block, 0, s>>>(c.H, raw, cu, total, k, w.part);
    kd_anchor_kernel<128><<<dim3(c.H, batch), dim3(128), 0, s>>>(c.H, cu, total, w.part, w.mu);
    kd_score_kernel<128><<<grid, block, 0, s>>>(c.H, cu, total, k, w.mu, scores, w.wsum);
  } else {
    kd_partial_kernel<64><<<grid, block, 0, s>>>(c.H, raw, cu, total, k, w.part);
    kd_anchor_kernel<64><<<dim3(c.H, batch), dim3(64), 0, s>>>(c.H, cu, total, w.part, w.mu);
    kd_score_kernel<64><<<grid, block, 0, s>>>(c.H, cu, total, k, w.mu, scores, w.wsum);
  }
  kd_norm_kernel<<<grid, block, 0, s>>>(c.H, cu, total, w.wsum, scores);
  return hipGetLastError();
}

}  // namespace dkv
