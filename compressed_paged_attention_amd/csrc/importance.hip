// importance.hip -- prompt-phase token importance on the GPU: the input of
// classification, computed from the prompt's own queries.
//
// What is computed (DiffKV notes, "KV compression policy", prompt phase): the
// importance of token i is the mean of the attention weights it receives from
// the tokens after it; the weights of the q heads that share a KV head are
// combined with max.  Causal attention: query j attends to keys 0..j with
// softmax(q_j . k / sqrt(d)).  For each later query j > i the group's weight
// of key i is max_g a^g_{j,i}; the importance is their mean over the N-1-i
// later queries (the token's own query excluded; the last token gets 0).
// A probe mode takes nq extra queries per request that see every token
// (count nq) -- the recipe of the tiny workload.
//
// MI355X mapping.  A dense contraction (every query against every earlier
// key), so the QK products run on the matrix units
// (v_mfma_f32_16x16x32_f16: A = 16 queries x 32 dims, B = 32 dims x 16 keys,
// lane l holds query rows 4(l/16)..+3 of key column l mod 16).  A workgroup
// of 4 waves owns a tile of 64 rows (16 per wave, kept in registers) and
// walks the other operand in 64-row tiles staged once per workgroup in LDS
// (rows padded by 32 bytes: a row stride of d/2 + 8 dwords puts the rows a
// 16-byte access serves together on disjoint banks -- the counters show no
// LDS bank conflicts with it, against 36-40 % of LDS cycles with 16 bytes),
// the next tile's global loads in flight during each tile's products:
//   imp_stats_kernel: per (64-query tile, q head) the softmax reference and
//     sum over the query's keys, lane-local online (each lane sees one key
//     column per block) merged over the 16 lanes of a row once; stores
//     c = -(max + log2 sum) in base 2, so a weight is 2^(x + c);
//   imp_sum_kernel: per (64-key tile, KV head) the keys stay in registers
//     while the workgroup walks the later query tiles and, per tile, the
//     group's heads (each head's query tile and references staged in LDS):
//     x + c masked to later queries, max over heads, then 2^ of it summed
//     per key;
//     the mean is written to scores[h][token].
// Both kernels loop over their tiles with a grid stride, so every length is
// covered whatever the grid.
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

namespace dkv {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kImpWaves = 4;  // waves per workgroup, each one 16-row block
constexpr float kL2e = 1.4426950408889634f;

__device__ inline float4_t mfma32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 fp16 of a row (16 bytes; rows are 16-byte aligned: d is a multiple of 8
// and the tensors start 16-byte aligned), or zeros for a row out of range
__device__ inline half8_t load8(const uint16_t* p, bool ok) {
  if (!ok) return half8_t{0, 0, 0, 0, 0, 0, 0, 0};
  return __builtin_bit_cast(half8_t, *(const uint4*)p);
}

// query row pointer of query j of request r, head qh
struct QRows {
  const uint16_t* q;
  int64_t base;     // causal: cu[r]; probe: r * nq
  int64_t stride;   // H * G * D
  __device__ const uint16_t* row(int64_t j, int qh, int D) const {
    return q + (base + j) * stride + (int64_t)qh * D;
  }
};

}  // namespace

constexpr int kTile = 64;  // rows per workgroup tile (16 per wave)

// A 64-row tile of fp16 rows of D, moved by the workgroup's 256 threads in
// 16-byte chunks: fetch (global -> registers, rows past `n` zero), then put
// (registers -> LDS rows of D + 8 halfs).
template <int D>
struct Tile {
  static constexpr int CPT = D / 32;  // chunks per thread: 64 rows x D/8 chunks / 256 threads
  static constexpr int LR = D + 16;   // LDS row, in halfs
  uint4 v[CPT];
  template <typename RowPtr>
  __device__ inline void fetch(int tid, int n0, int n, RowPtr row) {
#pragma unroll
    for (int e = 0; e < CPT; e++) {
      const int c = tid + 256 * e, rr = c / (D / 8), cc = c % (D / 8);
      const int x = n0 + rr;
      v[e] = x < n ? *(const uint4*)(row(x) + 8 * cc) : uint4{0u, 0u, 0u, 0u};
    }
  }
  __device__ inline void put(int tid, uint16_t* lds) const {
#pragma unroll
    for (int e = 0; e < CPT; e++) {
      const int c = tid + 256 * e, rr = c / (D / 8), cc = c % (D / 8);
      *(uint4*)(lds + rr * LR + 8 * cc) = v[e];
    }
  }
};

// the B / A operand slice a lane reads from an LDS tile: row 16 blk + col,
// dims 32 s + 8 rg .. + 7
template <int D>
__device__ inline half8_t lds8(const uint16_t* lds, int row, int s, int rg) {
  return __builtin_bit_cast(half8_t, *(const uint4*)(lds + row * Tile<D>::LR + 32 * s + 8 * rg));
}

// stats[qh][qtok] = -(M + log2 L) in base 2 over the keys query qtok sees.
template <int D>
__global__ __launch_bounds__(64 * kImpWaves) void imp_stats_kernel(int H, int G, int probe, int nq,
                                                                   const int64_t* __restrict__ cu,
                                                                   const uint16_t* __restrict__ q,
                                                                   const uint16_t* __restrict__ k,
                                                                   float* __restrict__ stats, int64_t nqtot,
                                                                   int64_t total, float scale_log2) {
  constexpr int NS = D / 32;
  __shared__ __align__(16) uint16_t ks[kTile * Tile<D>::LR];
  const int r = blockIdx.z, qh = blockIdx.y, h = qh / G;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int col = lane & 15, rg = lane >> 4;
  const int64_t c0 = cu[r];
  const int N = (int)(cu[r + 1] - c0);
  const int NQ = probe ? nq : N;
  if (N <= 0 || c0 < 0 || c0 + N > total) return;  // (a malformed cu_seqlens entry: nothing read)
  const QRows Q{q, probe ? (int64_t)r * nq : c0, (int64_t)H * G * D};
  auto krow = [&](int x) { return k + ((c0 + x) * H + h) * D; };
  for (int jt = blockIdx.x * kTile; jt < NQ; jt += gridDim.x * kTile) {
    // A operand: query jb + col, dims 8 rg + 32 s
    const int jb = jt + 16 * wid;
    half8_t a[NS];
    const int jq = jb + col;
#pragma unroll
    for (int s = 0; s < NS; s++) a[s] = load8(Q.row(min(jq, NQ - 1), qh, D) + 8 * rg + 32 * s, jq < NQ);
    float m[4], l[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
      m[t] = -INFINITY;
      l[t] = 0.0f;
    }
    // keys the tile's last query sees (workgroup-uniform)
    const int kend = probe ? N : min(N, jt + kTile);
    Tile<D> tl;
    tl.fetch(tid, 0, N, krow);
    for (int kt = 0; kt < kend; kt += kTile) {
      __syncthreads();  // the previous tile's reads are done
      tl.put(tid, ks);
      __syncthreads();
      if (kt + kTile < kend) tl.fetch(tid, kt + kTile, N, krow);  // in flight during the products
      if (!probe && kt > jb + 15) continue;  // (wave-uniform) every key after this wave's queries
      // a full tile (every key in range and before every query of the wave)
      // needs no mask; the rows' maxima move only when a tile exceeds them
      const bool full = kt + kTile <= N && (probe || kt + kTile - 1 <= jb);
      if (full) {
        float4_t acc[4];
#pragma unroll
        for (int kb = 0; kb < 4; kb++) {
          acc[kb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < NS; s++) acc[kb] = mfma32(a[s], lds8<D>(ks, 16 * kb + col, s, rg), acc[kb]);
        }
#pragma unroll
        for (int t = 0; t < 4; t++) {
          const float bm = fmaxf(fmaxf(acc[0][t], acc[1][t]), fmaxf(acc[2][t], acc[3][t])) * scale_log2;
          if (bm > m[t]) {
            l[t] *= __builtin_amdgcn_exp2f(m[t] - bm);  // (0 from an empty row: m = -inf)
            m[t] = bm;
          }
          float sacc = l[t];
#pragma unroll
          for (int kb = 0; kb < 4; kb++) sacc += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[kb][t], scale_log2, -m[t]));
          l[t] = sacc;
        }
        continue;
      }
      float x[4][4];  // [key block][row]
#pragma unroll
      for (int kb = 0; kb < 4; kb++) {
        const int ik = kt + 16 * kb + col;
        float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (kt + 16 * kb < kend && (probe || kt + 16 * kb <= jb + 15)) {
#pragma unroll
          for (int s = 0; s < NS; s++) acc = mfma32(a[s], lds8<D>(ks, 16 * kb + col, s, rg), acc);
        }
#pragma unroll
        for (int t = 0; t < 4; t++) {
          const int j = jb + 4 * rg + t;  // this lane's query rows
          const bool ok = ik < kend && (probe || ik <= j);
          x[kb][t] = ok ? acc[t] * scale_log2 : -INFINITY;
        }
      }
#pragma unroll
      for (int t = 0; t < 4; t++) {
        const float bm = fmaxf(fmaxf(x[0][t], x[1][t]), fmaxf(x[2][t], x[3][t]));
        const float mn = fmaxf(m[t], bm);
        if (mn != -INFINITY) {
          float sacc = l[t] * __builtin_amdgcn_exp2f(m[t] - mn);
#pragma unroll
          for (int kb = 0; kb < 4; kb++) sacc += __builtin_amdgcn_exp2f(x[kb][t] - mn);
          l[t] = sacc;
          m[t] = mn;
        }
      }
    }
    // merge over the 16 key columns of a row group (lanes of one DPP row)
#pragma unroll
    for (int t = 0; t < 4; t++) {
      const float M = group_reduce<16>(m[t], [](float a_, float b_) { return fmaxf(a_, b_); });
      const float part = M == -INFINITY ? 0.0f : l[t] * __builtin_amdgcn_exp2f(m[t] - M);
      const float L = group_reduce<16>(part, [](float a_, float b_) { return a_ + b_; });
      const int j = jb + 4 * rg + t;
      if (col == 0 && j < NQ)
        stats[(int64_t)qh * nqtot + (probe ? (int64_t)r * nq : c0) + j] =
            L > 0.0f ? -(M + __builtin_amdgcn_logf(L)) : -INFINITY;
    }
  }
}

// scores[h][c0 + i] = mean over the queries that count for key i of the max
// over the group's heads of 2^(x + c).
template <int D>
__global__ __launch_bounds__(64 * kImpWaves) void imp_sum_kernel(int H, int G, int probe, int nq,
                                                                 const int64_t* __restrict__ cu,
                                                                 const uint16_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ k,
                                                                 const float* __restrict__ stats, int64_t nqtot,
                                                                 int64_t total, float scale_log2,
                                                                 float* __restrict__ scores) {
  constexpr int NS = D / 32;
  __shared__ __align__(16) uint16_t qs[kTile * Tile<D>::LR];
  __shared__ __align__(16) float cs[kTile];
  const int r = blockIdx.z, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int col = lane & 15, rg = lane >> 4;
  const int64_t c0 = cu[r];
  const int N = (int)(cu[r + 1] - c0);
  const int NQ = probe ? nq : N;
  if (N <= 0 || c0 < 0 || c0 + N > total) return;  // (a malformed cu_seqlens entry: nothing read)
  const QRows Q{q, probe ? (int64_t)r * nq : c0, (int64_t)H * G * D};
  const int64_t sbase = probe ? (int64_t)r * nq : c0;
  for (int it = blockIdx.x * kTile; it < N; it += gridDim.x * kTile) {
    // B operand: key ib + col, dims 8 rg + 32 s (kept for the whole walk)
    const int ib = it + 16 * wid;
    const int ik = ib + col;
    half8_t kb[NS];
#pragma unroll
    for (int s = 0; s < NS; s++) kb[s] = load8(k + ((c0 + min(ik, N - 1)) * H + h) * D + 8 * rg + 32 * s, ik < N);
    float sum = 0.0f;
    // query tiles that can count for this tile's keys (causal: j > i >= it),
    // and per tile the group's heads; the (tile, head) pairs in that order,
    // the next pair's rows and references in flight during each pair's products
    const int jt0 = probe ? 0 : it;
    Tile<D> tl;
    float cpre = 0.0f;
    auto fetch = [&](int jt, int g) {
      const int qh = h * G + g;
      tl.fetch(tid, jt, NQ, [&](int x) { return Q.row(x, qh, D); });
      if (tid < kTile) cpre = stats[(int64_t)qh * nqtot + sbase + min(jt + tid, NQ - 1)];
    };
    if (jt0 < NQ) fetch(jt0, 0);
    for (int jt = jt0; jt < NQ; jt += kTile) {
      // [query block][row]: max over the heads so far of the exponent x + c
      // (2^ is increasing, so the max of the weights is 2^ of this max: one
      // exponential per (query, key) instead of one per head)
      float pm[4][4];
#pragma unroll
      for (int qb = 0; qb < 4; qb++)
#pragma unroll
        for (int t = 0; t < 4; t++) pm[qb][t] = -INFINITY;
      for (int g = 0; g < G; g++) {
        __syncthreads();  // the previous pair's reads are done
        tl.put(tid, qs);
        if (tid < kTile) cs[tid] = cpre;
        __syncthreads();
        if (g + 1 < G) fetch(jt, g + 1);
        else if (jt + kTile < NQ) fetch(jt + kTile, 0);
        if (!probe && jt + kTile - 1 <= ib) continue;  // (wave-uniform) no query after this wave's keys
        // a full tile (every query in range and after every key of the wave,
        // the wave's keys in range) needs no mask
        const bool full = jt + kTile <= NQ && ib + 16 <= N && (probe || jt >= ib + 16);
#pragma unroll
        for (int qb = 0; qb < 4; qb++) {
          if (!probe && jt + 16 * qb + 15 <= ib) continue;  // (wave-uniform)
          float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < NS; s++) acc = mfma32(lds8<D>(qs, 16 * qb + col, s, rg), kb[s], acc);
          const float4_t c4 = *(const float4_t*)(cs + 16 * qb + 4 * rg);  // the lane's four query rows
          if (full) {
#pragma unroll
            for (int t = 0; t < 4; t++) pm[qb][t] = fmaxf(pm[qb][t], __builtin_fmaf(acc[t], scale_log2, c4[t]));
          } else {
#pragma unroll
            for (int t = 0; t < 4; t++) {
              const int j = jt + 16 * qb + 4 * rg + t;
              const bool ok = j < NQ && ik < N && (probe || j > ik);
              pm[qb][t] = fmaxf(pm[qb][t], ok ? __builtin_fmaf(acc[t], scale_log2, c4[t]) : -INFINITY);
            }
          }
        }
      }
      // (2^-inf = 0: masked pairs, and queries whose references are -inf)
#pragma unroll
      for (int qb = 0; qb < 4; qb++)
        sum += (__builtin_amdgcn_exp2f(pm[qb][0]) + __builtin_amdgcn_exp2f(pm[qb][1])) +
               (__builtin_amdgcn_exp2f(pm[qb][2]) + __builtin_amdgcn_exp2f(pm[qb][3]));
    }
    // the four row groups of a key column: lanes col, col + 16, col + 32, col + 48
    sum += lane_xchg_t<4>(sum);
    sum += lane_xchg_t<5>(sum);
    if (rg == 0 && ik < N) {
      const int cnt = probe ? nq : N - 1 - ik;
      scores[(int64_t)h * total + c0 + ik] = cnt > 0 ? sum / (float)cnt : 0.0f;
    }
  }
}

size_t importance_workspace(const Cfg& c, int64_t nqtot) {
  return align_up((size_t)c.H * c.G * (size_t)(nqtot > 0 ? nqtot : 1) * sizeof(float), 256);
}

hipError_t launch_importance(const Cfg& c, int batch, int64_t total, const int64_t* cu, int probe, int nq,
                             const uint16_t* q, const uint16_t* k, float* scores, void* ws, hipStream_t s) {
  if (batch == 0 || total == 0) return hipSuccess;
  const int64_t nqtot = probe ? (int64_t)batch * nq : total;
  float* stats = (float*)ws;
  const float scale_log2 = (1.0f / sqrtf((float)c.d)) * kL2e;
  // blocks of 64 rows per workgroup; lengths up to max_seq_len in one pass
  // (longer ones by the kernels' grid-stride loops)
  const int64_t rows = probe ? nq : (c.S_max < total ? c.S_max : total);
  const unsigned gx = (unsigned)((rows + 16 * kImpWaves - 1) / (16 * kImpWaves));
  const int64_t keys = c.S_max < total ? c.S_max : total;
  const unsigned kx = (unsigned)((keys + 16 * kImpWaves - 1) / (16 * kImpWaves));
  const dim3 block(64 * kImpWaves);
  if (c.d == 128) {
    imp_stats_kernel<128><<<dim3(gx, c.H * c.G, batch), block, 0, s>>>(c.H, c.G, probe, nq, cu, q, k, stats, nqtot,
                                                                      total, scale_log2);
    imp_sum_kernel<128><<<dim3(kx, c.H, batch), block, 0, s>>>(c.H, c.G, probe, nq, cu, q, k, stats, nqtot, total,
                                                               scale_log2, scores);
  } else {
    imp_stats_kernel<64><<<dim3(gx, c.H * c.G, batch), block, 0, s>>>(c.H, c.G, probe, nq, cu, q, k, stats, nqtot,
                                                                     total, scale_log2);
    imp_sum_kernel<64><<<dim3(kx, c.H, batch), block, 0, s>>>(c.H, c.G, probe, nq, cu, q, k, stats, nqtot, total,
                                                              scale_log2, scores);
  }
  return hipGetLastError();
}

}  // namespace dkv
