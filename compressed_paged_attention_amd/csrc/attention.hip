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
// MI355X mapping.  One workgroup = (unit, split) with 4 waves; wave w takes
// the split's pages w, w+4, ...  Per page a wave uses 16x16x16 fp16 matrix
// instructions:
//   S (16 tokens x 16 heads)   = codes_K (16 x d) * Q^T (d x 16)
//   O^T (16 dims x 16 heads)  += codes_V^T (16 x 16 tokens) * P'^T (16 x 16)
// with P' = softmax weight * s_v.  The dequantization is algebraic:
//   q . k^ = s_k (q . c_k) + z_k sum(q)
//   sum_t p_t v^_t = sum_t (p_t s_v,t) c_t + (sum_t p_t z_v,t) * 1
// so only integer codes (exact in fp16) enter the matrix units.  P' is split
// into an fp16 head and an fp16 tail (two instructions) so the PV product
// keeps ~22 bits.  The S accumulator layout equals the P'^T operand layout,
// so softmax needs no data movement between the two products.  The codes of
// K are read token-major (lane: token l%16, a quarter of d); the codes of V
// are stored in 64 lane chunks so each lane issues one 16-byte load per page.
// The online softmax is fp32 in base 2.  Splits write (m, l, O) partials; the
// last workgroup of a unit (device-scope fences + one atomic counter) merges
// them and resets the counter.
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

namespace dkv {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ inline float4_t mfma16(half4_t a, half4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// two packed fp16 values (1024 + x) -> exact x
__device__ inline half2_t unbias(uint32_t w) {
  half2_t h = __builtin_bit_cast(half2_t, w);
  const half2_t k = {(_Float16)1024.0f, (_Float16)1024.0f};
  return h - k;
}
__device__ inline half4_t cat(half2_t a, half2_t b) { return half4_t{a.x, a.y, b.x, b.y}; }

// 4 u8 codes of one dword -> 4 fp16 values in order
__device__ inline half4_t u8x4_to_h4(uint32_t w) {
  const uint32_t a = (w & 0x000000FFu) | ((w & 0x0000FF00u) << 8) | 0x64006400u;
  const uint32_t b = ((w & 0x00FF0000u) >> 16) | ((w & 0xFF000000u) >> 8) | 0x64006400u;
  return cat(unbias(a), unbias(b));
}
// fields at bit s and s+16 of a dword, `mask` = field mask replicated at 0/16
__device__ inline half2_t pair(uint32_t w, int s, uint32_t mask) {
  return unbias(((w >> s) & mask) | 0x64006400u);
}

constexpr float kLog2e = 1.4426950408889634f;

struct Split {
  int S;
};

size_t attn_parts_offset(int64_t U) { return align_up((size_t)U * sizeof(int32_t), 256); }

int attn_splits(const Cfg& c, int batch) {
  const int64_t U = (int64_t)batch * c.H;
  if (U <= 0) return 1;
  int64_t S = (2048 + U - 1) / U;
  int64_t cap = c.L / 8;
  if (cap < 1) cap = 1;
  if (S > cap) S = cap;
  if (S > 64) S = 64;
  if (S < 1) S = 1;
  return (int)S;
}

struct AttnWs {
  int32_t* counters;  // [U] zero between calls
  float* part;        // [U][S][G][D + 2]
  float* ml;          // [U][G][2] final (max, sum) for the score update
  float* logits;      // [U][L][32][G] base-2 logits of every retained slot
};

static AttnWs attn_carve(const Cfg& c, int batch, bool scores, void* ws, size_t* bytes) {
  const int64_t U = (int64_t)batch * c.H;
  const int S = attn_splits(c, batch);
  uint8_t* b = (uint8_t*)ws;
  size_t off = 0;
  AttnWs w;
  w.counters = (int32_t*)(b + off);
  off = align_up(off + (size_t)U * sizeof(int32_t), 256);
  w.part = (float*)(b + off);
  off = align_up(off + (size_t)U * S * c.G * (c.d + 2) * sizeof(float), 256);
  w.ml = (float*)(b + off);
  off = align_up(off + (size_t)U * c.G * 2 * sizeof(float), 256);
  w.logits = (float*)(b + off);
  if (scores) off = align_up(off + (size_t)U * c.L * 32 * c.G * sizeof(float), 256);
  if (bytes) *bytes = off;
  return w;
}

size_t attn_workspace(const Cfg& c, int batch, bool scores) {
  size_t n = 0;
  attn_carve(c, batch, scores, nullptr, &n);
  return n;
}

// Unit validity, identical in every workgroup of the unit.
__device__ inline bool unit_ok(int nh, int nl, int ph, int pl, int L, int64_t P, const int32_t* row) {
  bool ok = nh >= 0 && nl >= 0 && ph == (int)cdiv(nh, kHiTokens) && pl == (int)cdiv(nl, kLoTokens) &&
            ph + pl <= L;
  int bad = 0;
  if (ok) {
    for (int j = threadIdx.x; j < ph + pl; j += blockDim.x) {
      const int32_t id = j < ph ? row[j] : row[L - 1 - (j - ph)];
      bad |= (id < 0 || id >= P);
    }
  }
  return __syncthreads_or(bad) == 0 && ok;
}

template <int D, bool SAVE>
__global__ __launch_bounds__(256) void attn_kernel(int H, int G, int L, int S, int64_t P, int page_bytes,
                                                   float scale_log2, const uint16_t* __restrict__ q,
                                                   const int32_t* __restrict__ table,
                                                   const int32_t* __restrict__ state,
                                                   const int32_t* __restrict__ seq_len,
                                                   const uint8_t* __restrict__ pages, float* __restrict__ out,
                                                   int32_t* counters, float* part, float* ml,
                                                   float* __restrict__ logits, uint32_t* status) {
  constexpr int NB = D / 16;  // 16-dim blocks (K-steps of QK, N-blocks of PV)
  constexpr int QD = D / 4;   // dims per lane group
  const int split = blockIdx.x;
  const int64_t u = blockIdx.y;
  const int b = (int)(u / H), h = (int)(u % H);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int i = lane & 15, qg = lane >> 4;
  const int32_t* row = table + u * L;
  const int32_t* s4 = state + 4 * u;
  const int nh = s4[0], nl = s4[1], ph = s4[2], pl = s4[3];
  const int N = seq_len[b];
  const bool ok = unit_ok(nh, nl, ph, pl, L, P, row);
  float* orow = out + ((int64_t)b * H * G + (int64_t)h * G) * D;
  if (N <= 0 || !ok || nh + nl == 0) {
    if (split == 0) {
      for (int x = tid; x < G * D; x += blockDim.x) orow[x] = 0.0f;
      if (SAVE)
        for (int x = tid; x < G; x += blockDim.x) {
          ml[(u * G + x) * 2 + 0] = -INFINITY;
          ml[(u * G + x) * 2 + 1] = 0.0f;
        }
      if (N > 0 && !ok && tid == 0) atomicOr(status, kStBadState);
    }
    return;
  }

  // ---- Q operands: lane (i, qg) holds head i, dims qg*QD .. qg*QD+QD-1 ----
  half4_t qhi[NB], qlo[NB];
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
    for (int kb = 0; kb < NB; kb++) {
      qhi[kb] = half4_t{H16(4 * kb), H16(4 * kb + 1), H16(4 * kb + 2), H16(4 * kb + 3)};
      const int w = kb >> 1, v = kb & 1, o = 8 * w + 2 * v;
      qlo[kb] = half4_t{H16(o), H16(o + 4), H16(o + 1), H16(o + 5)};
    }
    sumq += __shfl_xor(sumq, 16, 64);
    sumq += __shfl_xor(sumq, 32, 64);
  }

  // ---- page range of this split: hi pages first, then lo pages ----
  const int TPg = ph + pl;
  const int pps = (TPg + S - 1) / S;
  const int p0 = split * pps;
  const int p1 = min(TPg, p0 + pps);
  const Seg sh = tier_seg(D, true), sl = tier_seg(D, false);

  float m = -INFINITY, lsum = 0.0f, zsum = 0.0f;
  float4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; nb++) acc[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  for (int j = p0 + wid; j < p1; j += 4) {
    const bool is_hi = j < ph;
    const int jt = is_hi ? j : j - ph;
    const int tidx = is_hi ? jt : L - 1 - jt;
    const uint8_t* pg = pages + (int64_t)row[tidx] * page_bytes;
    if (is_hi) {
      const int nval = min(kHiTokens, nh - kHiTokens * jt);
      // loads
      uint32_t kw[NB];
      const uint4* kp = (const uint4*)(pg + sh.kc + i * D + qg * QD);
#pragma unroll
      for (int c = 0; c < NB / 4; c++) {
        const uint4 w = kp[c];
        kw[4 * c] = w.x;
        kw[4 * c + 1] = w.y;
        kw[4 * c + 2] = w.z;
        kw[4 * c + 3] = w.w;
      }
      const uint4 kmeta = *(const uint4*)(pg + sh.km + 16 * qg);
      const uint4 vmeta = *(const uint4*)(pg + sh.vm + 16 * qg);
      uint32_t vw[D / 32];
      if constexpr (D == 128) {
        const uint4 w = *(const uint4*)(pg + sh.vc + lane * 16);
        vw[0] = w.x;
        vw[1] = w.y;
        vw[2] = w.z;
        vw[3] = w.w;
      } else {
        const uint2 w = *(const uint2*)(pg + sh.vc + lane * 8);
        vw[0] = w.x;
        vw[1] = w.y;
      }
      // S = codes_K * Q^T
      float4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < NB; kb++) s = mfma16(u8x4_to_h4(kw[kb]), qhi[kb], s);
      const uint32_t km[4] = {kmeta.x, kmeta.y, kmeta.z, kmeta.w};
      const uint32_t vm[4] = {vmeta.x, vmeta.y, vmeta.z, vmeta.w};
      float x[4];
      float pm = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const float ks = h2f((uint16_t)km[r]), kz = h2f((uint16_t)(km[r] >> 16));
        x[r] = (ks * s[r] + kz * sumq) * scale_log2;
        if (4 * qg + r >= nval) x[r] = -INFINITY;
        pm = fmaxf(pm, x[r]);
      }
      if (SAVE && i < G) {
        float* lg = logits + (((int64_t)u * L + tidx) * 32 + 4 * qg) * G + i;
#pragma unroll
        for (int r = 0; r < 4; r++) lg[r * G] = x[r];
      }
      pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
      pm = fmaxf(pm, __shfl_xor(pm, 32, 64));
      const float mn = fmaxf(m, pm);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      float p[4], ps = 0.0f, pz = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        p[r] = __builtin_amdgcn_exp2f(x[r] - mn);
        ps += p[r];
        pz += p[r] * h2f((uint16_t)(vm[r] >> 16));
      }
      lsum = lsum * alpha + ps;
      zsum = zsum * alpha + pz;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int nb = 0; nb < NB; nb++) acc[nb] *= alpha;
      }
      m = mn;
      _Float16 ph16[4], pl16[4];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const float pp = p[r] * h2f((uint16_t)vm[r]);
        ph16[r] = (_Float16)pp;
        pl16[r] = (_Float16)(pp - (float)ph16[r]);
      }
      const half4_t bh = {ph16[0], ph16[1], ph16[2], ph16[3]};
      const half4_t bl = {pl16[0], pl16[1], pl16[2], pl16[3]};
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
        const uint32_t w = vw[nb >> 1];
        const int s0 = 8 * (nb & 1);
        const half4_t a = cat(pair(w, s0, 0x000F000Fu), pair(w, s0 + 4, 0x000F000Fu));
        acc[nb] = mfma16(a, bh, acc[nb]);
        acc[nb] = mfma16(a, bl, acc[nb]);
      }
    } else {
      const int nval = min(kLoTokens, nl - kLoTokens * jt);
      uint32_t kw[2][NB / 2];
#pragma unroll
      for (int mb = 0; mb < 2; mb++) {
        if constexpr (D == 128) {
          const uint4 w = *(const uint4*)(pg + sl.kc + (i + 16 * mb) * (D / 2) + qg * (QD / 2));
          kw[mb][0] = w.x;
          kw[mb][1] = w.y;
          kw[mb][2] = w.z;
          kw[mb][3] = w.w;
        } else {
          const uint2 w = *(const uint2*)(pg + sl.kc + (i + 16 * mb) * (D / 2) + qg * (QD / 2));
          kw[mb][0] = w.x;
          kw[mb][1] = w.y;
        }
      }
      uint4 kmeta[2], vmeta[2];
#pragma unroll
      for (int mb = 0; mb < 2; mb++) {
        kmeta[mb] = *(const uint4*)(pg + sl.km + 64 * mb + 16 * qg);
        vmeta[mb] = *(const uint4*)(pg + sl.vm + 64 * mb + 16 * qg);
      }
      uint32_t vw[D / 32];
      if constexpr (D == 128) {
        const uint4 w = *(const uint4*)(pg + sl.vc + lane * 16);
        vw[0] = w.x;
        vw[1] = w.y;
        vw[2] = w.z;
        vw[3] = w.w;
      } else {
        const uint2 w = *(const uint2*)(pg + sl.vc + lane * 8);
        vw[0] = w.x;
        vw[1] = w.y;
      }
      float x[2][4];
      float pm = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; mb++) {
        float4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < NB; kb++) {
          const uint32_t w = kw[mb][kb >> 1];
          const int s0 = 8 * (kb & 1);
          s = mfma16(cat(pair(w, s0, 0x000F000Fu), pair(w, s0 + 4, 0x000F000Fu)), qlo[kb], s);
        }
        const uint32_t km[4] = {kmeta[mb].x, kmeta[mb].y, kmeta[mb].z, kmeta[mb].w};
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const float ks = h2f((uint16_t)km[r]), kz = h2f((uint16_t)(km[r] >> 16));
          float xv = (ks * s[r] + kz * sumq) * scale_log2;
          if (16 * mb + 4 * qg + r >= nval) xv = -INFINITY;
          x[mb][r] = xv;
          pm = fmaxf(pm, xv);
        }
      }
      if (SAVE && i < G) {
#pragma unroll
        for (int mb = 0; mb < 2; mb++) {
          float* lg = logits + (((int64_t)u * L + tidx) * 32 + 16 * mb + 4 * qg) * G + i;
#pragma unroll
          for (int r = 0; r < 4; r++) lg[r * G] = x[mb][r];
        }
      }
      pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
      pm = fmaxf(pm, __shfl_xor(pm, 32, 64));
      const float mn = fmaxf(m, pm);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      float p[2][4], ps = 0.0f, pz = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; mb++) {
        const uint32_t vm[4] = {vmeta[mb].x, vmeta[mb].y, vmeta[mb].z, vmeta[mb].w};
#pragma unroll
        for (int r = 0; r < 4; r++) {
          p[mb][r] = __builtin_amdgcn_exp2f(x[mb][r] - mn);
          ps += p[mb][r];
          pz += p[mb][r] * h2f((uint16_t)(vm[r] >> 16));
        }
      }
      lsum = lsum * alpha + ps;
      zsum = zsum * alpha + pz;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int nb = 0; nb < NB; nb++) acc[nb] *= alpha;
      }
      m = mn;
#pragma unroll
      for (int ks = 0; ks < 2; ks++) {
        const uint32_t vm[4] = {vmeta[ks].x, vmeta[ks].y, vmeta[ks].z, vmeta[ks].w};
        _Float16 ph16[4], pl16[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const float pp = p[ks][r] * h2f((uint16_t)vm[r]);
          ph16[r] = (_Float16)pp;
          pl16[r] = (_Float16)(pp - (float)ph16[r]);
        }
        const half4_t bh = {ph16[0], ph16[1], ph16[2], ph16[3]};
        const half4_t bl = {pl16[0], pl16[1], pl16[2], pl16[3]};
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
          const int M = 2 * nb + ks;
          const int P0 = 2 * M, P1 = 2 * M + 1;
          const half4_t a = cat(pair(vw[P0 >> 3], 2 * (P0 & 7), 0x00030003u),
                                pair(vw[P1 >> 3], 2 * (P1 & 7), 0x00030003u));
          acc[nb] = mfma16(a, bh, acc[nb]);
          acc[nb] = mfma16(a, bl, acc[nb]);
        }
      }
    }
  }

  // ---- combine the 4 waves of the workgroup ----
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  zsum += __shfl_xor(zsum, 16, 64);
  zsum += __shfl_xor(zsum, 32, 64);
  __shared__ float wm[4][16], wl[4][16];
  __shared__ float wo[4][16][D + 1];
  if (qg == 0) {
    wm[wid][i] = m;
    wl[wid][i] = lsum;
  }
#pragma unroll
  for (int nb = 0; nb < NB; nb++)
#pragma unroll
    for (int r = 0; r < 4; r++) wo[wid][i][16 * nb + 4 * qg + r] = acc[nb][r] + zsum;
  __syncthreads();
  // per (head, dim) combination; the partial of this workgroup
  float* mypart = part + (((int64_t)u * S + split) * G) * (D + 2);
  for (int x = tid; x < G * D; x += blockDim.x) {
    const int g = x / D, dd = x % D;
    float M = fmaxf(fmaxf(wm[0][g], wm[1][g]), fmaxf(wm[2][g], wm[3][g]));
    float o = 0.0f, l = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; w++) {
        const float f = __builtin_amdgcn_exp2f(wm[w][g] - M);
        o += wo[w][g][dd] * f;
        l += wl[w][g] * f;
      }
    }
    if (S == 1) {
      orow[x] = o / l;
      if (SAVE && dd == 0) {
        ml[(u * G + g) * 2 + 0] = M;
        ml[(u * G + g) * 2 + 1] = l;
      }
    } else {
      mypart[g * (D + 2) + dd] = o;
      if (dd == 0) {
        mypart[g * (D + 2) + D] = M;
        mypart[g * (D + 2) + D + 1] = l;
      }
    }
  }
  if (S == 1) return;

  // ---- the last workgroup of the unit merges the split partials ----
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&counters[u], 1) == S - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* up = part + ((int64_t)u * S * G) * (D + 2);
  for (int x = tid; x < G * D; x += blockDim.x) {
    const int g = x / D, dd = x % D;
    float M = -INFINITY;
    for (int sp = 0; sp < S; sp++) M = fmaxf(M, __builtin_nontemporal_load(&up[(sp * G + g) * (D + 2) + D]));
    float o = 0.0f, l = 0.0f;
    for (int sp = 0; sp < S; sp++) {
      const float* pp = up + (sp * G + g) * (D + 2);
      const float ms = __builtin_nontemporal_load(&pp[D]);
      if (ms == -INFINITY) continue;
      const float f = __builtin_amdgcn_exp2f(ms - M);
      o += __builtin_nontemporal_load(&pp[dd]) * f;
      l += __builtin_nontemporal_load(&pp[D + 1]) * f;
    }
    orow[x] = o / l;
    if (SAVE && dd == 0) {
      ml[(u * G + g) * 2 + 0] = M;
      ml[(u * G + g) * 2 + 1] = l;
    }
  }
  if (tid == 0) counters[u] = 0;
}

// Score update: each retained token other than the query's own adds the max
// over the group's q heads of its softmax weight to its stored sum.
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
  if (N <= 0 || nh + nl == 0) return;
  if (!unit_ok(nh, nl, ph, pl, L, P, row)) return;
  __shared__ float sM[16], sL[16];
  if (tid < G) {
    sM[tid] = ml[(u * G + tid) * 2 + 0];
    sL[tid] = 1.0f / ml[(u * G + tid) * 2 + 1];
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
    uint8_t* pg = pages + (int64_t)row[tidx] * page_bytes;
    const Seg& sg = is_hi ? sh : sl;
    const int32_t pos = *(const int32_t*)(pg + sg.ps + 4 * t);
    if (pos >= N) continue;
    const float* lg = logits + (((int64_t)u * L + tidx) * 32 + t) * G;
    float mx = 0.0f;
    for (int g = 0; g < G; g++) mx = fmaxf(mx, __builtin_amdgcn_exp2f(lg[g] - sM[g]) * sL[g]);
    float* sc = (float*)(pg + sg.sc + 4 * t);
    *sc = *sc + mx;
  }
}

hipError_t launch_attn(const Cfg& c, const Pool& p, int batch, const uint16_t* q, const int32_t* table,
                       const int32_t* state, const int32_t* seq_len, float* out, bool update_scores, void* ws,
                       hipStream_t s) {
  const int64_t U = (int64_t)batch * c.H;
  if (U == 0) return hipSuccess;
  const int S = attn_splits(c, batch);
  AttnWs w = attn_carve(c, batch, update_scores, ws, nullptr);
  const float scale_log2 = (1.0f / sqrtf((float)c.d)) * kLog2e;
  const dim3 grid(S, (unsigned)U), block(256);
#define DKV_ATTN(D, SV)                                                                                   \
  attn_kernel<D, SV><<<grid, block, 0, s>>>(c.H, c.G, c.L, S, p.P, p.page_bytes, scale_log2, q, table, \
                                            state, seq_len, p.pages, out, w.counters, w.part, w.ml,      \
                                            w.logits, p.status)
  if (c.d == 128) {
    if (update_scores) DKV_ATTN(128, true);
    else DKV_ATTN(128, false);
  } else {
    if (update_scores) DKV_ATTN(64, true);
    else DKV_ATTN(64, false);
  }
#undef DKV_ATTN
  if (update_scores) {
    if (c.d == 128)
      score_kernel<128><<<grid, block, 0, s>>>(c.H, c.G, c.L, S, p.P, p.page_bytes, table, state, seq_len, w.ml,
                                               w.logits, p.pages);
    else
      score_kernel<64><<<grid, block, 0, s>>>(c.H, c.G, c.L, S, p.P, p.page_bytes, table, state, seq_len, w.ml,
                                              w.logits, p.pages);
  }
  return hipGetLastError();
}

}  // namespace dkv
