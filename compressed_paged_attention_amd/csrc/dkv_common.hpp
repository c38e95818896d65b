// dkv_common.hpp -- device-side definitions shared by the libdiffkv kernels:
// unified-page layout, the per-vector codec, and wave/block primitives for
// gfx950 (wave64).
//
// Unified page ("Memory management" section of the DiffKV notes: six
// segments -- quantized K, K metadata, quantized V, V metadata, token score,
// position -- with a per-precision token count).  Segment order follows the
// notes; every segment starts on a 16-byte boundary.
//   high tier: 16 tokens, K 8 bit token-major [16][d], V 4 bit
//   low tier : 32 tokens, K 4 bit token-major [32][d/2] (dims 8w..8w+7 in
//              word w, even dims in the low half-word), V 2 bit
//   metadata : one 32-bit word per token, fp16 scale in bits 0-15, fp16 zero
//              in bits 16-31
//   score    : fp32 running sum of received attention; position: int32
// V codes are token-vectorized and cut into 64 lane chunks of d/8 bytes so
// that lane L = i + 16q of a wave reads exactly the operand it feeds to a
// 16x16x16 matrix instruction: chunk L holds dims i + 16 nb of tokens
// 4q..4q+3 (high; low: tokens 16 ks + 4q .. +3).  Inside a chunk, field
// h = r mod 2 of pair P = 2M + r/2 (r = token mod 4; M = nb for high,
// M = 2 nb + ks for low) sits in 32-bit word w at bit b:
//   high: w = P / 4, b = 4 (P mod 4) + 16 h
//   low : w = P / 8, b = 2 (P mod 8) + 16 h
// so one AND/OR with 0x000F000F (0x00030003) after a shift yields a packed
// pair of fp16 operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dkv {

constexpr int kHiTokens = 16;
constexpr int kLoTokens = 32;
constexpr int kTierPrune = 0, kTierLo = 1, kTierHi = 2;
constexpr uint32_t kStExhausted = 1u, kStOverflow = 2u, kStBadState = 4u, kStStale = 8u;
constexpr uint32_t kStAll = 15u;  // every status bit

struct Seg {
  int T, kbits, vbits, kc, km, vc, vm, sc, ps, bytes;
};

__host__ __device__ constexpr int r16(int x) { return (x + 15) & ~15; }

__host__ __device__ constexpr Seg tier_seg(int d, bool hi) {
  const int T = hi ? kHiTokens : kLoTokens;
  const int kb = hi ? 8 : 4, vb = hi ? 4 : 2;
  const int kc = 0;
  const int km = kc + r16(T * d * kb / 8);
  const int vc = km + r16(4 * T);
  const int vm = vc + r16(T * d * vb / 8);
  const int sc = vm + r16(4 * T);
  const int ps = sc + r16(4 * T);
  const int end = ps + r16(4 * T);
  return Seg{T, kb, vb, kc, km, vc, vm, sc, ps, end};
}

__host__ __device__ constexpr int page_bytes_for(int d) {
  return tier_seg(d, true).bytes > tier_seg(d, false).bytes ? tier_seg(d, true).bytes
                                                           : tier_seg(d, false).bytes;
}

// Byte offset (from the page start) and bit shift of V code (tok, j).
__host__ __device__ inline void v_field(int d, bool hi, int tok, int j, int& byte, int& shift) {
  const Seg s = tier_seg(d, hi);
  const int i = j & 15, nb = j >> 4, r = tok & 3, h = r & 1;
  int lane, w, bit;
  if (hi) {
    const int P = 2 * nb + (r >> 1);
    lane = i + 16 * (tok >> 2);
    w = P >> 2;
    bit = 4 * (P & 3) + 16 * h;
  } else {
    const int P = 2 * (2 * nb + (tok >> 4)) + (r >> 1);
    lane = i + 16 * ((tok & 15) >> 2);
    w = P >> 3;
    bit = 2 * (P & 7) + 16 * h;
  }
  byte = s.vc + lane * (d / 8) + 4 * w + (bit >> 3);
  shift = bit & 7;
}

// Byte offset and shift of K code (tok, j).  4-bit: dim 8w+e of a token is
// nibble e/2 + 4(e&1) of the token's word w, so one shift-and-mask yields an
// fp16 pair of consecutive dims.
__host__ __device__ inline void k_field(int d, bool hi, int tok, int j, int& byte, int& shift) {
  if (hi) {
    byte = tok * d + j;
    shift = 0;
  } else {
    const int e = j & 7, n = (e >> 1) + 4 * (e & 1);
    byte = tok * (d / 2) + 4 * (j >> 3) + (n >> 1);
    shift = 4 * (n & 1);
  }
}

// ---------------------------------------------------------------------------
// Tier codec variants ("Results": the bit-split ablation compares K and V
// code widths such as K8V4, K4V8, K4V2, K2V4, K8V2, K4V1).  Widths other
// than the default pair (or the default pair given explicitly) use the plain
// layout: the same six segments and token counts, K and V codes token-major
// and packed from bit 0 -- code (t, j) at bit (t d + j) b of its segment --
// so a width in {1, 2, 4, 8} never splits a code across bytes.
// ---------------------------------------------------------------------------
struct Codec {
  int kb_hi, vb_hi, kb_lo, vb_lo;
};

// The plain layout of T tokens with K and V code widths kb, vb.
__host__ __device__ inline Seg level_seg(int d, int T, int kb, int vb) {
  const int kc = 0;
  const int km = kc + r16(T * d * kb / 8);
  const int vc = km + r16(4 * T);
  const int vm = vc + r16(T * d * vb / 8);
  const int sc = vm + r16(4 * T);
  const int ps = sc + r16(4 * T);
  const int end = ps + r16(4 * T);
  return Seg{T, kb, vb, kc, km, vc, vm, sc, ps, end};
}

__host__ __device__ inline Seg plain_seg(int d, bool hi, const Codec& c) {
  const int T = hi ? kHiTokens : kLoTokens;
  const int kb = hi ? c.kb_hi : c.kb_lo, vb = hi ? c.vb_hi : c.vb_lo;
  const int kc = 0;
  const int km = kc + r16(T * d * kb / 8);
  const int vc = km + r16(4 * T);
  const int vm = vc + r16(T * d * vb / 8);
  const int sc = vm + r16(4 * T);
  const int ps = sc + r16(4 * T);
  const int end = ps + r16(4 * T);
  return Seg{T, kb, vb, kc, km, vc, vm, sc, ps, end};
}

__host__ __device__ inline int plain_page_bytes(int d, const Codec& c) {
  const int a = plain_seg(d, true, c).bytes, b = plain_seg(d, false, c).bytes;
  return a > b ? a : b;
}

// the largest plain page: 8-bit K and V in both tiers
__host__ __device__ constexpr int plain_page_max(int d) { return 32 * d * 2 + 4 * 4 * 32; }

__host__ __device__ inline void plain_field(int seg_off, int d, int bits, int tok, int j, int& byte, int& shift) {
  const int bit = (tok * d + j) * bits;
  byte = seg_off + (bit >> 3);
  shift = bit & 7;
}

// The page layout as seen by the kernels that serve either kind (commit,
// plan, bounds): the default layout above, or the plain layout of a codec.
struct Lay {
  int d;
  bool plain;
  Seg s[2];  // [low, high]
  __host__ __device__ Lay(int d_, bool plain_, const Codec& c) : d(d_), plain(plain_) {
    s[0] = plain_ ? plain_seg(d_, false, c) : tier_seg(d_, false);
    s[1] = plain_ ? plain_seg(d_, true, c) : tier_seg(d_, true);
  }
  __host__ __device__ const Seg& seg(bool hi) const { return s[hi ? 1 : 0]; }
  __host__ __device__ void kf(bool hi, int tok, int j, int& byte, int& shift) const {
    if (plain) plain_field(s[hi ? 1 : 0].kc, d, s[hi ? 1 : 0].kbits, tok, j, byte, shift);
    else k_field(d, hi, tok, j, byte, shift);
  }
  __host__ __device__ void vf(bool hi, int tok, int j, int& byte, int& shift) const {
    if (plain) plain_field(s[hi ? 1 : 0].vc, d, s[hi ? 1 : 0].vbits, tok, j, byte, shift);
    else v_field(d, hi, tok, j, byte, shift);
  }
};

// ---------------------------------------------------------------------------
// fp16 helpers (IEEE binary16, round to nearest even via v_cvt_f16_f32).
// ---------------------------------------------------------------------------
__device__ inline uint16_t f2h_bits(float x) {
  _Float16 h = (_Float16)x;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ inline float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// ---------------------------------------------------------------------------
// Per-vector asymmetric codec ("Background": Q = round((X - z)/s),
// X^ = s Q + z).  z = fp16(min), s = fp16((max - min) / (2^b - 1)); codes use
// the stored fp16 values, IEEE fp32 division and round-half-even, clamped to
// [0, 2^b - 1]; s == 0 gives code 0.  Must match the CPU reference bit for
// bit, so nothing here may be contracted or approximated.
// ---------------------------------------------------------------------------
__device__ inline void codec_params(float mn, float mx, int bits, uint16_t& s16, uint16_t& z16,
                                    float& s, float& z) {
  const float qmax = (float)((1 << bits) - 1);
  const float range = __fsub_rn(mx, mn);
  const float scale = __fdiv_rn(range, qmax);
  s16 = f2h_bits(scale);
  z16 = f2h_bits(mn);
  s = h2f(s16);
  z = h2f(z16);
}

__device__ inline uint32_t codec_code(float x, float s, float z, int bits) {
  if (s == 0.0f) return 0u;
  const float t = __fdiv_rn(__fsub_rn(x, z), s);
  float r = rintf(t);
  const float qmax = (float)((1 << bits) - 1);
  r = fminf(fmaxf(r, 0.0f), qmax);
  return (uint32_t)r;
}

// Dequantized value; the product of an fp16 scale and a code of <= 8 bits is
// exact in fp32, so this is a single rounding.
__device__ inline float dequant(float s, float z, uint32_t code) {
  return __fadd_rn(__fmul_rn(s, (float)code), z);
}

// ---------------------------------------------------------------------------
// wave64 / block primitives
// ---------------------------------------------------------------------------
// Butterfly partner of level LVL across a 64-lane wave, without LDS: levels
// 0-3 by DPP inside rows of 16 lanes (xor 1, xor 2, half-row mirror, row
// mirror), levels 4-5 by row swaps (xor 16, xor 32).  Combining a value with
// its partner at levels 0..5 under an associative, commutative operation
// leaves the reduction of all 64 lanes in every lane.
template <int LVL>
__device__ inline uint32_t lane_xchg(uint32_t v) {
  if constexpr (LVL == 0) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  } else if constexpr (LVL == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  } else if constexpr (LVL == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  } else if constexpr (LVL == 3) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);  // row_mirror
  } else if constexpr (LVL == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}

template <int LVL, typename T>
__device__ inline T lane_xchg_t(T v) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, lane_xchg<LVL>(__builtin_bit_cast(uint32_t, v)));
  } else {
    static_assert(sizeof(T) == 8, "32- or 64-bit values");
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = lane_xchg<LVL>((uint32_t)u), hi = lane_xchg<LVL>((uint32_t)(u >> 32));
    return __builtin_bit_cast(T, lo | (hi << 32));
  }
}

template <typename T, typename Op>
__device__ inline T wave_reduce(T v, Op op) {
  v = op(v, lane_xchg_t<0>(v));
  v = op(v, lane_xchg_t<1>(v));
  v = op(v, lane_xchg_t<2>(v));
  v = op(v, lane_xchg_t<3>(v));
  v = op(v, lane_xchg_t<4>(v));
  v = op(v, lane_xchg_t<5>(v));
  return v;
}

// Reduction inside aligned groups of N lanes (N a power of two <= 64).
template <int N, typename T, typename Op>
__device__ inline T group_reduce(T v, Op op) {
  if constexpr (N > 1) v = op(v, lane_xchg_t<0>(v));
  if constexpr (N > 2) v = op(v, lane_xchg_t<1>(v));
  if constexpr (N > 4) v = op(v, lane_xchg_t<2>(v));
  if constexpr (N > 8) v = op(v, lane_xchg_t<3>(v));
  if constexpr (N > 16) v = op(v, lane_xchg_t<4>(v));
  if constexpr (N > 32) v = op(v, lane_xchg_t<5>(v));
  return v;
}

// Same with a wave-uniform group size n.
template <typename T, typename Op>
__device__ inline T group_reduce(T v, int n, Op op) {
  if (n > 1) v = op(v, lane_xchg_t<0>(v));
  if (n > 2) v = op(v, lane_xchg_t<1>(v));
  if (n > 4) v = op(v, lane_xchg_t<2>(v));
  if (n > 8) v = op(v, lane_xchg_t<3>(v));
  if (n > 16) v = op(v, lane_xchg_t<4>(v));
  if (n > 32) v = op(v, lane_xchg_t<5>(v));
  return v;
}

template <typename T>
__device__ inline T wave_sum(T v) {
  return wave_reduce(v, [](T a, T b) { return a + b; });
}
__device__ inline float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ inline float wave_min(float v) {
  return wave_reduce(v, [](float a, float b) { return fminf(a, b); });
}

// Inclusive scan across a wave (Hillis-Steele over 64 lanes).
template <typename T>
__device__ inline T wave_incl_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive block scan of one value per thread; `lds` holds >= blockDim/64
// elements; returns the exclusive prefix and writes the block total.
template <typename T>
__device__ inline T block_excl_scan(T v, T* lds, T& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  T inc = wave_incl_scan(v);
  if (lane == 63) lds[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    T x = lane < nw ? lds[lane] : T(0);
    T xi = wave_incl_scan(x);
    if (lane < nw) lds[lane] = xi - x;
    if (lane == nw - 1) lds[nw] = xi;
  }
  __syncthreads();
  T res = inc - v + lds[wid];
  total = lds[nw];
  __syncthreads();
  return res;
}

// Exclusive block-wide count of a predicate (ballot + lane mask count per
// wave, then the wave totals); `lds` holds >= blockDim/64 ints.  Returns the
// number of threads below this one with pred set and the block total.
__device__ inline int block_excl_count(bool pred, int* lds, int& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  const uint64_t m = __ballot(pred);
  const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  if (lane == 0) lds[wid] = __popcll(m);
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < nw; w++) {
    const int c = lds[w];
    before += w < wid ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + below;
}

__device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace dkv
