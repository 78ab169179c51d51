// Device helpers shared by the window-mode and token-mode kernels of the qkv
// library (gfx950): operand types, matrix-core wrappers, the exact unpack of
// 2-bit codes, cross-lane reductions and the online-softmax block update.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "qkv_internal.h"

namespace qkv {

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ inline floatx4 mfma_bf16_k32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline floatx4 mfma_f16_k32(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline floatx4 mfma_bf16_k16(short4v a, short4v b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ inline floatx4 mfma_f16_k16(half4 a, half4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// 2-bit codes to exact fp16 operands.  A code dword is first masked to
// 0x33333333 (directly, or after a shift by 2): every byte then holds two
// nibbles 00cc, which are the e2m1 (FP4) values cc/2, and the scaled FP4
// conversion with scale 2 turns byte b into the fp16 pair (low nibble, high
// nibble) = two codes, exactly.  The slot placement of the ledger
// (kcode_slot / vcode_slot) puts the codes an operand needs in these pairs.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
template <int B>
__device__ __forceinline__ half2v fp4_pair(uint32_t m) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, B);
}
__device__ __forceinline__ half2v fp4_pair_sel(uint32_t m, int b) {   // b is a constant after unrolling
  switch (b & 3) {
    case 0: return fp4_pair<0>(m);
    case 1: return fp4_pair<1>(m);
    case 2: return fp4_pair<2>(m);
    default: return fp4_pair<3>(m);
  }
}
__device__ __forceinline__ uint32_t code_half(uint32_t x, int odd) {   // slots 4k+odd, 4k+odd+2 of each byte
  return (odd ? (x >> 2) : x) & 0x33333333u;
}
// 4-bit codes to exact fp16 operands: a code dword is masked to 0x0F0F0F0F
// (directly, or after a shift by 4), so every byte is 0000cccc, which as an
// E4M3 FP8 value is cccc * 2^-9 (the subnormal and first normal binade are
// one linear range); the scaled FP8 conversion with scale 2^9 turns bytes
// (2w, 2w+1) into the fp16 pair (cccc, cccc) exactly.
template <bool W>
__device__ __forceinline__ half2v fp8_pair(uint32_t m) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m, 512.0f, W);
}
// the 8 codes of one 4-bit code dword whose code e sits at nibble 2e (e < 4)
// or 2(e-4)+1 (e >= 4), in order e = 0..7
__device__ __forceinline__ half8 codes8_int4(uint32_t x) {
  const uint32_t m0 = x & 0x0F0F0F0Fu, m1 = (x >> 4) & 0x0F0F0F0Fu;
  const half4 lo = __builtin_shufflevector(fp8_pair<false>(m0), fp8_pair<true>(m0), 0, 1, 2, 3);
  const half4 hi = __builtin_shufflevector(fp8_pair<false>(m1), fp8_pair<true>(m1), 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// the 8 codes of a masked dword (bytes 0..3) as one half8 operand
__device__ __forceinline__ half8 codes8(uint32_t m) {
  const half4 lo = __builtin_shufflevector(fp4_pair<0>(m), fp4_pair<1>(m), 0, 1, 2, 3);
  const half4 hi = __builtin_shufflevector(fp4_pair<2>(m), fp4_pair<3>(m), 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ inline float neg_inf() { return -__builtin_inff(); }

// float32 rounding of a double that a following float16 conversion must see:
// without the barrier the compiler folds double -> float -> half into one
// double -> half rounding, which differs from the two-step rounding whenever
// the float32 value is a float16 tie
__device__ __forceinline__ float f64_to_f32_kept(double x) {
  float f = (float)x;
  asm volatile("" : "+v"(f));
  return f;
}

// Rotary embedding of one channel pair (x_i, x_{i+d/2}) by a table entry
// (cos, sin): float64 products of the float32 operands (exact), one rounding
// of each difference or sum, then float32.
__device__ __forceinline__ void rope_pair(float lo, float hi, float c, float s, float &rlo, float &rhi) {
  const double l = lo, h = hi, cd = c, sd = s;
  rlo = f64_to_f32_kept(l * cd - h * sd);
  rhi = f64_to_f32_kept(h * cd + l * sd);
}

// Streaming loads of cache tiles: read once per decode step, so they are
// issued nontemporal (they do not displace reused lines in the caches, and
// HBM read throughput is measurably higher than with ordinary loads).
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream16(const void *p) {
  const u32x4v v = __builtin_nontemporal_load((const u32x4v *)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ u32x4v ld_stream16v(const void *p) { return __builtin_nontemporal_load((const u32x4v *)p); }
__device__ __forceinline__ uint2 ld_stream8(const void *p) {
  const u32x2v v = __builtin_nontemporal_load((const u32x2v *)p);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ld_stream4(const void *p) {
  return __builtin_nontemporal_load((const uint32_t *)p);
}

// uniform quantizer of one value (see the codec definition): code of x in a
// group with float16 step s16 and zero z16
__device__ inline uint32_t quant_code(float x, half_t s16, half_t z16, float levels) {
  float s = (float)s16;
  if (s == 0.0f) return 0u;
  float r = (x - (float)z16) / s;
  r = rintf(r);
  r = fminf(fmaxf(r, 0.0f), levels);
  return (uint32_t)r;
}

template <int D>
struct WaveState {
  floatx4 acc[D / 16];   // output rows (head, limb) x columns of each 16-channel tile
  floatx4 zacc;          // value-zero term per (row, channel group) of quantized tiles
  float m;               // running max of this lane's column (log2 units)
  float l;               // partial sum of probabilities over this lane's tokens
};

// order a wave's LDS writes before its own later LDS reads (no cross-wave sharing)
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// reductions over lane pairs (l, l^16) and (l, l^32) with the row-swap
// permutes of gfx950 (VALU, no LDS traffic); both lanes get identical bits
__device__ __forceinline__ float sum_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// s + (s of the lane 8 columns away): folds the low-limb column 8+h into
// column h and vice versa (a row rotation by 8, so both get the same sum)
__device__ __forceinline__ float fold8(float x) {
  // row_ror:8 reads inside the row for every lane, so bound_ctrl changes
  // nothing; with it the move folds into the add (one DPP add)
  const float y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, true));
  return x + y;
}

// Four per-lane values a, b, c, d -> lane group g (lanes 16g .. 16g+15) gets
// the sum of the g-th value over the four lane groups of its column
// (a reduce-scatter: three row-swap permutes and three adds)
__device__ __forceinline__ float reduce_scatter4(float a, float b, float c, float d) {
  // lanes 0-31 keep a (b) summed with lanes 32-63; lanes 32-63 keep c (d)
  const auto r1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(c), false, false);
  const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(b), __float_as_uint(d), false, false);
  const float u = __uint_as_float(r1[0]) + __uint_as_float(r1[1]);
  const float v = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
  // within each half: lanes of the lower 16 keep u, the upper 16 keep v
  const auto r3 = __builtin_amdgcn_permlane16_swap(__float_as_uint(u), __float_as_uint(v), false, false);
  return __uint_as_float(r3[0]) + __uint_as_float(r3[1]);
}

// Online-softmax update for NT 16-token tiles of log2-domain logits x in C
// layout (empty rows hold -inf): writes the probabilities p and each lane's
// per-tile sums ts (over its own 4 rows), and rescales the running state when
// the running max grows.
template <int D, int NT>
__device__ inline void softmax_rows(WaveState<D> &ws, const float (*x)[4], float (*p)[4], float *ts) {
  float mx = neg_inf();
#pragma unroll
  for (int t = 0; t < NT; ++t) mx = fmaxf(mx, fmaxf(fmaxf(x[t][0], x[t][1]), fmaxf(x[t][2], x[t][3])));
  mx = max_x16(mx);
  mx = max_x32(mx);
  const float m_new = fmaxf(ws.m, mx);
  const bool grow = m_new > ws.m;
  if (__any(grow)) {
    const float alpha = grow ? __builtin_amdgcn_exp2f(ws.m - m_new) : 1.0f;
    ws.l *= alpha;
    const int lq = (int)(__lane_id() >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ar = __shfl(alpha, 4 * lq + i);
#pragma unroll
      for (int ct = 0; ct < D / 16; ++ct) ws.acc[ct][i] *= ar;
      ws.zacc[i] *= ar;
    }
    ws.m = m_new;
  }
  float lsum = 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[t][i] = __builtin_amdgcn_exp2f(x[t][i] - ws.m);
    ts[t] = (p[t][0] + p[t][1]) + (p[t][2] + p[t][3]);
    lsum += ts[t];
  }
  ws.l += lsum;
}

// online-softmax update for a block of NT 16-token tiles (scores in C layout;
// rows lo[t] <= r < hi[t] of tile t are valid); writes probabilities p[t][i]
// and each tile's probability sum ts[t] (summed over the tile's 16 tokens) and
// rescales the running state when the running max grows.
template <int D, int NT>
__device__ inline void softmax_block(WaveState<D> &ws, const floatx4 *s, float sc, const int *lo, const int *hi,
                                     int lq, float (*p)[4], float *ts) {
  float x[NT][4];
  float mx = neg_inf();
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * lq + i;
      x[t][i] = (row >= lo[t] && row < hi[t]) ? s[t][i] * sc : neg_inf();
      mx = fmaxf(mx, x[t][i]);
    }
  mx = max_x16(mx);
  mx = max_x32(mx);
  const float m_new = fmaxf(ws.m, mx);
  const bool grow = m_new > ws.m;
  if (__any(grow)) {
    const float alpha = grow ? __builtin_amdgcn_exp2f(ws.m - m_new) : 1.0f;   // exp2(-inf) = 0 on the first block
    ws.l *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ar = __shfl(alpha, 4 * lq + i);   // factor of output row 4*lq+i
#pragma unroll
      for (int ct = 0; ct < D / 16; ++ct) ws.acc[ct][i] *= ar;
      ws.zacc[i] *= ar;
    }
    ws.m = m_new;
  }
  float lsum = 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    ts[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[t][i] = __builtin_amdgcn_exp2f(x[t][i] - ws.m);
      ts[t] += p[t][i];
    }
    lsum += ts[t];
  }
  ws.l += lsum;
#pragma unroll
  for (int t = 0; t < NT; ++t) ts[t] = sum_x32(sum_x16(ts[t]));
}

// fp16 limbs.  opaque_neg1() is -1.0 that the compiler cannot see, so that
// lo_limb's fma(hi, -1, x) stays one mixed-precision FMA with an fp16
// result (v_fma_mixlo_f16) instead of being folded into a conversion of hi
// and a subtraction; x - hi is exact in float32 when hi is x rounded to
// fp16, so the result is that remainder rounded once.
__device__ __forceinline__ float opaque_neg1() {
  float v = -1.0f;
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ half_t lo_limb(half_t hi, float x, float neg1) {
  return (half_t)__builtin_fmaf((float)hi, neg1, x);
}
// two floats cut toward zero to fp16 (one packed conversion)
__device__ __forceinline__ half2v rtz_pair(float a, float b) {
  return __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// Minimum and maximum that return NaN when either operand is NaN, as a
// float reduction over the values does: a quantizer's group that holds a NaN
// then gets a NaN step, which latches the range error, instead of the NaN
// being skipped and coded as if it were in range.
__device__ __forceinline__ float min_nan(float a, float b) { return a != a ? a : (b != b ? b : fminf(a, b)); }
__device__ __forceinline__ float max_nan(float a, float b) { return a != a ? a : (b != b ? b : fmaxf(a, b)); }

// Outputs of one (sequence, KV head) from its split partials: thread t folds
// outputs t, t + 256, ... (G*D of them, [head][channel]) with the LSE rule in
// split order; the loads of two outputs and CH splits go out together.
template <int G, int CH>
__device__ inline void merge_outputs(const float2 *ml, const float *po, int S, int D, float *out) {
  constexpr int PT = 2;
  const int n = G * D;
  for (int it0 = threadIdx.x; it0 < n; it0 += PT * blockDim.x) {
    float m[PT], l[PT], o[PT];
    int hh[PT], c[PT];
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int it = min(it0 + p * (int)blockDim.x, n - 1);
      hh[p] = it / D;
      c[p] = it % D;
      m[p] = neg_inf();
      l[p] = 0.0f;
      o[p] = 0.0f;
    }
    for (int s0 = 0; s0 < S; s0 += CH) {
      float2 mls[PT][CH];
      float os[PT][CH];
#pragma unroll
      for (int p = 0; p < PT; ++p)
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          const int sp = min(s0 + k, S - 1);
          mls[p][k] = ml[sp * G + hh[p]];
          os[p][k] = po[(size_t)(sp * G + hh[p]) * D + c[p]];
        }
#pragma unroll
      for (int p = 0; p < PT; ++p)
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          if (s0 + k >= S || mls[p][k].x == neg_inf()) continue;
          const float mn = fmaxf(m[p], mls[p][k].x);
          const float a = m[p] == neg_inf() ? 0.0f : exp2f(m[p] - mn), w = exp2f(mls[p][k].x - mn);
          l[p] = l[p] * a + mls[p][k].y * w;
          o[p] = o[p] * a + os[p][k] * w;
          m[p] = mn;
        }
    }
#pragma unroll
    for (int p = 0; p < PT; ++p)
      if (it0 + p * (int)blockDim.x < n) out[hh[p] * D + c[p]] = o[p] / l[p];
  }
}

}  // namespace qkv
