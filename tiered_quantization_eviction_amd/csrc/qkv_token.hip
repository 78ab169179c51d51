// Token-mode kernels of the tiered decode path (gfx950): H2O heavy-hitter
// eviction, where every token is its own unit and scores are kept per
// (sequence, KV head).
//
// H2O notes, sections 1.1-2.1 and the GQA paragraph: append the new token,
// attend over the kept set plus the new token, add each kept token's weight
// (summed over the query heads that share the KV head) to its score, keep the
// newest B_r tokens and the sinks, and evict from the older tokens the
// lowest-scored ones so that B_h heavy hitters remain (one per step once the
// budget is reached; the whole surplus when the scored prompt is trimmed).
//
// Kept older tokens live in compact tiles gathered at each routing call; the
// sinks and the tokens not yet ranked are read from the position pages.  The
// attention kernel streams [sink tile][compact tiles][recent position tiles]
// with the same 16x16x32 bf16 matrix-core tiling as the window mode, and emits
// per token slot the head's probability relative to the running maximum; the
// merge kernel normalizes those with the global (max, sum) of each head and
// adds them into the per-token scores in a fixed order (no atomics).
#include "qkv_device.h"

namespace qkv {

namespace {

constexpr size_t TOK_ALIGN = 256;
inline size_t tok_align(size_t x) { return (x + TOK_ALIGN - 1) / TOK_ALIGN * TOK_ALIGN; }

}  // namespace

size_t tok_carve(const TokGeom &g, char *base, TokState &st) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *p = base ? base + off : nullptr;
    off = tok_align(off + bytes);
    return (void *)p;
  };
  const size_t BH = (size_t)g.B * g.Hkv;
  const size_t tile_elems = (size_t)2 * TS * g.d;
  st.pages = (uint16_t *)take(BH * g.NPT * tile_elems * 2);
  st.cpages = (uint16_t *)take(BH * g.NCT * tile_elems * 2);
  st.cpos = (int32_t *)take(BH * g.NCT * TS * 4);
  st.tier = (uint8_t *)take(BH * g.T);
  st.score = (float *)take(BH * g.T * 4);
  st.part_o = (float *)take(BH * g.n_splits * g.G * g.d * 4);
  st.part_ml = (float *)take(BH * g.n_splits * g.G * 2 * 4);
  st.mrho = (float *)take(BH * (g.TILES + 1) * g.G * TS * 4);
  st.mref = (float *)take(BH * (g.TILES + 1) * g.G * 4);
  st.scratch_out = (float *)take((size_t)g.B * g.Hq * g.d * 4);
  st.status = (int32_t *)take(16);
  return off;
}

// ---------------------------------------------------------------------------
// append: new tokens into the position pages
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void tok_append_kernel(TokGeom g, TokState st, const uint16_t *__restrict__ k,
                                                         const uint16_t *__restrict__ v, int n_tokens, int pos0) {
  const int chunks = g.d / 8;
  const long long total = (long long)g.B * g.Hkv * n_tokens * chunks;
  for (long long it = (long long)blockIdx.x * blockDim.x + threadIdx.x; it < total;
       it += (long long)gridDim.x * blockDim.x) {
    const int ch = (int)(it % chunks);
    long long r = it / chunks;
    const int tok = (int)(r % n_tokens);
    r /= n_tokens;
    const int h = (int)(r % g.Hkv);
    const int b = (int)(r / g.Hkv);
    const int pos = pos0 + tok;
    uint16_t *kt = st.pages + tok_page_offset(g, b, h, pos / TS);
    uint16_t *vt = kt + TS * g.d;
    const int t = pos % TS, c0 = ch * 8;
    const size_t src = (((size_t)b * g.Hkv + h) * n_tokens + tok) * g.d + c0;
    *(uint4 *)(kt + k_tile_index(t, c0)) = *(const uint4 *)(k + src);
#pragma unroll
    for (int j = 0; j < 8; ++j) vt[v_tile_index(t, c0 + j)] = v[src + j];
    if (ch == 0) {
      const size_t u = ((size_t)b * g.Hkv + h) * g.T + pos;
      st.tier[u] = pos < g.n_sink ? T_SINK : T_RECENT;
      st.score[u] = 0.0f;
    }
  }
}

hipError_t tok_launch_append(const TokGeom &g, const TokState &st, const uint16_t *k, const uint16_t *v,
                             int n_tokens, int pos0, hipStream_t s) {
  const long long total = (long long)g.B * g.Hkv * n_tokens * (g.d / 8);
  int grid = (int)((total + 255) / 256);
  grid = grid > 16384 ? 16384 : (grid < 1 ? 1 : grid);
  hipLaunchKernelGGL(tok_append_kernel, dim3(grid), dim3(256), 0, s, g, st, k, v, n_tokens, pos0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// attention over [sink tile][compact tiles][recent position tiles]
// ---------------------------------------------------------------------------

struct TokList {
  int s0, nC, nR, rt0;   // sink tile present, compact tiles, recent tiles, first recent tile
  __device__ int count() const { return s0 + nC + nR; }
};

__device__ __forceinline__ TokList tok_list(const TokGeom &g, const TokStep &ts) {
  TokList L;
  L.s0 = (g.n_sink > 0 && ts.N > 0) ? 1 : 0;
  L.nC = (ts.n_cmp + TS - 1) / TS;
  L.rt0 = ts.rstart / TS;
  L.nR = ts.N > ts.rstart ? (ts.N - 1) / TS - L.rt0 + 1 : 0;
  return L;
}

// tile k of the list: page address and valid rows [lo, hi)
__device__ __forceinline__ const uint16_t *tok_tile(const TokGeom &g, const TokState &st, const TokStep &ts,
                                                    const TokList &L, int b, int h, int k, int &lo, int &hi) {
  if (k < L.s0) {
    lo = 0;
    hi = min(ts.N, g.n_sink);
    return st.pages + tok_page_offset(g, b, h, 0);
  }
  if (k < L.s0 + L.nC) {
    const int c = k - L.s0;
    lo = 0;
    hi = min(TS, ts.n_cmp - c * TS);
    return st.cpages + tok_cpage_offset(g, b, h, c);
  }
  const int rt = L.rt0 + (k - L.s0 - L.nC);
  lo = max(ts.rstart - rt * TS, 0);
  hi = min(ts.N - rt * TS, TS);
  return st.pages + tok_page_offset(g, b, h, rt);
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void tok_attend_kernel(
    TokGeom g, TokState st, TokStep ts, const uint16_t *__restrict__ q, size_t q_bstride, float scale_log2) {
  constexpr int KB = D / 32, CT = D / 16, CP = D / 32;
  const int S = g.n_splits;
  const int split = blockIdx.x % S;
  const int bh = blockIdx.x / S;
  const int h = bh % g.Hkv;
  const int b = bh / g.Hkv;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int lq = lane >> 4;
  const int G = g.G;
  const bool is_hi = col < G;
  const bool is_lo = col >= 8 && col < 8 + G;
  const bool has_q = is_hi || is_lo;
  const int hc = is_hi ? col : (is_lo ? col - 8 : 0);

  __shared__ float sm_m[ATT_WAVES][8];
  __shared__ float sm_l[ATT_WAVES][8];
  __shared__ float sm_o[ATT_WAVES][8][D];

  const TokList L = tok_list(g, ts);
  const int E = L.count();
  const int NS = 4 * S, gi = split * 4 + wave;
  const int ea = (int)((long long)E * gi / NS), eb = (int)((long long)E * (gi + 1) / NS);

  WaveState<D> ws;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) ws.acc[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
  ws.zacc = floatx4{0.f, 0.f, 0.f, 0.f};
  ws.m = has_q ? neg_inf() : 0.0f;   // columns without a head keep a finite reference
  ws.l = 0.0f;

  // query B operands (columns h and 8+h carry head h)
  bf16x8 bq[KB];
  {
    const uint16_t *qrow = q + (size_t)b * q_bstride + ((size_t)h * G + hc) * D;
    const uint32_t keep = has_q ? 0xffffffffu : 0u;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint4 r = *(const uint4 *)(qrow + kb * 32 + lq * 8);
      bq[kb] = __builtin_bit_cast(bf16x8, make_uint4(r.x & keep, r.y & keep, r.z & keep, r.w & keep));
    }
  }
  float *mrho = st.mrho + (size_t)bh * (g.TILES + 1) * G * TS;
  float *mref = st.mref + (size_t)bh * (g.TILES + 1) * G;

  if (ea < eb) {
    const int n_blocks = (eb - ea + 1) >> 1;
    // block i = tiles ea+2i, ea+2i+1 (a missing second tile repeats the first, masked)
    auto block = [&](int i, const uint16_t *(&ptr)[2], int (&lo)[2], int (&hi)[2], int (&e)[2]) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int k = ea + 2 * i + t;
        const bool valid = k < eb;
        ptr[t] = tok_tile(g, st, ts, L, b, h, valid ? k : ea + 2 * i, lo[t], hi[t]);
        if (!valid || !has_q) {
          lo[t] = 0;
          hi[t] = 0;
        }
        e[t] = valid ? k : g.TILES;
      }
    };
    const uint16_t *cp[2], *np[2];
    int clo[2], chi[2], ce[2], nlo[2], nhi[2], ne[2];
    block(0, cp, clo, chi, ce);
    uint4 kr[2][KB], vr[2][CP];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kr[t][kb] = *(const uint4 *)(cp[t] + (kb * 64 + lane) * 8);
#pragma unroll
      for (int p = 0; p < CP; ++p) vr[t][p] = *(const uint4 *)(cp[t] + TS * D + (p * 64 + lane) * 8);
    }
    for (int i = 0; i < n_blocks; ++i) {
      block(min(i + 1, n_blocks - 1), np, nlo, nhi, ne);   // the last block re-reads itself
      floatx4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) s[t] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, kr[t][kb]), bq[kb], s[t]);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) kr[t][kb] = *(const uint4 *)(np[t] + (kb * 64 + lane) * 8);
      float p[2][4], tsum[2];
      softmax_block<D, 2>(ws, s, scale_log2, clo, chi, lq, p, tsum);
      // per-slot probabilities of the heads (lanes of column h < G hold rows 4*lq..+3)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int er = is_hi ? ce[t] : g.TILES;
        *(float4 *)(mrho + ((size_t)er * G + (col & (G - 1))) * TS + 4 * lq) =
            make_float4(p[t][0], p[t][1], p[t][2], p[t][3]);
        const int em = (is_hi && lq == 0) ? ce[t] : g.TILES;
        mref[(size_t)em * G + (col & (G - 1))] = ws.m;
      }
      // rows h carry bf16(p), rows 8+h carry bf16(p - bf16(p))
      bf16x8 ap;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const float hi_ = (float)(__bf16)p[t][i2];
          ap[t * 4 + i2] = (__bf16)(is_lo ? p[t][i2] - hi_ : p[t][i2]);
        }
#pragma unroll
      for (int p2 = 0; p2 < CP; ++p2) {
        const uint4 v0 = make_uint4(vr[0][p2].x, vr[0][p2].y, vr[1][p2].x, vr[1][p2].y);
        const uint4 v1 = make_uint4(vr[0][p2].z, vr[0][p2].w, vr[1][p2].z, vr[1][p2].w);
        ws.acc[2 * p2] = mfma_bf16_k32(ap, __builtin_bit_cast(bf16x8, v0), ws.acc[2 * p2]);
        ws.acc[2 * p2 + 1] = mfma_bf16_k32(ap, __builtin_bit_cast(bf16x8, v1), ws.acc[2 * p2 + 1]);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int p2 = 0; p2 < CP; ++p2) vr[t][p2] = *(const uint4 *)(np[t] + TS * D + (p2 * 64 + lane) * 8);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        cp[t] = np[t];
        clo[t] = nlo[t];
        chi[t] = nhi[t];
        ce[t] = ne[t];
      }
    }
  }

  // ---- wave epilogue: fold the low-limb rows 8+h onto rows h ----
  float l_tot = sum_x32(sum_x16(ws.l));
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.acc[ct][i] += __shfl_down(ws.acc[ct][i], 32);

  // ---- workgroup merge ----
  if (lq == 0 && col < G) {
    sm_m[wave][col] = ws.m;
    sm_l[wave][col] = l_tot;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * lq + i;
    if (r < G) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) sm_o[wave][r][ct * 16 + col] = ws.acc[ct][i];
    }
  }
  __syncthreads();
  const size_t pbase = ((size_t)bh * S + split) * G;
  for (int it = threadIdx.x; it < G * D; it += blockDim.x) {
    const int hh = it / D, c = it % D;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w) M = fmaxf(M, sm_m[w][hh]);
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w)
      if (sm_m[w][hh] != neg_inf()) o += sm_o[w][hh][c] * exp2f(sm_m[w][hh] - M);
    st.part_o[(pbase + hh) * D + c] = o;
    if (c == 0) {
      float l = 0.0f;
#pragma unroll
      for (int w = 0; w < ATT_WAVES; ++w)
        if (sm_m[w][hh] != neg_inf()) l += sm_l[w][hh] * exp2f(sm_m[w][hh] - M);
      st.part_ml[(pbase + hh) * 2 + 0] = M;
      st.part_ml[(pbase + hh) * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// merge: outputs per (sequence, KV head); per-token masses -> scores
// ---------------------------------------------------------------------------

__device__ inline void tok_split_stats(const TokGeom &g, const TokState &st, int bh, int hh, float &M, float &invL) {
  const int S = g.n_splits, G = g.G;
  const float *ml = st.part_ml + ((size_t)bh * S * G + hh) * 2;
  float m = neg_inf(), l = 0.0f;
  for (int s = 0; s < S; ++s) {
    const float ms = ml[(size_t)s * G * 2], ls = ml[(size_t)s * G * 2 + 1];
    if (ms == neg_inf()) continue;
    const float mn = fmaxf(m, ms);
    l = (m == neg_inf() ? 0.0f : l * exp2f(m - mn)) + ls * exp2f(ms - mn);
    m = mn;
  }
  M = m;
  invL = 1.0f / l;
}

template <int G>
__global__ __launch_bounds__(256) void tok_merge_kernel(TokGeom g, TokState st, TokStep ts, float *__restrict__ out,
                                                        float *__restrict__ mass_out, int n_chunks) {
  constexpr int CH = 8;
  const int S = g.n_splits, D = g.d;
  const int n_out_blocks = g.B * g.Hkv;
  if ((int)blockIdx.x < n_out_blocks) {
    const int bh = blockIdx.x;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const float2 *ml = (const float2 *)st.part_ml + (size_t)bh * S * G;
    const float *po = st.part_o + (size_t)bh * S * G * D;
    for (int it = threadIdx.x; it < G * D; it += blockDim.x) {
      const int hh = it / D, c = it % D;
      float m = neg_inf(), l = 0.0f, o = 0.0f;
      for (int s0 = 0; s0 < S; s0 += CH) {
        float2 mls[CH];
        float os[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          const int sp = min(s0 + k, S - 1);
          mls[k] = ml[sp * G + hh];
          os[k] = po[(size_t)(sp * G + hh) * D + c];
        }
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          if (s0 + k >= S || mls[k].x == neg_inf()) continue;
          const float mn = fmaxf(m, mls[k].x);
          const float a = m == neg_inf() ? 0.0f : exp2f(m - mn), w = exp2f(mls[k].x - mn);
          l = l * a + mls[k].y * w;
          o = o * a + os[k] * w;
          m = mn;
        }
      }
      out[((size_t)b * g.Hq + (size_t)h * G + hh) * D + c] = o / l;
    }
    return;
  }
  // masses: 256 token slots (16 tiles) of one (sequence, KV head) per block
  __shared__ float sM[G], sInvL[G];
  const int mb = blockIdx.x - n_out_blocks;
  const int bh = mb / n_chunks, chunk = mb % n_chunks;
  const int b = bh / g.Hkv, h = bh % g.Hkv;
  const TokList L = tok_list(g, ts);
  const int k = chunk * (256 / TS) + (int)threadIdx.x / TS;   // tile
  const int slot = threadIdx.x % TS;
  if ((int)threadIdx.x < G) tok_split_stats(g, st, bh, threadIdx.x, sM[threadIdx.x], sInvL[threadIdx.x]);
  __syncthreads();
  if (k >= L.count()) return;
  int lo, hi;
  (void)tok_tile(g, st, ts, L, b, h, k, lo, hi);
  if (slot < lo || slot >= hi) return;
  int pos;
  if (k < L.s0)
    pos = slot;
  else if (k < L.s0 + L.nC)
    pos = st.cpos[(size_t)bh * g.NCT * TS + (k - L.s0) * TS + slot];
  else
    pos = (L.rt0 + (k - L.s0 - L.nC)) * TS + slot;
  const float *rho = st.mrho + ((size_t)bh * (g.TILES + 1) + k) * G * TS;
  const float *ref = st.mref + ((size_t)bh * (g.TILES + 1) + k) * G;
  float mass = 0.0f;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float v = rho[hh * TS + slot] * exp2f(ref[hh] - sM[hh]) * sInvL[hh];
    if (!(v >= 1.17549435e-38f)) v = 0.0f;   // a head's weight below FLT_MIN counts as 0
    mass += v;
  }
  const size_t u = (size_t)bh * g.T + pos;
  if (mass_out) mass_out[u] = mass;
  st.score[u] += mass;
}

hipError_t tok_launch_attend(const TokGeom &g, const TokState &st, const TokStep &ts, const uint16_t *q,
                             size_t q_bstride, float *out, float *mass_out, hipStream_t s, hipEvent_t ev_start,
                             hipEvent_t ev_stop) {
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)g.d));
  const int grid = g.B * g.Hkv * g.n_splits;
  hipError_t e;
  if (ev_start && (e = hipEventRecord(ev_start, s)) != hipSuccess) return e;
  if (g.d == 128)
    hipLaunchKernelGGL(tok_attend_kernel<128>, dim3(grid), dim3(256), 0, s, g, st, ts, q, q_bstride, scale_log2);
  else
    hipLaunchKernelGGL(tok_attend_kernel<64>, dim3(grid), dim3(256), 0, s, g, st, ts, q, q_bstride, scale_log2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev_stop && (e = hipEventRecord(ev_stop, s)) != hipSuccess) return e;
  if (mass_out && (e = launch_clear(mass_out, (size_t)g.B * g.Hkv * g.T * sizeof(float), s)) != hipSuccess) return e;
  const int n_tiles = (g.n_sink > 0 ? 1 : 0) + (ts.n_cmp + TS - 1) / TS +
                      (ts.N > ts.rstart ? (ts.N - 1) / TS - ts.rstart / TS + 1 : 0);
  const int n_chunks = (n_tiles * TS + 255) / 256;
  const dim3 mgrid(g.B * g.Hkv + g.B * g.Hkv * n_chunks);
  if (g.G == 4)
    hipLaunchKernelGGL(tok_merge_kernel<4>, mgrid, dim3(256), 0, s, g, st, ts, out, mass_out, n_chunks);
  else
    hipLaunchKernelGGL(tok_merge_kernel<8>, mgrid, dim3(256), 0, s, g, st, ts, out, mass_out, n_chunks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// routing (H2O): rank the kept older tokens and the newly aged ones per
// (sequence, KV head), keep the best k_heavy, gather them into compact tiles
// ---------------------------------------------------------------------------

__device__ inline void tok_bitonic_desc(unsigned long long *keys, int n) {
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long a = keys[i], c = keys[ixj];
          const bool desc = (i & k) == 0;
          if ((a < c) == desc) {
            keys[i] = c;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
}

__global__ __launch_bounds__(1024) void tok_route_h2o_kernel(TokGeom g, TokState st, int n_old, int a0, int a1,
                                                             int npow) {
  extern __shared__ unsigned long long keys[];
  const int bh = blockIdx.x;
  const int b = bh / g.Hkv, h = bh % g.Hkv;
  const int n = n_old + (a1 - a0);
  const size_t tb = (size_t)bh * g.T;
  int32_t *cpos = st.cpos + (size_t)bh * g.NCT * TS;
  // key: score bits (non-negative floats order like their bits), then position + 1
  for (int i = threadIdx.x; i < npow; i += blockDim.x) {
    unsigned long long key = 0ull;
    if (i < n) {
      const int pos = i < n_old ? cpos[i] : a0 + (i - n_old);
      key = ((unsigned long long)__float_as_uint(st.score[tb + pos]) << 32) | (unsigned)(pos + 1);
    }
    keys[i] = key;
  }
  __syncthreads();
  tok_bitonic_desc(keys, npow);
  const int keep = n < g.k_heavy ? n : g.k_heavy;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int pos = (int)(keys[i] & 0xffffffffull) - 1;
    st.tier[tb + pos] = i < keep ? T_FULL : T_EVICTED;
    if (i < keep) cpos[i] = pos;
  }
  // gather the kept tokens (rank order) into the compact tiles
  const int D = g.d, chunks = D / 8;
  for (int it = threadIdx.x; it < keep * chunks; it += blockDim.x) {
    const int i = it / chunks, c0 = (it % chunks) * 8;
    const int pos = (int)(keys[i] & 0xffffffffull) - 1;
    const uint16_t *sk = st.pages + tok_page_offset(g, b, h, pos / TS);
    const uint16_t *sv = sk + TS * D;
    uint16_t *dk = st.cpages + tok_cpage_offset(g, b, h, i / TS);
    uint16_t *dv = dk + TS * D;
    const int ts_ = pos % TS, td = i % TS;
    *(uint4 *)(dk + k_tile_index(td, c0)) = *(const uint4 *)(sk + k_tile_index(ts_, c0));
#pragma unroll
    for (int j = 0; j < 8; ++j) dv[v_tile_index(td, c0 + j)] = sv[v_tile_index(ts_, c0 + j)];
  }
}

hipError_t tok_launch_route(const TokGeom &g, const TokState &st, const TokStep &ts, int a0, int a1, int n_cand,
                            hipStream_t s) {
  int npow = 1;
  while (npow < n_cand) npow <<= 1;
  hipLaunchKernelGGL(tok_route_h2o_kernel, dim3(g.B * g.Hkv), dim3(1024), npow * sizeof(unsigned long long), s, g,
                     st, ts.n_cmp, a0, a1, npow);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// export: tiers and scores per (sequence, KV head, position)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void tok_export_kernel(TokGeom g, TokState st, int what, void *dst) {
  const size_t n = (size_t)g.B * g.Hkv * g.T;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    if (what == QKV_EXPORT_TIERS)
      ((uint8_t *)dst)[i] = st.tier[i];
    else
      ((float *)dst)[i] = st.score[i];
  }
}

hipError_t tok_launch_export(const TokGeom &g, const TokState &st, int what, void *dst, hipStream_t s) {
  const size_t n = (size_t)g.B * g.Hkv * g.T;
  int grid = (int)((n + 255) / 256);
  grid = grid > 4096 ? 4096 : (grid < 1 ? 1 : grid);
  hipLaunchKernelGGL(tok_export_kernel, dim3(grid), dim3(256), 0, s, g, st, what, dst);
  return hipGetLastError();
}

}  // namespace qkv
