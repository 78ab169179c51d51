// Token-mode kernels of the tiered decode path (gfx950): H2O heavy-hitter
// eviction and HqeKV five-tier assignment, where every token is its own unit
// and scores are kept per (sequence, KV head).
//
// H2O notes, sections 1.1-2.1 and the GQA paragraph: append the new token,
// attend over the kept set plus the new token, add each kept token's weight
// (summed over the query heads that share the KV head) to its score, keep the
// newest B_r tokens and the sinks, and evict from the older tokens the
// lowest-scored ones so that B_h heavy hitters remain.
//
// HqeKV notes, sections 3.2-3.5: every T steps the tokens ranked so far are
// ordered by accumulated attention times value range and cut by the tier
// shares into BF16 / INT4 / INT2 / INT1 (normalized) / evicted; a token only
// moves to a lower precision, re-quantized from its current values (keys and
// values per token, groups of 32 channels; INT1: mean and deviation).
//
// Ranked tokens live in compact tiles per tier, gathered at each routing
// call; tokens not yet ranked (and H2O's sinks) are read from the position
// pages.  The attention kernel streams [sink][BF16 compact][INT4][INT2][INT1]
// [recent] tiles: full-precision tiles feed bf16 matrix-core operands;
// quantized tiles feed their integer codes to fp16 matrix-core operations
// against the (exactly scaled) fp16 query, with the per-token scales and
// zeros applied in float32 and the value scale folded into the probabilities
// as two fp16 limbs (about 22 bits).  Each token slot's probability is emitted relative to the running
// maximum; the merge kernel normalizes those with the global (max, sum) of
// each head and adds each token's mass into an accumulator kept in list order
// (coalesced; the lists only change at routing calls).  Before a routing call
// or an export of the scores, the accumulators are added into the per-token
// scores and cleared.  With a routing period of 1 the merge adds into the
// per-token scores directly.
#include <hip/hip_ext.h>

#include "qkv_device.h"

namespace qkv {

namespace {

constexpr size_t TOK_ALIGN = 256;
inline size_t tok_align(size_t x) { return (x + TOK_ALIGN - 1) / TOK_ALIGN * TOK_ALIGN; }
constexpr float KAPPA1 = 0.6744897501960817f;   // Phi^-1(3/4): INT1 centres are mean -/+ KAPPA1 * std

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
  st.tacc = (float *)take(BH * g.TILES * TS * 4);
  st.scratch_out = (float *)take((size_t)g.B * g.Hq * g.d * 4);
  st.status = (int32_t *)take(16);
  st.vrange = nullptr;
  st.qrec = nullptr;
  st.cnt = nullptr;
  st.cuts = nullptr;
  st.hqold = nullptr;
  st.hqkey = nullptr;
  st.event = nullptr;
  st.victims = nullptr;
  if (g.policy == QKV_POLICY_H2O || g.policy == QKV_POLICY_HQEKV) {
    st.event = (int32_t *)take(BH * EV_WORDS * 4);
    st.victims = (int32_t *)take(BH * g.T * 4);
  }
  for (int k = 0; k < 3; ++k) {
    st.qtiles[k] = nullptr;
    st.qpos[k] = nullptr;
  }
  if (g.policy == QKV_POLICY_HQEKV) {
    st.vrange = (float *)take(BH * g.T * 4);
    st.qrec = (uint8_t *)take(BH * g.T * g.rec_bytes);
    for (int k = 0; k < 3; ++k) {
      st.qtiles[k] = (uint8_t *)take(BH * g.NCT * g.qtile_bytes[k]);
      st.qpos[k] = (int32_t *)take(BH * g.NCT * TS * 4);
    }
    st.cnt = (int32_t *)take(BH * 4 * 4);
    st.cuts = (unsigned long long *)take(BH * 4 * 8);
    st.hqold = (uint8_t *)take(BH * g.T);
    st.hqkey = (uint32_t *)take(BH * hq_key_stride(g) * 4);
  }
  return off;
}

// ---------------------------------------------------------------------------
// append: new tokens into the position pages (HqeKV: and their value range)
// ---------------------------------------------------------------------------

// one block row per (sequence, KV head); thread it of the row copies 16-byte
// chunk it % (D/8) of token it / (D/8)
template <int D>
__global__ __launch_bounds__(256) void tok_append_kernel(TokGeom g, TokState st, const uint16_t *__restrict__ k,
                                                         const uint16_t *__restrict__ v, int n_tokens, int pos0) {
  constexpr int CH = D / 8;
  const int bh = blockIdx.x;
  const int b = bh / g.Hkv, h = bh - b * g.Hkv;
  const int total = n_tokens * CH;
  for (int it = blockIdx.y * blockDim.x + threadIdx.x; it < total; it += gridDim.y * blockDim.x) {
    const int tok = it / CH, c0 = (it % CH) * 8;
    const int pos = pos0 + tok;
    uint16_t *kt = st.pages + tok_page_offset(g, b, h, pos / TS);
    uint16_t *vt = kt + TS * D;
    const int t = pos % TS;
    const size_t row = ((size_t)bh * n_tokens + tok) * D;
    *(uint4 *)(kt + k_tile_index(t, c0)) = *(const uint4 *)(k + row + c0);
    const uint4 vq = *(const uint4 *)(v + row + c0);
    const uint16_t *vs = (const uint16_t *)&vq;
#pragma unroll
    for (int j = 0; j < 8; ++j) vt[v_tile_index(t, c0 + j)] = vs[j];
    const size_t u = (size_t)bh * g.T + pos;
    if (c0 == 0) {
      st.tier[u] = pos < g.n_sink ? T_SINK : T_RECENT;
      st.score[u] = 0.0f;
    }
    if (st.vrange) {
      // value range over the token's channels (HqeKV section 3.2): the token's
      // D/8 chunks are adjacent lanes of one wave (the stride is a multiple
      // of 64 and the chunk count divides 64), reduced by shuffles
      float mn = bf16_to_f32(vs[0]), mx = mn;
#pragma unroll
      for (int j = 1; j < 8; ++j) {
        mn = fminf(mn, bf16_to_f32(vs[j]));
        mx = fmaxf(mx, bf16_to_f32(vs[j]));
      }
#pragma unroll
      for (int off = 1; off < CH; off <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, off));
        mx = fmaxf(mx, __shfl_xor(mx, off));
      }
      if (c0 == 0) st.vrange[u] = mx - mn;
    }
  }
}

hipError_t tok_launch_append(const TokGeom &g, const TokState &st, const uint16_t *k, const uint16_t *v,
                             int n_tokens, int pos0, hipStream_t s) {
  if ((long long)n_tokens * (g.d / 8) > 0x7fffffffLL) return hipErrorInvalidValue;
  const int total = n_tokens * (g.d / 8);
  const int threads = total <= 64 ? 64 : 256;
  int rows = (total + threads - 1) / threads;
  if (rows > 65535) rows = 65535;
  const dim3 grid(g.B * g.Hkv, rows);
  if (g.d == 128)
    hipLaunchKernelGGL(tok_append_kernel<128>, grid, dim3(threads), 0, s, g, st, k, v, n_tokens, pos0);
  else
    hipLaunchKernelGGL(tok_append_kernel<64>, grid, dim3(threads), 0, s, g, st, k, v, n_tokens, pos0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// live tiles of one (sequence, KV head):
//   [sink][BF16 compact][INT4][INT2][INT1][recent position tiles]
// ---------------------------------------------------------------------------

struct TokList {
  int s0, nC, nQ[3], nR, rt0;   // tiles of each part; first recent position tile
  int nCtok, nQtok[3];          // tokens in the compact lists
  __device__ int base_q(int k) const {
    int b = s0 + nC;
    for (int j = 0; j < k; ++j) b += nQ[j];
    return b;
  }
  __device__ int base_r() const { return s0 + nC + nQ[0] + nQ[1] + nQ[2]; }
  __device__ int count() const { return base_r() + nR; }
};

__device__ __forceinline__ TokList tok_list(const TokGeom &g, const TokState &st, const TokStep &ts, int bh) {
  TokList L;
  L.s0 = (g.n_sink > 0 && ts.N > 0) ? 1 : 0;
  if (g.policy == QKV_POLICY_HQEKV) {
    L.nCtok = st.cnt[bh * 4 + 0];
    for (int k = 0; k < 3; ++k) L.nQtok[k] = st.cnt[bh * 4 + 1 + k];
  } else {
    L.nCtok = ts.n_cmp;
    for (int k = 0; k < 3; ++k) L.nQtok[k] = 0;
  }
  L.nC = (L.nCtok + TS - 1) / TS;
  for (int k = 0; k < 3; ++k) L.nQ[k] = (L.nQtok[k] + TS - 1) / TS;
  L.rt0 = ts.rstart / TS;
  L.nR = ts.N > ts.rstart ? (ts.N - 1) / TS - L.rt0 + 1 : 0;
  return L;
}

// full-precision tile k of the list (sink, compact or recent): page address, valid rows [lo, hi)
__device__ __forceinline__ const uint16_t *tok_ftile(const TokGeom &g, const TokState &st, const TokStep &ts,
                                                     const TokList &L, int b, int h, int k, int &lo, int &hi) {
  if (k < L.s0) {
    lo = 0;
    hi = min(ts.N, g.n_sink);
    return st.pages + tok_page_offset(g, b, h, 0);
  }
  if (k < L.s0 + L.nC) {
    const int c = k - L.s0;
    lo = 0;
    hi = min(TS, L.nCtok - c * TS);
    return st.cpages + tok_cpage_offset(g, b, h, c);
  }
  const int rt = L.rt0 + (k - L.base_r());
  lo = max(ts.rstart - rt * TS, 0);
  hi = min(ts.N - rt * TS, TS);
  return st.pages + tok_page_offset(g, b, h, rt);
}

// position of slot `slot` of list tile k of (sequence, KV head) bh; -1 when
// the slot holds no token.  Without LOOKUP only validity is decided (0).
template <bool LOOKUP>
__device__ __forceinline__ int tok_slot_pos(const TokGeom &g, const TokState &st, const TokStep &ts, const TokList &L,
                                            int bh, int k, int slot) {
  if (k < L.s0 + L.nC || k >= L.base_r()) {
    int lo, hi;
    (void)tok_ftile(g, st, ts, L, bh / g.Hkv, bh % g.Hkv, k, lo, hi);
    if (slot < lo || slot >= hi) return -1;
    if (!LOOKUP) return 0;
    if (k < L.s0) return slot;
    if (k < L.s0 + L.nC) return st.cpos[(size_t)bh * g.NCT * TS + (k - L.s0) * TS + slot];
    return (L.rt0 + (k - L.base_r())) * TS + slot;
  }
  int f = 0;
  while (k >= L.base_q(f + 1)) ++f;
  const int idx = (k - L.base_q(f)) * TS + slot;
  if (idx >= L.nQtok[f]) return -1;
  return LOOKUP ? st.qpos[f][(size_t)bh * g.NCT * TS + idx] : 0;
}

// valid slots [lo, hi) of list tile k of (sequence, KV head) bh
__device__ __forceinline__ void tok_tile_range(const TokGeom &g, const TokState &st, const TokStep &ts,
                                               const TokList &L, int bh, int k, int &lo, int &hi) {
  if (k < L.s0 + L.nC || k >= L.base_r()) {
    (void)tok_ftile(g, st, ts, L, bh / g.Hkv, bh % g.Hkv, k, lo, hi);
    return;
  }
  int f = 0;
  while (k >= L.base_q(f + 1)) ++f;
  lo = 0;
  hi = min(TS, L.nQtok[f] - (k - L.base_q(f)) * TS);
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------

struct TokCtx {
  const TokGeom *g;
  const TokState *st;
  const TokStep *ts;
  const TokList *L;
  int b, h, bh, lane, col, lq, G;
  bool is_hi, is_lo, has_q;
  int slot;               // channel-group slot of this lane's A row in the paired value product
  float *mrho, *mref;
  uint32_t *lds_par;      // per wave: raw params of a block's two quantized tiles
  float *lds_ks;          // per wave: their key scales as float32 [2][groups][16]
};

// per-slot probabilities of a tile (lanes of column h < G hold rows 4*lq..+3)
// and the running max they are relative to; other lanes write the spare row
template <int GP>
__device__ __forceinline__ void tok_store_mass(const TokCtx &c, int e, const float *p, float m) {
  constexpr int G = GP == 2 ? 4 : 8;
  const bool mass_lane = c.col < G;
  const int er = mass_lane ? e : c.g->TILES;
  *(float4 *)(c.mrho + ((size_t)er * G + (c.col & (G - 1))) * TS + 4 * c.lq) = make_float4(p[0], p[1], p[2], p[3]);
  const int em = (mass_lane && c.lq == 0) ? e : c.g->TILES;
  c.mref[(size_t)em * G + (c.col & (G - 1))] = m;
}

// full-precision tiles (sink, compact, recent) of virtual range [ea, eb);
// virtual index v < s0 + nC is list tile v, above it list tile v + (quantized tiles)
template <int D, int GP>
__device__ __forceinline__ void tok_run_bf16(WaveState<D> &ws, const TokCtx &c, const bf16x8 (&bq)[D / 32], float sc, int ea,
                             int eb) {
  if (ea >= eb) return;
  constexpr int KB = D / 32, CP = D / 32;
  const TokList &L = *c.L;
  const int skip = L.base_r() - (L.s0 + L.nC);   // quantized tiles between compact and recent
  const int n_blocks = (eb - ea + 1) >> 1;
  auto block = [&](int i, const uint16_t *(&ptr)[2], int (&lo)[2], int (&hi)[2], int (&e)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int vk = ea + 2 * i + t;
      const bool valid = vk < eb;
      const int v = valid ? vk : ea + 2 * i;
      const int k = v < L.s0 + L.nC ? v : v + skip;
      ptr[t] = tok_ftile(*c.g, *c.st, *c.ts, L, c.b, c.h, k, lo[t], hi[t]);
      if (!valid || !c.has_q) {
        lo[t] = 0;
        hi[t] = 0;
      }
      e[t] = valid ? k : c.g->TILES;
    }
  };
  const uint16_t *cp[2], *np[2];
  int clo[2], chi[2], ce[2], nlo[2], nhi[2], ne[2];
  block(0, cp, clo, chi, ce);
  u32x4v kr[2][KB], vr[2][CP];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) kr[t][kb] = ld_stream16v(cp[t] + (kb * 64 + c.lane) * 8);
#pragma unroll
    for (int p = 0; p < CP; ++p) vr[t][p] = ld_stream16v(cp[t] + TS * D + (p * 64 + c.lane) * 8);
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
      for (int kb = 0; kb < KB; ++kb) kr[t][kb] = ld_stream16v(np[t] + (kb * 64 + c.lane) * 8);
    float p[2][4], tsum[2];
    softmax_block<D, 2>(ws, s, sc, clo, chi, c.lq, p, tsum);
#pragma unroll
    for (int t = 0; t < 2; ++t) tok_store_mass<GP>(c, ce[t], p[t], ws.m);
    // rows h carry bf16(p), rows 8+h carry bf16(p - bf16(p))
    bf16x8 ap;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        const float hi_ = (float)(__bf16)p[t][i2];
        ap[t * 4 + i2] = (__bf16)(c.is_lo ? p[t][i2] - hi_ : p[t][i2]);
      }
#pragma unroll
    for (int p2 = 0; p2 < CP; ++p2) {
      const u32x4v v0 = __builtin_shufflevector(vr[0][p2], vr[1][p2], 0, 1, 4, 5);
      const u32x4v v1 = __builtin_shufflevector(vr[0][p2], vr[1][p2], 2, 3, 6, 7);
      ws.acc[2 * p2] = mfma_bf16_k32(ap, __builtin_bit_cast(bf16x8, v0), ws.acc[2 * p2]);
      ws.acc[2 * p2 + 1] = mfma_bf16_k32(ap, __builtin_bit_cast(bf16x8, v1), ws.acc[2 * p2 + 1]);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int p2 = 0; p2 < CP; ++p2) vr[t][p2] = ld_stream16v(np[t] + TS * D + (p2 * 64 + c.lane) * 8);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      cp[t] = np[t];
      clo[t] = nlo[t];
      chi[t] = nhi[t];
      ce[t] = ne[t];
    }
  }
}

// INT4 and INT2 compact tiles (F = 0, 1) are laid out in the order the
// matrix-core operands are built, so that the attention kernel never
// dequantizes an element:
//   K codes  [64 lanes][CW dwords]: lane l holds token l%16, channels
//            kb*32 + 8*(l/16) + e (e < 8) of every k-block kb (ql_kslot)
//   V codes  [64 lanes][CW dwords]: lane l holds channel ct*16 + l%16 of
//            every column tile ct, tokens 4*(l/16) + tt (tt < 4) (ql_vslot)
//   params   K scale [NG][16], K zero [16][NG] (token-major), V scale [NG][16],
//            V zero [NG][16], fp16, one (scale, zero) per 32-channel group
// INT2 places codes as the window ledger does (two 2-bit codes per byte
// nibble pair, unpacked by the FP4 conversion); INT4 puts code e of a k-block
// at nibble 2e (e < 4) or 2(e-4)+1, and value token tt of column tile ct at
// nibble 2tt + ct%2 of dword ct/2 (unpacked by the FP8 conversion).
template <int D, int F>
struct QL {
  static constexpr int KB = D / 32, CT = D / 16, NG = D / 32, NKD = D / 64;
  static constexpr int CW = F == 0 ? KB : NKD;   // code dwords per lane, keys and values alike
  static constexpr int VC = 256 * CW, PAR = 512 * CW;
  static constexpr int KS = PAR, KZ = PAR + 32 * NG, VS = PAR + 64 * NG, VZ = PAR + 96 * NG;
  static constexpr int BYTES = PAR + 128 * NG;
};

// INT1 compact tiles: one code dword per lane for keys and one for values,
// each bit a code, placed so that (x >> j) & 0x11111111 leaves eight codes as
// the nibbles 000b of four bytes (the FP4 conversion then gives 0 or 1):
//   keys: code of k-block kb, element e at bit 4e + kb
//   values: column tile ct, token tt at bit 8*(2*(ct%2) + tt/2) + 4*(tt%2) + ct/2
//   params: K std [16], K mean [16], V std [16], V mean [16], fp16
template <int D>
struct Q1 {
  static constexpr int KB = D / 32, CT = D / 16, NG = D / 32;
  static constexpr int VC = 256, PAR = 512;
  static constexpr int KSD = PAR, KM = PAR + 32, VSD = PAR + 64, VM = PAR + 96;
  static constexpr int BYTES = PAR + 128;
};
__host__ __device__ inline int q1_kbit(int kb, int e) { return 4 * e + kb; }
__host__ __device__ inline int q1_vbit(int ct, int tt) { return 8 * (2 * (ct & 1) + (tt >> 1)) + 4 * (tt & 1) + (ct >> 1); }

template <int F>
__host__ __device__ inline void ql_kslot(int kb, int e, int &dw, int &bit) {
  if (F == 0) {
    dw = kb;
    bit = 4 * (e < 4 ? 2 * e : 2 * (e - 4) + 1);
  } else {
    dw = kb >> 1;
    bit = 2 * (4 * (e >> 1) + (kb & 1) + 2 * (e & 1));
  }
}
template <int F>
__host__ __device__ inline void ql_vslot(int ct, int tt, int &dw, int &bit) {
  if (F == 0) {
    dw = ct >> 1;
    bit = 4 * (2 * tt + (ct & 1));
  } else {
    dw = ct >> 2;
    bit = 2 * (4 * (ct & 3) + (tt >> 1) + 2 * (tt & 1));
  }
}

__device__ __forceinline__ float h_lo(uint32_t w) { return (float)__builtin_bit_cast(half_t, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float h_hi(uint32_t w) { return (float)__builtin_bit_cast(half_t, (uint16_t)(w >> 16)); }

// INT4 / INT2 tiles (QL layout), two per block.  Keys: one MFMA per k-block
// on the exact integer codes against the fp16 query (high columns only), kept
// per k-block and combined with each token's group scales in float32; the
// key-zero term sum_g z[t][g] * (sum of q over group g) is one 16x16x16 MFMA
// whose B operand holds the group sums as two fp16 limbs (high columns, low
// columns), folded with the rest by one DPP add.  Values: the value step is
// folded into the probabilities (fp16(p*s) on high rows, the exact remainder
// on low rows), against the exact integer codes; the value-zero term is one
// MFMA per block.
template <int D, int F, int GP>
__device__ __forceinline__ void tok_run_ql(WaveState<D> &ws, const TokCtx &c, const half8 (&bqk)[D / 32], half4 bQ, float sc,
                           int ea, int eb) {
  if (ea >= eb) return;
  using Q = QL<D, F>;
  constexpr int KB = Q::KB, NG = Q::NG, CW = Q::CW;
  const float neg1 = opaque_neg1();
  const TokList &L = *c.L;
  const int base = L.base_q(F);
  const int ntok = L.nQtok[F];
  const uint8_t *tiles = c.st->qtiles[F] + (size_t)c.bh * c.g->NCT * Q::BYTES;
  const int n_blocks = (eb - ea + 1) >> 1;
  auto block = [&](int i, const uint8_t *(&ptr)[2], int (&hi)[2], int (&e)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int qk = ea + 2 * i + t;
      const bool valid = qk < eb;
      const int qq = valid ? qk : ea + 2 * i;
      ptr[t] = tiles + (size_t)qq * Q::BYTES;
      hi[t] = valid ? min(TS, ntok - qq * TS) : 0;
      e[t] = valid ? base + qq : c.g->TILES;
    }
  };
  struct Buf {
    uint32_t kc[2][CW], vc[2][CW];
    uint32_t par[NG];   // this lane's 4*NG bytes of the params of tile lane/32
  };
  auto load = [&](const uint8_t *const (&ptr)[2], Buf &bf) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t *kc = (const uint32_t *)(ptr[t] + c.lane * 4 * CW);
      const uint32_t *vc = (const uint32_t *)(ptr[t] + Q::VC + c.lane * 4 * CW);
#pragma unroll
      for (int w = 0; w < CW; ++w) {
        bf.kc[t][w] = ld_stream4(kc + w);
        bf.vc[t][w] = ld_stream4(vc + w);
      }
    }
    // both tiles' params: lanes 0-31 the first tile's, 32-63 the second's
    const uint8_t *pp = (c.lane < 32 ? ptr[0] : ptr[1]) + Q::PAR + (c.lane & 31) * 4 * NG;
#pragma unroll
    for (int w = 0; w < NG; ++w) bf.par[w] = ld_stream4(pp + 4 * w);
  };
  const uint8_t *cp[2], *np[2];
  int chi[2], ce[2], nhi[2], ne[2];
  block(0, cp, chi, ce);
  Buf buf0, buf1;
  load(cp, buf0);
  const half4 zero4 = {(half_t)0, (half_t)0, (half_t)0, (half_t)0};
  auto step = [&](const int i, Buf &cur, Buf &nxt) __attribute__((always_inline)) {
    block(min(i + 1, n_blocks - 1), np, nhi, ne);   // the last block re-reads itself
    load(np, nxt);
    // stage params: raw bytes, and the key scales as float32
    {
      uint32_t *dst = c.lds_par + (c.lane >> 5) * 32 * NG + (c.lane & 31) * NG;
#pragma unroll
      for (int w = 0; w < NG; ++w) dst[w] = cur.par[w];
      if ((c.lane & 31) < 8) {   // these lanes hold the key scales [NG][16]
        float *ks = c.lds_ks + (c.lane >> 5) * 16 * NG + (c.lane & 31) * 2 * NG;
#pragma unroll
        for (int w = 0; w < NG; ++w) {
          ks[2 * w] = h_lo(cur.par[w]);
          ks[2 * w + 1] = h_hi(cur.par[w]);
        }
      }
    }
    wave_lds_sync();
    // ---- keys ----
    float x[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      floatx4 acc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const half8 a = F == 0 ? codes8_int4(cur.kc[t][kb]) : codes8(code_half(cur.kc[t][kb >> 1], kb & 1));
        acc[kb] = mfma_f16_k32(a, bqk[kb], floatx4{0.f, 0.f, 0.f, 0.f});
      }
      // key-zero term: A row = token (lanes 0-15), k = group
      half4 za = zero4;
      {
        const half_t *kz = (const half_t *)((const uint8_t *)c.lds_par + t * 128 * NG + (Q::KZ - Q::PAR)) +
                           (c.lane & 15) * NG;
        half4 zr;
        if (NG == 4) {
          zr = *(const half4 *)kz;
        } else {
          zr = half4{kz[0], kz[1], (half_t)0, (half_t)0};
        }
        za = c.lane < 16 ? zr : zero4;
      }
      floatx4 sco = mfma_f16_k16(za, bQ, floatx4{0.f, 0.f, 0.f, 0.f});
      const float *ks = c.lds_ks + t * 16 * NG;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const float4 s4 = *(const float4 *)(ks + kb * 16 + 4 * c.lq);
        sco[0] = __builtin_fmaf(s4.x, acc[kb][0], sco[0]);
        sco[1] = __builtin_fmaf(s4.y, acc[kb][1], sco[1]);
        sco[2] = __builtin_fmaf(s4.z, acc[kb][2], sco[2]);
        sco[3] = __builtin_fmaf(s4.w, acc[kb][3], sco[3]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = fold8(sco[r]);
        x[t][r] = 4 * c.lq + r < chi[t] ? f * sc : neg_inf();
      }
    }
    float p[2][4], tsum[2];
    softmax_rows<D, 2>(ws, x, p, tsum);
#pragma unroll
    for (int t = 0; t < 2; ++t) tok_store_mass<GP>(c, ce[t], p[t], ws.m);
    // ---- values ----
    // fp16 limbs of p (p cut toward zero to fp16, exact remainder); (P1, P2)
    // = (0, phi) on high rows, (phi, plo) on low rows
    half4 P1[2], P2[2];
    const uint32_t lo_keep = c.is_lo ? 0xffffffffu : 0u;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      half4 phi, plo;
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const half2v h = rtz_pair(p[t][r], p[t][r + 1]);
        phi[r] = h[0];
        phi[r + 1] = h[1];
        plo[r] = lo_limb(h[0], p[t][r], neg1);
        plo[r + 1] = lo_limb(h[1], p[t][r + 1], neg1);
      }
      const uint2 hb = __builtin_bit_cast(uint2, phi), lb = __builtin_bit_cast(uint2, plo);
      P1[t] = __builtin_bit_cast(half4, make_uint2(hb.x & lo_keep, hb.y & lo_keep));
      P2[t] = __builtin_bit_cast(half4, make_uint2(c.is_lo ? lb.x : hb.x, c.is_lo ? lb.y : hb.y));
    }
    const half_t *vs = (const half_t *)((const uint8_t *)c.lds_par + (Q::VS - Q::PAR));
    const half_t *vz = (const half_t *)((const uint8_t *)c.lds_par + (Q::VZ - Q::PAR));
#pragma unroll
    for (int gb = 0; gb < NG; gb += GP) {
      const int grp_l = gb + (GP == 1 ? 0 : c.slot);
      const half4 s40 = *(const half4 *)(vs + grp_l * TS + 4 * c.lq);
      const half4 s41 = *(const half4 *)(vs + 64 * NG + grp_l * TS + 4 * c.lq);
      const half4 t0 = P1[0] * s40, t1 = P1[1] * s41;
      const half4 ag0 = __builtin_elementwise_fma(P2[0], s40, __builtin_elementwise_fma(P1[0], s40, -t0));
      const half4 ag1 = __builtin_elementwise_fma(P2[1], s41, __builtin_elementwise_fma(P1[1], s41, -t1));
      const half8 ag = __builtin_shufflevector(ag0, ag1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int c2 = 0; c2 < 2 * GP; ++c2) {
        const int ct = gb * 2 + c2;
        half4 b0, b1;
        if (F == 0) {
          const uint32_t x0 = cur.vc[0][ct >> 1], x1 = cur.vc[1][ct >> 1];
          const uint32_t m0 = ((ct & 1) ? (x0 >> 4) : x0) & 0x0F0F0F0Fu;
          const uint32_t m1 = ((ct & 1) ? (x1 >> 4) : x1) & 0x0F0F0F0Fu;
          b0 = __builtin_shufflevector(fp8_pair<false>(m0), fp8_pair<true>(m0), 0, 1, 2, 3);
          b1 = __builtin_shufflevector(fp8_pair<false>(m1), fp8_pair<true>(m1), 0, 1, 2, 3);
        } else {
          const uint32_t v0 = cur.vc[0][ct >> 2], v1 = cur.vc[1][ct >> 2];
          b0 = __builtin_shufflevector(fp4_pair_sel(code_half(v0, 0), ct), fp4_pair_sel(code_half(v0, 1), ct), 0, 1,
                                       2, 3);
          b1 = __builtin_shufflevector(fp4_pair_sel(code_half(v1, 0), ct), fp4_pair_sel(code_half(v1, 1), ct), 0, 1,
                                       2, 3);
        }
        ws.acc[ct] = mfma_f16_k32(ag, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), ws.acc[ct]);
      }
    }
    {
      // value-zero term: B column = group (col < NG), k = the lane's four tokens of each tile
      const int zc = c.col < NG ? c.col : 0;
      const half4 z0 = *(const half4 *)(vz + zc * TS + 4 * c.lq);
      const half4 z1 = *(const half4 *)(vz + 64 * NG + zc * TS + 4 * c.lq);
      const half4 bz0 = c.col < NG ? z0 : zero4, bz1 = c.col < NG ? z1 : zero4;
      ws.zacc = mfma_f16_k32(__builtin_shufflevector(P2[0], P2[1], 0, 1, 2, 3, 4, 5, 6, 7),
                             __builtin_shufflevector(bz0, bz1, 0, 1, 2, 3, 4, 5, 6, 7), ws.zacc);
    }
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      cp[t] = np[t];
      chi[t] = nhi[t];
      ce[t] = ne[t];
    }
  };
  // two blocks per trip with the buffers' roles swapped, so that no buffer
  // whose loads are still in flight is copied at the end of a block
  int i = 0;
  for (; i + 1 < n_blocks; i += 2) {
    step(i, buf0, buf1);
    step(i + 1, buf1, buf0);
  }
  if (i < n_blocks) step(i, buf0, buf1);
}

// INT1 tiles (Q1 layout), two per block.  A token's values are
// mean + KAPPA1 * std * (2b - 1), so with a = 2 KAPPA1 std and
// c = mean - KAPPA1 std (float32, per token):
//   keys:   score = a * sum_c q_c b_c + c * sum_c q_c, one MFMA chain over the
//           0/1 codes against the fp16 query (high columns), then per row;
//   values: o = sum_t (p_t a_t) b_t + sum_t p_t c_t, with p*a split into two
//           fp16 limbs (high rows, low rows) against the 0/1 codes, and the
//           zero term as two MFMAs over the fp16 limbs of c.
template <int D, int GP>
__device__ __forceinline__ void tok_run_q1(WaveState<D> &ws, const TokCtx &c, const half8 (&bqk)[D / 32], float qall, float sc,
                           int ea, int eb) {
  if (ea >= eb) return;
  using Q = Q1<D>;
  constexpr int KB = Q::KB, CT = Q::CT, NG = Q::NG;
  const TokList &L = *c.L;
  const int base = L.base_q(2);
  const int ntok = L.nQtok[2];
  const uint8_t *tiles = c.st->qtiles[2] + (size_t)c.bh * c.g->NCT * Q::BYTES;
  const int n_blocks = (eb - ea + 1) >> 1;
  auto block = [&](int i, const uint8_t *(&ptr)[2], int (&hi)[2], int (&e)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int qk = ea + 2 * i + t;
      const bool valid = qk < eb;
      const int qq = valid ? qk : ea + 2 * i;
      ptr[t] = tiles + (size_t)qq * Q::BYTES;
      hi[t] = valid ? min(TS, ntok - qq * TS) : 0;
      e[t] = valid ? base + qq : c.g->TILES;
    }
  };
  struct Buf {
    uint32_t kc[2], vc[2];
    uint32_t par;   // this lane's 4 bytes of the params of tile lane/32
  };
  auto load = [&](const uint8_t *const (&ptr)[2], Buf &bf) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf.kc[t] = ld_stream4(ptr[t] + 4 * c.lane);
      bf.vc[t] = ld_stream4(ptr[t] + Q::VC + 4 * c.lane);
    }
    bf.par = ld_stream4((c.lane < 32 ? ptr[0] : ptr[1]) + Q::PAR + 4 * (c.lane & 31));
  };
  const uint8_t *cp[2], *np[2];
  int chi[2], ce[2], nhi[2], ne[2];
  block(0, cp, chi, ce);
  Buf buf0, buf1;
  load(cp, buf0);
  const half4 zero4 = {(half_t)0, (half_t)0, (half_t)0, (half_t)0};
  const half_t *par16 = (const half_t *)c.lds_par;   // [2 tiles][K std 16][K mean 16][V std 16][V mean 16]
  auto step = [&](const int i, Buf &cur, Buf &nxt) __attribute__((always_inline)) {
    block(min(i + 1, n_blocks - 1), np, nhi, ne);   // the last block re-reads itself
    load(np, nxt);
    c.lds_par[c.lane] = cur.par;
    wave_lds_sync();
    // ---- keys ----
    float x[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        acc = mfma_f16_k32(codes8((cur.kc[t] >> kb) & 0x11111111u), bqk[kb], acc);
      const half4 sd = *(const half4 *)(par16 + t * 64 + 4 * c.lq);
      const half4 mn = *(const half4 *)(par16 + t * 64 + 16 + 4 * c.lq);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = 2.0f * KAPPA1 * (float)sd[r];
        const float cz = __builtin_fmaf(-KAPPA1, (float)sd[r], (float)mn[r]);
        const float f = fold8(__builtin_fmaf(a, acc[r], c.is_hi ? cz * qall : 0.0f));
        x[t][r] = 4 * c.lq + r < chi[t] ? f * sc : neg_inf();
      }
    }
    float p[2][4], tsum[2];
    softmax_rows<D, 2>(ws, x, p, tsum);
#pragma unroll
    for (int t = 0; t < 2; ++t) tok_store_mass<GP>(c, ce[t], p[t], ws.m);
    // ---- values ----
    half8 ag, cz_hi, cz_lo;
    half4 P2[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const half4 sd = *(const half4 *)(par16 + t * 64 + 32 + 4 * c.lq);
      const half4 mn = *(const half4 *)(par16 + t * 64 + 48 + 4 * c.lq);
      half4 phi, plo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // p * a as a high part cut to 11 bits and the exact remainder
        const float pa = p[t][r] * (2.0f * KAPPA1 * (float)sd[r]);
        const float ah = __uint_as_float(__float_as_uint(pa) & 0xffffe000u);
        ag[t * 4 + r] = c.is_lo ? (half_t)(pa - ah) : (half_t)ah;
        const float ph = __uint_as_float(__float_as_uint(p[t][r]) & 0xffffe000u);
        phi[r] = (half_t)ph;
        plo[r] = (half_t)(p[t][r] - ph);
        const float cz = __builtin_fmaf(-KAPPA1, (float)sd[r], (float)mn[r]);
        const half_t czh = (half_t)cz;
        cz_hi[t * 4 + r] = c.col < NG ? czh : (half_t)0;
        cz_lo[t * 4 + r] = c.col < NG ? (half_t)(cz - (float)czh) : (half_t)0;
      }
      P2[t] = c.is_lo ? plo : phi;
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int B0 = 2 * (ct & 1);
      const uint32_t m0 = (cur.vc[0] >> (ct >> 1)) & 0x11111111u;
      const uint32_t m1 = (cur.vc[1] >> (ct >> 1)) & 0x11111111u;
      const half4 b0 = __builtin_shufflevector(fp4_pair_sel(m0, B0), fp4_pair_sel(m0, B0 + 1), 0, 1, 2, 3);
      const half4 b1 = __builtin_shufflevector(fp4_pair_sel(m1, B0), fp4_pair_sel(m1, B0 + 1), 0, 1, 2, 3);
      ws.acc[ct] = mfma_f16_k32(ag, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), ws.acc[ct]);
    }
    {
      const half8 pp = __builtin_shufflevector(P2[0], P2[1], 0, 1, 2, 3, 4, 5, 6, 7);
      ws.zacc = mfma_f16_k32(pp, cz_hi, ws.zacc);
      ws.zacc = mfma_f16_k32(pp, cz_lo, ws.zacc);
    }
    wave_lds_sync();
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      cp[t] = np[t];
      chi[t] = nhi[t];
      ce[t] = ne[t];
    }
  };
  // two blocks per trip with the buffers' roles swapped, so that no buffer
  // whose loads are still in flight is copied at the end of a block
  int i = 0;
  for (; i + 1 < n_blocks; i += 2) {
    step(i, buf0, buf1);
    step(i + 1, buf1, buf0);
  }
  if (i < n_blocks) step(i, buf0, buf1);
}

// NW waves per workgroup (8: the two waves on a SIMD belong to one
// workgroup; 4: two workgroups per compute unit)
template <int D, int GP, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void tok_attend_kernel(
    TokGeom g, TokState st, TokStep ts, const uint16_t *__restrict__ q, size_t q_bstride, float scale_log2) {
  constexpr int KB = D / 32, CT = D / 16, NG = D / 32;
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
  // columns 0..7 take high limbs, 8..15 low limbs; within each half column c
  // serves head (c mod 8) mod G, so every lane carries a head
  const bool is_hi = col < 8;
  const bool is_lo = col >= 8;
  const int hc = (col & 7) & (G - 1);

  __shared__ float sm_m[NW][8];
  __shared__ float sm_l[NW][8];
  __shared__ float sm_o[NW][8][D];
  __shared__ __attribute__((aligned(16))) uint32_t s_par[NW][2 * 32 * NG];
  __shared__ __attribute__((aligned(16))) float s_ks[NW][2 * 16 * NG];

  const TokList L = tok_list(g, st, ts, bh);
  TokCtx c;
  c.g = &g;
  c.st = &st;
  c.ts = &ts;
  c.L = &L;
  c.b = b;
  c.h = h;
  c.bh = bh;
  c.lane = lane;
  c.col = col;
  c.lq = lq;
  c.G = G;
  c.is_hi = is_hi;
  c.is_lo = is_lo;
  c.has_q = true;
  c.slot = min((col & 7) / G, GP - 1);
  c.mrho = st.mrho + (size_t)bh * (g.TILES + 1) * G * TS;
  c.mref = st.mref + (size_t)bh * (g.TILES + 1) * G;
  c.lds_par = &s_par[wave][0];
  c.lds_ks = &s_ks[wave][0];

  WaveState<D> ws;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) ws.acc[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
  ws.zacc = floatx4{0.f, 0.f, 0.f, 0.f};
  ws.m = neg_inf();
  ws.l = 0.0f;

  // query operands: bf16 for full-precision tiles; fp16 scaled by 2^-e (one e
  // per KV head, exact) for quantized ones -- in every column for INT1 tiles,
  // in the high columns only for INT4 / INT2 tiles, whose key-zero term takes
  // the per-group sums of the scaled query as two fp16 limbs (bQ: lanes 0-15,
  // k = group; high limb in the high columns, low limb in the low ones).
  bf16x8 bq[KB];
  half8 bqf[KB], bqk[KB];
  half4 bQ;
  float qall;   // sum of the scaled query over all channels, for this lane's head
  float scq = scale_log2;
  {
    const uint16_t *qrow = q + (size_t)b * q_bstride + ((size_t)h * G + hc) * D;
    float amax = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint4 r = *(const uint4 *)(qrow + kb * 32 + lq * 8);
      bq[kb] = __builtin_bit_cast(bf16x8, r);
      const uint16_t *e = (const uint16_t *)&r;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(bf16_to_f32(e[j])));
    }
    amax = max_x32(max_x16(amax));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    amax = fmaxf(amax, __shfl_xor(amax, 8));
    int qexp = 0;
    if (amax > 0.0f) frexpf(amax, &qexp);
    const half8 zero8 = {(half_t)0, (half_t)0, (half_t)0, (half_t)0, (half_t)0, (half_t)0, (half_t)0, (half_t)0};
    float gsum[KB];
    qall = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint16_t *e = (const uint16_t *)&bq[kb];
      float sum = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bqf[kb][j] = (half_t)ldexpf(bf16_to_f32(e[j]), -qexp);
        sum += (float)bqf[kb][j];
      }
      gsum[kb] = sum_x32(sum_x16(sum));   // the 32 channels of group kb, for this lane's head
      qall += gsum[kb];
      bqk[kb] = is_hi ? bqf[kb] : zero8;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float qs = k < KB ? gsum[k < KB ? k : 0] : 0.0f;
      const half_t qh = (half_t)qs;
      const half_t ql = (half_t)(qs - (float)qh);
      bQ[k] = lq == 0 ? (is_hi ? qh : ql) : (half_t)0;
    }
    scq = ldexpf(scale_log2, qexp);
  }

  // this wave's share: slice gi of NW*S of every part of the list
  const int NS = NW * S, gi = split * NW + wave;
  auto slice = [&](int n, int &a, int &z) {
    a = (int)((long long)n * gi / NS);
    z = (int)((long long)n * (gi + 1) / NS);
  };
  int fa, fz;
  slice(L.s0 + L.nC + L.nR, fa, fz);   // full-precision tiles (virtual order: sink, compact, recent)
  int qa[3], qz[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) slice(L.nQ[k], qa[k], qz[k]);
  auto quantized = [&]() __attribute__((always_inline)) {
    if (g.policy == QKV_POLICY_HQEKV) {
      tok_run_ql<D, 0, GP>(ws, c, bqk, bQ, scq, qa[0], qz[0]);
      tok_run_ql<D, 1, GP>(ws, c, bqk, bQ, scq, qa[1], qz[1]);
      tok_run_q1<D, GP>(ws, c, bqk, qall, scq, qa[2], qz[2]);
    }
  };
  // Opposite orders for the two waves that share a SIMD (w and w + 4 when
  // the waves are dealt round-robin, 2k and 2k + 1 when dealt in pairs): one
  // streams full-precision tiles while the other unpacks quantized ones.
  if (((wave & 1) ^ (wave >> 2)) & 1) {
    quantized();
    tok_run_bf16<D, GP>(ws, c, bq, scale_log2, fa, fz);
  } else {
    tok_run_bf16<D, GP>(ws, c, bq, scale_log2, fa, fz);
    quantized();
  }

  // ---- wave epilogue: value-zero term, then the low-limb rows 8+h onto rows h ----
  const float l_tot = sum_x32(sum_x16(ws.l));
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.acc[ct][i] += __shfl(ws.zacc[i], lq * 16 + (ct >> 1));
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.acc[ct][i] += __shfl_down(ws.acc[ct][i], 32);

  // ---- workgroup merge ----
  if (lq == 0 && col < G) {
    sm_m[wave][col] = ws.m;
    sm_l[wave][col] = l_tot;
  }
  // row r < 8 holds head r mod G; a channel tile's values are read from the
  // rows of its group's slot (r / G == group mod GP)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * lq + i;
    if (r < 8) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        if (r / G == ((ct >> 1) % GP)) sm_o[wave][r & (G - 1)][ct * 16 + col] = ws.acc[ct][i];
    }
  }
  __syncthreads();
  const size_t pbase = ((size_t)bh * S + split) * G;
  for (int it = threadIdx.x; it < G * D; it += blockDim.x) {
    const int hh = it / D, cc = it % D;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][hh]);
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (sm_m[w][hh] != neg_inf()) o += sm_o[w][hh][cc] * exp2f(sm_m[w][hh] - M);
    st.part_o[(pbase + hh) * D + cc] = o;
    if (cc == 0) {
      float l = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w)
        if (sm_m[w][hh] != neg_inf()) l += sm_l[w][hh] * exp2f(sm_m[w][hh] - M);
      st.part_ml[(pbase + hh) * 2 + 0] = M;
      st.part_ml[(pbase + hh) * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// merge: outputs per (sequence, KV head); per-token masses -> scores
// ---------------------------------------------------------------------------

// global (max, 1/sum) of each head of (sequence, KV head) bh over the
// splits, for the whole block: the splits' pairs are staged in LDS by all
// threads at once, then combined in split order by thread hh < G
template <int G>
__device__ inline void tok_split_stats(const TokGeom &g, const TokState &st, int bh, float *sM, float *sInvL) {
  __shared__ float2 sml[256];
  constexpr int PER = 256 / G;   // splits staged per round
  const int S = g.n_splits, tid = threadIdx.x;
  const float2 *ml = (const float2 *)st.part_ml + (size_t)bh * S * G;
  float m = neg_inf(), l = 0.0f;
  for (int r0 = 0; r0 < S; r0 += PER) {
    const int ns = min(S - r0, PER);
    if (tid < ns * G) sml[tid] = ml[(size_t)r0 * G + tid];
    __syncthreads();
    if (tid < G) {
      for (int s = 0; s < ns; ++s) {
        const float2 v = sml[s * G + tid];
        if (v.x == neg_inf()) continue;
        const float mn = fmaxf(m, v.x);
        l = (m == neg_inf() ? 0.0f : l * exp2f(m - mn)) + v.y * exp2f(v.x - mn);
        m = mn;
      }
    }
    __syncthreads();
  }
  if (tid < G) {
    sM[tid] = m;
    sInvL[tid] = 1.0f / l;
  }
  __syncthreads();
}

template <int G>
__global__ __launch_bounds__(256) void tok_merge_kernel(TokGeom g, TokState st, TokStep ts, float *__restrict__ out,
                                                        float *__restrict__ mass_out, int n_parts) {
  constexpr int CH = 8;
  const int S = g.n_splits, D = g.d;
  const int n_out_blocks = g.B * g.Hkv;
  if ((int)blockIdx.x < n_out_blocks) {
    const int bh = blockIdx.x;
    const int b = bh / g.Hkv, h = bh % g.Hkv;
    const float2 *ml = (const float2 *)st.part_ml + (size_t)bh * S * G;
    const float *po = st.part_o + (size_t)bh * S * G * D;
    merge_outputs<G, CH>(ml, po, S, D, out + ((size_t)b * g.Hq + (size_t)h * G) * D);
    return;
  }
  // masses: block `part` of n_parts per (sequence, KV head) strides over its
  // live tiles, four token slots per thread
  __shared__ float sM[G], sInvL[G];
  const int mb = blockIdx.x - n_out_blocks;
  const int bh = mb / n_parts, part = mb % n_parts;
  const TokList L = tok_list(g, st, ts, bh);   // issued ahead of the statistics wait
  const int n_live = min(L.count(), g.TILES);
  tok_split_stats<G>(g, st, bh, sM, sInvL);
  const int s0 = ((int)threadIdx.x % (TS / 4)) * 4;
  const bool list_order = g.omega > 1;   // routing every step: straight into the scores
  const bool need_pos = mass_out || !list_order;
  const int stride = n_parts * (256 * 4 / TS);
  // two tiles per trip, all loads first (the second index is clamped so its
  // loads stay valid; its results are dropped when it is past the list)
  for (int k = part * (256 * 4 / TS) + (int)threadIdx.x / (TS / 4); k < n_live; k += 2 * stride) {
    const int kt[2] = {k, min(k + stride, n_live - 1)};
    const bool live[2] = {true, k + stride < n_live};
    float4 r[2][G], acc[2];
    float ref[2][G];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float *rho = st.mrho + ((size_t)bh * (g.TILES + 1) + kt[u]) * G * TS + s0;
      const float *rf = st.mref + ((size_t)bh * (g.TILES + 1) + kt[u]) * G;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) r[u][hh] = *(const float4 *)(rho + hh * TS);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) ref[u][hh] = rf[hh];
      acc[u] = list_order ? *(const float4 *)(st.tacc + ((size_t)bh * g.TILES + kt[u]) * TS + s0)
                          : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!live[u]) continue;
      int lo, hi;
      tok_tile_range(g, st, ts, L, bh, kt[u], lo, hi);
      float w[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) w[hh] = exp2f(ref[u][hh] - sM[hh]);
      float *ap = (float *)&acc[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (s0 + e < lo || s0 + e >= hi) continue;
        float mass = 0.0f;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float v = ((const float *)&r[u][hh])[e] * w[hh] * sInvL[hh];
          if (!(v >= 1.17549435e-38f)) v = 0.0f;   // a head's weight below FLT_MIN counts as 0
          mass += v;
        }
        if (list_order && !ts.skip) ap[e] += mass;
        if (need_pos) {
          const int pos = tok_slot_pos<true>(g, st, ts, L, bh, kt[u], s0 + e);
          if (!list_order && !ts.skip) st.score[(size_t)bh * g.T + pos] += mass;
          if (mass_out) mass_out[(size_t)bh * g.T + pos] = mass;
        }
      }
      // list order: coalesced, and stable until the next route (which flushes first)
      if (list_order) *(float4 *)(st.tacc + ((size_t)bh * g.TILES + kt[u]) * TS + s0) = acc[u];
    }
  }
}

// pending list-order masses -> per-token scores (before anything reads the
// scores or a route changes the lists); the accumulators are cleared
__global__ __launch_bounds__(256) void tok_flush_kernel(TokGeom g, TokState st, TokStep ts, int n_chunks) {
  const int bh = blockIdx.x / n_chunks, chunk = blockIdx.x % n_chunks;
  const TokList L = tok_list(g, st, ts, bh);
  const int k = chunk * (256 / TS) + (int)threadIdx.x / TS;
  const int slot = threadIdx.x % TS;
  if (k >= L.count() || k >= g.TILES) return;
  float *acc = st.tacc + ((size_t)bh * g.TILES + k) * TS + slot;
  const float a = *acc;
  if (a == 0.0f) return;
  const int pos = tok_slot_pos<true>(g, st, ts, L, bh, k, slot);
  if (pos < 0) return;
  st.score[(size_t)bh * g.T + pos] += a;
  *acc = 0.0f;
}

namespace {
// live tiles per (sequence, KV head): at most the ranked tokens' tiles (one
// partial tile per tier) plus the sink and recent tiles
int tok_live_tiles(const TokGeom &g, const TokStep &ts) {
  const int ranked = g.policy == QKV_POLICY_HQEKV ? ts.rstart : ts.n_cmp;
  const int n = (g.n_sink > 0 ? 1 : 0) + (ranked + TS - 1) / TS + (g.policy == QKV_POLICY_HQEKV ? 4 : 0) +
                (ts.N > ts.rstart ? (ts.N - 1) / TS - ts.rstart / TS + 1 : 0);
  return n > g.TILES ? g.TILES : n;
}
}  // namespace

hipError_t tok_launch_flush(const TokGeom &g, const TokState &st, const TokStep &ts, hipStream_t s) {
  const int n_chunks = (tok_live_tiles(g, ts) * TS + 255) / 256;
  if (n_chunks < 1) return hipSuccess;
  hipLaunchKernelGGL(tok_flush_kernel, dim3(g.B * g.Hkv * n_chunks), dim3(256), 0, s, g, st, ts, n_chunks);
  return hipGetLastError();
}

hipError_t tok_launch_attend(const TokGeom &g, const TokState &st, const TokStep &ts, const uint16_t *q,
                             size_t q_bstride, float *out, float *mass_out, hipStream_t s, hipEvent_t ev_start,
                             hipEvent_t ev_stop) {
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)g.d));
  const int grid = g.B * g.Hkv * g.n_splits;
  hipError_t e;
  // the optional events are attached to the dispatch (kernel execution time);
  // four heads per KV head: value operands shared by channel-group pairs
  const bool pair = g.G == 4;
  const void *fn;
  if (g.att_waves == ATT_WAVES)
    fn = g.d == 128 ? (pair ? (const void *)tok_attend_kernel<128, 2, ATT_WAVES> : (const void *)tok_attend_kernel<128, 1, ATT_WAVES>)
                    : (pair ? (const void *)tok_attend_kernel<64, 2, ATT_WAVES> : (const void *)tok_attend_kernel<64, 1, ATT_WAVES>);
  else
    fn = g.d == 128 ? (pair ? (const void *)tok_attend_kernel<128, 2, ATT_WAVES / 2> : (const void *)tok_attend_kernel<128, 1, ATT_WAVES / 2>)
                    : (pair ? (const void *)tok_attend_kernel<64, 2, ATT_WAVES / 2> : (const void *)tok_attend_kernel<64, 1, ATT_WAVES / 2>);
  TokGeom ga = g;
  TokState sa = st;
  TokStep tsa = ts;
  const uint16_t *qa = q;
  size_t qb = q_bstride;
  float sl = scale_log2;
  void *args[] = {&ga, &sa, &tsa, &qa, &qb, &sl};
  e = hipExtLaunchKernel(fn, dim3(grid), dim3(64 * g.att_waves), args, 0, s, ev_start, ev_stop, 0);
  if (e != hipSuccess) return e;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (mass_out && (e = launch_clear(mass_out, (size_t)g.B * g.Hkv * g.T * sizeof(float), s)) != hipSuccess) return e;
  // mass blocks: about 2048 in all (a few per CU), at most one per 64 live tiles
  const int BH = g.B * g.Hkv;
  const int per_block = 256 * 4 / TS;
  int n_parts = (tok_live_tiles(g, ts) + per_block - 1) / per_block;
  const int want = (2048 + BH - 1) / BH;
  if (n_parts > want) n_parts = want;
  if (n_parts < 1) n_parts = 1;
  // a step outside the rolling score window adds nothing to the scores:
  // without a mass output its mass blocks are left out
  const dim3 mgrid(mass_out || !ts.skip ? BH + BH * n_parts : BH);
  if (g.G == 4)
    hipLaunchKernelGGL(tok_merge_kernel<4>, mgrid, dim3(256), 0, s, g, st, ts, out, mass_out, n_parts);
  else
    hipLaunchKernelGGL(tok_merge_kernel<8>, mgrid, dim3(256), 0, s, g, st, ts, out, mass_out, n_parts);
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

// copy token `pos` of the position pages into slot i of compact tiles `dst`
__device__ __forceinline__ void tok_copy_token(const TokGeom &g, const uint16_t *pages_bh, uint16_t *dst_bh, int pos,
                                               int i, int c0) {
  const int D = g.d;
  const uint16_t *sk = pages_bh + (size_t)(pos / TS) * 2 * TS * D;
  const uint16_t *sv = sk + TS * D;
  uint16_t *dk = dst_bh + (size_t)(i / TS) * 2 * TS * D;
  uint16_t *dv = dk + TS * D;
  const int ts_ = pos % TS, td = i % TS;
  *(uint4 *)(dk + k_tile_index(td, c0)) = *(const uint4 *)(sk + k_tile_index(ts_, c0));
#pragma unroll
  for (int j = 0; j < 8; ++j) dv[v_tile_index(td, c0 + j)] = sv[v_tile_index(ts_, c0 + j)];
}

// exclusive prefix of v over the threads of a workgroup of whole waves (in
// thread order), and the workgroup's total; wsum holds one int per wave
__device__ inline int block_excl_scan(int v, int *wsum, int &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int k = 0; k < nw; ++k) {
    const int x = wsum[k];
    if (k < w) base += x;
    tot += x;
  }
  __syncthreads();   // wsum may be reused
  total = tot;
  return base + inc - v;
}

__global__ __launch_bounds__(1024) void tok_route_h2o_kernel(TokGeom g, TokState st, int n_old, int a0, int a1,
                                                             int npow, int N) {
  extern __shared__ unsigned long long keys[];
  __shared__ int wsum[16];
  const int bh = blockIdx.x;
  const int b = bh / g.Hkv, h = bh % g.Hkv;
  const int n_new = a1 > a0 ? a1 - a0 : 0;
  const int n = n_old + n_new;
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
  int32_t *vic = st.victims + tb;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int pos = (int)(keys[i] & 0xffffffffull) - 1;
    st.tier[tb + pos] = i < keep ? T_FULL : T_EVICTED;
    if (i >= keep) vic[i - keep] = pos;
  }
  for (int i = n - keep + threadIdx.x; i < g.T; i += blockDim.x) vic[i] = -1;
  if (threadIdx.x == 0) {
    // the eviction record: candidates, kept, evicted and the relative score
    // gap across the cut (lowest kept minus highest evicted, over the larger)
    int32_t *ev = st.event + (size_t)bh * EV_WORDS;
    float m = __builtin_inff();
    if (keep > 0 && keep < n) {
      const float hi = __uint_as_float((uint32_t)(keys[keep - 1] >> 32)), lo = __uint_as_float((uint32_t)(keys[keep] >> 32));
      m = (hi - lo) / fmaxf(fmaxf(fabsf(hi), fabsf(lo)), 1.17549435e-38f);
    }
    for (int k = 0; k < EV_WORDS; ++k) ev[k] = 0;
    ev[EV_TOKENS] = N;
    ev[EV_CANDIDATES] = n;
    ev[EV_FULL] = keep;
    ev[EV_EVICTED] = n - keep;
    ev[EV_MARGIN_FULL] = __float_as_int(m);
    ev[EV_MARGIN_QUANT] = __float_as_int(__builtin_inff());
    ev[EV_MARGIN_MIN] = __float_as_int(m);
  }
  __syncthreads();   // tiers written; the sorted keys are not read below, their LDS is reused
  // The compact list keeps its slots: a kept token stays where it is, the
  // slot of an evicted one (and, while the list grows, slots n_old .. keep-1)
  // takes a kept newcomer, the k-th free slot in slot order the k-th
  // newcomer in position order, and only the newcomers are copied into the
  // compact tiles.
  int *freeslot = (int *)keys;   // keep <= npow entries
  int n_free = 0;
  {
    const int per = (keep + (int)blockDim.x - 1) / (int)blockDim.x;
    const int j0 = (int)threadIdx.x * per, j1 = min(keep, j0 + per);
    auto is_free = [&](int j) { return j >= n_old || st.tier[tb + cpos[j]] == T_EVICTED; };
    int cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += is_free(j) ? 1 : 0;
    int r = block_excl_scan(cnt, wsum, n_free);
    for (int j = j0; j < j1; ++j)
      if (is_free(j)) freeslot[r++] = j;
  }
  __syncthreads();
  {
    const int per = (n_new + (int)blockDim.x - 1) / (int)blockDim.x;
    const int e0 = (int)threadIdx.x * per, e1 = min(n_new, e0 + per);
    auto kept_new = [&](int e) { return st.tier[tb + a0 + e] == T_FULL; };
    int cnt = 0;
    for (int e = e0; e < e1; ++e) cnt += kept_new(e) ? 1 : 0;
    int total;
    int r = block_excl_scan(cnt, wsum, total);
    for (int e = e0; e < e1; ++e) {
      if (!kept_new(e)) continue;
      if (r < n_free) cpos[freeslot[r]] = a0 + e;
      else st.status[0] = QKV_ECAPACITY;   // more newcomers than free slots: cannot happen
      ++r;
    }
  }
  __syncthreads();
  const int chunks = g.d / 8;
  const uint16_t *pages_bh = st.pages + tok_page_offset(g, b, h, 0);
  uint16_t *cpages_bh = st.cpages + tok_cpage_offset(g, b, h, 0);
  for (int it = threadIdx.x; it < n_free * chunks; it += blockDim.x) {
    const int slot = freeslot[it / chunks];
    tok_copy_token(g, pages_bh, cpages_bh, cpos[slot], slot, (it % chunks) * 8);
  }
}

hipError_t tok_launch_route(const TokGeom &g, const TokState &st, const TokStep &ts, int a0, int a1, int n_cand,
                            hipStream_t s) {
  int npow = 1;
  while (npow < n_cand) npow <<= 1;
  if (npow > ROUTE_SORT_MAX) return hipErrorInvalidValue;   // 8-byte keys, at most 128 KB of LDS
  hipLaunchKernelGGL(tok_route_h2o_kernel, dim3(g.B * g.Hkv), dim3(1024), npow * sizeof(unsigned long long), s, g,
                     st, ts.n_cmp, a0, a1, npow, ts.N);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// HqeKV assignment event, one workgroup of 1024 threads per (sequence, KV head)
// ---------------------------------------------------------------------------

__device__ __forceinline__ int hq_level(uint8_t t) {
  switch (t) {
    case T_INT4: return HQ_INT4;
    case T_QUANT: return HQ_INT2;
    case T_INT1: return HQ_INT1;
    case T_EVICTED: return HQ_EVICT;
    default: return HQ_BF16;   // ranked or not-yet-ranked full precision
  }
}
__device__ __forceinline__ uint8_t hq_code(int level) {
  switch (level) {
    case HQ_INT4: return T_INT4;
    case HQ_INT2: return T_QUANT;
    case HQ_INT1: return T_INT1;
    case HQ_EVICT: return T_EVICTED;
    default: return T_FULL;
  }
}

// Record of a quantized token (canonical per-token packing, element c of a
// b-bit code stream at bit b*(c mod (8/b)) of byte c*b/8):
//   [K codes, d/2 B][V codes, d/2 B][K params d/32 x (s, z) fp16][V params]
// INT1 keeps (mean, std) fp16 in the first params pair.
__device__ __forceinline__ int rec_kc(const TokGeom &) { return 0; }
__device__ __forceinline__ int rec_vc(const TokGeom &g) { return g.d / 2; }
__device__ __forceinline__ int rec_kp(const TokGeom &g) { return g.d; }
__device__ __forceinline__ int rec_vp(const TokGeom &g) { return g.d + (g.d / 32) * 4; }

// Re-quantization of the tokens an assignment event moved to a quantized
// tier.  Each token row (keys, values) is handled by 16 lanes, lane i owning
// channels CPL*i .. CPL*i + CPL-1 (CPL = d/16), so a wave rebuilds two tokens
// at a time and the whole grid works through the changed tokens of every
// (sequence, KV head).  The current values are read first (float32: the bf16
// page, or the dequantized record of the previous level), then the record is
// written in canonical per-token packing.
template <int D>
__global__ __launch_bounds__(256) void hq_requant_kernel(TokGeom g, TokState st, int elig_end) {
  constexpr int CPL = D / 16;                // channels per lane
  constexpr int LPG = 32 / CPL;              // lanes per 32-channel group
  const int bh = blockIdx.y;
  const int b = bh / g.Hkv, h = bh % g.Hkv;
  const size_t tb = (size_t)bh * g.T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp16 = lane >> 4, li = lane & 15;  // 16-lane group: token grp16/2, row grp16%2
  const int w = grp16 & 1;
  const int c0 = CPL * li;
  const int base = (blockIdx.x * 4 + wave) * 64;
  const int mypos = base + lane;
  const bool pending = mypos < elig_end && st.hqold[tb + mypos] != 0;
  unsigned long long todo = __ballot(pending);
  while (todo) {
    // two tokens per pass (the second may repeat the first when one is left)
    const int l0 = __builtin_ctzll(todo);
    todo &= todo - 1;
    const int l1 = todo ? __builtin_ctzll(todo) : l0;
    if (todo) todo &= todo - 1;
    const int pos = base + ((grp16 >> 1) ? l1 : l0);
    const int old = (int)st.hqold[tb + pos] - 1;
    const int lvl = hq_level(st.tier[tb + pos]);
    // ---- current values of this lane's channels ----
    float x[CPL];
    uint8_t *rec = st.qrec + (tb + pos) * g.rec_bytes;
    if (old == HQ_BF16) {
      const uint16_t *kt = st.pages + tok_page_offset(g, b, h, pos / TS);
      const int t = pos % TS;
      if (w == 0) {
        const uint16_t *src = kt + k_tile_index(t, c0);   // CPL consecutive channels
#pragma unroll
        for (int e = 0; e < CPL; ++e) x[e] = bf16_to_f32(src[e]);
      } else {
#pragma unroll
        for (int e = 0; e < CPL; ++e) x[e] = bf16_to_f32(kt[TS * D + v_tile_index(t, c0 + e)]);
      }
    } else {
      const uint8_t *codes = rec + (w ? rec_vc(g) : rec_kc(g));
      const uint16_t *par = (const uint16_t *)(rec + (w ? rec_vp(g) : rec_kp(g)));
      if (old == HQ_INT1) {
        const uint32_t bits = codes[c0 >> 3] >> (c0 & 7);
        const float m = (float)__builtin_bit_cast(half_t, par[0]), sd = (float)__builtin_bit_cast(half_t, par[1]);
#pragma unroll
        for (int e = 0; e < CPL; ++e) x[e] = __builtin_fmaf(((bits >> e) & 1u) ? KAPPA1 : -KAPPA1, sd, m);
      } else {
        const int bits = old == HQ_INT4 ? 4 : 2;
        uint32_t word = 0u;   // the lane's CPL codes, bits * CPL <= 32
#pragma unroll
        for (int k = 0; k < CPL * 4 / 8; ++k)
          if (k * 8 < bits * CPL) word |= (uint32_t)codes[c0 * bits / 8 + k] << (8 * k);
        const int gi = c0 >> 5;
        const float sc = (float)__builtin_bit_cast(half_t, par[2 * gi]);
        const float zc = (float)__builtin_bit_cast(half_t, par[2 * gi + 1]);
#pragma unroll
        for (int e = 0; e < CPL; ++e)
          x[e] = __builtin_fmaf((float)((word >> (bits * e)) & ((1u << bits) - 1u)), sc, zc);
      }
    }
    __builtin_amdgcn_wave_barrier();
    // ---- new record (all reads of this token are done) ----
    uint8_t *codes = rec + (w ? rec_vc(g) : rec_kc(g));
    uint16_t *par = (uint16_t *)(rec + (w ? rec_vp(g) : rec_kp(g)));
    if (lvl == HQ_INT1) {
      // mean and population deviation in float64 over the row, rounded to float32, then fp16
      double sum = 0.0;
#pragma unroll
      for (int e = 0; e < CPL; ++e) sum += (double)x[e];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off);
      const float m32 = f64_to_f32_kept(sum / D);
      double ss = 0.0;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        const double dv = (double)x[e] - (double)m32;
        ss += dv * dv;
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) ss += __shfl_xor(ss, off);
      const float sd32 = f64_to_f32_kept(sqrt(ss / D));
      const half_t m16 = (half_t)m32, sd16 = (half_t)sd32;
      if (!isfinite((float)m16) || !isfinite((float)sd16)) st.status[0] = QKV_ERANGE;
      uint32_t cb = 0u;   // bit c of the row: x_c > mean
#pragma unroll
      for (int e = 0; e < CPL; ++e) cb |= ((double)x[e] > (double)m32 ? 1u : 0u) << e;
      if (CPL == 8) {
        codes[c0 >> 3] = (uint8_t)cb;
      } else {   // four channels per lane: lane pairs share a byte
        const uint32_t other = __shfl_xor(cb, 1);
        if ((li & 1) == 0) codes[c0 >> 3] = (uint8_t)(cb | (other << 4));
      }
      if (li == 0) {
        par[0] = __builtin_bit_cast(uint16_t, m16);
        par[1] = __builtin_bit_cast(uint16_t, sd16);
      }
    } else {
      const int bits = lvl == HQ_INT4 ? 4 : 2;
      const float levels = (float)((1 << bits) - 1);
      float mn = x[0], mx = x[0];
#pragma unroll
      for (int e = 1; e < CPL; ++e) {
        mn = min_nan(mn, x[e]);
        mx = max_nan(mx, x[e]);
      }
#pragma unroll
      for (int off = 1; off < LPG; off <<= 1) {
        mn = min_nan(mn, __shfl_xor(mn, off));
        mx = max_nan(mx, __shfl_xor(mx, off));
      }
      const half_t s16 = (half_t)((mx - mn) / levels);
      const half_t z16 = (half_t)mn;
      if (!isfinite((float)s16) || !isfinite((float)z16)) st.status[0] = QKV_ERANGE;
      uint32_t word = 0u;
#pragma unroll
      for (int e = 0; e < CPL; ++e) word |= quant_code(x[e], s16, z16, levels) << (bits * e);
#pragma unroll
      for (int k = 0; k < CPL * 4 / 8; ++k)
        if (k * 8 < bits * CPL) codes[c0 * bits / 8 + k] = (uint8_t)(word >> (8 * k));
      if ((li % LPG) == 0) {
        const int gi = c0 >> 5;
        par[2 * gi] = __builtin_bit_cast(uint16_t, s16);
        par[2 * gi + 1] = __builtin_bit_cast(uint16_t, z16);
      }
    }
    if (li == 0 && w == 0) st.hqold[tb + pos] = 0;
  }
}

constexpr uint32_t HQ_KEY_NONE = 0xffffffffu;   // key slot of a token that is not ranked
constexpr int HQ_TIE_CAP = 1024;                 // tied tokens at a cut resolved from one LDS list

// One radix digit of every active cut, chosen by the whole block: count(j, b)
// is the number of cut j's candidate keys whose digit is b (NB bins, a higher
// bin ranking first).  The bin holding the key of rank rem[j] (0 = highest)
// is or-ed into pref[j] at bit sh; rem[j] becomes the rank inside that bin
// and bin_n[j] its key count.
template <int NB, typename CountF>
__device__ void hq_choose_digit(CountF count, int sh, uint32_t *pref, int *rem, int *bin_n, const bool *active,
                                int (*wtot)[4]) {
  constexpr int BPT = NB >= 1024 ? NB / 1024 : 1;   // bins per thread, thread order = descending bins
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool has = tid * BPT < NB;
  int r[4], s[4], incl[4];
  bool act[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    act[j] = active[j];
    r[j] = rem[j];
    s[j] = 0;
    if (act[j] && has)
      for (int i = 0; i < BPT; ++i) s[j] += count(j, NB - 1 - (tid * BPT + i));
    int v = s[j];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(v, off);
      if (lane >= off) v += t;
    }
    incl[j] = v;
    if (lane == 63) wtot[wave][j] = v;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    for (int w = 0; w < wave; ++w) incl[j] += wtot[w][j];
    const int excl = incl[j] - s[j];
    if (act[j] && s[j] > 0 && excl <= r[j] && r[j] < incl[j]) {
      int acc = excl;
      for (int i = 0; i < BPT; ++i) {
        const int b = NB - 1 - (tid * BPT + i);
        const int c = count(j, b);
        if (acc + c > r[j]) {
          pref[j] |= (uint32_t)b << sh;
          rem[j] = r[j] - acc;
          bin_n[j] = c;
          break;
        }
        acc += c;
      }
    }
  }
  __syncthreads();
}

// Chunk targets of an assignment event (HqeKV notes 3.3, implementation
// note): chunk c holds positions [c*C, (c+1)*C) below elig_end and its metric
// is the mean of its ranked tokens' keys (the fp32 joint metric), summed in
// fp64 in position order; chunks are ordered by (mean desc, index desc), rank
// r takes the tier of the cumulative chunk counts c0..c3 (the rest evicted),
// and ranks 0 and 1 are BF16 whatever the counts.  ctgt[c] is left unset for
// a chunk without a ranked token (no token reads it).
__device__ void hq_rank_chunks(const TokGeom &g, const uint32_t *keys, int elig_end, int c0, int c1, int c2, int c3,
                               uint8_t *ctgt) {
  __shared__ double km[HQ_CHUNK_MAX];
  __shared__ int ki[HQ_CHUNK_MAX];
  const int C = g.chunk, tid = threadIdx.x, nthr = blockDim.x;
  const int nC = (elig_end + C - 1) / C;   // at most HQ_CHUNK_MAX (checked at create)
  int npow = 1;
  while (npow < nC) npow <<= 1;
  for (int c = tid; c < npow; c += nthr) {
    double sum = 0.0;
    int n = 0;
    if (c < nC) {
      const int p1 = min((c + 1) * C, elig_end);
#pragma unroll 8
      for (int p = c * C; p < p1; ++p) {
        const uint32_t k = keys[p];
        if (k != HQ_KEY_NONE) {
          sum += (double)__uint_as_float(k);
          ++n;
        }
      }
    }
    km[c] = n > 0 ? sum / n : -1.0;   // chunks without a ranked token sort last
    ki[c] = c;
  }
  __syncthreads();
  for (int k = 2; k <= npow; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < npow; i += nthr) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const double a = km[i], b = km[ixj];
          const int ia = ki[i], ib = ki[ixj];
          const bool a_first = a > b || (a == b && ia > ib);
          if (a_first != ((i & k) == 0)) {
            km[i] = b;
            km[ixj] = a;
            ki[i] = ib;
            ki[ixj] = ia;
          }
        }
      }
      __syncthreads();
    }
  const int cum0 = c0, cum1 = c0 + c1, cum2 = cum1 + c2, cum3 = cum2 + c3;
  for (int r = tid; r < nC; r += nthr) {
    if (km[r] < 0.0) continue;
    const int t = (r < 2 || r < cum0) ? HQ_BF16 : r < cum1 ? 1 : r < cum2 ? 2 : r < cum3 ? 3 : HQ_EVICT;
    ctgt[ki[r]] = (uint8_t)t;
  }
  __syncthreads();
}

// Assignment event of one (sequence, KV head) (HqeKV section 3.3 with the
// shares of its tier table): the joint metric (accumulated attention x value
// range) ranks every token appended before the previous event; the cuts at
// ranks cum[j] = c0 + ... + cj are found by radix selection on the metric's
// float bits (ties: the newer token first), each token moves down to its
// target tier if that is lower (a token that moves to a quantized tier
// keeps its previous level in hqold until hq_requant_kernel has rebuilt its
// record), and the per-tier position lists are rebuilt in position order.
__global__ __launch_bounds__(1024) void hq_event_kernel(TokGeom g, TokState st, int N, int elig_end, int c0, int c1,
                                                        int c2, int c3) {
  const int bh = blockIdx.x;
  const size_t tb = (size_t)bh * g.T;
  uint32_t *keys = st.hqkey + (size_t)bh * hq_key_stride(g);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n_waves = blockDim.x >> 6;
  const int nthr = blockDim.x;
  __shared__ uint32_t hist[4][2048];
  __shared__ int wtot[16][4];
  __shared__ uint32_t pref[4], ppref[4];
  __shared__ int rem[4], prem[4], bin_n[4], pbin_n[4], n_tie[4], pcut[4];
  __shared__ bool active[4], big[4];
  __shared__ int s_E;
  __shared__ unsigned long long thr[4];
  __shared__ int tie_pos[4][HQ_TIE_CAP];
  __shared__ int run[5];                   // list lengths: BF16, INT4, INT2, INT1, evicted at this event
  __shared__ unsigned long long below[4];
  __shared__ int n_moved, n_evicted;

  // ---- keys: metric bits of every eligible token, four positions per thread ----
  if (tid == 0) s_E = 0;
  __syncthreads();
  {
    int cnt = 0;
    for (int p0 = 4 * tid; p0 < elig_end; p0 += 4 * nthr) {
      uint32_t k4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = p0 + e;
        k4[e] = HQ_KEY_NONE;
        if (pos < elig_end) {
          const uint8_t t = st.tier[tb + pos];
          const float metric = st.score[tb + pos] * st.vrange[tb + pos];
          if (t != T_EVICTED && t != T_EMPTY) {
            const uint32_t k = __float_as_uint(metric);
            k4[e] = k == HQ_KEY_NONE ? k - 1u : k;   // (an all-ones NaN keeps its place among NaNs)
            ++cnt;
          }
        }
      }
      *(u32x4v *)(keys + p0) = u32x4v{k4[0], k4[1], k4[2], k4[3]};
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    if (lane == 0) atomicAdd(&s_E, cnt);
  }
  __syncthreads();
  const long long E = s_E;
  const long long cum[4] = {c0, (long long)c0 + c1, (long long)c0 + c1 + c2, (long long)c0 + c1 + c2 + c3};
  if (tid < 4) {
    const long long r = cum[tid] - 1;
    active[tid] = r >= 0 && r < E;
    rem[tid] = active[tid] ? (int)r : 0;
    pref[tid] = 0u;
    ppref[tid] = 0u;
    bin_n[tid] = 0;
    n_tie[tid] = 0;
    pcut[tid] = -1;
  }
  // every key of the block's positions, 16 per thread per round (loads first)
  auto for_keys = [&](auto fn) {
    for (int p0 = 4 * tid; p0 < elig_end; p0 += 16 * nthr) {
      u32x4v k4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = p0 + u * 4 * nthr;
        k4[u] = q < elig_end ? *(const u32x4v *)(keys + q) : u32x4v{HQ_KEY_NONE, HQ_KEY_NONE, HQ_KEY_NONE, HQ_KEY_NONE};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) fn(k4[u][e], p0 + u * 4 * nthr + e);
    }
  };
  auto clear_hist = [&]() {
    for (int i = tid; i < 4 * 2048; i += nthr) (&hist[0][0])[i] = 0u;
    __syncthreads();
  };
  __shared__ uint8_t ctgt[HQ_CHUNK_MAX];
  if (g.chunk > 0) {
    hq_rank_chunks(g, keys, elig_end, c0, c1, c2, c3, ctgt);
  } else {
  // ---- digit [31..21]: one histogram for all cuts (four copies against contention) ----
  clear_hist();
  for_keys([&](uint32_t k, int) {
    if (k != HQ_KEY_NONE) atomicAdd(&hist[wave & 3][k >> 21], 1u);
  });
  __syncthreads();
  hq_choose_digit<2048>([&](int, int b) { return (int)(hist[0][b] + hist[1][b] + hist[2][b] + hist[3][b]); }, 21,
                        pref, rem, bin_n, active, wtot);
  // ---- digit [20..10], then [9..0], per cut among the keys of its prefix ----
  clear_hist();
  for_keys([&](uint32_t k, int) {
    if (k == HQ_KEY_NONE) return;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (active[j] && (k >> 21) == (pref[j] >> 21)) atomicAdd(&hist[j][(k >> 10) & 2047u], 1u);
  });
  __syncthreads();
  hq_choose_digit<2048>([&](int j, int b) { return (int)hist[j][b]; }, 10, pref, rem, bin_n, active, wtot);
  clear_hist();
  for_keys([&](uint32_t k, int) {
    if (k == HQ_KEY_NONE) return;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (active[j] && (k >> 10) == (pref[j] >> 10)) atomicAdd(&hist[j][k & 1023u], 1u);
  });
  __syncthreads();
  hq_choose_digit<1024>([&](int j, int b) { return (int)hist[j][b]; }, 0, pref, rem, bin_n, active, wtot);
  // ---- ties at each cut's metric: the newer token ranks first ----
  if (tid < 4) big[tid] = active[tid] && bin_n[tid] > HQ_TIE_CAP;
  __syncthreads();
  for_keys([&](uint32_t k, int pos) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (active[j] && !big[j] && k == pref[j]) {
        const int i = atomicAdd(&n_tie[j], 1);
        if (i < HQ_TIE_CAP) tie_pos[j][i] = pos;
      }
  });
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (!active[j] || big[j]) continue;
    const int n = min(n_tie[j], HQ_TIE_CAP);
    for (int i = tid; i < n; i += nthr) {
      const int p = tie_pos[j][i];
      int r = 0;
      for (int q = 0; q < n; ++q) r += tie_pos[j][q] > p ? 1 : 0;
      if (r == rem[j]) pcut[j] = p;
    }
  }
  if (big[0] || big[1] || big[2] || big[3]) {
    // many equal metrics: radix selection on the positions of the tied tokens
    if (tid < 4) {
      prem[tid] = rem[tid];
      ppref[tid] = 0u;
    }
    __syncthreads();
    const int shs[3] = {20, 9, 0};
    for (int d = 0; d < 3; ++d) {
      const int sh = shs[d], top = d == 0 ? 31 : shs[d - 1];
      const uint32_t dmask = d == 2 ? 511u : 2047u;
      clear_hist();
      for_keys([&](uint32_t k, int pos) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (big[j] && k == pref[j] && ((uint32_t)pos >> top) == (ppref[j] >> top))
            atomicAdd(&hist[j][((uint32_t)pos >> sh) & dmask], 1u);
      });
      __syncthreads();
      if (d < 2)
        hq_choose_digit<2048>([&](int j, int b) { return (int)hist[j][b]; }, sh, ppref, prem, pbin_n, big, wtot);
      else
        hq_choose_digit<512>([&](int j, int b) { return (int)hist[j][b]; }, sh, ppref, prem, pbin_n, big, wtot);
    }
    if (tid < 4 && big[tid]) pcut[tid] = (int)ppref[tid];
  }
  }   // per-token ranking
  __syncthreads();
  if (tid < 4) {
    // keys >= thr[j] have rank < cum[j]: all of them when cum[j] >= E, none when cum[j] <= 0
    const long long c = cum[tid];
    thr[tid] = c >= E ? 0ull
             : (c <= 0 ? ~0ull : (((unsigned long long)pref[tid] << 32) | (unsigned)(pcut[tid] + 1)));
    st.cuts[bh * 4 + tid] = thr[tid];
    run[tid] = 0;
    below[tid] = 0ull;
  }
  if (tid == 0) {
    run[4] = 0;
    n_moved = 0;
    n_evicted = 0;
  }
  __syncthreads();
  // ---- the key just below each cut (the best-ranked one the cut drops), for
  // the event record's margins (per-token ranking only) ----
  if (g.chunk == 0) {
    unsigned long long lb[4] = {0ull, 0ull, 0ull, 0ull};
    for_keys([&](uint32_t k, int pos) {
      if (k == HQ_KEY_NONE) return;
      const unsigned long long key = ((unsigned long long)k << 32) | (unsigned)(pos + 1);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (key < thr[j] && key > lb[j]) lb[j] = key;
    });
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      unsigned long long v = lb[j];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const unsigned long long o = ((unsigned long long)(uint32_t)__shfl_xor((int)(v >> 32), off) << 32) |
                                     (uint32_t)__shfl_xor((int)(uint32_t)v, off);
        v = o > v ? o : v;
      }
      if (lane == 0 && v != 0ull) atomicMax(&below[j], v);
    }
  }
  __syncthreads();
  // ---- targets (downgrade only) and the per-tier position lists, in position order ----
  __shared__ int wsum[16][5];
  int my_moved = 0, my_evicted = 0;
  for (int base = 0; base < elig_end; base += 4 * nthr) {
    const int p0 = base + 4 * tid;
    int lv[4], cnt[5] = {0, 0, 0, 0, 0};
    bool gone[4] = {false, false, false, false};   // evicted at this event
    const u32x4v k4 = p0 < elig_end ? *(const u32x4v *)(keys + p0)
                                    : u32x4v{HQ_KEY_NONE, HQ_KEY_NONE, HQ_KEY_NONE, HQ_KEY_NONE};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pos = p0 + e;
      lv[e] = HQ_EVICT;
      if (pos >= elig_end) continue;
      const int old = hq_level(st.tier[tb + pos]);
      lv[e] = old;
      if (k4[e] != HQ_KEY_NONE) {
        const unsigned long long key = ((unsigned long long)k4[e] << 32) | (unsigned)(pos + 1);
        int target = 0;
        if (g.chunk > 0) {
          target = ctgt[pos / g.chunk];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (!(cum[j] >= E ? true : (cum[j] > 0 && key >= thr[j]))) ++target;
        }
        if (target > old) {
          st.tier[tb + pos] = hq_code(target);
          if (target != HQ_EVICT) st.hqold[tb + pos] = (uint8_t)(old + 1);
          lv[e] = target;
          ++my_moved;
          if (target == HQ_EVICT) {
            ++my_evicted;
            gone[e] = true;
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (lv[e] < 4) ++cnt[lv[e]];
      if (gone[e]) ++cnt[4];
    }
    int incl[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      int v = cnt[k];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off);
        if (lane >= off) v += t;
      }
      incl[k] = v;
      if (lane == 63) wsum[wave][k] = v;
    }
    __syncthreads();
    int off[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      off[k] = run[k] + incl[k] - cnt[k];
      for (int w2 = 0; w2 < wave; ++w2) off[k] += wsum[w2][k];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (gone[e]) st.victims[tb + off[4]++] = p0 + e;   // position order
      const int l = lv[e];
      if (l >= 4) continue;
      const int o = l == 0 ? off[0]++ : l == 1 ? off[1]++ : l == 2 ? off[2]++ : off[3]++;
      if (l == HQ_BF16)
        st.cpos[(size_t)bh * g.NCT * TS + o] = p0 + e;
      else
        st.qpos[l - 1][(size_t)bh * g.NCT * TS + o] = p0 + e;
    }
    __syncthreads();
    if (tid < 5) {
      int t = 0;
      for (int w2 = 0; w2 < n_waves; ++w2) t += wsum[w2][tid];
      run[tid] += t;
    }
    __syncthreads();
  }
  if (tid < 4) st.cnt[bh * 4 + tid] = run[tid];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    my_moved += __shfl_xor(my_moved, off);
    my_evicted += __shfl_xor(my_evicted, off);
  }
  if (lane == 0) {
    atomicAdd(&n_moved, my_moved);
    atomicAdd(&n_evicted, my_evicted);
  }
  __syncthreads();
  // the victims list ends at -1; the event record (layout in the header)
  for (int i = run[4] + tid; i < g.T; i += nthr) st.victims[tb + i] = -1;
  if (tid == 0) {
    int32_t *ev = st.event + (size_t)bh * EV_WORDS;
    float m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m[j] = __builtin_inff();
      if (g.chunk == 0 && cum[j] > 0 && cum[j] < E) {
        const float hi = __uint_as_float((uint32_t)(thr[j] >> 32)), lo = __uint_as_float((uint32_t)(below[j] >> 32));
        m[j] = (hi - lo) / fmaxf(fmaxf(fabsf(hi), fabsf(lo)), 1.17549435e-38f);
      }
    }
    for (int k = 0; k < EV_WORDS; ++k) ev[k] = 0;
    ev[EV_TOKENS] = N;
    ev[EV_CANDIDATES] = (int)E;
    ev[EV_FULL] = run[0];
    ev[EV_QUANT] = run[2];
    ev[EV_EVICTED] = n_evicted;
    ev[EV_DEMOTED] = n_moved;
    ev[EV_HQ_REQUANTIZED] = n_moved - n_evicted;
    ev[EV_HQ_INT4] = run[1];
    ev[EV_HQ_INT1] = run[3];
    ev[EV_MARGIN_FULL] = __float_as_int(m[0]);
    ev[EV_MARGIN_QUANT] = __float_as_int(m[1]);
    ev[EV_HQ_MARGIN_INT1] = __float_as_int(m[2]);
    ev[EV_HQ_MARGIN_EVICT] = __float_as_int(m[3]);
    ev[EV_MARGIN_MIN] = __float_as_int(fminf(fminf(m[0], m[1]), fminf(m[2], m[3])));
  }
}

__device__ __forceinline__ size_t tb_of(const TokGeom &g, int bh) { return (size_t)bh * g.T; }

// The records (canonical per-token packing, see the re-quantization kernel)
// of a compact tile's 16 token slots, staged in LDS by one wave with 16-byte
// loads; slots past the tier's count read as zeros.
template <int D>
__device__ __forceinline__ void hq_stage_records(const uint8_t *rec0, const int32_t *qpos, int tile, int nq, int lane,
                                                 uint8_t *lds) {
  constexpr int R = D + (D / 32) * 8, NCH = R / 16;
  for (int i = lane; i < TS * NCH; i += 64) {
    const int tk = i / NCH, part = i - tk * NCH;
    const int sl = tile * TS + tk;
    u32x4v v = {0u, 0u, 0u, 0u};
    if (sl < nq) v = *(const u32x4v *)(rec0 + (size_t)qpos[sl] * R + part * 16);
    *(u32x4v *)(lds + tk * R + part * 16) = v;
  }
  wave_lds_sync();
}

template <int CW>
__device__ __forceinline__ void store_words(uint8_t *dst, const uint32_t (&w)[CW]) {
  if constexpr (CW == 4) {
    *(u32x4v *)dst = u32x4v{w[0], w[1], w[2], w[3]};
  } else if constexpr (CW == 2) {
    *(u32x2v *)dst = u32x2v{w[0], w[1]};
  } else {
#pragma unroll
    for (int k = 0; k < CW; ++k) ((uint32_t *)dst)[k] = w[k];
  }
}

// INT4 / INT2 tiles of one (sequence, KV head) in operand order (QL), one
// wave per tile (tiles gw, gw + n_gw, ...)
template <int D, int F>
__device__ void hq_gather_ql(const TokGeom &g, const TokState &st, int bh, uint8_t *lds, int gw, int n_gw, int lane) {
  using Q = QL<D, F>;
  constexpr int R = D + (D / 32) * 8;
  constexpr int bits = F == 0 ? 4 : 2;
  constexpr uint32_t mask = (1u << bits) - 1u;
  const int nq = st.cnt[bh * 4 + 1 + F];
  const int ntiles = (nq + TS - 1) / TS;
  uint8_t *tiles = st.qtiles[F] + (size_t)bh * g.NCT * Q::BYTES;
  const int32_t *qpos = st.qpos[F] + (size_t)bh * g.NCT * TS;
  const uint8_t *rec0 = st.qrec + tb_of(g, bh) * R;
  const int t = lane & 15, lq = lane >> 4;
  for (int tile = gw; tile < ntiles; tile += n_gw) {
    hq_stage_records<D>(rec0, qpos, tile, nq, lane, lds);
    uint8_t *T = tiles + (size_t)tile * Q::BYTES;
    // keys: token slot t, channels kb*32 + 8*lq + e (one code word per k-block)
    uint32_t kw[Q::CW], vw[Q::CW];
#pragma unroll
    for (int w = 0; w < Q::CW; ++w) kw[w] = vw[w] = 0u;
#pragma unroll
    for (int kb = 0; kb < Q::KB; ++kb) {
      const uint32_t x = F == 0 ? *(const uint32_t *)(lds + t * R + 16 * kb + 4 * lq)
                                : (uint32_t) * (const uint16_t *)(lds + t * R + 8 * kb + 2 * lq);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int dw, bit;
        ql_kslot<F>(kb, e, dw, bit);
        kw[dw] |= ((x >> (bits * e)) & mask) << bit;
      }
    }
    // values: channel ct*16 + t of token slots 4*lq + tt
    const int vsh = bits * (t % (8 / bits)), vby = t * bits / 8;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const uint8_t *vr = lds + (4 * lq + tt) * R + D / 2 + vby;
#pragma unroll
      for (int ct = 0; ct < Q::CT; ++ct) {
        int dw, bit;
        ql_vslot<F>(ct, tt, dw, bit);
        vw[dw] |= (((uint32_t)vr[ct * 16 * bits / 8] >> vsh) & mask) << bit;
      }
    }
    store_words<Q::CW>(T + lane * 4 * Q::CW, kw);
    store_words<Q::CW>(T + Q::VC + lane * 4 * Q::CW, vw);
    // params of token slot t, written by the lanes of row lq == 0
    if (lq == 0) {
      const uint16_t *par = (const uint16_t *)(lds + t * R + D);
      uint16_t *ksc = (uint16_t *)(T + Q::KS), *kzr = (uint16_t *)(T + Q::KZ);
      uint16_t *vsc = (uint16_t *)(T + Q::VS), *vzr = (uint16_t *)(T + Q::VZ);
#pragma unroll
      for (int gi = 0; gi < Q::NG; ++gi) {
        ksc[gi * TS + t] = par[2 * gi];
        kzr[t * Q::NG + gi] = par[2 * gi + 1];
        vsc[gi * TS + t] = par[2 * Q::NG + 2 * gi];
        vzr[gi * TS + t] = par[2 * Q::NG + 2 * gi + 1];
      }
    }
    wave_lds_sync();   // the next tile's records overwrite these
  }
}

// INT1 tiles of one (sequence, KV head) (Q1 layout), one wave per tile
template <int D>
__device__ void hq_gather_q1(const TokGeom &g, const TokState &st, int bh, uint8_t *lds, int gw, int n_gw, int lane) {
  using Q = Q1<D>;
  constexpr int R = D + (D / 32) * 8;
  const int nq = st.cnt[bh * 4 + 3];
  const int ntiles = (nq + TS - 1) / TS;
  uint8_t *tiles = st.qtiles[2] + (size_t)bh * g.NCT * Q::BYTES;
  const int32_t *qpos = st.qpos[2] + (size_t)bh * g.NCT * TS;
  const uint8_t *rec0 = st.qrec + tb_of(g, bh) * R;
  const int t = lane & 15, lq = lane >> 4;
  for (int tile = gw; tile < ntiles; tile += n_gw) {
    hq_stage_records<D>(rec0, qpos, tile, nq, lane, lds);
    uint8_t *T = tiles + (size_t)tile * Q::BYTES;
    uint32_t kw = 0u, vw = 0u;
#pragma unroll
    for (int kb = 0; kb < Q::KB; ++kb) {
      const uint32_t x = lds[t * R + 4 * kb + lq];   // channels kb*32 + 8*lq + e at bit e
#pragma unroll
      for (int e = 0; e < 8; ++e) kw |= ((x >> e) & 1u) << q1_kbit(kb, e);
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const uint8_t *vr = lds + (4 * lq + tt) * R + D / 2 + (t >> 3);
#pragma unroll
      for (int ct = 0; ct < Q::CT; ++ct) vw |= (((uint32_t)vr[2 * ct] >> (t & 7)) & 1u) << q1_vbit(ct, tt);
    }
    ((uint32_t *)T)[lane] = kw;
    ((uint32_t *)(T + Q::VC))[lane] = vw;
    if (lq == 0) {
      // records keep (mean, std) in the first params pair of keys and of values
      const uint16_t *par = (const uint16_t *)(lds + t * R + D);
      ((uint16_t *)(T + Q::KSD))[t] = par[1];
      ((uint16_t *)(T + Q::KM))[t] = par[0];
      ((uint16_t *)(T + Q::VSD))[t] = par[2 * Q::NG + 1];
      ((uint16_t *)(T + Q::VM))[t] = par[2 * Q::NG];
    }
    wave_lds_sync();
  }
}

// Compact BF16 tiles of one (sequence, KV head) from the position pages, one
// wave per tile, all accesses 16 bytes wide: key chunks (one token, eight
// channels) are copied as they are; a value chunk of the tile layout (four
// tokens of two channels c, c + 16) is assembled from the four source chunks
// that hold those channels of each token.  Slots past the count are zeros.
template <int D>
__device__ void hq_gather_bf16(const TokGeom &g, const TokState &st, int bh, int gw, int n_gw, int lane) {
  const int b = bh / g.Hkv, h = bh % g.Hkv;
  const int nb = st.cnt[bh * 4 + 0];
  const int ntiles = (nb + TS - 1) / TS;
  const uint16_t *src = st.pages + tok_page_offset(g, b, h, 0);
  const int32_t *cpos = st.cpos + (size_t)bh * g.NCT * TS;
  const u32x4v zero = {0u, 0u, 0u, 0u};
  for (int tile = gw; tile < ntiles; tile += n_gw) {
    uint16_t *dk = st.cpages + tok_cpage_offset(g, b, h, tile);
    uint16_t *dv = dk + TS * D;
    for (int it = lane; it < TS * D / 8; it += 64) {
      const int tk = it / (D / 8), c0 = (it % (D / 8)) * 8;
      const int i = tile * TS + tk;
      u32x4v v = zero;
      if (i < nb) {
        const int pos = cpos[i];
        v = *(const u32x4v *)(src + (size_t)(pos / TS) * 2 * TS * D + k_tile_index(pos % TS, c0));
      }
      *(u32x4v *)(dk + k_tile_index(tk, c0)) = v;
    }
    for (int it = lane; it < 4 * (D / 2); it += 64) {
      const int q = it / (D / 2), cp = it % (D / 2);
      const int cb = (cp >> 4) * 32 + (cp & 15);   // channels cb and cb + 16
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        lo[tt] = hi[tt] = 0u;
        const int i = tile * TS + 4 * q + tt;
        if (i < nb) {
          const int pos = cpos[i], ts = pos % TS, e = ts & 3;
          const u32x4v sv = *(const u32x4v *)(src + (size_t)(pos / TS) * 2 * TS * D + TS * D + v_tile_index(ts & ~3, cb));
          lo[tt] = ((e < 2 ? sv[0] : sv[1]) >> (16 * (e & 1))) & 0xffffu;
          hi[tt] = ((e < 2 ? sv[2] : sv[3]) >> (16 * (e & 1))) & 0xffffu;
        }
      }
      *(u32x4v *)(dv + v_tile_index(4 * q, cb)) =
          u32x4v{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
    }
  }
}

// compact tiles of every tier from the position lists, one wave per tile
template <int D>
__global__ __launch_bounds__(256) void hq_gather_kernel(TokGeom g, TokState st) {
  const int bh = blockIdx.y;
  __shared__ __attribute__((aligned(16))) uint8_t s_rec[4][TS * (D + (D / 32) * 8)];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + wave, n_gw = gridDim.x * 4;
  hq_gather_bf16<D>(g, st, bh, gw, n_gw, lane);
  hq_gather_ql<D, 0>(g, st, bh, s_rec[wave], gw, n_gw, lane);
  hq_gather_ql<D, 1>(g, st, bh, s_rec[wave], gw, n_gw, lane);
  hq_gather_q1<D>(g, st, bh, s_rec[wave], gw, n_gw, lane);
}

hipError_t hq_launch_event(const TokGeom &g, const TokState &st, int N, int elig_end, const int *counts,
                           hipStream_t s) {
  hipLaunchKernelGGL(hq_event_kernel, dim3(g.B * g.Hkv), dim3(1024), 0, s, g, st, N, elig_end, counts[0], counts[1],
                     counts[2], counts[3]);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (elig_end > 0) {
    const dim3 rgrid((elig_end + 255) / 256, g.B * g.Hkv);
    if (g.d == 128)
      hipLaunchKernelGGL(hq_requant_kernel<128>, rgrid, dim3(256), 0, s, g, st, elig_end);
    else
      hipLaunchKernelGGL(hq_requant_kernel<64>, rgrid, dim3(256), 0, s, g, st, elig_end);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 grid(256, g.B * g.Hkv);   // 1024 waves per (sequence, KV head): 555 us at 8 x 64K, 614 with 64 blocks
  if (g.d == 128)
    hipLaunchKernelGGL(hq_gather_kernel<128>, grid, dim3(256), 0, s, g, st);
  else
    hipLaunchKernelGGL(hq_gather_kernel<64>, grid, dim3(256), 0, s, g, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// export: tiers and scores per (sequence, KV head, position); HqeKV records
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void tok_export_kernel(TokGeom g, TokState st, int what, void *dst) {
  const size_t n = (size_t)g.B * g.Hkv * g.T;
  if (what == QKV_EXPORT_KEYS || what == QKV_EXPORT_VALUES) {
    // the appended originals from the position pages: [B][Hkv][T][d]
    const int D = g.d;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n * D; i += (size_t)gridDim.x * blockDim.x) {
      const int c = (int)(i % D);
      const size_t row = i / D;                       // bh * T + pos
      const int pos = (int)(row % g.T);
      const size_t bh = row / g.T;
      const uint16_t *kt = st.pages + tok_page_offset(g, (int)(bh / g.Hkv), (int)(bh % g.Hkv), pos / TS);
      ((uint16_t *)dst)[i] = what == QKV_EXPORT_KEYS ? kt[k_tile_index(pos % TS, c)]
                                                     : kt[TS * D + v_tile_index(pos % TS, c)];
    }
    return;
  }
  if (what == QKV_EXPORT_TIERS || what == QKV_EXPORT_SCORES) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
      if (what == QKV_EXPORT_TIERS)
        ((uint8_t *)dst)[i] = st.tier[i];
      else
        ((float *)dst)[i] = st.score[i];
    }
    return;
  }
  // records: KCODES / VCODES [.., d/2] bytes, KPARAMS / VPARAMS [.., d/32, 2] fp16
  const int off = what == QKV_EXPORT_KCODES ? 0 : what == QKV_EXPORT_VCODES ? g.d / 2
                : what == QKV_EXPORT_KPARAMS ? g.d : g.d + (g.d / 32) * 4;
  const int len = (what == QKV_EXPORT_KCODES || what == QKV_EXPORT_VCODES) ? g.d / 2 : (g.d / 32) * 4;
  const size_t total = n * len;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x)
    ((uint8_t *)dst)[i] = st.qrec[(i / len) * g.rec_bytes + off + (i % len)];
}

hipError_t tok_launch_export(const TokGeom &g, const TokState &st, int what, void *dst, hipStream_t s) {
  const size_t n = (size_t)g.B * g.Hkv * g.T;
  if (what == QKV_EXPORT_EVENT)
    return hipMemcpyAsync(dst, st.event, (size_t)g.B * g.Hkv * EV_WORDS * 4, hipMemcpyDeviceToDevice, s);
  if (what == QKV_EXPORT_VICTIMS) return hipMemcpyAsync(dst, st.victims, n * 4, hipMemcpyDeviceToDevice, s);
  int grid = (int)((n + 255) / 256);
  grid = grid > 4096 ? 4096 : (grid < 1 ? 1 : grid);
  hipLaunchKernelGGL(tok_export_kernel, dim3(grid), dim3(256), 0, s, g, st, what, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// session snapshot: ranked lists, canonical -> internal layouts, compact tiles
// ---------------------------------------------------------------------------

// ROUTED [B][Hkv][4 + 4 L]: counts of the full-precision, INT4, INT2, INT1
// lists, then the lists (L entries each; -1 where a policy has no list)
__global__ __launch_bounds__(256) void tok_routed_kernel(TokGeom g, TokState st, int n_cmp, int32_t *dst,
                                                         int to_state) {
  const int bh = blockIdx.x;
  const int Lc = tok_list_cap(g);
  int32_t *row = dst + (size_t)bh * (4 + 4 * Lc);
  const bool hq = g.policy == QKV_POLICY_HQEKV;
  if (!to_state) {
    for (int i = threadIdx.x; i < 4 + 4 * Lc; i += blockDim.x) {
      int32_t v = -1;
      if (i < 4) {
        v = hq ? st.cnt[bh * 4 + i] : (i == 0 ? n_cmp : 0);
      } else {
        const int k = (i - 4) / Lc, e = (i - 4) % Lc;
        if (k == 0)
          v = st.cpos[(size_t)bh * Lc + e];
        else if (hq)
          v = st.qpos[k - 1][(size_t)bh * Lc + e];
      }
      row[i] = v;
    }
    return;
  }
  for (int i = threadIdx.x; i < 4 + 4 * Lc; i += blockDim.x) {
    const int32_t v = row[i];
    if (i < 4) {
      if (hq) st.cnt[bh * 4 + i] = v;
    } else {
      const int k = (i - 4) / Lc, e = (i - 4) % Lc;
      if (k == 0)
        st.cpos[(size_t)bh * Lc + e] = v;
      else if (hq)
        st.qpos[k - 1][(size_t)bh * Lc + e] = v;
    }
  }
}

hipError_t tok_launch_export_routed(const TokGeom &g, const TokState &st, int n_cmp, void *dst, hipStream_t s) {
  hipLaunchKernelGGL(tok_routed_kernel, dim3(g.B * g.Hkv), dim3(256), 0, s, g, st, n_cmp, (int32_t *)dst, 0);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void tok_import_kernel(TokGeom g, TokState st, int what, const void *__restrict__ src) {
  const size_t n = (size_t)g.B * g.Hkv * g.T;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (what == QKV_EXPORT_KEYS || what == QKV_EXPORT_VALUES) {
    const int D = g.d;
    const uint16_t *xs = (const uint16_t *)src;
    for (size_t i = i0; i < n * D; i += stride) {
      const int c = (int)(i % D);
      const size_t row = i / D;
      const int pos = (int)(row % g.T);
      const size_t bh = row / g.T;
      uint16_t *kt = st.pages + tok_page_offset(g, (int)(bh / g.Hkv), (int)(bh % g.Hkv), pos / TS);
      if (what == QKV_EXPORT_KEYS)
        kt[k_tile_index(pos % TS, c)] = xs[i];
      else
        kt[TS * D + v_tile_index(pos % TS, c)] = xs[i];
    }
    return;
  }
  // per-token records: KCODES / VCODES [.., d/2] bytes, KPARAMS / VPARAMS [.., d/32, 2] fp16
  const int off = what == QKV_EXPORT_KCODES ? 0 : what == QKV_EXPORT_VCODES ? g.d / 2
                : what == QKV_EXPORT_KPARAMS ? g.d : g.d + (g.d / 32) * 4;
  const int len = (what == QKV_EXPORT_KCODES || what == QKV_EXPORT_VCODES) ? g.d / 2 : (g.d / 32) * 4;
  for (size_t i = i0; i < n * len; i += stride)
    st.qrec[(i / len) * g.rec_bytes + off + (i % len)] = ((const uint8_t *)src)[i];
}

// value range of every position's original value row (as the append kernel
// forms it: max - min over the row, exact in any order)
__global__ __launch_bounds__(256) void tok_vrange_kernel(TokGeom g, TokState st) {
  const size_t n = (size_t)g.B * g.Hkv * g.T;
  const int D = g.d;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int pos = (int)(i % g.T);
    const size_t bh = i / g.T;
    const uint16_t *vt = st.pages + tok_page_offset(g, (int)(bh / g.Hkv), (int)(bh % g.Hkv), pos / TS) + TS * D;
    float mn = bf16_to_f32(vt[v_tile_index(pos % TS, 0)]), mx = mn;
    for (int c = 1; c < D; ++c) {
      const float x = bf16_to_f32(vt[v_tile_index(pos % TS, c)]);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    st.vrange[i] = mx - mn;
  }
}

hipError_t tok_launch_import(const TokGeom &g, const TokState &st, int what, const void *src, hipStream_t s) {
  const size_t n = (size_t)g.B * g.Hkv * g.T;
  switch (what) {
    case QKV_EXPORT_TIERS: return hipMemcpyAsync(st.tier, src, n, hipMemcpyDeviceToDevice, s);
    case QKV_EXPORT_SCORES: {
      // the imported scores already hold every pending mass
      hipError_t e = hipMemcpyAsync(st.score, src, n * sizeof(float), hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return e;
      return launch_clear(st.tacc, (size_t)g.B * g.Hkv * g.TILES * TS * sizeof(float), s);
    }
    case QKV_EXPORT_ROUTED:
      hipLaunchKernelGGL(tok_routed_kernel, dim3(g.B * g.Hkv), dim3(256), 0, s, g, st, 0,
                         (int32_t *)const_cast<void *>(src), 1);
      return hipGetLastError();
    default: break;
  }
  hipLaunchKernelGGL(tok_import_kernel, dim3(2048), dim3(256), 0, s, g, st, what, src);
  return hipGetLastError();
}

// H2O: the kept heavy hitters of each (sequence, KV head) gathered, in list
// order, into the compact tiles
__global__ __launch_bounds__(256) void tok_regather_kernel(TokGeom g, TokState st, int n_cmp) {
  const int bh = blockIdx.y;
  const int b = bh / g.Hkv, h = bh % g.Hkv;
  const int chunks = g.d / 8;
  const int32_t *cpos = st.cpos + (size_t)bh * g.NCT * TS;
  const uint16_t *pages_bh = st.pages + tok_page_offset(g, b, h, 0);
  uint16_t *cpages_bh = st.cpages + tok_cpage_offset(g, b, h, 0);
  for (int it = blockIdx.x * blockDim.x + threadIdx.x; it < n_cmp * chunks; it += gridDim.x * blockDim.x)
    tok_copy_token(g, pages_bh, cpages_bh, min(max(cpos[it / chunks], 0), g.T - 1), it / chunks, (it % chunks) * 8);
}

hipError_t tok_launch_rebuild(const TokGeom &g, const TokState &st, int n_cmp, hipStream_t s) {
  if (g.policy == QKV_POLICY_HQEKV) {
    const size_t n = (size_t)g.B * g.Hkv * g.T;
    int grid = (int)((n + 255) / 256);
    grid = grid > 4096 ? 4096 : (grid < 1 ? 1 : grid);
    hipLaunchKernelGGL(tok_vrange_kernel, dim3(grid), dim3(256), 0, s, g, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 ggrid(64, g.B * g.Hkv);
    if (g.d == 128)
      hipLaunchKernelGGL(hq_gather_kernel<128>, ggrid, dim3(256), 0, s, g, st);
    else
      hipLaunchKernelGGL(hq_gather_kernel<64>, ggrid, dim3(256), 0, s, g, st);
    return hipGetLastError();
  }
  if (n_cmp > 0) {
    const int chunks = g.d / 8;
    const dim3 grid((n_cmp * chunks + 255) / 256, g.B * g.Hkv);
    hipLaunchKernelGGL(tok_regather_kernel, grid, dim3(256), 0, s, g, st, n_cmp);
  }
  return hipGetLastError();
}

}  // namespace qkv
