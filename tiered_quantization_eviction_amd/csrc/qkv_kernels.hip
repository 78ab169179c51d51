// HIP kernels of the tiered decode path for gfx950 (CDNA4).
//
// Decode attention (QEvict notes section 4.1, Eq. attention) runs split-K over
// each (sequence, KV head): a workgroup of 4 waves streams a contiguous range
// of live units; scores S^T = K Q^T and the output P V use 16x16 matrix-core
// ops with the G query heads of the KV head as the narrow dimension.  Full
// precision tiles feed bf16 operands straight from HBM; quantized tiles are
// unpacked to exact fp16 integers in registers with the per-channel key scale
// folded into the query (q' = q*s split into two fp16 limbs) and the
// per-token value scale folded into the probabilities -- so no dequantized
// tile is ever materialized.  Each wave keeps an online softmax and emits,
// per unit, the head's partial mass with the reference maximum it is relative
// to; the merge kernel normalizes those with the global (max, sum) and adds
// them into the window scores (QEvict Eq.(1)) in a fixed order (no atomics).
#include <hip/hip_ext.h>

#include "qkv_device.h"

namespace qkv {

__device__ int g_quant_status;   // latched by the stateless quantizer

// ---------------------------------------------------------------------------
// fill
// ---------------------------------------------------------------------------

__global__ void fill_zero_kernel(uint32_t *p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_clear(void *p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  size_t words = bytes / 4;
  int grid = (int)((words + 255) / 256);
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, s, (uint32_t *)p, words);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// append: new positions into their unit's page (swizzled tiles)
// ---------------------------------------------------------------------------

// one block row per (sequence, KV head); thread it of the row copies 16-byte
// chunk it % (D/8) of token it / (D/8) (32-bit indices: a prompt is far below 2^31 chunks).
// ROPE: the key arrives before the rotary embedding; it is kept as given (the
// quantized tier is packed from it) and the page takes its rotation at the
// token's position, so the thread of chunk c0 < D/2 also handles the key
// chunk c0 + D/2 that pairs with it.
template <int D, bool ROPE>
__global__ __launch_bounds__(256) void append_kernel(Geom g, State st, const uint16_t *__restrict__ k,
                                                     const uint16_t *__restrict__ v, int n_tokens, int pos0) {
  constexpr int CH = D / 8;
  const int bh = blockIdx.x;
  const int b = bh / g.Hkv, h = bh - b * g.Hkv;
  const int total = n_tokens * CH;
  for (int it = blockIdx.y * blockDim.x + threadIdx.x; it < total; it += gridDim.y * blockDim.x) {
    const int tok = it / CH, c0 = (it % CH) * 8;
    const int pos = pos0 + tok;
    const int u = unit_of(g, pos);
    const int slot = pos - unit_start(g, u);
    const int tile = slot / TS, t = slot % TS;
    uint16_t *kt = st.pages + page_offset(g, b, u, h) + (size_t)tile * 2 * TS * D;
    uint16_t *vt = kt + TS * D;
    const size_t src = ((size_t)bh * n_tokens + tok) * D + c0;
    if (!ROPE) {
      *(uint4 *)(kt + k_tile_index(t, c0)) = *(const uint4 *)(k + src);
    } else if (c0 < D / 2) {
      const uint4 klo = *(const uint4 *)(k + src), khi = *(const uint4 *)(k + src + D / 2);
      uint16_t *kr = st.kraw + kraw_offset(g, b, u, h) + (size_t)tile * TS * D;
      *(uint4 *)(kr + k_tile_index(t, c0)) = klo;
      *(uint4 *)(kr + k_tile_index(t, c0 + D / 2)) = khi;
      const float4 *row = (const float4 *)(st.rope + ((size_t)pos * (D / 2) + c0) * 2);   // 8 (cos, sin) pairs
      float4 cs[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) cs[j] = row[j];
      const uint16_t *el = (const uint16_t *)&klo, *eh = (const uint16_t *)&khi;
      uint4 olo, ohi;
      uint16_t *ol = (uint16_t *)&olo, *oh = (uint16_t *)&ohi;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float cj = (j & 1) ? cs[j >> 1].z : cs[j >> 1].x, sj = (j & 1) ? cs[j >> 1].w : cs[j >> 1].y;
        float rl, rh;
        rope_pair(bf16_to_f32(el[j]), bf16_to_f32(eh[j]), cj, sj, rl, rh);
        ol[j] = f32_to_bf16_rne(rl);
        oh[j] = f32_to_bf16_rne(rh);
      }
      *(uint4 *)(kt + k_tile_index(t, c0)) = olo;
      *(uint4 *)(kt + k_tile_index(t, c0 + D / 2)) = ohi;
    }
    const uint4 vq = *(const uint4 *)(v + src);
    const uint16_t *vs = (const uint16_t *)&vq;
#pragma unroll
    for (int j = 0; j < 8; ++j) vt[v_tile_index(t, c0 + j)] = vs[j];
    if (h == 0 && c0 == 0 && (slot == 0 || tok == 0)) st.tier[b * g.U + u] = (u == 0) ? T_SINK : T_RECENT;
  }
}

hipError_t launch_append(const Geom &g, const State &st, const uint16_t *k, const uint16_t *v, int n_tokens,
                         int pos0, hipStream_t s) {
  if ((long long)n_tokens * (g.d / 8) > 0x7fffffffLL) return hipErrorInvalidValue;
  const int total = n_tokens * (g.d / 8);
  const int threads = total <= 64 ? 64 : 256;
  int rows = (total + threads - 1) / threads;
  if (rows > 65535) rows = 65535;
  const dim3 grid(g.B * g.Hkv, rows);
  if (g.rope && (!st.rope || !st.kraw || pos0 + n_tokens > st.rope_n)) return hipErrorInvalidValue;
  if (g.d == 128 && g.rope)
    hipLaunchKernelGGL((append_kernel<128, true>), grid, dim3(threads), 0, s, g, st, k, v, n_tokens, pos0);
  else if (g.d == 128)
    hipLaunchKernelGGL((append_kernel<128, false>), grid, dim3(threads), 0, s, g, st, k, v, n_tokens, pos0);
  else if (g.rope)
    hipLaunchKernelGGL((append_kernel<64, true>), grid, dim3(threads), 0, s, g, st, k, v, n_tokens, pos0);
  else
    hipLaunchKernelGGL((append_kernel<64, false>), grid, dim3(threads), 0, s, g, st, k, v, n_tokens, pos0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// live-entry list of one sequence (sink, ranked full, ranked quantized, recent)
// ---------------------------------------------------------------------------

struct EntryList {
  int s0, nF, nQ, nR, r0;
  __device__ int count() const { return s0 + nF + nQ + nR; }
};

__device__ inline EntryList make_list(const Geom &g, const State &st, const StepInfo &si, int b) {
  EntryList L;
  L.s0 = si.has_sink;
  // every sequence has the same candidate count, so the split of the ranked
  // windows follows from the host's count (the routing kernel stores the same
  // values in routed_nf / routed_nq)
  L.nF = min(si.n_routed, g.k_full);
  L.nQ = si.n_routed - L.nF;
  L.nR = si.r1 >= si.r0 ? si.r1 - si.r0 + 1 : 0;
  L.r0 = si.r0;
  return L;
}

// unit of entry e of list L (routed: the sequence's ranked list)
__device__ inline int entry_unit(const EntryList &L, const int32_t *routed, int e) {
  if (e < L.s0) return 0;
  const int r = e - L.s0;
  return r < L.nF + L.nQ ? routed[r] : L.r0 + (r - L.nF - L.nQ);
}

// ---------------------------------------------------------------------------
// attention: one workgroup per (sequence, KV head, split)
// ---------------------------------------------------------------------------
//
// The steady-state loops below keep every memory operation out of branches:
// a load or store under a branch makes the compiler wait for *all* loads in
// flight at the join, which would serialize the prefetch of the next block
// with the compute of the current one.  Unit ids are fetched two blocks
// ahead with clamped (always valid) indices, spare slots re-read valid tiles,
// and mass stores of unused lanes go to a spare slot.

// everything a wave needs while it walks its entries
struct Ctx {
  const Geom *g;
  const State *st;
  const StepInfo *si;
  const EntryList *L;
  const uint16_t *qrow;   // this lane's query row (head of its column; head 0 for other lanes)
  const uint16_t *qbase;  // query rows of the KV head's G heads
  int b, h, lane, col, lq, G, hc;
  bool is_hi, is_lo, has_q;
  int slot;               // channel-group slot of this lane's A row in the paired value product
  float scale_log2;
  float *mass_row;        // [(U+1)][G][2] of this (sequence, KV head); slot U is the spare
  size_t ledger_h;          // byte offset of this KV head's entry of ledger pool slot 0
  size_t ledger_stride;     // bytes from one pool slot to the next
  half_t *kp_lds;
  half_t *vp_lds;
  half_t *qs_lds;         // per window slot: q*s limbs [2][G][d] (fp16)
  float *rw_lds;          // rotary keys: table rows of the block's window starts [QT][d/2][2]
  const float *rd_lds;    // rotary keys: table rows 0..15 (token offsets in a window) [16][RD_STR]
  // a token appended by this launch (new_u < 0: none): its unit, tile and row;
  // lane l < d/4 holds 16-byte chunk l of its K and V rows ([2][d] bf16) in
  // new_chunk, which the wave that reads the token's tile stages in new_kv
  int new_u, new_tile, new_row;
  uint16_t *new_kv;        // LDS [2][d]
  uint4 new_chunk;
};

// unit id of entry e; `raw` is the routed-list value fetched for it (used
// for ranked entries only)
__device__ __forceinline__ int entry_id(const Ctx &c, int e, int raw) {
  const EntryList &L = *c.L;
  if (e < L.s0) return 0;
  const int r = e - L.s0;
  if (r < L.nF + L.nQ) return raw;
  return L.r0 + (r - L.nF - L.nQ);
}
// valid tokens of entry e (unit u)
__device__ __forceinline__ int entry_nv(const Ctx &c, int e, int u) {
  const EntryList &L = *c.L;
  if (e < L.s0) return min(c.si->N, c.g->n_sink);
  if (e - L.s0 < L.nF + L.nQ) return c.g->window;
  return min(c.si->N - unit_start(*c.g, u), c.g->window);
}
// routed-list values of entries e0 .. e0+3 in lanes j = 0..3 (mod 4); the
// index is clamped into the list so the load is valid and unconditional
__device__ __forceinline__ int ids_fetch(const Ctx &c, int e0) {
  const int r = min(max(e0 + (c.lane & 3) - c.L->s0, 0), c.g->U - 1);
  return c.st->routed[(size_t)c.b * c.g->U + r];
}
// the same for quantized entries: their ledger-pool slots (clamped into the pool)
__device__ __forceinline__ int slots_fetch(const Ctx &c, int e0) {
  const int r = min(max(e0 + (c.lane & 3) - c.L->s0, 0), c.g->U - 1);
  return min(max(c.st->qslot[(size_t)c.b * c.g->U + r], 0), c.g->pool_slots - 1);
}

// Mass partials of up to 4 units of a block in one store: lanes of row q
// (lq == q) and column h < G write unit slot q's (rho, m) when ok[q]; all
// other lanes write the spare slot.
template <int N>
__device__ __forceinline__ void store_mass(const Ctx &c, const int *e, const bool *ok, const float *rho, float m) {
  int slot = c.g->U;
  float r = 0.0f;
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const bool mine = (c.lq == q) && ok[q];
    slot = mine ? e[q] : slot;
    r = mine ? rho[q] : r;
  }
  if (c.col >= c.G) slot = c.g->U;
  *(float2 *)(c.mass_row + ((size_t)slot * c.G + (c.col & (c.G - 1))) * 2) = make_float2(r, m);
}

// query B operands: bf16 as given (columns h and G+h carry head h)
template <int D>
__device__ __forceinline__ void query_bf16(const Ctx &c, bf16x8 (&bq)[D / 32]) {
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb) {
    const uint32_t keep = c.has_q ? 0xffffffffu : 0u;   // lanes without a head get a zero query
    uint4 raw = *(const uint4 *)(c.qrow + kb * 32 + c.lq * 8);
    raw = make_uint4(raw.x & keep, raw.y & keep, raw.z & keep, raw.w & keep);
    bq[kb] = __builtin_bit_cast(bf16x8, raw);
  }
}
// Query for quantized tiles, as fp16 scaled by 2^-e (one e for the KV head's
// G heads, |q| 2^-e < 1, so q*s never leaves fp16).  qc: the compact operand
// of lane L -- heads (L/16) + 4r, channels 8*(L%16) .. +7 -- from which each
// window's q*s limbs are formed; bz: the B operand of the key-zero term
// (head h in column h, zero elsewhere).  Returns the softmax scale of the
// scores so formed.
template <int D>
__device__ __forceinline__ float query_f16(const Ctx &c, half8 (&qc)[2], half8 (&bz)[D / 32]) {
  constexpr int KB = D / 32;
  const int c0 = 8 * ((c.lane & 15) % (D / 8));
  uint4 rc[2];
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int hh = min((c.lane >> 4) + 4 * r, c.G - 1);
    rc[r] = *(const uint4 *)(c.qbase + (size_t)hh * D + c0);
    const uint16_t *e = (const uint16_t *)&rc[r];
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(bf16_to_f32(e[j])));
  }
  amax = max_x16(amax);
  amax = max_x32(amax);
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  amax = fmaxf(amax, __shfl_xor(amax, 8));
  int qexp = 0;
  if (amax > 0.0f) frexpf(amax, &qexp);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint16_t *e = (const uint16_t *)&rc[r];
#pragma unroll
    for (int j = 0; j < 8; ++j) qc[r][j] = (half_t)ldexpf(bf16_to_f32(e[j]), -qexp);
  }
  const uint32_t keep = c.is_hi ? 0xffffffffu : 0u;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const uint4 r = *(const uint4 *)(c.qrow + kb * 32 + c.lq * 8);
    const uint16_t *e = (const uint16_t *)&r;
#pragma unroll
    for (int j = 0; j < 8; ++j) bz[kb][j] = (half_t)ldexpf(bf16_to_f32(keep ? e[j] : (uint16_t)0), -qexp);
  }
  return ldexpf(c.scale_log2, qexp);
}

// ---- runs of full-precision units, two tiles (32 token slots) per block ----
// Tile k of a run is tile k % tpw of entry ea + k / tpw; block i holds tiles
// 2i and 2i+1, so with at most two tiles per unit a unit never straddles
// blocks.  A block's PV is one 16x16x32 op per column tile: the lane's eight
// k slots are tokens 4*lq..4*lq+3 of the first tile and of the second tile,
// the same order on the probability operand and on the value operand.

struct FBlock {
  int e[2], u[2], tile[2], nv[2];   // nv <= 0: an empty slot (its address repeats slot 0)
};

__device__ __forceinline__ void fblock_make(const Ctx &c, int ea, int n_tiles, int i, int ids, FBlock &fb) {
  const int tpw = c.g->tpw;
  const int e_first = ea + (2 * i) / tpw;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int k = 2 * i + s;
    const bool valid = k < n_tiles;
    const int kk = valid ? k : 2 * i;
    const int e = ea + kk / tpw;
    const int t = kk - (kk / tpw) * tpw;
    const int raw = __builtin_amdgcn_readlane(ids, e - e_first);
    const int u = entry_id(c, e, raw);
    fb.e[s] = e;
    fb.u[s] = u;
    fb.tile[s] = t;
    fb.nv[s] = valid ? entry_nv(c, e, u) - t * TS : 0;
  }
}

template <int D>
__device__ __forceinline__ const uint16_t *ftile_ptr(const Ctx &c, const FBlock &fb, int s) {
  return c.st->pages + page_offset(*c.g, c.b, fb.u[s], c.h) + (size_t)fb.tile[s] * 2 * TS * D;
}

// The tile that holds a token appended by this launch was read before the
// token reached the page: its row is patched in registers from the LDS copy
// (K: the lanes of the token's row; V: the lanes of its group of four
// tokens, element (channel half, token & 3) of each column-tile pair).
template <int D>
__device__ __forceinline__ void patch_new_token(const Ctx &c, u32x4v (&kr)[D / 32], u32x4v (&vr)[D / 32]) {
  if (c.lane < D / 4) *(uint4 *)(c.new_kv + c.lane * 8) = c.new_chunk;
  wave_lds_sync();
  const int row = c.new_row;
  if ((c.lane & 15) == row) {
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) kr[kb] = *(const u32x4v *)(c.new_kv + kb * 32 + c.lq * 8);
  }
  if (c.lq == (row >> 2)) {
#pragma unroll
    for (int cp = 0; cp < D / 32; ++cp)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int i = hf * 4 + (row & 3);   // the element of the lane's 8
        const uint32_t v = c.new_kv[D + 32 * cp + c.col + 16 * hf];
        uint32_t w = vr[cp][i >> 1];
        w = (i & 1) ? ((w & 0x0000ffffu) | (v << 16)) : ((w & 0xffff0000u) | v);
        vr[cp][i >> 1] = w;
      }
  }
}

// Attend over block `cur` (tiles in kr, vr); with PF the tiles of block
// `nxt` are loaded into kr and vr as soon as each has been consumed.
template <int D, bool PF>
__device__ __forceinline__ void full_step(WaveState<D> &ws, const Ctx &c, const bf16x8 (&bq)[D / 32],
                                          const FBlock &cur, const FBlock &nxt, u32x4v (&kr)[2][D / 32],
                                          u32x4v (&vr)[2][D / 32]) {
  constexpr int KB = D / 32, CP = D / 32;
  const int tpw = c.g->tpw;
  if (c.new_u >= 0) {   // wave-uniform; the patch reads LDS only, so no global wait lands here
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (cur.nv[t] > 0 && cur.u[t] == c.new_u && cur.tile[t] == c.new_tile) patch_new_token<D>(c, kr[t], vr[t]);
  }
  floatx4 s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) s[t] = mfma_bf16_k32(__builtin_bit_cast(bf16x8, kr[t][kb]), bq[kb], s[t]);
  if (PF) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t *kn = ftile_ptr<D>(c, nxt, t);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kr[t][kb] = ld_stream16v(kn + (kb * 64 + c.lane) * 8);
    }
  }
  const int lo[2] = {0, 0};
  const int hi[2] = {c.has_q ? cur.nv[0] : 0, c.has_q ? cur.nv[1] : 0};
  float p[2][4], ts[2];
  softmax_block<D, 2>(ws, s, c.scale_log2, lo, hi, c.lq, p, ts);
  {
    // tpw == 1: each slot is a unit; tpw == 2: the block is one unit
    const int e[2] = {cur.e[0], cur.e[1]};
    const bool ok[2] = {true, tpw == 1 && cur.nv[1] > 0};
    const float rho[2] = {tpw == 1 ? ts[0] : ts[0] + ts[1], ts[1]};
    store_mass<2>(c, e, ok, rho, ws.m);
  }
  // rows h carry bf16(p), rows G+h carry bf16(p - bf16(p))
  bf16x8 ap;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const float hi = (float)(__bf16)p[t][i2];
      ap[t * 4 + i2] = (__bf16)(c.is_lo ? p[t][i2] - hi : p[t][i2]);
    }
#pragma unroll
  for (int cp = 0; cp < CP; ++cp) {
    const u32x4v v0 = __builtin_shufflevector(vr[0][cp], vr[1][cp], 0, 1, 4, 5);
    const u32x4v v1 = __builtin_shufflevector(vr[0][cp], vr[1][cp], 2, 3, 6, 7);
    ws.acc[2 * cp] = mfma_bf16_k32(ap, __builtin_bit_cast(bf16x8, v0), ws.acc[2 * cp]);
    ws.acc[2 * cp + 1] = mfma_bf16_k32(ap, __builtin_bit_cast(bf16x8, v1), ws.acc[2 * cp + 1]);
  }
  if (PF) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t *kn = ftile_ptr<D>(c, nxt, t);
#pragma unroll
      for (int cp = 0; cp < CP; ++cp) vr[t][cp] = ld_stream16v(kn + TS * D + (cp * 64 + c.lane) * 8);
    }
  }
}

// Run of full-precision entries [ea, eb), two tiles per block; the next
// block is in flight while one computes, and the last block is peeled off so
// that nothing past the run is read.
template <int D>
__device__ void run_full(WaveState<D> &ws, const Ctx &c, int ea, int eb) {
  if (ea >= eb) return;
  constexpr int KB = D / 32, CP = D / 32;
  const int tpw = c.g->tpw;
  const int n_tiles = (eb - ea) * tpw;
  const int n_blocks = (n_tiles + 1) >> 1;
  bf16x8 bq[KB];
  query_bf16<D>(c, bq);
  int ids_a = ids_fetch(c, ea);
  int ids_b = ids_fetch(c, ea + (2 * min(1, n_blocks - 1)) / tpw);
  FBlock cur, nxt;
  fblock_make(c, ea, n_tiles, 0, ids_a, cur);
  u32x4v kr[2][KB], vr[2][CP];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const uint16_t *kt = ftile_ptr<D>(c, cur, s);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) kr[s][kb] = ld_stream16v(kt + (kb * 64 + c.lane) * 8);
#pragma unroll
    for (int cp = 0; cp < CP; ++cp) vr[s][cp] = ld_stream16v(kt + TS * D + (cp * 64 + c.lane) * 8);
  }
  for (int i = 0; i + 1 < n_blocks; ++i) {
    // unit ids two blocks ahead (clamped), the next block's tiles
    const int ids_c = ids_fetch(c, ea + (2 * min(i + 2, n_blocks - 1)) / tpw);
    fblock_make(c, ea, n_tiles, i + 1, ids_b, nxt);
    full_step<D, true>(ws, c, bq, cur, nxt, kr, vr);
    cur = nxt;
    ids_b = ids_c;
  }
  full_step<D, false>(ws, c, bq, cur, cur, kr, vr);
}

// ---- runs of quantized windows, QT tiles per block; the next block is in
// flight while one computes ----

constexpr int QT = 4;   // quantized tiles per block
// LDS strides (halfs), padded by 16 bytes so that rows and slots that are read
// together fall on different banks
template <int D> constexpr int PSTR = 2 * D + 8;   // parameter slot: [s(d), z(d)]
template <int D> constexpr int QSTR = D + 8;       // one q*s row
// window slots whose q*s limbs are staged in LDS at once: all of a block's,
// but half of them with eight heads per KV head at d = 128 (the LDS of eight
// waves holds no more), the block's windows then taking two rounds
template <int D, int GP> constexpr int QS_SLOTS = (GP == 1 && D == 128) ? QT / 2 : QT;

struct QBuf {
  uint4 code[QT];   // the lane's key code dwords, then value code dwords, of each tile
  uint4 code2[QT];  // 4-bit codes at d = 128: the lane's value code dwords
  uint2 kp[QT];     // the lane's 8 bytes of each window's key params (window slots)
  uint32_t vp[QT];  // the lane's 4 bytes of each tile's value params
  uint4 tr[2];      // rotary keys: the lane's 16-byte chunks of window (lane / 16)'s start row
};
// row stride (floats) of the offset rows of the rotary table in LDS
template <int D> constexpr int RD_STR = D + 4;

__device__ __forceinline__ uint32_t u4_at(const uint4 &v, int i) {   // i is a constant after unrolling
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// A operand of k-block kb of tile j: the lane's 8 key codes as exact fp16
template <int D, int BITS>
__device__ __forceinline__ half8 key_codes(const QBuf &buf, int j, int kb) {
  if (BITS == 2) return codes8(code_half(u4_at(buf.code[j], kb >> 1), kb & 1));
  return codes8_int4(u4_at(buf.code[j], kb));
}
// B operand half of column tile ct of tile j: the codes of the lane's four
// tokens (4 lq .. 4 lq + 3) of channel ct*16 + col, as exact fp16
template <int D, int BITS>
__device__ __forceinline__ half4 value_codes(const QBuf &buf, int j, int ct) {
  if (BITS == 2) {
    const uint32_t v = u4_at(buf.code[j], D == 128 ? 2 + (ct >> 2) : 1);
    return __builtin_shufflevector(fp4_pair_sel(code_half(v, 0), ct), fp4_pair_sel(code_half(v, 1), ct), 0, 1, 2, 3);
  }
  const uint32_t v = D == 128 ? u4_at(buf.code2[j], ct >> 1) : u4_at(buf.code[j], 2 + (ct >> 1));
  const uint32_t m = ((ct & 1) ? (v >> 4) : v) & 0x0F0F0F0Fu;
  return __builtin_shufflevector(fp8_pair<false>(m), fp8_pair<true>(m), 0, 1, 2, 3);
}
struct QBlock {
  int e, nwin;
  int u[QT];        // ledger-pool slots of the block's windows; spare slots repeat slot 0
  int p0;           // rotary keys: first position of window slot lane / 16 (per lane)
};

// window slot and tile-in-window of block tile j
__device__ __forceinline__ int qt_win(int j, int tpw) { return tpw == 1 ? j : j >> 1; }

template <bool ROPE>
__device__ __forceinline__ void qblock_make(const Ctx &c, int ea, int eb, int i, int ids, int units, QBlock &qb) {
  const int per = QT / c.g->tpw;
  const int e0 = ea + i * per;
  qb.e = e0;
  qb.nwin = min(per, eb - e0);
  // every entry of a quantized run is a ranked window, so the fetched value
  // is its pool slot (and, in `units`, its unit) as it stands
#pragma unroll
  for (int w = 0; w < QT; ++w) qb.u[w] = __builtin_amdgcn_readlane(ids, w < qb.nwin ? w : 0);
  qb.p0 = 0;
  if (ROPE) {
    // lane ww of `units` holds the routed unit of entry e0 + ww
    const int wl = c.lane >> 4, ww = wl < qb.nwin ? wl : 0;
    qb.p0 = min(max(unit_start(*c.g, __shfl(units, ww)), 0), c.st->rope_n - 1);
  }
}

template <int D, int BITS, bool ROPE>
__device__ __forceinline__ void quant_load(const Ctx &c, const QBlock &qb, QBuf &buf) {
  constexpr int DPL = D * BITS / 64;   // code dwords per lane per tile
  const Geom &g = *c.g;
  const int tpw = g.tpw;
  const int kl = c.lane & (g.kparam_bytes / 8 - 1);       // lanes past the params repeat them
  const int vl = c.lane & (g.tile_vparam_bytes / 4 - 1);
  // the windows' ledger offsets, one scalar product each; every address is
  // formed from the ledger base itself, so the loads stay global ones (a
  // pointer chosen among several would become a generic one, and generic
  // loads make every LDS wait wait for them as well)
  size_t Lw[QT];
#pragma unroll
  for (int w = 0; w < QT; ++w) Lw[w] = c.ledger_h + (size_t)(uint32_t)qb.u[w] * c.ledger_stride;
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    const int w = qt_win(j, tpw);
    const int tj = j - w * tpw;
    // both candidates are fixed indices: a run-time index would put Lw[] in scratch memory
    const uint8_t *Lb = c.st->ledger + (tpw == 1 ? Lw[j] : Lw[j >> 1]);
    const uint8_t *T = Lb + g.kparam_bytes + (size_t)tj * g.tile_block_bytes;
    if (DPL == 8) {
      buf.code[j] = ld_stream16(T + c.lane * 32);
      buf.code2[j] = ld_stream16(T + c.lane * 32 + 16);
    } else if (DPL == 4) {
      buf.code[j] = ld_stream16(T + c.lane * 16);
    } else {
      const uint2 cw = ld_stream8(T + c.lane * 8);
      buf.code[j] = make_uint4(cw.x, cw.y, 0u, 0u);
    }
    buf.vp[j] = ld_stream4(T + g.tile_kcode_bytes + g.tile_vcode_bytes + 4 * vl);
  }
#pragma unroll
  for (int w = 0; w < QT; ++w) buf.kp[w] = ld_stream8(c.st->ledger + Lw[w] + kl * 8);
  if (ROPE) {
    // lanes 16w .. 16w+15 fetch the table row of window slot w's first
    // position (D/2 (cos, sin) pairs, D/64 chunks of 16 bytes per lane); the
    // rows are shared by every KV head, so these are ordinary cached loads
    const float *row = c.st->rope + (size_t)qb.p0 * D;
#pragma unroll
    for (int r = 0; r < D / 64; ++r) buf.tr[r] = *(const uint4 *)(row + ((c.lane & 15) * (D / 64) + r) * 4);
  }
}

template <int D, int GP, int BITS, bool ROPE>
__device__ __forceinline__ void quant_compute(WaveState<D> &ws, const Ctx &c, const half8 (&qc)[2],
                                              const half8 (&qp)[2], const half8 (&bz)[D / 32], float sc_quant,
                                              const float (&row_bias)[4], const QBlock &qb, const QBuf &buf) {
  constexpr int KB = D / 32, NG = D / 32;
  const float neg1 = opaque_neg1();
  const Geom &g = *c.g;
  const int tpw = ROPE ? 1 : g.tpw;                          // rotary keys: one tile per window
  const int nws = QT / tpw;                                  // window slots per block
  constexpr int G = GP == 2 ? 4 : 8;   // query heads per KV head (the launcher pairs groups for four)
  const int kl = c.lane & (g.kparam_bytes / 8 - 1);
  const int vl = c.lane & (g.tile_vparam_bytes / 4 - 1);
  // stage key params (one slot per window) and value params (one slot per tile)
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    *(uint2 *)(c.kp_lds + j * PSTR<D> + kl * 4) = buf.kp[j];
    ((uint32_t *)(c.vp_lds + j * PSTR<D>))[vl] = buf.vp[j];
  }
  if constexpr (ROPE) {
#pragma unroll
    for (int r = 0; r < D / 64; ++r)
      *(uint4 *)(c.rw_lds + (c.lane >> 4) * D + ((c.lane & 15) * (D / 64) + r) * 4) = buf.tr[r];
  }
  wave_lds_sync();
  floatx4 s[QT];
  bool scored = false;   // the two-round path below forms the scores itself
  if constexpr (ROPE) {
    // Rotary keys.  A key of the window starting at p0 sits at p0 + t and
    // reads as R(p0 + t) k = R(p0) R(t) k, so q . R(p0 + t) k equals
    // (R(p0)^T q) . (R(t) k): the query is turned back by the window's start
    // once per (head, channel), and each dequantized key element is turned by
    // its offset t (the tile row, a lane constant).  q' = R(p0)^T q in two
    // fp16 limbs [limb][head][c]; the lane's channels pair with the lane
    // D/16 away (qp).
    const int c0 = 8 * ((c.lane & 15) % (D / 8));
    const int i0 = c0 & (D / 2 - 1);
    const bool lower = c0 < D / 2;
#pragma unroll
    for (int w = 0; w < QT; ++w) {
      float4 cs[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) cs[k] = *(const float4 *)(c.rw_lds + w * D + (i0 + 2 * k) * 2);
      half_t *qs = c.qs_lds + w * 2 * G * QSTR<D>;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (4 * r < G) {
          const int hh = (c.lane >> 4) + 4 * r;
          half8 hi, lo;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float cj = (j & 1) ? cs[j >> 1].z : cs[j >> 1].x, sj = (j & 1) ? cs[j >> 1].w : cs[j >> 1].y;
            const float o = (float)qp[r][j];
            const float v = __builtin_fmaf((float)qc[r][j], cj, (lower ? o : -o) * sj);
            hi[j] = (half_t)v;
            lo[j] = (half_t)(v - (float)hi[j]);
          }
          *(half8 *)(qs + hh * QSTR<D> + c0) = hi;
          *(half8 *)(qs + (G + hh) * QSTR<D> + c0) = lo;
        }
      }
    }
  } else if (QS_SLOTS<D, GP> < QT && nws > QS_SLOTS<D, GP>) {
    // the block's windows in two rounds of QS window slots: limbs of windows
    // w0 .. w0 + QS - 1, then the MFMAs of their tiles
    constexpr int QS = QS_SLOTS<D, GP>;
    const int c0 = 8 * ((c.lane & 15) % (D / 8));
    const int qrow = (c.is_lo ? G : 0) + c.hc;
    {
      // key-zero term of every window at once (reads the parameters only)
      floatx4 zb = {0.f, 0.f, 0.f, 0.f};
      const int zr = (c.lane & 15) % nws;
      half8 z8[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) z8[kb] = *(const half8 *)(c.kp_lds + zr * PSTR<D> + D + kb * 32 + c.lq * 8);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) zb = mfma_f16_k32(z8[kb], bz[kb], zb);
#pragma unroll
      for (int j = 0; j < QT; ++j) s[j] = floatx4{zb[j & 3] + row_bias[0], zb[j & 3] + row_bias[1],
                                                  zb[j & 3] + row_bias[2], zb[j & 3] + row_bias[3]};
    }
#pragma unroll
    for (int rd = 0; rd < QT / QS; ++rd) {
      if (rd > 0) {
        wave_lds_sync();   // the previous round's limbs have been read
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int w = 0; w < QS; ++w) {
        const half8 sw = *(const half8 *)(c.kp_lds + (rd * QS + w) * PSTR<D> + c0);
        half_t *qs = c.qs_lds + w * 2 * G * QSTR<D>;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if (4 * r < G) {
            const int hh = (c.lane >> 4) + 4 * r;
            const half8 hi = qc[r] * sw;
            const half8 lo = __builtin_elementwise_fma(qc[r], sw, -hi);
            *(half8 *)(qs + hh * QSTR<D> + c0) = hi;
            *(half8 *)(qs + (G + hh) * QSTR<D> + c0) = lo;
          }
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int w = 0; w < QS; ++w) {
          const int j = rd * QS + w;   // one tile per window
          const half8 bq = *(const half8 *)(c.qs_lds + (w * 2 * G + qrow) * QSTR<D> + kb * 32 + c.lq * 8);
          s[j] = mfma_f16_k32(key_codes<D, BITS>(buf, j, kb), bq, s[j]);
        }
    }
    scored = true;
  } else {
  // q*s of each window as two fp16 limbs (high, exact remainder), computed
  // once per (head, channel) in the compact layout and stored [limb][head][c]
  {
    const int c0 = 8 * ((c.lane & 15) % (D / 8));
    half8 s8[QT];   // all slots are staged (spare ones repeat slot 0), so the reads go out together
#pragma unroll
    for (int w = 0; w < QT; ++w) s8[w] = *(const half8 *)(c.kp_lds + w * PSTR<D> + c0);
#pragma unroll
    for (int w = 0; w < QT; ++w) {
      if (w < nws) {
        half_t *qs = c.qs_lds + w * 2 * G * QSTR<D>;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          if (4 * r < G) {
            const int hh = (c.lane >> 4) + 4 * r;
            const half8 hi = qc[r] * s8[w];
            const half8 lo = __builtin_elementwise_fma(qc[r], s8[w], -hi);
            *(half8 *)(qs + hh * QSTR<D> + c0) = hi;
            *(half8 *)(qs + (G + hh) * QSTR<D> + c0) = lo;
          }
        }
      }
    }
  }
  }
  wave_lds_sync();
  const int qrow = (c.is_lo ? G : 0) + c.hc;
  if constexpr (ROPE) {
    // A operand: the lane's 8 channels of k-block kb and their partners in
    // kb + KB/2, dequantized in float32 (code * s + z, one rounding), turned
    // by the row's offset and split into two fp16 limbs; each limb takes one
    // MFMA against the q' limbs (the key-zero term is inside the dequantized
    // values)
#pragma unroll
    for (int j = 0; j < QT; ++j) s[j] = floatx4{row_bias[0], row_bias[1], row_bias[2], row_bias[3]};
    const int t = c.lane & 15;
#pragma unroll
    for (int kb = 0; kb < KB / 2; ++kb) {
      const int ch = kb * 32 + c.lq * 8;
      float4 cs[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) cs[k] = *(const float4 *)(c.rd_lds + t * RD_STR<D> + (ch + 2 * k) * 2);
#pragma unroll
      for (int j = 0; j < QT; ++j) {
        const half_t *kp = c.kp_lds + j * PSTR<D>;
        const half8 sl = *(const half8 *)(kp + ch), sh = *(const half8 *)(kp + ch + D / 2);
        const half8 zl = *(const half8 *)(kp + D + ch), zh = *(const half8 *)(kp + D + ch + D / 2);
        const half8 cl = key_codes<D, BITS>(buf, j, kb), chh = key_codes<D, BITS>(buf, j, kb + KB / 2);
        half8 al, all, ah, ahl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xl = __builtin_fmaf((float)cl[e], (float)sl[e], (float)zl[e]);
          const float xh = __builtin_fmaf((float)chh[e], (float)sh[e], (float)zh[e]);
          const float ce = (e & 1) ? cs[e >> 1].z : cs[e >> 1].x, se = (e & 1) ? cs[e >> 1].w : cs[e >> 1].y;
          const float rl = __builtin_fmaf(xl, ce, -xh * se);
          const float rh = __builtin_fmaf(xh, ce, xl * se);
          al[e] = (half_t)rl;
          all[e] = lo_limb(al[e], rl, neg1);
          ah[e] = (half_t)rh;
          ahl[e] = lo_limb(ah[e], rh, neg1);
        }
        const half_t *qs = c.qs_lds + (j * 2 * G + qrow) * QSTR<D>;
        const half8 bl = *(const half8 *)(qs + ch), bh = *(const half8 *)(qs + ch + D / 2);
        s[j] = mfma_f16_k32(al, bl, s[j]);
        s[j] = mfma_f16_k32(all, bl, s[j]);
        s[j] = mfma_f16_k32(ah, bh, s[j]);
        s[j] = mfma_f16_k32(ahl, bh, s[j]);
        // one tile's operands at a time: letting the scheduler hoist the
        // next tiles' reads and arithmetic runs out of registers
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else if (!scored) {
  // key-zero term sum_c q_c z_c of every window at once: A rows r are the
  // zero vectors of window slot r % nws, so register i of every lane holds
  // the term of window slot i % nws for the lane's column (high columns only)
  floatx4 zb = {0.f, 0.f, 0.f, 0.f};
  const int zr = (c.lane & 15) % nws;
  half8 z8[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) z8[kb] = *(const half8 *)(c.kp_lds + zr * PSTR<D> + D + kb * 32 + c.lq * 8);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) zb = mfma_f16_k32(z8[kb], bz[kb], zb);
  // scores of the QT tiles: column h takes the high limb, column 8+h the low
  // limb, one MFMA per k-block; the two are folded after the last k-block
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    const float z = tpw == 1 ? zb[j & 3] : zb[(j >> 1) & 3];
    s[j] = floatx4{z + row_bias[0], z + row_bias[1], z + row_bias[2], z + row_bias[3]};
  }
  // the q*s operands are read two steps ahead of their MFMA, so that LDS
  // latency overlaps the matrix-core work instead of preceding every op
  auto bq_at = [&](int idx) {
    const int kb = idx / QT, j = idx % QT;
    return *(const half8 *)(c.qs_lds + (qt_win(j, tpw) * 2 * G + qrow) * QSTR<D> + kb * 32 + c.lq * 8);
  };
  half8 bqa = bq_at(0), bqb = bq_at(1);
#pragma unroll
  for (int idx = 0; idx < KB * QT; ++idx) {
    const int kb = idx / QT, j = idx % QT;
    const half8 bq = bqa;
    bqa = bqb;
    if (idx + 2 < KB * QT) bqb = bq_at(idx + 2);
    s[j] = mfma_f16_k32(key_codes<D, BITS>(buf, j, kb), bq, s[j]);
  }
  }
#pragma unroll
  for (int j = 0; j < QT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) s[j][i] = fold8(s[j][i]);
  // log2-domain logits.  Whether a tile holds tokens is uniform over the
  // wave, so an empty slot costs one scalar bias (-inf) instead of a
  // per-value mask; rows past a window shorter than a tile start from -inf
  // in the accumulator.  Columns without a head carry finite duplicates that
  // nothing reads.
  float x[QT][4];
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    const float bias = qt_win(j, tpw) < qb.nwin ? 0.0f : neg_inf();
#pragma unroll
    for (int i = 0; i < 4; ++i) x[j][i] = __builtin_fmaf(s[j][i], sc_quant, bias);
  }
  float p[QT][4], ts[QT];
  softmax_rows<D, QT>(ws, x, p, ts);
  // window masses: lane group lq ends with the sum over the 16 rows of
  // window slot lq (reduce-scatter over the four lane groups), which is the
  // slot its lanes store
  {
    const float a = tpw == 1 ? ts[0] : ts[0] + ts[1];
    const float b = tpw == 1 ? ts[1] : ts[2] + ts[3];
    const float cc = tpw == 1 ? ts[2] : 0.0f;
    const float d = tpw == 1 ? ts[3] : 0.0f;
    const float rho = reduce_scatter4(a, b, cc, d);
    const int slot = (c.lq < qb.nwin && c.col < G) ? qb.e + c.lq : g.U;
    *(float2 *)(c.mass_row + ((size_t)slot * G + (c.col & (G - 1))) * 2) = make_float2(rho, ws.m);
  }
  // value steps and zeros of the lane's tokens (all tiles, all group
  // batches): the LDS reads go out before the limb arithmetic below
  const half4 zero4 = {(half_t)0, (half_t)0, (half_t)0, (half_t)0};
  half4 sv[QT][NG / GP], zv[QT];
  {
    const int zc = c.col < NG ? c.col : 0;
#pragma unroll
    for (int j = 0; j < QT; ++j) {
#pragma unroll
      for (int gi = 0; gi < NG / GP; ++gi) {
        const int grp_l = gi * GP + (GP == 1 ? 0 : c.slot);
        sv[j][gi] = *(const half4 *)(c.vp_lds + j * PSTR<D> + (c.lq * NG + grp_l) * 8);
      }
      zv[j] = *(const half4 *)(c.vp_lds + j * PSTR<D> + (c.lq * NG + zc) * 8 + 4);
    }
  }
  // fp16 limbs of p; (P1, P2) = (0, phi) on hi lanes, (phi, plo) on lo lanes:
  // one FMA chain then yields fp16(p*s) on hi rows and the remainder on lo rows
  half4 P1[QT], P2[QT];
  const uint32_t lo_keep = c.is_lo ? 0xffffffffu : 0u;
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    // phi: p cut toward zero to fp16 (11 significant bits for p >= 2^-14);
    // plo: the exact fp32 remainder, rounded to fp16
    half4 phi, plo;
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const half2v h = rtz_pair(p[j][i], p[j][i + 1]);
      phi[i] = h[0];
      phi[i + 1] = h[1];
      plo[i] = lo_limb(h[0], p[j][i], neg1);
      plo[i + 1] = lo_limb(h[1], p[j][i + 1], neg1);
    }
    const uint2 ph = __builtin_bit_cast(uint2, phi), pl = __builtin_bit_cast(uint2, plo);
    P1[j] = __builtin_bit_cast(half4, make_uint2(ph.x & lo_keep, ph.y & lo_keep));
    P2[j] = __builtin_bit_cast(half4, make_uint2(c.is_lo ? pl.x : ph.x, c.is_lo ? pl.y : ph.y));
  }
  // PV over tile pairs: k slots = tokens 4*lq..+3 of tile 2pp, then of tile
  // 2pp+1.  The A operand scales p by the value step of one channel group;
  // with GP = 2 (four heads, each in two columns per limb) rows slot*G + h
  // take group gb + slot, so one operand serves two groups and each group's
  // MFMAs use its own rows.
#pragma unroll
  for (int pp = 0; pp < QT / 2; ++pp) {
    const int j0 = 2 * pp, j1 = 2 * pp + 1;
#pragma unroll
    for (int gb = 0; gb < NG; gb += GP) {
      const half4 s40 = sv[j0][gb / GP], s41 = sv[j1][gb / GP];
      const half4 t0 = P1[j0] * s40, t1 = P1[j1] * s41;
      const half4 ag0 = __builtin_elementwise_fma(P2[j0], s40, __builtin_elementwise_fma(P1[j0], s40, -t0));
      const half4 ag1 = __builtin_elementwise_fma(P2[j1], s41, __builtin_elementwise_fma(P1[j1], s41, -t1));
      const half8 ag = __builtin_shufflevector(ag0, ag1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int c2 = 0; c2 < 2 * GP; ++c2) {
        const int ct = gb * 2 + c2;
        const half4 b0 = value_codes<D, BITS>(buf, j0, ct), b1 = value_codes<D, BITS>(buf, j1, ct);
        const half8 bc = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        ws.acc[ct] = mfma_f16_k32(ag, bc, ws.acc[ct]);
      }
    }
    const half4 bz0 = c.col < NG ? zv[j0] : zero4, bz1 = c.col < NG ? zv[j1] : zero4;
    ws.zacc = mfma_f16_k32(__builtin_shufflevector(P2[j0], P2[j1], 0, 1, 2, 3, 4, 5, 6, 7),
                           __builtin_shufflevector(bz0, bz1, 0, 1, 2, 3, 4, 5, 6, 7), ws.zacc);
  }
  wave_lds_sync();
}

template <int D, int GP, int BITS, bool ROPE>
__device__ __forceinline__ void run_quant(WaveState<D> &ws, const Ctx &c, int ea, int eb) {
  if (ea >= eb) return;
  half8 qc[2], qp[2], bz[D / 32];
  const float sc_quant = query_f16<D>(c, qc, bz);
  // rotary keys: the compact query's pair partners (channel c +- D/2 sits
  // D/16 lanes away in the same head row)
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    uint4 w = __builtin_bit_cast(uint4, qc[r]);
    if (ROPE) {
      w.x = __shfl_xor(w.x, D / 16);
      w.y = __shfl_xor(w.y, D / 16);
      w.z = __shfl_xor(w.z, D / 16);
      w.w = __shfl_xor(w.w, D / 16);
    }
    qp[r] = __builtin_bit_cast(half8, w);
  }
  // rows of a tile past a window shorter than the tile hold no token
  float row_bias[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) row_bias[i] = 4 * c.lq + i < c.g->window ? 0.0f : neg_inf();
  const int per = QT / c.g->tpw;
  const int n_blocks = (eb - ea + per - 1) / per;
  // two-slot ring: one block in flight while one computes; unit ids two
  // blocks ahead (clamped, always valid); the loop body issues the same
  // loads on every trip, and the tail reads nothing past the run
  QBlock k0, k1;
  QBuf b0, b1;
  auto units = [&](int e0) { return ROPE ? ids_fetch(c, e0) : 0; };
  const int ids0 = slots_fetch(c, ea), un0 = units(ea);
  int ids1 = slots_fetch(c, ea + min(1, n_blocks - 1) * per), un1 = units(ea + min(1, n_blocks - 1) * per);
  qblock_make<ROPE>(c, ea, eb, 0, ids0, un0, k0);
  quant_load<D, BITS, ROPE>(c, k0, b0);
  // steady state: two blocks per trip, the following block always in flight
  int i = 0;
  for (; i + 2 < n_blocks; i += 2) {
    const int ids2 = slots_fetch(c, ea + min(i + 2, n_blocks - 1) * per), un2 = units(ea + min(i + 2, n_blocks - 1) * per);
    qblock_make<ROPE>(c, ea, eb, i + 1, ids1, un1, k1);
    quant_load<D, BITS, ROPE>(c, k1, b1);
    quant_compute<D, GP, BITS, ROPE>(ws, c, qc, qp, bz, sc_quant, row_bias, k0, b0);
    ids1 = slots_fetch(c, ea + min(i + 3, n_blocks - 1) * per);
    un1 = units(ea + min(i + 3, n_blocks - 1) * per);
    qblock_make<ROPE>(c, ea, eb, i + 2, ids2, un2, k0);
    quant_load<D, BITS, ROPE>(c, k0, b0);
    quant_compute<D, GP, BITS, ROPE>(ws, c, qc, qp, bz, sc_quant, row_bias, k1, b1);
  }
  // the last one or two blocks: nothing past the run is read
  if (i + 1 < n_blocks) {
    qblock_make<ROPE>(c, ea, eb, i + 1, ids1, un1, k1);
    quant_load<D, BITS, ROPE>(c, k1, b1);
    quant_compute<D, GP, BITS, ROPE>(ws, c, qc, qp, bz, sc_quant, row_bias, k0, b0);
    quant_compute<D, GP, BITS, ROPE>(ws, c, qc, qp, bz, sc_quant, row_bias, k1, b1);
  } else {
    quant_compute<D, GP, BITS, ROPE>(ws, c, qc, qp, bz, sc_quant, row_bias, k0, b0);
  }
}

// Waves per attention workgroup: one 8-wave workgroup per compute unit
// holds two waves on each SIMD.
constexpr int QW = 8;

template <int D, int GP, int BITS, bool ROPE>
__global__ __launch_bounds__(64 * QW) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_qevict_kernel(Geom g, State st, StepInfo si,
                                                            const uint16_t *__restrict__ q, float scale_log2,
                                                            const uint16_t *__restrict__ k_new,
                                                            const uint16_t *__restrict__ v_new) {
  constexpr int KB = D / 32;
  constexpr int CT = D / 16;
  const int S = g.n_splits;
  const int split = blockIdx.x % S;
  const int bh = blockIdx.x / S;
  const int h = bh % g.Hkv;
  const int b = bh / g.Hkv;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: ranges and loops stay scalar
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int lq = lane >> 4;
  constexpr int G = GP == 2 ? 4 : 8;   // the launcher passes GP = 2 exactly when G = 4 (G is 4 or 8)
  // Columns 0..7 take the high limb of quantized-tile scores, 8..15 the low
  // limb; within each half column c serves head (c mod 8) mod G, so with
  // fewer than 8 heads every head appears in several columns (identical
  // values) and no lane idles.
  const bool is_hi = col < 8;
  const bool is_lo = col >= 8;
  const int hc = (col & 7) & (G - 1);

  __shared__ __attribute__((aligned(16))) half_t s_kp[QW][QT][PSTR<D>];   // key scale/zero per window
  __shared__ __attribute__((aligned(16))) half_t s_vp[QW][QT][PSTR<D>];   // value params per tile
  __shared__ float sm_m[QW][8];
  __shared__ float sm_l[QW][8];
  __shared__ float sm_o[QW][8][D];
  // [QW][window slots][2][G][D+8] halfs; rotary keys: then [QW][QT][D] and
  // [16][RD_STR] floats (window-start rows, offset rows of the table)
  extern __shared__ __attribute__((aligned(16))) half_t s_qs[];

  // ---- this wave's share: slice gi of QW*S of the full-precision entries
  // (sink, ranked full, recent) and the same slice of the quantized windows,
  // so every workgroup (and so every XCD and CU) gets the same mix of
  // bandwidth-bound and arithmetic-bound work ----
  const EntryList L = make_list(g, st, si, b);
  const int A = L.s0 + L.nF, AQ = A + L.nQ, E = L.count();
  const int nB = A + (E - AQ);
  // The deal is static and fixed by (split, wave) alone, so every partial
  // sum, and with it every output and mass bit, is the same from run to run.
  const int NS = QW * S, gi = split * QW + wave;
  const int vb0 = (int)((long long)nB * gi / NS), vb1 = (int)((long long)nB * (gi + 1) / NS);
  const int q0 = A + (int)((long long)L.nQ * gi / NS), q1 = A + (int)((long long)L.nQ * (gi + 1) / NS);

  WaveState<D> ws;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) ws.acc[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
  ws.zacc = floatx4{0.f, 0.f, 0.f, 0.f};
  ws.m = neg_inf();
  ws.l = 0.0f;

  float *mass_row = st.mass_part + ((size_t)(b * g.Hkv + h) * (g.U + 1)) * G * 2;
  half_t *kp_lds = &s_kp[wave][0][0];
  half_t *vp_lds = &s_vp[wave][0][0];

  Ctx c;
  c.g = &g;
  c.st = &st;
  c.si = &si;
  c.L = &L;
  c.qrow = q + ((size_t)b * g.Hq + (size_t)h * G + hc) * D;
  c.qbase = q + ((size_t)b * g.Hq + (size_t)h * G) * D;
  c.hc = hc;
  c.b = b;
  c.h = h;
  c.lane = lane;
  c.col = col;
  c.lq = lq;
  c.G = G;
  c.is_hi = is_hi;
  c.is_lo = is_lo;
  c.has_q = true;
  c.slot = min((col & 7) / G, GP - 1);
  c.scale_log2 = scale_log2;
  c.mass_row = mass_row;
  c.ledger_h = (size_t)h * g.ledger_unit_bytes;
  c.ledger_stride = (size_t)g.Hkv * g.ledger_unit_bytes;
  c.kp_lds = kp_lds;
  c.vp_lds = vp_lds;
  const int qs_slots = ROPE ? QT : min(QT / g.tpw, QS_SLOTS<D, GP>);   // window slots of q*s limbs per wave
  c.qs_lds = s_qs + (size_t)wave * qs_slots * 2 * G * QSTR<D>;
  // Append folded into the launch (k_new, v_new: the step's token of every
  // (sequence, KV head), [B][Hkv][d]): lane l < d/4 of every wave loads
  // 16-byte chunk l of its K and V rows now (nothing waits for it here); the
  // one wave that reads the token's tile stages the chunks in LDS and patches
  // its row, and wave 0 of the split-0 workgroup stores the rows in the page
  // at the end (no wave of this launch reads that row from the page).
  __shared__ __attribute__((aligned(16))) uint16_t s_new[2 * D];
  const bool fused = !ROPE && k_new != nullptr;
  const int new_pos = si.N - 1;
  const int new_u = unit_of(g, new_pos), new_slot = new_pos - unit_start(g, new_u);
  c.new_u = fused ? new_u : -1;
  c.new_tile = new_slot / TS;
  c.new_row = new_slot % TS;
  c.new_kv = s_new;
  c.new_chunk = make_uint4(0u, 0u, 0u, 0u);
  if (!ROPE) {
    const int l = lane % (D / 4), kv = l / (D / 8), c0 = (l % (D / 8)) * 8;
    const uint16_t *src = fused ? (kv ? v_new : k_new) + (size_t)bh * D + c0 : q;   // q: any valid address
    c.new_chunk = *(const uint4 *)src;
  }
  if (ROPE) {
    float *rw = (float *)(s_qs + (size_t)QW * QT * 2 * G * QSTR<D>);
    float *rd = rw + QW * QT * D;
    c.rw_lds = rw + wave * QT * D;
    c.rd_lds = rd;
    // table rows 0..15 (the offsets of a window's tokens), D floats each
    for (int it = threadIdx.x; it < 16 * (D / 4); it += 64 * QW) {
      const int t = it / (D / 4), k = it % (D / 4);
      *(float4 *)(rd + t * RD_STR<D> + 4 * k) = *(const float4 *)(st.rope + (size_t)t * D + 4 * k);
    }
    __syncthreads();
  }
  // Opposite orders for the two waves that share a SIMD, whether the
  // workgroup's waves are dealt to the SIMDs round-robin (w, w+4) or in
  // pairs (2k, 2k+1): one streams full-precision tiles while the other
  // unpacks quantized ones.
  const int f0 = min(vb0, A), f1 = min(vb1, A);
  const int r0e = AQ + max(vb0 - A, 0), r1e = AQ + max(vb1 - A, 0);
  if (((wave & 1) ^ (wave >> 2)) & 1) {
    run_quant<D, GP, BITS, ROPE>(ws, c, q0, q1);
    run_full<D>(ws, c, f0, f1);      // sink and ranked full-precision windows
    run_full<D>(ws, c, r0e, r1e);    // windows not yet ranked
  } else {
    run_full<D>(ws, c, f0, f1);
    run_full<D>(ws, c, r0e, r1e);
    run_quant<D, GP, BITS, ROPE>(ws, c, q0, q1);
  }

  // ---- the appended token into its page (see above) ----
  if (fused && split == 0 && wave == 0) {
    uint16_t *kt = st.pages + page_offset(g, b, new_u, h) + (size_t)(new_slot / TS) * 2 * TS * D;
    const int kv = lane / (D / 8), c0 = (lane % (D / 8)) * 8;
    if (lane < D / 8) {
      *(uint4 *)(kt + k_tile_index(new_slot % TS, c0)) = c.new_chunk;
    } else if (lane < D / 4) {
      const uint16_t *e = (const uint16_t *)&c.new_chunk;
#pragma unroll
      for (int j = 0; j < 8; ++j) kt[TS * D + v_tile_index(new_slot % TS, c0 + j)] = e[j];
    }
    (void)kv;
    if (h == 0 && lane == 0) st.tier[b * g.U + new_u] = (new_u == 0) ? T_SINK : T_RECENT;
  }

  // ---- wave epilogue: fold value-zero term and limbs ----
  float l_tot = ws.l + __shfl_xor(ws.l, 16);
  l_tot += __shfl_xor(l_tot, 32);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.acc[ct][i] += __shfl(ws.zacc[i], lq * 16 + (ct >> 1));
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.acc[ct][i] += __shfl_down(ws.acc[ct][i], 32);   // rows 8+h onto rows h

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
  const size_t pbase = ((size_t)(b * g.Hkv + h) * S + split) * G;
  for (int it = threadIdx.x; it < G * D; it += blockDim.x) {
    const int hh = it / D, c = it % D;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < QW; ++w) M = fmaxf(M, sm_m[w][hh]);
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < QW; ++w)
      if (sm_m[w][hh] != neg_inf()) o += sm_o[w][hh][c] * exp2f(sm_m[w][hh] - M);
    st.part_o[(pbase + hh) * D + c] = o;
    if (c == 0) {
      float l = 0.0f;
#pragma unroll
      for (int w = 0; w < QW; ++w)
        if (sm_m[w][hh] != neg_inf()) l += sm_l[w][hh] * exp2f(sm_m[w][hh] - M);
      st.part_ml[(pbase + hh) * 2 + 0] = M;
      st.part_ml[(pbase + hh) * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// merge: outputs per (sequence, KV head); masses -> window scores per sequence
// ---------------------------------------------------------------------------

// global (max, 1/sum) of head hh of KV head h over the splits
__device__ inline void split_stats(const Geom &g, const State &st, int b, int h, int hh, float &M, float &invL) {
  constexpr int CH = 8;   // splits whose (max, sum) loads are issued together
  const int S = g.n_splits, G = g.G;
  const float2 *ml = (const float2 *)st.part_ml + (size_t)(b * g.Hkv + h) * S * G + hh;
  float m = neg_inf(), l = 0.0f;
  for (int s0 = 0; s0 < S; s0 += CH) {
    float2 p[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) p[k] = ml[(size_t)min(s0 + k, S - 1) * G];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      if (s0 + k >= S || p[k].x == neg_inf()) continue;
      const float mn = fmaxf(m, p[k].x);
      l = (m == neg_inf() ? 0.0f : l * exp2f(m - mn)) + p[k].y * exp2f(p[k].x - mn);
      m = mn;
    }
  }
  M = m;
  invL = 1.0f / l;
}

// Entries per mass block of the merge (four lanes per entry).
constexpr int MERGE_ENTRIES = 64;

template <int G>
__global__ __launch_bounds__(256) void merge_qevict_kernel(Geom g, State st, StepInfo si, float *__restrict__ out,
                                                           float *__restrict__ mass_out, int n_chunks) {
  constexpr int CH = 4;   // splits whose loads are issued together
  const int S = g.n_splits, D = g.d;
  const int n_out_blocks = g.B * g.Hkv;
  __shared__ float sM[128], sInvL[128];   // Hkv*G = Hq <= 128
  __shared__ float sPart[4][MERGE_ENTRIES];
  if ((int)blockIdx.x < n_out_blocks) {
    // outputs of one (sequence, KV head): each thread folds the split
    // partials of its outputs with the LSE rule on its own
    const int b = blockIdx.x / g.Hkv, h = blockIdx.x % g.Hkv;
    const float2 *ml = (const float2 *)st.part_ml + (size_t)(b * g.Hkv + h) * S * G;
    const float *po = st.part_o + (size_t)(b * g.Hkv + h) * S * G * D;
    merge_outputs<G, CH>(ml, po, S, D, out + ((size_t)b * g.Hq + (size_t)h * G) * D);
    return;
  }
  // masses of MERGE_ENTRIES live entries of one sequence -> list-order scores:
  // lane q of an entry's four sums the KV heads h = q, q + 4, ... (in that
  // order), and the four partial sums are added in order q = 0..3; the old
  // score and the lane's (rho, m) pairs are loaded before the wait for the
  // split statistics
  const int mb = blockIdx.x - n_out_blocks;
  const int b = mb / n_chunks, chunk = mb % n_chunks;
  const EntryList L = make_list(g, st, si, b);
  const int E = L.count();
  const int el = threadIdx.x % MERGE_ENTRIES, q = threadIdx.x / MERGE_ENTRIES;
  const int e = chunk * MERGE_ENTRIES + el;
  const int ee = min(e, E - 1);
  const int u_out = mass_out ? entry_unit(L, st.routed + b * g.U, ee) : 0;
  // the entry's list-order score: no other thread of the launch touches it
  const float old_score = q == 0 ? st.slist[b * g.U + ee] : 0.0f;
  constexpr int HPL = 2;   // KV heads per lane whose loads go out together
  float4 mp[HPL][G / 2];
  auto load_heads = [&](int h0) {
#pragma unroll
    for (int k = 0; k < HPL; ++k) {
      const int h = min(h0 + 4 * k, g.Hkv - 1);
      const float4 *src = (const float4 *)(st.mass_part + ((size_t)(b * g.Hkv + h) * (g.U + 1) + ee) * G * 2);
#pragma unroll
      for (int j = 0; j < G / 2; ++j) mp[k][j] = src[j];
    }
  };
  load_heads(q);
  for (int it = threadIdx.x; it < g.Hkv * G; it += blockDim.x) split_stats(g, st, b, it / G, it % G, sM[it], sInvL[it]);
  __syncthreads();
  float part = 0.0f;
  for (int h0 = q; h0 < g.Hkv; h0 += 4 * HPL) {
    if (h0 > q) load_heads(h0);
#pragma unroll
    for (int k = 0; k < HPL; ++k) {
      const int h = h0 + 4 * k;
      if (h >= g.Hkv) break;
      float gs = 0.0f;
#pragma unroll
      for (int j = 0; j < G / 2; ++j) {
        const float r2[2] = {mp[k][j].x, mp[k][j].z}, m2[2] = {mp[k][j].y, mp[k][j].w};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int hh = 2 * j + t;
          float v = (m2[t] == neg_inf()) ? 0.0f : r2[t] * exp2f(m2[t] - sM[h * G + hh]) * sInvL[h * G + hh];
          if (!(v >= 1.17549435e-38f)) v = 0.0f;   // a head's mass below FLT_MIN counts as 0
          gs += v;
        }
      }
      if (mass_out && e < E) mass_out[((size_t)b * g.Hkv + h) * g.U + u_out] = gs;
      part += gs;
    }
  }
  sPart[q][el] = part;
  __syncthreads();
  if (q == 0 && e < E) {
    const float total = (sPart[0][el] + sPart[1][el]) + (sPart[2][el] + sPart[3][el]);
    st.slist[b * g.U + e] = old_score + total;
  }
}

// LDS of one attention workgroup beyond its static arrays: the q*s limbs of
// every window slot of every wave
static size_t attend_qs_bytes(const Geom &g) {
  const int slots = g.rope ? QT : min(QT / g.tpw, (g.G == 8 && g.d == 128) ? QT / 2 : QT);   // QS_SLOTS
  size_t n = (size_t)QW * slots * 2 * g.G * (g.d + 8) * sizeof(half_t);
  if (g.rope) n += ((size_t)QW * QT * g.d + 16 * (size_t)(g.d + 4)) * sizeof(float);   // RD_STR
  return n;
}

// the attention kernel of a configuration: head dimension, four or eight heads
// per KV head (paired channel groups with four), 2- or 4-bit quantized tier,
// keys with or without the rotary embedding around the quantized tier
template <int D, int GP, bool ROPE>
static const void *attend_fn_bits(int bits) {
  return bits == 4 ? (const void *)attend_qevict_kernel<D, GP, 4, ROPE>
                   : (const void *)attend_qevict_kernel<D, GP, 2, ROPE>;
}
template <bool ROPE>
static const void *attend_fn_rope(const Geom &g) {
  if (g.d == 128) return g.G == 4 ? attend_fn_bits<128, 2, ROPE>(g.bits) : attend_fn_bits<128, 1, ROPE>(g.bits);
  return g.G == 4 ? attend_fn_bits<64, 2, ROPE>(g.bits) : attend_fn_bits<64, 1, ROPE>(g.bits);
}
static const void *attend_fn(const Geom &g) { return g.rope ? attend_fn_rope<true>(g) : attend_fn_rope<false>(g); }

hipError_t attend_lds_fits(const Geom &g, bool *fits) {
  hipFuncAttributes a;
  hipError_t e = hipFuncGetAttributes(&a, attend_fn(g));
  if (e != hipSuccess) return e;
  int dev = 0, max_lds = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev)) != hipSuccess) return e;
  *fits = a.sharedSizeBytes + attend_qs_bytes(g) <= (size_t)max_lds;
  return hipSuccess;
}

hipError_t launch_attend(const Geom &g, const State &st, const StepInfo &si, const uint16_t *q, float *out,
                         float *mass_out, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop,
                         const uint16_t *k_new, const uint16_t *v_new) {
  float scale_log2 = (float)(1.4426950408889634 / sqrt((double)g.d));
  const int grid = g.B * g.Hkv * g.n_splits;
  size_t qs_bytes = attend_qs_bytes(g);
  // The optional events are attached to the dispatch itself, so they time
  // the kernel's execution (no launch gap).
  Geom ga = g;
  State sa = st;
  StepInfo sia = si;
  const uint16_t *qa = q, *ka = k_new, *va = v_new;
  void *args[] = {&ga, &sa, &sia, &qa, &scale_log2, &ka, &va};
  hipError_t e = hipExtLaunchKernel(attend_fn(g), dim3(grid), dim3(64 * QW), args, qs_bytes, s, ev_start, ev_stop, 0);
  if (e != hipSuccess) return e;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (mass_out) {
    e = launch_clear(mass_out, (size_t)g.B * g.Hkv * g.U * sizeof(float), s);
    if (e != hipSuccess) return e;
  }
  const int n_live = si.has_sink + si.n_routed + (si.r1 >= si.r0 ? si.r1 - si.r0 + 1 : 0);   // entries this step
  const int n_chunks = (n_live + MERGE_ENTRIES - 1) / MERGE_ENTRIES;
  const dim3 mgrid(g.B * g.Hkv + g.B * n_chunks);
  if (g.G == 4)
    hipLaunchKernelGGL(merge_qevict_kernel<4>, mgrid, dim3(256), 0, s, g, st, si, out, mass_out, n_chunks);
  else
    hipLaunchKernelGGL(merge_qevict_kernel<8>, mgrid, dim3(256), 0, s, g, st, si, out, mass_out, n_chunks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// routing event: rank candidates per sequence in LDS (bitonic), assign tiers
// ---------------------------------------------------------------------------

// One key per thread (64 <= n <= blockDim.x, n a power of two): the
// compare-exchange partner of a stage with distance j < 64 is in the same
// wave and is read with a lane permute, so only the stages with j >= 64 go
// through LDS and a workgroup barrier (10 of the 55 stages at n = 1024).
__device__ inline void bitonic_desc_u64_regs(unsigned long long *keys, int n) {
  const int i = threadIdx.x;
  const bool mine = i < n;   // whole waves (n is a multiple of 64)
  unsigned long long key = mine ? keys[i] : 0ull;
  for (int k = 2; k <= n; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      unsigned long long other;
      if (j >= 64) {
        __syncthreads();
        if (mine) keys[i] = key;
        __syncthreads();
        other = mine ? keys[i ^ j] : 0ull;
      } else {
        const uint32_t lo = __shfl_xor((uint32_t)key, j), hi = __shfl_xor((uint32_t)(key >> 32), j);
        other = ((unsigned long long)hi << 32) | lo;
      }
      // the lower index of a pair keeps the larger key in a descending run
      const bool keep_max = ((i & j) == 0) == ((i & k) == 0);
      key = keep_max ? (key > other ? key : other) : (key < other ? key : other);
    }
  __syncthreads();
  if (mine) keys[i] = key;
  __syncthreads();
}

__device__ inline void bitonic_desc_u64(unsigned long long *keys, int n) {
  if (n >= 64 && n <= (int)blockDim.x) {
    bitonic_desc_u64_regs(keys, n);
    return;
  }
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

__global__ __launch_bounds__(1024) void route_qevict_kernel(Geom g, State st, StepInfo si, int a0, int a1, int npow) {
  extern __shared__ unsigned long long keys[];
  __shared__ int n_pack, n_prom, n_free, n_reuse, n_demote, s_top;
  const int b = blockIdx.x;
  const int nF = st.routed_nf[b], nQ = st.routed_nq[b];
  const int RC = nF + nQ;
  const int n = RC + (a1 > a0 ? a1 - a0 : 0);
  if (threadIdx.x == 0) {
    n_pack = 0;
    n_prom = 0;
    n_free = 0;
    n_reuse = 0;
    n_demote = 0;
  }
  // Candidate i sits at entry s0 + i of the list so far (the ranked windows,
  // then the windows aged since the last event, which lead the recent ones):
  // its list-order score is its key and goes back to its unit's score.  The
  // sink and the windows that stay recent (a1 .. r1) go back too.
  const int s0 = si.has_sink;
  const float *sl = st.slist + (size_t)b * g.U;
  const int n_keep = si.r1 >= a1 ? si.r1 - a1 + 1 : 0;
  for (int i = threadIdx.x; i < npow; i += blockDim.x) {
    unsigned long long key = 0ull;
    if (i < n) {
      const int u = i < RC ? st.routed[b * g.U + i] : a0 + (i - RC);
      const float sc = sl[s0 + i];
      st.score[b * g.U + u] = sc;
      key = ((unsigned long long)__float_as_uint(sc) << 32) |   // scores are >= 0: bits are monotone
            (unsigned long long)(uint32_t)(unit_start(g, u) + 1);
    }
    keys[i] = key;
  }
  for (int k = threadIdx.x; k < n_keep; k += blockDim.x) st.score[b * g.U + a1 + k] = sl[s0 + n + k];
  if (s0 && threadIdx.x == 0) st.score[b * g.U] = sl[0];
  __syncthreads();
  bitonic_desc_u64(keys, npow);
  const int KFQ = g.k_full + g.k_quant;
  for (int r = threadIdx.x; r < n; r += blockDim.x) {
    const int start = (int)(uint32_t)(keys[r] & 0xffffffffull) - 1;
    const int u = unit_of(g, start);
    const int idx = b * g.U + u;
    const uint8_t old = st.tier[idx];
    const uint8_t nt = r < g.k_full ? T_FULL : (r < KFQ ? T_QUANT : T_EVICTED);
    if (nt == T_QUANT && old != T_QUANT) {
      atomicAdd(&n_demote, 1);
      if (st.has_ledger[idx]) atomicAdd(&n_reuse, 1);
    }
    if (nt == T_QUANT && !st.has_ledger[idx]) {
      const int p = atomicAdd(&n_pack, 1);
      st.pack_list[b * g.U + p] = u;
      st.has_ledger[idx] = 1;
    }
    if (r >= KFQ) st.victims[b * g.U + (r - KFQ)] = u;
    if (nt == T_FULL && old == T_QUANT) {
      const int p = atomicAdd(&n_prom, 1);
      st.promote_list[b * g.U + p] = u;
    }
    if (nt == T_EVICTED && st.has_ledger[idx]) {   // its ledger slot goes back to the pool
      const int p = atomicAdd(&n_free, 1);
      st.free_list[b * g.U + p] = u;
      st.has_ledger[idx] = 0;
    }
    st.tier[idx] = nt;
    if (r < KFQ) st.routed[b * g.U + r] = u;
  }
  __syncthreads();
  // ledger slots: the evicted windows' go back on this (layer, sequence)'s
  // stack, then the windows packed for the first time take theirs (a failed
  // pop is latched and leaves the window without codes, never an
  // out-of-range access); then the new list's quantized entries get their
  // slots (qslot), which the attention kernel reads instead of window ids
  {
    const int range = st.layer * g.B + b, per = g.pool_per;
    int32_t *stack = st.pool_stack + (size_t)range * per;
    if (threadIdx.x == 0) s_top = st.pool_top[range];
    __syncthreads();
    for (int i = threadIdx.x; i < n_free; i += blockDim.x) {
      const int u = st.free_list[b * g.U + i];
      const int slot = st.lslot[b * g.U + u] - 1;
      st.lslot[b * g.U + u] = 0;
      if (slot < 0) continue;
      const int p = atomicAdd(&s_top, 1);
      if (p >= 0 && p < per)
        stack[p] = slot;
      else
        st.status[0] = QKV_ECAPACITY;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n_pack; i += blockDim.x) {
      const int u = st.pack_list[b * g.U + i];
      const int p = atomicSub(&s_top, 1) - 1;
      int slot = -1;
      if (p >= 0 && p < per)
        slot = stack[p];
      else
        st.status[0] = QKV_ECAPACITY;
      st.lslot[b * g.U + u] = slot + 1;
    }
    __syncthreads();
    if (threadIdx.x == 0) st.pool_top[range] = max(s_top, 0);
  }
  const int nF2 = min(n, g.k_full), nQ2 = max(0, min(n - g.k_full, g.k_quant));
  for (int r = nF2 + threadIdx.x; r < nF2 + nQ2; r += blockDim.x)
    st.qslot[b * g.U + r] = st.lslot[b * g.U + st.routed[b * g.U + r]] - 1;
  if (threadIdx.x == 0) {
    st.routed_nf[b] = nF2;
    st.routed_nq[b] = nQ2;
    st.pack_count[b] = n_pack;
    st.promote_count[b] = n_prom;
    st.free_count[b] = n_free;
    // the event record: counters and the relative score gaps across the cuts
    // (lowest kept minus highest dropped) of the sorted keys
    auto margin = [&](int cut) {
      if (cut <= 0 || cut >= n) return __builtin_inff();
      const float hi = __uint_as_float((uint32_t)(keys[cut - 1] >> 32)), lo = __uint_as_float((uint32_t)(keys[cut] >> 32));
      return (hi - lo) / fmaxf(fmaxf(fabsf(hi), fabsf(lo)), 1.17549435e-38f);
    };
    int32_t *ev = st.event + (size_t)b * EV_WORDS;
    const float mf = margin(g.k_full), mq = margin(KFQ);
    ev[EV_TOKENS] = si.N;
    ev[EV_CANDIDATES] = n;
    ev[EV_FULL] = nF2;
    ev[EV_QUANT] = nQ2;
    ev[EV_EVICTED] = n - nF2 - nQ2;
    ev[EV_PROMOTED] = n_prom;
    ev[EV_DEMOTED] = n_demote;
    ev[EV_FIRST_PACKS] = n_pack;
    ev[EV_REUSED] = n_reuse;
    ev[EV_FREED] = n_free;
    ev[EV_MARGIN_FULL] = __float_as_int(mf);
    ev[EV_MARGIN_QUANT] = __float_as_int(mq);
    ev[EV_MARGIN_MIN] = __float_as_int(fminf(mf, mq));
  }
  // list-order scores of the new list: the sink's is unchanged, the ranked
  // windows' are in their sorted keys, the recent windows' were written back
  // above; the slots past the list belong to windows not yet appended (0)
  {
    const int nFQ2 = nF2 + nQ2, E = s0 + nFQ2 + n_keep;
    for (int e = threadIdx.x; e < g.U; e += blockDim.x) {
      float v = 0.0f;
      if (e < s0)
        v = st.score[b * g.U];
      else if (e - s0 < nFQ2)
        v = __uint_as_float((uint32_t)(keys[e - s0] >> 32));
      else if (e < E)
        v = st.score[b * g.U + a1 + (e - s0 - nFQ2)];
      st.slist[b * g.U + e] = v;
      if (e >= n - nFQ2) st.victims[b * g.U + e] = -1;   // past this event's victims
    }
  }
}

// list-order scores -> per-unit scores of the live entries (before an export)
__global__ __launch_bounds__(256) void slist_sync_kernel(Geom g, State st, StepInfo si) {
  const int b = blockIdx.y;
  const EntryList L = make_list(g, st, si, b);
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < L.count()) st.score[b * g.U + entry_unit(L, st.routed + b * g.U, e)] = st.slist[b * g.U + e];
}

// Ledger pool: one range of pool_per slots per (layer, sequence), enough for
// the K_f + K_q windows it can hold; its free slots are a stack that only the
// routing workgroup of that (layer, sequence) touches.
__global__ void pool_init_kernel(int32_t *stack, int32_t *top, int n, int per) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) stack[i] = i;
  const int n_ranges = per > 0 ? n / per : 0;
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < n_ranges; r += gridDim.x * blockDim.x) top[r] = per;
}

hipError_t launch_pool_init(const Geom &g, const State &st, hipStream_t s) {
  hipLaunchKernelGGL(pool_init_kernel, dim3(64), dim3(256), 0, s, st.pool_stack, st.pool_top, g.pool_slots, g.pool_per);
  return hipGetLastError();
}

// pack (first demotion) and promote (quantized -> full) of listed windows;
// one (window, KV head) item at a time per 256-thread workgroup.  Every
// thread moves whole 16-byte tile chunks: a key chunk is 8 channels of one
// token, a value chunk 4 tokens of two channels (c, c + 16).
constexpr int TR_THREADS = 256;
template <int D> constexpr int TR_ROW = D + 8;   // LDS row (bf16), 16-byte aligned, rows on distinct banks

template <int D, int BITS>
__global__ __launch_bounds__(TR_THREADS) __attribute__((amdgpu_waves_per_eu(6))) void transitions_qevict_kernel(
    Geom g, State st, int per_seq) {
  constexpr int DPL = D * BITS / 64;   // code dwords per lane per tile
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  constexpr int CHUNKS = TS * D / 8;   // 16-byte chunks per K (or V) tile
  static_assert(CHUNKS <= TR_THREADS && D + 32 * (D / 32) <= TR_THREADS, "workgroup too small");
  __shared__ __attribute__((aligned(16))) uint16_t sk[2 * TS][TR_ROW<D>];   // bf16 of the window, [token][channel]
  __shared__ __attribute__((aligned(16))) uint16_t sv[2 * TS][TR_ROW<D>];
  __shared__ half_t s_ks[D], s_kz[D];
  __shared__ half_t s_vs[2 * TS][D / 32], s_vz[2 * TS][D / 32];
  const int b = blockIdx.x / per_seq;
  const int w0 = blockIdx.x % per_seq;
  const int npk = st.pack_count[b];
  const int npr = st.promote_count[b];
  const int items = (npk + npr) * g.Hkv;
  const int W = g.window, tpw = g.tpw;
  const float levels = (float)MASK;
  const int ci = threadIdx.x;
  const bool own = ci < CHUNKS;   // threads with a key and a value chunk of each tile
  // key chunk ci: token kt_t, channels kt_c .. +7; value chunk ci: tokens
  // 4 vt_q .. +3 of channels vt_c and vt_c + 16
  const int kt_t = ci % 16, kt_c = (ci / 64) * 32 + ((ci % 64) / 16) * 8;
  const int vt_q = (ci % 64) / 16, vt_c = (ci / 64) * 32 + ci % 16;
  // window of item it (the next item's is fetched while this one is worked on)
  auto item_unit = [&](int it) {
    const int i = min(it, items - 1) / g.Hkv;
    return i < npk ? st.pack_list[b * g.U + i] : st.promote_list[b * g.U + (i - npk)];
  };
  int u_next = items > w0 ? item_unit(w0) : 0;
  for (int it = w0; it < items; it += per_seq) {
    const int i = it / g.Hkv, h = it % g.Hkv;
    const bool pack = i < npk;
    const int u = u_next;
    u_next = item_unit(it + per_seq);
    uint16_t *pg = st.pages + page_offset(g, b, u, h);
    const int slot = st.lslot[b * g.U + u] - 1;
    if (slot < 0) continue;   // no slot (a latched pool error): nothing to pack or promote
    uint8_t *Lb = st.ledger + ledger_slot_offset(g, slot, h);
    half_t *kparam = (half_t *)Lb;
    if (pack) {
      // 1. tiles -> LDS in logical order (all loads issued before the stores)
      if (own) {
        uint4 kch[2], vch[2];
        // with the rotary embedding the ledger quantizes the keys as appended
        const uint16_t *kraw = g.rope ? st.kraw + kraw_offset(g, b, u, h) : nullptr;
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
          const uint16_t *kt = pg + (size_t)min(tile, tpw - 1) * 2 * TS * D;
          const uint16_t *ks = g.rope ? kraw + (size_t)min(tile, tpw - 1) * TS * D : kt;
          kch[tile] = *(const uint4 *)(ks + ci * 8);
          vch[tile] = *(const uint4 *)(kt + TS * D + ci * 8);
        }
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
          if (tile >= tpw) break;
          *(uint4 *)&sk[tile * TS + kt_t][kt_c] = kch[tile];
          const uint16_t *e = (const uint16_t *)&vch[tile];
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int j = 0; j < 4; ++j) sv[tile * TS + 4 * vt_q + j][vt_c + 16 * hf] = e[hf * 4 + j];
        }
      }
      __syncthreads();
      // 2. key parameters per channel over the window's tokens (threads
      // 0 .. D-1); value parameters per token and 32-channel group (the
      // upper half of the workgroup)
      if (ci < D) {
        const int c = ci;
        float mn = bf16_to_f32(sk[0][c]), mx = mn;
        for (int t0 = 0; t0 < W; t0 += 8)
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float x = bf16_to_f32(sk[t0 + k][c]);
            mn = min_nan(mn, x);
            mx = max_nan(mx, x);
          }
        const half_t s16 = (half_t)((mx - mn) / levels);
        const half_t z16 = (half_t)mn;
        if (!isfinite((float)s16) || !isfinite((float)z16)) st.status[0] = QKV_ERANGE;
        s_ks[c] = s16;
        s_kz[c] = z16;
        kparam[c] = s16;
        kparam[D + c] = z16;
      }
      if (ci >= TR_THREADS - W * (D / 32)) {
        const int it2 = ci - (TR_THREADS - W * (D / 32));
        const int t = it2 / (D / 32), grp = it2 % (D / 32);
        const uint4 *row = (const uint4 *)&sv[t][grp * 32];
        float mn = bf16_to_f32(sv[t][grp * 32]), mx = mn;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint4 r = row[q4];
          const uint16_t *e = (const uint16_t *)&r;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = bf16_to_f32(e[j]);
            mn = min_nan(mn, x);
            mx = max_nan(mx, x);
          }
        }
        const half_t s16 = (half_t)((mx - mn) / levels);
        const half_t z16 = (half_t)mn;
        if (!isfinite((float)s16) || !isfinite((float)z16)) st.status[0] = QKV_ERANGE;
        s_vs[t][grp] = s16;
        s_vz[t][grp] = z16;
        half_t *vp = (half_t *)(Lb + g.kparam_bytes + (t / TS) * g.tile_block_bytes + g.tile_kcode_bytes +
                                g.tile_vcode_bytes);
        vp[vparam_index(g, t % TS, grp, 0)] = s16;
        vp[vparam_index(g, t % TS, grp, 1)] = z16;
      }
      __syncthreads();
      // 3. codes in the matrix-core operand order: one thread per (tile, lane,
      // code dword), walking its slots (the inverse of kcode_slot / vcode_slot)
      for (int dw2 = ci; dw2 < tpw * 64 * DPL; dw2 += TR_THREADS) {
        const int tile = dw2 / (64 * DPL), r = dw2 % (64 * DPL), l = r / DPL, w = r % DPL;
        uint32_t word = 0u;
#pragma unroll
        for (int p = 0; p < 32 / BITS; ++p) {
          int t, c;
          const bool key = code_slot_elem(l, w, p, D, BITS, t, c);
          const int tt = tile * TS + t;
          uint32_t code = 0u;
          if (tt < W)
            code = key ? quant_code(bf16_to_f32(sk[tt][c]), s_ks[c], s_kz[c], levels)
                       : quant_code(bf16_to_f32(sv[tt][c]), s_vs[tt][c / 32], s_vz[tt][c / 32], levels);
          word |= code << (BITS * p);
        }
        ((uint32_t *)(Lb + g.kparam_bytes + tile * g.tile_block_bytes))[l * DPL + w] = word;
      }
      __syncthreads();
    } else {
      // promote: rebuild the full-precision tiles from the ledger, one key
      // chunk and one value chunk per thread and tile
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        if (tile >= tpw || !own) break;
        const uint8_t *T = Lb + g.kparam_bytes + tile * g.tile_block_bytes;
        const uint32_t *tc = (const uint32_t *)T;
        const half_t *vp = (const half_t *)(T + g.tile_kcode_bytes + g.tile_vcode_bytes);
        uint16_t *kt = pg + (size_t)tile * 2 * TS * D;
        // keys: the chunk's 8 channels share one code dword (kcode_slot)
        int kdw, vdw, sh;
        kcode_slot(kt_t, kt_c, D, BITS, kdw, sh);
        vcode_slot(4 * vt_q, vt_c, D, BITS, vdw, sh);
        const uint32_t kw = tc[kdw], vw = tc[vdw];
        const uint4 ks4 = *(const uint4 *)(kparam + kt_c), kz4 = *(const uint4 *)(kparam + D + kt_c);
        const uint4 vpar = *(const uint4 *)(vp + vparam_index(g, 4 * vt_q, vt_c / 32, 0));
        const half_t *ks = (const half_t *)&ks4, *kz = (const half_t *)&kz4, *vps = (const half_t *)&vpar;
        uint4 ko, vo;
        uint16_t *ke = (uint16_t *)&ko, *ve = (uint16_t *)&vo;
        if (!g.rope) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kcode_slot(kt_t, kt_c + e, D, BITS, kdw, sh);
            const float kcode = (float)((kw >> sh) & MASK);
            ke[e] = f32_to_bf16_rne(__builtin_fmaf(kcode, (float)ks[e], (float)kz[e]));
          }
          *(uint4 *)(kt + ci * 8) = ko;
        } else if (ci < CHUNKS / 2) {
          // rotary keys: the dequantized pair (kt_c + e, kt_c + e + D/2) is
          // rotated again at the token's position (chunk ci + CHUNKS/2 holds
          // the upper channels)
          int kdw2;
          kcode_slot(kt_t, kt_c + D / 2, D, BITS, kdw2, sh);
          const uint32_t kw2 = tc[kdw2];
          const uint4 ks24 = *(const uint4 *)(kparam + kt_c + D / 2), kz24 = *(const uint4 *)(kparam + D + kt_c + D / 2);
          const half_t *ks2 = (const half_t *)&ks24, *kz2 = (const half_t *)&kz24;
          const int row = min(unit_start(g, u) + tile * TS + kt_t, st.rope_n - 1);   // rows past the window hold no token
          const float4 *cs4 = (const float4 *)(st.rope + ((size_t)row * (D / 2) + kt_c) * 2);
          float4 cs[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) cs[j] = cs4[j];
          uint4 ko2;
          uint16_t *ke2 = (uint16_t *)&ko2;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kcode_slot(kt_t, kt_c + e, D, BITS, kdw, sh);
            const float xl = __builtin_fmaf((float)((kw >> sh) & MASK), (float)ks[e], (float)kz[e]);
            kcode_slot(kt_t, kt_c + D / 2 + e, D, BITS, kdw2, sh);
            const float xh = __builtin_fmaf((float)((kw2 >> sh) & MASK), (float)ks2[e], (float)kz2[e]);
            const float ce = (e & 1) ? cs[e >> 1].z : cs[e >> 1].x, se = (e & 1) ? cs[e >> 1].w : cs[e >> 1].y;
            float rl, rh;
            rope_pair(xl, xh, ce, se, rl, rh);
            ke[e] = f32_to_bf16_rne(rl);
            ke2[e] = f32_to_bf16_rne(rh);
          }
          *(uint4 *)(kt + ci * 8) = ko;
          *(uint4 *)(kt + (ci + CHUNKS / 2) * 8) = ko2;
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            vcode_slot(4 * vt_q + j, vt_c + 16 * hf, D, BITS, vdw, sh);
            const float vcode = (float)((vw >> sh) & MASK);
            ve[hf * 4 + j] = f32_to_bf16_rne(__builtin_fmaf(vcode, (float)vps[j], (float)vps[4 + j]));
          }
        *(uint4 *)(kt + TS * D + ci * 8) = vo;
      }
    }
  }
}

// pack/promote workgroups per sequence: as many as the device holds at once
// (the lists of a routing event are short after the first one)
hipError_t transitions_shape(Geom &g) {
  int dev = 0, n_cu = 0, per_cu = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  const void *f = g.d == 128 ? (g.bits == 4 ? (const void *)transitions_qevict_kernel<128, 4>
                                             : (const void *)transitions_qevict_kernel<128, 2>)
                             : (g.bits == 4 ? (const void *)transitions_qevict_kernel<64, 4>
                                             : (const void *)transitions_qevict_kernel<64, 2>);
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, TR_THREADS, 0)) != hipSuccess) return e;
  g.tr_per_seq = per_cu * n_cu / g.B > 1 ? per_cu * n_cu / g.B : 1;
  return hipSuccess;
}

hipError_t launch_route(const Geom &g, const State &st, const StepInfo &si, int a0, int a1, int n_cand,
                        hipStream_t s) {
  int bound = n_cand > 1 ? n_cand : 1;   // ranked windows + newly aged windows (same for every sequence)
  int npow = 1;
  while (npow < bound) npow <<= 1;
  if (npow > ROUTE_SORT_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(route_qevict_kernel, dim3(g.B), dim3(1024), npow * sizeof(unsigned long long), s, g, st, si, a0,
                     a1, npow);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int per_seq = g.tr_per_seq > 0 ? g.tr_per_seq : 128;
  const dim3 tg(g.B * per_seq), tb(TR_THREADS);
  if (g.d == 128 && g.bits == 4)
    hipLaunchKernelGGL((transitions_qevict_kernel<128, 4>), tg, tb, 0, s, g, st, per_seq);
  else if (g.d == 128)
    hipLaunchKernelGGL((transitions_qevict_kernel<128, 2>), tg, tb, 0, s, g, st, per_seq);
  else if (g.bits == 4)
    hipLaunchKernelGGL((transitions_qevict_kernel<64, 4>), tg, tb, 0, s, g, st, per_seq);
  else
    hipLaunchKernelGGL((transitions_qevict_kernel<64, 2>), tg, tb, 0, s, g, st, per_seq);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// stateless quantizer (canonical layout)
// ---------------------------------------------------------------------------

__device__ inline float load_x(const void *x, int dtype, size_t i) {
  return dtype == QKV_DTYPE_F32 ? ((const float *)x)[i] : bf16_to_f32(((const uint16_t *)x)[i]);
}

__global__ __launch_bounds__(256) void quantize_window_kernel(const void *__restrict__ x, int dtype, int n_blocks,
                                                              int tokens, int D, int bits, int group, int kind,
                                                              uint8_t *__restrict__ codes,
                                                              uint16_t *__restrict__ params) {
  const int per_byte = 8 / bits;
  const float levels = (float)((1 << bits) - 1);
  const size_t block_elems = (size_t)tokens * D;
  const size_t block_code_bytes = (block_elems * bits + 7) / 8;
  long long n_groups;
  int n_chunks = (tokens + group - 1) / group;
  if (kind == QKV_KIND_K_PER_CHANNEL) n_groups = (long long)D * n_chunks;
  else if (kind == QKV_KIND_PER_TOKEN) n_groups = (long long)tokens * (D / group);
  else n_groups = tokens;
  const long long total = n_groups * n_blocks;
  for (long long it = (long long)blockIdx.x * blockDim.x + threadIdx.x; it < total;
       it += (long long)gridDim.x * blockDim.x) {
    const int blk = (int)(it / n_groups);
    const long long gi = it % n_groups;
    const size_t xb = (size_t)blk * block_elems;
    uint8_t *cb = codes + (size_t)blk * block_code_bytes;
    if (kind == QKV_KIND_K_PER_CHANNEL) {
      const int c = (int)(gi / n_chunks), ch = (int)(gi % n_chunks);
      const int t0 = ch * group, t1 = min(tokens, t0 + group);
      float mn = load_x(x, dtype, xb + (size_t)t0 * D + c), mx = mn;
      for (int t = t0 + 1; t < t1; ++t) {
        const float v = load_x(x, dtype, xb + (size_t)t * D + c);
        mn = min_nan(mn, v);
        mx = max_nan(mx, v);
      }
      const half_t s16 = (half_t)((mx - mn) / levels), z16 = (half_t)mn;
      if (!isfinite((float)s16) || !isfinite((float)z16)) g_quant_status = QKV_ERANGE;
      uint16_t *pp = params + (((size_t)blk * D + c) * n_chunks + ch) * 2;
      pp[0] = __builtin_bit_cast(uint16_t, s16);
      pp[1] = __builtin_bit_cast(uint16_t, z16);
      for (int t = t0; t < t1; t += per_byte) {
        uint32_t byte = 0;
        for (int k = 0; k < per_byte && t + k < t1; ++k)
          byte |= quant_code(load_x(x, dtype, xb + (size_t)(t + k) * D + c), s16, z16, levels) << (bits * k);
        cb[((size_t)c * tokens + t) / per_byte] = (uint8_t)byte;
      }
    } else if (kind == QKV_KIND_PER_TOKEN) {
      const int t = (int)(gi / (D / group)), grp = (int)(gi % (D / group));
      const size_t row = xb + (size_t)t * D + (size_t)grp * group;
      float mn = load_x(x, dtype, row), mx = mn;
      for (int c = 1; c < group; ++c) {
        const float v = load_x(x, dtype, row + c);
        mn = min_nan(mn, v);
        mx = max_nan(mx, v);
      }
      const half_t s16 = (half_t)((mx - mn) / levels), z16 = (half_t)mn;
      if (!isfinite((float)s16) || !isfinite((float)z16)) g_quant_status = QKV_ERANGE;
      uint16_t *pp = params + (((size_t)blk * tokens + t) * (D / group) + grp) * 2;
      pp[0] = __builtin_bit_cast(uint16_t, s16);
      pp[1] = __builtin_bit_cast(uint16_t, z16);
      for (int c = 0; c < group; c += per_byte) {
        uint32_t byte = 0;
        for (int k = 0; k < per_byte; ++k) byte |= quant_code(load_x(x, dtype, row + c + k), s16, z16, levels) << (bits * k);
        cb[((size_t)t * D + grp * group + c) / per_byte] = (uint8_t)byte;
      }
    } else {
      const int t = (int)gi;
      const size_t row = xb + (size_t)t * D;
      double sum = 0.0;
      for (int c = 0; c < D; ++c) sum += (double)load_x(x, dtype, row + c);
      const float m32 = f64_to_f32_kept(sum / D);
      double ss = 0.0;
      for (int c = 0; c < D; ++c) {
        const double dv = (double)load_x(x, dtype, row + c) - (double)m32;
        ss += dv * dv;
      }
      const float sd32 = f64_to_f32_kept(sqrt(ss / D));
      const half_t m16 = (half_t)m32, sd16 = (half_t)sd32;
      if (!isfinite((float)m16) || !isfinite((float)sd16)) g_quant_status = QKV_ERANGE;
      uint16_t *pp = params + ((size_t)blk * tokens + t) * 2;
      pp[0] = __builtin_bit_cast(uint16_t, m16);
      pp[1] = __builtin_bit_cast(uint16_t, sd16);
      for (int c = 0; c < D; c += 8) {
        uint32_t byte = 0;
        for (int k = 0; k < 8; ++k) byte |= (load_x(x, dtype, row + c + k) > m32 ? 1u : 0u) << k;
        cb[((size_t)t * D + c) / 8] = (uint8_t)byte;
      }
    }
  }
}

hipError_t launch_quantize_window(const void *x, int x_dtype, int n_blocks, int tokens, int d, int bits, int group,
                                  int kind, uint8_t *codes, uint16_t *params, hipStream_t s) {
  long long groups = kind == QKV_KIND_K_PER_CHANNEL ? (long long)d * ((tokens + group - 1) / group)
                     : kind == QKV_KIND_PER_TOKEN ? (long long)tokens * (d / group)
                                                  : (long long)tokens;
  long long total = groups * n_blocks;
  int grid = (int)((total + 255) / 256);
  if (grid > 8192) grid = 8192;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(quantize_window_kernel, dim3(grid), dim3(256), 0, s, x, x_dtype, n_blocks, tokens, d, bits,
                     group, kind, codes, params);
  return hipGetLastError();
}

hipError_t read_quantize_status(int *flag, hipStream_t s) {
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbol(flag, HIP_SYMBOL(g_quant_status), sizeof(int), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  int zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_quant_status), &zero, sizeof(int), 0, hipMemcpyHostToDevice);
}

// ---------------------------------------------------------------------------
// stateless multi-tier ranking
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void rank_tiers_kernel(const float *__restrict__ score,
                                                          const int32_t *__restrict__ pos,
                                                          const uint8_t *__restrict__ eligible, int n,
                                                          const int32_t *__restrict__ counts, int n_tiers,
                                                          uint8_t *__restrict__ out, int npow) {
  extern __shared__ unsigned long long smem[];
  unsigned long long *keys = smem;                // (score, pos) order key
  int *idx = (int *)(smem + npow);
  __shared__ int n_elig;
  if (threadIdx.x == 0) n_elig = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    out[i] = 255;
    if (eligible[i]) atomicAdd(&n_elig, 1);
  }
  // ordered-integer images of (score, pos); padding sorts last
  for (int i = threadIdx.x; i < npow; i += blockDim.x) {
    unsigned long long key = 0ull;
    int id = -1;
    if (i < n && eligible[i]) {
      uint32_t sb = __float_as_uint(score[i]);
      sb = (sb & 0x80000000u) ? ~sb : (sb | 0x80000000u);
      const uint32_t pb = (uint32_t)pos[i] ^ 0x80000000u;
      key = ((unsigned long long)sb << 32) | pb;
      id = i;
    }
    keys[i] = key;
    idx[i] = id;
  }
  __syncthreads();
  // bitonic sort of (key, idx), key descending; padding (key 0) sorts last:
  // a real key is never 0 (its score image or position image is non-zero)
  for (int k = 2; k <= npow; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < npow; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long a = keys[i], c = keys[ixj];
          const bool desc = (i & k) == 0;
          if ((a < c) == desc && a != c) {
            keys[i] = c;
            keys[ixj] = a;
            const int t = idx[i];
            idx[i] = idx[ixj];
            idx[ixj] = t;
          }
        }
      }
      __syncthreads();
    }
  const int ne = n_elig;
  for (int r = threadIdx.x; r < ne; r += blockDim.x) {
    int t = 0, acc = 0;
    while (t < n_tiers && r >= acc + counts[t]) {
      acc += counts[t];
      ++t;
    }
    out[idx[r]] = (uint8_t)t;
  }
}

hipError_t launch_rank_tiers(const float *score, const int32_t *pos, const uint8_t *eligible, int n,
                             const int32_t *counts, int n_tiers, uint8_t *out, hipStream_t s) {
  int npow = 1;
  while (npow < n) npow <<= 1;
  size_t lds = (size_t)npow * (sizeof(unsigned long long) + sizeof(int));
  hipLaunchKernelGGL(rank_tiers_kernel, dim3(1), dim3(1024), lds, s, score, pos, eligible, n, counts, n_tiers, out,
                     npow);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// export in canonical layouts
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void export_kernel(Geom g, State st, int what, void *dst) {
  const int W = g.window, D = g.d;
  const size_t n_units = (size_t)g.B * g.U * g.Hkv;
  if (what == QKV_EXPORT_KCODES || what == QKV_EXPORT_VCODES) {
    const int bits = g.bits, per_byte = 8 / bits;
    const uint32_t mask = (1u << bits) - 1u;
    const int bytes_per = W * D * bits / 8;
    const size_t total = n_units * bytes_per;
    for (size_t it = (size_t)blockIdx.x * blockDim.x + threadIdx.x; it < total; it += (size_t)gridDim.x * blockDim.x) {
      const size_t blk = it / bytes_per;
      const int byte = (int)(it % bytes_per);
      const int h = (int)(blk % g.Hkv);
      const int u = (int)((blk / g.Hkv) % g.U);
      const int b = (int)(blk / ((size_t)g.Hkv * g.U));
      uint32_t val = 0;
      const int slot = st.lslot[b * g.U + u] - 1;
      if (st.has_ledger[b * g.U + u] && slot >= 0) {
        const uint8_t *Lb = st.ledger + ledger_slot_offset(g, slot, h);
        for (int k = 0; k < per_byte; ++k) {
          const int e = byte * per_byte + k;
          int t, c, dw, sh;
          if (what == QKV_EXPORT_KCODES) {
            c = e / W;
            t = e % W;
            kcode_slot(t % TS, c, D, bits, dw, sh);
          } else {
            t = e / D;
            c = e % D;
            vcode_slot(t % TS, c, D, bits, dw, sh);
          }
          const uint32_t *tc = (const uint32_t *)(Lb + g.kparam_bytes + (t / TS) * g.tile_block_bytes);
          val |= ((tc[dw] >> sh) & mask) << (bits * k);
        }
      }
      ((uint8_t *)dst)[it] = (uint8_t)val;
    }
  } else if (what == QKV_EXPORT_KPARAMS || what == QKV_EXPORT_VPARAMS) {
    const int per = what == QKV_EXPORT_KPARAMS ? D * 2 : W * (D / 32) * 2;
    const size_t total = n_units * per;
    for (size_t it = (size_t)blockIdx.x * blockDim.x + threadIdx.x; it < total; it += (size_t)gridDim.x * blockDim.x) {
      const size_t blk = it / per;
      const int k = (int)(it % per);
      const int h = (int)(blk % g.Hkv);
      const int u = (int)((blk / g.Hkv) % g.U);
      const int b = (int)(blk / ((size_t)g.Hkv * g.U));
      uint16_t val = 0;
      const int slot = st.lslot[b * g.U + u] - 1;
      if (st.has_ledger[b * g.U + u] && slot >= 0) {
        const uint8_t *Lb = st.ledger + ledger_slot_offset(g, slot, h);
        if (what == QKV_EXPORT_KPARAMS) {
          const int c = k / 2, which = k % 2;
          val = ((const uint16_t *)Lb)[which * D + c];
        } else {
          const int which = k % 2, grp = (k / 2) % (D / 32), t = k / 2 / (D / 32);
          const uint16_t *vp = (const uint16_t *)(Lb + g.kparam_bytes + (t / TS) * g.tile_block_bytes +
                                                  g.tile_kcode_bytes + g.tile_vcode_bytes);
          val = vp[vparam_index(g, t % TS, grp, which)];
        }
      }
      ((uint16_t *)dst)[it] = val;
    }
  } else {   // KEYS / VALUES
    const size_t total = (size_t)g.B * g.Hkv * g.max_ctx * D;
    for (size_t it = (size_t)blockIdx.x * blockDim.x + threadIdx.x; it < total; it += (size_t)gridDim.x * blockDim.x) {
      const int c = (int)(it % D);
      const int pos = (int)((it / D) % g.max_ctx);
      const int h = (int)((it / ((size_t)D * g.max_ctx)) % g.Hkv);
      const int b = (int)(it / ((size_t)D * g.max_ctx * g.Hkv));
      const int u = unit_of(g, pos);
      const int slot = pos - unit_start(g, u);
      const uint16_t *kt = st.pages + page_offset(g, b, u, h) + (size_t)(slot / TS) * 2 * TS * D;
      const int t = slot % TS;
      if (what == QKV_EXPORT_KEYS_RAW)   // the keys as appended (rotary caches), page key-half layout
        ((uint16_t *)dst)[it] = st.kraw[kraw_offset(g, b, u, h) + (size_t)(slot / TS) * TS * D + k_tile_index(t, c)];
      else
        ((uint16_t *)dst)[it] = what == QKV_EXPORT_KEYS ? kt[k_tile_index(t, c)] : kt[TS * D + v_tile_index(t, c)];
    }
  }
}

hipError_t launch_export(const Geom &g, const State &st, const StepInfo &si, int what, void *dst, hipStream_t s) {
  if (what == QKV_EXPORT_ROUTED)
    return hipMemcpyAsync(dst, st.routed, (size_t)g.B * g.U * sizeof(int32_t), hipMemcpyDeviceToDevice, s);
  if (what == QKV_EXPORT_TIERS)
    return hipMemcpyAsync(dst, st.tier, (size_t)g.B * g.U, hipMemcpyDeviceToDevice, s);
  if (what == QKV_EXPORT_SCORES) {
    hipLaunchKernelGGL(slist_sync_kernel, dim3((g.U + 255) / 256, g.B), dim3(256), 0, s, g, st, si);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipMemcpyAsync(dst, st.score, (size_t)g.B * g.U * sizeof(float), hipMemcpyDeviceToDevice, s);
  }
  if (what == QKV_EXPORT_LEDGER)
    return hipMemcpyAsync(dst, st.has_ledger, (size_t)g.B * g.U, hipMemcpyDeviceToDevice, s);
  if (what == QKV_EXPORT_EVENT)
    return hipMemcpyAsync(dst, st.event, (size_t)g.B * EV_WORDS * 4, hipMemcpyDeviceToDevice, s);
  if (what == QKV_EXPORT_VICTIMS)
    return hipMemcpyAsync(dst, st.victims, (size_t)g.B * g.U * 4, hipMemcpyDeviceToDevice, s);
  hipLaunchKernelGGL(export_kernel, dim3(2048), dim3(256), 0, s, g, st, what, dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// session snapshot: step scalars, canonical -> internal layouts, derived lists
// ---------------------------------------------------------------------------

__global__ void write_snapshot_kernel(Snapshot snap, long long *dst) {
  const int i = threadIdx.x;
  if (i < 16) dst[i] = snap.v[i];
}

hipError_t launch_write_snapshot(const Snapshot &snap, void *dst, hipStream_t s) {
  hipLaunchKernelGGL(write_snapshot_kernel, dim3(1), dim3(64), 0, s, snap, (long long *)dst);
  return hipGetLastError();
}

// The inverse of export_kernel: every internal element is written by one
// thread from the canonical copy (a code dword gathers its 16 slots, so no
// two threads write the same word).
__global__ __launch_bounds__(256) void import_kernel(Geom g, State st, int what, const void *__restrict__ src) {
  const int W = g.window, D = g.d;
  const size_t n_units = (size_t)g.B * g.U * g.Hkv;   // (b, u, h) blocks, in canonical order
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (what == QKV_EXPORT_KCODES || what == QKV_EXPORT_VCODES) {
    const bool keys = what == QKV_EXPORT_KCODES;
    const int bits = g.bits, dpl = code_dwords(D, bits), per_byte = 8 / bits;
    const int nkw = bits == 2 ? D / 64 : D / 32;     // key dwords per lane
    const int per_lane = keys ? nkw : dpl - nkw;     // this kind's dwords per lane
    const int per_unit = g.tpw * 64 * per_lane;      // this kind's code dwords per block
    const int cbytes = W * D * bits / 8;             // canonical bytes per block
    for (size_t it = i0; it < n_units * per_unit; it += stride) {
      const size_t blk = it / per_unit;
      const int r = (int)(it % per_unit);
      const int tile = r / (64 * per_lane), l = (r % (64 * per_lane)) / per_lane;
      const int w = (keys ? 0 : nkw) + r % per_lane;
      const uint8_t *cs = (const uint8_t *)src + blk * cbytes;
      uint32_t word = 0u;
      for (int p = 0; p < 32 / bits; ++p) {
        int t, c;
        (void)code_slot_elem(l, w, p, D, bits, t, c);
        const int tt = tile * TS + t;
        if (tt >= W) continue;
        const int e = keys ? c * W + tt : tt * D + c;
        word |= (uint32_t)((cs[e / per_byte] >> (bits * (e % per_byte))) & ((1 << bits) - 1)) << (bits * p);
      }
      const int slot = st.lslot[blk / g.Hkv] - 1;   // blk = (b * U + u) * Hkv + h
      if (slot < 0) continue;
      uint32_t *tc = (uint32_t *)(st.ledger + ledger_slot_offset(g, slot, (int)(blk % g.Hkv)) + g.kparam_bytes +
                                  (size_t)tile * g.tile_block_bytes);
      tc[l * dpl + w] = word;
    }
  } else if (what == QKV_EXPORT_KPARAMS) {
    const uint16_t *ps = (const uint16_t *)src;   // [blk][D][1][2]
    for (size_t it = i0; it < n_units * D * 2; it += stride) {
      const size_t blk = it / (D * 2);
      const int k = (int)(it % (D * 2)), c = k / 2, which = k % 2;
      const int slot = st.lslot[blk / g.Hkv] - 1;
      if (slot < 0) continue;
      ((uint16_t *)(st.ledger + ledger_slot_offset(g, slot, (int)(blk % g.Hkv))))[which * D + c] = ps[it];
    }
  } else if (what == QKV_EXPORT_VPARAMS) {
    const uint16_t *ps = (const uint16_t *)src;   // [blk][W][D/32][2]
    const int per = W * (D / 32) * 2;
    for (size_t it = i0; it < n_units * per; it += stride) {
      const size_t blk = it / per;
      const int k = (int)(it % per), which = k % 2, grp = (k / 2) % (D / 32), t = k / 2 / (D / 32);
      const int slot = st.lslot[blk / g.Hkv] - 1;
      if (slot < 0) continue;
      uint16_t *vp = (uint16_t *)(st.ledger + ledger_slot_offset(g, slot, (int)(blk % g.Hkv)) + g.kparam_bytes +
                                  (size_t)(t / TS) * g.tile_block_bytes + g.tile_kcode_bytes + g.tile_vcode_bytes);
      vp[vparam_index(g, t % TS, grp, which)] = ps[it];
    }
  } else {   // KEYS / VALUES: [B][Hkv][max_ctx][D]
    const uint16_t *xs = (const uint16_t *)src;
    const size_t total = (size_t)g.B * g.Hkv * g.max_ctx * D;
    for (size_t it = i0; it < total; it += stride) {
      const int c = (int)(it % D);
      const int pos = (int)((it / D) % g.max_ctx);
      const int h = (int)((it / ((size_t)D * g.max_ctx)) % g.Hkv);
      const int b = (int)(it / ((size_t)D * g.max_ctx * g.Hkv));
      const int u = unit_of(g, pos);
      const int slot = pos - unit_start(g, u);
      uint16_t *kt = st.pages + page_offset(g, b, u, h) + (size_t)(slot / TS) * 2 * TS * D;
      const int t = slot % TS;
      if (what == QKV_EXPORT_KEYS_RAW)
        st.kraw[kraw_offset(g, b, u, h) + (size_t)(slot / TS) * TS * D + k_tile_index(t, c)] = xs[it];
      else if (what == QKV_EXPORT_KEYS)
        kt[k_tile_index(t, c)] = xs[it];
      else
        kt[TS * D + v_tile_index(t, c)] = xs[it];
    }
  }
}

hipError_t launch_import(const Geom &g, const State &st, int what, const void *src, hipStream_t s) {
  const size_t BU = (size_t)g.B * g.U;
  switch (what) {
    case QKV_EXPORT_TIERS: return hipMemcpyAsync(st.tier, src, BU, hipMemcpyDeviceToDevice, s);
    case QKV_EXPORT_SCORES: return hipMemcpyAsync(st.score, src, BU * sizeof(float), hipMemcpyDeviceToDevice, s);
    case QKV_EXPORT_ROUTED: return hipMemcpyAsync(st.routed, src, BU * sizeof(int32_t), hipMemcpyDeviceToDevice, s);
    default: break;
  }
  hipLaunchKernelGGL(import_kernel, dim3(2048), dim3(256), 0, s, g, st, what, src);
  return hipGetLastError();
}

// After an import: the per-sequence full/quantized split of the ranked list
// and the list-order scores (sink, ranked, recent) from the per-unit scores;
// slots past the list hold 0, as a routing event leaves them.
__global__ __launch_bounds__(256) void rebuild_kernel(Geom g, State st, StepInfo si) {
  const int b = blockIdx.y;
  const EntryList L = make_list(g, st, si, b);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    st.routed_nf[b] = L.nF;
    st.routed_nq[b] = L.nQ;
  }
  for (int r = L.nF + blockIdx.x * blockDim.x + threadIdx.x; r < L.nF + L.nQ; r += gridDim.x * blockDim.x)
    st.qslot[(size_t)b * g.U + r] = st.lslot[(size_t)b * g.U + min(max(st.routed[(size_t)b * g.U + r], 0), g.U - 1)] - 1;
  const int E = L.count();
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < g.U; e += gridDim.x * blockDim.x) {
    const int u = min(max(entry_unit(L, st.routed + (size_t)b * g.U, e), 0), g.U - 1);
    st.slist[(size_t)b * g.U + e] = e < E ? st.score[(size_t)b * g.U + u] : 0.0f;
  }
}

hipError_t launch_rebuild(const Geom &g, const State &st, const StepInfo &si, hipStream_t s) {
  hipLaunchKernelGGL(rebuild_kernel, dim3((g.U + 255) / 256, g.B), dim3(256), 0, s, g, st, si);
  return hipGetLastError();
}

}  // namespace qkv
