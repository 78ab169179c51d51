// Internal geometry, device state and layout helpers of the qkv library.
//
// Memory layout in HBM (one workspace, carved at create time):
//
//   pages    bf16  [B][U][Hkv][tpw][2][TS*d]   full-precision content of every unit
//                  (unit 0 = sink prefix, unit 1+j = window j), tiles of TS=16
//                  token slots; K tiles and V tiles are stored in the order
//                  the matrix-core operands are read (see k_tile_index /
//                  v_tile_index), so each wavefront load is one contiguous block.
//   ledger   u8    [P][Hkv][ledger_unit_bytes]  pool of P ledger slots holding the
//                  persistent quantized codes of every window demoted and not
//                  evicted since (pack-once ledger); one pool for every layer and
//                  sequence of the cache, slots handed out and returned at routing
//                  events through a free-slot stack.  A layer's sequence never holds
//                  more than K_f + K_q ledgers (only Full and Quantized windows keep
//                  one), so P = layers * B * min(K_f + K_q, U) never runs out.
//   tier, has_ledger u8 [B][U]; score f32 [B][U]; lslot i32 [B][U] (pool slot + 1, 0: none)
//   routed   i32   [B][U]  ranked unit ids: full-precision windows first, then
//                  quantized windows (rank order); counts in routed_nf/nq.
//   pack/promote lists i32 [B][U] + counts; attention partials; mass partials.
//
// Units are addressed by their stable window id; a window's position span is
// fixed by its id, independent of its tier (the stable window <-> span map the
// routing recurrence needs).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qkv.h"

namespace qkv {

constexpr int TS = 16;           // token slots per tile
constexpr int WAVE = 64;
constexpr int ATT_WAVES = 8;     // most waves per token-mode attention workgroup
constexpr int SORT_MAX = 8192;          // largest LDS sort of the token policies and the stateless ranking
constexpr int ROUTE_SORT_MAX = 16384;   // largest window-policy candidate set (8-byte keys, 128 KB of LDS)

enum : uint8_t { T_EMPTY = 0, T_SINK = 1, T_RECENT = 2, T_FULL = 3, T_QUANT = 4, T_EVICTED = 5 };

struct Geom {
  int B, Hq, Hkv, G, d;
  int window, omega, n_sink, n_recent, k_full, k_quant, bits, group, max_ctx;
  int U;                 // units per sequence
  int tpw;               // tiles per unit
  int n_splits;
  // per (b,u,g) sizes
  int page_unit_elems;   // bf16 elements: tpw * 2 * TS * d
  int ledger_unit_bytes; // kparams + tpw * tile block
  int kparam_bytes;      // s[d], z[d] fp16
  int tile_kcode_bytes;  // TS * d / 4
  int tile_vcode_bytes;
  int tile_vparam_bytes; // 4 token quads * d/32 groups * 16 B
  int tile_block_bytes;
  int tr_per_seq;        // workgroups per sequence of the pack/promote launch (one resident round)
  int pool_slots;        // ledger-pool slots of the cache (every layer)
  int pool_per;          // slots of one (layer, sequence): its range of the pool
  int rope;              // keys arrive before the rotary embedding (table in State::rope)
};

struct State {
  uint16_t *pages;
  uint8_t *ledger;
  uint8_t *tier;
  uint8_t *has_ledger;
  float *score;      // [B][U] per unit
  int32_t *routed;
  int32_t *routed_nf;
  int32_t *routed_nq;
  int32_t *pack_list;
  int32_t *pack_count;
  int32_t *promote_list;
  int32_t *promote_count;
  float *part_o;     // [B][Hkv][S][G][d]
  float *part_ml;    // [B][Hkv][S][G][2]  (max in log2 units, sum)
  float *mass_part;  // [B][Hkv][U+1][G][2] (partial mass, reference max)
  float *slist;         // [B][U] scores of the live entries in list order (sink, ranked,
                        // recent): the per-step merge updates these; score[] is brought up
                        // to date from them by each routing event and before an export
  int32_t *status;   // [4] latched device errors
  int32_t *lslot;       // [B][U] ledger-pool slot + 1 of each window holding codes (0: none)
  int32_t *qslot;       // [B][U] pool slot of ranked entry r (its quantized part), set at each event
  int32_t *event;       // [B][EV_WORDS] record of the last routing event (EV_* fields)
  int32_t *victims;     // [B][U] windows the last routing event evicted, in rank order (-1 past them)
  int32_t *free_list;   // [B][U] windows whose ledger the last routing event released
  int32_t *free_count;  // [B]
  int32_t *pool_stack;  // [L*B][pool_per] free slots of each (layer, sequence)'s range of the pool
  int32_t *pool_top;    // [L*B] free slots on each stack
  int layer;            // this state's layer (its pool ranges are layer * B + b)
  // rotary embedding (Geom::rope): the caller's table [positions][d/2][cos, sin]
  // and the keys as appended, before the rotation, [B][U][Hkv][tpw*TS][d]
  // (packing reads them; the pages hold the rotated keys)
  const float *rope;
  int rope_n;           // rows of the table
  uint16_t *kraw;
};

// Per-step scalars the host knows without reading the device.
struct StepInfo {
  int N;        // tokens appended per sequence
  int r0, r1;   // recent (not yet ranked) windows: units r0..r1 (r1 < r0: none)
  int has_sink; // sink entry present
  int n_routed; // ranked (full + quantized) windows per sequence after the last routing event
};

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// position span of unit u
__host__ __device__ inline int unit_start(const Geom &g, int u) { return u == 0 ? 0 : g.n_sink + (u - 1) * g.window; }
__host__ __device__ inline int unit_len(const Geom &g, int u) { return u == 0 ? g.n_sink : g.window; }
__host__ __device__ inline int unit_of(const Geom &g, int pos) {
  return pos < g.n_sink ? 0 : 1 + (pos - g.n_sink) / g.window;
}

// Swizzled element index inside a K tile [TS tokens x d]: the A operand of a
// 16x16x32 matrix op reads, for k-block kb, lane l = token + 16*q, the 8
// channels kb*32 + 8q .. +7 -- stored as 16 contiguous bytes at (kb*64+l)*8.
__host__ __device__ inline int k_tile_index(int t, int c) {
  return ((c >> 5) * 64 + ((c & 31) >> 3) * 16 + t) * 8 + (c & 7);
}
// V tile: the B operand of a 16x16x32 op over a pair of tiles reads, for
// column tile ct, lane l = (t/4)*16 + c%16 the 4 tokens 4q..4q+3 of channel c
// of each tile; the column tiles 2p and 2p+1 of a lane sit side by side, so a
// lane reads 16 contiguous bytes per column-tile pair.
__host__ __device__ inline int v_tile_index(int t, int c) {
  return (((c >> 5) * 64 + (t >> 2) * 16 + (c & 15)) * 2 + ((c >> 4) & 1)) * 4 + (t & 3);
}

// Ledger code placement.  A tile's codes are DPL = d*bits/64 dwords per lane
// (code_dwords): the lane's key dwords, then its value dwords, so one or two
// 16-byte loads fetch all of a lane's codes.
//
// 2-bit codes (16 per dword, slot p at bits [2p, 2p+1]; nkd = d/64 key and
// nkd value dwords per lane).  Slots are placed for the unpack in the
// attention kernel: x & 0x33333333 keeps slots 4k and 4k+2 of byte k in the
// low bits of its two nibbles, (x >> 2) & 0x33333333 slots 4k+1 and 4k+3, and
// a scaled FP4 (e2m1) conversion of a byte then yields the two codes as an
// exact fp16 pair (a nibble 00cc is the e2m1 value cc/2).
//   Keys, for the A operand of k-block kb (lane l = ((c%32)/8)*16 + t holds
//   the 8 channels kb*32 + 8*(l/16) ..): dword l*DPL + kb/2; channel e = c%8
//   sits in byte e/2 of the kb%2 half: slot 4*(e/2) + kb%2 + 2*(e%2).
//   Values, for the B operand of column tile ct (lane l = (t/4)*16 + c%16
//   holds tokens 4*(l/16) .. +3 of channel ct*16 + l%16): dword l*DPL + nkd +
//   ct/4; byte ct%4; tokens (0,1) of the quad in the first half, (2,3) in the
//   second: slot 4*(ct%4) + (t%4)/2 + 2*(t%2).
// 4-bit codes (8 per dword, nibble p at bits [4p, 4p+3]; d/32 key and d/32
// value dwords per lane).  x & 0x0F0F0F0F keeps the even nibbles, (x >> 4) &
// 0x0F0F0F0F the odd ones, each as the low nibble of a byte, which the scaled
// FP8 conversion turns into an exact fp16 code.
//   Keys: dword l*DPL + kb; channel e = c%8 at nibble 2e (e < 4) or 2(e-4)+1.
//   Values: dword l*DPL + d/32 + ct/2; token t%4 of column tile ct at nibble
//   2*(t%4) + ct%2.
__host__ __device__ inline int code_dwords(int d, int bits) { return d * bits / 64; }
__host__ __device__ inline void kcode_slot(int t, int c, int d, int bits, int &dword, int &shift) {
  const int kb = c >> 5, l = ((c & 31) >> 3) * 16 + t, e = c & 7, dpl = code_dwords(d, bits);
  if (bits == 2) {
    dword = l * dpl + (kb >> 1);
    shift = 2 * (4 * (e >> 1) + (kb & 1) + 2 * (e & 1));
  } else {
    dword = l * dpl + kb;
    shift = 4 * (e < 4 ? 2 * e : 2 * (e - 4) + 1);
  }
}
__host__ __device__ inline void vcode_slot(int t, int c, int d, int bits, int &dword, int &shift) {
  const int ct = c >> 4, l = (t >> 2) * 16 + (c & 15), tt = t & 3, dpl = code_dwords(d, bits);
  if (bits == 2) {
    dword = l * dpl + d / 64 + (ct >> 2);
    shift = 2 * (4 * (ct & 3) + (tt >> 1) + 2 * (tt & 1));
  } else {
    dword = l * dpl + d / 32 + (ct >> 1);
    shift = 4 * (2 * tt + (ct & 1));
  }
}
// The inverse: code slot p of dword w of lane l (a key dword when w is below
// the lane's key-dword count) holds the element (token t, channel c).
__host__ __device__ inline bool code_slot_elem(int l, int w, int p, int d, int bits, int &t, int &c) {
  if (bits == 2) {
    const int nkd = d / 64, m = p >> 2, par = p & 1, hi = (p >> 1) & 1;
    if (w < nkd) {
      c = (2 * w + par) * 32 + (l / 16) * 8 + 2 * m + hi;
      t = l % 16;
      return true;
    }
    c = (4 * (w - nkd) + m) * 16 + l % 16;
    t = 4 * (l / 16) + 2 * par + hi;
    return false;
  }
  const int kbn = d / 32;
  if (w < kbn) {
    const int e = (p & 1) ? 4 + (p >> 1) : (p >> 1);
    c = w * 32 + (l / 16) * 8 + e;
    t = l % 16;
    return true;
  }
  c = (2 * (w - kbn) + (p & 1)) * 16 + l % 16;
  t = 4 * (l / 16) + (p >> 1);
  return false;
}
// V params of a tile: [token quad tq][group g][s x4, z x4] fp16
__host__ __device__ inline int vparam_index(const Geom &g, int t, int grp, int which /*0 s,1 z*/) {
  return ((t >> 2) * (g.d / 32) + grp) * 8 + which * 4 + (t & 3);
}

__host__ __device__ inline size_t page_offset(const Geom &g, int b, int u, int h) {
  return ((size_t)(b * g.U + u) * g.Hkv + h) * (size_t)g.page_unit_elems;
}
// Record of a routing event per (layer, sequence): int32 counters, then the
// float32 relative score gaps across the two cuts of the ranking.
enum {
  EV_TOKENS = 0,      // tokens in the cache at the event
  EV_CANDIDATES,      // windows ranked
  EV_FULL,            // windows kept in full precision
  EV_QUANT,           // windows kept quantized
  EV_EVICTED,         // windows evicted at this event
  EV_PROMOTED,        // quantized -> full precision
  EV_DEMOTED,         // full precision or recent -> quantized
  EV_FIRST_PACKS,     // demotions that packed the window (no ledger yet)
  EV_REUSED,          // demotions that reused the window's ledger
  EV_FREED,           // ledger slots released (evicted windows that held codes)
  EV_MARGIN_FULL,     // float: (s[Kf-1] - s[Kf]) / max(|s[Kf-1]|, |s[Kf]|), +inf without such a cut
  EV_MARGIN_QUANT,    // float: the same at Kf + Kq
  EV_MARGIN_MIN,      // float: the smaller of the two
  EV_WORDS = 16
};
// HqeKV's assignment event in the same record: EV_FULL, EV_QUANT = BF16 and
// INT2 tokens of the ranked range after it, EV_EVICTED / EV_DEMOTED = tokens
// it evicted / moved to a lower tier, margins at its four cuts
enum {
  EV_HQ_REQUANTIZED = EV_FIRST_PACKS,   // tokens moved to INT4, INT2 or INT1
  EV_HQ_INT4 = EV_REUSED,
  EV_HQ_INT1 = EV_FREED,
  EV_HQ_MARGIN_INT1 = 13,               // float: margin at the INT2 | INT1 cut
  EV_HQ_MARGIN_EVICT = 14,              // float: margin at the INT1 | evict cut
};

__host__ __device__ inline size_t kraw_offset(const Geom &g, int b, int u, int h) {
  return ((size_t)(b * g.U + u) * g.Hkv + h) * (size_t)(g.tpw * TS * g.d);
}
__host__ __device__ inline size_t ledger_slot_offset(const Geom &g, int slot, int h) {
  return ((size_t)slot * g.Hkv + h) * (size_t)g.ledger_unit_bytes;
}

// bf16 helpers
__host__ __device__ inline float bf16_to_f32(uint16_t h) {
  union { uint32_t u; float f; } x;
  x.u = (uint32_t)h << 16;
  return x.f;
}
__host__ __device__ inline uint16_t f32_to_bf16_rne(float f) {
  union { uint32_t u; float f; } x;
  x.f = f;
  uint32_t lsb = (x.u >> 16) & 1u;
  return (uint16_t)((x.u + 0x7FFFu + lsb) >> 16);
}

// ---------------------------------------------------------------------------
// Token mode (H2O, HqeKV): every token is its own scoring unit, scores are
// per (sequence, KV head), and the kept tokens are gathered into compact tiles.
//
//   pages   bf16 [B][Hkv][NPT][2][TS*d]  every appended token at its position
//                (tile pos/16, slot pos%16; same swizzle as the window pages)
//   cpages  bf16 [B][Hkv][NCT][2][TS*d]  compact full-precision tiles: kept
//                tokens (HqeKV: in rank order; H2O: each in the slot it keeps
//                until evicted); cpos [B][Hkv][NCT*TS] their positions
//   tier u8, score f32 [B][Hkv][T]       per token
//   mrho f32 [B][Hkv][TILES+1][G][TS]    per live tile and head: p of each slot
//   mref f32 [B][Hkv][TILES+1][G]        ... and the running max it is relative
//                to (row TILES is the spare row unused lanes write to)
//   tacc f32 [B][Hkv][TILES][TS]         masses summed in list order since the
//                last flush into score (flushed before a route or an export;
//                unused when the routing period is 1)
// ---------------------------------------------------------------------------

// HqeKV tiers of a ranked token (the per-token state of the five-tier method)
enum : int { HQ_BF16 = 0, HQ_INT4 = 1, HQ_INT2 = 2, HQ_INT1 = 3, HQ_EVICT = 4 };
// exported tier codes of token-mode tokens
enum : uint8_t { T_INT4 = 6, T_INT1 = 7 };   // besides T_FULL (BF16), T_QUANT (INT2), T_EVICTED

struct TokGeom {
  int B, Hq, Hkv, G, d;
  int policy;
  int T;            // token capacity per (sequence, KV head)
  int NPT;          // position tiles: ceil(T / TS)
  int NCT;          // compact tiles per (sequence, KV head) of each tier
  int TILES;        // live tiles per (sequence, KV head), upper bound
  int n_sink, n_recent, k_heavy, omega;
  int n_splits;
  int att_waves;    // waves per attention workgroup: 8 (HqeKV) or 4 (H2O)
  // HqeKV: per-position record of a quantized token (canonical per-token
  // packing): K codes [d/2 B], V codes [d/2 B], K params [d/32][2] fp16,
  // V params [d/32][2] fp16 (INT1: [mean, std] in the first pair)
  int rec_bytes;
  int qtile_bytes[3];   // compact tile bytes of INT4, INT2, INT1
  int chunk;            // HqeKV: positions per ranked chunk (0: tokens are ranked one by one)
};

constexpr int HQ_CHUNK_MAX = 4096;   // ranked chunks per (sequence, KV head), sorted in LDS

struct TokState {
  uint16_t *pages;
  uint16_t *cpages;
  int32_t *cpos;
  uint8_t *tier;
  float *score;
  float *part_o;     // [B][Hkv][S][G][d]
  float *part_ml;    // [B][Hkv][S][G][2]
  float *mrho;
  float *mref;
  float *tacc;       // [B][Hkv][TILES][TS] masses added since the last flush, in list order
  float *scratch_out;   // [B][Hq][d] outputs of scoring-only passes
  int32_t *status;
  // HqeKV
  float *vrange;        // [B][Hkv][T] max - min of the token's original value row
  uint8_t *qrec;        // [B][Hkv][T][rec_bytes]
  uint32_t *hqkey;      // [B][Hkv][hq_key_stride] metric keys of the last assignment event
  uint8_t *hqold;       // [B][Hkv][T] level + 1 a token held before the last event, until it is re-quantized (0: none)
  uint8_t *qtiles[3];   // [B][Hkv][NCT][qtile_bytes] compact INT4 / INT2 / INT1 tiles
  int32_t *qpos[3];     // [B][Hkv][NCT*TS] their positions
  int32_t *cnt;         // [B][Hkv][4] tokens per ranked tier (BF16, INT4, INT2, INT1)
  unsigned long long *cuts;   // [B][Hkv][4] cut keys of the last assignment
  // H2O
  int32_t *event;       // [B][Hkv][EV_WORDS] record of the last eviction call that ranked
  int32_t *victims;     // [B][Hkv][T] positions it evicted, best-ranked first (-1 past them)
};

// Per-call scalars the host knows: tokens so far, first position not yet
// ranked (positions [rstart, N) are read from the position pages), kept tokens.
struct TokStep {
  int N, rstart, n_cmp;
  int skip;   // 1: this step's masses do not enter the scores (outside a rolling score window)
};

// key slots per (sequence, KV head) of an assignment event (a multiple of 4)
__host__ __device__ inline int hq_key_stride(const TokGeom &g) { return (g.T + 3) & ~3; }

__host__ __device__ inline size_t tok_page_offset(const TokGeom &g, int b, int h, int tile) {
  return (((size_t)b * g.Hkv + h) * g.NPT + tile) * (size_t)(2 * TS * g.d);
}
__host__ __device__ inline size_t tok_cpage_offset(const TokGeom &g, int b, int h, int tile) {
  return (((size_t)b * g.Hkv + h) * g.NCT + tile) * (size_t)(2 * TS * g.d);
}

// Step scalars and geometry of a session snapshot (QKV_EXPORT_STATE): written
// to device memory by a kernel from its arguments, read back by an import.
struct Snapshot {
  long long v[16];
};
enum : int {
  SNAP_TAG = 0, SNAP_POLICY, SNAP_BATCH, SNAP_HQ, SNAP_HKV, SNAP_D, SNAP_WINDOW, SNAP_MAXCTX,
  SNAP_N, SNAP_R, SNAP_RANKED, SNAP_STEPS, SNAP_ROUTES, SNAP_SINCE_ROUTE, SNAP_LAST_EVENT, SNAP_SPARE
};
constexpr long long SNAP_TAG_VALUE = 0x514B5631;   // "QKV1"

// ---- launchers (defined in qkv_kernels.hip) ----
hipError_t launch_write_snapshot(const Snapshot &snap, void *dst, hipStream_t s);
hipError_t launch_import(const Geom &g, const State &st, int what, const void *src, hipStream_t s);
hipError_t launch_rebuild(const Geom &g, const State &st, const StepInfo &si, hipStream_t s);
hipError_t launch_pool_init(const Geom &g, const State &st, hipStream_t s);
constexpr int MAX_LAYERS = 128;   // layers of one cache
hipError_t launch_clear(void *p, size_t bytes, hipStream_t s);
hipError_t launch_append(const Geom &g, const State &st, const uint16_t *k, const uint16_t *v, int n_tokens,
                         int pos0, hipStream_t s);
hipError_t launch_attend(const Geom &g, const State &st, const StepInfo &si, const uint16_t *q, float *out,
                         float *mass_out, hipStream_t s, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
                         const uint16_t *k_new = nullptr, const uint16_t *v_new = nullptr);
hipError_t launch_route(const Geom &g, const State &st, const StepInfo &si, int a0, int a1, int n_cand,
                        hipStream_t s);
hipError_t attend_lds_fits(const Geom &g, bool *fits);   // the attention workgroup's LDS fits the device
hipError_t transitions_shape(Geom &g);
hipError_t launch_quantize_window(const void *x, int x_dtype, int n_blocks, int tokens, int d, int bits, int group,
                                  int kind, uint8_t *codes, uint16_t *params, hipStream_t s);
hipError_t launch_rank_tiers(const float *score, const int32_t *pos, const uint8_t *eligible, int n,
                             const int32_t *counts, int n_tiers, uint8_t *out, hipStream_t s);
hipError_t launch_export(const Geom &g, const State &st, const StepInfo &si, int what, void *dst, hipStream_t s);
hipError_t read_quantize_status(int *flag, hipStream_t s);

// ---- token-mode launchers (defined in qkv_token.hip) ----
size_t tok_carve(const TokGeom &g, char *base, TokState &st);
hipError_t tok_launch_append(const TokGeom &g, const TokState &st, const uint16_t *k, const uint16_t *v,
                             int n_tokens, int pos0, hipStream_t s);
hipError_t tok_launch_attend(const TokGeom &g, const TokState &st, const TokStep &ts, const uint16_t *q,
                             size_t q_bstride, float *out, float *mass_out, hipStream_t s,
                             hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t tok_launch_route(const TokGeom &g, const TokState &st, const TokStep &ts, int a0, int a1, int n_cand,
                            hipStream_t s);
hipError_t tok_launch_export(const TokGeom &g, const TokState &st, int what, void *dst, hipStream_t s);
hipError_t tok_launch_flush(const TokGeom &g, const TokState &st, const TokStep &ts, hipStream_t s);
hipError_t hq_launch_event(const TokGeom &g, const TokState &st, int N, int elig_end, const int *counts,
                           hipStream_t s);
hipError_t tok_launch_import(const TokGeom &g, const TokState &st, int what, const void *src, hipStream_t s);
hipError_t tok_launch_rebuild(const TokGeom &g, const TokState &st, int n_cmp, hipStream_t s);
hipError_t tok_launch_export_routed(const TokGeom &g, const TokState &st, int n_cmp, void *dst, hipStream_t s);
// entries per list of a token-mode ROUTED snapshot
__host__ __device__ inline int tok_list_cap(const TokGeom &g) { return g.NCT * TS; }

}  // namespace qkv
