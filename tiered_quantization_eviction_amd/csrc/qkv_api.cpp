// Host side of the qkv C ABI: configuration checks, geometry, workspace
// carving, and the per-step scalars (token count, recent range) that the host
// tracks so that no call has to read device state.
#include <hip/hip_runtime.h>

#include <math.h>
#include <new>
#include <vector>
#include <string.h>

#include "qkv_internal.h"

using namespace qkv;

struct qkv_cache {
  qkv_config cfg;
  bool tok;       // token mode (H2O): per-token units, per-(sequence, KV head) scores
  Geom g;
  int L;          // layers (window policy; 1 for the token policies)
  State sts[MAX_LAYERS];   // per layer; the ledger pool, its free-slot stack and the
                           // attention partials are shared by every layer
  int Nl[MAX_LAYERS];      // tokens appended per sequence, per layer
  bool ledger_ready;       // ledger slots assigned (always, except between importing a
                           // snapshot's state and its ledger flags)
  TokGeom tg;
  TokState ts;
  int r_tok;      // token mode: first position not yet ranked
  int n_cmp;      // token mode (H2O): kept older tokens per (sequence, KV head)
  int last_event_N;   // HqeKV: tokens at the previous assignment event (0: none yet)
  // token mode with a routing period above 1: masses wait in list order until
  // a flush (before a route or a score export)
  mutable bool tacc_dirty = false;
  int steps_since_route = 0;   // decode steps since the last routing / assignment event
  void *ws;
  size_t ws_bytes;
  int N;          // tokens appended per sequence
  int r0;         // first window not yet ranked
  int routed;     // ranked windows held (same for every sequence)
  long long steps;
  long long routes;
  // after an import: derived structures (list-order scores, compact tiles,
  // value ranges) are rebuilt before the next call that reads them
  bool rebuild_pending;
  // kernel timing
  hipEvent_t *ev;   // 2 * ev_n events
  int ev_n, ev_next, ev_stride, ev_calls;
};

namespace {

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

int validate(const qkv_config *c) {
  if (!c) return QKV_EINVAL;
  if (c->batch < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1) return QKV_EINVAL;
  if (c->n_q_heads % c->n_kv_heads) return QKV_EINVAL;
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 4 && G != 8) return QKV_EINVAL;            // query heads per KV head: 4 or 8
  if (c->n_q_heads > 128) return QKV_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return QKV_EINVAL;
  if (c->max_ctx < 1) return QKV_EINVAL;
  if (c->n_splits < 0 || c->n_splits > 256) return QKV_EINVAL;
  if (c->n_layers < 0 || c->n_layers > MAX_LAYERS) return QKV_EINVAL;
  if (c->n_layers > 1 && c->policy != QKV_POLICY_QEVICT) return QKV_EINVAL;   // layers: the window policy
  // rotary keys: the window policy, windows of at most one 16-token tile (the
  // attention kernel keeps a tile's offset rotations in registers)
  if (c->rope < 0 || c->rope > 1 || (c->rope && (c->policy != QKV_POLICY_QEVICT || c->window > TS))) return QKV_EINVAL;
  // a rolling score window is HqeKV's, at most one routing period long
  if (c->score_window < 0 || (c->score_window > 0 && (c->policy != QKV_POLICY_HQEKV || c->score_window > c->omega)))
    return QKV_EINVAL;
  // chunk ranking is HqeKV's, chunks of at most 64 positions, at most HQ_CHUNK_MAX of them
  if (c->chunk < 0 || c->chunk > 64) return QKV_EINVAL;
  if (c->chunk > 0 && (c->policy != QKV_POLICY_HQEKV || ((long long)c->max_ctx + c->chunk - 1) / c->chunk > HQ_CHUNK_MAX))
    return QKV_EINVAL;
  if (c->policy == QKV_POLICY_H2O) {
    // per-token heavy hitters: window 1, no quantized tier, scores per KV head
    if (c->window != 1 || c->omega < 1 || c->k_quant != 0 || c->k_full < 0 || c->n_recent < 0) return QKV_EINVAL;
    if (c->n_sink < 0 || c->n_sink > TS) return QKV_EINVAL;
    if (c->max_ctx > ROUTE_SORT_MAX) return QKV_EINVAL;   // routing candidates are ranked in LDS
    return QKV_OK;
  }
  if (c->policy == QKV_POLICY_HQEKV) {
    // per-token five-tier assignment: window 1, no sinks, shares in [0, 1] summing to 1
    if (c->window != 1 || c->omega < 1 || c->n_sink != 0) return QKV_EINVAL;
    float sum = 0.0f;
    for (int k = 0; k < 5; ++k) {
      if (!(c->ratios[k] >= 0.0f && c->ratios[k] <= 1.0f)) return QKV_EINVAL;
      sum += c->ratios[k];
    }
    if (sum < 0.999f || sum > 1.001f) return QKV_EINVAL;
    return QKV_OK;
  }
  if (c->policy != QKV_POLICY_QEVICT) return QKV_EINVAL;
  if (c->window != 8 && c->window != 16 && c->window != 32) return QKV_EINVAL;
  if (c->omega < 1) return QKV_EINVAL;
  if (c->n_sink < 0 || c->n_sink > TS || c->n_recent < 0) return QKV_EINVAL;
  if (c->k_full < 0 || c->k_quant < 0) return QKV_EINVAL;
  if ((c->quant_bits != 2 && c->quant_bits != 4) || c->group != 32) return QKV_EINVAL;
  // rotary keys with eight heads per KV head at d = 128: the attention
  // workgroup's LDS (rotated query limbs of every window slot of eight
  // waves, the table rows) exceeds the device's
  if (c->rope && c->head_dim == 128 && G == 8) return QKV_EINVAL;
  const long long U = 1 + ((long long)c->max_ctx - c->n_sink + c->window - 1) / c->window;
  if (U + 1 > ROUTE_SORT_MAX) return QKV_EINVAL;      // routing candidates are ranked in LDS
  return QKV_OK;
}

void make_geom(const qkv_config *c, Geom &g) {
  memset(&g, 0, sizeof g);
  g.B = c->batch;
  g.Hq = c->n_q_heads;
  g.Hkv = c->n_kv_heads;
  g.G = c->n_q_heads / c->n_kv_heads;
  g.d = c->head_dim;
  g.window = c->window;
  g.omega = c->omega;
  g.n_sink = c->n_sink;
  g.n_recent = c->n_recent;
  g.k_full = c->k_full;
  g.k_quant = c->k_quant;
  g.bits = c->quant_bits;
  g.group = c->group;
  g.max_ctx = c->max_ctx;
  g.U = 1 + (c->max_ctx - c->n_sink + c->window - 1) / c->window;
  if (g.U < 1) g.U = 1;
  g.tpw = (c->window + TS - 1) / TS;
  g.page_unit_elems = g.tpw * 2 * TS * g.d;
  g.kparam_bytes = 4 * g.d;
  g.tile_kcode_bytes = TS * g.d * g.bits / 8;
  g.tile_vcode_bytes = TS * g.d * g.bits / 8;
  g.tile_vparam_bytes = 4 * (g.d / 32) * 16;
  g.tile_block_bytes = g.tile_kcode_bytes + g.tile_vcode_bytes + g.tile_vparam_bytes;
  g.ledger_unit_bytes = g.kparam_bytes + g.tpw * g.tile_block_bytes;
  g.rope = c->rope;
  {
    // a layer's sequence holds at most K_f + K_q ledgers (Full and Quantized
    // windows only), and never more than it has windows
    const long long per = (long long)c->k_full + c->k_quant < g.U ? (long long)c->k_full + c->k_quant : g.U;
    const long long P = (long long)(c->n_layers > 1 ? c->n_layers : 1) * g.B * per;
    g.pool_slots = P > 0 ? (int)P : 1;
    g.pool_per = (int)per;
  }
  int S = c->n_splits;
  if (S == 0) {   // one resident round: 256 workgroups of 8 waves = 1 per compute unit, 2 waves per SIMD
    const int pairs = g.B * g.Hkv;
    S = (256 + pairs - 1) / pairs;
    const int cap = g.U / 8 > 1 ? g.U / 8 : 1;
    if (S > cap) S = cap;
    if (S > 64) S = 64;
    if (S < 1) S = 1;
  }
  g.n_splits = S;
}

void make_tok_geom(const qkv_config *c, TokGeom &g) {
  memset(&g, 0, sizeof g);
  g.B = c->batch;
  g.Hq = c->n_q_heads;
  g.Hkv = c->n_kv_heads;
  g.G = c->n_q_heads / c->n_kv_heads;
  g.d = c->head_dim;
  g.policy = c->policy;
  g.T = c->max_ctx;
  g.NPT = (c->max_ctx + TS - 1) / TS;
  if (c->policy == QKV_POLICY_HQEKV) {
    g.NCT = g.NPT;                 // any tier may hold every token
    g.TILES = 2 * g.NPT + 5;       // ranked tiles (one partial per tier) + recent tiles
    g.rec_bytes = g.d + (g.d / 32) * 8;
    const int KB = g.d / 32;
    const int bits[3] = {4, 2, 1};
    for (int f = 0; f < 3; ++f) {
      const int lb = KB * bits[f] < 4 ? 4 : KB * bits[f];
      const int pb = f == 2 ? 4 : KB * 4;
      g.qtile_bytes[f] = 128 * lb + 32 * pb;
    }
  } else {
    g.NCT = c->k_full > 0 ? (c->k_full + TS - 1) / TS : 1;
    g.TILES = 1 + g.NCT + g.NPT;
  }
  g.n_sink = c->n_sink;
  g.n_recent = c->n_recent;
  g.k_heavy = c->k_full;
  g.omega = c->omega;
  g.chunk = c->policy == QKV_POLICY_HQEKV ? c->chunk : 0;
  // HqeKV: 8-wave workgroups, whose two waves on a SIMD take the
  // full-precision and quantized tiers in opposite orders; H2O (a short
  // compact list and the recent tiles): 4-wave workgroups, twice as many
  g.att_waves = c->policy == QKV_POLICY_HQEKV ? ATT_WAVES : ATT_WAVES / 2;
  int S = c->n_splits;
  if (S == 0) {   // one resident round (two waves per SIMD), at least two tiles per wave
    const int pairs = g.B * g.Hkv;
    const int wgs = 256 * ATT_WAVES / g.att_waves;
    S = (wgs + pairs - 1) / pairs;
    const int cap = g.TILES / (2 * g.att_waves) > 1 ? g.TILES / (2 * g.att_waves) : 1;
    if (S > cap) S = cap;
    if (S > 64) S = 64;
  }
  g.n_splits = S;
}

// workspace carving for L layers; with base == nullptr only sizes are computed
size_t carve(const Geom &g, int L, char *base, State *sts) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *p = base ? base + off : nullptr;
    off = align_up(off + bytes);
    return (void *)p;
  };
  const size_t BU = (size_t)g.B * g.U;
  State sh;   // shared by every layer
  memset(&sh, 0, sizeof sh);
  sh.ledger = (uint8_t *)take((size_t)g.pool_slots * g.Hkv * (size_t)g.ledger_unit_bytes);
  sh.pool_stack = (int32_t *)take((size_t)g.pool_slots * 4);
  sh.pool_top = (int32_t *)take((size_t)L * g.B * 4);
  sh.part_o = (float *)take((size_t)g.B * g.Hkv * g.n_splits * g.G * g.d * 4);
  sh.part_ml = (float *)take((size_t)g.B * g.Hkv * g.n_splits * g.G * 2 * 4);
  sh.mass_part = (float *)take((size_t)g.B * g.Hkv * (g.U + 1) * g.G * 2 * 4);
  for (int l = 0; l < L; ++l) {
    State st = sh;
    st.layer = l;
    st.pages = (uint16_t *)take(BU * g.Hkv * (size_t)g.page_unit_elems * 2);
    st.tier = (uint8_t *)take(BU);
    st.has_ledger = (uint8_t *)take(BU);
    st.score = (float *)take(BU * 4);
    st.routed = (int32_t *)take(BU * 4);
    st.routed_nf = (int32_t *)take((size_t)g.B * 4);
    st.routed_nq = (int32_t *)take((size_t)g.B * 4);
    st.pack_list = (int32_t *)take(BU * 4);
    st.pack_count = (int32_t *)take((size_t)g.B * 4);
    st.promote_list = (int32_t *)take(BU * 4);
    st.promote_count = (int32_t *)take((size_t)g.B * 4);
    st.free_list = (int32_t *)take(BU * 4);
    st.free_count = (int32_t *)take((size_t)g.B * 4);
    st.event = (int32_t *)take((size_t)g.B * EV_WORDS * 4);
    st.victims = (int32_t *)take(BU * 4);
    st.lslot = (int32_t *)take(BU * 4);
    st.qslot = (int32_t *)take(BU * 4);
    st.slist = (float *)take(BU * 4);
    st.status = (int32_t *)take(16);
    st.kraw = g.rope ? (uint16_t *)take(BU * g.Hkv * (size_t)(g.tpw * TS * g.d) * 2) : nullptr;
    st.rope = nullptr;
    st.rope_n = 0;
    if (sts) sts[l] = st;
  }
  return off;
}

thread_local hipError_t g_last_hip = hipSuccess;   // the HIP error behind this thread's last QKV_EHIP

int hip_err(hipError_t e) {
  if (e == hipSuccess) return QKV_OK;
  g_last_hip = e;
  return QKV_EHIP;
}

StepInfo step_info(const qkv_cache *c, int layer = 0) {
  StepInfo si;
  const int N = c->Nl[layer];
  si.N = N;
  si.has_sink = (c->g.n_sink > 0 && N > 0) ? 1 : 0;
  si.r0 = c->r0;
  si.r1 = N > c->g.n_sink ? unit_of(c->g, N - 1) : 0;
  si.n_routed = c->routed;
  return si;
}

// every layer holds the same number of tokens (routing and snapshots need it)
bool layers_in_step(const qkv_cache *c) {
  for (int l = 1; l < c->L; ++l)
    if (c->Nl[l] != c->Nl[0]) return false;
  return true;
}

// rebuild what an import left pending, on the stream of the call that needs it
int settle(qkv_cache *c, hipStream_t s) {
  if (!c->rebuild_pending) return QKV_OK;
  int rc = QKV_OK;
  if (c->tok) {
    rc = hip_err(tok_launch_rebuild(c->tg, c->ts, c->n_cmp, s));
  } else {
    for (int l = 0; l < c->L && rc == QKV_OK; ++l) rc = hip_err(launch_rebuild(c->g, c->sts[l], step_info(c, l), s));
  }
  if (rc == QKV_OK) c->rebuild_pending = false;
  return rc;
}

Snapshot make_snapshot(const qkv_cache *c) {
  Snapshot sn;
  memset(&sn, 0, sizeof sn);
  sn.v[SNAP_TAG] = SNAP_TAG_VALUE;
  sn.v[SNAP_POLICY] = c->cfg.policy;
  sn.v[SNAP_BATCH] = c->cfg.batch;
  sn.v[SNAP_HQ] = c->cfg.n_q_heads;
  sn.v[SNAP_HKV] = c->cfg.n_kv_heads;
  sn.v[SNAP_D] = c->cfg.head_dim;
  sn.v[SNAP_WINDOW] = c->cfg.window;
  sn.v[SNAP_MAXCTX] = c->cfg.max_ctx;
  sn.v[SNAP_N] = c->N;
  sn.v[SNAP_R] = c->tok ? c->r_tok : c->r0;
  sn.v[SNAP_RANKED] = c->tok ? c->n_cmp : c->routed;
  sn.v[SNAP_STEPS] = c->steps;
  sn.v[SNAP_ROUTES] = c->routes;
  sn.v[SNAP_SINCE_ROUTE] = c->steps_since_route;
  sn.v[SNAP_LAST_EVENT] = c->last_event_N;
  sn.v[SNAP_SPARE] = c->L;
  return sn;
}

// a snapshot's step scalars are usable by this cache (same policy and
// geometry, values in range)
bool snapshot_fits(const qkv_cache *c, const Snapshot &sn) {
  const long long *v = sn.v;
  if (v[SNAP_TAG] != SNAP_TAG_VALUE || v[SNAP_POLICY] != c->cfg.policy || v[SNAP_BATCH] != c->cfg.batch ||
      v[SNAP_HQ] != c->cfg.n_q_heads || v[SNAP_HKV] != c->cfg.n_kv_heads || v[SNAP_D] != c->cfg.head_dim ||
      v[SNAP_WINDOW] != c->cfg.window || v[SNAP_MAXCTX] != c->cfg.max_ctx || v[SNAP_SPARE] != c->L)
    return false;
  const long long N = v[SNAP_N];
  if (N < 0 || N > c->cfg.max_ctx || v[SNAP_STEPS] < 0 || v[SNAP_ROUTES] < 0 || v[SNAP_SINCE_ROUTE] < 0) return false;
  if (v[SNAP_LAST_EVENT] < 0 || v[SNAP_LAST_EVENT] > N) return false;
  if (c->tok) {
    const long long cap = c->cfg.policy == QKV_POLICY_H2O ? c->cfg.k_full : 0;
    return v[SNAP_R] >= 0 && v[SNAP_R] <= N && v[SNAP_RANKED] >= 0 && v[SNAP_RANKED] <= cap;
  }
  const long long kfq = (long long)c->g.k_full + c->g.k_quant;
  return v[SNAP_R] >= 1 && v[SNAP_R] <= c->g.U && v[SNAP_RANKED] >= 0 && v[SNAP_RANKED] <= kfq &&
         v[SNAP_RANKED] <= c->g.U;
}

}  // namespace

extern "C" {

const char *qkv_strerror(int code) {
  switch (code) {
    case QKV_OK: return "ok";
    case QKV_EINVAL: return "invalid argument or configuration";
    case QKV_ECAPACITY: return "capacity exceeded";
    case QKV_ERANGE: return "quantization parameter outside float16 range";
    case QKV_EHIP: return "HIP runtime error";
    case QKV_ESTATE: return "call out of order";
    default: return "unknown error";
  }
}

int qkv_check_config(const qkv_config *cfg) { return validate(cfg); }

const char *qkv_hip_error_detail(void) { return hipGetErrorString(g_last_hip); }

int qkv_plan_capacities(const qkv_config *cfg, double budget_bytes, double q, int32_t layers, int32_t *k_full,
                        int32_t *k_quant) {
  if (!cfg || !k_full || !k_quant || validate(cfg) != QKV_OK || cfg->policy != QKV_POLICY_QEVICT) return QKV_EINVAL;
  if (layers < 1 || !(q >= 0.0 && q <= 1.0) || !(budget_bytes >= 0.0)) return QKV_EINVAL;
  const double per_token = (double)layers * 2.0 * cfg->n_kv_heads * cfg->head_dim * 2.0;   // K and V, BF16
  const double fixed = (double)(cfg->n_sink + cfg->n_recent) * per_token;
  const double b_hist = budget_bytes - fixed;
  if (b_hist < 0.0) return QKV_EINVAL;
  const int w = cfg->window, d = cfg->head_dim, grp = cfg->group;
  const double m_f = (double)w * per_token;
  const double ledger = 2.0 * w * d * cfg->quant_bits / 8.0 + (double)d * ((w + grp - 1) / grp) * 4.0 +
                        (double)w * (d / grp) * 4.0;
  const double m_q = (double)layers * cfg->n_kv_heads * ledger;
  const double kf = floor((1.0 - q) * b_hist / m_f), kq = floor(q * b_hist / m_q);
  if (kf > 2147483647.0 || kq > 2147483647.0) return QKV_EINVAL;
  *k_full = (int32_t)kf;
  *k_quant = (int32_t)kq;
  return QKV_OK;
}

size_t qkv_workspace_bytes(const qkv_config *cfg) {
  if (validate(cfg) != QKV_OK) return 0;
  if (cfg->policy == QKV_POLICY_H2O || cfg->policy == QKV_POLICY_HQEKV) {
    TokGeom tg;
    make_tok_geom(cfg, tg);
    TokState ts;
    return tok_carve(tg, nullptr, ts);
  }
  Geom g;
  make_geom(cfg, g);
  return carve(g, cfg->n_layers > 1 ? cfg->n_layers : 1, nullptr, nullptr);
}

}  // extern "C"

// Set up handle `c` (cleared here) for a cache over `workspace`; nothing is
// allocated.  Shared by qkv_create (a handle from the heap) and
// qkv_create_static (a per-device handle of this file).
static int create_into(qkv_cache *c, const qkv_config *cfg, void *workspace, size_t bytes, hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != QKV_OK) return rc;
  if (!workspace || ((uintptr_t)workspace % ALIGN)) return QKV_EINVAL;
  memset(c, 0, sizeof *c);
  c->cfg = *cfg;
  c->tok = cfg->policy == QKV_POLICY_H2O || cfg->policy == QKV_POLICY_HQEKV;
  size_t need;
  if (c->tok) {
    make_tok_geom(cfg, c->tg);
    need = tok_carve(c->tg, (char *)workspace, c->ts);
    c->r_tok = cfg->n_sink;
  } else {
    make_geom(cfg, c->g);
    bool fits = false;
    rc = hip_err(attend_lds_fits(c->g, &fits));
    if (rc != QKV_OK || !fits) return rc != QKV_OK ? rc : QKV_EINVAL;   // (d = 128, G = 8 needs 32-token windows)
    rc = hip_err(transitions_shape(c->g));
    if (rc != QKV_OK) return rc;
    c->L = cfg->n_layers > 1 ? cfg->n_layers : 1;
    need = carve(c->g, c->L, (char *)workspace, c->sts);
  }
  if (c->tok) c->L = 1;
  if (bytes < need) return QKV_ECAPACITY;
  c->ws = workspace;
  c->ws_bytes = need;
  c->r0 = 1;
  c->ledger_ready = true;
  rc = hip_err(launch_clear(workspace, need, stream));
  if (rc != QKV_OK || c->tok) return rc;
  return hip_err(launch_pool_init(c->g, c->sts[0], stream));
}

static void free_events(qkv_cache *c) {
  if (c->ev) {
    for (int i = 0; i < 2 * c->ev_n; ++i) (void)hipEventDestroy(c->ev[i]);
    delete[] c->ev;
  }
  c->ev = nullptr;
  c->ev_n = c->ev_next = 0;
}

namespace qkv {

// one handle per device for the caches of qkv_create_static
constexpr int STATIC_DEVICES = 64;
static qkv_cache g_static_handle[STATIC_DEVICES];
static bool g_static_live[STATIC_DEVICES];

int create_static_over(const qkv_config *cfg, void *workspace, size_t bytes, int dev, hipStream_t stream,
                       qkv_cache **out) {
  if (!out) return QKV_EINVAL;
  *out = nullptr;
  if (dev < 0 || dev >= STATIC_DEVICES) return QKV_EINVAL;
  qkv_cache *c = &g_static_handle[dev];
  if (g_static_live[dev]) free_events(c);   // the device's previous static cache ends here
  g_static_live[dev] = false;
  const int rc = create_into(c, cfg, workspace, bytes, stream);
  if (rc != QKV_OK) return rc;
  g_static_live[dev] = true;
  *out = c;
  return QKV_OK;
}

static bool is_static_handle(const qkv_cache *c) {
  return c >= g_static_handle && c < g_static_handle + STATIC_DEVICES;
}

}  // namespace qkv

extern "C" {

int qkv_create(const qkv_config *cfg, void *workspace, size_t bytes, qkv_stream stream, qkv_cache **out) {
  if (!out) return QKV_EINVAL;
  *out = nullptr;
  int rc = validate(cfg);
  if (rc != QKV_OK) return rc;
  qkv_cache *c = new (std::nothrow) qkv_cache;
  if (!c) return QKV_ECAPACITY;
  rc = create_into(c, cfg, workspace, bytes, (hipStream_t)stream);
  if (rc != QKV_OK) {
    delete c;
    return rc;
  }
  *out = c;
  return QKV_OK;
}


int qkv_destroy(qkv_cache *cache) {
  if (!cache) return QKV_OK;
  free_events(cache);
  if (is_static_handle(cache)) {
    g_static_live[cache - g_static_handle] = false;   // the handle stays with its device
    return QKV_OK;
  }
  delete cache;
  return QKV_OK;
}

int qkv_profile_start(qkv_cache *c, int32_t n, int32_t stride) {
  if (!c || n < 0 || n > (1 << 20) || stride < 1) return QKV_EINVAL;
  free_events(c);
  if (n == 0) return QKV_OK;
  c->ev = new (std::nothrow) hipEvent_t[2 * n];
  if (!c->ev) return QKV_ECAPACITY;
  for (int i = 0; i < 2 * n; ++i) {
    // timing only: no system-scope fence (cache writeback) when recorded
    if (hipEventCreateWithFlags(&c->ev[i], hipEventDisableSystemFence) != hipSuccess) {
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(c->ev[j]);
      delete[] c->ev;
      c->ev = nullptr;
      return QKV_EHIP;
    }
  }
  c->ev_n = n;
  c->ev_next = 0;
  c->ev_stride = stride;
  c->ev_calls = 0;
  return QKV_OK;
}

int qkv_profile_read(qkv_cache *c, float *ms, int32_t n) {
  if (!c || !ms || n < 0 || n > c->ev_next) return QKV_EINVAL;
  if (n == 0) return QKV_OK;
  if (hipEventSynchronize(c->ev[2 * (c->ev_next - 1) + 1]) != hipSuccess) return QKV_EHIP;
  for (int i = 0; i < n; ++i)
    if (hipEventElapsedTime(&ms[i], c->ev[2 * i], c->ev[2 * i + 1]) != hipSuccess) return QKV_EHIP;
  return QKV_OK;
}

int qkv_set_rope(qkv_cache *c, const float *table, int32_t n_positions) {
  if (!c || !table || c->tok || !c->g.rope) return QKV_EINVAL;
  if (n_positions < c->cfg.max_ctx || n_positions < 16 || ((uintptr_t)table & 15)) return QKV_EINVAL;
  for (int l = 0; l < c->L; ++l) {
    c->sts[l].rope = table;
    c->sts[l].rope_n = n_positions;
  }
  return QKV_OK;
}

int qkv_append_layer(qkv_cache *c, int32_t layer, const void *k, const void *v, int32_t n_tokens,
                     qkv_stream stream) {
  if (!c || !k || !v || n_tokens < 1 || layer < 0 || layer >= c->L) return QKV_EINVAL;
  if (!c->tok && c->g.rope && !c->sts[0].rope) return QKV_ESTATE;   // qkv_set_rope first
  if ((long long)c->Nl[layer] + n_tokens > c->cfg.max_ctx) return QKV_ECAPACITY;
  int rc = settle(c, (hipStream_t)stream);
  if (rc != QKV_OK) return rc;
  rc = c->tok ? hip_err(tok_launch_append(c->tg, c->ts, (const uint16_t *)k, (const uint16_t *)v, n_tokens,
                                          c->N, (hipStream_t)stream))
              : hip_err(launch_append(c->g, c->sts[layer], (const uint16_t *)k, (const uint16_t *)v, n_tokens,
                                      c->Nl[layer], (hipStream_t)stream));
  if (rc != QKV_OK) return rc;
  c->Nl[layer] += n_tokens;
  c->N = c->Nl[0];
  return QKV_OK;
}

int qkv_append(qkv_cache *c, const void *k, const void *v, int32_t n_tokens, qkv_stream stream) {
  return qkv_append_layer(c, 0, k, v, n_tokens, stream);
}

static int decode_attend(qkv_cache *c, int32_t layer, const void *q, float *out, float *mass_out, qkv_stream stream,
                         const void *k_new = nullptr, const void *v_new = nullptr);

int qkv_decode_attend_layer(qkv_cache *c, int32_t layer, const void *q, float *out, float *mass_out,
                            qkv_stream stream) {
  if (!c || !q || !out || layer < 0 || layer >= c->L) return QKV_EINVAL;
  if (c->Nl[layer] < 1) return QKV_ESTATE;
  if (settle(c, (hipStream_t)stream) != QKV_OK) return QKV_EHIP;
  return decode_attend(c, layer, q, out, mass_out, stream);
}

int qkv_decode_step_layer(qkv_cache *c, int32_t layer, const void *k, const void *v, const void *q, float *out,
                          float *mass_out, qkv_stream stream) {
  if (!c || !k || !v || !q || !out || layer < 0 || layer >= c->L) return QKV_EINVAL;
  if (c->tok || c->g.rope) {
    // token policies and rotary keys: the append kernel, then attention
    const int rc = qkv_append_layer(c, layer, k, v, 1, stream);
    if (rc != QKV_OK) return rc;
    return qkv_decode_attend_layer(c, layer, q, out, mass_out, stream);
  }
  if ((long long)c->Nl[layer] + 1 > c->cfg.max_ctx) return QKV_ECAPACITY;
  if (settle(c, (hipStream_t)stream) != QKV_OK) return QKV_EHIP;
  c->Nl[layer] += 1;   // the launch attends over the new token and stores it in its page
  c->N = c->Nl[0];
  return decode_attend(c, layer, q, out, mass_out, stream, k, v);
}

int qkv_decode_step(qkv_cache *c, const void *k, const void *v, const void *q, float *out, float *mass_out,
                    qkv_stream stream) {
  return qkv_decode_step_layer(c, 0, k, v, q, out, mass_out, stream);
}

static int decode_attend(qkv_cache *c, int32_t layer, const void *q, float *out, float *mass_out, qkv_stream stream,
                         const void *k_new, const void *v_new) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (c->ev && c->ev_next < c->ev_n && c->ev_calls++ % c->ev_stride == 0) {
    e0 = c->ev[2 * c->ev_next];
    e1 = c->ev[2 * c->ev_next + 1];
    c->ev_next++;
  }
  int rc;
  if (c->tok) {
    // with a rolling score window only the last score_window steps before
    // the next event add to the scores
    const int m = c->cfg.score_window;
    const TokStep ts = {c->N, c->r_tok, c->n_cmp, (m > 0 && c->steps_since_route < c->tg.omega - m) ? 1 : 0};
    rc = hip_err(tok_launch_attend(c->tg, c->ts, ts, (const uint16_t *)q, (size_t)c->tg.Hq * c->tg.d, out, mass_out,
                                   (hipStream_t)stream, e0, e1));
    if (c->tg.omega > 1) c->tacc_dirty = true;
    c->steps_since_route++;
  } else {
    rc = hip_err(launch_attend(c->g, c->sts[layer], step_info(c, layer), (const uint16_t *)q, out, mass_out,
                               (hipStream_t)stream, e0, e1, (const uint16_t *)k_new, (const uint16_t *)v_new));
  }
  if (rc != QKV_OK) return rc;
  if (layer == c->L - 1) c->steps++;   // a decode step of the model ends with its last layer
  return QKV_OK;
}

int qkv_decode_attend(qkv_cache *c, const void *q, float *out, float *mass_out, qkv_stream stream) {
  return qkv_decode_attend_layer(c, 0, q, out, mass_out, stream);
}

int qkv_prefill_score(qkv_cache *c, const void *q, int32_t n_queries, qkv_stream stream) {
  if (!c || !q || n_queries < 1) return QKV_EINVAL;
  if (!c->tok) return QKV_ESTATE;                        // window mode does not score the prompt
  if (n_queries > c->N) return QKV_EINVAL;
  // a scored position must not be older than a kept ranked token (it would see it)
  if (c->n_cmp > 0 && c->N - n_queries < c->r_tok) return QKV_ESTATE;
  if (settle(c, (hipStream_t)stream) != QKV_OK) return QKV_EHIP;
  const TokGeom &g = c->tg;
  const size_t row = (size_t)g.Hq * g.d;
  for (int i = 0; i < n_queries; ++i) {
    const TokStep ts = {c->N - n_queries + i + 1, c->r_tok, c->n_cmp};   // causal: positions <= its own
    int rc = hip_err(tok_launch_attend(g, c->ts, ts, (const uint16_t *)q + (size_t)i * row, (size_t)n_queries * row,
                                       c->ts.scratch_out, nullptr, (hipStream_t)stream));
    if (rc != QKV_OK) return rc;
    if (g.omega > 1) c->tacc_dirty = true;
  }
  return QKV_OK;
}

int qkv_route(qkv_cache *c, qkv_stream stream) {
  if (!c) return QKV_EINVAL;
  if (c->N < 1) return QKV_ESTATE;
  if (settle(c, (hipStream_t)stream) != QKV_OK) return QKV_EHIP;
  if (c->tok && c->tacc_dirty) {
    // masses accumulated in list order reach the per-token scores first
    const TokStep ts = {c->N, c->r_tok, c->n_cmp};
    int rc = hip_err(tok_launch_flush(c->tg, c->ts, ts, (hipStream_t)stream));
    if (rc != QKV_OK) return rc;
    c->tacc_dirty = false;
  }
  if (c->tok && c->tg.policy == QKV_POLICY_HQEKV) {
    // assignment event: tokens ranked before (all live ones at the first
    // event) get target tiers by their rank; shares floor(r_k * N) of all
    // tokens ever appended, in the order BF16, INT4, INT2, INT1
    const int elig_end = c->last_event_N == 0 ? c->N : c->last_event_N;
    // shares of all tokens ever appended, or of all chunks of them
    const int chunk = c->tg.chunk;
    const double units = chunk > 0 ? (double)((c->N + chunk - 1) / chunk) : (double)c->N;
    int counts[4];
    for (int k = 0; k < 4; ++k) counts[k] = (int)floor((double)c->cfg.ratios[k] * units);
    int rc = hip_err(hq_launch_event(c->tg, c->ts, c->N, elig_end, counts, (hipStream_t)stream));
    if (rc != QKV_OK) return rc;
    if (c->cfg.score_window > 0) {
      // rolling window: the next event ranks by the queries of its own window only
      rc = hip_err(launch_clear(c->ts.score, (size_t)c->tg.B * c->tg.Hkv * c->tg.T * sizeof(float),
                                (hipStream_t)stream));
      if (rc != QKV_OK) return rc;
    }
    c->r_tok = elig_end;
    c->last_event_N = c->N;
    c->routes++;
    c->steps_since_route = 0;
    return QKV_OK;
  }
  if (c->tok) {
    // tokens older than the newest n_recent join the kept ones; the best k_full stay
    const TokGeom &tg = c->tg;
    const int limit = c->N - tg.n_recent;
    const int a0 = c->r_tok, a1 = limit > a0 ? limit : a0;
    const int n_cand = c->n_cmp + (a1 - a0);
    if (n_cand > 0) {
      const TokStep ts = {c->N, c->r_tok, c->n_cmp};
      int rc = hip_err(tok_launch_route(tg, c->ts, ts, a0, a1, n_cand, (hipStream_t)stream));
      if (rc != QKV_OK) return rc;
    }
    c->r_tok = a1;
    c->n_cmp = n_cand < tg.k_heavy ? n_cand : tg.k_heavy;
    c->routes++;
    c->steps_since_route = 0;
    return QKV_OK;
  }
  const Geom &g = c->g;
  if (!layers_in_step(c)) return QKV_ESTATE;   // every layer must hold the same tokens
  // windows whose last position is older than the newest n_recent positions
  const long long limit = (long long)c->N - g.n_recent;
  const long long aged = limit > g.n_sink ? (limit - g.n_sink) / g.window : 0;
  const int a0 = c->r0;
  const int a1 = (int)(aged + 1 > a0 ? aged + 1 : a0);
  const int n_cand = c->routed + (a1 - a0);
  // each layer ranks its own windows by its own scores (QEvict notes 4.2:
  // one score per layer and window), with the same capacities
  for (int l = 0; l < c->L; ++l) {
    int rc = hip_err(launch_route(g, c->sts[l], step_info(c, l), a0, a1, n_cand, (hipStream_t)stream));
    if (rc != QKV_OK) return rc;
  }
  c->r0 = a1;
  const int kfq = g.k_full + g.k_quant;
  c->routed = n_cand < kfq ? n_cand : kfq;
  c->routes++;
  c->steps_since_route = 0;
  return QKV_OK;
}

int qkv_quantize_window(const void *x, int32_t x_dtype, int32_t n_blocks, int32_t tokens, int32_t head_dim,
                        int32_t bits, int32_t group, int32_t kind, uint8_t *codes, uint16_t *params,
                        qkv_stream stream) {
  if (!x || !codes || !params || n_blocks < 1 || tokens < 1 || head_dim < 8 || head_dim % 8) return QKV_EINVAL;
  if (x_dtype != QKV_DTYPE_BF16 && x_dtype != QKV_DTYPE_F32) return QKV_EINVAL;
  if (kind == QKV_KIND_K_PER_CHANNEL || kind == QKV_KIND_PER_TOKEN) {
    if (bits != 2 && bits != 4) return QKV_EINVAL;
    if (group < 8 || group % 8) return QKV_EINVAL;
    if (kind == QKV_KIND_K_PER_CHANNEL && tokens % 8) return QKV_EINVAL;   // whole bytes per channel run
    if (kind == QKV_KIND_PER_TOKEN && head_dim % group) return QKV_EINVAL;
  } else if (kind == QKV_KIND_INT1_NORMAL) {
    if (bits != 1) return QKV_EINVAL;
  } else {
    return QKV_EINVAL;
  }
  return hip_err(launch_quantize_window(x, x_dtype, n_blocks, tokens, head_dim, bits, group, kind, codes, params,
                                        (hipStream_t)stream));
}

int qkv_quantize_status(qkv_stream stream) {
  int flag = 0;
  int rc = hip_err(read_quantize_status(&flag, (hipStream_t)stream));
  if (rc != QKV_OK) return rc;
  return flag ? QKV_ERANGE : QKV_OK;
}

int qkv_rank_tiers(const float *score, const int32_t *pos, const uint8_t *eligible, int32_t n,
                   const int32_t *tier_counts, int32_t n_tiers, uint8_t *tier_out, qkv_stream stream) {
  if (!score || !pos || !eligible || !tier_counts || !tier_out) return QKV_EINVAL;
  if (n < 1 || n > SORT_MAX || n_tiers < 0 || n_tiers > 254) return QKV_EINVAL;
  return hip_err(launch_rank_tiers(score, pos, eligible, n, tier_counts, n_tiers, tier_out, (hipStream_t)stream));
}

size_t qkv_export_bytes(const qkv_cache *c, int32_t what) {
  if (!c) return 0;
  if (what == QKV_EXPORT_STATE) return sizeof(Snapshot);
  if (c->tok) {
    const size_t n = (size_t)c->tg.B * c->tg.Hkv * c->tg.T;
    switch (what) {
      case QKV_EXPORT_TIERS: return n;
      case QKV_EXPORT_SCORES: return n * 4;
      case QKV_EXPORT_KEYS:
      case QKV_EXPORT_VALUES: return n * c->tg.d * 2;
      case QKV_EXPORT_ROUTED: return (size_t)c->tg.B * c->tg.Hkv * (4 + 4 * (size_t)tok_list_cap(c->tg)) * 4;
      case QKV_EXPORT_KCODES:
      case QKV_EXPORT_VCODES: return c->tg.policy == QKV_POLICY_HQEKV ? n * (c->tg.d / 2) : 0;
      case QKV_EXPORT_KPARAMS:
      case QKV_EXPORT_VPARAMS: return c->tg.policy == QKV_POLICY_HQEKV ? n * (c->tg.d / 32) * 4 : 0;
      case QKV_EXPORT_EVENT: return c->tg.policy != QKV_POLICY_QEVICT ? (size_t)c->tg.B * c->tg.Hkv * EV_WORDS * 4 : 0;
      case QKV_EXPORT_VICTIMS: return c->tg.policy != QKV_POLICY_QEVICT ? n * 4 : 0;
      default: return 0;
    }
  }
  // window policy: one layer's array per layer, layer-major
  const Geom &g = c->g;
  const size_t BU = (size_t)g.B * g.U;
  size_t per = 0;
  switch (what) {
    case QKV_EXPORT_TIERS:
    case QKV_EXPORT_LEDGER: per = BU; break;
    case QKV_EXPORT_SCORES: per = BU * 4; break;
    case QKV_EXPORT_KCODES:
    case QKV_EXPORT_VCODES: per = BU * g.Hkv * (size_t)(g.window * g.d * g.bits / 8); break;
    case QKV_EXPORT_KPARAMS: per = BU * g.Hkv * (size_t)g.d * 2 * 2; break;
    case QKV_EXPORT_VPARAMS: per = BU * g.Hkv * (size_t)g.window * (g.d / g.group) * 2 * 2; break;
    case QKV_EXPORT_KEYS:
    case QKV_EXPORT_VALUES: per = (size_t)g.B * g.Hkv * g.max_ctx * g.d * 2; break;
    case QKV_EXPORT_KEYS_RAW: per = g.rope ? (size_t)g.B * g.Hkv * g.max_ctx * g.d * 2 : 0; break;
    case QKV_EXPORT_ROUTED: per = BU * 4; break;
    case QKV_EXPORT_EVENT: per = (size_t)g.B * EV_WORDS * 4; break;
    case QKV_EXPORT_VICTIMS: per = BU * 4; break;
    default: return 0;
  }
  return per * (size_t)c->L;
}

int qkv_export(const qkv_cache *cc, int32_t what, void *dst, size_t bytes, qkv_stream stream) {
  if (!cc || !dst) return QKV_EINVAL;
  const size_t need = qkv_export_bytes(cc, what);
  if (need == 0 || bytes != need) return QKV_EINVAL;
  // an export reads derived structures only once they are rebuilt (the
  // handle is const to the caller; its pending rebuild is not caller state)
  qkv_cache *c = const_cast<qkv_cache *>(cc);
  if (settle(c, (hipStream_t)stream) != QKV_OK) return QKV_EHIP;
  if (what == QKV_EXPORT_STATE) {
    if (!layers_in_step(c)) return QKV_ESTATE;
    return hip_err(launch_write_snapshot(make_snapshot(c), dst, (hipStream_t)stream));
  }
  if (c->tok && what == QKV_EXPORT_ROUTED)
    return hip_err(tok_launch_export_routed(c->tg, c->ts, c->n_cmp, dst, (hipStream_t)stream));
  if (c->tok) {
    if (what == QKV_EXPORT_SCORES && c->tacc_dirty) {
      const TokStep ts = {c->N, c->r_tok, c->n_cmp};
      int rc = hip_err(tok_launch_flush(c->tg, c->ts, ts, (hipStream_t)stream));
      if (rc != QKV_OK) return rc;
      c->tacc_dirty = false;
    }
    return hip_err(tok_launch_export(c->tg, c->ts, what, dst, (hipStream_t)stream));
  }
  const size_t per = need / c->L;
  for (int l = 0; l < c->L; ++l) {
    const int rc = hip_err(launch_export(c->g, c->sts[l], step_info(c, l), what, (char *)dst + per * l,
                                         (hipStream_t)stream));
    if (rc != QKV_OK) return rc;
  }
  return QKV_OK;
}

int qkv_import(qkv_cache *c, int32_t what, const void *src, size_t bytes, qkv_stream stream) {
  if (!c || !src) return QKV_EINVAL;
  const size_t need = qkv_export_bytes(c, what);
  if (need == 0 || bytes != need) return QKV_EINVAL;
  if (what == QKV_EXPORT_EVENT || what == QKV_EXPORT_VICTIMS) return QKV_EINVAL;   // diagnostics, export only
  const hipStream_t s = (hipStream_t)stream;
  if (what == QKV_EXPORT_STATE) {
    Snapshot sn;
    if (hipMemcpyAsync(&sn, src, sizeof sn, hipMemcpyDeviceToHost, s) != hipSuccess) return QKV_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return QKV_EHIP;
    if (!snapshot_fits(c, sn)) return QKV_EINVAL;
    c->N = (int)sn.v[SNAP_N];
    for (int l = 0; l < c->L; ++l) c->Nl[l] = c->N;
    c->steps = sn.v[SNAP_STEPS];
    c->routes = sn.v[SNAP_ROUTES];
    c->steps_since_route = (int)sn.v[SNAP_SINCE_ROUTE];
    c->last_event_N = (int)sn.v[SNAP_LAST_EVENT];
    if (c->tok) {
      c->r_tok = (int)sn.v[SNAP_R];
      c->n_cmp = (int)sn.v[SNAP_RANKED];
      c->tacc_dirty = false;   // the imported scores hold every pending mass
    } else {
      c->r0 = (int)sn.v[SNAP_R];
      c->routed = (int)sn.v[SNAP_RANKED];
    }
    c->rebuild_pending = true;
    return QKV_OK;
  }
  if (what == QKV_EXPORT_ROUTED) {
    // list entries index pages and records: checked on the host before they
    // reach a kernel (a restore is not on the decode path, so the read-back
    // is affordable)
    std::vector<int32_t> h(need / 4);
    if (hipMemcpyAsync(h.data(), src, need, hipMemcpyDeviceToHost, s) != hipSuccess) return QKV_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return QKV_EHIP;
    if (c->tok) {
      const int Lc = tok_list_cap(c->tg);
      for (size_t r = 0; r < (size_t)c->tg.B * c->tg.Hkv; ++r) {
        const int32_t *row = h.data() + r * (4 + 4 * (size_t)Lc);
        for (int k = 0; k < 4; ++k) {
          if (row[k] < 0 || row[k] > Lc) return QKV_EINVAL;
          for (int e = 0; e < row[k]; ++e)
            if (row[4 + k * Lc + e] < 0 || row[4 + k * Lc + e] >= c->tg.T) return QKV_EINVAL;
        }
      }
    } else {
      for (int32_t u : h)
        if (u < 0 || u >= c->g.U) return QKV_EINVAL;
    }
  }
  if (!c->tok && what == QKV_EXPORT_LEDGER) {
    // ledger flags of every layer: windows holding codes get pool slots in
    // order (layer, sequence, window), the rest of the pool is free
    std::vector<uint8_t> f(need);
    if (hipMemcpyAsync(f.data(), src, need, hipMemcpyDeviceToHost, s) != hipSuccess) return QKV_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return QKV_EHIP;
    // each (layer, sequence) takes the first slots of its range, in window
    // order; the rest of the range is its free stack
    const size_t BU = (size_t)c->g.B * c->g.U;
    const int per = c->g.pool_per, nR = c->L * c->g.B;
    std::vector<int32_t> slot(need, 0), stack((size_t)nR * per), top(nR);
    for (int r = 0; r < nR; ++r) {
      int next = 0;
      for (int u = 0; u < c->g.U; ++u)
        if (f[(size_t)r * c->g.U + u]) {
          if (next >= per) return QKV_EINVAL;   // more ledgers than the range holds
          slot[(size_t)r * c->g.U + u] = r * per + next + 1;
          ++next;
        }
      for (int i = next; i < per; ++i) stack[(size_t)r * per + (i - next)] = r * per + i;
      top[r] = per - next;
    }
    for (int l = 0; l < c->L; ++l) {
      const State &st = c->sts[l];
      if (hipMemcpyAsync(st.has_ledger, (const uint8_t *)src + BU * l, BU, hipMemcpyDeviceToDevice, s) != hipSuccess ||
          hipMemcpyAsync(st.lslot, slot.data() + BU * l, BU * 4, hipMemcpyHostToDevice, s) != hipSuccess)
        return QKV_EHIP;
    }
    const State &st0 = c->sts[0];
    if (hipMemcpyAsync(st0.pool_stack, stack.data(), stack.size() * 4, hipMemcpyHostToDevice, s) != hipSuccess ||
        hipMemcpyAsync(st0.pool_top, top.data(), top.size() * 4, hipMemcpyHostToDevice, s) != hipSuccess)
      return QKV_EHIP;
    if (hipStreamSynchronize(s) != hipSuccess) return QKV_EHIP;   // the host vectors go out of scope
    c->ledger_ready = true;
    c->rebuild_pending = true;
    return QKV_OK;
  }
  if (!c->tok && (what == QKV_EXPORT_KCODES || what == QKV_EXPORT_VCODES || what == QKV_EXPORT_KPARAMS ||
                  what == QKV_EXPORT_VPARAMS) && !c->ledger_ready)
    return QKV_ESTATE;   // codes go to the slots the ledger flags assign
  int rc = QKV_OK;
  if (c->tok) {
    rc = hip_err(tok_launch_import(c->tg, c->ts, what, src, s));
  } else {
    const size_t per = need / c->L;
    for (int l = 0; l < c->L && rc == QKV_OK; ++l)
      rc = hip_err(launch_import(c->g, c->sts[l], what, (const char *)src + per * l, s));
  }
  if (rc != QKV_OK) return rc;
  if (c->tok && what == QKV_EXPORT_SCORES) c->tacc_dirty = false;
  c->rebuild_pending = true;
  return QKV_OK;
}

int qkv_info(const qkv_cache *c, int32_t what, int64_t *value) {
  if (!c || !value) return QKV_EINVAL;
  switch (what) {
    case QKV_INFO_TOKENS: *value = c->N; return QKV_OK;
    case QKV_INFO_LAYERS: *value = c->L; return QKV_OK;
    case QKV_INFO_UNITS: *value = c->tok ? c->tg.T : c->g.U; return QKV_OK;
    case QKV_INFO_STEPS: *value = c->steps; return QKV_OK;
    case QKV_INFO_ROUTES: *value = c->routes; return QKV_OK;
    case QKV_INFO_SPLITS: *value = c->tok ? c->tg.n_splits : c->g.n_splits; return QKV_OK;
    case QKV_INFO_WORKSPACE: *value = (int64_t)c->ws_bytes; return QKV_OK;
    case QKV_INFO_LIST_CAPACITY: *value = c->tok ? tok_list_cap(c->tg) : 0; return QKV_OK;
    default: return QKV_EINVAL;
  }
}

int qkv_status(qkv_cache *c, qkv_stream stream) {
  if (!c) return QKV_EINVAL;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return QKV_EHIP;
  for (int l = 0; l < c->L; ++l) {
    int32_t flag = 0;
    if (hipMemcpy(&flag, c->tok ? c->ts.status : c->sts[l].status, sizeof flag, hipMemcpyDeviceToHost) != hipSuccess)
      return QKV_EHIP;
    if (flag == QKV_ECAPACITY) return QKV_ECAPACITY;
    if (flag) return QKV_ERANGE;
  }
  return QKV_OK;
}

}  // extern "C"
