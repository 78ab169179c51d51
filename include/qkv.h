/*
 * qkv.h -- C ABI of the tiered KV-cache decode path for MI355X (gfx950).
 *
 * One cache object holds one transformer layer's KV state for a batch of
 * sequences that advance in lockstep.  Its memory is a single caller-owned
 * device workspace; the library never allocates device memory after
 * qkv_create and never frees caller memory.  Every call that takes a stream
 * only enqueues work on that stream (NULL = the null stream) and returns;
 * routing decisions, transition lists and live-unit lists stay on the device,
 * so no call waits for the GPU.  All tensor arguments are device pointers,
 * row-major, densely packed.  bfloat16 tensors are passed as uint16 storage.
 *
 * Error convention: every int-returning call returns QKV_OK (0) or a negative
 * QKV_E* code; arguments are validated on the host before anything is
 * enqueued, so a call that fails leaves the cache unchanged.  A device-side
 * condition (a quantization parameter outside float16 range) is latched in
 * the cache and reported by qkv_status().  No call throws.  A cache is not
 * thread-safe: use one cache per stream.
 *
 * Non-finite inputs: K, V and q must be finite.  The attention path does not
 * check them (a check would cost a pass over the data): a NaN or infinity
 * reaches the outputs, masses and scores of its (sequence, KV head), and a
 * NaN score takes part in the ranking by its bit pattern.  Every quantizer
 * (the routing pack, HqeKV re-quantization, qkv_quantize_window) does check
 * its groups: a NaN or infinity in a group makes its scale or zero
 * non-finite, which latches QKV_ERANGE as an out-of-range value does; the
 * group's codes are then not meaningful.
 *
 * Notation follows the pages: H_q query heads, H_kv KV heads, G = H_q/H_kv,
 * d = head dim, window = tokens per window (omega_w), omega = routing period
 * (Omega), K_f / K_q = windows kept in full precision / quantized.
 */
#ifndef QKV_H
#define QKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct qkv_cache qkv_cache;
typedef void *qkv_stream; /* a hipStream_t */

enum {
  QKV_OK = 0,
  QKV_EINVAL = -1,    /* bad shape, argument or configuration               */
  QKV_ECAPACITY = -2, /* max_ctx, list or workspace capacity exceeded       */
  QKV_ERANGE = -3,    /* a quantization parameter does not fit float16      */
  QKV_EHIP = -4,      /* HIP runtime error                                  */
  QKV_ESTATE = -5,    /* call out of order for the cache's policy or state  */
};

enum { QKV_POLICY_QEVICT = 0, QKV_POLICY_H2O = 1, QKV_POLICY_HQEKV = 2 };

/* Quantizer kinds of qkv_quantize_window. */
enum {
  QKV_KIND_K_PER_CHANNEL = 0, /* keys: one group per channel along tokens     */
  QKV_KIND_PER_TOKEN = 1,     /* values (and HqeKV keys): per token, channel groups */
  QKV_KIND_INT1_NORMAL = 2,   /* one-bit normalized quantizer per token       */
};

enum { QKV_DTYPE_BF16 = 0, QKV_DTYPE_F32 = 1 };

/* Unit tiers as exported by qkv_export(QKV_EXPORT_TIERS). */
enum {
  QKV_TIER_EMPTY = 0,   /* not yet appended                                  */
  QKV_TIER_SINK = 1,    /* protected prefix, always full precision            */
  QKV_TIER_RECENT = 2,  /* full precision, not yet ranked                     */
  QKV_TIER_FULL = 3,    /* ranked into the full-precision tier               */
  QKV_TIER_QUANT = 4,   /* ranked into the quantized (recoverable) tier      */
  QKV_TIER_EVICTED = 5, /* dropped for good                                  */
};

typedef struct qkv_config {
  int32_t batch;      /* sequences                                          */
  int32_t n_q_heads;  /* H_q                                                */
  int32_t n_kv_heads; /* H_kv; H_q % H_kv == 0, G = H_q / H_kv <= 8          */
  int32_t head_dim;   /* d in {64, 128}                                     */
  int32_t policy;     /* QKV_POLICY_*                                       */
  int32_t window;     /* tokens per window: 8, 16 or 32 (QEvict)            */
  int32_t omega;      /* routing period in decode steps                     */
  int32_t n_sink;     /* protected prefix tokens (<= 16)                    */
  int32_t n_recent;   /* protected recent tokens                            */
  int32_t k_full;     /* K_f: windows kept in full precision                */
  int32_t k_quant;    /* K_q: windows kept quantized                        */
  float ratios[5];    /* HqeKV shares: BF16, INT4, INT2, INT1-normal, evict */
  int32_t quant_bits; /* bits of the recoverable tier (2)                    */
  int32_t group;      /* quantization group (32)                            */
  int32_t max_ctx;    /* capacity in tokens per sequence                    */
  int32_t n_splits;   /* attention splits per (sequence, KV head); 0 = auto */
  int32_t score_window; /* HqeKV: 0 = every decode step adds to the scores;
                         * m in [1, omega] = a rolling window of the last m
                         * queries (HqeKV notes 3.8, 3.10): only the last m
                         * decode steps before each event add, and the scores
                         * restart from 0 after every event.  0 otherwise.   */
  int32_t chunk;      /* HqeKV: 0 = tokens are ranked one by one; c in [1, 64]
                       * = positions are ranked in chunks of c by the mean of
                       * their tokens' metrics, shares counted in chunks, the
                       * two best chunks kept BF16 (HqeKV notes 3.3);
                       * ceil(max_ctx / c) <= 4096.  0 otherwise.            */
  int32_t n_layers;   /* QEvict: layers held by the cache (0 or 1: one layer;
                       * at most 128).  Each layer has its own pages, scores,
                       * tiers and lists and is ranked by its own scores with the
                       * same capacities k_full / k_quant (QEvict notes 4.2: one
                       * score per layer and window; 4.3 and 4.5: capacities of
                       * a budget over all layers, qkv_plan_capacities); the
                       * ledgers of every layer share one pool.  1 otherwise.  */
  int32_t rope;       /* QEvict: 1 = keys arrive before the rotary embedding
                       * (QEvict notes 4.4, Algorithm 1's promotion step and the
                       * paragraph on promoted keys' positions): qkv_set_rope
                       * gives the table; full-precision pages hold the keys
                       * rotated once at their positions, the ledger quantizes
                       * the keys before rotation, the quantized tier is read
                       * rotated at the tokens' positions and a promoted window
                       * is rotated again at them.  Queries are given rotated.
                       * Windows of at most 16 tokens.  0 otherwise.          */
} qkv_config;

/* Bytes of device workspace a cache with this configuration needs, or 0 if
 * the configuration is invalid (see qkv_check_config for the reason). */
size_t qkv_workspace_bytes(const qkv_config *cfg);

/* QEvict capacities from a byte budget (QEvict notes §4.3, Eq.(budget) and
 * Eq.(3); §4.5 works the arithmetic for Llama-3.1-8B).  The budget
 * `budget_bytes` covers `layers` layers of this configuration's KV geometry
 * (per sequence); sinks and the recent region are held in BF16 and paid
 * first; of the rest, a share q in [0, 1] buys quantized windows and 1 - q
 * full-precision windows:
 *   M_f = window * layers * 2 * n_kv_heads * head_dim * 2 bytes,
 *   M_q = layers * n_kv_heads * (2 * window * head_dim * bits / 8
 *         + head_dim * ceil(window / group) * 4 + window * (head_dim / group) * 4),
 *   K_f = floor((1 - q) * B_hist / M_f),  K_q = floor(q * B_hist / M_q).
 * Writes K_f and K_q (host pointers); QKV_EINVAL for a non-QEvict or invalid
 * configuration, layers < 1, q outside [0, 1], a negative budget, or a budget
 * that does not cover the sinks and the recent region. */
int qkv_plan_capacities(const qkv_config *cfg, double budget_bytes, double q, int32_t layers, int32_t *k_full,
                        int32_t *k_quant);

/* QKV_OK if the configuration is supported, else QKV_EINVAL.  Besides the
 * ranges above: QEvict with head_dim 128 and eight query heads per KV head
 * needs 32-token windows (the attention workgroup's LDS would not fit). */
int qkv_check_config(const qkv_config *cfg);

/* Create a cache over `workspace` (device memory, at least
 * qkv_workspace_bytes(cfg) bytes, 256-byte aligned, owned by the caller and
 * kept alive until qkv_destroy).  The workspace is cleared on `stream`.
 * QKV_EINVAL also when the attention workgroup of this configuration would
 * not fit the current device's LDS. */
int qkv_create(const qkv_config *cfg, void *workspace, size_t bytes, qkv_stream stream,
               qkv_cache **out);

/* The rotary table of a cache created with rope = 1: device float32
 * [n_positions][head_dim/2][2] holding (cos, sin) of position p and frequency
 * i, which rotates the channel pair (i, i + head_dim/2):
 *   r_i = x_i cos - x_{i+d/2} sin,   r_{i+d/2} = x_{i+d/2} cos + x_i sin.
 * The quantized tier composes the row of a window's first position with the
 * row of the token's offset in it, so row p must be the rotation by p times
 * fixed angles (what a model's table is).  n_positions >= max_ctx; the table
 * is the caller's and must stay valid while the cache is used.  Required
 * before the first append (QKV_ESTATE otherwise); QKV_EINVAL for a cache
 * without rope. */
int qkv_set_rope(qkv_cache *cache, const float *table, int32_t n_positions);

/* Release the host-side handle (the workspace stays the caller's). */
int qkv_destroy(qkv_cache *cache);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * cache as qkv_create, with its workspace in a device array inside the
 * library instead of caller memory.  Each GPU holds its own array of
 * QKV_STATIC_WORKSPACE_BYTES bytes until the process ends; nothing is
 * allocated by this call or by later calls on the cache.  The array is
 * cleared for the new cache on `stream`.
 * One such cache per device at a time: a second qkv_create_static on the same
 * device replaces the first (both handles then name the new cache), and calls
 * on caches that share a device's array race.  qkv_destroy releases the
 * handle.  Errors: QKV_ECAPACITY when qkv_workspace_bytes(cfg) exceeds
 * QKV_STATIC_WORKSPACE_BYTES; QKV_EINVAL as qkv_create.
 */
#define QKV_STATIC_WORKSPACE_BYTES (64u << 20)
int qkv_create_static(const qkv_config *cfg, qkv_stream stream, qkv_cache **out);

/*
 * Policies.
 * QKV_POLICY_QEVICT: window units (window = 8, 16 or 32 tokens), one score
 *   per (sequence, window) summed over all query heads, three tiers (full
 *   precision, INT2 or INT4 ledger, evicted); routing every omega steps.  At
 *   most 16383 windows per sequence (the routing sort holds 16384 keys in
 *   LDS): max_ctx up to about 262K tokens at window = 16.
 * QKV_POLICY_H2O (H2O notes, sections 1.1-2.1 and the GQA paragraph): token
 *   units (window = 1, k_quant = 0), one score per (sequence, KV head, token)
 *   summed over the G query heads of that KV head; k_full is the heavy-hitter
 *   budget B_h, n_recent the recent budget B_r, n_sink protected sinks; call
 *   qkv_route after every decode step (omega = 1) to evict down to the budget.
 *   The scored prompt (section 1.2, each position accumulates from its own
 *   causal row): append it, qkv_prefill_score with its
 *   queries, then one qkv_route trims it.  max_ctx <= 16384 (a routing
 *   event ranks its candidates in LDS).
 * QKV_POLICY_HQEKV (HqeKV notes, sections 3.2-3.5 and 3.8): token units
 *   (window = 1, n_sink = 0), one score per (sequence, KV head, token) summed
 *   over the G query heads; ratios[0..4] are the shares of full precision,
 *   INT4, INT2, INT1 (normalized quantizer) and evicted tokens, summing to 1;
 *   omega is the assignment period in decode steps.  The prompt: append it,
 *   qkv_prefill_score with its last 20 queries (section 3.10, m = 20), then
 *   qkv_route makes the first assignment.
 */

/*
 * Append n_tokens new positions to every sequence.
 *   k, v: bfloat16 [batch, n_kv_heads, n_tokens, head_dim].
 * QEvict: positions go to their windows (the first n_sink positions form the
 * sink unit); every appended window is full precision and not yet ranked
 * (QEvict notes, Fig.1 stage 1: all windows start in full precision).
 * Errors: QKV_ECAPACITY if the total would exceed max_ctx.
 */
int qkv_append(qkv_cache *cache, const void *k, const void *v, int32_t n_tokens, qkv_stream stream);

/*
 * Multi-layer caches (n_layers > 1): the same calls for one layer.  Layers are
 * appended and attended one at a time, in any order within a decode step;
 * qkv_append and qkv_decode_attend act on layer 0.  qkv_route needs every
 * layer to hold the same number of tokens (QKV_ESTATE otherwise) and routes
 * all of them.  QKV_EINVAL for a layer outside [0, n_layers).
 */
int qkv_append_layer(qkv_cache *cache, int32_t layer, const void *k, const void *v, int32_t n_tokens,
                     qkv_stream stream);
int qkv_decode_attend_layer(qkv_cache *cache, int32_t layer, const void *q, float *out, float *mass_out,
                            qkv_stream stream);

/*
 * One decode step of single-query attention over the accessible cache, with
 * the attention mass each unit receives accumulated into its score.
 *   q:        bfloat16 [batch, n_q_heads, head_dim]
 *   out:      float32  [batch, n_q_heads, head_dim]
 *   mass_out: optional float32 [batch, n_kv_heads, n_units]: this step's mass
 *             per unit summed over the G query heads of each KV head (0 for
 *             units that were not accessible).  n_units: qkv_info(QKV_INFO_UNITS).
 * Attention is softmax(q K^T / sqrt(d)) V over sinks, not-yet-ranked windows,
 * full-precision windows and dequantized quantized windows (QEvict notes
 * section 4.1, Eq. attention); each head's mass on a unit below FLT_MIN counts
 * as 0; QEvict scores add the mass of all query heads (section 4.2, Eq.(1),
 * without its constant 1/H_q).
 */
int qkv_decode_attend(qkv_cache *cache, const void *q, float *out, float *mass_out, qkv_stream stream);

/*
 * A whole decode step in one call: qkv_append of one token (k, v: bfloat16
 * [batch, n_kv_heads, 1, head_dim]) followed by qkv_decode_attend, with the
 * same results bit for bit (QEvict notes section 4.1: the step appends the
 * token, then attends over the accessible cache including it).  For the
 * window policy without rotary keys the append is part of the attention
 * launch (the new token's row is taken from k and v, and stored in its page
 * for later steps); otherwise the two calls run in turn.  Errors as for the
 * two calls.  The _layer form acts on one layer of a multi-layer cache.
 */
int qkv_decode_step(qkv_cache *cache, const void *k, const void *v, const void *q, float *out, float *mass_out,
                    qkv_stream stream);
int qkv_decode_step_layer(qkv_cache *cache, int32_t layer, const void *k, const void *v, const void *q, float *out,
                          float *mass_out, qkv_stream stream);

/*
 * Routing event (QEvict notes section 4.4, Eq.(4)-(6), Algorithm 1): the
 * previous full and quantized windows and the windows that aged out of the
 * recent region are ranked by score (descending, ties to the later window);
 * the first k_full are full precision, the next k_quant quantized, the rest
 * evicted.  A window demoted for the first time is packed (keys per channel,
 * values per token, float16 scale/zero per group) into its persistent ledger;
 * later demotions reuse those codes; a promoted window is rebuilt in
 * full precision from its ledger.
 */
int qkv_route(qkv_cache *cache, qkv_stream stream);
/* H2O: the same call is the per-step eviction: tokens older than the newest
 * n_recent join the kept older tokens, and of those the k_full best by
 * (score descending, position descending) stay, the rest are evicted for
 * good (H2O notes section 2.1; the tie rule is this library's reading).
 * HqeKV: the same call is an assignment event (HqeKV notes sections 3.2, 3.3
 * and 3.5): the tokens appended before the previous event (all tokens at the
 * first event) are ordered by accumulated score times the value range of
 * their original value row (max - min over head_dim), float32, descending,
 * ties to the later position; the first floor(ratios[k] * N) of them (N =
 * tokens appended so far, shares taken as float32) target tier k in the
 * order full precision, INT4, INT2, INT1, and the rest are evicted.  A
 * token's tier only moves down (new = max(old, target)); a token that moves
 * to a quantized tier is re-quantized from its current values, keys and
 * values per token in groups of 32 channels with float16 scale and zero
 * (INT4, INT2) or as signs around the row mean with float16 mean and
 * standard deviation (INT1). */

/*
 * Scored prompt (H2O notes section 1.2; HqeKV notes sections 3.8 and 3.10): the queries of the last n_queries
 * appended positions, each attending causally to the live tokens at or before
 * its own position, add their weights (summed over each KV head's query
 * heads, each below FLT_MIN counting as 0) to the token scores; no output.
 *   q: bfloat16 [batch, n_queries, n_q_heads, head_dim]
 * Errors: QKV_ESTATE for the window policy, or when a scored position is
 * older than a token already ranked and kept by qkv_route.
 */
int qkv_prefill_score(qkv_cache *cache, const void *q, int32_t n_queries, qkv_stream stream);

/*
 * Stateless quantizer (HqeKV notes section 2.3 Eq.(2) uniform; Eq.(3)-(4)
 * one-bit normalized) over n_blocks independent blocks of [tokens, head_dim].
 *   x:      [n_blocks, tokens, head_dim], bfloat16 or float32 (x_dtype)
 *   codes:  uint8, canonical packed layout, codes_bytes(kind) per block:
 *           K_PER_CHANNEL: element (channel c, token t) has index c*tokens+t;
 *           PER_TOKEN / INT1_NORMAL: index t*head_dim+c; element e sits at bit
 *           bits*(e mod (8/bits)) of byte e*bits/8.
 *   params: float16 pairs per group, per block:
 *           K_PER_CHANNEL: [head_dim][ceil(tokens/group)][scale, zero]
 *           PER_TOKEN:     [tokens][head_dim/group][scale, zero]
 *           INT1_NORMAL:   [tokens][mean, std]
 * bits: 2 or 4 for the uniform kinds, 1 for INT1_NORMAL.  Groups are `group`
 * tokens (K_PER_CHANNEL) or channels (PER_TOKEN).  A parameter outside float16
 * range, or a group holding a NaN or infinity, latches QKV_ERANGE, reported
 * by qkv_quantize_status().
 */
int qkv_quantize_window(const void *x, int32_t x_dtype, int32_t n_blocks, int32_t tokens, int32_t head_dim,
                        int32_t bits, int32_t group, int32_t kind, uint8_t *codes, uint16_t *params,
                        qkv_stream stream);

/*
 * Stateless multi-tier ranking (HqeKV notes section 3.7, the 8-token worked
 * example: tokens ordered by their importance and cut by the tier shares;
 * H2O notes section 2.1 and section 5.1: one fixed order with position as the
 * tie key).  Entries with eligible[i] != 0 are ordered by (score descending,
 * pos descending); the first tier_counts[0] get tier 0, the next
 * tier_counts[1] tier 1, ..., the remaining eligible entries tier n_tiers,
 * ineligible entries 255.  score float32 [n], pos int32 [n], eligible uint8
 * [n], tier_counts int32 [n_tiers] (non-negative), tier_out uint8 [n]; all
 * device memory owned by the caller.  1 <= n <= 8192 (the ranking is one LDS
 * sort), 0 <= n_tiers <= 254; QKV_EINVAL otherwise.
 */
int qkv_rank_tiers(const float *score, const int32_t *pos, const uint8_t *eligible, int32_t n,
                   const int32_t *tier_counts, int32_t n_tiers, uint8_t *tier_out, qkv_stream stream);

/* Export state into device memory `dst` (`bytes` must equal the size below).
 * The kinds are the pieces of a session's state that the pages name: the
 * tier of every unit and its accumulated score (QEvict notes section 4.2
 * Eq.(1), section 4.4 Eq.(4)-(6)), the pack-once ledger of codes and float16
 * scale/zero (section 4.4, Algorithm 1 and its migration-stable quantization
 * paragraph; section 10h asks for a ledger whose lifetime follows the
 * window's), the content read in full precision, and -- for a session
 * restore (H2O notes section 6.2: the heavy/recent boundary, scores,
 * positions and the update step count) -- the ranked list order and the step
 * scalars.  Codes and parameters are in the canonical packing:
 *   QKV_EXPORT_TIERS   uint8   [batch, n_units]
 *   QKV_EXPORT_SCORES  float32 [batch, n_units]
 *   QKV_EXPORT_LEDGER  uint8   [batch, n_units]   1 if the unit holds ledger codes
 *   QKV_EXPORT_KCODES  uint8   [batch, n_units, n_kv_heads, window*head_dim*bits/8] canonical
 *   QKV_EXPORT_VCODES  uint8   [batch, n_units, n_kv_heads, window*head_dim*bits/8] canonical
 *   QKV_EXPORT_KPARAMS uint16  [batch, n_units, n_kv_heads, head_dim, 1, 2]
 *   QKV_EXPORT_VPARAMS uint16  [batch, n_units, n_kv_heads, window, head_dim/group, 2]
 *   QKV_EXPORT_KEYS    uint16  [batch, n_kv_heads, max_ctx, head_dim]  full-precision content
 *   QKV_EXPORT_VALUES  uint16  [batch, n_kv_heads, max_ctx, head_dim]
 *   QKV_EXPORT_ROUTED  int32   [batch, n_units]   ranked windows in rank order (full precision
 *                                                  first, then quantized); entries past the
 *                                                  ranked count are unspecified
 *   QKV_EXPORT_STATE   int64   [16]               format tag, policy, geometry and step scalars
 *   QKV_EXPORT_KEYS_RAW uint16 [batch, n_kv_heads, max_ctx, head_dim]  caches with rope = 1: the
 *                                                  keys as appended, before the rotation (the
 *                                                  ledger packs from them); KEYS holds them
 *                                                  rotated
 *   QKV_EXPORT_EVENT   int32   [batch, 16]        the last routing event of each sequence (H2O
 *                                                  notes section 5.1: log what each eviction
 *                                                  decided and how close its cut was): tokens
 *                                                  in the cache, candidates, kept full, kept
 *                                                  quantized, evicted, promoted, demoted,
 *                                                  first packs, ledger reuses, ledger slots
 *                                                  freed (words 0..9); then float32 bits of the
 *                                                  relative score gap (lowest kept minus highest
 *                                                  dropped, over the larger) at the K_f cut, at
 *                                                  the K_f + K_q cut and their minimum (words
 *                                                  10..12; +inf where the ranking has no such
 *                                                  cut); zero before the first event
 *   QKV_EXPORT_VICTIMS int32   [batch, n_units]   windows the last event evicted, best-ranked
 *                                                  first (their scores: SCORES; their positions:
 *                                                  the window spans), -1 past them
 *   (EVENT and VICTIMS are diagnostics: export only)
 * H2O also writes them per (sequence, KV head) at every eviction call that
 * ranks: EVENT int32 [batch, n_kv_heads, 16] with tokens, candidates, kept
 * heavy hitters, evicted (words 0..4 with 1 and 3 as above: 2 kept, 3 zero,
 * 4 evicted), the margin at the heavy-hitter cut (word 10, also word 12;
 * word 11 +inf); VICTIMS int32 [batch, n_kv_heads, max_ctx] the evicted
 * positions, best-ranked first (their age is tokens - 1 - position).
 * HqeKV writes them per (sequence, KV head) at every assignment event:
 * EVENT words 0 tokens, 1 tokens ranked, 2 BF16, 3 INT2, 8 INT4 and 9 INT1
 * tokens of the ranked positions after the event, 4 tokens it evicted, 6
 * tokens it moved to a lower tier, 7 of them re-quantized (6 minus 4), 5
 * zero (downgrade only); float32 margins (the metric score x value range,
 * relative gap across the cut) at the BF16|INT4 (10), INT4|INT2 (11),
 * INT2|INT1 (13) and INT1|evict (14) cuts and their minimum (12), +inf where
 * a cut falls outside the ranking and with chunk ranking; VICTIMS int32
 * [batch, n_kv_heads, max_ctx] the positions the event evicted, in position
 * order, -1 past them.
 * (units without a ledger export zero codes and parameters).  A cache of
 * n_layers > 1 exports every per-layer kind as n_layers such arrays, layer
 * after layer (STATE once; QKV_ESTATE unless every layer holds the same
 * number of tokens).
 * Token policies (H2O, HqeKV), per (sequence, KV head, position):
 *   TIERS uint8 [batch, n_kv_heads, max_ctx]; SCORES float32 [same] (masses
 *   pending in list order are added first); KEYS / VALUES uint16 [batch,
 *   n_kv_heads, max_ctx, head_dim] (the appended originals); HqeKV also
 *   KCODES / VCODES uint8 [batch, n_kv_heads, max_ctx, head_dim/2] and
 *   KPARAMS / VPARAMS uint16 [batch, n_kv_heads, max_ctx, head_dim/32, 2]
 *   (per-token records); ROUTED int32 [batch, n_kv_heads, 4 + 4*L]: the token
 *   counts of the full-precision, INT4, INT2 and INT1 lists, then the four
 *   lists of positions in list order, L = qkv_info(QKV_INFO_LIST_CAPACITY)
 *   entries each (H2O: the kept heavy hitters in list 0); STATE as above.
 * A kind a policy does not hold is QKV_EINVAL.
 */
enum {
  QKV_EXPORT_TIERS = 0,
  QKV_EXPORT_SCORES = 1,
  QKV_EXPORT_LEDGER = 2,
  QKV_EXPORT_KCODES = 3,
  QKV_EXPORT_VCODES = 4,
  QKV_EXPORT_KPARAMS = 5,
  QKV_EXPORT_VPARAMS = 6,
  QKV_EXPORT_KEYS = 7,
  QKV_EXPORT_VALUES = 8,
  QKV_EXPORT_ROUTED = 9,
  QKV_EXPORT_STATE = 10,
  QKV_EXPORT_KEYS_RAW = 11,
  QKV_EXPORT_EVENT = 12,
  QKV_EXPORT_VICTIMS = 13,
};
int qkv_export(const qkv_cache *cache, int32_t what, void *dst, size_t bytes, qkv_stream stream);
size_t qkv_export_bytes(const qkv_cache *cache, int32_t what);

/*
 * Session restore (H2O notes section 6.2: restoring a session needs the
 * heavy/recent boundary, the scores, the positions and the update step
 * count; QEvict notes section 10h: the ledger of codes and scale/zero lives
 * as long as its window).  `src` is device memory in the layout qkv_export
 * writes for the same kind and `bytes` must equal qkv_export_bytes(cache,
 * what).  A full restore imports, into a cache created with the same
 * configuration, every kind the policy exports:
 *   QEvict: STATE, TIERS, SCORES, LEDGER, ROUTED, KCODES, VCODES, KPARAMS,
 *           VPARAMS, KEYS, VALUES;
 *   H2O:    STATE, TIERS, SCORES, ROUTED, KEYS, VALUES;
 *   HqeKV:  the H2O kinds plus KCODES, VCODES, KPARAMS, VPARAMS.
 * The order is free, except that QEvict's LEDGER (which hands out the ledger
 * pool's slots) comes before KCODES, VCODES, KPARAMS and VPARAMS (QKV_ESTATE
 * otherwise).  Structures derived from these (list-order scores, the
 * compact tiles of the ranked lists, value ranges) are rebuilt on `stream`
 * before the next append, attention, prompt scoring, routing or export, so a
 * restored cache continues exactly as the exported one does.  No pending
 * masses are carried: with a routing period above 1 the token policies keep
 * each step's masses in list order until the next routing call, and an
 * export of SCORES adds them into the scores first (the exported cache then
 * continues from those scores too; a cache never exported adds a period's
 * masses at once, which can differ from it in the last float32 bits).  STATE is read back to the
 * host, so importing it waits for `stream`.  Errors: QKV_EINVAL for a kind
 * the policy does not hold, a wrong size, or a STATE whose format tag,
 * policy or geometry differs from the cache's or whose step scalars are out
 * of range (the cache is then unchanged).
 */
int qkv_import(qkv_cache *cache, int32_t what, const void *src, size_t bytes, qkv_stream stream);

/* Host-side counters. */
enum {
  QKV_INFO_TOKENS = 0,      /* positions appended per sequence               */
  QKV_INFO_UNITS = 1,       /* units per sequence (sink unit + windows)      */
  QKV_INFO_STEPS = 2,       /* decode steps attended                         */
  QKV_INFO_ROUTES = 3,      /* routing events                                */
  QKV_INFO_SPLITS = 4,      /* attention splits per (sequence, KV head)      */
  QKV_INFO_WORKSPACE = 5,   /* workspace bytes in use                        */
  QKV_INFO_LIST_CAPACITY = 6, /* token policies: entries per list of QKV_EXPORT_ROUTED */
  QKV_INFO_LAYERS = 7,      /* layers held                                   */
};
int qkv_info(const qkv_cache *cache, int32_t what, int64_t *value);

/* Kernel timing: after qkv_profile_start(cache, n, stride), every stride-th of
 * the following qkv_decode_attend calls (the 1st, the (1+stride)-th, ...)
 * records a pair of HIP events on its stream around the attention kernel (not
 * the merge), n pairs in all.  Sampling keeps the event packets, which delay
 * the next launch, out of most steps.  qkv_profile_read waits for the last pair
 * and writes the recorded durations in milliseconds (n entries, at most as many
 * as were recorded).  Events are created by qkv_profile_start (no device
 * memory) and released by the next start or by qkv_destroy.  stride >= 1. */
int qkv_profile_start(qkv_cache *cache, int32_t n, int32_t stride);
int qkv_profile_read(qkv_cache *cache, float *ms, int32_t n);

/* Device-latched status of every layer: waits for `stream`, returns QKV_OK,
 * QKV_ERANGE (a quantization parameter outside float16 range, or a quantized
 * group holding a NaN or infinity) or
 * QKV_ECAPACITY (the ledger pool ran out: cannot happen with the pool sized
 * as qkv_workspace_bytes sizes it, latched rather than faulting). */
int qkv_status(qkv_cache *cache, qkv_stream stream);
/* Status latched by qkv_quantize_window calls since the last query (same rule). */
int qkv_quantize_status(qkv_stream stream);

const char *qkv_strerror(int code);
/* The HIP runtime's description of the error behind the calling thread's
 * most recent QKV_EHIP ("no error" if there was none). */
const char *qkv_hip_error_detail(void);

#ifdef __cplusplus
}
#endif
#endif /* QKV_H */
