/*
 * bkv.h -- C ABI of the BeaconKV eviction-step library (libbkv.so, gfx950).
 *
 * BeaconKV keeps, per attention head, a bounded buffer of pre-RoPE queries
 * maintained by continual farthest point sampling (FPS).  At each eviction it
 * scores every cached key with the buffered "beacon" queries rotated to the
 * current step plus the recent queries at their own positions, max-pools the
 * attention weights over queries and over the GQA group, keeps the prefix,
 * the recent window and the top-k keys, and compacts K/V in place.
 *
 * Citations name the reading notes "BeaconKV：用历史查询代表保护长推理的远程回看"
 * (liuzhao09.github.io, "Notes") and the rcap.io post "BeaconKV: Key-Value
 * Cache Compression Guided by Beacon Queries" ("Summary").
 *
 * Layout.  A unit is one (layer, batch element, KV head):
 *     u  = (l * batch + b) * n_kv_heads + g
 * and a query buffer is one (layer, batch element, query head):
 *     uq = (l * batch + b) * n_q_heads + h,   query head h reads KV head h / G,
 * G = n_q_heads / n_kv_heads.  Dense row-major arrays:
 *     K, V        bf16  [units][cap][head_dim]       K holds post-RoPE keys
 *     qbuf        bf16  [qbufs][qcap][head_dim]      pre-RoPE query buffers
 *     qcount      int32 [qbufs]                      valid rows per buffer
 *     q_new       bf16  [qbufs][head_dim]            this step's pre-RoPE query
 *     q_recent    bf16  [qbufs][n_recent_q][head_dim] pre-RoPE recent queries
 *     pos_recent  int32 [batch][n_recent_q]          their positions
 *     t           int32 [batch]                      current step per sequence
 *     rope_cs     fp32  [rope_rows][head_dim/2][2]   {cos, sin} table
 *     scores      fp32  [units][n_len]
 *     idx         int32 [units][budget]
 *     fps_sel     int32 [qbufs][n_beacon]
 * i.e. per layer the usual [batch][heads][seq][head_dim] cache layout, with
 * layers outermost.  Device pointers must be 16-byte aligned.
 *
 * Ownership.  The caller owns all memory; the library never allocates, frees
 * or keeps a pointer after a call returns.  In/out arguments are modified in
 * place as documented per call.
 *
 * Execution.  Every device call only enqueues kernels on `stream` (a
 * hipStream_t; NULL is the null stream) and returns without synchronising.
 * No call needs a workspace: every kernel keeps its intermediate results
 * (scores, keep sets, Gram matrices) on chip or in the caller's output
 * buffers.  The only global state is a per-device, per-head-size memo of
 * the FPS update kernel's resident workgroup count, filled by the first
 * call that needs it (written atomically; every writer stores the same
 * value); the library is re-entrant, and calls that overlap on the same
 * buffers race.
 *
 * Errors.  Calls return BKV_OK or a negative code.  Validation of shapes,
 * null and misaligned pointers, and every host query a call needs (the
 * occupancy memo above, device attributes) happen before its first launch,
 * so a call that fails with BKV_EINVAL, BKV_EUNSUPPORTED or BKV_ERANGE, or
 * with BKV_EHIP from such a query, has enqueued nothing.  A call that
 * enqueues several kernels (bkv_evict, bkv_decode_step) and gets BKV_EHIP
 * from a later launch may leave the earlier kernels enqueued.  Device data
 * (qcount, positions, idx) is clamped into the range the buffers allow,
 * never trusted for addressing.  Faults of a launched kernel surface at the
 * caller's next synchronisation.  No C++ exception crosses this interface.
 */
#ifndef BKV_H
#define BKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BKV_ABI_VERSION 5

typedef uint16_t bkv_bf16; /* raw bf16 bits */

enum {
    BKV_OK = 0,
    BKV_EINVAL = -1,       /* null/misaligned pointer, inconsistent shape */
    BKV_EUNSUPPORTED = -2, /* shape outside what the kernels implement */
    BKV_ERANGE = -3,       /* sizes out of range (n_len > cap, budget too small, ...) */
    BKV_EHIP = -4          /* a kernel launch failed */
};

/* flags */
#define BKV_CAUSAL_RECENT 1u /* recent query i sees only slots <= n_len - n_recent_q + i */
#define BKV_POOL_MEAN 2u     /* scores pool the weights by their mean, not their max (see bkv_score) */
/* Source of the beacons (at most one; neither = continual FPS, Notes §2.2).
 * The buffer, its count and the cycle stay as for continual FPS; only the
 * update, the merge and the prefill change:
 *   BKV_BEACON_INITIAL (Initial+Recent, Notes §3.4 Table 3): the first
 *     n_beacon queries a buffer is offered; later ones are ignored and the
 *     merge keeps the buffer.
 *   BKV_BEACON_RANDOM (random history, Notes §3.2 Fig. 6): a uniform random
 *     sample of n_beacon of all queries offered so far, by reservoir sampling
 *     (Vitter's Algorithm R).  qcount counts the offers; offer n (0-based)
 *     takes slot n while n < n_beacon, else slot floor(r (n + 1) / 2^32) if
 *     below n_beacon, where r is the first output word of Philox4x32-10
 *     (Salmon et al., SC 2011) at counter (n, uq, 0, 0) and key (seed, 0).
 *     Updates offer the step's query; the merge offers the recents in ring
 *     order. */
#define BKV_BEACON_INITIAL 4u
#define BKV_BEACON_RANDOM 8u
/* BKV_BEACON_NAIVE (naive full-history FPS, the memory-hungry baseline of
 * Notes §3.2 Fig. 7): the caller keeps every past query of each head in a
 * history (bkv_history_append) and, before each eviction, fills the buffers
 * with FPS(history, n_beacon) by bkv_fps_history.  The continual update and
 * the merge then leave the buffers alone (fps_sel receives -1s), and
 * bkv_decode_step touches no buffer in the collection phase. */
#define BKV_BEACON_NAIVE 16u

typedef struct bkv_shape {
    int32_t n_layers, batch, n_q_heads, n_kv_heads, head_dim; /* head_dim in {64, 128}; G <= 8 */
    int32_t cap;          /* rows allocated per unit in K and V */
    int32_t budget;       /* B_KV^min: rows kept by an eviction */
    int32_t n_prefix;     /* forced keep of the first rows */
    int32_t n_recent_kv;  /* forced keep of the last rows */
    int32_t n_beacon;     /* B_Q^min: beacons kept by FPS */
    int32_t n_recent_q;   /* recent queries; B_Q^max = n_beacon + n_recent_q <= 32 */
    int32_t qcap;         /* rows allocated per query buffer, >= B_Q^max */
    uint32_t flags;       /* BKV_CAUSAL_RECENT | BKV_POOL_MEAN | one BKV_BEACON_* */
    uint32_t seed;        /* key of the BKV_BEACON_RANDOM draws */
} bkv_shape;

/* ABI version (BKV_ABI_VERSION). */
int bkv_version(void);

/* Workspace a call needs for this shape and cache length: always 0 (no
 * kernel uses scratch memory, see Execution above).  Kept so that callers
 * sizing a workspace before each call need no special case. */
size_t bkv_workspace_bytes(const bkv_shape *shape, int32_t n_len);

/* Static text for an error code. */
const char *bkv_strerror(int code);

/* Host only.  RoPE table for positions [p0, p1):
 *   host_out[((p - p0) * head_dim/2 + i) * 2 + {0, 1}] = {cos, sin}(p * theta^(-2i/head_dim)),
 * angles in fp64, rounded to fp32; pairs are (i, i + head_dim/2), the
 * convention of the model families the Notes evaluate (§3.1).  The caller
 * uploads it once and passes it to bkv_score / bkv_evict with rope_rows =
 * p1 when p0 = 0.  Errors: BKV_EINVAL (null, odd or non-positive head_dim,
 * p0 < 0 or p1 <= p0). */
int bkv_rope_table(double theta, int32_t head_dim, int32_t p0, int32_t p1, float *host_out);

/* Continual FPS buffer update, one decode step (Notes §2.2 Eq. 9 and App.
 * Alg. 1; Summary, pseudocode).  For every buffer uq: append q_new[uq] at
 * slot qcount[uq]; if the count reaches B_Q^max, replace the buffer by
 * FPS(buffer, n_beacon) -- seed at the lowest mean cosine, then repeatedly
 * the row whose largest cosine to the rows taken is smallest, ties to the
 * lowest slot, cosines in a fixed fp32 order -- with the survivors in
 * ascending slot order, and set qcount to n_beacon.
 * In/out: qbuf (rows [0, qcount) valid afterwards), qcount.  fps_sel may be
 * NULL; else it receives the selection order, or -1s where no sampling ran.
 * qcount is clamped to [0, B_Q^max - 1] on entry.  Under BKV_BEACON_INITIAL
 * or BKV_BEACON_RANDOM the update is instead one offer of q_new[uq] by that
 * rule (see the flags; qcount < 0 reads as 0), and fps_sel receives -1s. */
int bkv_fps_update(const bkv_shape *shape, bkv_bf16 *qbuf, int32_t *qcount,
                   const bkv_bf16 *q_new, int32_t *fps_sel, void *stream);

/* Compression at the freeze point of a cycle (Notes §2.2 App. Alg. 2: the
 * beacons a cycle is scored with represent every query it collected).  Every
 * buffer holding more than n_beacon rows (qcount clamped to [0, B_Q^max - 1]
 * when read) becomes FPS(buffer, n_beacon) exactly as in bkv_fps_update,
 * survivors in ascending slot order and qcount = n_beacon; other buffers are
 * left as they are.  fps_sel (nullable) receives the selection order, or -1s
 * where no sampling ran.  bkv_decode_step runs it on the first step of the
 * recent phase.  A no-op under BKV_BEACON_INITIAL, _RANDOM or _NAIVE, whose
 * buffers never hold more than n_beacon beacons. */
int bkv_fps_compress(const bkv_shape *shape, bkv_bf16 *qbuf, int32_t *qcount, int32_t *fps_sel, void *stream);

/* Longest prompt bkv_fps_prefill takes. */
#define BKV_PREFILL_MAX 8192

/* Prefill initialisation of the query buffers (Notes §2.2: at prefill the
 * first representatives are sampled from the prompt's queries, by the FPS of
 * App. Alg. 1).  For every buffer uq, q_prompt[uq][0 : n_prompt) holds the
 * head's pre-RoPE prompt queries (bf16 [qbufs][n_prompt][head_dim]); the
 * buffer becomes FPS(prompt, n_beacon), survivors in ascending prompt order,
 * and qcount[uq] their number, min(n_prompt, n_beacon).  fps_sel (nullable)
 * receives the selection order, -1 past the last pick.
 * The FPS is that of bkv_fps_update except the seed: the mean cosine of row i
 * is computed as u_i . s / n with u_j = q_j * (1 / |q_j|) (0 for a zero row)
 * and s[k] the pairwise sum of u_j[k] over j (a balanced binary tree over the
 * row index, zero rows padding it to a power of two), which costs O(n d)
 * instead of O(n^2 d); the fma chains, norms, cosines, argmins and ties are
 * as in bkv_fps_update.  Inputs must be finite with finite squared norms.
 * Under BKV_BEACON_INITIAL the buffer takes the first min(n_prompt,
 * n_beacon) prompt rows (count likewise); under BKV_BEACON_RANDOM every
 * prompt row is offered in order (count n_prompt); fps_sel then holds the
 * prompt row kept in each slot (-1 for an empty slot).
 * Errors: BKV_EINVAL (null or misaligned pointer, n_prompt < 0),
 * BKV_EUNSUPPORTED (n_prompt > BKV_PREFILL_MAX). */
int bkv_fps_prefill(const bkv_shape *shape, const bkv_bf16 *q_prompt, int32_t n_prompt,
                    bkv_bf16 *qbuf, int32_t *qcount, int32_t *fps_sel, void *stream);

/* Query history of the naive full-history beacons (BKV_BEACON_NAIVE; Notes
 * §3.2 Fig. 7): for every buffer uq, hist[uq][hcount[uq]] = q_new[uq] and
 * hcount[uq] grows by one, while hcount[uq] < hcap (a full history takes no
 * more rows; a negative count reads as 0).  hist: bf16 [qbufs][hcap][head_dim];
 * hcount: int32 [qbufs]; q_new: bf16 [qbufs][head_dim].  In/out: hist, hcount.
 * Errors: BKV_EINVAL (null or misaligned pointer, hcap < 0). */
int bkv_history_append(const bkv_shape *shape, bkv_bf16 *hist, int32_t hcap, int32_t *hcount,
                       const bkv_bf16 *q_new, void *stream);

/* Beacons from the whole history (BKV_BEACON_NAIVE; Notes §3.2 Fig. 7, with
 * the FPS of App. Alg. 1): for every buffer uq, the buffer becomes
 * FPS(hist[uq][0 : n_rows), n_beacon) exactly as bkv_fps_prefill samples a
 * prompt (same seed rule, order and ties; survivors in ascending history
 * order, qcount = min(n_rows, n_beacon)).  The rows of buffer uq start at
 * hist + uq * hcap * head_dim; bkv_fps_prefill is the case hcap = n_rows.
 * fps_sel (nullable) receives the selection order.  Errors: BKV_EINVAL (null
 * or misaligned pointer, n_rows < 0 or > hcap), BKV_EUNSUPPORTED (n_rows >
 * BKV_PREFILL_MAX). */
int bkv_fps_history(const bkv_shape *shape, const bkv_bf16 *hist, int32_t hcap, int32_t n_rows,
                    bkv_bf16 *qbuf, int32_t *qcount, int32_t *fps_sel, void *stream);

/* Scores of every cached key (Notes §2.1 Eq. 4-5, §2.3 Eq. 7).  Per unit,
 * the observation rows of each of its G query heads are the beacons
 * qbuf[uq][0 : min(qcount, n_beacon)) rotated to t[b] and the recent queries
 * q_recent[uq][i] rotated to pos_recent[b][i] (rotation in fp32 with each
 * product and sum rounded, result rounded to bf16).  With z = q.k / sqrt(d)
 * over the keys a row sees (all n_len keys for beacons; for recent row i,
 * under BKV_CAUSAL_RECENT, keys <= n_len - n_recent_q + i):
 *   scores[u][j] = max over rows r of exp(z_rj - logsumexp_j' z_rj').
 * Under BKV_POOL_MEAN (Notes §2.1 Eq. 6, pooled over queries and heads as in
 * the Max/Mean ablation of Notes §3.3 Table 2) the max becomes the sum over
 * the rows divided by their number, sum_h min(qcount, n_beacon) + n_recent_q
 * over the group; a row's weight on a key it does not see counts as 0.
 * bf16 MFMA products with fp32 accumulation.  Positions are clamped to
 * [0, rope_rows).  Out: scores [units][n_len]. */
int bkv_score(const bkv_shape *shape, const bkv_bf16 *K, int32_t n_len,
              const bkv_bf16 *qbuf, const int32_t *qcount, const bkv_bf16 *q_recent,
              const int32_t *pos_recent, const int32_t *t,
              const float *rope_cs, int32_t rope_rows, float *scores, void *stream);

/* Keep set (Notes §2.3 Eq. 8, 0-based): I_keep = [0, n_prefix) U
 * [n_len - n_recent_kv, n_len); the budget - |I_keep| highest-scoring other
 * keys (ties to the lower index) join it; idx[u] lists the kept slots in
 * ascending order.  If n_len <= budget, idx[u] = 0..n_len-1 then -1s.
 * Scores must be >= 0 (weights are).  Out: idx [units][budget]. */
int bkv_select(const bkv_shape *shape, const float *scores, int32_t n_len,
               int32_t *idx, void *stream);

/* In-place compaction (Notes §2.3 Eq. 8: K^ = K[:, I_final, :], V^ likewise):
 * row r of K and V becomes row idx[u][r], r < min(n_len, budget).  idx[u]
 * must be strictly ascending (as bkv_select writes it); rows >= budget keep
 * stale data.  In/out: K, V. */
int bkv_compact(const bkv_shape *shape, bkv_bf16 *K, bkv_bf16 *V, int32_t n_len,
                const int32_t *idx, void *stream);

/* End-of-cycle merge (Notes §2.2, App. Alg. 2): per buffer, the beacons
 * qbuf[uq][0 : min(qcount, n_beacon)) followed by q_recent[uq] are reduced
 * by FPS to n_beacon rows (all of them if there are no more), written in
 * candidate order to qbuf[uq], and qcount becomes their number.  fps_sel
 * (nullable) receives the selection order (-1 padded).  Under
 * BKV_BEACON_INITIAL nothing changes; under BKV_BEACON_RANDOM the recents
 * are offered in ring order; fps_sel receives -1s for both. */
int bkv_fps_merge(const bkv_shape *shape, bkv_bf16 *qbuf, int32_t *qcount,
                  const bkv_bf16 *q_recent, int32_t *fps_sel, void *stream);

/* One whole eviction (Notes §2.2 App. Alg. 2 and §2.3; Summary,
 * pseudocode) over all units: the scores of bkv_score, the keep set of
 * bkv_select and the compaction of bkv_compact, computed per unit by one
 * workgroup without leaving the chip in between (so the unit's keys are
 * re-read from the on-die cache rather than from HBM), then bkv_fps_merge.
 * idx_out ([units][budget]), scores_out ([units][n_len]) and fps_sel_out
 * ([qbufs][n_beacon]) are optional copies of the intermediate results
 * (NULL: not written); the results equal those of the separate calls.
 * In/out: K, V, qbuf, qcount. */
int bkv_evict(const bkv_shape *shape, bkv_bf16 *K, bkv_bf16 *V, int32_t n_len,
              bkv_bf16 *qbuf, int32_t *qcount, const bkv_bf16 *q_recent,
              const int32_t *pos_recent, const int32_t *t,
              const float *rope_cs, int32_t rope_rows,
              int32_t *idx_out, float *scores_out, int32_t *fps_sel_out, void *stream);

/* One decode step of the eviction cycle (Notes §2.2 App. Alg. 2; Summary,
 * pseudocode) at cache length L: rows [0, L) of every unit are valid and
 * 0 <= L < cap.
 *   - Unit u appends k_new[u], rotated to position pos[b] exactly as
 *     bkv_score rotates its observation rows, at row L of K, and v_new[u]
 *     at row L of V.
 *   - Query buffer uq takes q_new[uq].  While L < cap - n_recent_q (the
 *     cycle's collection phase) it is appended by bkv_fps_update's rule.  In
 *     the last n_recent_q steps before the cache is full the buffer is left
 *     as it is (its first rows are this cycle's beacons) and the query goes
 *     to the recent ring: q_recent[uq][i] = q_new[uq], pos_recent[b][i] =
 *     pos[b], i = L - (cap - n_recent_q).  On the first of these steps the
 *     buffers are first compressed by bkv_fps_compress, so that the beacons
 *     represent every query of the collection phase.
 * After the step with L = cap - 1 the cache is full; the caller then runs
 * bkv_evict with n_len = cap and t = the last step's pos, which leaves
 * L = budget.
 * k_new, v_new: bf16 [units][head_dim] (k_new pre-RoPE); q_new: bf16
 * [qbufs][head_dim]; pos: int32 [batch].  Positions are clamped to
 * [0, rope_rows).  In/out: K, V (row L), qbuf, qcount, q_recent,
 * pos_recent.  fps_sel (nullable) as in bkv_fps_update; not written in the
 * ring phase.  Errors: BKV_ERANGE if L < 0, L >= cap or rope_rows <= 0;
 * BKV_EINVAL for null or misaligned pointers. */
int bkv_decode_step(const bkv_shape *shape, bkv_bf16 *K, bkv_bf16 *V, int32_t L,
                    const bkv_bf16 *k_new, const bkv_bf16 *v_new, const int32_t *pos,
                    bkv_bf16 *qbuf, int32_t *qcount, const bkv_bf16 *q_new,
                    bkv_bf16 *q_recent, int32_t *pos_recent,
                    const float *rope_cs, int32_t rope_rows, int32_t *fps_sel, void *stream);

/* Append of one decode step's key and value (the cache growth of Notes §2.1,
 * the second formula): per unit, K[u][L] = k_new[u] rotated to pos[b] (fp32,
 * each product and sum rounded, then bf16 round to nearest even) and V[u][L]
 * = v_new[u].  k_new, v_new: bf16 [units][head_dim] (k_new pre-RoPE); pos:
 * int32 [batch], clamped to [0, rope_rows).  This is the first half of
 * bkv_decode_step, for callers that run the plain decode loop (no
 * eviction).  Errors: BKV_ERANGE (L < 0, L >= cap, rope_rows <= 0). */
int bkv_append_kv(const bkv_shape *shape, bkv_bf16 *K, bkv_bf16 *V, int32_t L, const bkv_bf16 *k_new,
                  const bkv_bf16 *v_new, const int32_t *pos, const float *rope_cs, int32_t rope_rows,
                  void *stream);

/* One decode step's attention over the cache (Notes §2.1, the second
 * formula; the new key and value already appended): for every query buffer
 * uq = u * G + h, q[uq] (bf16 pre-RoPE, [qbufs][head_dim]) is rotated to
 * pos[b] as the scoring queries are, and
 *   out[uq][k] = sum_{j < n_len} w_j V[u][j][k],  w = softmax_j(q . K[u][j] / sqrt(head_dim)),
 * fp32 [qbufs][head_dim].  Logits by bf16 MFMA with fp32 accumulation, the
 * rest in fp32.  Errors: BKV_ERANGE (n_len < 1 or > cap, rope_rows <= 0). */
int bkv_decode_attention(const bkv_shape *shape, const bkv_bf16 *K, const bkv_bf16 *V, int32_t n_len,
                         const bkv_bf16 *q, const int32_t *pos, const float *rope_cs, int32_t rope_rows,
                         float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BKV_H */
