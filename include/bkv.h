/*
 * bkv.h -- C ABI of the BeaconKV eviction-step library for MI355X (gfx950).
 *
 * The library implements the data-parallel eviction step of BeaconKV
 * ("BeaconKV: Key-Value Cache Compression Guided by Beacon Queries for
 * Efficient Large Reasoning Model Inference"; cited below as *paper text*
 * for the paper's own prose, *summary* for the structured summary page whose
 * section "方法步骤详情" restates Algorithm 2 as steps (1)-(6), and *review*
 * for the jaehun.me review page).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers allocated and owned by the caller.
 *    The library allocates no device memory in these calls and keeps no
 *    state between calls; scratch memory comes from the caller's workspace
 *    (bkv_evict_noalloc alone uses a fixed array of the library instead).
 *  - bfloat16 tensors are passed as uint16_t bit patterns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work on `stream`; none synchronises the host.
 *  - Return codes: BKV_OK, or a negative error.  Arguments are validated on
 *    the host BEFORE anything is enqueued; on an error nothing is launched
 *    and bkv_last_error() describes the problem.  No C++ exception crosses
 *    this ABI.  A launch or runtime failure returns BKV_EHIP (work enqueued
 *    earlier in the same call may already be running).
 *  - Inputs are const.  Outputs must not alias inputs, except where a call
 *    documents an in-place mode.
 *  - Layouts (row-major; U = n_units KV groups, g = group, Uq = U*g query
 *    heads, d = d_head):
 *        K, V      bf16  [U, l_cap, d]   post-RoPE keys / values per slot
 *        kpos      int32 [U, l_cap]      absolute position of each slot
 *        score     fp32  [U, l_cap]      pooled attention score per slot
 *        kept      int32 [U, b_kv]       kept slots, ascending
 *        buf       fp32  [Uq, buf_cap, d] pre-RoPE query buffer per head
 *        count     int32 [Uq]            rows in use in buf
 *        recents   fp32  [Uq, n_recent_q, d] pre-RoPE recent queries
 *        lse_in    fp32  [U, g, 32]      softmax denominators by observation
 *                                        row (natural-log log-sum-exp)
 *        q, out    fp32  [Uq, d]         decode-step query, attention output
 *        lse_q     fp32  [Uq]; lse_obs fp32 [Uq, 16]
 *    Unit u is (layer * batch + b) * h_kv + kv_head; query head j of unit u
 *    is u * g + j.
 */
#ifndef BKV_H
#define BKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BKV_ABI_VERSION 1

enum {
    BKV_OK = 0,
    BKV_EINVAL = -1,  /* bad pointer, shape or parameter */
    BKV_ENOTSUP = -2, /* valid but unsupported (d_head, group, buffer size) */
    BKV_ENOSPC = -3,  /* workspace too small */
    BKV_EHIP = -4     /* HIP launch/runtime error */
};

/* Shape of the cache being processed. */
typedef struct bkv_dims {
    int64_t n_units; /* U: KV groups (layers x batch x KV heads); 0 is a no-op */
    int32_t group;   /* g: query heads sharing one KV head, 1..8 */
    int32_t d_head;  /* d: 64 or 128 */
    int64_t l_cap;   /* slot stride of K, V, kpos and score (>= L) */
} bkv_dims;

/* Policy flags.  BKV_FLAG_MEAN: pool the attention weights by their mean
 * over the group's rows instead of their maximum (the mean-aggregation
 * ablation: paper text §5.3 and Table 2; the average form of the importance
 * score, paper text §2.2). */
#define BKV_FLAG_MEAN 1
/* BKV_FLAG_UNSORTED: bkv_evict compacts with bkv_compact_unsorted (kept
 * tokens past b_kv fill the evicted slots below it; the cache is no longer in
 * position order). */
#define BKV_FLAG_UNSORTED 2

/* Method parameters.  Paper text §5.1 ("Implementation Details"): beacon
 * budget max 32 / min 16, recent query budget 16; summary step (5): prefix
 * and recent tokens always kept. */
typedef struct bkv_policy {
    int32_t n_beacon;   /* beacon rows per query head used for scoring: 16, or 0
                         * with n_recent_q = 32 (no beacons: the window of the 32
                         * most recent queries the baselines observe, paper
                         * text §2.2 and §3.2) */
    int32_t n_recent_q; /* recent queries per query head: 16 (or 32, above) */
    int32_t buf_cap;    /* rows per head in buf (32; up to 8192 for a prefill over a
                         * long prompt; beyond 256 rows, m <= 64) */
    int32_t prefix;     /* P: leading slots always kept */
    int32_t recent_tok; /* R: trailing slots always kept */
    int32_t flags;      /* 0, or BKV_FLAG_MEAN | BKV_FLAG_UNSORTED */
    double rope_theta;  /* RoPE base theta (> 0) */
    float sm_scale;     /* softmax scale; 0 means 1/sqrt(d_head) */
    int32_t reserved;   /* must be 0 */
} bkv_policy;

/* ABI version the library was built with (BKV_ABI_VERSION). */
int bkv_abi_version(void);

/* Message for the last error returned on the calling thread ("" if none).
 * The pointer stays valid until the next bkv_* call on the same thread. */
const char* bkv_last_error(void);

/* Workspace bytes.  With b_kv == 0: what bkv_score needs (the RoPE angle
 * table).  With b_kv > 0: what bkv_evict needs for (L, b_kv), which also
 * covers the score and kept arrays when the caller passes none.
 * Returns 0 on invalid arguments (see bkv_last_error).  The workspace holds
 * nothing between calls; calls that share a workspace must not overlap. */
size_t bkv_workspace_bytes(const bkv_dims* dims, const bkv_policy* pol,
                           int64_t L, int64_t b_kv);

/*
 * bkv_fps_update -- Continual-FPS fill and compress of the per-head buffers.
 *
 * Paper text §4.2 ("Continual FPS") and App. D.1 (Algorithm 1, FPS);
 * summary steps (2), (3) and (6).  For every query head q in [0, Uq):
 *   1. append: rows new_q[q, 0..n_new) are copied to buf[q, count[q] + i];
 *      count[q] += n_new.  A head whose rows would not fit
 *      (count + n_new > buf_cap) is left completely unchanged and, if
 *      n_overflow is non-NULL, *n_overflow is atomically incremented.
 *   2. compress: if count[q] >= trigger, FPS under cosine similarity picks m
 *      rows (seed: lowest average cosine to the whole buffer; then
 *      repeatedly the row whose largest cosine to the picked set is lowest;
 *      ties to the lower slot).  The picked rows are stored in ascending
 *      original slot order in buf[q, 0..m) and count[q] = m.  If sel_order is
 *      non-NULL, sel_order[q, i] is the original slot of the i-th pick
 *      (heads that do not compress get -1 there).
 * Typical calls: trigger = buf_cap = 32, m = 16 (fill and compress);
 * trigger = m + 1 (beacon fix: compress only heads holding more than m);
 * n_new = 16 recents with trigger 32 after an eviction (merge);
 * trigger = buf_cap + 1 (append only, never compress: collecting the recent
 * queries, summary step (3), in a buffer of n_recent_q rows).
 * The cosine matrix of a buffer of up to 32 rows is formed on bf16 MFMA
 * from a high/low split of the fp32 rows (each cosine within about 2^-15 of
 * fp32); other arithmetic is fp32.  Requires
 * 0 <= n_new <= buf_cap, new_q NULL iff n_new == 0 (and 16-byte aligned),
 * 1 <= m < trigger <= buf_cap + 1, buf_cap <= 8192 (and m <= 64 when
 * buf_cap > 256 and heads can compress), every count in
 * [0, buf_cap] on entry.  buf and count are updated in place; new_q must not
 * overlap buf.
 */
int bkv_fps_update(const bkv_dims* dims, const bkv_policy* pol, float* buf,
                   int32_t* count, const float* new_q, int32_t n_new,
                   int32_t trigger, int32_t m, int32_t* sel_order,
                   int32_t* n_overflow, void* stream);

/*
 * bkv_fps_update_strided -- bkv_fps_update with the new rows at strides.
 *
 * The same operation (paper text §4.2, "Continual FPS"; summary steps (2),
 * (3) and (6)), with head q's new row i read at
 * new_q + q * q_head_stride + i * q_row_stride (floats) instead of
 * new_q + (q * n_new + i) * d_head; bkv_fps_update is this call with
 * q_head_stride = n_new * d_head and q_row_stride = d_head.  It lets a
 * decode loop append a block of steps' queries held step-major
 * ([n_new, Uq, d_head]: q_head_stride = d_head, q_row_stride =
 * Uq * d_head) without first copying them into head-major order.
 * Requires, besides what bkv_fps_update requires: new_q 16-byte aligned,
 * both strides multiples of 4, q_head_stride >= 0 and
 * q_row_stride >= d_head; every row read must lie in the caller's
 * allocation (the library cannot check it) and must not overlap buf.
 * Buffers of more than 256 rows take other strides only for appends of
 * at most 64 16-byte chunks per head (BKV_ENOTSUP otherwise).
 */
int bkv_fps_update_strided(const bkv_dims* dims, const bkv_policy* pol, float* buf,
                           int32_t* count, const float* new_q, int32_t n_new,
                           int64_t q_head_stride, int64_t q_row_stride,
                           int32_t trigger, int32_t m, int32_t* sel_order,
                           int32_t* n_overflow, void* stream);

/*
 * bkv_score -- observation-set attention score of every live slot.
 *
 * Paper text §4.3 ("Query Construction and Alignment", "Importance Scoring
 * via Max-Aggregation"); summary step (4); review §4.3.  Per unit u, query
 * head h of its group:
 *   - beacon rows: buf rows 0..n_beacon-1 of head h (stride buf_cap rows),
 *     rotated by RoPE to position t;
 *   - recent rows: recents[h, i] rotated to tau_i = kpos[u, L-n_recent_q+i];
 *   RoPE pairs coordinate k with k + d/2 at angle pos * theta^(-2k/d),
 *   computed in fp64 and rounded to fp32 and then to bf16 (both RNE).
 *   logits s = q . k * sm_scale against K[u, 0..L) (bf16 in, fp32 accumulate);
 *   recent row i sees slots 0..L-n_recent_q+i, beacon rows see all L slots;
 *   W = row softmax over the visible slots (hidden entries are 0);
 *   score[u, j] = max over the g*(n_beacon+n_recent_q) rows of W[row, j],
 *   or with BKV_FLAG_MEAN their average (sum over the rows / that count).
 * Writes score[u, 0..L); other slots are untouched.  If qobs_out is non-NULL
 * it receives the bf16 observation rows, [U, g*(n_beacon+n_recent_q), d],
 * row = h*(n_beacon+n_recent_q) + (beacons first, then recents).
 * beacons may be NULL when n_beacon == 0.
 * Requires n_recent_q <= L <= l_cap, t >= 0,
 * ws_bytes >= bkv_workspace_bytes(dims, pol, L, 0).
 */
int bkv_score(const bkv_dims* dims, const bkv_policy* pol, const uint16_t* K,
              const int32_t* kpos, int64_t L, const float* beacons,
              const float* recents, int64_t t, float* score,
              uint16_t* qobs_out, void* ws, size_t ws_bytes, void* stream);

/*
 * bkv_score_lse -- bkv_score with the softmax denominators already known.
 *
 * Summary "未来方向" (fold beacon scoring into the attention kernel, so the
 * eviction step loses its extra pass); paper text §4.3 for the scores.  The
 * same scores as bkv_score (max pooling, or the average with
 * BKV_FLAG_MEAN), where lse_in[u, h, r] (float32, [U, g, 32], row r as in
 * bkv_score: beacons first) gives the natural-log log-sum-exp of row r's
 * scaled logits:
 *   - beacon rows: over slots [0, lse_from) only; slots [lse_from, L) are
 *     added here (bkv_decode_attend's lse_obs at the step the cache held
 *     lse_from slots, the beacons then being fixed);
 *   - recent rows: complete (each recent query's own bkv_decode_attend
 *     lse_q: that step's cache is exactly the slots the row sees).
 * The kernel then reads the keys once more for the scores instead of twice.
 * A beacon value may be -inf (no slots before lse_from) only if
 * lse_from < L; all values must otherwise be finite.
 * Requires 0 <= lse_from <= L and what bkv_score requires; no qobs output.
 */
int bkv_score_lse(const bkv_dims* dims, const bkv_policy* pol, const uint16_t* K,
                  const int32_t* kpos, int64_t L, const float* beacons,
                  const float* recents, int64_t t, const float* lse_in,
                  int64_t lse_from, float* score, void* ws, size_t ws_bytes,
                  void* stream);

/*
 * bkv_decode_attend -- decode attention, with the beacons' denominators.
 *
 * Paper text §2.1 (scaled dot-product attention softmax(q k^T / sqrt(d)) V
 * of the step's query over the cache); summary "未来方向" (beacon scoring
 * folded into the attention kernel).  Per unit u and query head h of its
 * group (qh = u * g + h):
 *   qhat = q[qh] (pre-RoPE float32, [U*g, d]) rotated to t_q as bkv_score
 *   rotates (fp64, then fp32, then bf16, both RNE);
 *   s_j = qhat . K[u, j] * sm_scale for j in [0, L) (the step's own key is
 *   already in slot L - 1, so every slot is visible);
 *   out[qh] = sum_j softmax(s)_j V[u, j] (float32, [U*g, d]);
 *   lse_q[qh] = log sum_j exp(s_j) (float32, [U*g]).
 * With beacons non-NULL (rows 0..15 of each head, stride buf_cap rows, as
 * for bkv_score), each beacon rotated to t_obs (the coming eviction's step)
 * gets lse_obs[qh, b] = log sum_j exp(qhat_b . K[u, j] * sm_scale) over the
 * same L slots (float32, [U*g, 16]); lse_obs may be NULL otherwise.
 * Keys and values are read once for both.  Requires 1 <= L <= l_cap,
 * t_q >= 0, t_obs >= 0 with beacons, n_beacon = 16 with beacons.
 */
int bkv_decode_attend(const bkv_dims* dims, const bkv_policy* pol, const uint16_t* K,
                      const uint16_t* V, int64_t L, const float* q, int64_t t_q,
                      const float* beacons, int64_t t_obs, float* out, float* lse_q,
                      float* lse_obs, void* stream);

/*
 * bkv_select -- keep set of every unit.
 *
 * Summary step (5); paper text §2.2 (retain the top-scoring pairs) and
 * App. D.2.  kept[u] = slots [0, P) U [L-R, L) U the b_kv-P-R middle slots
 * with the highest score (ties: lower slot first), written ascending.
 * Scores are compared as fp32 values (non-negative, so by their bits).
 * Requires P + R <= b_kv < L <= l_cap.
 */
int bkv_select(const bkv_dims* dims, const bkv_policy* pol,
               const float* score, int64_t L, int64_t b_kv, int32_t* kept,
               void* stream);

/*
 * bkv_compact -- gather the kept slots to the front of the cache.
 *
 * Paper text §2.2 (index the sequence dimension with the kept set); summary
 * step (5) (written back in position order).  For k < b_kv:
 *   K'[u, k] = K[u, kept[u, k]], V'[u, k] = V[u, kept[u, k]],
 *   kpos'[u, k] = kpos[u, kept[u, k]].
 * With K_out, V_out and kpos_out all NULL the update is in place (slots at
 * and beyond b_kv are left as they were); otherwise all three must be
 * non-NULL with slot stride out_cap >= b_kv and must not overlap the inputs.
 * kept must be strictly ascending with values in [0, L) (as bkv_select
 * writes it); in place relies on that order.  An entry outside [0, L) is
 * skipped (its destination slot is left as it was) rather than followed.
 * Requires 0 < b_kv <= L <= l_cap.
 */
int bkv_compact(const bkv_dims* dims, uint16_t* K, uint16_t* V, int32_t* kpos,
                int64_t L, const int32_t* kept, int64_t b_kv, uint16_t* K_out,
                uint16_t* V_out, int32_t* kpos_out, int64_t out_cap,
                void* stream);

/*
 * bkv_select_compact -- bkv_select, then an in-place bkv_compact, in one
 * call.
 *
 * Summary step (5) (keep prefix, recent and Top-K; write back in position
 * order); paper text §2.2.  The same kept sets (written to kept, [U, b_kv],
 * ascending) and the same compacted K, V and kpos as the two calls, which
 * it makes on the same stream.  Requires what bkv_select requires.
 */
int bkv_select_compact(const bkv_dims* dims, const bkv_policy* pol, const float* score,
                       int64_t L, int64_t b_kv, uint16_t* K, uint16_t* V, int32_t* kpos,
                       int32_t* kept, void* stream);

/*
 * bkv_compact_unsorted -- fill the evicted slots instead of shifting.
 *
 * Unsorted variant of bkv_compact, in place.  The ThinKV pages note that
 * attention is invariant to the order of the cached tokens and reuse evicted
 * slots where they are.  Here every kept slot below b_kv keeps its token;
 * the kept tokens at slots >= b_kv move into the evicted slots below b_kv,
 * the i-th lowest such slot taking the i-th lowest such token (K, V and
 * kpos).  Afterwards slots [0, b_kv) hold the kept set, not in position
 * order, and at most L - b_kv tokens have moved.  kept must be the ascending
 * keep set bkv_select writes; the kernel bounds-checks every access, so a
 * malformed list moves nothing outside [0, L) (some slots may then be left
 * as they were).  Requires 0 < b_kv <= L <= l_cap.
 */
int bkv_compact_unsorted(const bkv_dims* dims, uint16_t* K, uint16_t* V, int32_t* kpos,
                         int64_t L, const int32_t* kept, int64_t b_kv, void* stream);

/*
 * bkv_evict -- one full eviction event (summary steps (4)-(6)).
 *
 * Runs bkv_score, then bkv_select_compact (or bkv_select and
 * bkv_compact_unsorted with BKV_FLAG_UNSORTED) on K, V, kpos; then,
 * if buf is non-NULL, the rolling update of summary step (6): the recent
 * queries are appended to each head's buffer (which must hold exactly the
 * n_beacon beacons, count == n_beacon) and the buffer is compressed back to
 * n_beacon rows with FPS.  `beacons` is normally `buf` itself.
 * With n_beacon == 0 there is no rolling update and buf must be NULL.
 * score_out / kept_out, if non-NULL, receive the scores and kept slots;
 * otherwise they live in the workspace.
 * Requires what the three calls require and
 * ws_bytes >= bkv_workspace_bytes(dims, pol, L, b_kv).
 */
int bkv_evict(const bkv_dims* dims, const bkv_policy* pol, uint16_t* K,
              uint16_t* V, int32_t* kpos, int64_t L, const float* beacons,
              const float* recents, int64_t t, int64_t b_kv, float* buf,
              int32_t* count, float* score_out, int32_t* kept_out, void* ws,
              size_t ws_bytes, void* stream);

/*
 * bkv_evict_noalloc -- bkv_evict without a workspace, allocating nothing.
 *
 * For callers that cannot allocate device memory or pass a workspace: code
 * under stream capture, tight serving loops, harnesses that forbid
 * allocation.  The same eviction event as bkv_evict (same kernels, same
 * results), with its scratch -- the RoPE angle table and, when score_out /
 * kept_out are NULL, the score and kept arrays -- in a fixed 16 MiB array
 * compiled into the library: one copy per GPU, held until the process ends.
 * A call whose scratch would exceed 16 MiB returns BKV_ENOSPC before
 * anything is enqueued (for U units, l_cap slots and b_kv kept, about
 * U * (l_cap + b_kv) * 4 bytes when neither output is passed; pass score_out
 * and kept_out for large caches).  Calls that overlap on one GPU (two
 * streams, or two host threads) share that scratch and race; serialise them.
 * The first call on a device looks up that device's copy (no allocation).
 * Requires what bkv_evict requires, except ws.
 */
int bkv_evict_noalloc(const bkv_dims* dims, const bkv_policy* pol, uint16_t* K,
                      uint16_t* V, int32_t* kpos, int64_t L, const float* beacons,
                      const float* recents, int64_t t, int64_t b_kv, float* buf,
                      int32_t* count, float* score_out, int32_t* kept_out,
                      void* stream);

/*
 * bkv_evict_lse -- bkv_evict with the softmax denominators already known.
 *
 * Summary "未来方向" (beacon scoring folded into attention); summary steps
 * (4)-(6).  The eviction event of bkv_evict, its scores formed as
 * bkv_score_lse forms them from lse_in ([U, g, 32] natural-log LSE; beacon
 * rows over slots [0, lse_from), recent rows complete) with one read of the
 * keys.  Requires what bkv_evict and bkv_score_lse require.
 */
int bkv_evict_lse(const bkv_dims* dims, const bkv_policy* pol, uint16_t* K,
                  uint16_t* V, int32_t* kpos, int64_t L, const float* beacons,
                  const float* recents, int64_t t, const float* lse_in,
                  int64_t lse_from, int64_t b_kv, float* buf, int32_t* count,
                  float* score_out, int32_t* kept_out, void* ws, size_t ws_bytes,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BKV_H */
