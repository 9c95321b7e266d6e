// Host side of the C ABI: argument validation, workspace layout, error
// reporting and the launch sequence of each entry point.  Nothing here
// allocates device memory; every call enqueues work on the caller's stream.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "common.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char msg[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, sizeof msg, fmt, ap);
    va_end(ap);
    g_err = msg;
    return code;
}

int ok() {
    g_err.clear();
    return BKV_OK;
}

// Test hook: BKV_FAULT_INJECT=<entry point name> or "all" makes that entry
// point report a HIP failure after validation, without launching anything.
bool fault_injected(const char* name) {
    const char* e = getenv("BKV_FAULT_INJECT");
    return e && (strcmp(e, "all") == 0 || strcmp(e, name) == 0);
}

int hip_result(hipError_t e, const char* name) {
    if (e != hipSuccess)
        return fail(BKV_EHIP, "%s: HIP error %d (%s)", name, (int)e, hipGetErrorString(e));
    return ok();
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// Checks shared by every call that takes dims and (optionally) a policy.
int check_dims(const char* fn, const bkv_dims* d) {
    if (!d) return fail(BKV_EINVAL, "%s: dims is NULL", fn);
    if (d->n_units < 0) return fail(BKV_EINVAL, "%s: n_units %lld < 0", fn, (long long)d->n_units);
    if (d->group < 1 || d->group > 8)
        return fail(d->group < 1 ? BKV_EINVAL : BKV_ENOTSUP,
                    "%s: group %d not in [1, 8]", fn, d->group);
    if (d->d_head != 64 && d->d_head != 128)
        return fail(d->d_head <= 0 ? BKV_EINVAL : BKV_ENOTSUP,
                    "%s: d_head %d not supported (64 or 128)", fn, d->d_head);
    if (d->l_cap < 1) return fail(BKV_EINVAL, "%s: l_cap %lld < 1", fn, (long long)d->l_cap);
    int64_t cells, elems;
    if (!mul_ok(d->n_units, d->l_cap, &cells) || !mul_ok(cells, d->d_head, &elems) ||
        elems > INT64_MAX / 4)
        return fail(BKV_EINVAL, "%s: n_units * l_cap * d_head overflows", fn);
    return BKV_OK;
}

int check_policy(const char* fn, const bkv_policy* p) {
    if (!p) return fail(BKV_EINVAL, "%s: policy is NULL", fn);
    if ((p->flags & ~(BKV_FLAG_MEAN | BKV_FLAG_UNSORTED)) != 0 || p->reserved != 0)
        return fail(BKV_EINVAL, "%s: unknown policy flags or reserved field not 0", fn);
    // The observation set is 32 rows per query head: 16 beacons + 16 recent
    // queries (the method), or 32 recent queries (the baselines' window).
    if (!((p->n_beacon == 16 && p->n_recent_q == 16) || (p->n_beacon == 0 && p->n_recent_q == 32)))
        return fail(BKV_ENOTSUP,
                    "%s: n_beacon %d / n_recent_q %d: only 16 / 16 or 0 / 32 supported", fn,
                    p->n_beacon, p->n_recent_q);
    if (p->buf_cap < 1) return fail(BKV_EINVAL, "%s: buf_cap %d < 1", fn, p->buf_cap);
    if (p->buf_cap > 8192) return fail(BKV_ENOTSUP, "%s: buf_cap %d > 8192", fn, p->buf_cap);
    if (p->prefix < 0 || p->recent_tok < 0)
        return fail(BKV_EINVAL, "%s: prefix %d / recent_tok %d must be >= 0", fn, p->prefix,
                    p->recent_tok);
    if (!(p->rope_theta > 0.0) || !isfinite(p->rope_theta))
        return fail(BKV_EINVAL, "%s: rope_theta must be finite and > 0", fn);
    if (!(p->sm_scale >= 0.f) || !isfinite(p->sm_scale) || p->sm_scale > 1e4f)
        return fail(BKV_EINVAL, "%s: sm_scale must be in [0, 1e4]", fn);
    return BKV_OK;
}

float scale_of(const bkv_dims* d, const bkv_policy* p) {
    return p->sm_scale > 0.f ? p->sm_scale : (float)(1.0 / sqrt((double)d->d_head));
}

struct WsLayout {
    size_t table = 0, score = 0, kept = 0, total = 0;
};

// Workspace: RoPE angle table, then (bkv_evict) the score and kept arrays.
WsLayout ws_layout(const bkv_dims* d, const bkv_policy* p, int64_t b_kv) {
    WsLayout w;
    w.table = 0;
    size_t off = align_up(bkv::rope_table_bytes(p->n_recent_q, d->d_head));
    if (b_kv > 0) {
        w.score = off;
        off = align_up(off + (size_t)d->n_units * (size_t)d->l_cap * sizeof(float));
        w.kept = off;
        off = align_up(off + (size_t)d->n_units * (size_t)b_kv * sizeof(int32_t));
    }
    w.total = off;
    return w;
}

int check_score_args(const char* fn, const bkv_dims* d, const bkv_policy* p, const void* K,
                     const void* kpos, int64_t L, const void* beacons, const void* recents,
                     int64_t t) {
    if (!K || !kpos || !recents || (!beacons && p->n_beacon > 0))
        return fail(BKV_EINVAL, "%s: NULL tensor pointer", fn);
    if (L < p->n_recent_q || L > d->l_cap)
        return fail(BKV_EINVAL, "%s: L %lld not in [n_recent_q=%d, l_cap=%lld]", fn,
                    (long long)L, p->n_recent_q, (long long)d->l_cap);
    if (p->buf_cap < p->n_beacon)
        return fail(BKV_EINVAL, "%s: buf_cap %d < n_beacon %d", fn, p->buf_cap, p->n_beacon);
    if (t < 0) return fail(BKV_EINVAL, "%s: t %lld < 0", fn, (long long)t);
    // The scoring kernel addresses one unit's keys with 32-bit byte offsets.
    if (L * d->d_head * 2 > INT32_MAX)
        return fail(BKV_ENOTSUP, "%s: L %lld keys of d_head %d exceed 2^31 bytes per unit", fn,
                    (long long)L, d->d_head);
    return BKV_OK;
}

int check_select_args(const char* fn, const bkv_dims* d, const bkv_policy* p, int64_t L,
                      int64_t b_kv) {
    if (L < 1 || L > d->l_cap)
        return fail(BKV_EINVAL, "%s: L %lld not in [1, l_cap=%lld]", fn, (long long)L,
                    (long long)d->l_cap);
    if (!((int64_t)p->prefix + p->recent_tok <= b_kv && b_kv < L))
        return fail(BKV_EINVAL, "%s: need prefix + recent_tok (%d) <= b_kv (%lld) < L (%lld)", fn,
                    p->prefix + p->recent_tok, (long long)b_kv, (long long)L);
    if (L > INT32_MAX) return fail(BKV_ENOTSUP, "%s: L beyond int32 slots", fn);
    return BKV_OK;
}

#define CHECK(x)                     \
    do {                             \
        int rc_ = (x);               \
        if (rc_ != BKV_OK) return rc_; \
    } while (0)

// Scratch memory of bkv_evict_noalloc, for callers that cannot allocate:
// a fixed array in the library's device code, one copy on every GPU the
// library runs on, held until the process ends.  It holds the RoPE angle
// table and, when the caller passes no score or kept output, those arrays.
// Nothing in it needs to start at zero: each call writes every byte it
// reads.  Calls on one GPU share it, so calls that overlap on one GPU race.
constexpr size_t kScratchBytes = 16u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of each GPU's copy of `scratch` (host code never passes the
// array's own name, which on the host is only a stand-in): looked up once per
// device, on the first bkv_evict_noalloc call with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_of_current_device(const char* fn, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_result(e, fn);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(BKV_ENOTSUP, "%s: device %d beyond the %d the library tracks", fn, dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(BKV_EHIP, "%s: scratch address on device %d: HIP error %d (%s)", fn, dev,
                        (int)e, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return BKV_OK;
}

}  // namespace

extern "C" {

int bkv_abi_version(void) { return BKV_ABI_VERSION; }

const char* bkv_last_error(void) { return g_err.c_str(); }

size_t bkv_workspace_bytes(const bkv_dims* dims, const bkv_policy* pol, int64_t L,
                           int64_t b_kv) {
    const char* fn = "bkv_workspace_bytes";
    if (check_dims(fn, dims) != BKV_OK || check_policy(fn, pol) != BKV_OK) return 0;
    if (b_kv < 0 || L < 0 || L > dims->l_cap || (b_kv > 0 && b_kv >= L)) {
        fail(BKV_EINVAL, "%s: need 0 <= b_kv < L <= l_cap", fn);
        return 0;
    }
    ok();
    return ws_layout(dims, pol, b_kv).total;
}

static int fps_update_impl(const char* fn, const bkv_dims* dims, const bkv_policy* pol,
                           float* buf, int32_t* count, const float* new_q, int32_t n_new,
                           int64_t q_head_stride, int64_t q_row_stride, int32_t trigger,
                           int32_t m, int32_t* sel_order, int32_t* n_overflow, void* stream) {
    CHECK(check_dims(fn, dims));
    CHECK(check_policy(fn, pol));
    if (!buf || !count) return fail(BKV_EINVAL, "%s: NULL buf or count", fn);
    if (n_new < 0 || n_new > pol->buf_cap)
        return fail(BKV_EINVAL, "%s: n_new %d not in [0, buf_cap=%d]", fn, n_new, pol->buf_cap);
    if ((new_q == nullptr) != (n_new == 0))
        return fail(BKV_EINVAL, "%s: new_q must be NULL exactly when n_new == 0", fn);
    if (new_q && (q_head_stride < 0 || q_row_stride < dims->d_head || q_head_stride % 4 != 0 ||
                  q_row_stride % 4 != 0 || (reinterpret_cast<uintptr_t>(new_q) & 15) != 0))
        return fail(BKV_EINVAL,
                    "%s: new_q strides (head %lld, row %lld floats) must be multiples of 4, the row "
                    "stride at least d_head = %d, and new_q 16-byte aligned",
                    fn, (long long)q_head_stride, (long long)q_row_stride, dims->d_head);
    if (!(1 <= m && m < trigger && trigger <= pol->buf_cap + 1))
        return fail(BKV_EINVAL, "%s: need 1 <= m (%d) < trigger (%d) <= buf_cap + 1 (%d)", fn, m,
                    trigger, pol->buf_cap + 1);
    if (pol->buf_cap > 256 && m > 64 && trigger <= pol->buf_cap)
        return fail(BKV_ENOTSUP, "%s: buffers of more than 256 rows keep at most 64 (m = %d)", fn,
                    m);
    const int64_t nch = (int64_t)n_new * dims->d_head / 4;
    const bool append_kernel = trigger > pol->buf_cap && n_new > 0 && nch <= 64;
    if (pol->buf_cap > 256 && new_q && !append_kernel &&
        (q_row_stride != dims->d_head || q_head_stride != (int64_t)n_new * dims->d_head))
        return fail(BKV_ENOTSUP, "%s: buffers of more than 256 rows take head-major contiguous "
                    "new rows", fn);
    if (dims->n_units == 0) return ok();
    if (fault_injected(fn)) return fail(BKV_EHIP, "%s: injected HIP failure", fn);
    const int64_t n_heads = dims->n_units * dims->group;
    return hip_result(bkv::launch_fps(buf, count, new_q, n_new, q_head_stride, q_row_stride,
                                      n_heads, dims->d_head, pol->buf_cap, trigger, m, sel_order,
                                      n_overflow, (hipStream_t)stream),
                      fn);
}

int bkv_fps_update(const bkv_dims* dims, const bkv_policy* pol, float* buf, int32_t* count,
                   const float* new_q, int32_t n_new, int32_t trigger, int32_t m,
                   int32_t* sel_order, int32_t* n_overflow, void* stream) {
    const int64_t d = dims ? dims->d_head : 0;
    return fps_update_impl("bkv_fps_update", dims, pol, buf, count, new_q, n_new,
                           (int64_t)n_new * d, d, trigger, m, sel_order, n_overflow, stream);
}

int bkv_fps_update_strided(const bkv_dims* dims, const bkv_policy* pol, float* buf,
                           int32_t* count, const float* new_q, int32_t n_new,
                           int64_t q_head_stride, int64_t q_row_stride, int32_t trigger, int32_t m,
                           int32_t* sel_order, int32_t* n_overflow, void* stream) {
    return fps_update_impl("bkv_fps_update_strided", dims, pol, buf, count, new_q, n_new,
                           q_head_stride, q_row_stride, trigger, m, sel_order, n_overflow, stream);
}

static int score_impl(const char* fn, const bkv_dims* dims, const bkv_policy* pol,
                      const uint16_t* K, const int32_t* kpos, int64_t L, const float* beacons,
                      const float* recents, int64_t t, const float* lse_in, int64_t lse_from,
                      float* score, uint16_t* qobs_out, void* ws, size_t ws_bytes, void* stream) {
    CHECK(check_dims(fn, dims));
    CHECK(check_policy(fn, pol));
    CHECK(check_score_args(fn, dims, pol, K, kpos, L, beacons, recents, t));
    if (!score) return fail(BKV_EINVAL, "%s: NULL score", fn);
    const WsLayout w = ws_layout(dims, pol, 0);
    if (!ws || ws_bytes < w.total)
        return fail(BKV_ENOSPC, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, w.total);
    if (dims->n_units == 0) return ok();
    if (fault_injected(fn)) return fail(BKV_EHIP, "%s: injected HIP failure", fn);
    hipStream_t s = (hipStream_t)stream;
    double* table = (double*)((char*)ws + w.table);
    hipError_t e = bkv::launch_rope_table(table, t, pol->n_recent_q, dims->d_head,
                                          pol->rope_theta, s);
    if (e == hipSuccess)
        e = bkv::launch_score(K, kpos, dims->n_units, dims->group, dims->d_head, dims->l_cap,
                              L, beacons, pol->buf_cap, recents, pol->n_beacon,
                              pol->n_recent_q, t, pol->rope_theta, scale_of(dims, pol),
                              (pol->flags & BKV_FLAG_MEAN) != 0, table, score, qobs_out,
                              lse_in, lse_from, s);
    return hip_result(e, fn);
}

int bkv_score(const bkv_dims* dims, const bkv_policy* pol, const uint16_t* K,
              const int32_t* kpos, int64_t L, const float* beacons, const float* recents,
              int64_t t, float* score, uint16_t* qobs_out, void* ws, size_t ws_bytes,
              void* stream) {
    return score_impl("bkv_score", dims, pol, K, kpos, L, beacons, recents, t, nullptr, 0,
                      score, qobs_out, ws, ws_bytes, stream);
}

int bkv_score_lse(const bkv_dims* dims, const bkv_policy* pol, const uint16_t* K,
                  const int32_t* kpos, int64_t L, const float* beacons, const float* recents,
                  int64_t t, const float* lse_in, int64_t lse_from, float* score,
                  void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "bkv_score_lse";
    if (!lse_in) return fail(BKV_EINVAL, "%s: NULL lse_in", fn);
    if (!(0 <= lse_from && lse_from <= L))
        return fail(BKV_EINVAL, "%s: need 0 <= lse_from (%lld) <= L (%lld)", fn,
                    (long long)lse_from, (long long)L);
    return score_impl(fn, dims, pol, K, kpos, L, beacons, recents, t, lse_in, lse_from, score,
                      nullptr, ws, ws_bytes, stream);
}

int bkv_decode_attend(const bkv_dims* dims, const bkv_policy* pol, const uint16_t* K,
                      const uint16_t* V, int64_t L, const float* q, int64_t t_q,
                      const float* beacons, int64_t t_obs, float* out, float* lse_q,
                      float* lse_obs, void* stream) {
    const char* fn = "bkv_decode_attend";
    CHECK(check_dims(fn, dims));
    CHECK(check_policy(fn, pol));
    if (!K || !V || !q || !out || !lse_q) return fail(BKV_EINVAL, "%s: NULL tensor pointer", fn);
    if (beacons && !lse_obs) return fail(BKV_EINVAL, "%s: beacons given without lse_obs", fn);
    if (beacons && (pol->n_beacon != 16 || pol->buf_cap < 16))
        return fail(BKV_EINVAL, "%s: beacons need n_beacon 16 and buf_cap >= 16", fn);
    if (L < 1 || L > dims->l_cap)
        return fail(BKV_EINVAL, "%s: L %lld not in [1, l_cap=%lld]", fn, (long long)L,
                    (long long)dims->l_cap);
    if (t_q < 0 || (beacons && t_obs < 0))
        return fail(BKV_EINVAL, "%s: negative position", fn);
    if (L * dims->d_head * 2 > INT32_MAX)
        return fail(BKV_ENOTSUP, "%s: L %lld keys of d_head %d exceed 2^31 bytes per unit", fn,
                    (long long)L, dims->d_head);
    if (dims->n_units == 0) return ok();
    if (fault_injected(fn)) return fail(BKV_EHIP, "%s: injected HIP failure", fn);
    return hip_result(bkv::launch_decode(K, V, dims->n_units, dims->group, dims->d_head,
                                         dims->l_cap, L, q, t_q, beacons, pol->buf_cap, t_obs,
                                         pol->rope_theta, scale_of(dims, pol), out, lse_q,
                                         beacons ? lse_obs : nullptr, (hipStream_t)stream),
                      fn);
}

int bkv_select(const bkv_dims* dims, const bkv_policy* pol, const float* score, int64_t L,
               int64_t b_kv, int32_t* kept, void* stream) {
    const char* fn = "bkv_select";
    CHECK(check_dims(fn, dims));
    CHECK(check_policy(fn, pol));
    CHECK(check_select_args(fn, dims, pol, L, b_kv));
    if (!score || !kept) return fail(BKV_EINVAL, "%s: NULL score or kept", fn);
    if (dims->n_units == 0) return ok();
    if (fault_injected(fn)) return fail(BKV_EHIP, "%s: injected HIP failure", fn);
    return hip_result(bkv::launch_select(score, dims->n_units, dims->l_cap, L, b_kv,
                                         pol->prefix, pol->recent_tok, kept,
                                         (hipStream_t)stream),
                      fn);
}

int bkv_select_compact(const bkv_dims* dims, const bkv_policy* pol, const float* score,
                       int64_t L, int64_t b_kv, uint16_t* K, uint16_t* V, int32_t* kpos,
                       int32_t* kept, void* stream) {
    const char* fn = "bkv_select_compact";
    CHECK(check_dims(fn, dims));
    CHECK(check_policy(fn, pol));
    CHECK(check_select_args(fn, dims, pol, L, b_kv));
    if (!score || !kept || !K || !V || !kpos)
        return fail(BKV_EINVAL, "%s: NULL tensor pointer", fn);
    if (dims->n_units == 0) return ok();
    if (fault_injected(fn)) return fail(BKV_EHIP, "%s: injected HIP failure", fn);
    hipStream_t s = (hipStream_t)stream;
    return hip_result(bkv::launch_select_compact(K, V, kpos, dims->n_units, dims->d_head,
                                                 dims->l_cap, L, score, kept, b_kv, pol->prefix,
                                                 pol->recent_tok, s),
                      fn);
}

int bkv_compact_unsorted(const bkv_dims* dims, uint16_t* K, uint16_t* V, int32_t* kpos,
                         int64_t L, const int32_t* kept, int64_t b_kv, void* stream) {
    const char* fn = "bkv_compact_unsorted";
    CHECK(check_dims(fn, dims));
    if (!K || !V || !kpos || !kept) return fail(BKV_EINVAL, "%s: NULL tensor pointer", fn);
    if (!(0 < b_kv && b_kv <= L && L <= dims->l_cap))
        return fail(BKV_EINVAL, "%s: need 0 < b_kv (%lld) <= L (%lld) <= l_cap (%lld)", fn,
                    (long long)b_kv, (long long)L, (long long)dims->l_cap);
    if (L > INT32_MAX) return fail(BKV_ENOTSUP, "%s: L beyond int32 slots", fn);
    if (dims->n_units == 0) return ok();
    if (fault_injected(fn)) return fail(BKV_EHIP, "%s: injected HIP failure", fn);
    return hip_result(bkv::launch_compact_fill(K, V, kpos, dims->n_units, dims->d_head,
                                               dims->l_cap, L, kept, b_kv, (hipStream_t)stream),
                      fn);
}

int bkv_compact(const bkv_dims* dims, uint16_t* K, uint16_t* V, int32_t* kpos, int64_t L,
                const int32_t* kept, int64_t b_kv, uint16_t* K_out, uint16_t* V_out,
                int32_t* kpos_out, int64_t out_cap, void* stream) {
    const char* fn = "bkv_compact";
    CHECK(check_dims(fn, dims));
    if (!K || !V || !kpos || !kept) return fail(BKV_EINVAL, "%s: NULL tensor pointer", fn);
    if (!(0 < b_kv && b_kv <= L && L <= dims->l_cap))
        return fail(BKV_EINVAL, "%s: need 0 < b_kv (%lld) <= L (%lld) <= l_cap (%lld)", fn,
                    (long long)b_kv, (long long)L, (long long)dims->l_cap);
    const int n_out = (K_out != nullptr) + (V_out != nullptr) + (kpos_out != nullptr);
    if (n_out != 0 && n_out != 3)
        return fail(BKV_EINVAL, "%s: K_out, V_out, kpos_out must be all NULL or all set", fn);
    if (n_out == 3) {
        int64_t cells, elems;
        if (out_cap < b_kv || !mul_ok(dims->n_units, out_cap, &cells) ||
            !mul_ok(cells, dims->d_head, &elems))
            return fail(BKV_EINVAL, "%s: out_cap %lld < b_kv %lld", fn, (long long)out_cap,
                        (long long)b_kv);
        if (K_out == K || V_out == V || kpos_out == kpos)
            return fail(BKV_EINVAL, "%s: outputs alias inputs; pass NULL for in place", fn);
    }
    if (dims->n_units == 0) return ok();
    if (fault_injected(fn)) return fail(BKV_EHIP, "%s: injected HIP failure", fn);
    return hip_result(bkv::launch_compact(K, V, kpos, dims->n_units, dims->d_head, dims->l_cap,
                                          L, kept, b_kv, K_out, V_out, kpos_out,
                                          n_out ? out_cap : dims->l_cap, (hipStream_t)stream),
                      fn);
}

// Argument checks of bkv_evict and its variants (everything but the
// workspace).
static int evict_checks(const char* fn, const bkv_dims* dims, const bkv_policy* pol,
                        const uint16_t* K, const uint16_t* V, const int32_t* kpos, int64_t L,
                        const float* beacons, const float* recents, int64_t t, int64_t b_kv,
                        const float* buf, const int32_t* count) {
    CHECK(check_dims(fn, dims));
    CHECK(check_policy(fn, pol));
    CHECK(check_score_args(fn, dims, pol, K, kpos, L, beacons, recents, t));
    CHECK(check_select_args(fn, dims, pol, L, b_kv));
    if (!V) return fail(BKV_EINVAL, "%s: NULL V", fn);
    if ((buf == nullptr) != (count == nullptr))
        return fail(BKV_EINVAL, "%s: buf and count must both be set or both NULL", fn);
    if (buf && pol->n_beacon == 0)
        return fail(BKV_EINVAL, "%s: no beacons (n_beacon 0): pass buf = NULL", fn);
    if (buf && pol->buf_cap < pol->n_beacon + pol->n_recent_q)
        return fail(BKV_EINVAL, "%s: buf_cap %d cannot hold beacons + recents", fn,
                    pol->buf_cap);
    return BKV_OK;
}

// The launch sequence of one eviction event: RoPE table, scores, selection
// and compaction, then the merge.  table, score and kept are device memory.
static hipError_t evict_launch(const bkv_dims* dims, const bkv_policy* pol, uint16_t* K,
                               uint16_t* V, int32_t* kpos, int64_t L, const float* beacons,
                               const float* recents, int64_t t, const float* lse_in,
                               int64_t lse_from, int64_t b_kv, float* buf, int32_t* count,
                               double* table, float* score, int32_t* kept, hipStream_t s) {
    hipError_t e = bkv::launch_rope_table(table, t, pol->n_recent_q, dims->d_head,
                                          pol->rope_theta, s);
    if (e == hipSuccess)
        e = bkv::launch_score(K, kpos, dims->n_units, dims->group, dims->d_head, dims->l_cap,
                              L, beacons, pol->buf_cap, recents, pol->n_beacon,
                              pol->n_recent_q, t, pol->rope_theta, scale_of(dims, pol),
                              (pol->flags & BKV_FLAG_MEAN) != 0, table, score, nullptr,
                              lse_in, lse_from, s);
    const bool sorted = (pol->flags & BKV_FLAG_UNSORTED) == 0;
    if (e == hipSuccess)
        e = bkv::launch_select(score, dims->n_units, dims->l_cap, L, b_kv, pol->prefix,
                               pol->recent_tok, kept, s);
    if (e == hipSuccess && !sorted)
        e = bkv::launch_compact_fill(K, V, kpos, dims->n_units, dims->d_head, dims->l_cap, L,
                                     kept, b_kv, s);
    else if (e == hipSuccess)
        e = bkv::launch_compact(K, V, kpos, dims->n_units, dims->d_head, dims->l_cap, L, kept,
                                b_kv, nullptr, nullptr, nullptr, dims->l_cap, s);
    if (e == hipSuccess && buf)
        e = bkv::launch_fps(buf, count, recents, pol->n_recent_q,
                            (int64_t)pol->n_recent_q * dims->d_head, dims->d_head,
                            dims->n_units * dims->group, dims->d_head, pol->buf_cap,
                            pol->n_beacon + pol->n_recent_q, pol->n_beacon, nullptr, nullptr, s);
    return e;
}

static int evict_impl(const char* fn, const bkv_dims* dims, const bkv_policy* pol, uint16_t* K,
                      uint16_t* V, int32_t* kpos, int64_t L, const float* beacons,
                      const float* recents, int64_t t, const float* lse_in, int64_t lse_from,
                      int64_t b_kv, float* buf, int32_t* count, float* score_out,
                      int32_t* kept_out, void* ws, size_t ws_bytes, void* stream) {
    CHECK(evict_checks(fn, dims, pol, K, V, kpos, L, beacons, recents, t, b_kv, buf, count));
    const WsLayout w = ws_layout(dims, pol, b_kv);
    if (!ws || ws_bytes < w.total)
        return fail(BKV_ENOSPC, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, w.total);
    if (dims->n_units == 0) return ok();
    if (fault_injected(fn)) return fail(BKV_EHIP, "%s: injected HIP failure", fn);
    double* table = (double*)((char*)ws + w.table);
    float* score = score_out ? score_out : (float*)((char*)ws + w.score);
    int32_t* kept = kept_out ? kept_out : (int32_t*)((char*)ws + w.kept);
    return hip_result(evict_launch(dims, pol, K, V, kpos, L, beacons, recents, t, lse_in,
                                   lse_from, b_kv, buf, count, table, score, kept,
                                   (hipStream_t)stream),
                      fn);
}

int bkv_evict(const bkv_dims* dims, const bkv_policy* pol, uint16_t* K, uint16_t* V,
              int32_t* kpos, int64_t L, const float* beacons, const float* recents, int64_t t,
              int64_t b_kv, float* buf, int32_t* count, float* score_out, int32_t* kept_out,
              void* ws, size_t ws_bytes, void* stream) {
    return evict_impl("bkv_evict", dims, pol, K, V, kpos, L, beacons, recents, t, nullptr, 0,
                      b_kv, buf, count, score_out, kept_out, ws, ws_bytes, stream);
}

int bkv_evict_noalloc(const bkv_dims* dims, const bkv_policy* pol, uint16_t* K, uint16_t* V,
                      int32_t* kpos, int64_t L, const float* beacons, const float* recents,
                      int64_t t, int64_t b_kv, float* buf, int32_t* count, float* score_out,
                      int32_t* kept_out, void* stream) {
    const char* fn = "bkv_evict_noalloc";
    CHECK(evict_checks(fn, dims, pol, K, V, kpos, L, beacons, recents, t, b_kv, buf, count));
    // Scratch layout: the table, then score and kept where the caller passes
    // no output for them.  Checked before any HIP call.
    size_t off = align_up(bkv::rope_table_bytes(pol->n_recent_q, dims->d_head));
    size_t score_off = 0, kept_off = 0;
    if (!score_out) {
        score_off = off;
        off = align_up(off + (size_t)dims->n_units * (size_t)dims->l_cap * sizeof(float));
    }
    if (!kept_out) {
        kept_off = off;
        off = align_up(off + (size_t)dims->n_units * (size_t)b_kv * sizeof(int32_t));
    }
    if (off > kScratchBytes)
        return fail(BKV_ENOSPC,
                    "%s: needs %zu bytes of scratch, the library's fixed scratch holds %zu; "
                    "pass score_out and kept_out, or use bkv_evict with a workspace",
                    fn, off, kScratchBytes);
    if (dims->n_units == 0) return ok();
    if (fault_injected(fn)) return fail(BKV_EHIP, "%s: injected HIP failure", fn);
    void* base = nullptr;
    CHECK(scratch_of_current_device(fn, &base));
    char* ws = (char*)base;
    float* score = score_out ? score_out : (float*)(ws + score_off);
    int32_t* kept = kept_out ? kept_out : (int32_t*)(ws + kept_off);
    return hip_result(evict_launch(dims, pol, K, V, kpos, L, beacons, recents, t, nullptr, 0,
                                   b_kv, buf, count, (double*)ws, score, kept,
                                   (hipStream_t)stream),
                      fn);
}

int bkv_evict_lse(const bkv_dims* dims, const bkv_policy* pol, uint16_t* K, uint16_t* V,
                  int32_t* kpos, int64_t L, const float* beacons, const float* recents,
                  int64_t t, const float* lse_in, int64_t lse_from, int64_t b_kv, float* buf,
                  int32_t* count, float* score_out, int32_t* kept_out, void* ws,
                  size_t ws_bytes, void* stream) {
    const char* fn = "bkv_evict_lse";
    if (!lse_in) return fail(BKV_EINVAL, "%s: NULL lse_in", fn);
    if (!(0 <= lse_from && lse_from <= L))
        return fail(BKV_EINVAL, "%s: need 0 <= lse_from (%lld) <= L (%lld)", fn,
                    (long long)lse_from, (long long)L);
    return evict_impl(fn, dims, pol, K, V, kpos, L, beacons, recents, t, lse_in, lse_from, b_kv,
                      buf, count, score_out, kept_out, ws, ws_bytes, stream);
}

}  // extern "C"
