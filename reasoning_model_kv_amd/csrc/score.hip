// Observation-set scoring: RoPE alignment, Q_obs . K^T on bf16 MFMA,
// row softmax and the max over the GQA group.
//
// Paper text §4.3: beacons rotated to the current step t, recent queries to
// their own positions tau; attention weights W (|Q_obs| x L) against the
// current cache, max-pooled over all queries and heads of the KV group
// (summary step (4); review §4.3: Score[j] = max_{h in g} max_q W[h,q,j]).
//
// Mapping (one workgroup per KV group, one wavefront per query head):
//  * A wavefront owns its head's 32 observation rows (16 beacons, 16
//    recents).  It rotates them in fp64 straight into the A operand of
//    v_mfma_f32_32x32x16_bf16: lane (row i = lane % 32, half h = lane / 32)
//    holds dims 16 s + 8 h + e for MFMA step s, element e; the RoPE partner
//    of dim k < d/2 (dim k + d/2) sits in the same lane at step s + d/32.
//  * Keys stream through LDS in tiles of 64 (double-buffered, loaded with
//    global_load_lds_dwordx4, 16-byte chunks XOR-swizzled by row so the
//    32 lanes that read one chunk column hit distinct banks).  All g
//    wavefronts of the group read the same tile.
//  * Pass 1: per 64-key tile each wavefront forms a 32 x 64 logit block and
//    keeps a per-lane running (max, sum of exp2) for its 16 rows; the 32
//    lanes of a half are merged once at the end into each row's LSE.
//  * Pass 2: the logits are formed again, shifted by the row LSE, reduced
//    over the lane's 16 rows, the other half (permlane32 swap) and the g
//    wavefronts (LDS), and written as score = exp2(max).
//  Output layout of the 32x32 MFMA: lane l, accumulator v holds
//  row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.

#include "common.h"

namespace bkv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int KT = 64;               // keys per tile
constexpr float kNegBig = -1.0e30f;  // finite "no key seen yet" running max
constexpr float kRescaleLog2 = 64.f; // lazy rescale threshold (log2 units)

__device__ __forceinline__ void rope_cs(double pos, int i, int d, double theta,
                                        double* c, double* s) {
    const double w = pow(theta, (-2.0 * (double)i) / (double)d);
    sincos(pos * w, s, c);
}

__global__ void rope_table_kernel(double* table, int64_t t, int n_recent_q,
                                  int d, double theta) {
    const int half = d / 2;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (1 + n_recent_q) * half) return;
    const int p = idx / half, i = idx % half;
    const int64_t pos = p == 0 ? t : t - n_recent_q + (p - 1);
    double c, s;
    rope_cs((double)pos, i, d, theta, &c, &s);
    table[2 * idx] = c;
    table[2 * idx + 1] = s;
}

struct ScoreArgs {
    const uint16_t* K;
    const int32_t* kpos;
    int64_t l_cap;
    int64_t L;
    const float* beacons;
    const float* recents;
    int buf_cap;
    int n_recent_q;
    int64_t t;
    double theta;
    float c2;  // sm_scale * log2(e)
    const double* table;
    float* score;
    uint16_t* qobs;
};

__device__ __forceinline__ int acc_row(int v, int lane) {
    return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// Build this lane's A fragments (bf16) for MFMA steps 0..D/16-1.
template <int D>
__device__ __forceinline__ void build_queries(const ScoreArgs& a, int64_t u, int g,
                                              int h, int lane, bf16x8 (&frag)[D / 16]) {
#pragma clang fp contract(off)
    constexpr int NS = D / 16;
    const int i = lane & 31;
    const int hh = lane >> 5;
    const int64_t qh = u * g + h;
    const float* src;
    int64_t pos;
    const double* tab = nullptr;
    if (i < 16) {
        src = a.beacons + (qh * a.buf_cap + i) * (int64_t)D;
        pos = a.t;
        tab = a.table;
    } else {
        const int r = i - 16;
        src = a.recents + (qh * a.n_recent_q + r) * (int64_t)D;
        pos = a.kpos[u * a.l_cap + a.L - a.n_recent_q + r];
        if (pos == a.t - a.n_recent_q + r) tab = a.table + (int64_t)(1 + r) * D;
    }
    uint16_t out[NS][8];
#pragma unroll
    for (int s = 0; s < NS / 2; ++s) {
        const int d0 = 16 * s + 8 * hh;
        float x1[8], x2[8];
        const float4 p0 = *reinterpret_cast<const float4*>(src + d0);
        const float4 p1 = *reinterpret_cast<const float4*>(src + d0 + 4);
        const float4 q0 = *reinterpret_cast<const float4*>(src + d0 + D / 2);
        const float4 q1 = *reinterpret_cast<const float4*>(src + d0 + D / 2 + 4);
        x1[0] = p0.x; x1[1] = p0.y; x1[2] = p0.z; x1[3] = p0.w;
        x1[4] = p1.x; x1[5] = p1.y; x1[6] = p1.z; x1[7] = p1.w;
        x2[0] = q0.x; x2[1] = q0.y; x2[2] = q0.z; x2[3] = q0.w;
        x2[4] = q1.x; x2[5] = q1.y; x2[6] = q1.z; x2[7] = q1.w;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = d0 + e;
            double c, sn;
            if (tab) {
                c = tab[2 * k];
                sn = tab[2 * k + 1];
            } else {
                rope_cs((double)pos, k, D, a.theta, &c, &sn);
            }
            const double a1 = (double)x1[e], a2 = (double)x2[e];
            const double p = a1 * c;
            const double q = a2 * sn;
            const double y1 = p - q;
            const double r1 = a2 * c;
            const double r2 = a1 * sn;
            const double y2 = r1 + r2;
            out[s][e] = f32_to_bf16_rne((float)y1);
            out[s + NS / 2][e] = f32_to_bf16_rne((float)y2);
        }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        uint4 w;
        w.x = (uint32_t)out[s][0] | ((uint32_t)out[s][1] << 16);
        w.y = (uint32_t)out[s][2] | ((uint32_t)out[s][3] << 16);
        w.z = (uint32_t)out[s][4] | ((uint32_t)out[s][5] << 16);
        w.w = (uint32_t)out[s][6] | ((uint32_t)out[s][7] << 16);
        frag[s] = __builtin_bit_cast(bf16x8, w);
        if (a.qobs) {
            const int64_t row = (int64_t)h * 32 + i;
            *reinterpret_cast<uint4*>(a.qobs + ((u * g * 32) + row) * D + 16 * s + 8 * hh) = w;
        }
    }
}

// RoPE alignment (paper text §4.3) as its own step: one wavefront per query
// head rotates its 32 observation rows once and writes them as bf16 to
// a.qobs ([U, g*32, d]); the scoring kernel reads them as MFMA A operands.
template <int D>
__global__ __launch_bounds__(256) void rope_align_kernel(ScoreArgs a, int g, int64_t n_heads) {
    const int64_t qh = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (qh >= n_heads) return;
    bf16x8 frag[D / 16];
    build_queries<D>(a, qh / g, g, (int)(qh % g), threadIdx.x & 63, frag);
}

// A fragments of query head h of unit u: this lane's row (lane % 32) and
// dims (16 s + 8 (lane / 32) .. + 8) of the bf16 observation rows.
template <int D>
__device__ __forceinline__ void load_frag(const uint16_t* qobs, int64_t u, int g, int h,
                                          int lane, bf16x8 (&frag)[D / 16]) {
    const uint16_t* qrow =
        qobs + ((u * g + h) * 32 + (lane & 31)) * (int64_t)D + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
        frag[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + 16 * s));
}

// Causal limit of accumulator entry v as an offset from the first recent
// slot L - nrq: a key at offset d is visible iff d <= limit.  Beacon rows
// see every live slot (offset nrq - 1 is slot L - 1); recent row i sees
// slots up to its own, offset i.
__device__ __forceinline__ int row_lim(int v, int lane, int nrq) {
    const int r = acc_row(v, lane);
    return r < 16 ? nrq - 1 : r - 16;
}

// exp2 without the denormal-range fix-up: results below 2^-126 flush to 0.
// Used for the softmax sums, where such terms are negligible next to the
// row maximum's term of 1.
__device__ __forceinline__ float exp2_sum(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt on the vector-memory counter only (expcnt and lgkmcnt at their
// no-wait maxima): at most N vector memory operations of this wavefront may
// still be outstanding; they complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Direct-to-LDS loads of one key tile by the first NL wavefronts: NPW
// instructions per loader lane, in the same chunk order and XOR swizzle as
// load_tile.
template <int D, int NL>
__device__ __forceinline__ void load_tile_nl(const uint16_t* Ku, int64_t L, int64_t base,
                                             uint16_t* lds_tile, int wave, int lane) {
    constexpr int CPR = D / 8;
    constexpr int NPW = KT * CPR / (64 * NL);
    static_assert(NPW * 64 * NL == KT * CPR, "tile split");
#pragma unroll
    for (int k = 0; k < NPW; ++k) {
        const int p0 = (k * NL + wave) * 64;
        const int p = p0 + lane;
        const int j = p / CPR;
        const int c = (p % CPR) ^ (j % CPR);
        int64_t key = base + j;
        key = key < L ? key : L - 1;
        __builtin_amdgcn_global_load_lds(
            (const void*)(Ku + key * D + 8 * c),
            (__attribute__((address_space(3))) void*)(lds_tile + (int64_t)p0 * 8), 16, 0, 0);
    }
}

// Issue the direct-to-LDS loads of one key tile.  LDS chunk p (16 bytes) of
// the tile holds global chunk (row j, column c) with p = j*CPR + (c ^ (j%CPR)).
template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* Ku, int64_t L, int64_t base,
                                          uint16_t* lds_tile, int tid, int nthreads) {
    constexpr int CPR = D / 8;  // 16-byte chunks per key row
    constexpr int NCH = KT * CPR;
    const int wave = tid >> 6, lane = tid & 63;
    for (int p0 = wave * 64; p0 < NCH; p0 += nthreads) {
        const int p = p0 + lane;
        const int j = p / CPR;
        const int c = (p % CPR) ^ (j % CPR);
        int64_t key = base + j;
        key = key < L ? key : L - 1;  // tail: any valid row, masked later
        const uint16_t* gsrc = Ku + key * D + 8 * c;
        __builtin_amdgcn_global_load_lds(
            (const void*)gsrc,
            (__attribute__((address_space(3))) void*)(lds_tile + (int64_t)p0 * 8), 16, 0, 0);
    }
}

template <int D>
__device__ __forceinline__ void tile_logits(const uint16_t* lds_tile, int lane,
                                            const bf16x8 (&frag)[D / 16], f32x16& acc0,
                                            f32x16& acc1) {
    constexpr int NS = D / 16;
    constexpr int CPR = D / 8;
    const int hh = lane >> 5;
    acc0 = f32x16{};
    acc1 = f32x16{};
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int j = cb * 32 + (lane & 31);
        const uint16_t* rowp = lds_tile + j * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int c = (2 * s + hh) ^ (j % CPR);
            const uint4 w = *reinterpret_cast<const uint4*>(rowp + 8 * c);
            const bf16x8 b = __builtin_bit_cast(bf16x8, w);
            if (cb == 0)
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[s], b, acc0, 0, 0, 0);
            else
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[s], b, acc1, 0, 0, 0);
        }
    }
}

// One workgroup per unit (one wavefront per query head); with about 140
// VGPRs, 3 workgroups share a CU.
template <int D, int NL>
__global__ __launch_bounds__(512)
void score_kernel(ScoreArgs a, int g) {
    // Three separately declared tiles (not one array) so that the compiler
    // can tell the tiles being loaded by the direct-to-LDS loads from the tile
    // being read, and does not wait for the former before reading the latter.
    __shared__ __attribute__((aligned(16))) uint16_t tile0[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t tile1[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t tile2[KT * D];
    __shared__ float red[8][KT];
    constexpr int NPW = KT * (D / 8) / (64 * NL);  // loads per loader lane per tile

    const int tid = threadIdx.x;
    const int h = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lane = tid & 63;
    const bool loader = h < NL;
    const int64_t u = blockIdx.x;
    const int64_t L = a.L;
    const uint16_t* Ku = a.K + u * a.l_cap * D;
    const int ntiles = (int)((L + KT - 1) / KT);
    const int64_t mask_from = L - a.n_recent_q;  // tiles reaching past this need masks
    const float c2 = a.c2;

    bf16x8 frag[D / 16];
    load_frag<D>(a.qobs, u, g, h, lane, frag);

// One tile iteration: wait until tile `it` (in CUR) has landed while tile
// it+1 may still be in flight (loader wavefronts; NST extra stores may be
// younger than tile it+1's loads), start loading tile it+2 into NXT2, then
// run BODY on CUR.  Lane-derived addresses are recomputed every iteration
// (ti), not kept live across the loop.
#define BKV_TILE_ITER(it, NST, CUR, NXT2, ...)                                     \
    do {                                                                           \
        int ti = tid;                                                              \
        asm volatile("" : "+v"(ti));                                               \
        if (loader) {                                                              \
            if ((it) + 1 >= ntiles) wait_vm<0>();                                  \
            else if (NST) wait_vm<NPW + 1>();                                      \
            else wait_vm<NPW>();                                                   \
        }                                                                          \
        __syncthreads();                                                           \
        if (loader && (it) + 2 < ntiles)                                           \
            load_tile_nl<D, NL>(Ku, L, (int64_t)((it) + 2) * KT, NXT2, h, ti & 63); \
        f32x16 acc0, acc1;                                                         \
        tile_logits<D>(CUR, ti & 63, frag, acc0, acc1);                            \
        const int64_t base = (int64_t)(it) * KT;                                   \
        __VA_ARGS__;                                                               \
    } while (0)
// Tiles rotate through tile0, tile1, tile2; SDEL is 1 when wavefront 0
// issues a score store in each iteration (pass 2), which the wait of the
// next iteration must allow for.
#define BKV_TILE_LOOP(SDEL, ...)                                                   \
    do {                                                                           \
        if (loader) {                                                              \
            load_tile_nl<D, NL>(Ku, L, 0, tile0, h, lane);                          \
            if (1 < ntiles) load_tile_nl<D, NL>(Ku, L, KT, tile1, h, lane);         \
        }                                                                          \
        for (int it = 0; it < ntiles; it += 3) {                                   \
            BKV_TILE_ITER(it, (SDEL) && h == 0 && it > 0, tile0, tile2, __VA_ARGS__); \
            if (it + 1 < ntiles)                                                   \
                BKV_TILE_ITER(it + 1, (SDEL) && h == 0, tile1, tile0, __VA_ARGS__); \
            if (it + 2 < ntiles)                                                   \
                BKV_TILE_ITER(it + 2, (SDEL) && h == 0, tile2, tile1, __VA_ARGS__); \
        }                                                                          \
    } while (0)

    // ---------------- pass 1: per-row running max and sum of exp2 ----------
    float m[16], l[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) { m[v] = kNegBig; l[v] = 0.f; }
    const float thr = kRescaleLog2 / c2;
#define BKV_PASS1                                                                  \
    if (base + KT > mask_from) {                                                   \
        const int ln = ti & 63;                                                    \
        const int d0 = (int)(base - mask_from) + (ln & 31), d1 = d0 + 32;          \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
            const int lim = row_lim(v, ln, a.n_recent_q);                          \
            if (d0 > lim) acc0[v] = -__builtin_inff();                             \
            if (d1 > lim) acc1[v] = -__builtin_inff();                             \
        }                                                                          \
    }                                                                              \
    bool need = false;                                                             \
    _Pragma("unroll") for (int v = 0; v < 16; ++v)                                 \
        need |= fmaxf(acc0[v], acc1[v]) > m[v] + thr;                              \
    if (__builtin_amdgcn_ballot_w64(need) != 0) {                                  \
        /* Subtract before scaling: with the finite sentinel, m - mn is */         \
        /* exactly 0 when nothing visible has been seen yet. */                    \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
            const float mn = fmaxf(m[v], fmaxf(acc0[v], acc1[v]));                 \
            l[v] = l[v] * exp2_sum((m[v] - mn) * c2) + exp2_sum((acc0[v] - mn) * c2) + \
                   exp2_sum((acc1[v] - mn) * c2);                                  \
            m[v] = mn;                                                             \
        }                                                                          \
    } else {                                                                       \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
            const float mc = m[v] * c2;                                            \
            l[v] += exp2_sum(fmaf(acc0[v], c2, -mc)) + exp2_sum(fmaf(acc1[v], c2, -mc)); \
        }                                                                          \
    }
    BKV_TILE_LOOP(0, BKV_PASS1);
#undef BKV_PASS1
    // Merge the 32 lanes of each half: every lane ends with its rows' LSE.
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float m2 = __shfl_xor(m[v], o);
            const float l2 = __shfl_xor(l[v], o);
            const float mn = fmaxf(m[v], m2);
            l[v] = l[v] * exp2_sum((m[v] - mn) * c2) + l2 * exp2_sum((m2 - mn) * c2);
            m[v] = mn;
        }
    }
    float lse[16];  // log2-domain LSE in units of (logit * c2)
#pragma unroll
    for (int v = 0; v < 16; ++v) lse[v] = fmaf(m[v], c2, log2f(l[v]));

    // ---------------- pass 2: max over rows of (s - LSE) -------------------
    __syncthreads();  // everyone is done with the tiles
    float* score_u = a.score + u * a.l_cap;
#define BKV_PASS2                                                                  \
    float c0 = -__builtin_inff(), c1 = -__builtin_inff();                          \
    if (base + KT > mask_from) {                                                   \
        const int ln = ti & 63;                                                    \
        const int d0 = (int)(base - mask_from) + (ln & 31), d1 = d0 + 32;          \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
            const int lim = row_lim(v, ln, a.n_recent_q);                          \
            const float y0 = fmaf(acc0[v], c2, -lse[v]);                           \
            const float y1 = fmaf(acc1[v], c2, -lse[v]);                           \
            if (d0 <= lim) c0 = fmaxf(c0, y0);                                     \
            if (d1 <= lim) c1 = fmaxf(c1, y1);                                     \
        }                                                                          \
    } else {                                                                       \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
            c0 = fmaxf(c0, fmaf(acc0[v], c2, -lse[v]));                            \
            c1 = fmaxf(c1, fmaf(acc1[v], c2, -lse[v]));                            \
        }                                                                          \
    }                                                                              \
    /* Other half of the rows lives in lane ^ 32. */                               \
    c0 = fmaxf(c0, __shfl_xor(c0, 32));                                            \
    c1 = fmaxf(c1, __shfl_xor(c1, 32));                                            \
    if (lane < 32) {                                                               \
        red[h][lane] = c0;                                                         \
        red[h][32 + lane] = c1;                                                    \
    }                                                                              \
    __syncthreads();                                                               \
    if (tid < KT) {                                                                \
        float best = red[0][tid];                                                  \
        for (int w = 1; w < g; ++w) best = fmaxf(best, red[w][tid]);               \
        const int64_t key = base + tid;                                            \
        if (key < L) score_u[key] = exp2f(best);                                   \
    }
    BKV_TILE_LOOP(1, BKV_PASS2);
#undef BKV_PASS2
#undef BKV_TILE_LOOP
#undef BKV_TILE_ITER
}

}  // namespace

hipError_t launch_rope_table(double* table, int64_t t, int n_recent_q, int d,
                             double theta, hipStream_t s) {
    const int n = (1 + n_recent_q) * (d / 2);
    rope_table_kernel<<<(n + 255) / 256, 256, 0, s>>>(table, t, n_recent_q, d, theta);
    return hipGetLastError();
}

hipError_t launch_score(const uint16_t* K, const int32_t* kpos, int64_t n_units,
                        int g, int d, int64_t l_cap, int64_t L,
                        const float* beacons, int buf_cap, const float* recents,
                        int n_beacon, int n_recent_q, int64_t t, double theta,
                        float sm_scale, const double* table, float* score,
                        uint16_t* qobs_out, uint16_t* qobs_ws, hipStream_t s) {
    (void)n_beacon;
    if (n_units <= 0) return hipSuccess;
    ScoreArgs a;
    a.K = K;
    a.kpos = kpos;
    a.l_cap = l_cap;
    a.L = L;
    a.beacons = beacons;
    a.recents = recents;
    a.buf_cap = buf_cap;
    a.n_recent_q = n_recent_q;
    a.t = t;
    a.theta = theta;
    a.c2 = sm_scale * 1.4426950408889634f;
    a.table = table;
    a.score = score;
    a.qobs = qobs_out ? qobs_out : qobs_ws;
    const int64_t n_heads = n_units * g;
    const unsigned rblocks = (unsigned)((n_heads + 3) / 4);
    if (d == 128)
        rope_align_kernel<128><<<rblocks, 256, 0, s>>>(a, g, n_heads);
    else
        rope_align_kernel<64><<<rblocks, 256, 0, s>>>(a, g, n_heads);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)n_units);
    const dim3 block(64 * g);
    // Loader wavefronts: the largest power of two <= g, at most 4.
    const int nl = g >= 4 ? 4 : (g >= 2 ? 2 : 1);
    if (d == 128) {
        if (nl == 4) score_kernel<128, 4><<<grid, block, 0, s>>>(a, g);
        else if (nl == 2) score_kernel<128, 2><<<grid, block, 0, s>>>(a, g);
        else score_kernel<128, 1><<<grid, block, 0, s>>>(a, g);
    } else {
        if (nl == 4) score_kernel<64, 4><<<grid, block, 0, s>>>(a, g);
        else if (nl == 2) score_kernel<64, 2><<<grid, block, 0, s>>>(a, g);
        else score_kernel<64, 1><<<grid, block, 0, s>>>(a, g);
    }
    return hipGetLastError();
}

}  // namespace bkv
