// Observation-set scoring: RoPE alignment, Q_obs . K^T on bf16 MFMA,
// row softmax and the max over the GQA group.
//
// Paper text §4.3: beacons rotated to the current step t, recent queries to
// their own positions tau; attention weights W (|Q_obs| x L) against the
// current cache, max-pooled over all queries and heads of the KV group
// (summary step (4); review §4.3: Score[j] = max_{h in g} max_q W[h,q,j]).
//
// Two kernels:
//  * rope_align_kernel (one wavefront per query head) rotates the head's 32
//    observation rows (16 beacons, 16 recents) once in fp64 and writes them
//    as bf16 rows, the A operands of v_mfma_f32_32x32x16_bf16.
//  * score_kernel (one workgroup per KV group, one wavefront per query
//    head) holds its head's rows in registers as A fragments (lane: row
//    lane % 32, dims 16 s + 8 (lane / 32) .. + 8 for MFMA step s).  Keys
//    stream through a ring of three LDS tiles of 64 keys, loaded two tiles
//    ahead by buffer_load ... lds (16-byte chunks XOR-swizzled by row so the
//    32 lanes that read one chunk column hit distinct banks); all g
//    wavefronts of the group read the same tile.
//  * Pass 1: per tile each wavefront forms a 32 x 64 logit block and keeps a
//    per-lane running (max, sum of exp2) for its 16 rows; the 32 lanes of a
//    half are merged once at the end into each row's LSE.
//  * Pass 2: the logits are formed again, shifted by the row LSE, reduced
//    over the lane's 16 rows, the other half (lane ^ 32) and the g
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
// Buffer-resource flags word (gfx9 family: raw 32-bit data, no swizzle).
constexpr int kBufferFlags = 0x00020000;
constexpr float kRescaleBig = 0x1p64f; // lazy rescale: largest tile term sum kept

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
    int64_t n_units;
    int split;  // 1: each unit's heads are scored by two workgroups (scores pre-zeroed, max-combined)
};

__device__ __forceinline__ int acc_row(int v, int lane) {
    return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// RoPE alignment (paper text §4.3) as its own step, one wavefront per query
// head: lane k owns the RoPE pair (k, k + D/2) (for D = 64 the two halves of
// the wavefront take two rows at a time), walks the head's 32 observation
// rows (16 beacons at position t, 16 recents at their own positions) and
// writes them as bf16 rows to a.qobs ([U, g*32, D]), the MFMA A operands of
// the scoring kernel.  Rotation in fp64 (products rounded separately, as
// the plain definition computes them), then fp64 -> fp32 -> bf16, both
// round-to-nearest-even.  The cos/sin pairs come from the table for t and
// t-16..t-1; a recent row at any other position computes its own.
template <int D>
__device__ __forceinline__ void rotate_store(uint16_t* row, int k, float x1f, float x2f,
                                             double c, double sn) {
#pragma clang fp contract(off)
    const double x1 = (double)x1f, x2 = (double)x2f;
    const double p = x1 * c;
    const double q = x2 * sn;
    const double y1 = p - q;
    const double r1 = x2 * c;
    const double r2 = x1 * sn;
    const double y2 = r1 + r2;
    row[k] = f32_to_bf16_rne((float)y1);
    row[k + D / 2] = f32_to_bf16_rne((float)y2);
}

template <int D>
__global__ __launch_bounds__(256) void rope_align_kernel(ScoreArgs a, int g, int64_t n_heads) {
    constexpr int HALF = D / 2;
    constexpr int RPS = 64 / HALF;  // rows per step
    constexpr int NB = 16 / RPS;    // steps per 16 rows
    const int64_t qh = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (qh >= n_heads) return;
    const int lane = threadIdx.x & 63;
    const int k = lane % HALF, sub = lane / HALF;
    const int64_t u = qh / g;
    const int h = (int)(qh % g);
    if (a.split) {
        // The two workgroups of a split unit combine their scores with an
        // atomic maximum: clear the unit's score slots first (the g waves of
        // the unit take interleaved runs of 64).
        float* su = a.score + u * a.l_cap;
        for (int64_t j = (int64_t)h * 64 + lane; j < a.L; j += (int64_t)g * 64) su[j] = 0.f;
    }
    const double2* tab = reinterpret_cast<const double2*>(a.table);
    uint16_t* out = a.qobs + (u * g + h) * 32 * (int64_t)D;
    // Positions of the 16 recent rows: lane r (mod 16) holds row r's.
    const int64_t rpos = a.kpos[u * a.l_cap + a.L - a.n_recent_q + (lane & 15)];

    // Beacons (rows 0..15) at position t.  All loads are issued before any
    // arithmetic so that they overlap.
    {
        float x1[NB], x2[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const float* src = a.beacons + (qh * a.buf_cap + j * RPS + sub) * (int64_t)D;
            x1[j] = src[k];
            x2[j] = src[k + HALF];
        }
        const double2 cs = tab[k];
#pragma unroll
        for (int j = 0; j < NB; ++j)
            rotate_store<D>(out + (j * RPS + sub) * D, k, x1[j], x2[j], cs.x, cs.y);
    }
    // Recents (rows 16..31): recent r at its own position, tabulated when it
    // is t - 16 + r, else computed here.
    {
        float x1[NB], x2[NB];
        double2 cs[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int r = j * RPS + sub;
            const float* src = a.recents + (qh * a.n_recent_q + r) * (int64_t)D;
            x1[j] = src[k];
            x2[j] = src[k + HALF];
            cs[j] = tab[(1 + r) * HALF + k];
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int r = j * RPS + sub;
            const int64_t pos = __shfl(rpos, r);
            if (pos != a.t - a.n_recent_q + r) {
                double c, sn;
                rope_cs((double)pos, k, D, a.theta, &c, &sn);
                cs[j].x = c;
                cs[j].y = sn;
            }
            rotate_store<D>(out + (16 + r) * D, k, x1[j], x2[j], cs[j].x, cs[j].y);
        }
    }
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

// Maximum of two or three floats as one v_maximum(3)_f32.  The operands are
// logits, LSE offsets or their exp2 (never NaN for finite inputs); unlike
// fmaxf this needs no canonicalisation of its inputs.
__device__ __forceinline__ float vmax(float x, float y) {
    return __builtin_elementwise_maximum(x, y);
}
__device__ __forceinline__ float vmax3(float x, float y, float z) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z);
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

// Key tiles in LDS: chunk p (16 bytes) of a tile holds global chunk (row j,
// column c) of the tile's keys with p = j*CPR + (c ^ (j % CPR)), CPR = D/8
// chunks per row; the XOR swizzle by row makes the 32 lanes that read one
// chunk column for an MFMA B operand hit distinct banks.
//
// Loads go through a buffer resource whose base is the tile's first key and
// whose size ends at key L - 1: chunks of keys at or past L read as zero
// (the hardware range check, no memory access) and are masked later.  The
// first NL wavefronts load, NPW direct-to-LDS instructions per lane and
// tile; each lane's byte offsets within a tile are the same for every tile.
template <int D, int NL>
struct TileLoad {
    static constexpr int CPR = D / 8;
    static constexpr int NPW = KT * CPR / (64 * NL);
    static_assert(NPW * 64 * NL == KT * CPR, "tile split");
    // One load instruction fills 64 / CPR key rows (1 KB).  Load k of
    // wavefront w starts at row (k*NL + w) * 64/CPR; the swizzle term of a
    // lane repeats with period NP in k, so NP offsets serve all NPW loads
    // and the rest of the displacement (k * NL KB) moves the buffer base.
    static constexpr int ROWS = 64 / CPR;
    static constexpr int NP = (CPR / ROWS) / NL > 1 ? (CPR / ROWS) / NL : 1;
    int voff[NP];

    __device__ __forceinline__ TileLoad(int wave, int lane) {
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int j = (k * NL + wave) * ROWS + lane / CPR;
            const int c = (lane % CPR) ^ (j % CPR);
            voff[k] = (((k * NL + wave) * ROWS) * D + (lane / CPR) * D + 8 * c) * 2 - k * NL * 1024;
        }
    }

    // Issue the loads of keys [base, base + KT) of Ku (L keys) into lds_tile.
    __device__ __forceinline__ void issue(const uint16_t* Ku, int64_t L, int64_t base,
                                          uint16_t* lds_tile, int wave) const {
        const int bytes = (int)((L - base) * D * 2);
#pragma unroll
        for (int k = 0; k < NPW; ++k) {
            const int shift = k * NL * 1024;
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)((const char*)(Ku + base * D) + shift), 0,
                bytes > shift ? bytes - shift : 0, kBufferFlags);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc,
                (__attribute__((address_space(3))) void*)(lds_tile + (k * NL + wave) * 64 * 8),
                16, voff[k % NP], 0, 0, 0);
        }
    }
};

// Byte offsets (within a tile) of this lane's B-operand chunks for MFMA
// steps s = 0..D/16-1 of the first 32 keys; the second 32 keys are
// 32*D*2 bytes further.
template <int D>
struct TileRead {
    static constexpr int NS = D / 16;
    uint32_t off[NS];
    __device__ __forceinline__ explicit TileRead(int lane) {
        constexpr int CPR = D / 8;
        const int j = lane & 31, hh = lane >> 5;
#pragma unroll
        for (int s = 0; s < NS; ++s) off[s] = (uint32_t)(j * D + 8 * ((2 * s + hh) ^ (j % CPR))) * 2;
    }
};

template <int D>
__device__ __forceinline__ void tile_logits(const uint16_t* lds_tile, const TileRead<D>& rd,
                                            const bf16x8 (&frag)[D / 16], f32x16& acc0,
                                            f32x16& acc1) {
    constexpr int NS = D / 16;
    const char* t = reinterpret_cast<const char*>(lds_tile);
    acc0 = f32x16{};
    acc1 = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const uint4 w0 = *reinterpret_cast<const uint4*>(t + rd.off[s]);
        const uint4 w1 = *reinterpret_cast<const uint4*>(t + rd.off[s] + 32 * D * 2);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[s], __builtin_bit_cast(bf16x8, w0),
                                                       acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[s], __builtin_bit_cast(bf16x8, w1),
                                                       acc1, 0, 0, 0);
    }
}

// One workgroup per unit, one wavefront per query head; with 162 VGPRs, 12
// wavefronts share a CU.  For g > 4 (a.split) a unit's heads are shared by
// two workgroups of hs wavefronts each (the second may have an idle
// wavefront, which loads and keeps the barriers but computes nothing), so
// that more than one group fits on a CU; the pair runs on one XCD
// (blocks b and b + 8), where the second read of each key tile is likely to
// hit L2, and combines its column maxima with an atomic maximum on the
// score bits (non-negative floats order like their bit patterns).
template <int D, int NL, bool SPLIT>
__global__ __launch_bounds__(512)
void score_kernel(ScoreArgs a, int g, int hs) {
    // Three separately declared tiles (not one array) so that the compiler
    // can tell the tiles being loaded by the direct-to-LDS loads from the tile
    // being read, and does not wait for the former before reading the latter.
    __shared__ __attribute__((aligned(16))) uint16_t tile0[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t tile1[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t tile2[KT * D];
    __shared__ float red[8][KT];
    constexpr int NPW = TileLoad<D, NL>::NPW;  // loads per loader lane per tile

    const int tid = threadIdx.x;
    const int h = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lane = tid & 63;
    const bool loader = h < NL;
    int64_t u = blockIdx.x;
    int hg = h;  // query head of the group this wavefront scores
    if (SPLIT) {
        const int64_t b = blockIdx.x;
        u = (b / 16) * 8 + (b % 8);
        hg = (int)((b / 8) & 1) * hs + h;
        if (u >= a.n_units) return;  // whole workgroup, before any barrier
    }
    const bool active = !SPLIT || hg < g;
    const int nw = (int)(blockDim.x / 64);
    const int64_t L = a.L;
    const uint16_t* Ku = a.K + u * a.l_cap * D;
    const int ntiles = (int)((L + KT - 1) / KT);
    const int64_t mask_from = L - a.n_recent_q;  // tiles reaching past this need masks
    const float c2 = a.c2;

    bf16x8 frag[D / 16];
    if (active) load_frag<D>(a.qobs, u, g, hg, lane, frag);
    const TileLoad<D, NL> ld(h, lane);
    const TileRead<D> rd(lane);

// One tile iteration: wait until tile `it` (in CUR) has landed while tile
// it+1 may still be in flight (loader wavefronts; NST extra stores may be
// younger than tile it+1's loads), start loading tile it+2 into NXT2, then
// run BODY on CUR.
#define BKV_TILE_ITER(it, NST, CUR, NXT2, ...)                                     \
    do {                                                                           \
        if (loader) {                                                              \
            if ((it) + 1 >= ntiles) wait_vm<0>();                                  \
            else if (NST) wait_vm<NPW + 1>();                                      \
            else wait_vm<NPW>();                                                   \
        }                                                                          \
        __syncthreads();                                                           \
        if (loader && (it) + 2 < ntiles)                                           \
            ld.issue(Ku, L, (int64_t)((it) + 2) * KT, NXT2, h);                    \
        f32x16 acc0, acc1;                                                         \
        if (SPLIT && !active) { acc0 = f32x16{}; acc1 = f32x16{}; }                \
        else tile_logits<D>(CUR, rd, frag, acc0, acc1);                            \
        const int64_t base = (int64_t)(it) * KT;                                   \
        __VA_ARGS__;                                                               \
    } while (0)
// Tiles rotate through tile0, tile1, tile2; SDEL is 1 when wavefront 0
// issues a score store in each iteration (pass 2), which the wait of the
// next iteration must allow for.
#define BKV_TILE_LOOP(SDEL, ...)                                                   \
    do {                                                                           \
        if (loader) {                                                              \
            ld.issue(Ku, L, 0, tile0, h);                                          \
            if (1 < ntiles) ld.issue(Ku, L, KT, tile1, h);                         \
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
    // mc[v]: running maximum of row v's logits in log2 units (logit * c2),
    // starting at a finite sentinel; l[v]: sum of exp2(logit * c2 - mc[v]).
    // The maximum is updated lazily: a tile whose terms stay below
    // kRescaleBig (logits at most ~64 log2 units above mc) is summed against
    // the stale mc; otherwise (and for the first tile, where every term
    // overflows against the sentinel) the tile is redone with a rescale.
    float mc[16], l[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) { mc[v] = kNegBig; l[v] = 0.f; }
#define BKV_PASS1                                                                  \
    if (active) {                                                                  \
    if (base + KT > mask_from) {                                                   \
        const int ln = lane;                                                       \
        const int d0 = (int)(base - mask_from) + (ln & 31), d1 = d0 + 32;          \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
            const int lim = row_lim(v, ln, a.n_recent_q);                          \
            if (d0 > lim) acc0[v] = -__builtin_inff();                             \
            if (d1 > lim) acc1[v] = -__builtin_inff();                             \
        }                                                                          \
    }                                                                              \
    BKV_PASS1_HALF(0);                                                             \
    BKV_PASS1_HALF(8);                                                             \
    }
// Rows v0..v0+7 of one tile: sum against the stale maxima if every term
// stays below kRescaleBig, else rescale those rows.
#define BKV_PASS1_HALF(v0)                                                         \
    do {                                                                           \
        float tsum[8];                                                             \
        float big = 0.f;                                                           \
        _Pragma("unroll") for (int v = 0; v < 8; ++v) {                            \
            tsum[v] = exp2_sum(fmaf(acc0[(v0) + v], c2, -mc[(v0) + v])) +          \
                      exp2_sum(fmaf(acc1[(v0) + v], c2, -mc[(v0) + v]));           \
            if (v & 1) big = vmax3(big, tsum[v - 1], tsum[v]);                      \
        }                                                                          \
        if (__builtin_amdgcn_ballot_w64(!(big <= kRescaleBig)) == 0) {             \
            _Pragma("unroll") for (int v = 0; v < 8; ++v) l[(v0) + v] += tsum[v];  \
        } else {                                                                   \
            _Pragma("unroll") for (int v = (v0); v < (v0) + 8; ++v) {              \
                const float mn = vmax3(mc[v], acc0[v] * c2, acc1[v] * c2);         \
                l[v] = l[v] * exp2_sum(mc[v] - mn) + exp2_sum(fmaf(acc0[v], c2, -mn)) + \
                       exp2_sum(fmaf(acc1[v], c2, -mn));                           \
                mc[v] = mn;                                                        \
            }                                                                      \
        }                                                                          \
    } while (0)
    BKV_TILE_LOOP(0, BKV_PASS1);
#undef BKV_PASS1
#undef BKV_PASS1_HALF
    // Merge the 32 lanes of each half: every lane ends with its rows' LSE.
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float m2 = __shfl_xor(mc[v], o);
            const float l2 = __shfl_xor(l[v], o);
            const float mn = fmaxf(mc[v], m2);
            l[v] = l[v] * exp2_sum(mc[v] - mn) + l2 * exp2_sum(m2 - mn);
            mc[v] = mn;
        }
    }
    float lse[16];  // log2-domain LSE in units of (logit * c2)
#pragma unroll
    for (int v = 0; v < 16; ++v) lse[v] = mc[v] + log2f(l[v]);

    // ---------------- pass 2: max over rows of (s - LSE) -------------------
    __syncthreads();
    float* score_u = a.score + u * a.l_cap;
#define BKV_PASS2                                                                  \
    float c0 = -__builtin_inff(), c1 = -__builtin_inff();                          \
    if (base + KT > mask_from) {                                                   \
        const int ln = lane;                                                       \
        const int d0 = (int)(base - mask_from) + (ln & 31), d1 = d0 + 32;          \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
            const int lim = row_lim(v, ln, a.n_recent_q);                          \
            const float y0 = fmaf(acc0[v], c2, -lse[v]);                           \
            const float y1 = fmaf(acc1[v], c2, -lse[v]);                           \
            if (d0 <= lim) c0 = vmax(c0, y0);                                      \
            if (d1 <= lim) c1 = vmax(c1, y1);                                      \
        }                                                                          \
    } else {                                                                       \
        _Pragma("unroll") for (int v = 0; v < 16; v += 2) {                        \
            c0 = vmax3(c0, fmaf(acc0[v], c2, -lse[v]), fmaf(acc0[v + 1], c2, -lse[v + 1])); \
            c1 = vmax3(c1, fmaf(acc1[v], c2, -lse[v]), fmaf(acc1[v + 1], c2, -lse[v + 1])); \
        }                                                                          \
    }                                                                              \
    /* Other half of the rows lives in lane ^ 32. */                               \
    c0 = vmax(c0, __shfl_xor(c0, 32));                                             \
    c1 = vmax(c1, __shfl_xor(c1, 32));                                             \
    if (lane < 32) {                                                               \
        red[h][lane] = active ? c0 : -__builtin_inff();                            \
        red[h][32 + lane] = active ? c1 : -__builtin_inff();                       \
    }                                                                              \
    __syncthreads();                                                               \
    if (tid < KT) {                                                                \
        float best = red[0][tid];                                                  \
        for (int w = 1; w < nw; ++w) best = vmax(best, red[w][tid]);               \
        const int64_t key = base + tid;                                            \
        if (key < L) {                                                             \
            if (SPLIT)                                                             \
                atomicMax(reinterpret_cast<unsigned int*>(score_u + key),          \
                          __float_as_uint(exp2f(best)));                           \
            else                                                                   \
                score_u[key] = exp2f(best);                                        \
        }                                                                          \
    }
// Pass 2 walks the tiles backwards: at the end of pass 1 the last three
// tiles are still in LDS (tile T in buffer T % 3), so they are scored
// without being read again, and the rest stream in from the end with the
// same ring, two tiles ahead.  Iteration j scores tile T = ntiles - 1 - j
// from CUR and loads tile T - 2 into NXT (the buffer tile T + 1 used).
#define BKV_REV_ITER(j, CUR, NXT, ...)                                             \
    do {                                                                           \
        const int T = ntiles - 1 - (j);                                            \
        if (loader && T < ntiles - 3) {                                            \
            if (T == 0) wait_vm<0>();                                              \
            else if (h == 0) wait_vm<NPW + 1>();                                   \
            else wait_vm<NPW>();                                                   \
        }                                                                          \
        __syncthreads();                                                           \
        if (loader && T - 2 >= 0 && T - 2 < ntiles - 3)                            \
            ld.issue(Ku, L, (int64_t)(T - 2) * KT, NXT, h);                        \
        f32x16 acc0, acc1;                                                         \
        if (SPLIT && !active) { acc0 = f32x16{}; acc1 = f32x16{}; }                \
        else tile_logits<D>(CUR, rd, frag, acc0, acc1);                            \
        const int64_t base = (int64_t)T * KT;                                      \
        __VA_ARGS__;                                                               \
    } while (0)
#define BKV_REV_LOOP(B0, B1, B2, ...)                                              \
    for (int j = 0; j < ntiles; j += 3) {                                          \
        BKV_REV_ITER(j, B0, B1, __VA_ARGS__);                                      \
        if (j + 1 < ntiles) BKV_REV_ITER(j + 1, B2, B0, __VA_ARGS__);              \
        if (j + 2 < ntiles) BKV_REV_ITER(j + 2, B1, B2, __VA_ARGS__);              \
    }
    // Buffers visited from the last tile down: tile T lives in buffer T % 3.
    switch ((ntiles - 1) % 3) {
        case 0: BKV_REV_LOOP(tile0, tile1, tile2, BKV_PASS2); break;
        case 1: BKV_REV_LOOP(tile1, tile2, tile0, BKV_PASS2); break;
        default: BKV_REV_LOOP(tile2, tile0, tile1, BKV_PASS2); break;
    }
#undef BKV_REV_LOOP
#undef BKV_REV_ITER
#undef BKV_PASS2
#undef BKV_TILE_LOOP
#undef BKV_TILE_ITER
}

// Every variant is instantiated explicitly, so each gets its host launch stub
// even though it is launched from one branch of a conditional.
template __global__ void score_kernel<128, 4, false>(ScoreArgs, int, int);
template __global__ void score_kernel<128, 2, false>(ScoreArgs, int, int);
template __global__ void score_kernel<128, 1, false>(ScoreArgs, int, int);
template __global__ void score_kernel<64, 4, false>(ScoreArgs, int, int);
template __global__ void score_kernel<64, 2, false>(ScoreArgs, int, int);
template __global__ void score_kernel<64, 1, false>(ScoreArgs, int, int);
template __global__ void score_kernel<128, 4, true>(ScoreArgs, int, int);
template __global__ void score_kernel<128, 2, true>(ScoreArgs, int, int);
template __global__ void score_kernel<128, 1, true>(ScoreArgs, int, int);
template __global__ void score_kernel<64, 4, true>(ScoreArgs, int, int);
template __global__ void score_kernel<64, 2, true>(ScoreArgs, int, int);
template __global__ void score_kernel<64, 1, true>(ScoreArgs, int, int);

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
    a.n_units = n_units;
    // Groups of more than 4 heads: two workgroups per unit (see score_kernel).
    a.split = g > 4 ? 1 : 0;
    const int hs = a.split ? (g + 1) / 2 : g;
    const int64_t n_heads = n_units * g;
    const unsigned rblocks = (unsigned)((n_heads + 3) / 4);
    if (d == 128)
        rope_align_kernel<128><<<rblocks, 256, 0, s>>>(a, g, n_heads);
    else
        rope_align_kernel<64><<<rblocks, 256, 0, s>>>(a, g, n_heads);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid(a.split ? (unsigned)((n_units + 7) / 8 * 16) : (unsigned)n_units);
    const dim3 block(64 * hs);
    // Loader wavefronts: the largest power of two <= hs, at most 4.
    const int nl = hs >= 4 ? 4 : (hs >= 2 ? 2 : 1);
#define BKV_LAUNCH(DD, NN)                                                        \
    do {                                                                          \
        if (a.split) score_kernel<DD, NN, true><<<grid, block, 0, s>>>(a, g, hs);  \
        else score_kernel<DD, NN, false><<<grid, block, 0, s>>>(a, g, hs);         \
    } while (0)
    if (d == 128) {
        if (nl == 4) BKV_LAUNCH(128, 4);
        else if (nl == 2) BKV_LAUNCH(128, 2);
        else BKV_LAUNCH(128, 1);
    } else {
        if (nl == 4) BKV_LAUNCH(64, 4);
        else if (nl == 2) BKV_LAUNCH(64, 2);
        else BKV_LAUNCH(64, 1);
    }
#undef BKV_LAUNCH
    return hipGetLastError();
}

}  // namespace bkv
