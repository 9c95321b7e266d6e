// Observation-set scoring: RoPE alignment, Q_obs . K^T on bf16 MFMA,
// row softmax and the max over the GQA group.
//
// Paper text §4.3: beacons rotated to the current step t, recent queries to
// their own positions tau; attention weights W (|Q_obs| x L) against the
// current cache, max-pooled over all queries and heads of the KV group
// (summary step (4); review §4.3: Score[j] = max_{h in g} max_q W[h,q,j]).
//
// Mapping: one workgroup per KV group, one wavefront per query head.
//  * Prologue: the cos/sin table rows go to LDS and each wavefront loads its
//    head's 32 observation rows (16 beacons, 16 recents) ahead of the first
//    two key tiles; while those are in flight it rotates the rows in fp64
//    (lane = 4 RoPE pairs of a row), stages them as bf16 in LDS and reads
//    them back as the A operands of v_mfma_f32_32x32x16_bf16 (lane: row
//    lane % 32, dims 16 s + 8 (lane / 32) .. + 8 for MFMA step s).
//  * Keys stream through a ring of three LDS tiles of 64 keys, loaded two
//    tiles ahead by buffer_load ... lds (16-byte chunks XOR-swizzled by row
//    so the 32 lanes that read one chunk column hit distinct banks); all
//    wavefronts of the group read the same tile.
//  * Pass 1: per tile each wavefront forms a 32 x 64 logit block and adds
//    exp2 of its scaled logits to a per-lane sum for each of its 16 rows
//    (against a fixed reference: exact in fp32 while the row totals stay in
//    [2^-60, 2^100]; a workgroup with a row outside redoes pass 1 with a
//    running maximum); the 32 lanes of a half are merged once at the end
//    into each row's LSE.
//  * Pass 2 walks the tiles backwards (the last three are still in LDS): the
//    logits are formed again, shifted by the row LSE, reduced over the
//    lane's 16 rows, the other half (lane ^ 32) and the wavefronts (LDS,
//    two buffers: a tile's last step runs after the next tile's barrier, one
//    barrier per tile), and written as score = exp2(max).
//  * Groups of five to eight heads run a variant held to 128 VGPRs, so that
//    two workgroups share a CU.
//  Output layout of the 32x32 MFMA: lane l, accumulator v holds
//  row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32.

#include "common.h"

namespace bkv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;

constexpr int KT = 64;               // keys per tile
// Key tiles in the scoring kernel's LDS ring: loads run two tiles ahead, so
// the ring's last three tiles of pass 1 are still resident when pass 2
// starts from the end.  (Four tiles, at two workgroups per CU instead of
// three, streamed fewer units at once and were slower.)
constexpr int kRing = 3;
constexpr float kNegBig = -1.0e30f;  // finite "no key seen yet" running max
// Buffer-resource flags word (gfx9 family: raw 32-bit data, no swizzle).
constexpr int kBufferFlags = 0x00020000;
constexpr float kRescaleBig = 0x1p64f; // lazy rescale: largest tile term sum kept
constexpr float kRescaleExp = 64.0f;    // the same bound on an exponent (log2 units)
// Cache-policy word of a load whose data is not read again (non-temporal:
// it does not displace lines that other loads will reuse).
constexpr int kLoadStreaming = 2;

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
    float inv_rows;  // 1 / (g * 32): the mean pooling's divisor
    // Known softmax denominators (natural-log LSE of the scaled logits),
    // [U, g, 32] by observation row, or NULL.  Beacon rows' values cover
    // slots [0, lse_from) and pass 1 adds [lse_from, L); recent rows' values
    // are complete and pass 1 adds nothing to them.
    const float* lse_in;
    int64_t lse_from;
};

__device__ __forceinline__ int acc_row(int v, int lane) {
    return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// RoPE alignment (paper text §4.3) of one query head's 32 observation rows
// (16 beacons at position t, 16 recents at their own positions), done by
// the head's wavefront in the scoring kernel's prologue.
//
// rotate4: rotation of four RoPE pairs (x1[p], x2[p]) by (cs[p].x, cs[p].y)
// in fp64, each product rounded separately as the plain definition computes
// them, then fp64 -> fp32 -> bf16, both round-to-nearest-even (the hardware
// conversions in the default rounding mode).  Returns the four rotated
// first halves (two packed words, lower pair index in the low half) then
// the four second halves.
__device__ __forceinline__ uint4 rotate4(float4 x1, float4 x2, const double2 (&cs)[4]) {
#pragma clang fp contract(off)
    const float a1[4] = {x1.x, x1.y, x1.z, x1.w}, a2[4] = {x2.x, x2.y, x2.z, x2.w};
    float y1[4], y2[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const double u1 = (double)a1[p], u2 = (double)a2[p];
        const double m1 = u1 * cs[p].x;
        const double m2 = u2 * cs[p].y;
        const double m3 = u2 * cs[p].x;
        const double m4 = u1 * cs[p].y;
        y1[p] = (float)(m1 - m2);
        y2[p] = (float)(m3 + m4);
    }
    const auto pk = [](float lo, float hi) {
        const f32x2 v = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    };
    return uint4{pk(y1[0], y1[1]), pk(y1[2], y1[3]), pk(y2[0], y2[1]), pk(y2[2], y2[3])};
}

// The rows as loaded: lane = (row sub of each step, pairs 4q .. 4q+3 of
// the D/2 RoPE pairs (k, k + D/2)).  Observation rows 0..15 come from src1
// (the beacons, or the first 16 recent queries when the window is 32
// recent queries) and rows 16..31 from src2 (the last 16 recent queries);
// each is 16 consecutive rows of D floats.  Loading and rotating are
// separate steps so that the loads can be in flight together with the
// first key tiles.
template <int D>
struct ObsRows {
    static constexpr int HALF = D / 2;
    static constexpr int QPR = HALF / 4;  // lanes per row
    static constexpr int RPS = 64 / QPR;  // rows per step
    static constexpr int NB = 16 / RPS;   // steps per 16 rows
    float4 bx1[NB], bx2[NB], rx1[NB], rx2[NB];

    __device__ __forceinline__ void load(const float* src1, const float* src2, int lane) {
        const int q = lane % QPR, sub = lane / QPR;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const float* src = src1 + (j * RPS + sub) * (int64_t)D + 4 * q;
            bx1[j] = *reinterpret_cast<const float4*>(src);
            bx2[j] = *reinterpret_cast<const float4*>(src + HALF);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const float* src = src2 + (j * RPS + sub) * (int64_t)D + 4 * q;
            rx1[j] = *reinterpret_cast<const float4*>(src);
            rx2[j] = *reinterpret_cast<const float4*>(src + HALF);
        }
    }

    // out[j]: observation row j * RPS + sub; out[NB + j]: row 16 + j * RPS +
    // sub; each as rotate4 returns it.  Row r < 16 takes its cos/sin pairs
    // from tab1[r * stride1 + pair] (stride1 = 0: the beacons' single row for
    // t), row 16 + r from tab2[r * D/2 + pair]; all in LDS.
    __device__ __forceinline__ void rotate(int lane, const double2* tab1, int stride1,
                                           const double2* tab2, uint4 (&out)[2 * NB]) const {
        const int q = lane % QPR, sub = lane / QPR;
        double2 cs[4];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            const int r = j * RPS + sub;
#pragma unroll
            for (int p = 0; p < 4; ++p) cs[p] = tab1[r * stride1 + 4 * q + p];
            out[j] = rotate4(bx1[j], bx2[j], cs);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            // One row's cos/sin pairs at a time (the scheduler would
            // otherwise read all of them up front, 16 registers a row).
            __builtin_amdgcn_sched_barrier(0);
            const int r = j * RPS + sub;
#pragma unroll
            for (int p = 0; p < 4; ++p) cs[p] = tab2[r * HALF + 4 * q + p];
            out[NB + j] = rotate4(rx1[j], rx2[j], cs);
        }
    }
};

// The table holds the cos/sin pairs for positions t-nrq..t-1 (nrq = 16 or
// 32 recent queries); recent rows of the unit at other positions (lane r
// (mod nrq) holds row r's position in rpos) get theirs computed into the
// LDS copy (rows 0..15 at rtab_lo, rows 16..31 at rtab_hi, [16][D/2]
// double2 each) by the whole workgroup.  Every wavefront of the workgroup
// sees the same positions, so all take the same branch.  Returns whether
// any row moved.
template <int D>
__device__ __forceinline__ bool fix_recent_table(const ScoreArgs& a, int64_t u, int32_t rpos,
                                                 int lane, int tid, int nthreads,
                                                 double2* rtab_lo, double2* rtab_hi) {
    const int nrq = a.n_recent_q;
    const int32_t first = (int32_t)(a.t - nrq);
    if (__ballot(rpos != first + (lane & (nrq - 1))) == 0) return false;
    const int32_t* rp = a.kpos + u * a.l_cap + a.L - nrq;
    for (int e = tid; e < nrq * (D / 2); e += nthreads) {
        const int r = e / (D / 2), k = e % (D / 2);
        const int32_t pos = rp[r];
        if (pos != first + r) {
            double c, sn;
            rope_cs((double)pos, k, D, a.theta, &c, &sn);
            (r < 16 ? rtab_lo : rtab_hi)[(r % 16) * (D / 2) + k] = double2{c, sn};
        }
    }
    __syncthreads();
    return true;
}

// Writes rotated rows to `stage` (LDS, 32 rows in the swizzled layout of a
// key tile): per row, 4 consecutive dims of each half.
template <int D>
__device__ __forceinline__ void put_rows(const uint4 (&v)[2 * ObsRows<D>::NB], int lane,
                                         uint16_t* stage) {
    using O = ObsRows<D>;
    constexpr int CPR = D / 8;
    const int q = lane % O::QPR, sub = lane / O::QPR;
#pragma unroll
    for (int i = 0; i < 2 * O::NB; ++i) {
        const int r = (i / O::NB) * 16 + (i % O::NB) * O::RPS + sub;
        const int c1 = q >> 1, c2 = O::HALF / 8 + (q >> 1), e = 4 * (q & 1);
        *reinterpret_cast<uint2*>(stage + (r * CPR + (c1 ^ (r % CPR))) * 8 + e) =
            uint2{v[i].x, v[i].y};
        *reinterpret_cast<uint2*>(stage + (r * CPR + (c2 ^ (r % CPR))) * 8 + e) =
            uint2{v[i].z, v[i].w};
    }
}

// Causal limit of accumulator entry v as an offset from the first recent
// slot L - nrq: a key at offset d is visible iff d <= limit.  Beacon rows
// see every live slot (offset nrq - 1 is slot L - 1); recent row i sees
// slots up to its own, offset i.  nrq is 16 (after 16 beacon rows) or 32.
__device__ __forceinline__ int row_lim(int v, int lane, int nrq) {
    const int r = acc_row(v, lane);
    // 32 recent rows: row r is recent row r.  16 beacons + 16 recents: the
    // beacons are rows 0..15, i.e. accumulator entries v < 8 (a compile-time
    // fact once v is unrolled).
    if (nrq == 32) return r;
    return v < 8 ? nrq - 1 : r - 16;
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

// Workgroup barrier of the scoring kernel.  HIP's __syncthreads() carries a
// workgroup-scope release fence, which on this target waits for every
// outstanding vector memory operation -- including the direct-to-LDS loads
// of the key tiles still ahead -- and so would drain the prefetch at every
// tile.  Here each wavefront has already waited (vmcnt) for its share of
// every tile read after the barrier; the barrier drains only LDS traffic
// (lgkmcnt: earlier reads of a buffer about to be refilled, writes of the
// reduction buffer), and wavefront-scope fences keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unbounded
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
template <int D, int NL, int TK = KT>
struct TileLoad {
    static constexpr int CPR = D / 8;
    static constexpr int NPW = TK * CPR / (64 * NL);
    static_assert(NPW * 64 * NL == TK * CPR, "tile split");
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

    // Issue the loads of keys [base, base + TK) of Ku (L keys) into lds_tile,
    // with cache policy AUX (0, or kLoadStreaming for a last read).
    template <int AUX = 0>
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
                16, voff[k % NP], 0, 0, AUX);
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

// One workgroup per unit, one wavefront per query head; with 165 VGPRs, 12
// wavefronts share a CU.  OCC > 0 holds the kernel to the registers of OCC
// wavefronts per SIMD (groups of 5 to 8 heads: see launch_score).
template <int D, int NL, bool MEAN, int OCC = 0>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(OCC > 0 ? OCC : 1, 8)))
void score_kernel(ScoreArgs a, int g) {
    // Three separately declared tiles (not one array) so that the compiler
    // can tell the tiles being loaded by the direct-to-LDS loads from the tile
    // being read, and does not wait for the former before reading the latter.
    __shared__ __attribute__((aligned(16))) uint16_t tile0[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t tile1[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t tile2[KT * D];
    __shared__ float red[2][8][KT];  // pass 2: one buffer per tile parity
    constexpr int NPW = TileLoad<D, NL>::NPW;  // loads per loader lane per tile

    const int tid = threadIdx.x;
    const int h = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lane = tid & 63;
    const bool loader = h < NL;
    const int64_t u = blockIdx.x;
    const int hg = h;  // query head of the group this wavefront scores
    const int nw = (int)(blockDim.x / 64);
    const int64_t L = a.L;
    const uint16_t* Ku = a.K + u * a.l_cap * D;
    const int ntiles = (int)((L + KT - 1) / KT);
    const int64_t mask_from = L - a.n_recent_q;  // tiles reaching past this need masks
    // With known denominators pass 1 covers only the tiles from the one
    // holding slot lse_from (at least the last tile): tiles t0 .. ntiles-1.
    const bool lse_mode = a.lse_in != nullptr;
    const int t0 = lse_mode ? (int)(a.lse_from / KT < ntiles - 1 ? a.lse_from / KT : ntiles - 1) : 0;
    const int nt1 = ntiles - t0;
    // The prologue's second tile: the next one of pass 1, or, when pass 1
    // has a single tile, the first one pass 2 needs beyond it (tile
    // ntiles-2, into buffer 1; pass 2 then visits the buffers in the
    // reflected order 0, 1, 2).
    const bool reflect = lse_mode && nt1 == 1 && ntiles >= 2;
    const int second = nt1 >= 2 ? t0 + 1 : (reflect ? ntiles - 2 : -1);
    const float c2 = a.c2;

    const TileLoad<D, NL> ld(h, lane);

    // Prologue.  The table's cos/sin rows for the recent positions
    // t-nrq..t-1 (nrq x D/2 pairs of doubles: one tile buffer per 16 rows)
    // go to the third tile buffer (and, for 32 recent queries, the second)
    // and the row for t to the reduction buffer by direct-to-LDS loads, each
    // wavefront loads its head's observation rows, then the loader
    // wavefronts issue the first key tiles (two, unless the second buffer
    // holds table rows) and wait for everything older.  The rows are rotated
    // while the tiles are in flight and staged, two heads at a time, through
    // the third tile buffer, from where each wavefront reads its MFMA A
    // fragments (lane: row lane % 32, dims 16 s + 8 (lane / 32) .. + 8 for
    // step s; the same swizzled layout as a key tile).
    const int64_t qh = u * g + hg;
    const int nrq = a.n_recent_q;
    const bool wide = nrq == 32;  // window of 32 recent queries, no beacons
    {
        constexpr int NIT = KT * D * 2 / 1024;  // 1 KB loads per tile buffer (16 table rows)
        static_assert(D / 2 * 16 <= (int)sizeof(red), "table row for t fits the reduction buffer");
        const int NI = wide ? 2 * NIT : NIT;
        const char* tab = reinterpret_cast<const char*>(a.table);
        for (int i = h; i <= NI; i += nw) {
            const bool row0 = i == NI;
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(tab + (row0 ? 0 : (D / 2) * 16 + i * 1024)), 0, row0 ? (D / 2) * 16 : 1024,
                kBufferFlags);
            uint16_t* dst = (i < NIT ? tile2 : tile1) + (i % NIT) * 512;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc,
                (__attribute__((address_space(3))) void*)(row0 ? (void*)&red[0][0][0] : (void*)dst),
                16, lane * 16, 0, 0, 0);
        }
    }
    const int32_t rpos = a.kpos[u * a.l_cap + L - nrq + (lane & (nrq - 1))];
    const float* src1 = wide ? a.recents + qh * nrq * (int64_t)D
                             : a.beacons + qh * a.buf_cap * (int64_t)D;
    const float* src2 = a.recents + (qh * nrq + nrq - 16) * (int64_t)D;
    ObsRows<D> obs;
    obs.load(src1, src2, lane);
    if (loader) {
        ld.issue(Ku, L, (int64_t)t0 * KT, tile0, h);
        if (!wide && second >= 0) {
            ld.issue(Ku, L, (int64_t)second * KT, tile1, h);
            wait_vm<2 * NPW>();
        } else {
            wait_vm<NPW>();
        }
    } else {
        wait_vm<0>();
    }
    lds_barrier();  // the cos/sin rows have landed
    double2* rtab_lo = reinterpret_cast<double2*>(tile2);
    double2* rtab_hi = reinterpret_cast<double2*>(tile1);
    if (fix_recent_table<D>(a, u, rpos, lane, tid, 64 * nw, rtab_lo, rtab_hi)) {
        // Rare path: the rows are loaded again, so that their first copy is
        // dead while the cos/sin pairs are computed and its registers free.
        obs.load(src1, src2, lane);
    }
    bf16x8 frag[D / 16];
    {
        uint4 rows[2 * ObsRows<D>::NB];
        {
            // Rows 0..15: the beacons' row for t, or recent rows 0..15; rows
            // 16..31: the last 16 recent rows.
            const double2* tab1 = wide ? rtab_lo : reinterpret_cast<const double2*>(&red[0][0][0]);
            obs.rotate(lane, tab1, wide ? D / 2 : 0, wide ? rtab_hi : rtab_lo, rows);
        }
        // The rotated words pass through an empty asm before the barrier, so
        // the arithmetic stays ahead of it (sunk past it, it would keep every
        // cos/sin pair read before the barrier in registers at once).
#pragma unroll
        for (int i = 0; i < 2 * ObsRows<D>::NB; ++i)
            asm volatile("" : "+v"(rows[i].x), "+v"(rows[i].y), "+v"(rows[i].z), "+v"(rows[i].w));
        lds_barrier();  // the cos/sin rows are no longer needed
        uint16_t* stage = tile2 + (h & 1) * 32 * D;
        for (int rnd = 0; 2 * rnd < nw; ++rnd) {
            const bool mine = (h >> 1) == rnd;
            // A fresh copy of the lane index per round keeps the staging
            // addresses from being hoisted out of the loop into registers.
            int ln = lane;
            asm volatile("" : "+v"(ln));
            if (mine) put_rows<D>(rows, ln, stage);
            lds_barrier();
            if (mine) {
                const TileRead<D> rs(ln);
                const char* st = reinterpret_cast<const char*>(stage);
#pragma unroll
                for (int s = 0; s < D / 16; ++s)
                    frag[s] = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const uint4*>(st + rs.off[s]));
                // Observation rows out (a.qobs: [U, g*32, D] bf16): lane
                // holds 8 consecutive dims per step.
                if (a.qobs) {
                    uint16_t* q = a.qobs + (qh * 32 + (ln & 31)) * (int64_t)D + 8 * (ln >> 5);
#pragma unroll
                    for (int s = 0; s < D / 16; ++s)
                        *reinterpret_cast<uint4*>(q + 16 * s) = __builtin_bit_cast(uint4, frag[s]);
                }
            }
            lds_barrier();
        }
    }

    // With 32 recent queries the second tile buffer held table rows: its key
    // tile is issued now.
    if (loader && wide && second >= 0) ld.issue(Ku, L, (int64_t)second * KT, tile1, h);

    // Per-lane LDS offsets of the key tiles' B operands, formed after the
    // prologue (from a fresh copy of the lane index) so that they do not
    // occupy registers during it.
    int lane_rd = lane;
    asm volatile("" : "+v"(lane_rd));
    const TileRead<D> rd(lane_rd);

// One tile iteration: wait until tile `it` (in CUR) has landed while tile
// it+1 may still be in flight (loader wavefronts; NST extra stores may be
// younger than tile it+1's loads), start loading tile it+2 into NXT2, then
// run BODY on CUR.
#define BKV_TILE_ITER(it, NST, CUR, NXT2, ...)                                     \
    do {                                                                           \
        if (loader) {                                                              \
            if ((it) + 1 >= nt1) wait_vm<0>();                                     \
            else if (NST) wait_vm<NPW + 1>();                                      \
            else wait_vm<NPW>();                                                   \
        }                                                                          \
        lds_barrier();                                                           \
        if (loader && (it) + 2 < nt1)                                              \
            ld.issue(Ku, L, (int64_t)(t0 + (it) + 2) * KT, NXT2, h);               \
        f32x16 acc0, acc1;                                                         \
        tile_logits<D>(CUR, rd, frag, acc0, acc1);                                 \
        const int64_t base = (int64_t)(t0 + (it)) * KT;                            \
        __VA_ARGS__;                                                               \
    } while (0)
// Tiles rotate through tile0 .. tile2 (tiles 0 and 1 are issued by the
// prologue); SDEL is 1 when wavefront 0 issues a score store in each
// iteration, which the wait of the next iteration must allow for.
#define BKV_TILE_LOOP(SDEL, ...)                                                   \
    do {                                                                           \
        for (int it = 0; it < nt1; it += 3) {                                      \
            BKV_TILE_ITER(it, (SDEL) && h == 0 && it > 0, tile0, tile2, __VA_ARGS__); \
            if (it + 1 < nt1)                                                      \
                BKV_TILE_ITER(it + 1, (SDEL) && h == 0, tile1, tile0, __VA_ARGS__); \
            if (it + 2 < nt1)                                                      \
                BKV_TILE_ITER(it + 2, (SDEL) && h == 0, tile2, tile1, __VA_ARGS__); \
        }                                                                          \
    } while (0)

    // ---------------- pass 1: the rows' log-sum-exp --------------------------
    // Fast path: ls[v] sums exp2(logit * c2) for row v over the lane's
    // columns against a fixed reference of 0 (log2 units): one multiply, one
    // exp2 and one add per logit, no running maximum and no branch.  In fp32
    // this is as exact as the running-maximum form while every row's total
    // lies in [2^-60, 2^100]: no partial sum overflows, and terms flushed to
    // zero (below 2^-126) are under 2^-53 of the row's largest term.  That
    // covers row log-sum-exps from about -41 to 69 (natural log).  A
    // workgroup with any row outside redoes pass 1 with the running maximum
    // (exact for any logits), so the range only decides the speed.
    // With known denominators, column 0 of each row starts from the row's
    // value (in log2 units: LSE * log2(e)); -inf (no slots before lse_from)
    // starts empty.
#define BKV_PASS1_MASKS                                                            \
    if (lse_mode) {                                                                \
        /* Beacon rows add the slots in [lse_from, L); recent rows none. */       \
        int ln = lane; /* fresh copy: the limits are not hoisted */                \
        asm volatile("" : "+v"(ln));                                              \
        const int64_t k0 = base + (ln & 31), k1 = k0 + 32;                         \
        const bool in0 = k0 >= a.lse_from && k0 < L;                               \
        const bool in1 = k1 >= a.lse_from && k1 < L;                               \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
            const bool brow = !wide && v < 8;                                      \
            if (!(brow && in0)) acc0[v] = -__builtin_inff();                       \
            if (!(brow && in1)) acc1[v] = -__builtin_inff();                       \
        }                                                                          \
    } else if (base + KT > mask_from) {                                            \
        int ln = lane; /* fresh copy: the limits are not hoisted */                \
        asm volatile("" : "+v"(ln));                                              \
        const int d0 = (int)(base - mask_from) + (ln & 31), d1 = d0 + 32;          \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
            const int lim = row_lim(v, ln, a.n_recent_q);                          \
            if (d0 > lim) acc0[v] = -__builtin_inff();                             \
            if (d1 > lim) acc1[v] = -__builtin_inff();                             \
        }                                                                          \
    }
    float ls[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) ls[v] = 0.f;
    if (lse_mode && (lane & 31) == 0) {
        const float* li = a.lse_in + qh * 32;
#pragma unroll
        for (int v = 0; v < 16; ++v) ls[v] = exp2_sum(li[acc_row(v, lane)] * 1.4426950408889634f);
    }
#define BKV_PASS1_FAST                                                             \
    do {                                                                           \
        BKV_PASS1_MASKS                                                            \
        _Pragma("unroll") for (int v = 0; v < 16; ++v)                             \
            ls[v] += exp2_sum(acc0[v] * c2) + exp2_sum(acc1[v] * c2);              \
    } while (0)
    BKV_TILE_LOOP(0, BKV_PASS1_FAST);
#undef BKV_PASS1_FAST
    // Totals over the 32 lanes of each half.
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
#pragma unroll
        for (int v = 0; v < 16; ++v) ls[v] += __shfl_xor(ls[v], o);
    }
    int out_of_range = 0;
#pragma unroll
    for (int v = 0; v < 16; ++v) out_of_range |= !(ls[v] >= 0x1p-60f && ls[v] <= 0x1p100f);
    float lse[16];  // log2-domain LSE in units of (logit * c2)
    if (!__syncthreads_or(out_of_range)) {
#pragma unroll
        for (int v = 0; v < 16; ++v) lse[v] = log2f(ls[v]);
    } else {
        // Pass 1 again with a running maximum.  Every wavefront is past the
        // barrier, so no tile buffer is still being read; the loads start
        // over as the prologue issued them.
        if (loader) {
            ld.issue(Ku, L, (int64_t)t0 * KT, tile0, h);
            if (second >= 0) ld.issue(Ku, L, (int64_t)second * KT, tile1, h);
        }
        // mc[v]: running maximum of row v's logits in log2 units (logit * c2),
        // starting at a finite sentinel; l[v]: sum of exp2(logit * c2 - mc[v]).
        // The maximum is updated lazily: a tile whose terms stay below
        // kRescaleBig (logits at most ~64 log2 units above mc) is summed
        // against the stale mc; otherwise (and for the first tile, where every
        // term overflows against the sentinel) the tile is redone with a
        // rescale.  Known denominators start column 0 at their value with a
        // sum of 1.
        float mc[16], l[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) { mc[v] = kNegBig; l[v] = 0.f; }
        if (lse_mode && (lane & 31) == 0) {
            const float* li = a.lse_in + qh * 32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float x = li[acc_row(v, lane)] * 1.4426950408889634f;
                if (x > kNegBig) { mc[v] = x; l[v] = 1.f; }
            }
        }
#define BKV_PASS1                                                                  \
    do {                                                                           \
        BKV_PASS1_MASKS                                                            \
        BKV_PASS1_HALF(0);                                                         \
        BKV_PASS1_HALF(8);                                                         \
    } while (0)
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
#pragma unroll
        for (int v = 0; v < 16; ++v) lse[v] = mc[v] + log2f(l[v]);
    }
#undef BKV_PASS1_MASKS

    // ---------------- pass 2: max over rows of (s - LSE) -------------------
    // Tiles t_res .. ntiles-1 are in LDS and complete (tile T in buffer
    // (T - t0) mod 3, or (ntiles - 1 - T) mod 3 when reflected); every other
    // tile is loaded by the walk two iterations ahead, the first of them at
    // iteration 0 when fewer than three tiles are resident.
    const int t_res = reflect ? ntiles - 2 : (t0 > ntiles - kRing ? t0 : ntiles - kRing);
    // Pass 1 has waited for all its loads in its last iteration; saying so
    // here (free at run time) tells the compiler that no tile load is still
    // in flight when pass 2 starts, so that its first reads need no wait.
    wait_vm<0>();
    lds_barrier();
    float* score_u = a.score + u * a.l_cap;
    // The cross-wavefront step of a tile's reduction (wavefront rw, lane =
    // key), run after the next tile's barrier: the tiles alternate between
    // the two halves of red, so pass 2 needs one barrier per tile.  With five
    // to seven wavefronts, wavefront 3 is the one alone on its SIMD (waves
    // are placed round-robin on the four), so it takes this extra work.
    static_assert(KT == 64, "one lane per key of a tile");
    const int rw = (nw >= 5 && nw <= 7) ? 3 : 0;
    auto p2_reduce = [&](int64_t kb, int b) {
        if (h == rw) {
            const int64_t key = kb + lane;
            if constexpr (MEAN) {
                float tot = red[b][0][lane];
                for (int w = 1; w < nw; ++w) tot += red[b][w][lane];
                if (key < L) score_u[key] = tot * a.inv_rows;
            } else {
                float best = red[b][0][lane];
                for (int w = 1; w < nw; ++w) best = vmax(best, red[b][w][lane]);
                if (key < L) score_u[key] = exp2f(best);
            }
        }
    };
#define BKV_PASS2                                                                  \
    if constexpr (MEAN) {                                                          \
        BKV_PASS2_MEAN;                                                            \
    } else {                                                                       \
        BKV_PASS2_MAX;                                                             \
    }
// Max pooling: the largest (s - LSE) over the lane's rows, the other half
// and the wavefronts, then one exp2 per key.
#define BKV_PASS2_MAX                                                              \
    float c0 = -__builtin_inff(), c1 = -__builtin_inff();                          \
    if (base + KT > mask_from) {                                                   \
        int ln = lane; /* fresh copy: the limits are not hoisted */                \
        asm volatile("" : "+v"(ln));                                              \
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
        red[rb][h][lane] = c0;                                                     \
        red[rb][h][32 + lane] = c1;                                                \
    }
// Mean pooling: the sum of exp2(s - LSE) = W over the lane's rows (hidden
// entries add nothing), the other half and the wavefronts, divided by the
// group's g * 32 rows.  Terms below 2^-126 flush to zero, far below any
// score that matters (at most 256 of them).
#define BKV_PASS2_MEAN                                                             \
    float c0 = 0.f, c1 = 0.f;                                                      \
    if (base + KT > mask_from) {                                                   \
        int ln = lane; /* fresh copy: the limits are not hoisted */                \
        asm volatile("" : "+v"(ln));                                              \
        const int d0 = (int)(base - mask_from) + (ln & 31), d1 = d0 + 32;          \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
            const int lim = row_lim(v, ln, a.n_recent_q);                          \
            const float e0 = exp2_sum(fmaf(acc0[v], c2, -lse[v]));                 \
            const float e1 = exp2_sum(fmaf(acc1[v], c2, -lse[v]));                 \
            c0 += d0 <= lim ? e0 : 0.f;                                            \
            c1 += d1 <= lim ? e1 : 0.f;                                            \
        }                                                                          \
    } else {                                                                       \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) {                           \
            c0 += exp2_sum(fmaf(acc0[v], c2, -lse[v]));                            \
            c1 += exp2_sum(fmaf(acc1[v], c2, -lse[v]));                            \
        }                                                                          \
    }                                                                              \
    c0 += __shfl_xor(c0, 32);                                                      \
    c1 += __shfl_xor(c1, 32);                                                      \
    if (lane < 32) {                                                               \
        red[rb][h][lane] = c0;                                                     \
        red[rb][h][32 + lane] = c1;                                                \
    }
// Pass 2 walks the tiles backwards: at the end of pass 1 the last tiles
// (three, or the ones pass 1 covered plus the prologue's second tile) are
// still in LDS, so they are scored without being read again, and the rest
// stream in from the end with the same ring, two tiles ahead, as streaming
// (non-temporal) loads: it is their last read, and left out of the caches
// they do not push out the tiles pass 1 of other workgroups will read again
// (6% faster than plain loads; pass 1's loads stay plain, as pass 2 reads
// its last tiles from L2).  Iteration j scores tile T = ntiles - 1 - j from
// CUR and loads tile T - 2 into NXT (the buffer tile T + 1 used, or an unused
// one at j = 0); from j = 1 on, wavefront rw then stores tile T + 1's scores,
// one store younger than those loads, which its wait allows for.
#define BKV_REV_STEP(j, CUR, NXT, LOAD, ...)                                       \
    do {                                                                           \
        const int T = ntiles - 1 - (j);                                            \
        if (loader && T < t_res) {                                                 \
            if (T == 0) wait_vm<0>();                                              \
            else if (h == rw) wait_vm<NPW + 1>();                                  \
            else wait_vm<NPW>();                                                   \
        }                                                                          \
        lds_barrier();                                                           \
        if (LOAD)                                                                  \
            ld.template issue<kLoadStreaming>(Ku, L, (int64_t)(T - 2) * KT, NXT, h); \
        if ((j) > 0) p2_reduce((int64_t)(T + 1) * KT, ((j) - 1) & 1);            \
        f32x16 acc0, acc1;                                                         \
        tile_logits<D>(CUR, rd, frag, acc0, acc1);                                 \
        const int64_t base = (int64_t)T * KT;                                      \
        const int rb = (j) & 1;                                                    \
        __VA_ARGS__;                                                               \
    } while (0)
#define BKV_REV_ITER(j, CUR, NXT, ...)                                             \
    BKV_REV_STEP(j, CUR, NXT, loader && T - 2 >= 0 && T - 2 < t_res, __VA_ARGS__)
#define BKV_REV_LOOP(B0, B1, B2, ...)                                              \
    for (int j = 0; j < ntiles; j += 3) {                                          \
        BKV_REV_ITER(j, B0, B1, __VA_ARGS__);                                      \
        if (j + 1 < ntiles) BKV_REV_ITER(j + 1, B2, B0, __VA_ARGS__);              \
        if (j + 2 < ntiles) BKV_REV_ITER(j + 2, B1, B2, __VA_ARGS__);              \
    }
// The loader wavefronts from iteration j on, X0 being the buffer iteration j
// scores: whole rounds of three iterations that each load a tile (no branch
// around a load inside the loop: with loads that some paths through the loop
// skip, the compiler cannot count which loads are still in flight and waits
// for all of them before reading a tile -- one round trip to memory in every
// third iteration), then the last one to four iterations, whose loads stop
// at tile 0.
#define BKV_REV_FAST(X0, X1, X2, ...)                                              \
    wait_vm<0>();                                                                  \
    for (; j + 3 <= ntiles - 2; j += 3) {                                          \
        BKV_REV_STEP(j, X0, X1, true, __VA_ARGS__);                                \
        BKV_REV_STEP(j + 1, X2, X0, true, __VA_ARGS__);                            \
        BKV_REV_STEP(j + 2, X1, X2, true, __VA_ARGS__);                            \
    }                                                                              \
    if (j < ntiles) BKV_REV_STEP(j, X0, X1, T >= 2, __VA_ARGS__);                  \
    if (j + 1 < ntiles) BKV_REV_STEP(j + 1, X2, X0, T >= 2, __VA_ARGS__);          \
    if (j + 2 < ntiles) BKV_REV_STEP(j + 2, X1, X2, T >= 2, __VA_ARGS__);          \
    if (j + 3 < ntiles) BKV_REV_STEP(j + 3, X0, X1, T >= 2, __VA_ARGS__)
    // Buffers visited from the last tile down.
    {
        if (loader && (reflect || t0 <= ntiles - 3)) {
            // Reflected: no tile is resident beyond the two pass 1 left, so
            // every iteration from the first loads (t_res = ntiles - 2).
            // Otherwise the first iteration scores the last tile, resident,
            // and loads nothing (t_res = ntiles - 3); the rounds start at
            // iteration 1, one buffer further round the ring.
            int j = 0;
            if (reflect) {
                BKV_REV_FAST(tile0, tile2, tile1, BKV_PASS2);
            } else {
                switch ((ntiles - 1 - t0) % 3) {
                    case 0:
                        BKV_REV_STEP(0, tile0, tile1, false, BKV_PASS2);
                        j = 1;
                        BKV_REV_FAST(tile2, tile0, tile1, BKV_PASS2);
                        break;
                    case 1:
                        BKV_REV_STEP(0, tile1, tile2, false, BKV_PASS2);
                        j = 1;
                        BKV_REV_FAST(tile0, tile1, tile2, BKV_PASS2);
                        break;
                    default:
                        BKV_REV_STEP(0, tile2, tile0, false, BKV_PASS2);
                        j = 1;
                        BKV_REV_FAST(tile1, tile2, tile0, BKV_PASS2);
                        break;
                }
            }
        } else if (reflect) {
            BKV_REV_LOOP(tile0, tile2, tile1, BKV_PASS2);
        } else {
            switch ((ntiles - 1 - t0) % 3) {
                case 0: BKV_REV_LOOP(tile0, tile1, tile2, BKV_PASS2); break;
                case 1: BKV_REV_LOOP(tile1, tile2, tile0, BKV_PASS2); break;
                default: BKV_REV_LOOP(tile2, tile0, tile1, BKV_PASS2); break;
            }
        }
    }
    lds_barrier();
    p2_reduce(0, (ntiles - 1) & 1);  // the last tile walked is tile 0
#undef BKV_REV_FAST
#undef BKV_REV_LOOP
#undef BKV_REV_ITER
#undef BKV_REV_STEP
#undef BKV_PASS2
#undef BKV_PASS2_MAX
#undef BKV_PASS2_MEAN
#undef BKV_TILE_LOOP
#undef BKV_TILE_ITER
}

// ---------------------------------------------------------------------------
// Decode attention with the beacons' softmax denominators.
//
// Paper text §2.1: the decode step's attention softmax(q k^T / sqrt(d)) V of
// each query head's new query over its KV head's cache; summary "未来方向":
// beacon scoring folded into the attention kernel.  While the keys stream
// through, the same MFMA blocks give the logits of the head's 16 beacons
// (rotated to the coming eviction's step t_obs), whose log-sum-exp over the
// cache is the beacon rows' softmax denominator; the new query's own
// log-sum-exp is a recent row's denominator at the next eviction.
//
// Mapping: one workgroup per unit, one wavefront per query head (groups of
// more than four heads in a 128-VGPR form, see decode_kernel).
// A fragments (rows of the 32 x 32 x 16 MFMA): rows 0..15 the beacons, rows
// 16 and 20 the new query, the other rows zero; each lane rotates its own
// row's dims (16 s + 8 (lane / 32) .. + 8 for step s pair with the same dims
// of step s + D/32) in fp64 and rounds through fp32 to bf16.  Keys and
// values stream through rings of three LDS tiles of 32 rows.  Per tile: one
// 32 x 32 logit block; the beacon rows update a per-lane running (max, sum
// of exp2) as the scoring's pass 1 does; the new query's 32 logits
// (accumulator 8: row 16 in lanes 0..31, its copy in row 20 in lanes
// 32..63) update a lazily raised running max and a per-lane sum, and the
// weights times the value tile run on the matrix cores (see vt_offset).
// Keys and values are read once, with streaming (non-temporal) loads.
constexpr int DT = 32;  // keys per tile of the decode kernel

struct DecodeArgs {
    const uint16_t* K;
    const uint16_t* V;
    int64_t l_cap;
    int64_t L;
    const float* q;         // [U * g, D] pre-RoPE, rotated to t_q
    int64_t t_q;
    const float* beacons;   // [U * g, buf_cap, D] rows 0..15, rotated to t_obs; or NULL
    int buf_cap;
    int64_t t_obs;
    double theta;
    float c2;               // sm_scale * log2(e)
    float* out;             // [U * g, D]
    float* lse_q;           // [U * g]
    float* lse_obs;         // [U * g, 16] (when beacons != NULL)
    int64_t n_units;
};

// Value products on the matrix cores: one 16 x 16 x 32 bf16 MFMA per 16
// dims of the output.  B is the value tile (32 keys x 16 dims); A holds the
// query's 32 weights, a bf16 high part (the top 16 bits of the fp32 weight)
// in the even rows and the truncated remainder in the odd rows, so that
// accumulators 0 and 1 of a lane (rows 4 (lane / 16) and 4 (lane / 16) + 1,
// column lane % 16) add up to sum_j p_j V[j][dim] with each weight kept to
// about 2^-14 relative.  Key slots 0..7 of lane group q (lanes 16 q ..
// 16 q + 15) are keys 4 q + i and 16 + 4 q + i (i < 4): the two halves read
// rows with the same XOR swizzle, 16 rows apart.  Each half is one LDS
// transpose read (ds_read_b64_tr_b16): in a group of 16 lanes, lane 4 r + c
// reads dims 4 c .. 4 c + 3 of the block from key row r of the half, and
// lane n receives the four rows' values of dim n.  vt_offset is this lane's
// byte offset for block 0 and the first half; block b is that offset XOR
// 32 b (the swizzle permutes 16-byte chunks within a row), the second half
// is 32 D bytes further.
template <int D>
__device__ __forceinline__ uint32_t vt_offset(int lane) {
    constexpr int CPR = D / 8;
    const int q = (lane >> 4) & 3, t = lane & 15;
    const int j = 4 * q + (t >> 2);
    const int c = ((t & 3) >> 1) ^ (j % CPR);
    return (uint32_t)(j * D * 2 + c * 16 + (t & 1) * 8);
}

__device__ __forceinline__ i16x4 lds_read_tr16(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
}

// The running max of the new query's logits (log2 units) is raised only
// when a logit exceeds it by more than this, so that the value accumulators
// are rescaled rarely; weights stay below 2^8.
constexpr float kQueryLazy = 8.0f;

// One workgroup per unit, one wavefront per query head.  Groups of more
// than four heads (WIDE) are held to 128 VGPRs, four wavefronts per SIMD, so
// that two groups of up to eight wavefronts share a CU (R1-Distill-Qwen-7B
// shape, g = 7: 1.50 ms per call against 1.68 for two workgroups of four
// wavefronts per unit, whose second workgroup re-read the keys and values
// partly from HBM); smaller groups keep three per SIMD and more registers.
template <int D, int NL, bool WIDE>
__global__ __launch_bounds__(512, WIDE ? 4 : 1) void decode_kernel(DecodeArgs a, int g) {
    __shared__ __attribute__((aligned(16))) uint16_t k0[DT * D];
    __shared__ __attribute__((aligned(16))) uint16_t k1[DT * D];
    __shared__ __attribute__((aligned(16))) uint16_t k2[DT * D];
    __shared__ __attribute__((aligned(16))) uint16_t v0[DT * D];
    __shared__ __attribute__((aligned(16))) uint16_t v1[DT * D];
    __shared__ __attribute__((aligned(16))) uint16_t v2[DT * D];
    __shared__ double2 tab[2][D / 2];  // cos/sin at t_obs (beacons), at t_q (new query)
    constexpr int NPW = TileLoad<D, NL, DT>::NPW;
    constexpr int NS = D / 16;
    constexpr int NB = D / 16;  // 16-dim output blocks

    const int tid = threadIdx.x;
    const int h = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const bool loader = h < NL;
    const int64_t u = blockIdx.x;
    const int64_t qh = u * g + h;
    const int64_t L = a.L;
    const uint16_t* Ku = a.K + u * a.l_cap * D;
    const uint16_t* Vu = a.V + u * a.l_cap * D;
    const int ntiles = (int)((L + DT - 1) / DT);
    const bool obs = a.beacons != nullptr;
    const TileLoad<D, NL, DT> ld(h, lane);

    // The cos/sin pairs at t_obs and t_q (fp64), first, so that their
    // registers are free before the rows arrive.
    for (int e = tid; e < D; e += (int)blockDim.x) {
        const int which = e / (D / 2), k = e % (D / 2);
        double c, sn;
        rope_cs((double)(which == 0 ? a.t_obs : a.t_q), k, D, a.theta, &c, &sn);
        tab[which][k] = double2{c, sn};
    }
    // This lane's row (beacon r < 16, new query r == 16, zero beyond) is
    // loaded before the first two tiles of keys and values are issued, so
    // that waiting for it does not wait for the tiles.  Keys and values are
    // read once here: streaming (non-temporal) loads, 8% faster than plain
    // ones without the beacon rows.
    const int r = lane & 31, hh = lane >> 5;
    const float* src = nullptr;
    if (r < 16 && obs) src = a.beacons + (qh * a.buf_cap + r) * (int64_t)D;
    else if (r == 16 || r == 20) src = a.q + qh * (int64_t)D;
    float4 x1[NS / 2][2], x2[NS / 2][2];
#pragma unroll
    for (int s = 0; s < NS / 2; ++s) {
        const int k = 16 * s + 8 * hh;
        x1[s][0] = x1[s][1] = x2[s][0] = x2[s][1] = float4{0.f, 0.f, 0.f, 0.f};
        if (src) {
            x1[s][0] = *reinterpret_cast<const float4*>(src + k);
            x1[s][1] = *reinterpret_cast<const float4*>(src + k + 4);
            x2[s][0] = *reinterpret_cast<const float4*>(src + k + D / 2);
            x2[s][1] = *reinterpret_cast<const float4*>(src + k + D / 2 + 4);
        }
    }
    auto load_tile = [&](int64_t base, uint16_t* kd, uint16_t* vd) {
        ld.template issue<kLoadStreaming>(Ku, L, base, kd, h);
        ld.template issue<kLoadStreaming>(Vu, L, base, vd, h);
    };
    if (loader) {
        load_tile(0, k0, v0);
        if (1 < ntiles) load_tile(DT, k1, v1);
    }
    // A full barrier here and in the tile loop: with the LDS-only barrier the
    // decode kernel's beacon rows took 946 instead of 907 us (Qwen3-4B shape).
    __syncthreads();  // the cos/sin table

    // A fragments: rotate in fp64, round through fp32 to bf16 (zero rows
    // rotate to zero).
    bf16x8 frag[NS];
    {
        const double2* cs_tab = tab[(r == 16 || r == 20) ? 1 : 0];
#pragma unroll
        for (int s = 0; s < NS / 2; ++s) {
            const int k = 16 * s + 8 * hh;
            double2 csa[4], csb[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) { csa[p] = cs_tab[k + p]; csb[p] = cs_tab[k + 4 + p]; }
            const uint4 ra = rotate4(x1[s][0], x2[s][0], csa);
            const uint4 rb = rotate4(x1[s][1], x2[s][1], csb);
            frag[s] = __builtin_bit_cast(bf16x8, (uint4{ra.x, ra.y, rb.x, rb.y}));
            frag[s + NS / 2] = __builtin_bit_cast(bf16x8, (uint4{ra.z, ra.w, rb.z, rb.w}));
        }
    }
    // Byte offsets of this lane's key chunks for MFMA step s and of its value
    // transpose reads for block b are koff ^ 32 s and vto ^ 32 b (the XOR
    // swizzle permutes 16-byte chunks within a row).  The wide form forms
    // them per tile from the two bases rather than holding sixteen registers.
    const uint32_t koff = TileRead<D>(lane).off[0];
    const float c2 = a.c2;

    // Beacon rows (accumulators 0..7): running max and sum of exp2, lazily
    // rescaled as in the scoring's pass 1.  New query: running max m (in
    // log2 units, wave-uniform), per-lane partial sum ls and output o.
    float mc[8], l[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) { mc[v] = kNegBig; l[v] = 0.f; }
    float m = -__builtin_inff(), ls = 0.f;
    f32x4 pv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) pv[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t vto = vt_offset<D>(lane);
    // Source lane (times 4) of this lane's first weight pair: lane group q
    // takes keys 4 q .. 4 q + 3 and 16 + 4 q .. 16 + 4 q + 3, even rows the
    // high parts (lanes 0..31), odd rows the remainders (lanes 32..63).
    const int wsrc = 4 * ((lane & 1) * 32 + 4 * ((lane >> 4) & 3));

#define BKV_DEC_ITER(it, KC, VC, KN, VN)                                           \
    do {                                                                           \
        if (loader) {                                                              \
            if ((it) + 1 >= ntiles) wait_vm<0>();                                  \
            else wait_vm<2 * NPW>();                                               \
        }                                                                          \
        __syncthreads();                                                           \
        if (loader && (it) + 2 < ntiles) load_tile((int64_t)((it) + 2) * DT, KN, VN); \
        uint32_t kb = koff, vb = vto;                                              \
        if constexpr (WIDE) asm volatile("" : "+v"(kb), "+v"(vb));                 \
        f32x16 acc = f32x16{};                                                     \
        {                                                                          \
            const char* kt = reinterpret_cast<const char*>(KC);                    \
            _Pragma("unroll") for (int s = 0; s < NS; ++s) {                       \
                const uint4 w = *reinterpret_cast<const uint4*>(kt + (kb ^ (uint32_t)(32 * s))); \
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                     \
                    frag[s], __builtin_bit_cast(bf16x8, w), acc, 0, 0, 0);         \
            }                                                                      \
        }                                                                          \
        if ((int64_t)((it) + 1) * DT > L) {  /* only the last tile is partial */  \
            if ((int64_t)(it) * DT + (lane & 31) >= L) {                           \
                _Pragma("unroll") for (int v = 0; v < 16; ++v) acc[v] = -__builtin_inff(); \
            }                                                                      \
        }                                                                          \
        if (obs) {                                                                 \
            /* exponents against the running maxima; raise those only when a  \
               term would pass kRescaleBig (log2 64), then add the terms */    \
            float e[8];                                                            \
            float big = -__builtin_inff();                                         \
            _Pragma("unroll") for (int v = 0; v < 8; ++v) {                        \
                e[v] = fmaf(acc[v], c2, -mc[v]);                                   \
                big = vmax(big, e[v]);                                             \
            }                                                                      \
            if (__builtin_amdgcn_ballot_w64(!(big <= kRescaleExp)) != 0) {         \
                _Pragma("unroll") for (int v = 0; v < 8; ++v) {                    \
                    const float mn = vmax(mc[v], acc[v] * c2);                     \
                    l[v] *= exp2_sum(mc[v] - mn);                                  \
                    mc[v] = mn;                                                    \
                    e[v] = fmaf(acc[v], c2, -mn);                                  \
                }                                                                  \
            }                                                                      \
            _Pragma("unroll") for (int v = 0; v < 8; ++v) l[v] += exp2_sum(e[v]);  \
        }                                                                          \
        /* New query: logits in accumulator 8 (rows 16 and 20 of the block both \
           hold the query, so lanes j and 32 + j both have key j's logit). */  \
        const float x = acc[8] * c2;                                               \
        if (__builtin_amdgcn_ballot_w64(x > m + kQueryLazy) != 0) {                \
            float tm = x;                                                          \
            _Pragma("unroll") for (int o = 1; o < 32; o <<= 1) tm = vmax(tm, __shfl_xor(tm, o)); \
            const float mt = __builtin_bit_cast(float,                             \
                __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, tm)));      \
            const float alpha = exp2_sum(m - mt);                                  \
            m = mt;                                                                \
            ls *= alpha;                                                           \
            _Pragma("unroll") for (int b = 0; b < NB; ++b) pv[b] *= alpha;         \
        }                                                                          \
        const float p = exp2_sum(x - m);                                           \
        ls += p;  /* lanes 0..31 are summed at the end */                         \
        bf16x8 wa;                                                                 \
        {   /* lanes 0..31 hold the high parts, lanes 32..63 the remainders;      \
               even lanes pack keys j, j + 1, then the A operand is gathered */   \
            const uint32_t pb = __float_as_uint(p);                                \
            const uint32_t wb = lane < 32 ? pb                                     \
                : __float_as_uint(p - __uint_as_float(pb & 0xffff0000u));          \
            const uint32_t nb = (uint32_t)__builtin_amdgcn_mov_dpp((int)wb, 0xB1, 0xF, 0xF, false); \
            const int pk = (int)__builtin_amdgcn_perm(nb, wb, 0x07060302u);       \
            const uint4 g4 = uint4{(uint32_t)__builtin_amdgcn_ds_bpermute(wsrc, pk),      \
                                   (uint32_t)__builtin_amdgcn_ds_bpermute(wsrc + 8, pk),  \
                                   (uint32_t)__builtin_amdgcn_ds_bpermute(wsrc + 64, pk), \
                                   (uint32_t)__builtin_amdgcn_ds_bpermute(wsrc + 72, pk)};\
            wa = __builtin_bit_cast(bf16x8, g4);                                   \
        }                                                                          \
        {                                                                          \
            const char* vt = reinterpret_cast<const char*>(VC);                    \
            _Pragma("unroll") for (int b = 0; b < NB; ++b) {                       \
                const char* pa = vt + (vb ^ (uint32_t)(32 * b));                   \
                const i16x4 lo4 = lds_read_tr16(pa);                               \
                const i16x4 hi4 = lds_read_tr16(pa + 32 * D);                      \
                const bf16x8 vb = __builtin_bit_cast(bf16x8,                       \
                    __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));    \
                pv[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, vb, pv[b], 0, 0, 0); \
            }                                                                      \
        }                                                                          \
    } while (0)

    for (int it = 0; it < ntiles; it += 3) {
        BKV_DEC_ITER(it, k0, v0, k2, v2);
        if (it + 1 < ntiles) BKV_DEC_ITER(it + 1, k1, v1, k0, v0);
        if (it + 2 < ntiles) BKV_DEC_ITER(it + 2, k2, v2, k1, v1);
    }
#undef BKV_DEC_ITER

    // New query: total sum over the 32 lanes, then the output and its LSE.
    float lt = ls;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) lt += __shfl_xor(lt, o);
    lt = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, lt)));
    const float inv = 1.0f / lt;
    {
        const int q = (lane >> 4) & 3;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (b % 4 == q) a.out[qh * (int64_t)D + 16 * b + (lane & 15)] = (pv[b][0] + pv[b][1]) * inv;
    }
    constexpr float kLn2 = 0.6931471805599453f;
    if (lane == 0) a.lse_q[qh] = (m + log2f(lt)) * kLn2;
    if (obs) {
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const float m2 = __shfl_xor(mc[v], o);
                const float l2 = __shfl_xor(l[v], o);
                const float mm = fmaxf(mc[v], m2);
                l[v] = l[v] * exp2_sum(mc[v] - mm) + l2 * exp2_sum(m2 - mm);
                mc[v] = mm;
            }
        }
        if ((lane & 31) == 0) {
#pragma unroll
            for (int v = 0; v < 8; ++v)
                a.lse_obs[qh * 16 + acc_row(v, lane)] = (mc[v] + log2f(l[v])) * kLn2;
        }
    }
}

template __global__ void decode_kernel<128, 4, false>(DecodeArgs, int);
template __global__ void decode_kernel<128, 2, false>(DecodeArgs, int);
template __global__ void decode_kernel<128, 1, false>(DecodeArgs, int);
template __global__ void decode_kernel<64, 4, false>(DecodeArgs, int);
template __global__ void decode_kernel<64, 2, false>(DecodeArgs, int);
template __global__ void decode_kernel<64, 1, false>(DecodeArgs, int);
template __global__ void decode_kernel<128, 4, true>(DecodeArgs, int);
template __global__ void decode_kernel<64, 4, true>(DecodeArgs, int);

// Every variant is instantiated explicitly, so each gets its host launch stub
// even though it is launched from one branch of a conditional.
template __global__ void score_kernel<128, 4, false>(ScoreArgs, int);
template __global__ void score_kernel<128, 2, false>(ScoreArgs, int);
template __global__ void score_kernel<128, 1, false>(ScoreArgs, int);
template __global__ void score_kernel<64, 4, false>(ScoreArgs, int);
template __global__ void score_kernel<64, 2, false>(ScoreArgs, int);
template __global__ void score_kernel<64, 1, false>(ScoreArgs, int);
template __global__ void score_kernel<128, 4, true>(ScoreArgs, int);
template __global__ void score_kernel<128, 2, true>(ScoreArgs, int);
template __global__ void score_kernel<128, 1, true>(ScoreArgs, int);
template __global__ void score_kernel<64, 4, true>(ScoreArgs, int);
template __global__ void score_kernel<64, 2, true>(ScoreArgs, int);
template __global__ void score_kernel<64, 1, true>(ScoreArgs, int);
template __global__ void score_kernel<128, 4, false, 4>(ScoreArgs, int);
template __global__ void score_kernel<128, 4, true, 4>(ScoreArgs, int);
template __global__ void score_kernel<64, 4, false, 4>(ScoreArgs, int);
template __global__ void score_kernel<64, 4, true, 4>(ScoreArgs, int);

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
                        float sm_scale, bool mean, const double* table, float* score,
                        uint16_t* qobs_out, const float* lse_in, int64_t lse_from,
                        hipStream_t s) {
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
    a.qobs = qobs_out;
    a.lse_in = lse_in;
    a.lse_from = lse_from;
    a.n_units = n_units;
    // One workgroup per unit, one wavefront per query head.  Groups of 5 to 8
    // heads take the variant held to 128 VGPRs (four wavefronts per SIMD, its
    // spills confined to the rare running-maximum pass 1), so that two or
    // three workgroups share a CU: R1-Distill-Qwen-7B shape (g = 7) 2.50 ->
    // 2.05 ms and Qwen3-14B shape (g = 5) 2.94 -> 2.50 ms against splitting a
    // group over two workgroups, each of which read every key.
    a.inv_rows = 1.0f / (float)(g * 32);
    const bool capped = g >= 5;
    const dim3 grid((unsigned)n_units);
    const dim3 block(64 * g);
    // Loader wavefronts: the largest power of two <= g, at most 4.
    const int nl = g >= 4 ? 4 : (g >= 2 ? 2 : 1);
#define BKV_LAUNCH_M(DD, NN, MM)                                                   \
    do {                                                                           \
        if (capped) score_kernel<DD, 4, MM, 4><<<grid, block, 0, s>>>(a, g);       \
        else score_kernel<DD, NN, MM><<<grid, block, 0, s>>>(a, g);                \
    } while (0)
#define BKV_LAUNCH(DD, NN)                                                         \
    do {                                                                           \
        if (mean) BKV_LAUNCH_M(DD, NN, true);                                      \
        else BKV_LAUNCH_M(DD, NN, false);                                          \
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
#undef BKV_LAUNCH_M
    return hipGetLastError();
}

hipError_t launch_decode(const uint16_t* K, const uint16_t* V, int64_t n_units, int g, int d,
                         int64_t l_cap, int64_t L, const float* q, int64_t t_q,
                         const float* beacons, int buf_cap, int64_t t_obs, double theta,
                         float sm_scale, float* out, float* lse_q, float* lse_obs,
                         hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    DecodeArgs a;
    a.K = K;
    a.V = V;
    a.l_cap = l_cap;
    a.L = L;
    a.q = q;
    a.t_q = t_q;
    a.beacons = beacons;
    a.buf_cap = buf_cap;
    a.t_obs = t_obs;
    a.theta = theta;
    a.c2 = sm_scale * 1.4426950408889634f;
    a.out = out;
    a.lse_q = lse_q;
    a.lse_obs = lse_obs;
    a.n_units = n_units;
    // Groups of more than four heads: the 128-VGPR form (see decode_kernel).
    const bool wide = g > 4;
    const dim3 grid((unsigned)n_units);
    const dim3 block(64 * g);
    const int nl = g >= 4 ? 4 : (g >= 2 ? 2 : 1);
#define BKV_LAUNCH_DEC(DD, NN, WW) decode_kernel<DD, NN, WW><<<grid, block, 0, s>>>(a, g)
    if (d == 128) {
        if (wide) BKV_LAUNCH_DEC(128, 4, true);
        else if (nl == 4) BKV_LAUNCH_DEC(128, 4, false);
        else if (nl == 2) BKV_LAUNCH_DEC(128, 2, false);
        else BKV_LAUNCH_DEC(128, 1, false);
    } else {
        if (wide) BKV_LAUNCH_DEC(64, 4, true);
        else if (nl == 4) BKV_LAUNCH_DEC(64, 4, false);
        else if (nl == 2) BKV_LAUNCH_DEC(64, 2, false);
        else BKV_LAUNCH_DEC(64, 1, false);
    }
#undef BKV_LAUNCH_DEC
    return hipGetLastError();
}

}  // namespace bkv
