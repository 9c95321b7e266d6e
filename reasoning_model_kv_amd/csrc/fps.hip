// Continual-FPS fill-and-compress of the per-head pre-RoPE query buffers.
//
// Paper text §4.2 ("Continual FPS") and App. D.1 (Algorithm 1, FPS):
// average cosine similarity picks the seed (lowest), then the row whose
// largest cosine to the picked set is lowest joins it, until m rows remain.
//
// Mapping.  Buffers of up to 32 rows: one wavefront per query head forms
// the 32 x 32 cosine matrix once on bf16 MFMAs (each fp32 value split into
// a high and a low bf16 part) and runs the greedy picks on it (see
// fps_wave_kernel).  Buffers of up to 256 rows (prefill) use one
// workgroup per head and one thread per row; there the average cosine of
// row i uses the sum of all normalised rows (sum_j cos(q_i, q_j) equals
// q_i/|q_i| . sum_j q_j/|q_j|) and each pick broadcasts the new member's
// row through LDS.  Longer buffers (up to 8192 rows) are read in three full
// passes, after which the greedy runs lazily on a shortlist of rows gathered
// from memory (fps_long_kernel).
//
// Arithmetic is fp32; ties go to the lower slot.

#include <algorithm>

#include "common.h"

namespace bkv {
namespace {

constexpr float kNormFloor = 1e-12f;

__device__ __forceinline__ void argmin_pair(float& v, int& i, float ov, int oi) {
    if (ov < v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}

// Cross-lane moves for the wavefront reductions: DPP within rows of 16
// lanes, a bitmask swizzle for lane ^ 16 within 32.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, x)));
}
__device__ __forceinline__ int swap16_i(int x) { return __builtin_amdgcn_ds_swizzle(x, 0x401F); }
__device__ __forceinline__ float swap16_f(float x) {
    return __builtin_bit_cast(float, swap16_i(__builtin_bit_cast(int, x)));
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// Eight fp32 values split into bf16 high parts (the top 16 bits, exact) and
// low parts (the remainder, exact in fp32, rounded to bf16): hi + lo equals
// each value to within 2^-16 of it.  Packed in dimension order.
__device__ __forceinline__ void split_bf16(const float* v, uint4& hi, uint4& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t b0 = __float_as_uint(v[2 * i]), b1 = __float_as_uint(v[2 * i + 1]);
        h[i] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
        const f32x2 r = {v[2 * i] - __uint_as_float(b0 & 0xFFFF0000u),
                         v[2 * i + 1] - __uint_as_float(b1 & 0xFFFF0000u)};
        l[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
    }
    hi = uint4{h[0], h[1], h[2], h[3]};
    lo = uint4{l[0], l[1], l[2], l[3]};
}

// A candidate as one 32-bit key that orders like (value, row): the float's
// bits made monotone (larger value, larger key), the low 5 mantissa bits
// replaced by the row (0..31).  Values within 32 ulps (2^-18 relative)
// compare equal and go to the lower row, well inside the method's
// tolerance and about the size of the fp32 cosines' own rounding.
// kNoCandidate is larger than every real key (+inf included).
constexpr uint32_t kNoCandidate = 0xFFFFFFFFu;
__device__ __forceinline__ uint32_t pick_key(float v, int row) {
    uint32_t b = __float_as_uint(v);
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return (b & ~31u) | (uint32_t)row;
}

// Minimum key over each 32-lane half (both halves hold the same 32
// candidates), one v_min_u32 per step with the cross-lane move as its DPP
// operand where the compiler can fold it; returns the winning row.
__device__ __forceinline__ int half_argmin_key(uint32_t k) {
    k = min(k, (uint32_t)dpp_i<0xB1>((int)k));
    k = min(k, (uint32_t)dpp_i<0x4E>((int)k));
    k = min(k, (uint32_t)dpp_i<0x141>((int)k));
    k = min(k, (uint32_t)dpp_i<0x140>((int)k));
    k = min(k, (uint32_t)swap16_i((int)k));
    return __builtin_amdgcn_readlane((int)k, 0) & 31;
}

// Buffers of up to 32 rows: one wavefront per query head.
//  * Lane pair (2r, 2r+1) loads row r (half of its d fp32 values each) into
//    registers, where the rows stay until the kept ones are written back.
//  * The unit-normalised rows go to LDS row-major, one half of the dims at a
//    time, each value split into bf16 high and low parts (hi + lo within
//    2^-16 of it), and the 32 x 32 cosine matrix C = Qn Qn^T is formed as
//    Hi Hi^T + Hi Lo^T + Lo Hi^T on bf16 MFMAs (v_mfma_f32_32x32x16_bf16,
//    fp32 accumulate; lane l supplies row l % 32, dims 16 s + 8 (l / 32) ..
//    + 8 of step s, which serve as both operands since C = Qn Qn^T): 3 d/16
//    MFMAs instead of the d/2 of 32x32x2 fp32 ones.  The dropped Lo Lo^T
//    term and the rounding leave each cosine within about 2^-15 of fp32.
//  * Lane l then stands for row l % 32.  The average cosine of row j is the
//    sum of column j of C (C is symmetric) over N; the seed is its argmin.
//    Each further pick p adds column p of C (one LDS read per lane) to the
//    running max S, and the next pick is the argmin of S over the rows not
//    yet picked.
//  * The kept rows leave through LDS, eight at a time, as contiguous stores.
//  LDS stays at about 8 KB (d = 128) and registers at 128 or fewer, so 16
//  wavefronts share a CU.
template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void fps_wave_kernel(
    float* __restrict__ buf, int32_t* __restrict__ count,
    const float* __restrict__ new_q, int n_new, int64_t qhs, int64_t qrs, int cap, int trigger,
    int m, int32_t* __restrict__ sel_order, int32_t* __restrict__ n_overflow) {
    constexpr int HD = D / 2;   // dims held by one lane of a pair
    constexpr int TS = 33;      // LDS stride (floats) of the transposed rows and of C
    constexpr int RS = D + 4;   // LDS stride (floats) of a staged output row
    constexpr int C4 = D / 4;   // 16-byte chunks per row
    constexpr int SR = 8;       // output rows staged per write-back round
    constexpr int LDSF = HD * TS;
    static_assert(LDSF >= 32 * TS && LDSF >= SR * RS, "LDS reuse");
    // In turn: Qn^T of one half of the dims (qt[dim * TS + row]), C
    // (qt[i * TS + j]), and output rows (qt[r * RS + dim]) for the write-back.
    // Half the transposed rows at a time keeps the footprint at 8 KB (d = 128).
    __shared__ __attribute__((aligned(16))) float qt[LDSF];

    const int lane = threadIdx.x;
    const int64_t head = blockIdx.x;
    const int row = lane >> 1;
    const int half = lane & 1;
    float* hb = buf + head * (int64_t)cap * D;
    const float* nq = new_q ? new_q + head * qhs : nullptr;  // row r at nq + r * qrs

    const int cnt = count[head];
    const int N = cnt + n_new;
    const bool compress = (cnt >= 0 && N <= cap && N >= trigger && N > m);
    if (sel_order && !compress && lane < m) sel_order[head * m + lane] = -1;
    if (cnt < 0 || N > cap) {
        if (lane == 0 && n_overflow) atomicAdd(n_overflow, 1);
        return;
    }
    if (!compress) {
        // Append only.
        for (int e = lane * 4; e < n_new * D; e += 64 * 4)
            *reinterpret_cast<float4*>(hb + (int64_t)cnt * D + e) =
                *reinterpret_cast<const float4*>(nq + (int64_t)(e / D) * qrs + e % D);
        if (lane == 0) count[head] = N;
        return;
    }

    // Load this lane's half row (rows >= N are padding); all 16-byte loads
    // of a lane are in flight together.
    float x[HD];
    const bool valid = row < N;
    if (valid) {
        const float* src = row < cnt ? hb + (int64_t)row * D : nq + (int64_t)(row - cnt) * qrs;
        src += half * HD;
#pragma unroll
        for (int k = 0; k < HD; k += 4) {
            float4 f = *reinterpret_cast<const float4*>(src + k);
            x[k] = f.x; x[k + 1] = f.y; x[k + 2] = f.z; x[k + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < HD; ++k) x[k] = 0.f;
    }

    float nn = 0.f;
#pragma unroll
    for (int k = 0; k < HD; ++k) nn = fmaf(x[k], x[k], nn);
    nn += dpp_f<0xB1>(nn);  // the lane pair's other half (quad_perm [1,0,3,2])
    const float inv = 1.0f / fmaxf(sqrtf(nn), kNormFloor);

    // C over two rounds, one per half of the dims: the lanes holding that half
    // store it (hi and lo parts, rows of HD bf16 each, 16-byte chunks
    // XOR-swizzled by row so the fragment reads spread over the banks), then
    // 3 * HD / 16 MFMAs add it.  Lane l ends with C[i][l % 32] for
    // i = 8 (v / 4) + 4 (l / 32) + v % 4.
    const int r32 = lane & 31;
    const int kk = lane >> 5;
    constexpr int CH = HD / 8;  // 16-byte chunks per half row
    uint4* qh4 = reinterpret_cast<uint4*>(qt);           // hi parts: [32][CH]
    uint4* ql4 = reinterpret_cast<uint4*>(qt) + 32 * CH;  // lo parts: [32][CH]
    static_assert(2 * 32 * CH * 16 <= LDSF * 4, "hi/lo halves fit the LDS buffer");
    f32x16 acc = f32x16{};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        if (hf) wave_sync_lds();  // the first round's operand reads are done
        if (half == hf) {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = x[8 * c + e] * inv;
                uint4 h4, l4;
                split_bf16(v, h4, l4);
                const int pc = row * CH + (c ^ (row % CH));
                qh4[pc] = h4;
                ql4[pc] = l4;
            }
        }
        wave_sync_lds();
#pragma unroll
        for (int st = 0; st < HD / 16; ++st) {
            const int pc = r32 * CH + ((2 * st + kk) ^ (r32 % CH));
            const bf16x8 a = __builtin_bit_cast(bf16x8, qh4[pc]);
            const bf16x8 b = __builtin_bit_cast(bf16x8, ql4[pc]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc, 0, 0, 0);
        }
    }
    float colsum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) colsum += acc[v];
    colsum += __shfl_xor(colsum, 32);  // the other 16 rows of the column
    wave_sync_lds();                   // every operand read of Qn^T is done
#pragma unroll
    for (int v = 0; v < 16; ++v) qt[(8 * (v >> 2) + 4 * kk + (v & 3)) * TS + r32] = acc[v];
    wave_sync_lds();

    // Lane l stands for row l % 32 from here on.
    const bool valid32 = r32 < N;
    int pick = half_argmin_key(valid32 ? pick_key(colsum / (float)N, r32) : kNoCandidate);
    uint32_t sel = 1u << pick;
    int my_pick = (lane == 0) ? pick : -1;
    float S = qt[pick * TS + r32];
    for (int it = 1; it < m; ++it) {
        const bool cand = valid32 && !((sel >> r32) & 1u);
        pick = half_argmin_key(cand ? pick_key(S, r32) : kNoCandidate);
        sel |= 1u << pick;
        if (lane == it) my_pick = pick;
        S = fmaxf(S, qt[pick * TS + r32]);
    }

    // Keep the picked rows in ascending slot order: SR output rows at a time
    // go from registers to LDS (in C's place), then out with contiguous
    // 16-byte stores.  Every row was loaded before any store.
    const int dst = ((sel >> row) & 1u) ? __popc(sel & ((1u << row) - 1u)) : -1;
    for (int r0 = 0; r0 < m; r0 += SR) {
        wave_sync_lds();  // C's last reads, or the previous round's stores
        if (dst >= r0 && dst < r0 + SR) {
#pragma unroll
            for (int k = 0; k < HD; k += 4)
                *reinterpret_cast<float4*>(qt + (dst - r0) * RS + half * HD + k) =
                    make_float4(x[k], x[k + 1], x[k + 2], x[k + 3]);
        }
        wave_sync_lds();
        const int nrow = m - r0 < SR ? m - r0 : SR;
        for (int id = lane; id < nrow * C4; id += 64) {
            const int r = id / C4, c4 = id % C4;
            *reinterpret_cast<float4*>(hb + (int64_t)(r0 + r) * D + 4 * c4) =
                *reinterpret_cast<const float4*>(qt + r * RS + 4 * c4);
        }
    }
    if (sel_order && lane < m) sel_order[head * m + lane] = my_pick;
    if (lane == 0) count[head] = m;
}

// One workgroup per head, one thread per row (rows up to 256).
template <int D>
__global__ __launch_bounds__(256) void fps_block_kernel(
    float* __restrict__ buf, int32_t* __restrict__ count,
    const float* __restrict__ new_q, int n_new, int64_t qhs, int64_t qrs, int cap, int trigger,
    int m, int32_t* __restrict__ sel_order, int32_t* __restrict__ n_overflow) {
    __shared__ float svec[D];
    __shared__ float bc[D];
    __shared__ float inv_s[256];
    __shared__ float red_v[4];
    __shared__ int red_i[4];
    __shared__ int rank_s[4];
    __shared__ int pick_s;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int64_t head = blockIdx.x;
    float* hb = buf + head * (int64_t)cap * D;
    const float* nq = new_q ? new_q + head * qhs : nullptr;  // row r at nq + r * qrs

    const int cnt = count[head];
    const int N = cnt + n_new;
    const bool compress = (cnt >= 0 && N <= cap && N >= trigger && N > m);
    if (sel_order && !compress && tid < m) sel_order[head * m + tid] = -1;
    if (cnt < 0 || N > cap) {
        if (tid == 0 && n_overflow) atomicAdd(n_overflow, 1);
        return;
    }
    if (!compress) {
        for (int e = tid * 4; e < n_new * D; e += 256 * 4)
            *reinterpret_cast<float4*>(hb + (int64_t)cnt * D + e) =
                *reinterpret_cast<const float4*>(nq + (int64_t)(e / D) * qrs + e % D);
        if (tid == 0) count[head] = N;
        return;
    }

    auto row_ptr = [&](int j) -> const float* {
        return j < cnt ? hb + (int64_t)j * D : nq + (int64_t)(j - cnt) * qrs;
    };

    const int row = tid;
    const bool valid = row < N;
    float x[D];
    if (valid) {
        const float* src = row_ptr(row);
#pragma unroll
        for (int k = 0; k < D; k += 4) {
            float4 f = *reinterpret_cast<const float4*>(src + k);
            x[k] = f.x; x[k + 1] = f.y; x[k + 2] = f.z; x[k + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < D; ++k) x[k] = 0.f;
    }
    float nn = 0.f;
#pragma unroll
    for (int k = 0; k < D; ++k) nn = fmaf(x[k], x[k], nn);
    const float inv = 1.0f / fmaxf(sqrtf(nn), kNormFloor);
    inv_s[tid] = inv;
    __syncthreads();
    for (int k = tid; k < D; k += 256) {
        float s = 0.f;
        for (int j = 0; j < N; ++j) s += row_ptr(j)[k] * inv_s[j];
        svec[k] = s;
    }
    __syncthreads();

    auto dot_with = [&](const float* v) {
        float a = 0.f;
#pragma unroll
        for (int k = 0; k < D; ++k) a = fmaf(x[k], v[k], a);
        return a * inv;
    };
    auto block_argmin = [&](float v) -> int {
        int i = row;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            float ov = __shfl_xor(v, o);
            int oi = __shfl_xor(i, o);
            argmin_pair(v, i, ov, oi);
        }
        if (lane == 0) { red_v[wave] = v; red_i[wave] = i; }
        __syncthreads();
        if (tid == 0) {
            float bv = red_v[0];
            int bi = red_i[0];
            for (int w = 1; w < 4; ++w) argmin_pair(bv, bi, red_v[w], red_i[w]);
            pick_s = bi;
        }
        __syncthreads();
        return pick_s;
    };
    auto broadcast_row = [&](int r) {
        if (row == r) {
#pragma unroll
            for (int k = 0; k < D; ++k) bc[k] = x[k] * inv;
        }
        __syncthreads();
    };

    const float inf = __builtin_inff();
    const float avg = dot_with(svec) / (float)N;
    int pick = block_argmin(valid ? avg : inf);
    bool selected = (row == pick);
    if (sel_order && tid == 0) sel_order[head * m] = pick;
    broadcast_row(pick);
    float S = dot_with(bc);
    for (int it = 1; it < m; ++it) {
        __syncthreads();  // everyone has read bc
        pick = block_argmin((valid && !selected) ? S : inf);
        if (row == pick) selected = true;
        if (sel_order && tid == 0) sel_order[head * m + it] = pick;
        broadcast_row(pick);
        S = fmaxf(S, dot_with(bc));
    }

    // Rank of each selected row among the selected rows, in slot order.
    const unsigned long long bal = __ballot(selected);
    const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) rank_s[wave] = __popcll(bal);
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += rank_s[w];
    if (selected) {
        float* dst = hb + (int64_t)(base + in_wave) * D;
#pragma unroll
        for (int k = 0; k < D; k += 4)
            *reinterpret_cast<float4*>(dst + k) = make_float4(x[k], x[k + 1], x[k + 2], x[k + 3]);
    }
    if (tid == 0) count[head] = m;
}

// Buffers of more than 256 rows (up to kLongCap; the prefill FPS over a
// long prompt, or FPS over a whole query history): one workgroup of
// kLongThreads per head, with the rows left in memory.  A wavefront
// instruction reads RPI = 64 / (D/4) whole rows, one float4 per lane, and a
// row's dot products reduce over its D/4 lanes with xor shuffles; a row's
// norm is re-formed from the same loads wherever the row is read.
//  * pass 1: the sum of the normalised rows (then the average cosine of row
//    i is q_i/|q_i| . sum / N, as in fps_block_kernel);
//  * pass 2: the average cosines; the seed is their argmin;
//  * pass 3: every row's cosine with the seed.
// From then on each row keeps in LDS a lower bound lb of its S (its largest
// cosine to the picked set): the largest cosine over the ep picks applied
// to it so far.  The greedy's next pick, the row of least (S, slot), is
// found lazily.  The kShort rows of least (lb, slot) form a shortlist whose
// bound T is the least (lb, slot) outside it; their rows are gathered into
// registers and take the cosines with the picks they lack, so their S are
// exact.  Every row outside has S >= lb and (lb, slot) >= T, so while the
// least (S, slot) of the shortlist is below T it is the greedy's pick; the
// shortlist rows then take the new pick's cosine and the test repeats.
// Once it fails, the bounds go back to LDS and a new shortlist is formed.
// Each (row, pick) cosine is formed once, in the same fp32 arithmetic as a
// pass over all rows would form it, so the picks are those of the plain
// greedy over these cosines.  The shortlist's bound comes from a radix
// select over (lb, slot) keys in LDS, stopped as soon as at least
// kShort / 2 rows fall below a digit boundary.  The picked rows' normalised
// rows stay in LDS (pick rows [m][D]) for the gathers.
constexpr int kLongCap = 8192;
constexpr int kLongM = 64;
constexpr int kLongThreads = 512;
constexpr int kLongWaves = kLongThreads / 64;
constexpr int kShort = 128;        // shortlist rows
constexpr uint32_t kPicked = 0xff;  // ep of a picked row

// (value, slot) as one 45-bit key that orders like the pair: the float's
// bits made monotone (-0 folded onto +0), then the slot (below 2^13).
__device__ __forceinline__ uint64_t order_key(float v, int j) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0;
    u ^= (u >> 31) ? 0xffffffffu : 0x80000000u;
    return ((uint64_t)u << 13) | (uint32_t)j;
}

// The value of the lane that differs from this one in bit b of its index
// within 32.  The DPP mirror pairings differ in bits 2 and 3 (and in the
// bits below), so every step pairs lanes by XOR with a constant and a
// reduction over steps 0..4 leaves the same result in all 32 lanes.
__device__ __forceinline__ int lane_xchg_i(int x, int b) {
    switch (b) {
        case 0: return dpp_i<0xB1>(x);   // quad_perm [1,0,3,2]
        case 1: return dpp_i<0x4E>(x);   // quad_perm [2,3,0,1]
        case 2: return dpp_i<0x141>(x);  // row_half_mirror
        case 3: return dpp_i<0x140>(x);  // row_mirror
        default: return swap16_i(x);
    }
}
__device__ __forceinline__ float lane_xchg(float x, int b) {
    return __builtin_bit_cast(float, lane_xchg_i(__builtin_bit_cast(int, x), b));
}

// Least value over the wavefront, returned as a wavefront-uniform value.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
    for (int b = 0; b < 5; ++b) x = min(x, (uint32_t)lane_xchg_i((int)x, b));
    return min((uint32_t)__builtin_amdgcn_readlane((int)x, 0),
               (uint32_t)__builtin_amdgcn_readlane((int)x, 32));
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t x) {
#pragma unroll
    for (int b = 0; b < 5; ++b) {
        const uint64_t y = ((uint64_t)(uint32_t)lane_xchg_i((int)(x >> 32), b) << 32) |
                           (uint32_t)lane_xchg_i((int)x, b);
        x = y < x ? y : x;
    }
    const uint64_t a = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), 0) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
    const uint64_t c = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), 32) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
    return c < a ? c : a;
}

// Sums of NI rows' partial sums over the C4 lanes that hold each row: a
// reduce-scatter (each step trades half of the values with the partner lane
// and adds) leaves row i's total in the C4/NI lanes with c4 / (C4/NI) == i.
template <int C4, int NI>
__device__ __forceinline__ float rows_sum_scatter(float (&v)[NI], int c4) {
    constexpr int LC4 = __builtin_ctz(C4), LNI = __builtin_ctz(NI);
#pragma unroll
    for (int s = 0; s < LNI; ++s) {
        const int b = LC4 - 1 - s, h = NI >> (s + 1);
        const bool hi = (c4 >> b) & 1;
#pragma unroll
        for (int k = 0; k < h; ++k) {
            float lo_v = v[k], hi_v = v[k + h];
            // Values, not array slots: keeps the choice below a register
            // select instead of a run-time index into v.
            asm volatile("" : "+v"(lo_v), "+v"(hi_v));
            const float send = hi ? lo_v : hi_v;
            const float keep = hi ? hi_v : lo_v;
            v[k] = keep + lane_xchg(send, b);
        }
    }
    float x = v[0];
#pragma unroll
    for (int b = LC4 - LNI - 1; b >= 0; --b) x += lane_xchg(x, b);
    return x;
}

// At most 80 VGPRs (six wavefronts per SIMD): three workgroups per CU, so
// that one workgroup's shortlist work overlaps the others' passes.
template <int D>
__global__ __launch_bounds__(kLongThreads, 6) void fps_long_kernel(
    float* __restrict__ buf, int32_t* __restrict__ count, const float* __restrict__ new_q,
    int n_new, int cap, int trigger, int m, int32_t* __restrict__ sel_order,
    int32_t* __restrict__ n_overflow) {
    extern __shared__ float dyn[];  // pick rows [m][D], then lb [cap], then ep [cap] bytes
    __shared__ float bc[D];
    __shared__ float part[kLongWaves][D];
    __shared__ uint32_t hist[256];
    __shared__ int eidx[kShort];
    __shared__ uint64_t red_k[kLongWaves];
    __shared__ float red_v[kLongWaves];
    __shared__ int red_i[kLongWaves];
    __shared__ int picks[kLongM];
    __shared__ int sh_n;
    __shared__ uint32_t sh_digit, sh_below;
    constexpr int NT = kLongThreads, NW = kLongWaves;
    constexpr int C4 = D / 4;                // float4 chunks per row
    constexpr int RPI = 64 / C4;             // rows per wavefront instruction
    constexpr int STEP = NW * RPI;           // rows per pass iteration of the workgroup
    constexpr int NI = kShort / NW / RPI;    // shortlist rows per lane group
    constexpr int U = 4;                     // row loads in flight per lane in a pass
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int sub = lane / C4, c4 = lane % C4;
    const int64_t head = blockIdx.x;
    float* hb = buf + head * (int64_t)cap * D;
    const float* nq = new_q ? new_q + head * (int64_t)n_new * D : nullptr;

    const int cnt = count[head];
    const int N = cnt + n_new;
    const bool compress = (cnt >= 0 && N <= cap && N >= trigger && N > m);
    if (sel_order && !compress)
        for (int i = tid; i < m; i += NT) sel_order[head * m + i] = -1;
    if (cnt < 0 || N > cap) {
        if (tid == 0 && n_overflow) atomicAdd(n_overflow, 1);
        return;
    }
    if (!compress) {
        for (int e = tid * 4; e < n_new * D; e += NT * 4)
            *reinterpret_cast<float4*>(hb + (int64_t)cnt * D + e) =
                *reinterpret_cast<const float4*>(nq + e);
        if (tid == 0) count[head] = N;
        return;
    }
    float* P = dyn;
    float* lb = dyn + min(m, kLongM) * D;
    uint8_t* ep = reinterpret_cast<uint8_t*>(lb + cap);

    auto row_ptr = [&](int j) -> const float* {
        return j < cnt ? hb + (int64_t)j * D : nq + (int64_t)(j - cnt) * D;
    };
    auto load4 = [&](int j) -> float4 {
        return (j >= 0 && j < N) ? *reinterpret_cast<const float4*>(row_ptr(j) + 4 * c4)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    auto row_sum = [&](float x) {  // over the C4 lanes of a row, the same in each
#pragma unroll
        for (int b = 0; (1 << b) < C4; ++b) x += lane_xchg(x, b);
        return x;
    };
    auto dot4 = [](float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; };
    auto inv_norm = [&](float4 v) {
        return 1.0f / fmaxf(sqrtf(row_sum(dot4(v, v))), kNormFloor);
    };
    // A pass over all rows, U row loads in flight per lane.
    auto stream = [&](auto&& body) {
        for (int j0 = wave * RPI + sub; j0 < N + sub; j0 += U * STEP) {
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = load4(j0 + u * STEP);
#pragma unroll
            for (int u = 0; u < U; ++u) body(j0 + u * STEP, v[u]);
        }
    };
    // (value, index) argmin where index kNone means "no candidate": any
    // candidate beats none, so the result is a real row even if every value
    // is NaN (garbage in, but never an index out of range).
    constexpr int kNone = 0x7fffffff;
    auto take = [](float& v, int& i, float ov, int oi) {
        if (oi != kNone && (i == kNone || ov < v || (ov == v && oi < i))) {
            v = ov;
            i = oi;
        }
    };
    auto block_argmin = [&](float v, int i) -> int {
#pragma unroll
        for (int b = 0; b < 5; ++b) take(v, i, lane_xchg(v, b), lane_xchg_i(i, b));
        const float v32 = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
        const int i32 = __builtin_amdgcn_readlane(i, 32);
        if (lane == 0) {
            take(v, i, v32, i32);
            red_v[wave] = v;
            red_i[wave] = i;
        }
        __syncthreads();
        float bv = red_v[0];
        int bi = red_i[0];
        for (int w = 1; w < NW; ++w) take(bv, bi, red_v[w], red_i[w]);
        __syncthreads();  // red_* are free again
        return bi;
    };
    const float inf = __builtin_inff();

    // Pass 1: sum of the normalised rows.
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    stream([&](int j, float4 v) {
        const float inv = inv_norm(v);
        if (j < N) {
            acc.x = fmaf(v.x, inv, acc.x);
            acc.y = fmaf(v.y, inv, acc.y);
            acc.z = fmaf(v.z, inv, acc.z);
            acc.w = fmaf(v.w, inv, acc.w);
        }
    });
#pragma unroll
    for (int o = C4; o < 64; o <<= 1) {
        acc.x += __shfl_xor(acc.x, o);
        acc.y += __shfl_xor(acc.y, o);
        acc.z += __shfl_xor(acc.z, o);
        acc.w += __shfl_xor(acc.w, o);
    }
    if (sub == 0) *reinterpret_cast<float4*>(&part[wave][4 * c4]) = acc;
    __syncthreads();
    if (tid < D) {
        float s = part[0][tid];
        for (int w = 1; w < NW; ++w) s += part[w][tid];
        bc[tid] = s;
    }
    __syncthreads();

    // Pass 2: average cosines; the seed is their argmin.
    const float invN = 1.0f / (float)N;
    float bv = inf;
    int bi = kNone;
    {
        const float4 sv = *reinterpret_cast<const float4*>(&bc[4 * c4]);
        stream([&](int j, float4 v) {
            const float inv = inv_norm(v);
            const float a = row_sum(dot4(v, sv)) * inv * invN;
            if (j < N) take(bv, bi, a, j);
        });
    }
    const int seed = block_argmin(bv, bi);
    if (tid == 0) {
        picks[0] = seed;
        if (sel_order) sel_order[head * m] = seed;
    }
    if (wave == 0) {  // the seed's normalised row
        const float4 v = sub == 0 ? *reinterpret_cast<const float4*>(row_ptr(seed) + 4 * c4)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
        const float inv = inv_norm(v);
        if (sub == 0)
            *reinterpret_cast<float4*>(&P[4 * c4]) =
                make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
    }
    __syncthreads();

    // Pass 3: every row's cosine with the seed.
    {
        const float4 b4 = *reinterpret_cast<const float4*>(&P[4 * c4]);
        stream([&](int j, float4 v) {
            const float inv = inv_norm(v);
            const float c = row_sum(dot4(v, b4)) * inv;
            if (j < N && c4 == 0) {
                lb[j] = fmaxf(-inf, c);  // a NaN cosine leaves -inf
                ep[j] = j == seed ? kPicked : 1;
            }
        });
    }
    __syncthreads();

    // A refill that makes no pick brings at least one stale row up to date
    // (were every shortlist row current, its least key would be below T), so
    // there are at most N + 1 refills per pick; the cap only guarantees that
    // the workgroup finishes whatever its input.
    int npk = 1;
    const int64_t refill_cap = (int64_t)m * (N + 1);
    for (int64_t refills = 0; npk < m && refills < refill_cap; ++refills) {
        // The shortlist bound T (exclusive) over the keys of the unpicked
        // rows: the kShort-th least key, or an earlier digit boundary with at
        // least kShort / 2 keys below it.  8-bit digits from the top.
        uint64_t T = ~0ull;
        if (N - npk > kShort) {
            uint64_t prefix = 0;
            uint32_t rank = kShort, below = 0;
            int sh = 45;
            while (sh > 0) {
                const int width = sh >= 8 ? 8 : sh;
                sh -= width;
                if (tid < 256) hist[tid] = 0;
                __syncthreads();
                for (int j = tid; j < N; j += NT) {
                    if (ep[j] == kPicked) continue;
                    const uint64_t k = order_key(lb[j], j);
                    if ((k >> (sh + width)) == prefix)
                        atomicAdd(&hist[(uint32_t)(k >> sh) & ((1u << width) - 1)], 1u);
                }
                __syncthreads();
                if (wave == 0) {  // the bin that holds rank `rank`
                    uint32_t h[4], s = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        h[q] = hist[4 * lane + q];
                        s += h[q];
                    }
                    // Inclusive scan: within rows of 16 lanes by DPP row
                    // shifts (lanes shifted in from outside the row read 0),
                    // then the totals of the rows below.
                    uint32_t incl = s;
                    incl += (uint32_t)dpp_i<0x111>((int)incl);  // row_shr:1
                    incl += (uint32_t)dpp_i<0x112>((int)incl);  // row_shr:2
                    incl += (uint32_t)dpp_i<0x114>((int)incl);  // row_shr:4
                    incl += (uint32_t)dpp_i<0x118>((int)incl);  // row_shr:8
                    const uint32_t r0 = __builtin_amdgcn_readlane((int)incl, 15);
                    const uint32_t r1 = __builtin_amdgcn_readlane((int)incl, 31);
                    const uint32_t r2 = __builtin_amdgcn_readlane((int)incl, 47);
                    const int row16 = lane >> 4;
                    incl += (row16 >= 1 ? r0 : 0u) + (row16 >= 2 ? r1 : 0u) + (row16 >= 3 ? r2 : 0u);
                    uint32_t c = incl - s;
                    if (c <= rank && rank < incl) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            if (rank < c + h[q]) {
                                sh_digit = 4 * lane + q;
                                sh_below = c;
                                break;
                            }
                            c += h[q];
                        }
                    }
                }
                __syncthreads();
                const uint32_t dg = __builtin_amdgcn_readfirstlane(sh_digit);
                const uint32_t cb = __builtin_amdgcn_readfirstlane(sh_below);
                prefix = (prefix << width) | dg;
                below += cb;
                rank -= cb;
                if (below >= kShort / 2) break;
            }
            T = prefix << sh;
        }
        if (tid == 0) sh_n = 0;
        __syncthreads();
        for (int j = tid; j < N; j += NT) {
            if (ep[j] != kPicked && order_key(lb[j], j) < T) {
                const int s = atomicAdd(&sh_n, 1);
                if (s < kShort) eidx[s] = j;
            }
        }
        __syncthreads();
        const int ne = __builtin_amdgcn_readfirstlane(min(sh_n, kShort));

        // Gather the shortlist rows and apply the picks each one lacks.  Lane
        // group `sub` holds rows i = 0..NI-1 of its share in er[i]; the
        // bookkeeping of row i (slot, S, 1/|q|, picks applied) sits in the G
        // lanes with c4 / G == i, where rows_sum_scatter leaves its sums.
        constexpr int G = C4 / NI;
        const int my_row = c4 / G;
        float4 er[NI];
        int my_j = -1, my_ep = npk;
        float my_s = inf, my_inv;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int s = (wave * NI + i) * RPI + sub;
            const int j = s < ne ? eidx[s] : -1;
            er[i] = load4(j);
            if (my_row == i) my_j = j;
        }
        if (my_j >= 0) {
            my_ep = ep[my_j];
            my_s = lb[my_j];
        }
        const int emin = (int)wave_min_u32((uint32_t)my_ep);
        {
            float t[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) t[i] = dot4(er[i], er[i]);
            my_inv = 1.0f / fmaxf(sqrtf(rows_sum_scatter<C4, NI>(t, c4)), kNormFloor);
        }
        for (int k = emin; k < npk; ++k) {
            const float4 b4 = *reinterpret_cast<const float4*>(&P[k * D + 4 * c4]);
            float t[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) t[i] = dot4(er[i], b4);
            const float d = rows_sum_scatter<C4, NI>(t, c4);
            if (k >= my_ep) my_s = fmaxf(my_s, d * my_inv);
        }

        // Greedy picks while the shortlist's least key is below T.
        for (;;) {
            uint64_t kb = my_j >= 0 ? order_key(my_s, my_j) : ~0ull;
            kb = wave_min_u64(kb);
            if (lane == 0) red_k[wave] = kb;
            __syncthreads();
            uint64_t best = red_k[0];
            for (int w = 1; w < NW; ++w) best = red_k[w] < best ? red_k[w] : best;
            // (readfirstlane returns int: each half goes through uint32_t so
            // that the low half is not sign-extended into the high one.)
            best = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(best >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)best);
            if (best >= T) break;
            const int pj = (int)(best & 0x1fff);
            const unsigned long long hold = __ballot(my_j == pj);
            if (hold) {  // this wavefront holds the pick: row (L % C4) / G of group L / C4
                const int L = __builtin_ctzll(hold);
                const int ri = (L % C4) / G;
                const float inv = __shfl(my_inv, L);
                if (sub == L / C4) {
                    float4 v = er[0];
#pragma unroll
                    for (int i = 1; i < NI; ++i)
                        if (ri == i) v = er[i];
                    *reinterpret_cast<float4*>(&P[npk * D + 4 * c4]) =
                        make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
                    if (c4 == ri * G) ep[pj] = kPicked;
                }
                if (my_j == pj) my_j = -1;
            }
            if (tid == 0) {
                picks[npk] = pj;
                if (sel_order) sel_order[head * m + npk] = pj;
            }
            ++npk;
            __syncthreads();  // the pick row is in LDS; red_k is free again
            if (npk == m) break;
            const float4 b4 = *reinterpret_cast<const float4*>(&P[(npk - 1) * D + 4 * c4]);
            float t[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i) t[i] = dot4(er[i], b4);
            const float d = rows_sum_scatter<C4, NI>(t, c4);
            my_s = fmaxf(my_s, d * my_inv);
        }
        if (my_j >= 0 && c4 % G == 0) {
            lb[my_j] = my_s;
            ep[my_j] = (uint8_t)npk;
        }
        __syncthreads();
    }

    if (npk < m) {  // past the cap (not reached): the lowest unpicked slots
        if (tid == 0)
            for (int j = 0; j < N && npk < m; ++j)
                if (ep[j] != kPicked) {
                    ep[j] = kPicked;
                    picks[npk] = j;
                    if (sel_order) sel_order[head * m + npk] = j;
                    ++npk;
                }
        __syncthreads();
    }

    // Write back the picks in ascending slot order.
    if (tid == 0) {
        for (int a = 1; a < m; ++a) {
            const int x = picks[a];
            int b = a - 1;
            while (b >= 0 && picks[b] > x) {
                picks[b + 1] = picks[b];
                --b;
            }
            picks[b + 1] = x;
        }
    }
    __syncthreads();
    // (Native vector type: an array of the float4 struct would live in scratch.)
    typedef float v4f __attribute__((ext_vector_type(4)));
    constexpr int KS = kLongM * C4 / NT;  // staged chunks per thread
    v4f stg[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int e = tid + NT * k;
        stg[k] = e < m * C4
                     ? *reinterpret_cast<const v4f*>(row_ptr(picks[e / C4]) + 4 * (e % C4))
                     : v4f{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int e = tid + NT * k;
        if (e < m * C4)
            *reinterpret_cast<v4f*>(hb + (int64_t)(e / C4) * D + 4 * (e % C4)) = stg[k];
    }
    if (tid == 0) count[head] = m;
}

// Append only (trigger > buf_cap, so no head can compress), when one head's
// new rows are at most 64 16-byte chunks: CPH lanes (a power of two) per
// head, 256 / CPH heads per workgroup.  All lanes of a head are in one
// wavefront and read count before its chunk-0 lane writes the new count.
template <int CPH>
__global__ __launch_bounds__(256) void fps_append_kernel(
    float* __restrict__ buf, int32_t* __restrict__ count, const float* __restrict__ new_q,
    int n_new, int64_t qhs, int64_t qrs, int d, int cap, int m, int32_t* __restrict__ sel_order,
    int32_t* __restrict__ n_overflow, int64_t n_heads) {
    const int64_t head = ((int64_t)blockIdx.x * 256 + threadIdx.x) / CPH;
    const int c = threadIdx.x % CPH;
    if (head >= n_heads) return;
    const int nch = n_new * d / 4;  // 16-byte chunks to append
    const int cnt = count[head];
    if (sel_order)
        for (int i = c; i < m; i += CPH) sel_order[head * m + i] = -1;
    if (cnt < 0 || cnt + n_new > cap) {
        if (c == 0 && n_overflow) atomicAdd(n_overflow, 1);
        return;
    }
    if (c < nch)
        reinterpret_cast<float4*>(buf + (head * cap + cnt) * (int64_t)d)[c] =
            *reinterpret_cast<const float4*>(new_q + head * qhs + (int64_t)(c / (d / 4)) * qrs +
                                             (c % (d / 4)) * 4);
    if (c == 0) count[head] = cnt + n_new;
}

}  // namespace

hipError_t launch_fps(float* buf, int32_t* count, const float* new_q,
                      int32_t n_new, int64_t qhs, int64_t qrs, int64_t n_heads, int d, int buf_cap,
                      int trigger, int m, int32_t* sel_order,
                      int32_t* n_overflow, hipStream_t s) {
    if (n_heads <= 0) return hipSuccess;
    const int nch = n_new * d / 4;
    if (trigger > buf_cap && n_new > 0 && nch <= 64) {
        // Append only: many heads per workgroup.
        const unsigned blocks32 = (unsigned)((n_heads * 32 + 255) / 256);
        const unsigned blocks64 = (unsigned)((n_heads * 64 + 255) / 256);
        if (nch <= 32)
            fps_append_kernel<32><<<blocks32, 256, 0, s>>>(buf, count, new_q, n_new, qhs, qrs, d, buf_cap,
                                                           m, sel_order, n_overflow, n_heads);
        else
            fps_append_kernel<64><<<blocks64, 256, 0, s>>>(buf, count, new_q, n_new, qhs, qrs, d, buf_cap,
                                                           m, sel_order, n_overflow, n_heads);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)n_heads);
    if (buf_cap <= 32) {
        if (d == 128)
            fps_wave_kernel<128><<<grid, 64, 0, s>>>(buf, count, new_q, n_new, qhs, qrs, buf_cap,
                                                     trigger, m, sel_order, n_overflow);
        else
            fps_wave_kernel<64><<<grid, 64, 0, s>>>(buf, count, new_q, n_new, qhs, qrs, buf_cap,
                                                    trigger, m, sel_order, n_overflow);
    } else if (buf_cap <= 256) {
        if (d == 128)
            fps_block_kernel<128><<<grid, 256, 0, s>>>(buf, count, new_q, n_new, qhs, qrs, buf_cap,
                                                       trigger, m, sel_order, n_overflow);
        else
            fps_block_kernel<64><<<grid, 256, 0, s>>>(buf, count, new_q, n_new, qhs, qrs, buf_cap,
                                                      trigger, m, sel_order, n_overflow);
    } else {
        if (buf_cap > kLongCap || (m > kLongM && trigger <= buf_cap)) return hipErrorInvalidValue;
        // Long buffers take their new rows head-major and contiguous.
        if (n_new > 0 && (qrs != d || qhs != (int64_t)n_new * d)) return hipErrorInvalidValue;
        // Pick rows [min(m, kLongM)][d] floats, lb [buf_cap] floats, ep [buf_cap] bytes.
        const size_t lds = ((size_t)std::min(m, kLongM) * d * 4 + (size_t)buf_cap * 5 + 15) &
                           ~(size_t)15;
        if (d == 128) {
            if (lds > 65536) {
                const hipError_t e = hipFuncSetAttribute(
                    reinterpret_cast<const void*>(&fps_long_kernel<128>),
                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                if (e != hipSuccess) return e;
            }
            fps_long_kernel<128><<<grid, kLongThreads, lds, s>>>(
                buf, count, new_q, n_new, buf_cap, trigger, m, sel_order, n_overflow);
        } else {
            fps_long_kernel<64><<<grid, kLongThreads, lds, s>>>(
                buf, count, new_q, n_new, buf_cap, trigger, m, sel_order, n_overflow);
        }
    }
    return hipGetLastError();
}

}  // namespace bkv
