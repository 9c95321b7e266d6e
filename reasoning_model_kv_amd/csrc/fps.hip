// Continual-FPS fill-and-compress of the per-head pre-RoPE query buffers.
//
// Paper text §4.2 ("Continual FPS") and App. D.1 (Algorithm 1, FPS):
// average cosine similarity picks the seed (lowest), then the row whose
// largest cosine to the picked set is lowest joins it, until m rows remain.
//
// Mapping.  Buffers of up to 32 rows: one wavefront per query head forms
// the 32 x 32 cosine matrix once on fp32 MFMA and runs the greedy picks on
// it (see fps_wave_kernel).  Buffers of up to 256 rows (prefill) use one
// workgroup per head and one thread per row; there the average cosine of
// row i uses the sum of all normalised rows (sum_j cos(q_i, q_j) equals
// q_i/|q_i| . sum_j q_j/|q_j|) and each pick broadcasts the new member's
// row through LDS.
//
// Arithmetic is fp32; ties go to the lower slot.

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

// Wavefront argmin over (value, index) within each 32-lane half (both halves
// hold the same 32 candidates, one per lane), returned wave-uniform:
// lane ^ 1 and ^ 2 (quad_perm), the other quad of 8 (row_half_mirror), the
// other 8 of 16 (row_mirror), lane ^ 16 (swizzle).  (value, index) pairs
// compare lexicographically, so the order of the steps does not matter.
__device__ __forceinline__ int half_argmin(float v, int i) {
    argmin_pair(v, i, dpp_f<0xB1>(v), dpp_i<0xB1>(i));
    argmin_pair(v, i, dpp_f<0x4E>(v), dpp_i<0x4E>(i));
    argmin_pair(v, i, dpp_f<0x141>(v), dpp_i<0x141>(i));
    argmin_pair(v, i, dpp_f<0x140>(v), dpp_i<0x140>(i));
    argmin_pair(v, i, swap16_f(v), swap16_i(i));
    return __builtin_amdgcn_readlane(i, 0);
}

// Buffers of up to 32 rows: one wavefront per query head.
//  * Lane pair (2r, 2r+1) loads row r (half of its d fp32 values each) into
//    registers, where the rows stay until the kept ones are written back.
//  * The unit-normalised rows go to LDS transposed (dim-major), one half of
//    the dims at a time, and the 32 x 32 cosine matrix C = Qn Qn^T is formed
//    with d/2 fp32 MFMAs (v_mfma_f32_32x32x2_f32; lane l supplies row
//    l % 32, dim 2t + l / 32 of the half in LDS).
//  * Lane l then stands for row l % 32.  The average cosine of row j is the
//    sum of column j of C (C is symmetric) over N; the seed is its argmin.
//    Each further pick p adds column p of C (one LDS read per lane) to the
//    running max S, and the next pick is the argmin of S over the rows not
//    yet picked.
//  * The kept rows leave through LDS, eight at a time, as contiguous stores.
//  LDS stays at about 8 KB (d = 128), so some 18 wavefronts share a CU.
template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(5))) void fps_wave_kernel(
    float* __restrict__ buf, int32_t* __restrict__ count,
    const float* __restrict__ new_q, int n_new, int cap, int trigger, int m,
    int32_t* __restrict__ sel_order, int32_t* __restrict__ n_overflow) {
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
    const float* nq = new_q ? new_q + head * (int64_t)n_new * D : nullptr;

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
                *reinterpret_cast<const float4*>(nq + e);
        if (lane == 0) count[head] = N;
        return;
    }

    // Load this lane's half row (rows >= N are padding); all 16-byte loads
    // of a lane are in flight together.
    float x[HD];
    const bool valid = row < N;
    if (valid) {
        const float* src = row < cnt ? hb + (int64_t)row * D : nq + (int64_t)(row - cnt) * D;
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

    // C = Qn Qn^T over two rounds, one per half of the dims: the lanes holding
    // that half store it transposed to LDS (padding rows are zero rows), then
    // d/4 MFMAs add it.  Lane l ends with C[i][l % 32] for
    // i = 8 (v / 4) + 4 (l / 32) + v % 4.
    const int r32 = lane & 31;
    const int kk = lane >> 5;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        if (hf) wave_sync_lds();  // the first round's operand reads are done
        if (half == hf) {
#pragma unroll
            for (int k = 0; k < HD; ++k) qt[k * TS + row] = x[k] * inv;
        }
        wave_sync_lds();
#pragma unroll 8
        for (int t = 0; t < HD / 2; ++t) {
            const float a = qt[(2 * t + kk) * TS + r32];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, a, acc, 0, 0, 0);
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
    const float inf = __builtin_inff();
    int pick = half_argmin(valid32 ? colsum / (float)N : inf, r32);
    uint32_t sel = 1u << pick;
    int my_pick = (lane == 0) ? pick : -1;
    float S = qt[pick * TS + r32];
    for (int it = 1; it < m; ++it) {
        const bool cand = valid32 && !((sel >> r32) & 1u);
        pick = half_argmin(cand ? S : inf, r32);
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
    const float* __restrict__ new_q, int n_new, int cap, int trigger, int m,
    int32_t* __restrict__ sel_order, int32_t* __restrict__ n_overflow) {
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
    const float* nq = new_q ? new_q + head * (int64_t)n_new * D : nullptr;

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
                *reinterpret_cast<const float4*>(nq + e);
        if (tid == 0) count[head] = N;
        return;
    }

    auto row_ptr = [&](int j) -> const float* {
        return j < cnt ? hb + (int64_t)j * D : nq + (int64_t)(j - cnt) * D;
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

// Append only (trigger > buf_cap, so no head can compress), when one head's
// new rows are at most 64 16-byte chunks: CPH lanes (a power of two) per
// head, 256 / CPH heads per workgroup.  All lanes of a head are in one
// wavefront and read count before its chunk-0 lane writes the new count.
template <int CPH>
__global__ __launch_bounds__(256) void fps_append_kernel(
    float* __restrict__ buf, int32_t* __restrict__ count, const float* __restrict__ new_q,
    int n_new, int d, int cap, int m, int32_t* __restrict__ sel_order,
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
            reinterpret_cast<const float4*>(new_q + head * (int64_t)n_new * d)[c];
    if (c == 0) count[head] = cnt + n_new;
}

}  // namespace

hipError_t launch_fps(float* buf, int32_t* count, const float* new_q,
                      int32_t n_new, int64_t n_heads, int d, int buf_cap,
                      int trigger, int m, int32_t* sel_order,
                      int32_t* n_overflow, hipStream_t s) {
    if (n_heads <= 0) return hipSuccess;
    const int nch = n_new * d / 4;
    if (trigger > buf_cap && n_new > 0 && nch <= 64) {
        // Append only: many heads per workgroup.
        const unsigned blocks32 = (unsigned)((n_heads * 32 + 255) / 256);
        const unsigned blocks64 = (unsigned)((n_heads * 64 + 255) / 256);
        if (nch <= 32)
            fps_append_kernel<32><<<blocks32, 256, 0, s>>>(buf, count, new_q, n_new, d, buf_cap,
                                                           m, sel_order, n_overflow, n_heads);
        else
            fps_append_kernel<64><<<blocks64, 256, 0, s>>>(buf, count, new_q, n_new, d, buf_cap,
                                                           m, sel_order, n_overflow, n_heads);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)n_heads);
    if (buf_cap <= 32) {
        if (d == 128)
            fps_wave_kernel<128><<<grid, 64, 0, s>>>(buf, count, new_q, n_new, buf_cap,
                                                     trigger, m, sel_order, n_overflow);
        else
            fps_wave_kernel<64><<<grid, 64, 0, s>>>(buf, count, new_q, n_new, buf_cap,
                                                    trigger, m, sel_order, n_overflow);
    } else {
        if (d == 128)
            fps_block_kernel<128><<<grid, 256, 0, s>>>(buf, count, new_q, n_new, buf_cap,
                                                       trigger, m, sel_order, n_overflow);
        else
            fps_block_kernel<64><<<grid, 256, 0, s>>>(buf, count, new_q, n_new, buf_cap,
                                                      trigger, m, sel_order, n_overflow);
    }
    return hipGetLastError();
}

}  // namespace bkv
