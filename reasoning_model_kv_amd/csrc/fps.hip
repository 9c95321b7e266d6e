// Continual-FPS fill-and-compress of the per-head pre-RoPE query buffers.
//
// Paper text §4.2 ("Continual FPS") and App. D.1 (Algorithm 1, FPS):
// average cosine similarity picks the seed (lowest), then the row whose
// largest cosine to the picked set is lowest joins it, until m rows remain.
//
// Mapping.  Buffers of up to 32 rows: one wavefront per query head, two
// lanes per row, each lane holding half of the row (d/2 fp32 values) in
// registers.  The unit-normalised rows are staged in LDS once; each pick
// then broadcasts the new member's row from LDS to all lanes (same-address
// reads, no bank conflicts), every lane pair forms its row's cosine with
// it, and a wavefront argmin chooses the next pick.  The average cosine of
// row i uses the sum of all normalised rows: sum_j cos(q_i, q_j) equals
// q_i/|q_i| . sum_j q_j/|q_j|, one dot product instead of a row of the Gram
// matrix.  Buffers of up to 256 rows (prefill) use one workgroup per head
// and one thread per row.
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

// Wavefront argmin over (value, index); every lane receives the result.
// Lanes 2r and 2r+1 carry the same candidate, so xor 1 is skipped.
__device__ __forceinline__ int wave_argmin_rows(float v, int i) {
#pragma unroll
    for (int o = 2; o < 64; o <<= 1) {
        float ov = __shfl_xor(v, o);
        int oi = __shfl_xor(i, o);
        argmin_pair(v, i, ov, oi);
    }
    return i;
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__global__ __launch_bounds__(64) void fps_wave_kernel(
    float* __restrict__ buf, int32_t* __restrict__ count,
    const float* __restrict__ new_q, int n_new, int cap, int trigger, int m,
    int32_t* __restrict__ sel_order, int32_t* __restrict__ n_overflow) {
    constexpr int HD = D / 2;       // dims held by one lane
    constexpr int STRIDE = D + 4;   // LDS row stride (floats)
    __shared__ float qn[32 * STRIDE];
    __shared__ float svec[D];

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

    // Load this lane's half row (rows >= N are padding).
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
    nn += __shfl_xor(nn, 1);
    const float inv = 1.0f / fmaxf(sqrtf(nn), kNormFloor);

    float* myrow = qn + row * STRIDE + half * HD;
#pragma unroll
    for (int k = 0; k < HD; k += 4)
        *reinterpret_cast<float4*>(myrow + k) =
            make_float4(x[k] * inv, x[k + 1] * inv, x[k + 2] * inv, x[k + 3] * inv);
    wave_sync_lds();

    // Sum of the normalised rows, one or two dims per lane.
    for (int k = lane; k < D; k += 64) {
        float s = 0.f;
        for (int j = 0; j < N; ++j) s += qn[j * STRIDE + k];
        svec[k] = s;
    }
    wave_sync_lds();

    auto dot_with = [&](const float* v) {
        float a = 0.f;
#pragma unroll
        for (int k = 0; k < HD; k += 4) {
            float4 f = *reinterpret_cast<const float4*>(v + half * HD + k);
            a = fmaf(x[k], f.x, a);
            a = fmaf(x[k + 1], f.y, a);
            a = fmaf(x[k + 2], f.z, a);
            a = fmaf(x[k + 3], f.w, a);
        }
        a += __shfl_xor(a, 1);
        return a * inv;
    };

    const float avg = dot_with(svec) / (float)N;
    const float inf = __builtin_inff();
    int pick = wave_argmin_rows(valid ? avg : inf, row);
    uint32_t sel = 1u << pick;
    int my_pick = (lane == 0) ? pick : -1;
    float S = dot_with(qn + pick * STRIDE);

    for (int it = 1; it < m; ++it) {
        const bool cand = valid && !((sel >> row) & 1u);
        pick = wave_argmin_rows(cand ? S : inf, row);
        sel |= 1u << pick;
        if (lane == it) my_pick = pick;
        S = fmaxf(S, dot_with(qn + pick * STRIDE));
    }

    // Keep the picked rows in ascending slot order, from registers.
    if ((sel >> row) & 1u) {
        const int rank = __popc(sel & ((1u << row) - 1u));
        float* dst = hb + (int64_t)rank * D + half * HD;
#pragma unroll
        for (int k = 0; k < HD; k += 4)
            *reinterpret_cast<float4*>(dst + k) = make_float4(x[k], x[k + 1], x[k + 2], x[k + 3]);
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

}  // namespace

hipError_t launch_fps(float* buf, int32_t* count, const float* new_q,
                      int32_t n_new, int64_t n_heads, int d, int buf_cap,
                      int trigger, int m, int32_t* sel_order,
                      int32_t* n_overflow, hipStream_t s) {
    if (n_heads <= 0) return hipSuccess;
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
