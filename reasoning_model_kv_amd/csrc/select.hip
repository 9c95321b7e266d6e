// Keep-set selection: forced prefix and recent slots plus Top-K of the rest.
//
// Summary step (5): the prefix tokens and the most recent tokens are always
// kept, the remaining budget is filled with the highest-scoring slots and
// the kept entries are written back in position order (paper text §2.2,
// App. D.2).  Ties go to the lower slot.
//
// Mapping: one workgroup per KV group.  Scores are non-negative fp32, so
// their bit patterns order like the values; a 4-pass MSB-first radix select
// (8-bit digits, LDS histogram, block scan over the digits from the top)
// finds the exact value T of the K'-th largest middle score and how many
// entries equal to T are needed.  A final pass over the slots in order
// scans the "keep" flags (block ballot + prefix) and writes the kept slots
// ascending; entries equal to T are taken lowest slot first.

#include "common.h"

namespace bkv {
namespace {

constexpr int NT = 256;

// Inclusive scan of one value per thread over the workgroup; also returns
// the total.  Uses `wsum` (NT/64 words of LDS).
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* wsum,
                                                         uint32_t* total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t n = __shfl_up(v, o);
        if (lane >= o) v += n;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t s = wsum[w];
        if (w < wave) off += s;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return v + off;
}

__global__ __launch_bounds__(NT) void select_kernel(const float* __restrict__ score,
                                                    int64_t l_cap, int64_t L, int64_t b_kv,
                                                    int prefix, int recent_tok,
                                                    int32_t* __restrict__ kept) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wsum[NT / 64];
    __shared__ uint32_t sh_digit, sh_krem;

    const int tid = threadIdx.x;
    const int64_t u = blockIdx.x;
    const uint32_t* bits = reinterpret_cast<const uint32_t*>(score + u * l_cap);
    int32_t* out = kept + u * b_kv;
    const int64_t lo = prefix, hi = L - recent_tok;  // middle slots [lo, hi)
    const int64_t want = b_kv - prefix - recent_tok;

    uint32_t thr = 0, pmask = 0;
    uint32_t krem = (uint32_t)want;
    if (want > 0) {
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            hist[tid] = 0;
            __syncthreads();
            for (int64_t j = lo + tid; j < hi; j += NT) {
                const uint32_t b = bits[j];
                if ((b & pmask) == thr) atomicAdd(&hist[(b >> shift) & 255u], 1u);
            }
            __syncthreads();
            // Digits from the top: thread t looks at digit 255 - t.
            const uint32_t c = hist[255 - tid];
            uint32_t tot;
            const uint32_t inc = block_inclusive_scan(c, wsum, &tot);
            if (inc >= krem && inc - c < krem) {
                sh_digit = 255u - (uint32_t)tid;
                sh_krem = krem - (inc - c);
            }
            __syncthreads();
            thr |= sh_digit << shift;
            pmask |= 0xFFu << shift;
            krem = sh_krem;
            __syncthreads();
        }
    }

    // thr: exact bits of the K'-th largest middle score; krem: how many of
    // the entries equal to thr are kept (the lowest slots).
    uint32_t written = 0, eq_seen = 0;
    for (int64_t j0 = 0; j0 < L; j0 += NT) {
        const int64_t j = j0 + tid;
        const bool in = j < L;
        const bool forced = in && (j < lo || j >= hi);
        const bool mid = in && !forced && want > 0;
        const uint32_t b = mid ? bits[j] : 0u;
        const bool eq = mid && b == thr;
        uint32_t tot_eq;
        const uint32_t eq_inc = block_inclusive_scan(eq ? 1u : 0u, wsum, &tot_eq);
        const uint32_t eq_rank = eq_seen + eq_inc - (eq ? 1u : 0u);
        const bool take = forced || (mid && b > thr) || (eq && eq_rank < krem);
        uint32_t tot_take;
        const uint32_t t_inc = block_inclusive_scan(take ? 1u : 0u, wsum, &tot_take);
        const uint32_t pos = written + t_inc - 1;
        if (take && pos < (uint32_t)b_kv) out[pos] = (int32_t)j;
        written += tot_take;
        eq_seen += tot_eq;
    }
}

}  // namespace

hipError_t launch_select(const float* score, int64_t n_units, int64_t l_cap,
                         int64_t L, int64_t b_kv, int prefix, int recent_tok,
                         int32_t* kept, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    select_kernel<<<dim3((unsigned)n_units), NT, 0, s>>>(score, l_cap, L, b_kv, prefix,
                                                         recent_tok, kept);
    return hipGetLastError();
}

}  // namespace bkv
