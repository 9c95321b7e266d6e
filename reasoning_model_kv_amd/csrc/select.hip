// Keep-set selection: forced prefix and recent slots plus Top-K of the rest.
//
// Summary step (5): the prefix tokens and the most recent tokens are always
// kept, the remaining budget is filled with the highest-scoring slots and
// the kept entries are written back in position order (paper text §2.2,
// App. D.2).  Ties go to the lower slot.
//
// Mapping: one wavefront per KV group up to 8192 slots -- with the scores in
// registers up to 4608 slots (select_reg_kernel), staged in LDS beyond
// (select_wave_kernel) -- and one workgroup per KV group beyond 8192.  Scores are non-negative fp32, so
// their bit patterns order like the values; a 4-pass MSB-first radix select
// (8-bit digits, LDS histogram, block scan over the digits from the top)
// finds the exact value T of the K'-th largest middle score and how many
// entries equal to T are needed.  A final pass over the slots in order
// scans the "keep" flags (block ballot + prefix) and writes the kept slots
// ascending; entries equal to T are taken lowest slot first.

#include "common.h"
#include "select_wave.h"

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

// Wavefront-wide synchronisation of LDS between the lanes of one wavefront.
__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Single-wavefront variant (units of up to kWaveSlots slots): the unit's
// scores are copied once into LDS (all loads in flight together), and every
// later step reads LDS and is wavefront-wide, with no workgroup barriers.
// Each radix pass counts into an LDS histogram with LDS atomics; the digits
// are scanned from the top with a wavefront scan (four digits per lane); the
// final pass takes the slots in chunks of 64 with ballots, which order equal
// entries and kept slots by slot.  Dynamic LDS: 256 + L words.
__global__ __launch_bounds__(64) void select_wave_kernel(const float* __restrict__ score,
                                                         int64_t l_cap, int64_t L, int64_t b_kv,
                                                         int prefix, int recent_tok,
                                                         int32_t* __restrict__ kept) {
    extern __shared__ uint32_t lds_words[];
    uint32_t* hist = lds_words;       // 256 digit counts
    uint32_t* sc = lds_words + 256;   // the unit's score bits, [L]
    const int lane = threadIdx.x;
    const int64_t u = blockIdx.x;
    const uint32_t* bits = reinterpret_cast<const uint32_t*>(score + u * l_cap);
    int32_t* out = kept + u * b_kv;
    const int n = (int)L;
    const int lo = prefix, hi = n - recent_tok;  // middle slots [lo, hi)
    const int64_t want = b_kv - prefix - recent_tok;

    // Copy in batches of 32 loads per lane, all in flight before any store.
    for (int j0 = 0; j0 < n; j0 += 64 * 32) {
        uint32_t t[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int j = j0 + lane + 64 * i;
            t[i] = j < n ? bits[j] : 0u;
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int j = j0 + lane + 64 * i;
            if (j < n) sc[j] = t[i];
        }
    }
    wave_sync_lds();

    uint32_t thr = 0, pmask = 0;
    uint32_t krem = (uint32_t)want;
    if (want > 0) {
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
#pragma unroll
            for (int k = 0; k < 4; ++k) hist[lane + 64 * k] = 0;
            wave_sync_lds();
#pragma unroll 4
            for (int j = lo + lane; j < hi; j += 64) {
                const uint32_t b = sc[j];
                if ((b & pmask) == thr) atomicAdd(&hist[(b >> shift) & 255u], 1u);
            }
            wave_sync_lds();
            // Lane l takes digits 255 - 4l .. 252 - 4l (descending).
            uint32_t c[4], cs = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                c[k] = hist[255 - 4 * lane - k];
                cs += c[k];
            }
            uint32_t inc = cs;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t t = __shfl_up(inc, o);
                if (lane >= o) inc += t;
            }
            const uint32_t exc = inc - cs;
            const bool here = exc < krem && inc >= krem;  // exactly one lane
            uint32_t digit = 0, kr = 0;
            if (here) {
                uint32_t e = exc;
                bool found = false;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if (!found) {
                        if (e + c[k] >= krem) {
                            digit = 255u - 4u * (uint32_t)lane - (uint32_t)k;
                            kr = krem - e;
                            found = true;
                        } else {
                            e += c[k];
                        }
                    }
                }
            }
            const uint64_t who = __ballot(here);
            const int src = who ? (int)__builtin_ctzll(who) : 0;
            thr |= (uint32_t)__builtin_amdgcn_readlane((int)digit, src) << shift;
            pmask |= 0xFFu << shift;
            krem = (uint32_t)__builtin_amdgcn_readlane((int)kr, src);
            wave_sync_lds();  // every lane has read the histogram
        }
    }

    // thr: exact bits of the K'-th largest middle score; krem: how many of
    // the entries equal to thr are kept (the lowest slots).
    uint32_t written = 0, eq_seen = 0;
    for (int j0 = 0; j0 < n; j0 += 64) {
        const int j = j0 + lane;
        const bool in = j < n;
        const bool forced = in && (j < lo || j >= hi);
        const bool mid = in && !forced && want > 0;
        const uint32_t b = mid ? sc[j] : 0u;
        const bool eq = mid && b == thr;
        const uint64_t eqm = __ballot(eq);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(eqm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eqm, 0u));
        const bool take = forced || (mid && b > thr) || (eq && eq_seen + below < krem);
        const uint64_t tm = __ballot(take);
        const uint32_t pos = written + __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(tm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)tm, 0u));
        if (take && pos < (uint32_t)b_kv) out[pos] = j;
        written += (uint32_t)__builtin_popcountll(tm);
        eq_seen += (uint32_t)__builtin_popcountll(eqm);
    }
}

// Register-resident variant (units of up to 64 * NR slots): the scores stay
// in registers, so only the 256-bin histogram lives in LDS and every unit of
// a large launch is resident at once (the LDS-staged kernel keeps (256 + L)
// words per wavefront, which at L = 2176 caps a CU at 16 wavefronts).
template <int NR>
__global__ __launch_bounds__(64) void select_reg_kernel(const float* __restrict__ score,
                                                        int64_t l_cap, int64_t L, int64_t b_kv,
                                                        int prefix, int recent_tok,
                                                        int32_t* __restrict__ kept) {
    __shared__ uint32_t hist[256];
    const int64_t u = blockIdx.x;
    select_wave_reg<NR>(score + u * l_cap, L, b_kv, prefix, recent_tok, kept + u * b_kv, hist,
                        threadIdx.x);
}

// Largest unit handled by one wavefront (beyond it a workgroup shares the
// sweeps).
constexpr int64_t kWaveSlots = 8192;

}  // namespace

hipError_t launch_select(const float* score, int64_t n_units, int64_t l_cap,
                         int64_t L, int64_t b_kv, int prefix, int recent_tok,
                         int32_t* kept, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    const dim3 g1((unsigned)n_units);
#define BKV_SEL_REG(NR)                                                                  \
    if (L <= 64 * (NR)) {                                                                \
        select_reg_kernel<NR><<<g1, 64, 0, s>>>(score, l_cap, L, b_kv, prefix, recent_tok, \
                                                kept);                                   \
        return hipGetLastError();                                                        \
    }
    BKV_SEL_REG(8)
    BKV_SEL_REG(16)
    BKV_SEL_REG(36)
    BKV_SEL_REG(72)
#undef BKV_SEL_REG
    if (L <= kWaveSlots)
        select_wave_kernel<<<dim3((unsigned)n_units), 64, (size_t)(256 + L) * 4, s>>>(
            score, l_cap, L, b_kv, prefix, recent_tok, kept);
    else
        select_kernel<<<dim3((unsigned)n_units), NT, 0, s>>>(score, l_cap, L, b_kv, prefix,
                                                             recent_tok, kept);
    return hipGetLastError();
}

}  // namespace bkv
