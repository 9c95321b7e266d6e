// Keep-set selection of one unit by one wavefront, scores in registers:
// shared by the select kernel and the fused select-and-compact kernel.
//
// Summary step (5): the prefix tokens and the most recent tokens are always
// kept, the remaining budget is filled with the highest-scoring slots,
// written in position order (paper text §2.2, App. D.2); ties go to the
// lower slot.  Lane l holds the score bits of slots l + 64 r, r < NR (units
// of up to 64 * NR slots; scores are non-negative fp32, so their bits order
// like the values); four MSB-first 8-bit radix passes over a 256-bin LDS
// histogram find the value T of the K'-th largest middle score and how many
// entries equal to T are taken; a final pass over the slots in order takes
// the kept ones with ballots (register r of every lane is the chunk of slots
// [64 r, 64 r + 64)) and writes them ascending.
#pragma once

#include "common.h"

namespace bkv {
namespace {

__device__ __forceinline__ void sel_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// score_u: the unit's scores [L]; out: its kept list [b_kv]; hist: 256
// words of LDS owned by this wavefront.
template <int NR>
__device__ __forceinline__ void select_wave_reg(const float* __restrict__ score_u, int64_t L,
                                                int64_t b_kv, int prefix, int recent_tok,
                                                int32_t* __restrict__ out, uint32_t* hist,
                                                int lane) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(score_u);
    const int n = (int)L;
    const int lo = prefix, hi = n - recent_tok;  // middle slots [lo, hi)
    const int64_t want = b_kv - prefix - recent_tok;

    // Unconditional loads (slots past the end read slot n - 1 and are never
    // used): no branch per chunk, all loads in flight together.
    uint32_t bits[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int j = lane + 64 * r;
        bits[r] = src[j < n ? j : n - 1];
    }
    // Bit r of midm[r / 32]: slot lane + 64 r is a middle slot.
    constexpr int NW = (NR + 31) / 32;
    uint32_t midm[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) midm[w] = 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int j = lane + 64 * r;
        if (j >= lo && j < hi) midm[r / 32] |= 1u << (r % 32);
    }

    uint32_t thr = 0, pmask = 0;
    uint32_t krem = (uint32_t)want;
    if (want > 0) {
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
#pragma unroll
            for (int k = 0; k < 4; ++k) hist[lane + 64 * k] = 0;
            sel_wave_sync();
            // Fresh copies of the masks per pass: the per-slot conditions
            // are not hoisted out of the pass loop (as 64-bit exec masks,
            // one per slot chunk, they would not fit in scalar registers).
            uint32_t mm[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                mm[w] = midm[w];
                asm volatile("" : "+v"(mm[w]));
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const uint32_t b = bits[r];
                if (((mm[r / 32] >> (r % 32)) & 1u) && (b & pmask) == thr)
                    atomicAdd(&hist[(b >> shift) & 255u], 1u);
            }
            sel_wave_sync();
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
            const int srcl = who ? (int)__builtin_ctzll(who) : 0;
            thr |= (uint32_t)__builtin_amdgcn_readlane((int)digit, srcl) << shift;
            pmask |= 0xFFu << shift;
            krem = (uint32_t)__builtin_amdgcn_readlane((int)kr, srcl);
            sel_wave_sync();  // every lane has read the histogram
        }
    }

    uint32_t written = 0, eq_seen = 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        // One chunk at a time: unfenced, the scheduler hoists every chunk's
        // ballot masks and runs out of scalar registers.
        __builtin_amdgcn_sched_barrier(0);
        const int j = lane + 64 * r;
        const bool in = j < n;
        const bool forced = in && (j < lo || j >= hi);
        const bool mid = in && !forced && want > 0;
        const uint32_t b = mid ? bits[r] : 0u;
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

}  // namespace
}  // namespace bkv
