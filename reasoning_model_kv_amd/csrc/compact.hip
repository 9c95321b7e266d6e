// Compaction: gather the kept slots to the front of each unit's cache.
//
// Paper text §2.2: the compressed cache indexes the sequence dimension with
// the retained set; summary step (5): written back in position order.
//
// Mapping: one workgroup of W wavefronts per tensor part of a KV group (the
// key rows and the positions, or the value rows), which walks the kept list
// in ascending order in rounds of W x 32 tokens; wavefront w moves tokens
// [base + 32 w, base + 32 w + 32) of the round starting at base (a bf16 row
// of d = 128 is 16 lanes x 16 bytes, so one load instruction moves 4 rows),
// and the next round's rows are in flight while this round's are stored.
// In place, tokens before the first evicted slot do not move and are
// skipped.
//
// Why it is safe in place.  kept is strictly ascending and kept[k] >= k, so
// the source of token k lies at or above every destination of the tokens
// before it: a round's stores land below every source of the later rounds,
// and only overwrite sources of the same or earlier rounds.  Each round
// therefore waits, in every wavefront, for that wavefront's loads of the
// round to land, then meets at a workgroup barrier, and only then stores;
// the loads of the next round may already be in flight (their sources lie
// above this round's destinations).  The barrier carries no memory fence:
// the hazard is between loads that have returned their data and stores
// issued after the barrier, which needs no cache visibility.
//
// Why a workgroup per part rather than a wavefront: with one wavefront per
// part (about 9,000 independent streams at the Qwen3-4B shape), moving
// 9.7 GB took 1.90 ms (5.1 TB/s); with sixteen wavefronts walking one part
// together (about 500 streams of 512 tokens per round) 1.75 ms (5.5 TB/s,
// the rate of a plain device copy of the same bytes on this GPU).

#include "common.h"

namespace bkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte store: the compacted rows are not read
// again by this step.
__device__ __forceinline__ void st_nt(uint16_t* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st_nt(uint16_t* p, uint4 v) {
    st_nt(p, __builtin_bit_cast(u32x4, v));
}
// Streaming (non-temporal) 16-byte load: each moved row is read once.
__device__ __forceinline__ u32x4 ld_nt(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
constexpr int TPB = 32;  // tokens per wavefront per round

// Write-only sink for the stores of tokens past the end of the kept list (or
// of malformed entries): every store is issued unconditionally, so that the
// compiler's vmcnt waits count exactly (a conditional store makes it assume
// the store may be missing and wait for loads still in flight).  Never read.
__device__ u32x4 g_sink[64];

// First index k whose kept slot is not k (kept[k] - k never decreases), or
// b_kv if nothing moves.
__device__ __forceinline__ int64_t first_moved(const int32_t* __restrict__ ku, int64_t b_kv,
                                               int lane) {
    for (int64_t k0 = 0; k0 < b_kv; k0 += 64) {
        const int64_t k = k0 + lane;
        const bool moved = k < b_kv && ku[k] != (int32_t)k;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(moved);
        if (bal) return k0 + __builtin_ctzll(bal);
    }
    return b_kv;
}

// Workgroup barrier without a memory fence (see the header): the
// wavefront-scope fences only keep the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void round_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Stand-in source of the positions for the value part, whose position loads
// are discarded: one cached line instead of a second read of the positions.
__device__ int32_t g_nopos[64];

// The walk of one tensor of unit u by wavefront w of W: rows Ts[kept[k]] go
// to Td[k] (Ts == Td in place), and with pos the positions ps[kept[k]] to
// pd[k].  Tokens before k0 are not moved.  Every wavefront of the workgroup
// runs the same number of rounds (the loop bounds depend on k0 and b_kv
// only), so the barriers match.  Both parts run this one code path (pos is
// a runtime flag): with the two parts specialised into two inlined loops the
// same walk took 2.8 instead of 1.75 ms at the Qwen3-4B shape.
template <int D, int W>
__device__ __forceinline__ void coop_walk(const uint16_t* Ts, uint16_t* Td, const int32_t* ps,
                                          int32_t* pd, bool pos, const int32_t* __restrict__ ku,
                                          int64_t L, int64_t b_kv, int64_t k0, int w, int lane) {
    constexpr int LPT = D / 8;        // lanes per token row (16-byte chunks)
    constexpr int TPW = 64 / LPT;     // tokens per wave instruction
    constexpr int NI = TPB / TPW;     // instructions per round (<= 8)
    constexpr int RS = W * TPB;       // tokens per round
    static_assert(NI >= 1 && NI <= 8, "tokens per round");
    const int st = lane / LPT;  // token within an instruction
    const int ch = lane % LPT;  // 16-byte chunk within the row
    const int64_t off = 8 * ch;
    const int tl = lane & (TPB - 1);
    // Raw kept entries of this wavefront's tokens of the round at base (lane
    // j (mod TPB): kept[base + TPB w + j]); checked only where they are used,
    // so that the load is not waited for at once.
    auto load_kept = [&](int64_t base) -> int32_t {
        const int64_t k = base + TPB * w + tl;
        return ku[k < b_kv ? k : b_kv - 1];
    };
    // -1 past b_kv or for an entry outside [0, L) (a malformed list is
    // skipped, never followed).
    auto checked = [&](int64_t base, int32_t v) -> int32_t {
        const int64_t k = base + TPB * w + tl;
        return (k < b_kv && v >= 0 && v < L) ? v : -1;
    };
    // One round's rows and positions.  Invalid tokens load slot 0 (the loads
    // stay unconditional, so the compiler's waits count exactly) and are
    // stored into the sink.
    struct Batch {
        u32x4 r[NI];
        int32_t s[NI];
        int32_t p;
        bool pv;
    };
    auto load_rows = [&](int64_t base, int32_t raw, Batch& b) {
        const int32_t kv = checked(base, raw);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            b.s[i] = __shfl(kv, st + i * TPW);
            const int64_t r = b.s[i] >= 0 ? b.s[i] : 0;
            b.r[i] = ld_nt(Ts + r * D + off);
        }
        b.pv = pos && kv >= 0;
        b.p = ps[pos && kv >= 0 ? kv : 0];
    };
    // Waits until this wavefront's loads of b have returned their data.
    auto landed = [&](const Batch& b) {
#pragma unroll
        for (int i = 0; i < NI; ++i) asm volatile("" ::"v"(b.r[i]));
        asm volatile("" ::"v"(b.p));
    };
    // Every lane stores: invalid tokens into the sink; lanes TPB.. repeat the
    // position stores of lanes 0..TPB-1 (same address, same value).
    auto store_rows = [&](int64_t base, const Batch& b) {
        const int64_t bw = base + TPB * w;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int64_t kb = bw + st + i * TPW;
            const bool ok = b.s[i] >= 0;
            st_nt(ok ? Td + kb * D + off : reinterpret_cast<uint16_t*>(&g_sink[lane]), b.r[i]);
        }
        *(b.pv ? pd + bw + tl : reinterpret_cast<int32_t*>(&g_sink[lane])) = b.p;
    };

    // Software pipeline over two register buffers (no register with a load
    // in flight is ever copied): the raw kept entries of the round after
    // next and the rows of the next round are loaded before this round's
    // barrier and stores.
    Batch A, B;
    int32_t kvA = load_kept(k0);
    load_rows(k0, kvA, A);
    int32_t kvB = load_kept(k0 + RS);
    for (int64_t base = k0;;) {
        kvA = load_kept(base + 2 * RS);
        load_rows(base + RS, kvB, B);
        landed(A);
        round_barrier();
        store_rows(base, A);
        base += RS;
        if (base >= b_kv) break;
        kvB = load_kept(base + 2 * RS);
        load_rows(base + RS, kvA, A);
        landed(B);
        round_barrier();
        store_rows(base, B);
        base += RS;
        if (base >= b_kv) break;
    }
    // Keeps the kept-entry loads where they are issued: with no use on the
    // exit path the compiler sinks them below the loop's exit test, next to
    // their first use, and the wait there drains every load and store in
    // flight (the counter is in order).
    asm volatile("" ::"v"(kvA), "v"(kvB));
}

// Workgroup b: unit b / 2, part b % 2 (0: keys and positions, 1: values);
// Ko == nullptr means in place.
template <int D, int W>
__global__ __launch_bounds__(64 * W) void compact_kernel(
    uint16_t* K, uint16_t* V, int32_t* kpos, int64_t l_cap, const int32_t* __restrict__ kept,
    int64_t L, int64_t b_kv, uint16_t* Ko, uint16_t* Vo, int32_t* kposo, int64_t out_cap,
    int64_t n_units) {
    const int64_t u = (int64_t)(blockIdx.x >> 1);
    const int part = (int)(blockIdx.x & 1);
    if (u >= n_units) return;  // uniform over the workgroup
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool inplace = (Ko == nullptr);
    const int32_t* ku = kept + u * b_kv;
    const int64_t k0 = inplace ? first_moved(ku, b_kv, lane) : 0;
    if (k0 >= b_kv) return;  // uniform: every wavefront finds the same k0
    const int64_t so = u * l_cap * D, dof = inplace ? so : u * out_cap * D;
    uint16_t* src = (part == 0 ? K : V) + so;
    uint16_t* dst = (inplace ? src : (part == 0 ? Ko : Vo) + dof);
    int32_t* pdst = inplace ? kpos + u * l_cap : kposo + u * out_cap;
    coop_walk<D, W>(src, dst, part == 0 ? kpos + u * l_cap : g_nopos, pdst, part == 0, ku, L,
                    b_kv, k0, w, lane);
}

constexpr int WAVES = 4;  // wavefronts per workgroup of the unsorted compaction

// Wavefront-wide synchronisation of LDS between the lanes of one wavefront.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Holes handled per pass of the unsorted compaction (LDS per wavefront).
constexpr int kFillPass = 1024;

// Unsorted compaction (hole filling): the kept tokens at slots >= b_kv move
// into the evicted slots below b_kv -- the i-th lowest such hole takes the
// i-th lowest such token -- and every other kept token stays where it is.
// One wavefront per KV group:
//  * c = the number of kept entries below b_kv (kept is ascending), by 64
//    probes and then a scan of the one block they narrow it to;
//  * the holes just below kept entry k are the slots between kept[k-1] and
//    kept[k] (kept[c] taken as b_kv), and hole h there has rank h - k (the
//    slots below it less the kept entries below it), so every lane walks its
//    own entry's gap and records hole[rank] = h in LDS, no prefix sums;
//  * the moves read token kept[c + rank] and write it to hole[rank]: sources
//    are all >= b_kv and destinations < b_kv, so they are independent; 16
//    lanes move one 256-byte row, four rows per instruction.
// Ranks are handled kFillPass at a time.  Every access is bounds-checked: a
// kept list that is not strictly ascending within [0, L) moves nothing
// outside [0, L) (it may leave holes unfilled).
template <int D>
__global__ __launch_bounds__(64 * WAVES) void fill_kernel(uint16_t* K, uint16_t* V,
                                                          int32_t* kpos, int64_t l_cap,
                                                          const int32_t* __restrict__ kept,
                                                          int64_t L, int64_t b_kv,
                                                          int64_t n_units) {
    constexpr int LPT = D / 8;     // lanes per token row
    constexpr int TPW = 64 / LPT;  // rows per instruction
    __shared__ int32_t hole_lds[WAVES][kFillPass];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t u = (int64_t)blockIdx.x * WAVES + wv;
    if (u >= n_units) return;
    int32_t* hole = hole_lds[wv];
    const int32_t* ku = kept + u * b_kv;
    uint16_t* Ku = K + u * l_cap * D;
    uint16_t* Vu = V + u * l_cap * D;
    int32_t* pu = kpos + u * l_cap;
    const int32_t b = (int32_t)b_kv;

    // c: first index whose entry is >= b (b if none).  Probe i reads entry
    // i * step (step = ceil(b / 64), so the probes cover [0, b)); the first
    // probe at or above b, f, bounds c to (probe f-1, probe f]; with none,
    // c lies after the last probe.  One scan of at most step - 1 entries
    // finishes it.
    int32_t c;
    {
        const int32_t step = (b + 63) / 64;
        const int32_t pi = lane * step;
        const uint64_t m = __ballot(pi < b && ku[pi] >= b);
        int32_t lo, hi;
        if (m == 0) {
            const int32_t last = ((b - 1) / step) * step;  // last probe below b
            lo = last + 1;
            hi = b;
        } else {
            const int32_t f = (int32_t)__builtin_ctzll(m);
            lo = f == 0 ? 0 : (f - 1) * step + 1;
            hi = f * step;
        }
        c = hi;
        for (int32_t k0 = lo; k0 < hi; k0 += 64) {
            const int32_t k = k0 + lane;
            const uint64_t mm = __ballot(k < hi && ku[k] >= b);
            if (mm) {
                c = k0 + (int32_t)__builtin_ctzll(mm);
                break;
            }
        }
    }
    const int32_t n_tail = b - c;
    const int st = lane / LPT, ch = lane % LPT;
    const int64_t off = 8 * ch;
    for (int32_t base = 0; base < n_tail; base += kFillPass) {
        const int32_t n = n_tail - base < kFillPass ? n_tail - base : kFillPass;
        for (int i = lane; i < kFillPass; i += 64) hole[i] = -1;
        wave_sync();
        // Gaps of entries 0..c (entry c stands for b): ranks [base, base + n).
        int32_t carry = -1;  // entry before the chunk
        for (int32_t k0 = 0; k0 <= c; k0 += 64) {
            const int32_t k = k0 + lane;
            const int32_t cur = k < c ? ku[k] : (k == c ? b : 0);
            int32_t prev = __shfl_up(cur, 1);
            if (lane == 0) prev = carry;
            carry = __shfl(cur, 63);
            if (k <= c) {
                // holes h in (prev, cur) with rank h - k in [base, base + n)
                int32_t h0 = prev + 1, h1 = cur - 1;
                if (h0 < base + k) h0 = base + k;
                if (h1 > base + n - 1 + k) h1 = base + n - 1 + k;
                if (h1 >= b) h1 = b - 1;
                for (int32_t h = h0; h <= h1; ++h) hole[h - k - base] = h;
            }
        }
        wave_sync();
        // Moves: 64 holes per round, TPW rows per instruction.
        for (int32_t i0 = 0; i0 < n; i0 += 64) {
            const int32_t my = i0 + lane;
            const int32_t hsrc = my < n ? ku[c + base + my] : -1;  // source of rank base+my
#pragma unroll 4
            for (int r0 = 0; r0 < 64; r0 += TPW) {
                const int j = r0 + st;  // row within the round
                const int32_t s_ = __shfl(hsrc, j);
                const int32_t h = i0 + j < n ? hole[i0 + j] : -1;
                const bool ok = i0 + j < n && h >= 0 && h < b && s_ >= b && s_ < L;
                if (ok) {
                    const uint4 kr = *(const uint4*)(Ku + (int64_t)s_ * D + off);
                    const uint4 vr = *(const uint4*)(Vu + (int64_t)s_ * D + off);
                    st_nt(Ku + (int64_t)h * D + off, kr);
                    st_nt(Vu + (int64_t)h * D + off, vr);
                    if (ch == 0) pu[h] = pu[s_];
                }
            }
        }
        wave_sync();
    }
}

}  // namespace

hipError_t launch_compact(uint16_t* K, uint16_t* V, int32_t* kpos,
                          int64_t n_units, int d, int64_t l_cap, int64_t L,
                          const int32_t* kept, int64_t b_kv, uint16_t* K_out,
                          uint16_t* V_out, int32_t* kpos_out, int64_t out_cap,
                          hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    if (n_units > (int64_t)1 << 30) return hipErrorInvalidValue;
    // Two workgroups per unit; rounds of W x 32 tokens, W sized to the kept
    // list so that short lists do not leave most wavefronts idle.
    const dim3 grid((unsigned)(2 * n_units));
#define BKV_CMP(DD, WW)                                                                 \
    compact_kernel<DD, WW><<<grid, 64 * (WW), 0, s>>>(K, V, kpos, l_cap, kept, L, b_kv, \
                                                      K_out, V_out, kpos_out, out_cap,  \
                                                      n_units)
#define BKV_CMP_W(DD)                                                                   \
    if (b_kv >= 1024) BKV_CMP(DD, 16);                                                  \
    else if (b_kv >= 512) BKV_CMP(DD, 8);                                               \
    else BKV_CMP(DD, 4)
    if (d == 128) { BKV_CMP_W(128); }
    else { BKV_CMP_W(64); }
#undef BKV_CMP_W
#undef BKV_CMP
    return hipGetLastError();
}

hipError_t launch_select_compact(uint16_t* K, uint16_t* V, int32_t* kpos, int64_t n_units,
                                 int d, int64_t l_cap, int64_t L, const float* score,
                                 int32_t* kept, int64_t b_kv, int prefix, int recent_tok,
                                 hipStream_t s) {
    hipError_t e = launch_select(score, n_units, l_cap, L, b_kv, prefix, recent_tok, kept, s);
    if (e == hipSuccess)
        e = launch_compact(K, V, kpos, n_units, d, l_cap, L, kept, b_kv, nullptr, nullptr,
                           nullptr, l_cap, s);
    return e;
}

}  // namespace bkv

namespace bkv {

hipError_t launch_compact_fill(uint16_t* K, uint16_t* V, int32_t* kpos, int64_t n_units, int d,
                               int64_t l_cap, int64_t L, const int32_t* kept, int64_t b_kv,
                               hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n_units + WAVES - 1) / WAVES));
    if (d == 128)
        fill_kernel<128><<<grid, 64 * WAVES, 0, s>>>(K, V, kpos, l_cap, kept, L, b_kv, n_units);
    else
        fill_kernel<64><<<grid, 64 * WAVES, 0, s>>>(K, V, kpos, l_cap, kept, L, b_kv, n_units);
    return hipGetLastError();
}

}  // namespace bkv
