// Compaction: gather the kept slots to the front of each unit's cache.
//
// Paper text §2.2: the compressed cache indexes the sequence dimension with
// the retained set; summary step (5): written back in position order.
//
// Mapping: two wavefronts per KV group, one moving the key rows and the
// positions, the other the value rows.  Each walks the kept list in
// ascending order, 32 tokens per iteration (a bf16 row of d = 128 is 16
// lanes x 16 bytes, so one load instruction moves 4 rows), with the next
// iteration's rows in flight while this one's are stored.  In place, tokens
// before the first evicted slot do not move and are skipped.  The walk is
// safe in place without any barrier: kept is strictly ascending, so the
// source of token k is at a slot >= k and every destination written by an
// iteration lies below every source read by later iterations; a destination
// can only be the source of the same or an earlier token, whose load has
// completed before the store that needs its data is issued; and the two
// wavefronts of a group touch disjoint tensors.  Splitting a group's moves
// over two wavefronts (rather than one wavefront moving both tensors) keeps
// twice as many groups' streams in flight: 5.1 against 4.9 TB/s.

#include "common.h"
#include "select_wave.h"

namespace bkv {
namespace {

constexpr int WAVES = 4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte store: the compacted rows are not read
// again by this step.
__device__ __forceinline__ void st_nt(uint16_t* p, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}
// Streaming (non-temporal) 16-byte load: each moved row is read once.
__device__ __forceinline__ uint4 ld_nt(const uint16_t* p) {
    return __builtin_bit_cast(uint4,
                              __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
constexpr int TPI = 32;  // tokens per iteration

// Write-only sink for the stores of tokens past the end of the kept list (or
// of malformed entries): every store is issued unconditionally, so that the
// compiler's vmcnt waits count exactly (a conditional store makes it assume
// the store may be missing and wait for loads still in flight).  Never read.
__device__ uint4 g_sink[64];

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

// The walk of one tensor of unit u by one wavefront: rows Ts[kept[k]] go to
// Td[k] (Ts == Td in place), and with POS the positions ps[kept[k]] to
// pd[k].  Tokens before k0 are not moved.
template <int D, bool POS>
__device__ __forceinline__ void compact_walk(const uint16_t* Ts, uint16_t* Td, const int32_t* ps,
                                             int32_t* pd, const int32_t* __restrict__ ku,
                                             int64_t L, int64_t b_kv, int64_t k0, int lane) {
    constexpr int LPT = D / 8;        // lanes per token row (16-byte chunks)
    constexpr int TPW = 64 / LPT;     // tokens per wave instruction
    constexpr int NI = TPI / TPW;     // instructions per iteration (<= 8)
    static_assert(NI >= 1 && NI <= 8, "tokens per iteration");
    const int st = lane / LPT;  // token within an instruction
    const int ch = lane % LPT;  // 16-byte chunk within the row
    const int64_t off = 8 * ch;
    // Kept entries of tokens [base, base + TPI): lane j (mod TPI) holds
    // kept[base + j], or -1 past b_kv or for an entry outside [0, L) (a
    // malformed list is skipped, never followed).  One load per lane.
    auto load_kept = [&](int64_t base) -> int32_t {
        const int64_t k = base + (lane & (TPI - 1));
        const int32_t v = ku[k < b_kv ? k : b_kv - 1];
        return (k < b_kv && v >= 0 && v < L) ? v : -1;
    };
    // One iteration's rows (and positions).  Invalid tokens load slot 0 (the
    // loads stay unconditional, so the compiler's waits count exactly) and
    // are stored into the sink.
    struct Batch {
        uint4 r[NI];
        int32_t s[NI];
        int32_t p;
        bool pv;
    };
    auto load_rows = [&](int32_t kv, Batch& b) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            b.s[i] = __shfl(kv, st + i * TPW);
            const int64_t r = b.s[i] >= 0 ? b.s[i] : 0;
            b.r[i] = ld_nt(Ts + r * D + off);
        }
        if (POS) {
            b.pv = kv >= 0;
            b.p = ps[kv >= 0 ? kv : 0];
        }
    };
    // Every lane stores: invalid tokens into the sink; lanes TPI.. repeat the
    // position stores of lanes 0..TPI-1 (same address, same value).
    auto store_rows = [&](int64_t base, const Batch& b) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int64_t kb = base + st + i * TPW;
            const bool ok = b.s[i] >= 0;
            st_nt(ok ? Td + kb * D + off : reinterpret_cast<uint16_t*>(&g_sink[lane]), b.r[i]);
        }
        if (POS)
            *(b.pv ? pd + base + (lane & (TPI - 1)) : reinterpret_cast<int32_t*>(&g_sink[lane])) =
                b.p;
    };

    // Software pipeline: the kept entries of the iteration after next and
    // the rows of the next iteration are loaded before this iteration's rows
    // are stored.  Unrolled by two over two buffers, so that no register
    // with a load in flight is ever copied (a copy would wait for the load).
    // Safe in place: every destination written by an iteration lies below
    // every source read by the later ones (kept is strictly ascending and
    // kept[k] >= k).
    Batch A, B;
    int32_t kvA = load_kept(k0);
    load_rows(kvA, A);
    int32_t kvB = load_kept(k0 + TPI);
    for (int64_t base = k0;;) {
        kvA = load_kept(base + 2 * TPI);
        load_rows(kvB, B);
        store_rows(base, A);
        base += TPI;
        if (base >= b_kv) break;
        kvB = load_kept(base + 2 * TPI);
        load_rows(kvA, A);
        store_rows(base, B);
        base += TPI;
        if (base >= b_kv) break;
    }
}

// Wavefront `part` (0: keys and positions, 1: values) of unit u's
// compaction; Ko == nullptr means in place.
template <int D>
__device__ __forceinline__ void compact_part(uint16_t* K, uint16_t* V, int32_t* kpos,
                                             int64_t l_cap, const int32_t* __restrict__ kept,
                                             int64_t L, int64_t b_kv, uint16_t* Ko,
                                             uint16_t* Vo, int32_t* kposo, int64_t out_cap,
                                             int64_t u, int part, int lane) {
    const bool inplace = (Ko == nullptr);
    const int32_t* ku = kept + u * b_kv;
    const int64_t k0 = inplace ? first_moved(ku, b_kv, lane) : 0;
    if (k0 >= b_kv) return;
    const int64_t so = u * l_cap * D, dof = inplace ? so : u * out_cap * D;
    if (part == 0) {
        compact_walk<D, true>(K + so, (inplace ? K : Ko) + dof, kpos + u * l_cap,
                              inplace ? kpos + u * l_cap : kposo + u * out_cap, ku, L, b_kv, k0,
                              lane);
    } else {
        compact_walk<D, false>(V + so, (inplace ? V : Vo) + dof, nullptr, nullptr, ku, L, b_kv,
                               k0, lane);
    }
}

// Wavefront w of workgroup b: unit (4 b + w) / 2, part w % 2.
template <int D>
__global__ __launch_bounds__(64 * WAVES) void compact_kernel(
    uint16_t* K, uint16_t* V, int32_t* kpos, int64_t l_cap, const int32_t* __restrict__ kept,
    int64_t L, int64_t b_kv, uint16_t* Ko, uint16_t* Vo, int32_t* kposo, int64_t out_cap,
    int64_t n_units) {
    const int64_t gw = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
    const int64_t u = gw >> 1;
    if (u >= n_units) return;
    compact_part<D>(K, V, kpos, l_cap, kept, L, b_kv, Ko, Vo, kposo, out_cap, u, (int)(gw & 1),
                    threadIdx.x & 63);
}

// Selection and in-place compaction in one launch (summary step (5)): a
// workgroup of four wavefronts takes two units.  Wavefronts 0 and 1 select
// the keep sets of the two units (select_wave_reg, units of up to 64 * NR
// slots) and write them to kept; after a workgroup barrier, which makes
// those writes visible to the whole workgroup, wavefronts 2u' and 2u' + 1
// move unit u''s keys and positions and its values.  A unit's selection is
// latency-bound and its walk bandwidth-bound: the wavefronts of other
// workgroups keep HBM busy meanwhile.
template <int D, int NR>
__device__ __forceinline__ void select_compact_group(
    uint16_t* K, uint16_t* V, int32_t* kpos, int64_t l_cap, const float* __restrict__ score,
    int32_t* kept, int64_t L, int64_t b_kv, int prefix, int recent_tok, int64_t n_units,
    uint32_t (*hist)[256]) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t u0 = (int64_t)blockIdx.x * 2;
    if (w < 2 && u0 + w < n_units)
        select_wave_reg<NR>(score + (u0 + w) * l_cap, L, b_kv, prefix, recent_tok,
                            kept + (u0 + w) * b_kv, hist[w], lane);
    __syncthreads();
    const int64_t u = u0 + (w >> 1);
    if (u < n_units)
        compact_part<D>(K, V, kpos, l_cap, kept, L, b_kv, nullptr, nullptr, nullptr, 0, u, w & 1,
                        lane);
}

// Units of up to 64 * 36 slots: held to 128 VGPRs, four wavefronts per SIMD
// as in compact_kernel.
template <int D, int NR>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(4)))
void select_compact_kernel(uint16_t* K, uint16_t* V, int32_t* kpos, int64_t l_cap,
                           const float* __restrict__ score, int32_t* kept, int64_t L,
                           int64_t b_kv, int prefix, int recent_tok, int64_t n_units) {
    __shared__ uint32_t hist[2][256];
    select_compact_group<D, NR>(K, V, kpos, l_cap, score, kept, L, b_kv, prefix, recent_tok,
                                n_units, hist);
}

// Up to 64 * 72 slots: the 72 score registers per lane need more than 128
// VGPRs (held to 128 they spill), so three wavefronts per SIMD.
template <int D>
__global__ __launch_bounds__(64 * WAVES) void select_compact_kernel_wide(
    uint16_t* K, uint16_t* V, int32_t* kpos, int64_t l_cap, const float* __restrict__ score,
    int32_t* kept, int64_t L, int64_t b_kv, int prefix, int recent_tok, int64_t n_units) {
    __shared__ uint32_t hist[2][256];
    select_compact_group<D, 72>(K, V, kpos, l_cap, score, kept, L, b_kv, prefix, recent_tok,
                                n_units, hist);
}

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
    // Two wavefronts per unit.
    const dim3 grid((unsigned)((2 * n_units + WAVES - 1) / WAVES));
    if (d == 128)
        compact_kernel<128><<<grid, 64 * WAVES, 0, s>>>(K, V, kpos, l_cap, kept, L, b_kv, K_out,
                                                        V_out, kpos_out, out_cap, n_units);
    else
        compact_kernel<64><<<grid, 64 * WAVES, 0, s>>>(K, V, kpos, l_cap, kept, L, b_kv, K_out,
                                                       V_out, kpos_out, out_cap, n_units);
    return hipGetLastError();
}

bool select_compact_fits(int64_t L) { return L <= 64 * 72; }

hipError_t launch_select_compact(uint16_t* K, uint16_t* V, int32_t* kpos, int64_t n_units,
                                 int d, int64_t l_cap, int64_t L, const float* score,
                                 int32_t* kept, int64_t b_kv, int prefix, int recent_tok,
                                 hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    if (!select_compact_fits(L)) return hipErrorInvalidValue;
    // Two units per workgroup.
    const dim3 grid((unsigned)((n_units + 1) / 2));
#define BKV_SC(DD, NR)                                                                    \
    select_compact_kernel<DD, NR><<<grid, 64 * WAVES, 0, s>>>(K, V, kpos, l_cap, score, kept, \
                                                              L, b_kv, prefix, recent_tok, n_units)
#define BKV_SC_D(NR)                                                                      \
    if (d == 128) BKV_SC(128, NR); else BKV_SC(64, NR)
    if (L <= 64 * 8) { BKV_SC_D(8); }
    else if (L <= 64 * 16) { BKV_SC_D(16); }
    else if (L <= 64 * 36) { BKV_SC_D(36); }
    else if (d == 128) {
        select_compact_kernel_wide<128><<<grid, 64 * WAVES, 0, s>>>(
            K, V, kpos, l_cap, score, kept, L, b_kv, prefix, recent_tok, n_units);
    } else {
        select_compact_kernel_wide<64><<<grid, 64 * WAVES, 0, s>>>(
            K, V, kpos, l_cap, score, kept, L, b_kv, prefix, recent_tok, n_units);
    }
#undef BKV_SC_D
#undef BKV_SC
    return hipGetLastError();
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
