// Compaction: gather the kept slots to the front of each unit's cache.
//
// Paper text §2.2: the compressed cache indexes the sequence dimension with
// the retained set; summary step (5): written back in position order.
//
// Mapping: one wavefront per KV group walks its kept list in ascending
// order, 16 tokens per iteration (a bf16 row of d = 128 is 16 lanes x 16
// bytes, so one load instruction moves 4 rows).  In place, tokens before
// the first evicted slot do not move and are skipped.  The walk is safe in
// place without any barrier: kept is strictly ascending, so the source of
// token k is at a slot >= k and every destination written by an iteration
// lies below every source read by later iterations; a destination can only
// be the source of the same or an earlier token, whose load has completed
// before the store that needs its data is issued.

#include "common.h"

namespace bkv {
namespace {

constexpr int WAVES = 4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte store: the compacted rows are not read
// again by this step.
__device__ __forceinline__ void st_nt(uint16_t* p, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}
constexpr int TPI = 16;  // tokens per iteration

template <int D>
__global__ __launch_bounds__(64 * WAVES) void compact_kernel(
    uint16_t* K, uint16_t* V, int32_t* kpos, int64_t l_cap, const int32_t* __restrict__ kept,
    int64_t L, int64_t b_kv, uint16_t* Ko, uint16_t* Vo, int32_t* kposo, int64_t out_cap,
    int64_t n_units) {
    constexpr int LPT = D / 8;        // lanes per token row (16-byte chunks)
    constexpr int TPW = 64 / LPT;     // tokens per wave instruction
    constexpr int NI = TPI / TPW;     // instructions per tensor per iteration (<= 4)
    static_assert(NI >= 1 && NI <= 4, "tokens per iteration");
    const int lane = threadIdx.x & 63;
    const int64_t u = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
    if (u >= n_units) return;
    const bool inplace = (Ko == nullptr);
    const int32_t* ku = kept + u * b_kv;
    const uint16_t* Ks = K + u * l_cap * D;
    const uint16_t* Vs = V + u * l_cap * D;
    const int32_t* ps = kpos + u * l_cap;
    uint16_t* Kd = inplace ? K + u * l_cap * D : Ko + u * out_cap * D;
    uint16_t* Vd = inplace ? V + u * l_cap * D : Vo + u * out_cap * D;
    int32_t* pd = inplace ? kpos + u * l_cap : kposo + u * out_cap;

    int64_t k0 = 0;
    if (inplace) {
        // First index whose slot changes (kept[k] - k never decreases).
        for (k0 = 0; k0 < b_kv; k0 += 64) {
            const int64_t k = k0 + lane;
            const bool moved = k < b_kv && ku[k] != (int32_t)k;
            const uint64_t bal = __builtin_amdgcn_ballot_w64(moved);
            if (bal) {
                k0 += __builtin_ctzll(bal);
                break;
            }
        }
        if (k0 >= b_kv) return;
    }

    const int st = lane / LPT;  // token within an instruction
    const int ch = lane % LPT;  // 16-byte chunk within the row
    for (int64_t base = k0; base < b_kv; base += TPI) {
        // Source slots of this lane's NI tokens (kept[k] >= 0 always; -1 = past the end).
        // Entries outside [0, L) (a malformed kept list) are skipped, never followed.
        auto src_of = [&](int64_t k) -> int32_t {
            if (k >= b_kv) return -1;
            const int32_t v = ku[k];
            return (v >= 0 && v < L) ? v : -1;
        };
        const int64_t kb = base + st;
        const int32_t s0 = src_of(kb);
        const int32_t s1 = NI > 1 ? src_of(kb + TPW) : -1;
        const int32_t s2 = NI > 2 ? src_of(kb + 2 * TPW) : -1;
        const int32_t s3 = NI > 3 ? src_of(kb + 3 * TPW) : -1;
        const int32_t psrc = lane < TPI ? src_of(base + lane) : -1;
        uint4 k0r{}, k1r{}, k2r{}, k3r{}, v0r{}, v1r{}, v2r{}, v3r{};
        const int64_t off = 8 * ch;
        if (s0 >= 0) { k0r = *(const uint4*)(Ks + (int64_t)s0 * D + off); v0r = *(const uint4*)(Vs + (int64_t)s0 * D + off); }
        if (s1 >= 0) { k1r = *(const uint4*)(Ks + (int64_t)s1 * D + off); v1r = *(const uint4*)(Vs + (int64_t)s1 * D + off); }
        if (s2 >= 0) { k2r = *(const uint4*)(Ks + (int64_t)s2 * D + off); v2r = *(const uint4*)(Vs + (int64_t)s2 * D + off); }
        if (s3 >= 0) { k3r = *(const uint4*)(Ks + (int64_t)s3 * D + off); v3r = *(const uint4*)(Vs + (int64_t)s3 * D + off); }
        int32_t pr = 0;
        if (psrc >= 0) pr = ps[psrc];
        if (s0 >= 0) { st_nt(Kd + kb * D + off, k0r); st_nt(Vd + kb * D + off, v0r); }
        if (s1 >= 0) { st_nt(Kd + (kb + TPW) * D + off, k1r); st_nt(Vd + (kb + TPW) * D + off, v1r); }
        if (s2 >= 0) { st_nt(Kd + (kb + 2 * TPW) * D + off, k2r); st_nt(Vd + (kb + 2 * TPW) * D + off, v2r); }
        if (s3 >= 0) { st_nt(Kd + (kb + 3 * TPW) * D + off, k3r); st_nt(Vd + (kb + 3 * TPW) * D + off, v3r); }
        if (psrc >= 0) pd[base + lane] = pr;
    }
}

}  // namespace

hipError_t launch_compact(uint16_t* K, uint16_t* V, int32_t* kpos,
                          int64_t n_units, int d, int64_t l_cap, int64_t L,
                          const int32_t* kept, int64_t b_kv, uint16_t* K_out,
                          uint16_t* V_out, int32_t* kpos_out, int64_t out_cap,
                          hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n_units + WAVES - 1) / WAVES));
    if (d == 128)
        compact_kernel<128><<<grid, 64 * WAVES, 0, s>>>(K, V, kpos, l_cap, kept, L, b_kv, K_out,
                                                        V_out, kpos_out, out_cap, n_units);
    else
        compact_kernel<64><<<grid, 64 * WAVES, 0, s>>>(K, V, kpos, l_cap, kept, L, b_kv, K_out,
                                                       V_out, kpos_out, out_cap, n_units);
    return hipGetLastError();
}

}  // namespace bkv
