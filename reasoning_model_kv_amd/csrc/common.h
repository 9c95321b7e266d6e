// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bkv.h"

namespace bkv {

// Launchers: enqueue kernels, return hipSuccess or the launch error.
// new_q: head h's new row r at new_q + h * qhs + r * qrs (floats).
hipError_t launch_fps(float* buf, int32_t* count, const float* new_q,
                      int32_t n_new, int64_t qhs, int64_t qrs, int64_t n_heads, int d, int buf_cap,
                      int trigger, int m, int32_t* sel_order,
                      int32_t* n_overflow, hipStream_t s);

hipError_t launch_rope_table(double* table, int64_t t, int n_recent_q, int d,
                             double theta, hipStream_t s);

// lse_in: known softmax denominators by observation row ([U, g, 32],
// natural log) or NULL; see bkv_score_lse.
hipError_t launch_score(const uint16_t* K, const int32_t* kpos, int64_t n_units,
                        int g, int d, int64_t l_cap, int64_t L,
                        const float* beacons, int buf_cap, const float* recents,
                        int n_beacon, int n_recent_q, int64_t t, double theta,
                        float sm_scale, bool mean, const double* table, float* score,
                        uint16_t* qobs_out, const float* lse_in, int64_t lse_from,
                        hipStream_t s);

// Decode attention of each query head's new query (rotated to t_q) over
// K, V [0, L), with the beacons' (rotated to t_obs) log-sum-exp when
// beacons is non-NULL; see bkv_decode_attend.
hipError_t launch_decode(const uint16_t* K, const uint16_t* V, int64_t n_units, int g, int d,
                         int64_t l_cap, int64_t L, const float* q, int64_t t_q,
                         const float* beacons, int buf_cap, int64_t t_obs, double theta,
                         float sm_scale, float* out, float* lse_q, float* lse_obs,
                         hipStream_t s);

hipError_t launch_select(const float* score, int64_t n_units, int64_t l_cap,
                         int64_t L, int64_t b_kv, int prefix, int recent_tok,
                         int32_t* kept, hipStream_t s);

// Keep-set selection, then in-place position-ordered compaction; kept
// receives the keep sets as launch_select writes them.
hipError_t launch_select_compact(uint16_t* K, uint16_t* V, int32_t* kpos, int64_t n_units,
                                 int d, int64_t l_cap, int64_t L, const float* score,
                                 int32_t* kept, int64_t b_kv, int prefix, int recent_tok,
                                 hipStream_t s);

// Unsorted compaction in place: kept tokens at slots >= b_kv fill the
// evicted slots below b_kv.
hipError_t launch_compact_fill(uint16_t* K, uint16_t* V, int32_t* kpos, int64_t n_units, int d,
                               int64_t l_cap, int64_t L, const int32_t* kept, int64_t b_kv,
                               hipStream_t s);
hipError_t launch_compact(uint16_t* K, uint16_t* V, int32_t* kpos,
                          int64_t n_units, int d, int64_t l_cap, int64_t L,
                          const int32_t* kept, int64_t b_kv, uint16_t* K_out,
                          uint16_t* V_out, int32_t* kpos_out, int64_t out_cap,
                          hipStream_t s);

// RoPE angle table: (1 + n_recent_q) positions x d/2 pairs x {cos, sin}.
// Entry 0 is position t; entry 1 + i is position t - n_recent_q + i.
inline size_t rope_table_bytes(int n_recent_q, int d) {
    return (size_t)(1 + n_recent_q) * (size_t)(d / 2) * 2 * sizeof(double);
}

// ---------------------------------------------------------------- device --

// float -> bfloat16 bits, round to nearest, ties to even (finite inputs;
// NaN becomes a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

}  // namespace bkv
