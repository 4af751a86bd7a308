// Internal helpers shared by the HIP kernels of libspec_hip (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "spec.h"

namespace spec {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// launch geometry shared by host launchers and workspace sizing
// ---------------------------------------------------------------------------

// Logit rows are cut into chunks of 16 KB (8192 bf16 or 4096 fp32 entries: a
// workgroup of 256 threads reads one with four 16-byte loads per thread),
// fewer entries for short rows so that a row still spans about four chunks
// (a multiple of 64 entries keeps 16-byte alignment).
struct RowSplit {
    int64_t chunk;   // elements per chunk
    int32_t splits;  // chunks per row
};

constexpr int kChunkBytes = 16384;

inline RowSplit row_split(int32_t vocab, int elem_bytes)
{
    const int64_t full = kChunkBytes / elem_bytes;
    int64_t chunk = (vocab + 3) / 4;
    chunk = (chunk + 63) / 64 * 64;
    if (chunk > full) chunk = full;
    if (chunk < 64) chunk = 64;
    RowSplit s;
    s.chunk = chunk;
    s.splits = (int32_t)((vocab + chunk - 1) / chunk);
    return s;
}

constexpr int32_t kMaxSplits = 2048;             // rows up to 8,388,608 entries

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

template <typename T>
__device__ __forceinline__ T wave_max(T v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        T u = __shfl_xor(v, o, kWave);
        v = u > v ? u : v;
    }
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2,
// 4 and 8 within each row of 16 lanes, then the last lane of row 0 (and of
// row 2) added to row 1 (and row 3), then the last lane of row 1 added to rows
// 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t v)
{
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return (uint32_t)x;
}

// One DPP step of the same pattern on a double (both halves moved alike;
// lanes the step does not reach read 0).
template <int CTRL, int ROWS, bool BOUND>
__device__ __forceinline__ double dpp_f64(double v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS, 0xf, BOUND);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS, 0xf, BOUND);
    return __hiloint2double(hi, lo);
}

// Inclusive prefix sum over the 64 lanes of a wave in fp64 (the scan pattern
// of wave_incl_add): lane l gets v_0 + ... + v_l, in a fixed order.
__device__ __forceinline__ double wave_incl_f64(double v)
{
    v += dpp_f64<0x111, 0xf, true>(v);
    v += dpp_f64<0x112, 0xf, true>(v);
    v += dpp_f64<0x114, 0xf, true>(v);
    v += dpp_f64<0x118, 0xf, true>(v);
    v += dpp_f64<0x142, 0xa, false>(v);
    v += dpp_f64<0x143, 0xc, false>(v);
    return v;
}

// Sum over the 64 lanes of a wave, valid in lane 63.
__device__ __forceinline__ double wave_total_f64(double v) { return wave_incl_f64(v); }

// Lane l's double (l wave-uniform), in every lane.
__device__ __forceinline__ double wave_bcast_f64(double v, int l)
{
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), l);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), l);
    return __hiloint2double(hi, lo);
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v |= __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        uint64_t u = __shfl_xor(v, o, kWave);
        v = u > v ? u : v;
    }
    return v;
}

// Top-2 of unique 64-bit keys (0 = empty).
struct Top2 {
    uint64_t a, b;  // a > b or b == 0
};

__device__ __forceinline__ Top2 top2_merge(Top2 x, Top2 y)
{
    Top2 r;
    if (x.a >= y.a) {
        r.a = x.a;
        r.b = x.b > y.a ? x.b : y.a;
    } else {
        r.a = y.a;
        r.b = y.b > x.a ? y.b : x.a;
    }
    return r;
}

__device__ __forceinline__ Top2 top2_insert(Top2 t, uint64_t k)
{
    if (k > t.a) {
        t.b = t.a;
        t.a = k;
    } else if (k > t.b) {
        t.b = k;
    }
    return t;
}

__device__ __forceinline__ Top2 wave_top2(Top2 t)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        Top2 u;
        u.a = __shfl_xor(t.a, o, kWave);
        u.b = __shfl_xor(t.b, o, kWave);
        t = top2_merge(t, u);
    }
    return t;
}

}  // namespace spec

// Host-side launch status bookkeeping (defined in abi.hip).
int spec_record_hip_error(hipError_t e);
