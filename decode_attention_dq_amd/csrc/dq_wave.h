// Wave-level helpers shared by the attention kernels: cross-lane reductions,
// the in-register 128-point Walsh-Hadamard transform and scalar conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dq {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Wave-wide maxima returned as wave-uniform values, by DPP moves: butterflies
// inside each 16-lane row (quad swaps, half-row and row mirrors), then row
// 15 -> row 1/3 and lane 31 -> rows 2/3 broadcasts, after which lane 63 holds
// the maximum of all 64 lanes. Every lane must be active.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_mov(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ float wave_max_uniform(float v) {
    v = fmaxf(v, __int_as_float(dpp_mov<0xB1>(__float_as_int(v))));        // quad_perm [1,0,3,2]
    v = fmaxf(v, __int_as_float(dpp_mov<0x4E>(__float_as_int(v))));        // quad_perm [2,3,0,1]
    v = fmaxf(v, __int_as_float(dpp_mov<0x141>(__float_as_int(v))));       // row_half_mirror
    v = fmaxf(v, __int_as_float(dpp_mov<0x140>(__float_as_int(v))));       // row_mirror
    v = fmaxf(v, __int_as_float(dpp_mov<0x142, 0xA>(__float_as_int(v))));  // row_bcast:15
    v = fmaxf(v, __int_as_float(dpp_mov<0x143, 0xC>(__float_as_int(v))));  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Wave-wide sum returned as a wave-uniform value, by the same DPP pattern
// (the row broadcasts add zero in the rows they do not write).
__device__ __forceinline__ float wave_sum_uniform(float v) {
    v += __int_as_float(dpp_mov<0xB1>(__float_as_int(v)));
    v += __int_as_float(dpp_mov<0x4E>(__float_as_int(v)));
    v += __int_as_float(dpp_mov<0x141>(__float_as_int(v)));
    v += __int_as_float(dpp_mov<0x140>(__float_as_int(v)));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ int wave_max_uniform_i(int v) {
    v = max(v, dpp_mov<0xB1>(v));
    v = max(v, dpp_mov<0x4E>(v));
    v = max(v, dpp_mov<0x141>(v));
    v = max(v, dpp_mov<0x140>(v));
    v = max(v, dpp_mov<0x142, 0xA>(v));
    v = max(v, dpp_mov<0x143, 0xC>(v));
    return __builtin_amdgcn_readlane(v, 63);
}

// In-register 128-point Walsh-Hadamard transform (H x, entries +-1) of a row
// held as v0 = x[lane], v1 = x[lane + 64]: butterflies of span 1..32 across
// lanes, then span 64 inside the lane.
__device__ __forceinline__ void fwht128_f32(float& v0, float& v1, int lane) {
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
        const float p0 = __shfl_xor(v0, h), p1 = __shfl_xor(v1, h);
        const bool lo = (lane & h) == 0;
        v0 = lo ? v0 + p0 : p0 - v0;
        v1 = lo ? v1 + p1 : p1 - v1;
    }
    const float a = v0, b = v1;
    v0 = a + b;
    v1 = a - b;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return (float)v;
}
__device__ __forceinline__ int f32_exponent(float v) {   // floor(log2 v) for v > 0 normal
    return (int)((__float_as_uint(v) >> 23) & 255u) - 127;
}

}  // namespace dq
