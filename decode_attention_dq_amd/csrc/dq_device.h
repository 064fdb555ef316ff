// Device helpers shared by the decode-attention kernel and the symbol-decode
// test hook: LDS staging of fixed-stride containers and the rANS decode step.
#pragma once

#include "dq_internal.h"

namespace dq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Orders this wave's earlier LDS accesses before its later ones as seen by
// the other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One rANS decode step (D-Quant section 3.1, Dec): the slot x mod 2^p selects
// the table entry of the symbol m that owns it, the state becomes
// f_m * floor(x / 2^p) + (slot - c_m), and one byte is shifted in when the
// state drops below 2^16 (at most one, since f_m >= 2^(p-8)). `ptr` is the
// LDS address of the next container byte; the byte is always read and used
// only when needed, so the step has no branch. Returns the entry.
typedef __attribute__((address_space(3))) const uint8_t lds_u8;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;

// `ptr` and `tab` are absolute LDS byte addresses.
__device__ __forceinline__ uint32_t rans_dec_step(uint32_t& x, uint32_t& ptr, uint32_t tab, uint32_t mask,
                                                  uint32_t p) {
    const uint32_t e = *(lds_u32*)(size_t)(tab + ((x & mask) << 2));
    const uint32_t b = *(lds_u8*)(size_t)ptr;
    const uint32_t f = (e >> 18) & 1023u;
    const uint32_t bias = (e >> 8) & 1023u;
    x = __umul24(f, x >> p) + bias;       // f < 2^10, x >> p < 2^14
    const bool need = x < kStateLow;
    // The shifted-in state is formed unconditionally and passed through an
    // empty asm so that the select stays a v_cndmask: otherwise the byte load
    // is sunk into a branch and each step pays two dependent LDS trips.
    uint32_t t = (x << 8) | b;
    asm volatile("" : "+v"(t));
    x = need ? t : x;
    ptr += need ? 1u : 0u;
    // opaque running pointer: otherwise the compiler rewrites it as base + the
    // sum of all renormalisation flags and keeps every flag live
    asm volatile("" : "+v"(ptr));
    return e;
}

// Two fp16 levels (entries e0 for the lower channel, e1 for the upper) packed
// into one dword: the level's high byte sits in bits 0..7 of an entry and its
// low byte is zero.
__device__ __forceinline__ uint32_t pack_levels(uint32_t e0, uint32_t e1) {
    return __builtin_amdgcn_perm(e1, e0, 0x040C000Cu);
}

}  // namespace dq
