// Device helpers shared by the decode-attention kernel and the symbol-decode
// test hook: LDS staging of fixed-stride containers and the rANS decode step.
#pragma once

#include "dq_internal.h"

namespace dq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Orders this wave's earlier LDS accesses before its later ones as seen by
// the other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef __attribute__((address_space(3))) const uint8_t lds_u8;
typedef __attribute__((address_space(3))) const uint32_t lds_u32;
typedef __attribute__((address_space(3))) const u32x2 lds_u32x2;

// Per-lane rANS decoder state. The container bytes are read through a
// 4-byte window refilled every 4 steps (at most one byte is consumed per
// step), so a step needs one LDS access (the table) instead of two. The
// per-token kernel refills it from HBM; tiles staged in LDS use RansLaneCarry.
struct RansLane {
    uint32_t x;     // state, in [2^16, 2^24) between steps
    uint32_t ptr;   // address of the window's first byte
    uint32_t win;   // the 4 bytes at ptr (first byte in bits 0..7)
    uint32_t sel;   // v_perm selector kSel0 + bytes consumed from the window
};
constexpr uint32_t kSel0 = 0x06050400u;   // result bytes: win[k], x[0], x[1], x[2]

// The decoder for a tile in LDS. A refill carries the window's two aligned
// dwords (lo at a, hi at a + 4) on to the next refill. At most 4
// bytes go between refills, so the new aligned start is a or a + 4: the new lo
// is the old lo or the old hi, and only the dword after it is read. One 4-byte
// read per refill costs the LDS about half of reading both dwords when the
// lanes' windows sit at different offsets (6 against 12 cycles per wave
// instruction at a 37-byte lane stride, by the SQ counters of a microbenchmark).
// KEEP_A holds the aligned start a in a register; without it the refill
// compares the old and new window addresses instead (one VALU instruction
// more per refill, one register less per chain).
template <bool KEEP_A>
struct RansLaneCarry {
    uint32_t x, ptr, win, sel;   // as in RansLane
    uint32_t a;                  // ptr rounded down to a dword (held when KEEP_A)
    uint32_t lo, hi;             // the dwords at a and a + 4
};
// State from the 3-byte little-endian flush at LDS address `base`.
template <bool KEEP_A>
__device__ __forceinline__ void rans_init(RansLaneCarry<KEEP_A>& r, uint32_t base) {
    r.x = (uint32_t)(*(lds_u8*)(size_t)base) | ((uint32_t)(*(lds_u8*)(size_t)(base + 1)) << 8) |
          ((uint32_t)(*(lds_u8*)(size_t)(base + 2)) << 16);
    r.ptr = base + kStateBytes;
    r.win = 0;
    r.sel = kSel0;
    r.a = r.ptr & ~3u;
    r.lo = *(lds_u32*)(size_t)r.a;
    r.hi = 0;   // read by the first refill (its aligned start is still a)
}
template <bool KEEP_A>
__device__ __forceinline__ void rans_refill(RansLaneCarry<KEEP_A>& r) {
    const uint32_t np = r.ptr + (r.sel - kSel0);
    const uint32_t na = np & ~3u;
    // the window moved to the next dword when its address crossed a multiple of
    // 4 (it moved by at most 4 bytes)
    const bool up = KEEP_A ? na != r.a : (np ^ r.ptr) >= 4u;
    r.lo = up ? r.hi : r.lo;
    r.hi = *(lds_u32*)(size_t)(na + 4u);
    r.win = __builtin_amdgcn_alignbyte(r.hi, r.lo, np);
    r.ptr = np;
    r.a = na;
    r.sel = kSel0;
}
// Bytes consumed since rans_init.
template <bool KEEP_A>
__device__ __forceinline__ uint32_t rans_consumed(const RansLaneCarry<KEEP_A>& r, uint32_t base) {
    return r.ptr + (r.sel - kSel0) - base;
}

// One rANS decode step (D-Quant section 3.1, Dec): the slot x mod 2^p selects
// the table entry of the symbol m that owns it, the state becomes
// f_m * floor(x / 2^p) + (slot - c_m), and one byte is shifted in when the
// state drops below 2^16 (at most one, since f_m >= 2^(p-8)). The byte comes
// from the window; the shift-in is a v_perm whose selector counts the bytes
// already taken, so the step has no branch. `tab` is the table's absolute
// LDS address. Returns the entry. At most 4 steps may run between refills.
template <class Lane>
__device__ __forceinline__ uint32_t rans_dec_step(Lane& r, uint32_t tab, uint32_t mask, uint32_t p) {
    const uint32_t e = *(lds_u32*)(size_t)(tab + ((r.x & mask) << 2));
    const uint32_t f = (e >> 18) & 1023u;
    const uint32_t bias = (e >> 8) & 1023u;
    const uint32_t xn = __umul24(f, r.x >> p) + bias;       // f < 2^10, x >> p < 2^14
    const uint32_t t = __builtin_amdgcn_perm(xn, r.win, r.sel);
    const bool need = xn < kStateLow;
    r.x = need ? t : xn;
    r.sel += need ? 1u : 0u;
    asm volatile("" : "+v"(r.sel));   // one carry-in add per step (no 0/1 temporaries summed in a tree)
    return e;
}

// The same step from a two-dword entry (wide_entry_pack): one 8-byte table
// read, and the 24-bit multiply-add takes f_m and the bias straight from it.
// The entry's dword 0 carries the level's fp16 high byte in bits 24..31.
template <class Lane>
__device__ __forceinline__ u32x2 rans_lookup_wide(const Lane& r, uint32_t tab, uint32_t mask) {
    return *(lds_u32x2*)(size_t)(tab + ((r.x & mask) << 3));
}
template <class Lane>
__device__ __forceinline__ void rans_advance_wide(Lane& r, u32x2 e, uint32_t p) {
    const uint32_t xn = __umul24(e.x, r.x >> p) + e.y;      // e.x & 0xFFFFFF = f_m
    const uint32_t t = __builtin_amdgcn_perm(xn, r.win, r.sel);
    const bool need = xn < kStateLow;
    r.x = need ? t : xn;
    r.sel += need ? 1u : 0u;
    asm volatile("" : "+v"(r.sel));
}

// Two fp16 levels (dword 0 of the two-dword entries e0 for the lower channel
// and e1 for the upper) packed into one dword: the level's high byte sits in
// bits 24..31 of an entry and its low byte is zero.
__device__ __forceinline__ uint32_t pack_levels_wide(uint32_t e0, uint32_t e1) {
    return __builtin_amdgcn_perm(e1, e0, 0x070C030Cu);
}

}  // namespace dq
