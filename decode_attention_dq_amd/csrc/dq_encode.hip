// Cache write (D-Quant sections 4.1-4.3 and 4.5 "Encoding"): rotation,
// normalisation, nearest-level quantisation, drift and rANS encoding of
// (token, KV head) streams of K and V, bit-exact to the specification: every
// floating-point decision is an IEEE fp64 operation in a fixed order with no
// contraction (this file is compiled with -ffp-contract=off).
//
// Work decomposition: a wave takes up to kPerWave (24) consecutive streams.
//   1. lane = channel, one stream after another (the next stream's inputs are
//      already in flight): rotation, norm, nearest level, the drift candidates
//      and their (key, channel) ranks. What stays in LDS per stream is the
//      symbol row of the minimal candidate prefix and the channels of the
//      next candidates in order.
//   2. lane = stream: the serial rANS encodes run side by side, each in one
//      pass that counts the bytes and keeps them in LDS. A stream whose
//      encoding overflows takes the next candidate and encodes again.
//   3. the whole wave, one stream after another: each container is written
//      from its state and kept bytes, with one store per 64 bytes.
// The table constants the phases read are staged in LDS once per work-group.
// A stream that the first drift round cannot fit (no prefix fits, or it needs
// more extensions than were staged) is redone from scratch by the complete
// per-stream procedure, which also runs the fallback rounds.
#include "dq_token.h"

#include <algorithm>

#pragma clang fp contract(off)

namespace dq {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxRounds = 64;
constexpr int kTail = 16;         // candidates staged per stream beyond the minimal prefix
constexpr int kPerWave = 24;      // most streams a wave takes (lanes of the serial phase)
constexpr int kRow = 132;         // LDS bytes per stream symbol row (an odd number of dwords)

// fp64 -> fp16 bits with a single rounding to nearest even; overflow gives inf.
__device__ uint16_t f64_to_f16_rne(double d) {
    const uint64_t b = (uint64_t)__double_as_longlong(d);
    const uint32_t sign = (uint32_t)(b >> 63) << 15;
    const int exp = (int)((b >> 52) & 0x7FF);
    uint64_t mant = b & ((1ull << 52) - 1);
    if (exp == 0x7FF) return (uint16_t)(sign | 0x7C00u | (mant ? 0x200u : 0u));
    if (exp == 0) return (uint16_t)sign;
    const int e = exp - 1023;
    int shift;
    uint32_t base;
    if (e >= -14) {
        shift = 42;
        base = (uint32_t)(e + 15) << 10;
    } else {
        shift = 28 - e;
        base = 0;
        mant |= 1ull << 52;
        if (shift > 62) return (uint16_t)sign;
    }
    uint64_t q = mant >> shift;
    const uint64_t rem = mant & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) q++;
    const uint32_t r = base + (uint32_t)q;
    return (uint16_t)(r >= 0x7C00u ? (sign | 0x7C00u) : (sign | r));
}

__device__ __forceinline__ double dq_sqrt(double v) { return __builtin_sqrt(v); }

// Order-preserving map of an fp64 key to uint64 (for finite keys).
__device__ __forceinline__ uint64_t order_key(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    return (b >> 63) ? ~b : (b | (1ull << 63));
}

// Integer wave reductions by DPP row operations (no LDS round trips; exact in
// any order). A source lane outside the row reads 0.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xF, true);
}
constexpr int kDppRowShr = 0x110, kDppRowMirror = 0x140, kDppRowHalfMirror = 0x141, kDppBcast15 = 0x142,
              kDppBcast31 = 0x143, kDppQuadSwap1 = 0xB1, kDppQuadSwap2 = 0x4E;

// Sum over the wave, in every lane.
__device__ __forceinline__ int wave_sum_i(int v) {
    v += dpp_i<kDppQuadSwap1>(v);       // lane pairs
    v += dpp_i<kDppQuadSwap2>(v);       // quads
    v += dpp_i<kDppRowHalfMirror>(v);   // half rows
    v += dpp_i<kDppRowMirror>(v);       // rows of 16: every lane holds its row's sum
    v += dpp_i<kDppBcast15, 0xA>(v);    // rows 1, 3 add rows 0, 2
    v += dpp_i<kDppBcast31, 0xC>(v);    // rows 2, 3 add rows 0 + 1: lane 63 holds the total
    return __builtin_amdgcn_readlane(v, 63);
}

// Inclusive prefix sum over the wave's lanes: shifts by 1, 2, 4, 8 inside each
// row of 16, then each row adds the totals of the rows before it.
__device__ __forceinline__ int wave_incl_scan_i(int v, int lane) {
    (void)lane;
    v += dpp_i<kDppRowShr + 1>(v);
    v += dpp_i<kDppRowShr + 2>(v);
    v += dpp_i<kDppRowShr + 4>(v);
    v += dpp_i<kDppRowShr + 8>(v);
    v += dpp_i<kDppBcast15, 0xA>(v);
    v += dpp_i<kDppBcast31, 0xC>(v);
    return v;
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per-symbol encode constants of both tables, staged in LDS.
struct SymConst {
    uint32_t freq, cum, lim, magic, shift, inner, pad0, pad1;
};

// One stream's ranking scratch (phase 1 and the per-stream procedure).
struct Scratch {
    uint64_t key[128];
    int32_t dr[128];
    uint8_t sym[128];
    uint8_t buf[136];
};

struct WaveLds {
    Scratch sc;                   // phase 1; in phases 2 and 3 the streams' byte buffers
    uint8_t sym[kPerWave][kRow];  // symbol row of each stream
    uint8_t ord[kPerWave][kTail]; // channels of the staged candidates, in (key, channel) order
    int32_t kmin[kPerWave];       // candidates in the minimal prefix
    int32_t staged[kPerWave];     // staged candidates; -1: redo with the per-stream procedure
    int32_t meta[kPerWave];       // bit 0: over budget before drift; bits 16..31: rho16
    int32_t cnt[kPerWave];        // phase 2 result: emitted bytes, or -1 (nothing to write here)
    uint32_t xfin[kPerWave];      // phase 2 result: final state
    uint64_t idx[kPerWave];       // phase 2 result: the container's index in its cache
};
// Byte buffer of a phase-2 stream: cap + 1 = C - 2 bytes; the streams of a
// wave share the Scratch area.
constexpr int kBufArea = (int)sizeof(Scratch);
static_assert(kBufArea >= 128 - 2, "a wave must hold the buffer of one stream of the largest container");

// rANS encode of sym[127..0] (section 3.1, Enc) by one lane: before each
// symbol the state is renormalised into [2^(16-p) f, 2^(24-p) f) by emitting
// its low byte (at most once), then x <- floor(x/f) 2^p + (x mod f) + c.
// Returns the number of emitted bytes, or -1 once more than cap were emitted.
__device__ int rans_encode_lane(const uint8_t* sym, const SymConst* sc, int p, int cap, uint8_t* buf,
                                uint32_t& state) {
    uint32_t x = kStateLow;
    int cnt = 0;
    for (int i = kHeadDim - 1; i >= 0; --i) {
        const SymConst c = sc[sym[i]];
        if (x >= c.lim) {
            if (cnt >= cap) return -1;
            buf[cnt++] = (uint8_t)(x & 255u);
            x >>= 8;
        }
        const uint32_t q = __umulhi(x, c.magic) >> c.shift;
        x = x + c.cum + q * ((1u << p) - c.freq);
    }
    state = x;
    return cnt;
}

// Per-symbol encode record, one 16-byte LDS read per step: lim, magic, c_m,
// 2^p - f_m, where lim = 2^(24-p) f_m is the emission threshold and
// floor(x / f_m) = umulhi(x, magic) >> (magic & 31) for x < 2^24 (the host
// chooses the magic so that its low 5 bits are the shift). The records of a
// table sit in one 256-byte aligned block, 16 bytes per symbol.
typedef uint32_t u32x4e __attribute__((ext_vector_type(4)));

// The same encode by one lane in a single pass that both counts and keeps the
// bytes, without branches: the k-th emitted byte goes to buf[cap - k]. Every
// step stores the state's low byte at the emission pointer e = buf + cap -
// (bytes emitted so far), clamped to buf[0], and moves e down only when the
// renormalisation emits; with cnt <= cap emitted bytes they lie in decode
// order at buf[cap + 1 - cnt .. cap] (buf holds cap + 1 bytes). Two groups of
// four records alternate: one group is read while the other is encoded.
// Returns cnt, or -1 when it exceeds cap; xo gets the final state.
__device__ __forceinline__ void rans_emit_group(uint32_t& x, int& e, int lo, const u32x4e (&c)[4]) {
#pragma unroll
    for (int b = 3; b >= 0; --b) {
        const u32x4e r = c[b];
        const bool emit = x >= r.x;
        *(__attribute__((address_space(3))) uint8_t*)(size_t)(uint32_t)max(e, lo) = (uint8_t)(x & 255u);
        e -= emit ? 1 : 0;
        x = emit ? x >> 8 : x;
        const uint32_t q = __umulhi(x, r.y) >> (r.y & 31u);
        x = x + r.z + __umul24(q, r.w);
    }
}
// The records of the 4 symbols of row word w (sym[i .. i + 3]): symbols are
// below 16, so in the word shifted left by 4 byte b is 16 x symbol b, and a
// byte permute puts it under the block's address (whose low byte is zero).
__device__ __forceinline__ void rans_emit_records(uint32_t w, uint32_t rec, u32x4e (&c)[4]) {
    const uint32_t w4 = w << 4;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        c[b] = *(const __attribute__((address_space(3))) u32x4e*)(size_t)__builtin_amdgcn_perm(w4, rec, 0x03020104u + b);
}
__device__ __forceinline__ int rans_emit_lane(const uint8_t* sym, uint32_t rec, int cap, uint8_t* buf, uint32_t& xo) {
    // LDS addresses as int: e goes at most 128 - cap below lo
    const int lo = (int)(uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)buf;
    const int top = lo + cap;
    const uint32_t* words = (const uint32_t*)sym;
    uint32_t x = kStateLow;
    int e = top;
    u32x4e ca[4], cb[4];
    rans_emit_records(words[kHeadDim / 4 - 1], rec, ca);
    uint32_t wb = words[kHeadDim / 4 - 2];
    // word k holds symbols 4k .. 4k + 3; each word is read a group before its records
    for (int k = kHeadDim / 4 - 1; k >= 1; k -= 2) {
        rans_emit_records(wb, rec, cb);
        const uint32_t wa = words[max(k - 2, 0)];   // (clamped reads: no branch, so no early wait)
        rans_emit_group(x, e, lo, ca);
        rans_emit_records(wa, rec, ca);
        wb = words[max(k - 3, 0)];
        rans_emit_group(x, e, lo, cb);
    }
    xo = x;
    // e went below lo only after more than cap emissions
    return e >= lo ? top - e : -1;
}

struct StreamId {
    int kv, token, head;
};
// (32-bit arithmetic: the host keeps 2 num_tokens num_kv_heads below 2^30)
__device__ __forceinline__ StreamId stream_id(const EncArgs& a, long sid) {
    const int nstreams = a.num_tokens * a.num_kv_heads;
    StreamId s;
    s.kv = (int)sid >= nstreams ? 1 : 0;
    const int rem = (int)sid - s.kv * nstreams;
    s.token = rem / a.num_kv_heads;
    s.head = rem - s.token * a.num_kv_heads;
    return s;
}

// Inputs of one stream, widened exactly to fp64; lane holds channels lane and lane + 64.
__device__ __forceinline__ void load_row(const EncArgs& a, const StreamId& s, int lane, double& y0, double& y1) {
    const size_t off = ((size_t)s.token * a.num_kv_heads + s.head) * kHeadDim;
    const void* src = s.kv ? a.v : a.k;
    if (a.dtype == DQ_DTYPE_BF16) {
        const uint16_t* p = (const uint16_t*)src + off;
        y0 = (double)__uint_as_float((uint32_t)p[lane] << 16);
        y1 = (double)__uint_as_float((uint32_t)p[lane + 64] << 16);
    } else {
        const float* p = (const float*)src + off;
        y0 = (double)p[lane];
        y1 = (double)p[lane + 64];
    }
}

// Key channel-mean removal (sections 3.2 and 5): the mean row of the
// 128-token block that starts at call token `first`, found from that token's
// slot; false when the slot is missing or not where a block starts.
__device__ __forceinline__ bool mean_row_at(const int32_t* slot_mapping, int P, int num_kv_heads, int first,
                                            int head, size_t& row) {
    const int slot = slot_mapping[first];
    if (slot < 0) return false;
    const int page = slot / P, off = slot - page * P;
    if (off % (P < kMeanBlock ? P : kMeanBlock) != 0) return false;
    row = ((size_t)page * num_kv_heads + head) * (size_t)mean_rows_per_page(P) + (size_t)(off / kMeanBlock);
    return true;
}

__device__ __forceinline__ bool mean_row(const EncArgs& a, int first, int head, size_t& row) {
    return mean_row_at(a.slot_mapping, a.page_size, a.num_kv_heads, first, head, row);
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return (double)(float)v;   // both conversions exact
}

// The dequantised block mean q * s16 a key stream subtracts after the rotation
// (0 for values and when the removal is off); false when the stream's block has
// no valid mean row.
__device__ __forceinline__ bool stream_mean(const EncArgs& a, const StreamId& id, int lane, double& mh0,
                                            double& mh1) {
    mh0 = 0.0;
    mh1 = 0.0;
    if (!a.k_mean || id.kv != 0) return true;
    size_t row;
    if (!mean_row(a, id.token / kMeanBlock * kMeanBlock, id.head, row)) return false;
    const double sd = f16_bits_to_f64(a.k_mean_scale[row]);
    mh0 = (double)a.k_mean[row * kHeadDim + lane] * sd;
    mh1 = (double)a.k_mean[row * kHeadDim + lane + 64] * sd;
    return true;
}

// Rotation y = H x (Sylvester, entries +-1): butterflies of span 1, 2, ..., 64,
// (a, b) -> (a + b, a - b) for the pair (i, i + h), i mod 2h < h.
__device__ __forceinline__ void fwht_f64(double& y0, double& y1, int lane) {
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
        const double p0 = __shfl_xor(y0, h), p1 = __shfl_xor(y1, h);
        const bool lo = (lane & h) == 0;
        y0 = lo ? y0 + p0 : p0 - y0;
        y1 = lo ? y1 + p1 : p1 - y1;
    }
    const double u = y0, v = y1;
    y0 = u + v;
    y1 = u - v;
}

// The norm S by the fixed tree s_j += s_{j+w}, w = 64, 32, ..., 1,
// rho = sqrt(S / 128), rho16 rounded once, and the unit-RMS values z = y / rho.
__device__ __forceinline__ void normalise(double y0, double y1, int lane, double& z0, double& z1,
                                          uint16_t& rho16) {
    double s = y0 * y0;
    {
        const double s1 = y1 * y1;
        s = s + s1;
    }
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) {
        const double o = __shfl_xor(s, w);
        s = s + o;   // meaningful for lane < w only, as the tree requires
    }
    const double S = __shfl(s, 0);
    const double rho = dq_sqrt(S / 128.0);
    rho16 = f64_to_f16_rne(rho);
    z0 = 0.0;
    z1 = 0.0;
    if (S > 0.0) {
        z0 = y0 / rho;
        z1 = y1 / rho;
    }
}

// Nearest level; an exact midpoint goes to the inner level.
// (unrolled over the largest table, so the boundary reads go out together)
__device__ __forceinline__ int nearest_level(double z, const EncTable* T, int M) {
    int m = 0;
#pragma unroll
    for (int j = 0; j + 1 < kMaxLevels; ++j) {
        if (j + 1 < M) {
            const double bj = T->bounds[j];
            m += (bj >= 0.0 ? z > bj : z >= bj) ? 1 : 0;
        }
    }
    return m;
}

// The drift candidates of the current symbols m0, m1 (one level inward and
// strictly cheaper, section 4.3) with their keys dd / dr, compacted into W in
// channel order; then each candidate's rank in (key, channel) order and the
// rate removed by every candidate ahead of it.
struct Cands {
    int i0, i1, dr0, dr1, rank0, rank1, cb0, cb1, pos0, pos1, nc, tot;
    bool c0, c1;
};
__device__ __forceinline__ Cands rank_candidates(const EncTable* T, double z0, double z1, int m0, int m1,
                                                 int lane, Scratch& W) {
    Cands r;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    r.i0 = T->inner[m0];
    r.i1 = T->inner[m1];
    r.dr0 = r.i0 >= 0 ? T->cost[m0] - T->cost[r.i0] : 0;
    r.dr1 = r.i1 >= 0 ? T->cost[m1] - T->cost[r.i1] : 0;
    r.c0 = r.i0 >= 0 && r.dr0 > 0;
    r.c1 = r.i1 >= 0 && r.dr1 > 0;
    uint64_t k0 = 0, k1 = 0;
    if (r.c0) {
        const double a0 = z0 - T->recon[r.i0], b0 = z0 - T->recon[m0];
        const double dd = a0 * a0 - b0 * b0;
        k0 = order_key(dd / (double)r.dr0);
    }
    if (r.c1) {
        const double a1 = z1 - T->recon[r.i1], b1 = z1 - T->recon[m1];
        const double dd = a1 * a1 - b1 * b1;
        k1 = order_key(dd / (double)r.dr1);
    }
    const uint64_t bal0 = __ballot(r.c0), bal1 = __ballot(r.c1);
    r.pos0 = __popcll(bal0 & lt_mask);
    r.pos1 = __popcll(bal0) + __popcll(bal1 & lt_mask);
    r.nc = __popcll(bal0) + __popcll(bal1);
    if (r.c0) W.key[r.pos0] = k0;
    if (r.c1) W.key[r.pos1] = k1;
    wave_sync();
    // Ranks by key alone. Distinct keys give distinct ranks; candidates with
    // equal keys share one, and only then is the channel order needed.
    r.rank0 = 0; r.rank1 = 0; r.cb0 = 0; r.cb1 = 0; r.tot = 0;
    for (int j = 0; j < r.nc; ++j) {
        const uint64_t kj = W.key[j];
        r.rank0 += kj < k0 ? 1 : 0;
        r.rank1 += kj < k1 ? 1 : 0;
    }
    if (r.c0) W.dr[r.rank0] = r.pos0;
    if (r.c1) W.dr[r.rank1] = r.pos1;
    wave_sync();
    const bool clash = (r.c0 && W.dr[r.rank0] != r.pos0) || (r.c1 && W.dr[r.rank1] != r.pos1);
    wave_sync();
    if (__ballot(clash)) {
        // equal keys: (key, channel) order, counted against every candidate
        if (r.c0) W.dr[r.pos0] = r.dr0;
        if (r.c1) W.dr[r.pos1] = r.dr1;
        wave_sync();
        r.rank0 = 0; r.rank1 = 0;
        for (int j = 0; j < r.nc; ++j) {
            const uint64_t kj = W.key[j];
            const int dj = W.dr[j];
            r.tot += dj;
            const bool a0 = kj < k0 || (kj == k0 && j < r.pos0);
            const bool a1 = kj < k1 || (kj == k1 && j < r.pos1);
            r.rank0 += a0;
            r.cb0 += a0 ? dj : 0;
            r.rank1 += a1;
            r.cb1 += a1 ? dj : 0;
        }
        wave_sync();
        return r;
    }
    // the rate removed ahead of each candidate: exclusive prefix sums of the
    // rates in rank order (lane holds ranks lane and lane + 64)
    if (r.c0) W.dr[r.rank0] = r.dr0;
    if (r.c1) W.dr[r.rank1] = r.dr1;
    wave_sync();
    const int d0 = lane < r.nc ? W.dr[lane] : 0, d1 = lane + 64 < r.nc ? W.dr[lane + 64] : 0;
    const int s0 = wave_incl_scan_i(d0, lane), s1 = wave_incl_scan_i(d1, lane);
    const int t0 = __shfl(s0, 63), t1 = __shfl(s1, 63);
    wave_sync();
    W.dr[lane] = s0 - d0;
    W.dr[lane + 64] = t0 + s1 - d1;
    wave_sync();
    r.tot = t0 + t1;
    if (r.c0) r.cb0 = W.dr[r.rank0];
    if (r.c1) r.cb1 = W.dr[r.rank1];
    wave_sync();
    return r;
}

// The complete per-stream procedure (one wave, lane = channel), including the
// fallback rounds: for the streams the batched path hands back.
__device__ void encode_one(const EncArgs& a, long sid, int lane, Scratch& W, const SymConst (*sconst)[16]) {
    const StreamId id = stream_id(a, sid);
    const int slot = a.slot_mapping[id.token];
    if (slot < 0) return;
    const EncTable* T = a.tables + id.kv;
    const SymConst* sc = sconst[id.kv];
    const int M = T->levels, C = T->container, p = T->prob_bits;
    const int32_t budget = T->budget_fx;
    double y0, y1, z0, z1, mh0, mh1;
    uint16_t rho16;
    if (!stream_mean(a, id, lane, mh0, mh1)) return;   // the mean pass flagged this key block
    load_row(a, id, lane, y0, y1);
    fwht_f64(y0, y1, lane);
    y0 = y0 - mh0;
    y1 = y1 - mh1;
    normalise(y0, y1, lane, z0, z1, rho16);
    int m0 = nearest_level(z0, T, M), m1 = nearest_level(z1, T, M);
    const int n0 = m0, n1 = m1;
    int R = wave_sum_i(T->cost[m0] + T->cost[m1]);

    int rounds = 0;
    bool done = false, failed = false;
    uint32_t state = 0;
    int nbytes = 0;

    // streams already within budget whose encoding fits need no drift
    if (R <= budget) {
        W.sym[lane] = (uint8_t)m0;
        W.sym[lane + 64] = (uint8_t)m1;
        wave_sync();
        int cnt = 0;
        uint32_t st = 0;
        if (lane == 0) cnt = rans_encode_lane(W.sym, sc, p, C - kStateBytes, W.buf, st);
        cnt = __shfl(cnt, 0);
        if (cnt >= 0) {
            done = true;
            nbytes = cnt;
            state = __shfl(st, 0);
        }
        wave_sync();
    }

    while (!done) {
        if (++rounds > kMaxRounds) { failed = true; break; }
        const Cands c = rank_candidates(T, z0, z1, m0, m1, lane, W);
        const int need = R - budget;
        if (c.tot >= need) {
            int kmin = 0;
            if (need > 0) kmin = __popcll(__ballot(c.c0 && c.cb0 < need)) + __popcll(__ballot(c.c1 && c.cb1 < need));
            for (int k = kmin; k <= c.nc; ++k) {
                const int s0 = (c.c0 && c.rank0 < k) ? c.i0 : m0;
                const int s1 = (c.c1 && c.rank1 < k) ? c.i1 : m1;
                W.sym[lane] = (uint8_t)s0;
                W.sym[lane + 64] = (uint8_t)s1;
                wave_sync();
                int cnt = 0;
                uint32_t st = 0;
                if (lane == 0) cnt = rans_encode_lane(W.sym, sc, p, C - kStateBytes, W.buf, st);
                cnt = __shfl(cnt, 0);
                wave_sync();
                if (cnt >= 0) {
                    done = true;
                    nbytes = cnt;
                    state = __shfl(st, 0);
                    m0 = s0;
                    m1 = s1;
                    break;
                }
            }
        }
        if (!done) {
            if (c.nc == 0) { failed = true; break; }
            // fallback round: every candidate moves, and drift starts again from there
            m0 = c.c0 ? c.i0 : m0;
            m1 = c.c1 ? c.i1 : m1;
            R = wave_sum_i(T->cost[m0] + T->cost[m1]);
        }
    }

    // ---- store: [state, 3 bytes LE][bytes in decode order][zeros]
    const int page = slot / a.page_size, po = slot - page * a.page_size;
    const size_t idx = ((size_t)page * a.num_kv_heads + id.head) * a.page_size + po;
    uint8_t* dst = a.cache[id.kv] + idx * C;
    for (int j = lane; j < C; j += 64) {
        uint8_t v = 0;
        if (!failed) {
            if (j < kStateBytes) v = (uint8_t)(state >> (8 * j));
            else if (j < kStateBytes + nbytes) v = W.buf[nbytes - 1 - (j - kStateBytes)];
        }
        dst[j] = v;
    }
    const int changed = wave_sum_i((m0 != n0) + (m1 != n1));
    if (lane == 0) {
        a.norm[id.kv][idx] = rho16;
        if (a.drift_stats)
            a.drift_stats[((size_t)id.token * a.num_kv_heads + id.head) * 2 + id.kv] =
                (uint16_t)((changed & 255) | ((rounds > 255 ? 255 : rounds) << 8));
        if (failed && a.err_word) atomicOr(a.err_word, DQ_DEVERR_ENCODE);
    }
}

// The key channel means of the call's 128-token blocks (sections 3.2, 5): one
// wave per (block, KV head). The rotated rows are added in token order in
// fp64 and divided by 128; the INT8 code takes one fp16 scale
// s16 = fp16(max |mu| / 127) and q = rint(mu / s16) clamped to +-127.
__global__ __launch_bounds__(64 * kWaves) void mean_kernel(EncArgs a) {
    const int lane = threadIdx.x & 63;
    const long w = (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int nblocks = a.num_tokens / kMeanBlock;
    if (w >= (long)nblocks * a.num_kv_heads) return;
    const int blk = (int)(w / a.num_kv_heads), head = (int)(w % a.num_kv_heads);
    size_t row;
    if (!mean_row(a, blk * kMeanBlock, head, row)) {
        if (lane == 0 && a.err_word) atomicOr(a.err_word, DQ_DEVERR_MEAN_SLOT);
        return;
    }
    double acc0 = 0.0, acc1 = 0.0;
    for (int t0 = 0; t0 < kMeanBlock; t0 += 8) {
        double y0[8], y1[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            StreamId id;
            id.kv = 0;
            id.token = blk * kMeanBlock + t0 + u;
            id.head = head;
            load_row(a, id, lane, y0[u], y1[u]);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            fwht_f64(y0[u], y1[u], lane);
            acc0 = acc0 + y0[u];
            acc1 = acc1 + y1[u];
        }
    }
    const double mu0 = acc0 / 128.0, mu1 = acc1 / 128.0;
    double mx = fmax(fabs(mu0), fabs(mu1));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    const uint16_t s16 = f64_to_f16_rne(mx / 127.0);
    const double sd = f16_bits_to_f64(s16);
    int q0 = 0, q1 = 0;
    if (sd > 0.0) {
        q0 = (int)fmin(fmax(__builtin_rint(mu0 / sd), -127.0), 127.0);
        q1 = (int)fmin(fmax(__builtin_rint(mu1 / sd), -127.0), 127.0);
    }
    a.k_mean[row * kHeadDim + lane] = (int8_t)q0;
    a.k_mean[row * kHeadDim + lane + 64] = (int8_t)q1;
    if (lane == 0) a.k_mean_scale[row] = s16;
}

__global__ __launch_bounds__(64 * kWaves, 6) void encode_kernel(EncArgs a, int per_wave) {
    __shared__ WaveLds wl_all[kWaves];
    __shared__ SymConst sconst[2][16];
    __shared__ __attribute__((aligned(256))) u32x4e erec[2][16];
    __shared__ EncTable tl[2];   // the tables' constants, read by phase 1 from LDS
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    WaveLds& W = wl_all[wave];
    const long total = 2l * a.num_tokens * a.num_kv_heads;
    const long sid0 = ((long)blockIdx.x * kWaves + wave) * per_wave;
    const int nb = (int)max(0l, min((long)per_wave, total - sid0));   // streams of this wave, <= kPerWave

    // the first stream's inputs go out before the tables are staged (a row is
    // read whatever its slot: every token of the call has one), and the
    // table loads go out before the first stream's rotation and norm, which
    // need no table (no branch before them: the loads are clamped instead)
    int slot_n = -1;
    double y0n = 0.0, y1n = 0.0, mh0n = 0.0, mh1n = 0.0;
    bool ok_n = false;
    StreamId idn = {0, 0, 0};
    if (nb > 0) {
        idn = stream_id(a, sid0);
        slot_n = a.slot_mapping[idn.token];
        load_row(a, idn, lane, y0n, y1n);
        ok_n = stream_mean(a, idn, lane, mh0n, mh1n);
    }
    constexpr int kTabDw = (int)(2 * sizeof(EncTable) / 4);
    static_assert(kTabDw <= 2 * 64 * kWaves, "two table dwords per thread");
    const uint32_t* tsrc = (const uint32_t*)a.tables;
    const uint32_t tv0 = tsrc[min(tid, kTabDw - 1)], tv1 = tsrc[min(tid + 64 * kWaves, kTabDw - 1)];
    const EncTable* tt = a.tables + ((tid >> 4) & 1);
    const int tm = tid & 15;
    const uint32_t cfreq = tt->freq[tm], ccum = tt->cum[tm], clim = tt->renorm_lim[tm], cmagic = tt->div_magic[tm],
                   cshift = tt->div_shift[tm], cinner = (uint32_t)tt->inner[tm], cp = (uint32_t)tt->prob_bits;
    double z0f = 0.0, z1f = 0.0;
    uint16_t rho16f = 0;
    if (nb > 0) {
        double y0 = y0n, y1 = y1n;
        fwht_f64(y0, y1, lane);
        y0 = y0 - mh0n;
        y1 = y1 - mh1n;
        normalise(y0, y1, lane, z0f, z1f, rho16f);
    }
    if (tid < kTabDw) ((uint32_t*)tl)[tid] = tv0;
    if (tid + 64 * kWaves < kTabDw) ((uint32_t*)tl)[tid + 64 * kWaves] = tv1;
    if (tid < 32) {
        SymConst c;
        c.freq = cfreq;
        c.cum = ccum;
        c.lim = clim;
        c.magic = cmagic;
        c.shift = cshift;
        c.inner = cinner;
        c.pad0 = c.pad1 = 0;
        sconst[tid >> 4][tm] = c;
        erec[tid >> 4][tm] = u32x4e{clim, cmagic, ccum, (1u << cp) - cfreq};
    }
    __syncthreads();
    if (nb == 0) return;
    auto rec_addr = [&](int kv) { return (uint32_t)(size_t)(__attribute__((address_space(3))) u32x4e*)&erec[kv][0]; };

    // ---- phase 1: lane = channel, one stream at a time
    for (int s = 0; s < nb; ++s) {
        const StreamId id = idn;
        const int slot = slot_n;
        const bool ok = ok_n;
        double y0 = y0n, y1 = y1n;
        const double mh0 = mh0n, mh1 = mh1n;
        if (s + 1 < nb) {   // the next stream's inputs go out before this one's work
            idn = stream_id(a, sid0 + s + 1);
            slot_n = a.slot_mapping[idn.token];
            load_row(a, idn, lane, y0n, y1n);
            ok_n = stream_mean(a, idn, lane, mh0n, mh1n);
        }
        if (slot < 0 || !ok) {
            if (lane == 0) W.staged[s] = -2;   // no slot, or a flagged key block: nothing is written
            continue;
        }
        const EncTable* T = &tl[id.kv];
        const int M = T->levels;
        double z0 = z0f, z1 = z1f;   // stream 0's, computed before the barrier
        uint16_t rho16 = rho16f;
        if (s > 0) {
            fwht_f64(y0, y1, lane);
            y0 = y0 - mh0;
            y1 = y1 - mh1;
            normalise(y0, y1, lane, z0, z1, rho16);
        }
        const int m0 = nearest_level(z0, T, M), m1 = nearest_level(z1, T, M);
        const int R = wave_sum_i(T->cost[m0] + T->cost[m1]);
        const Cands c = rank_candidates(T, z0, z1, m0, m1, lane, W.sc);
        const int need = R - T->budget_fx;
        int kmin = 0;
        if (need > 0) kmin = __popcll(__ballot(c.c0 && c.cb0 < need)) + __popcll(__ballot(c.c1 && c.cb1 < need));
        W.sym[s][lane] = (uint8_t)((c.c0 && c.rank0 < kmin) ? c.i0 : m0);
        W.sym[s][lane + 64] = (uint8_t)((c.c1 && c.rank1 < kmin) ? c.i1 : m1);
        if (c.c0 && c.rank0 >= kmin && c.rank0 < kmin + kTail) W.ord[s][c.rank0 - kmin] = (uint8_t)lane;
        if (c.c1 && c.rank1 >= kmin && c.rank1 < kmin + kTail) W.ord[s][c.rank1 - kmin] = (uint8_t)(lane + 64);
        if (lane == 0) {
            // a prefix must remove the excess rate; otherwise the per-stream procedure takes over
            const bool fits = need <= 0 || c.tot >= need;
            W.kmin[s] = kmin;
            W.staged[s] = fits ? min(c.nc - kmin, kTail) : -1;
            W.meta[s] = (need > 0 ? 1 : 0) | ((int)rho16 << 16) | (c.nc - kmin > kTail ? 2 : 0);
        }
    }
    wave_sync();

    // ---- phase 2: lane = stream, the bytes kept in the Scratch area. A wave
    // with a single stream runs its trials side by side instead: lane j
    // encodes the row with the first j staged candidates moved (in a symbol
    // row of its own), and the smallest j that fits is the serial loop's choice.
    const int bstride = a.max_c - 2;
    uint8_t* const bufs = (uint8_t*)&W.sc;
    bool slow = false;
    int bsel0 = 0;   // buffer of stream 0 (the fitting trial's, with trials side by side)
    const int staged0 = W.staged[0];
    if (nb == 1 && staged0 >= 0 && (staged0 + 1) * bstride <= kBufArea) {
        const StreamId id = stream_id(a, sid0);
        const EncTable* T = &tl[id.kv];
        const SymConst* sc = sconst[id.kv];
        const int C = T->container;
        {   // rows 1 .. staged0 start as copies of row 0: lane l copies dwords 8 (l % 4) .. + 7 into row 1 + l / 4
            const uint32_t* src = (const uint32_t*)W.sym[0] + 8 * (lane & 3);
            uint32_t d[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) d[u] = src[u];
            if ((lane >> 2) < staged0) {
                uint32_t* dst = (uint32_t*)W.sym[1 + (lane >> 2)] + 8 * (lane & 3);
#pragma unroll
                for (int u = 0; u < 8; ++u) dst[u] = d[u];
            }
        }
        wave_sync();
        // candidate m moves in the rows of trials j > m: lane m writes its
        // channel's inner level into each of those rows
        if (lane < staged0) {
            const int ch = W.ord[0][lane];
            const uint8_t alt = (uint8_t)sc[W.sym[0][ch]].inner;
            for (int j = lane + 1; j <= staged0; ++j) W.sym[j][ch] = alt;
        }
        wave_sync();
        int cnt = -1;
        uint32_t xo = 0;
        if (lane <= staged0) cnt = rans_emit_lane(W.sym[lane], rec_addr(id.kv), C - kStateBytes, bufs + lane * bstride, xo);
        const uint64_t fit = __ballot(cnt >= 0);
        if (!fit) {
            slow = lane == 0;   // no staged prefix suffices
            if (lane == 0) W.cnt[0] = -1;
        } else {
            bsel0 = __ffsll((long long)fit) - 1;
            if (lane == bsel0) {
                const int slot = a.slot_mapping[id.token];
                const int page = slot / a.page_size, po = slot - page * a.page_size;
                const size_t idx = ((size_t)page * a.num_kv_heads + id.head) * a.page_size + po;
                W.xfin[0] = xo;
                W.idx[0] = idx;
                W.cnt[0] = cnt;
                const int meta = W.meta[0];
                a.norm[id.kv][idx] = (uint16_t)((uint32_t)meta >> 16);
                if (a.drift_stats) {
                    const int k = W.kmin[0] + bsel0;
                    const int rounds = ((meta & 1) || k > 0) ? 1 : 0;
                    a.drift_stats[((size_t)id.token * a.num_kv_heads + id.head) * 2 + id.kv] =
                        (uint16_t)((k & 255) | (rounds << 8));
                }
            }
        }
    } else if (lane < nb) {
        int res = -1;
        if (W.staged[lane] >= 0) {
            const StreamId id = stream_id(a, sid0 + lane);
            const EncTable* T = &tl[id.kv];
            const SymConst* sc = sconst[id.kv];
            const int C = T->container;
            uint8_t* row = W.sym[lane];
            uint8_t* buf = bufs + lane * bstride;
            const int staged = W.staged[lane];
            int used = 0, cnt;
            uint32_t xo = 0;
            while ((cnt = rans_emit_lane(row, rec_addr(id.kv), C - kStateBytes, buf, xo)) < 0 && used < staged) {
                const int ch = W.ord[lane][used++];   // the next candidate moves one level inward
                row[ch] = (uint8_t)sc[row[ch]].inner;
            }
            if (cnt < 0) {
                slow = true;   // the staged candidates did not suffice
            } else {
                const int slot = a.slot_mapping[id.token];
                const int page = slot / a.page_size, po = slot - page * a.page_size;
                const size_t idx = ((size_t)page * a.num_kv_heads + id.head) * a.page_size + po;
                W.xfin[lane] = xo;
                W.idx[lane] = idx;
                res = cnt;
                const int meta = W.meta[lane];
                a.norm[id.kv][idx] = (uint16_t)((uint32_t)meta >> 16);
                if (a.drift_stats) {
                    const int k = W.kmin[lane] + used;
                    const int rounds = ((meta & 1) || k > 0) ? 1 : 0;
                    a.drift_stats[((size_t)id.token * a.num_kv_heads + id.head) * 2 + id.kv] =
                        (uint16_t)((k & 255) | (rounds << 8));
                }
            }
        } else if (W.staged[lane] == -1) {
            slow = true;
        }
        W.cnt[lane] = res;
    }
    wave_sync();

    // ---- phase 3: the whole wave writes each container: [state, 3 bytes LE]
    // [bytes in decode order][zeros]
    for (int s = 0; s < nb; ++s) {
        const int cnt = W.cnt[s];
        if (cnt < 0) continue;
        const StreamId id = stream_id(a, sid0 + s);
        const int C = tl[id.kv].container, cap = C - kStateBytes;
        const uint32_t x = W.xfin[s];
        const uint8_t* buf = bufs + (s == 0 ? bsel0 : s) * bstride;
        uint8_t* dst = a.cache[id.kv] + W.idx[s] * (size_t)C;
        for (int j = lane; j < C; j += 64) {
            uint8_t v = 0;
            if (j < kStateBytes) v = (uint8_t)(x >> (8 * j));
            else if (j < kStateBytes + cnt) v = buf[cap + 1 - cnt + (j - kStateBytes)];
            dst[j] = v;
        }
    }
    wave_sync();   // the slow path below reuses the Scratch area

    // streams handed back: the complete per-stream procedure, from scratch
    uint64_t back = __ballot(slow);
    while (back) {
        const int s = __ffsll((long long)back) - 1;
        back &= back - 1;
        encode_one(a, sid0 + s, lane, W.sc, sconst);
    }
}

__global__ void selftest_kernel(const double* __restrict__ a, const double* __restrict__ b, int n,
                                double* __restrict__ sq, double* __restrict__ dv, uint16_t* __restrict__ f16) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const double x = a[i];
    sq[i] = x >= 0.0 ? dq_sqrt(x) : 0.0;
    dv[i] = x / b[i];
    f16[i] = f64_to_f16_rne(x);
}

// ---------------------------------------------------------------------------
// Per-token format (sections 4.5 "Encoding", 5.1; appendix "Compared
// configurations"): one stream of the 8
// KV heads' 1024 rotated values per token. Lane l holds channels l and l + 64
// of every head, i.e. stream positions 128h + l and 128h + 64 + l: value i of
// a lane (i = 2h + j) sits at position tok_pos(i, lane).
//
// Work decomposition: a wave takes up to kTokBatch consecutive streams.
//   A. lane = channel, one stream after another: load and rotation, the
//      min-max grid and nearest symbols, and the first drift round up to the
//      minimal prefix that brings the rate under the budget; the symbol row
//      stays in LDS.
//   B. lane = stream: the serial rANS encodes run side by side.
//   C. lane = channel, one stream after another: the least-squares refit of
//      (o, s) to the final symbols, the container, the metadata.
// A stream that the first round's minimal prefix does not fit (its bytes
// overflow the container, or no prefix brings the rate under the budget) is
// redone in phase C by the complete per-stream procedure (further candidates,
// further rounds, one lane encoding), so containers, metadata and drift
// statistics are the same. With the configured tables the prefix nearly
// always fits: the rate model is conservative against the coder's bytes.

constexpr int kTokBatch = 8;                   // most streams a wave takes
constexpr int kTokRow = kTokN + 4;             // LDS bytes per symbol row (rows on different banks)
constexpr int kTokSkip = 1 << 30, kTokSlow = 1 << 29;   // stream flags in TokWave::info

__device__ __forceinline__ int tok_pos(int i, int lane) { return 128 * (i >> 1) + 64 * (i & 1) + lane; }

// One wave's LDS for nb streams: the symbol rows, the emission buffers
// (buf_stride bytes per stream, C - 1 used) and the per-stream results.
struct TokWave {
    uint8_t* row;          // [nb][kTokRow]
    uint8_t* buf;          // [nb][buf_stride]
    int32_t* info;         // [nb] rounds << 8 | flags
    int32_t* cnt;          // [nb] emitted bytes
    uint32_t* xfin;        // [nb] final state
};
constexpr int kTokWgLds = 39 * 1024;           // dynamic LDS of a work-group: 4 fit on a CU
__host__ __device__ inline int tok_buf_stride(int max_c) { return (max_c + 3) & ~3; }
__host__ __device__ inline int tok_stream_bytes(int max_c) { return kTokRow + tok_buf_stride(max_c) + 12; }
static_assert(kTokWgLds / kWaves >= kTokRow + kTokMaxC + 12, "a wave must hold at least one stream");
// streams per wave: kTokBatch, fewer when the LDS of kTokBatch would not fit
__host__ __device__ inline int tok_per_wave(int max_c) {
    const int n = kTokWgLds / kWaves / tok_stream_bytes(max_c);
    return n < kTokBatch ? n : kTokBatch;
}

// The rANS encode of one symbol row (section 3.1, Enc) by one lane, storing
// each emitted byte as it goes, without branches: every step stores the
// state's low byte at the next emission slot buf[last - cnt] (clamped to
// buf[0]) and advances cnt only when the renormalisation emits, so the k-th
// emitted byte sits at buf[last - k], and with cnt <= cap < last the cnt
// bytes end up in decode order at buf[last + 1 - cnt ..]. Returns cnt, or -1
// when it exceeds cap; xo gets the final state. One pass serves as both the
// trial and the write.
__device__ int tok_rans_emit(const uint8_t* sym, const SymConst* sc, int p, int cap, uint8_t* buf, int last,
                             uint32_t& xo) {
    uint32_t x = kStateLow;
    int cnt = 0;
    for (int i = kTokN - 4; i >= 0; i -= 4) {
        const uint32_t w = *(const uint32_t*)(sym + i);
#pragma unroll
        for (int b = 3; b >= 0; --b) {
            const SymConst c = sc[(w >> (8 * b)) & 255u];
            const bool emit = x >= c.lim;
            buf[last - min(cnt, last)] = (uint8_t)(x & 255u);
            cnt += emit ? 1 : 0;
            x = emit ? x >> 8 : x;
            const uint32_t q = __umulhi(x, c.magic) >> c.shift;
            x = x + c.cum + q * ((1u << p) - c.freq);
        }
    }
    xo = x;
    return cnt <= cap ? cnt : -1;
}

// Sum of the 16 values of every lane by the fixed halving tree over stream
// positions (v_j += v_{j+w}, w = 512, 256, .., 1): w = 512, 256, 128 pair
// heads inside a lane, w = 64 the lane's two channels, w = 32 .. 1 lanes.
// Every lane gets the total.
__device__ __forceinline__ double tok_fold_sum(const double (&t)[16]) {
    double a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = t[i] + t[i + 8];       // heads h, h + 4
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = a[i] + a[i + 4];       // heads h, h + 2
    const double b0 = a[0] + a[2], b1 = a[1] + a[3];          // heads 0, 1
    double v = b0 + b1;                                        // channels l, l + 64
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) {
        const double o = __shfl_xor(v, w);
        v = v + o;   // meaningful for lane < w, as the tree requires
    }
    return __shfl(v, 0);
}

// The 16 symbols of a lane (value i at stream position tok_pos(i, lane)) as
// 4-bit fields, so that a wave's registers stay small.
struct Nib16 {
    uint32_t w[2];
    __device__ __forceinline__ int get(int i) const { return (int)((w[i >> 3] >> (4 * (i & 7))) & 15u); }
    __device__ __forceinline__ void set(int i, int v) {
        w[i >> 3] = (w[i >> 3] & ~(15u << (4 * (i & 7)))) | ((uint32_t)v << (4 * (i & 7)));
    }
};

// y = H x per head from exact fp64 inputs, minus the dequantised key block
// mean (the stream codes the residual); false when the key stream's block has
// no mean row (the mean pass flagged it; the stream stays unwritten).
__device__ __forceinline__ bool tok_rotated(const TokEncArgs& a, int token, int kv, int lane, double (&y)[16]) {
    const size_t base = (size_t)token * kTokN;
    const void* src = kv ? a.v : a.k;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const size_t at = base + tok_pos(i, lane);
        y[i] = a.dtype == DQ_DTYPE_BF16 ? (double)__uint_as_float((uint32_t)((const uint16_t*)src)[at] << 16)
                                        : (double)((const float*)src)[at];
    }
#pragma unroll
    for (int h = 0; h < 8; ++h) fwht_f64(y[2 * h], y[2 * h + 1], lane);
    if (kv == 0 && a.k_mean) {
        const int first = token / kMeanBlock * kMeanBlock;
#pragma unroll
        for (int h = 0; h < kTokHeads; ++h) {
            size_t row;
            if (!mean_row_at(a.slot_mapping, a.page_size, kTokHeads, first, h, row)) return false;
            const double sd = f16_bits_to_f64(a.k_mean_scale[row]);
            y[2 * h] = y[2 * h] - (double)a.k_mean[row * kHeadDim + lane] * sd;
            y[2 * h + 1] = y[2 * h + 1] - (double)a.k_mean[row * kHeadDim + lane + 64] * sd;
        }
    }
    return true;
}

// The token-wise min-max grid, o = min, s = (max - min) / (M - 1), and the
// nearest grid symbols of u = (y - o) / s (an exact midpoint goes inward).
__device__ __forceinline__ Nib16 tok_nearest(const double (&y)[16], int M, double& go, double& gs) {
    double mn = y[0], mx = y[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
        mn = fmin(mn, y[i]);
        mx = fmax(mx, y[i]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        mn = fmin(mn, __shfl_xor(mn, o));
        mx = fmax(mx, __shfl_xor(mx, o));
    }
    go = mn;
    gs = (mx - mn) / (double)(M - 1);
    const double half = (double)(M - 1) / 2.0;
    Nib16 m = {{0u, 0u}};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        int q = (M - 1) / 2;
        if (gs > 0.0) {
            const double u = (y[i] - go) / gs;
            q = 0;
            for (int j = 1; j < M; ++j) {
                const double b = (double)j - 0.5;
                q += b >= half ? (u > b) : (u >= b);
            }
        }
        m.set(i, q);
    }
    return m;
}

__device__ __forceinline__ void tok_put_row(uint8_t* row, Nib16 m, int lane) {
#pragma unroll
    for (int i = 0; i < 16; ++i) row[tok_pos(i, lane)] = (uint8_t)m.get(i);
}

// The drift candidates of a round that starts at symbols mr (the per-head
// coder's rule in grid units): a symbol whose inward neighbour is strictly
// cheaper, keyed by distortion increase over rate decrease. Returns the
// stream's rate R; `any` tells whether the stream has a candidate.
__device__ __forceinline__ int tok_keys(const double (&y)[16], Nib16 mr, const SymConst* sc, double go, double gs,
                                        uint64_t (&key)[16], bool& any) {
    bool has = false;
    int R = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int mi = mr.get(i);
        const SymConst ci = sc[mi];
        R += (int)ci.pad0;
        const int inn = (int)ci.inner;
        const int dr = inn >= 0 ? (int)ci.pad0 - (int)sc[inn].pad0 : 0;
        key[i] = ~0ull;
        if (inn >= 0 && dr > 0) {
            const double u = gs > 0.0 ? (y[i] - go) / gs : 0.0;
            const double e1 = u - (double)inn, e0 = u - (double)mi;
            const double dd = e1 * e1 - e0 * e0;
            key[i] = order_key(dd / (double)dr);
            has = true;
        }
    }
    any = __any(has);
    return wave_sum_i(R);
}

// The next candidate in (key, position) order: its stream position (every
// lane gets it), or -1 when none is left. Its key is retired.
__device__ __forceinline__ int tok_next(uint64_t (&key)[16], int lane) {
    uint64_t bk = ~0ull;
    int bi = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (key[i] < bk) {   // positions grow with i: the first minimum has the lowest position
            bk = key[i];
            bi = i;
        }
    int bp = tok_pos(bi, lane);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t ok = __shfl_xor(bk, o);
        const int op = __shfl_xor(bp, o);
        if (ok < bk || (ok == bk && op < bp)) {
            bk = ok;
            bp = op;
        }
    }
    if (bk == ~0ull) return -1;
    const int owner = bp & 63, wi = 2 * (bp >> 7) + ((bp >> 6) & 1);
    if (lane == owner) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (i == wi) key[i] = ~0ull;
    }
    return bp;
}

// Moves the symbol at position bp one level inward, from its round-start
// level, in m and in the LDS row; returns the rate it removes (every lane).
__device__ __forceinline__ int tok_move(int bp, Nib16 mr, Nib16& m, const SymConst* sc, uint8_t* row, int lane) {
    const int owner = bp & 63, wi = 2 * (bp >> 7) + ((bp >> 6) & 1);
    int d = 0;
    if (lane == owner) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (i == wi) {
                const int mi = mr.get(i);
                const int inn = (int)sc[mi].inner;
                d = (int)sc[mi].pad0 - (int)sc[inn].pad0;
                m.set(i, inn);
                row[bp] = (uint8_t)inn;
            }
    }
    return __shfl(d, owner);
}

// Least-squares refit of (o, s) to the stored symbols (sums by the halving
// tree), then the container as dwords interleaved across the page's slots
// (dword j of slot po at row j of the page, zero-padded to whole dwords:
// the flushed state for bytes 0..2, then the cnt emitted bytes in decode
// order at bytes[0..cnt), then zeros), (o16, s16) at the slot and the drift
// statistics.
__device__ void tok_store(const TokEncArgs& a, int token, int kv, int slot, int lane, const double (&y)[16],
                          Nib16 m, Nib16 nearest, int rounds, int cnt, uint32_t xs, const uint8_t* bytes, int C) {
    double t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = (double)m.get(i);
    const double mbar = tok_fold_sum(t) / (double)kTokN;
    const double ybar = tok_fold_sum(y) / (double)kTokN;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const double dm = (double)m.get(i) - mbar;
        t[i] = dm * dm;
    }
    const double smm = tok_fold_sum(t);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const double dm = (double)m.get(i) - mbar;
        const double dy = y[i] - ybar;
        t[i] = dm * dy;
    }
    const double smy = tok_fold_sum(t);
    const double s_star = smm > 0.0 ? smy / smm : 0.0;
    const double o_star = ybar - s_star * mbar;

    const int C4 = (C + 3) >> 2;
    const int page = slot / a.page_size, po = slot - page * a.page_size;
    const size_t idx = (size_t)page * a.page_size + po;
    uint32_t* dst = (uint32_t*)a.cache[kv] + (size_t)page * C4 * a.page_size + po;
    for (int j = lane; j < C4; j += 64) {
        uint32_t d = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int b = 4 * j + k;
            const uint32_t v = b < kStateBytes ? (xs >> (8 * b)) & 255u
                               : (b < kStateBytes + cnt ? (uint32_t)bytes[b - kStateBytes] : 0u);
            d |= v << (8 * k);
        }
        dst[(size_t)j * a.page_size] = d;
    }
    if (lane == 0) {
        a.meta[kv][2 * idx] = f64_to_f16_rne(o_star);
        a.meta[kv][2 * idx + 1] = f64_to_f16_rne(s_star);
    }
    if (a.drift_stats) {
        int changed = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) changed += m.get(i) != nearest.get(i);
        changed = wave_sum_i(changed);
        if (lane == 0) a.drift_stats[(size_t)token * 2 + kv] = (uint32_t)changed | ((uint32_t)rounds << 16);
    }
}

// The complete per-stream procedure (one wave, one lane encoding): the
// nearest symbols, then drift rounds whose candidates leave in (key,
// position) order, each round up to the minimal prefix that brings the rate
// under the budget and then one more at a time until the rANS stream fits
// the container; a round that runs out of candidates moves them all and the
// next round starts. `row` and `buf` (C - 1 bytes) are this wave's LDS.
__device__ void tok_encode_one(const TokEncArgs& a, int token, int kv, int lane, const SymConst* sc, uint8_t* row,
                               uint8_t* buf) {
    const int slot = a.slot_mapping[token];
    if (slot < 0) return;
    const EncTable* T = a.tables + kv;
    const int M = T->levels, C = T->container, p = T->prob_bits;
    const int B = T->budget_fx, cap = C - kStateBytes, last = C - 2;
    double y[16];
    if (!tok_rotated(a, token, kv, lane, y)) return;
    double go, gs;
    const Nib16 nearest = tok_nearest(y, M, go, gs);
    Nib16 m = nearest;
    wave_sync();
    tok_put_row(row, m, lane);
    int R = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) R += (int)sc[m.get(i)].pad0;
    R = wave_sum_i(R);
    bool done = false, failed = false;
    int cnt = -1, rounds = 0;
    uint32_t xfin = 0;
    auto emit = [&]() {
        wave_sync();
        if (lane == 0) cnt = tok_rans_emit(row, sc, p, cap, buf, last, xfin);
        cnt = __shfl(cnt, 0);
        return cnt >= 0;
    };
    if (R <= B) done = emit();
    while (!done) {
        if (++rounds > kMaxRounds) {
            failed = true;
            break;
        }
        const Nib16 mr = m;   // the round's starting symbols
        uint64_t key[16];
        bool any;
        R = tok_keys(y, mr, sc, go, gs, key, any);
        if (!any) {
            failed = true;
            break;
        }
        int removed = 0, bp = 0;
        while (R - removed > B && (bp = tok_next(key, lane)) >= 0) removed += tok_move(bp, mr, m, sc, row, lane);
        if (R - removed <= B) {
            for (;;) {
                if (emit()) {
                    done = true;
                    break;
                }
                if ((bp = tok_next(key, lane)) < 0) break;
                tok_move(bp, mr, m, sc, row, lane);
            }
        }
    }
    if (failed) {
        if (lane == 0 && a.err_word) atomicOr(a.err_word, DQ_DEVERR_ENCODE);
        return;
    }
    const uint32_t xs = (uint32_t)__shfl((int)xfin, 0);
    wave_sync();
    tok_store(a, token, kv, slot, lane, y, m, nearest, rounds, cnt, xs, buf + last + 1 - cnt, C);
}

// 4 waves per SIMD (4 work-groups per CU, the register bound spills): 5.7 ms for
// 262,144 streams, against 6.5 ms at 3 and 6.1-6.3 ms at 5-6 waves per SIMD.
__global__ __launch_bounds__(64 * kWaves, 4) void token_encode_kernel(TokEncArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t tok_lds[];
    __shared__ SymConst sconst[2][16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < 32) {
        const EncTable* t = a.tables + (tid >> 4);
        const int m = tid & 15;
        SymConst c;
        c.freq = t->freq[m];
        c.cum = t->cum[m];
        c.lim = t->renorm_lim[m];
        c.magic = t->div_magic[m];
        c.shift = t->div_shift[m];
        c.inner = (uint32_t)t->inner[m];
        c.pad0 = (uint32_t)t->cost[m];   // the symbol's fixed-point cost
        c.pad1 = 0;
        sconst[tid >> 4][m] = c;
    }
    __syncthreads();
    const int per_wave = tok_per_wave(a.max_c);
    const long total = 2l * a.num_tokens;
    const long sid0 = ((long)blockIdx.x * kWaves + wave) * per_wave;
    if (sid0 >= total) return;
    const int nb = (int)min((long)per_wave, total - sid0);
    const int bstride = tok_buf_stride(a.max_c);
    uint8_t* base = tok_lds + (size_t)wave * per_wave * tok_stream_bytes(a.max_c);
    TokWave W;
    W.row = base;
    W.buf = W.row + per_wave * kTokRow;
    W.info = (int32_t*)(W.buf + per_wave * bstride);
    W.cnt = W.info + per_wave;
    W.xfin = (uint32_t*)(W.cnt + per_wave);

    // ---- phase A: lane = channel, one stream at a time
    for (int s = 0; s < nb; ++s) {
        const long sid = sid0 + s;
        const int token = (int)(sid >> 1), kv = (int)(sid & 1);
        const EncTable* T = a.tables + kv;
        const SymConst* sc = sconst[kv];
        const int M = T->levels, B = T->budget_fx;
        uint8_t* row = W.row + s * kTokRow;
        double y[16];
        if (a.slot_mapping[token] < 0 || !tok_rotated(a, token, kv, lane, y)) {
            if (lane == 0) W.info[s] = kTokSkip;
            continue;
        }
        double go, gs;
        Nib16 m = tok_nearest(y, M, go, gs);
        tok_put_row(row, m, lane);
        int R = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) R += (int)sc[m.get(i)].pad0;
        R = wave_sum_i(R);
        // over the budget: the first round's candidates move up to the minimal
        // prefix
        int info = 0;
        if (R > B) {
            const Nib16 mr = m;
            uint64_t key[16];
            bool any;
            tok_keys(y, mr, sc, go, gs, key, any);
            int removed = 0, bp = 0;
            while (R - removed > B && (bp = tok_next(key, lane)) >= 0) removed += tok_move(bp, mr, m, sc, row, lane);
            info = R - removed > B ? kTokSlow : 1 << 8;   // no prefix fits: later rounds, in the per-stream procedure
        }
        if (lane == 0) W.info[s] = info;
    }
    wave_sync();

    // ---- phase B: lane = stream, the serial encodes side by side
    if (lane < nb && !(W.info[lane] & (kTokSkip | kTokSlow))) {
        const int kv = (int)((sid0 + lane) & 1);
        const EncTable* T = a.tables + kv;
        const SymConst* sc = sconst[kv];
        const int C = T->container, p = T->prob_bits;
        uint8_t* row = W.row + lane * kTokRow;
        uint8_t* buf = W.buf + lane * bstride;
        uint32_t xf;
        const int cnt = tok_rans_emit(row, sc, p, C - kStateBytes, buf, C - 2, xf);
        if (cnt < 0) W.info[lane] |= kTokSlow;   // the bytes overflow: further candidates, per stream
        W.cnt[lane] = cnt;
        W.xfin[lane] = xf;
    }
    wave_sync();

    // ---- phase C: lane = channel, one stream at a time
    for (int s = 0; s < nb; ++s) {
        const int info = W.info[s];
        if (info & kTokSkip) continue;
        const long sid = sid0 + s;
        const int token = (int)(sid >> 1), kv = (int)(sid & 1);
        const SymConst* sc = sconst[kv];
        const EncTable* T = a.tables + kv;
        const int C = T->container;
        uint8_t* row = W.row + s * kTokRow;
        uint8_t* buf = W.buf + s * bstride;
        if (info & kTokSlow) {
            tok_encode_one(a, token, kv, lane, sc, row, buf);
            continue;
        }
        double y[16];
        tok_rotated(a, token, kv, lane, y);
        double go, gs;
        const Nib16 nearest = tok_nearest(y, T->levels, go, gs);
        Nib16 m = {{0u, 0u}};
#pragma unroll
        for (int i = 0; i < 16; ++i) m.set(i, row[tok_pos(i, lane)]);
        const int cnt = W.cnt[s];
        tok_store(a, token, kv, a.slot_mapping[token], lane, y, m, nearest, (info >> 8) & 1, cnt, W.xfin[s],
                  buf + (C - 2) + 1 - cnt, C);
    }
}

// Symbols of per-token containers, one stream per thread, straight from the
// container bytes (a plain decoder for checking the cache write): slot =
// x mod 2^p, m = the symbol whose [c_m, c_m + f_m) holds the slot, x =
// f_m floor(x / 2^p) + slot - c_m, one byte shifted in while x < 2^16.
__global__ void token_decode_symbols_kernel(const EncTable* __restrict__ T, const uint8_t* __restrict__ cont,
                                            int n, uint8_t* __restrict__ out, uint32_t* err) {
    const int sid = blockIdx.x * blockDim.x + threadIdx.x;
    if (sid >= n) return;
    const int M = T->levels, C = T->container, p = T->prob_bits;
    const uint8_t* c = cont + (size_t)sid * C;
    uint32_t x = (uint32_t)c[0] | ((uint32_t)c[1] << 8) | ((uint32_t)c[2] << 16);
    int ptr = kStateBytes;
    bool ok = true;
    for (int i = 0; i < kTokN; ++i) {
        const uint32_t slot = x & ((1u << p) - 1u);
        int s = 0;
        while (s + 1 < M && T->cum[s + 1] <= slot) ++s;
        x = T->freq[s] * (x >> p) + slot - T->cum[s];
        if (x < kStateLow) {
            x = (x << 8) | (ptr < C ? c[ptr] : 0u);
            ++ptr;
            if (x < kStateLow) ok = false;
        }
        out[(size_t)sid * kTokN + i] = (uint8_t)s;
    }
    if (!(ok && x == kStateLow && ptr <= C) && err) atomicOr(err, DQ_DEVERR_DECODE);
}

}  // namespace

// Streams per wave: kPerWave (one per lane in the serial phase) for large
// writes; fewer when that would leave the chip short of waves (about 6144 fit
// at once: 256 CUs x 24), since a wave walks its streams one at a time first.
// Waves stalled on fp64 divide chains and cross-lane moves are hidden by
// occupancy: 24 streams per wave keep the LDS at 24 KB per work-group and the
// launch bound holds the registers to 80 (a few spill), so 6 waves share a
// SIMD (Llama-shaped write: 4.07 ms at 32 streams and 5 waves, 3.98 ms here).
hipError_t launch_encode(const EncArgs& a, hipStream_t s) {
    if (a.k_mean) {
        const long waves = (long)(a.num_tokens / kMeanBlock) * a.num_kv_heads;
        hipLaunchKernelGGL(mean_kernel, dim3((unsigned)((waves + kWaves - 1) / kWaves)), dim3(64 * kWaves), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long streams = 2l * a.num_tokens * a.num_kv_heads;
    const long waves_wanted = 6144;
    const int buf_streams = kBufArea / (a.max_c - 2);   // byte buffers that fit in a wave's Scratch area
    const int per_wave = (int)std::min((long)std::min(kPerWave, buf_streams),
                                       std::max(1l, (streams + waves_wanted - 1) / waves_wanted));
    const long per_block = (long)per_wave * kWaves;
    dim3 grid((unsigned)((streams + per_block - 1) / per_block));
    hipLaunchKernelGGL(encode_kernel, grid, dim3(64 * kWaves), 0, s, a, per_wave);
    return hipGetLastError();
}

hipError_t launch_token_encode(const TokEncArgs& a, hipStream_t s) {
    if (a.k_mean) {
        // the per-head mean pass over [num_tokens][8][128] key rows
        EncArgs m = {};
        m.k = a.k;
        m.dtype = a.dtype;
        m.num_tokens = a.num_tokens;
        m.num_kv_heads = kTokHeads;
        m.page_size = a.page_size;
        m.slot_mapping = a.slot_mapping;
        m.err_word = a.err_word;
        m.k_mean = a.k_mean;
        m.k_mean_scale = a.k_mean_scale;
        const long waves = (long)(a.num_tokens / kMeanBlock) * kTokHeads;
        hipLaunchKernelGGL(mean_kernel, dim3((unsigned)((waves + kWaves - 1) / kWaves)), dim3(64 * kWaves), 0, s, m);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long streams = 2l * a.num_tokens;
    const int per_wave = tok_per_wave(a.max_c);
    const long per_block = (long)per_wave * kWaves;
    dim3 grid((unsigned)((streams + per_block - 1) / per_block));
    hipLaunchKernelGGL(token_encode_kernel, grid, dim3(64 * kWaves),
                       (size_t)kWaves * per_wave * tok_stream_bytes(a.max_c), s, a);
    return hipGetLastError();
}

hipError_t launch_token_decode_symbols(const EncTable* table, const uint8_t* containers, int n, uint8_t* out,
                                       uint32_t* err, hipStream_t s) {
    hipLaunchKernelGGL(token_decode_symbols_kernel, dim3((n + 63) / 64), dim3(64), 0, s, table, containers, n,
                       out, err);
    return hipGetLastError();
}

hipError_t launch_selftest_fp64(const double* a, const double* b, int n, double* sq, double* dv, uint16_t* f16,
                                hipStream_t s) {
    hipLaunchKernelGGL(selftest_kernel, dim3((n + 255) / 256), dim3(256), 0, s, a, b, n, sq, dv, f16);
    return hipGetLastError();
}

}  // namespace dq
