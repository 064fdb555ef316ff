// Cache write (D-Quant sections 4.1-4.3 and 4.5 "Encoding"): rotation,
// normalisation, nearest-level quantisation, drift and rANS encoding of one
// (token, KV head) stream of K or V per wave, bit-exact to the specification:
// every floating-point decision is an IEEE fp64 operation in a fixed order
// with no contraction (this file is compiled with -ffp-contract=off).
#include "dq_internal.h"

#pragma clang fp contract(off)

namespace dq {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxRounds = 64;

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

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per-symbol encode constants of both tables, staged in LDS.
struct SymConst {
    uint32_t freq, cum, lim, magic, shift, pad0, pad1, pad2;
};

struct WaveLds {
    uint64_t key[128];
    int32_t dr[128];
    uint8_t sym[128];
    uint8_t buf[136];
};

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

__global__ __launch_bounds__(64 * kWaves) void encode_kernel(EncArgs a) {
    __shared__ WaveLds wl_all[kWaves];
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
        c.pad0 = c.pad1 = c.pad2 = 0;
        sconst[tid >> 4][m] = c;
    }
    __syncthreads();

    const long nstreams = (long)a.num_tokens * a.num_kv_heads;
    const long sid = (long)blockIdx.x * kWaves + wave;
    if (sid >= 2 * nstreams) return;
    const int kv = sid >= nstreams ? 1 : 0;
    const long rem = sid - kv * nstreams;
    const int token = (int)(rem / a.num_kv_heads), head = (int)(rem % a.num_kv_heads);
    const int slot = a.slot_mapping[token];
    if (slot < 0) return;
    const EncTable* T = a.tables + kv;
    const SymConst* sc = sconst[kv];
    WaveLds& W = wl_all[wave];
    const int M = T->levels, C = T->container, p = T->prob_bits;
    const int32_t budget = T->budget_fx;

    // ---- load (exact widening to fp64); lane holds channels lane and lane+64
    const size_t off = ((size_t)token * a.num_kv_heads + head) * kHeadDim;
    const void* src = kv ? a.v : a.k;
    double y0, y1;
    if (a.dtype == DQ_DTYPE_BF16) {
        const uint16_t* s = (const uint16_t*)src + off;
        y0 = (double)__uint_as_float((uint32_t)s[lane] << 16);
        y1 = (double)__uint_as_float((uint32_t)s[lane + 64] << 16);
    } else {
        const float* s = (const float*)src + off;
        y0 = (double)s[lane];
        y1 = (double)s[lane + 64];
    }

    // ---- rotation y = H x (Sylvester, entries +-1): butterflies of span 1, 2, ..., 64,
    // (a, b) -> (a + b, a - b) for the pair (i, i + h), i mod 2h < h
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
        const double p0 = __shfl_xor(y0, h), p1 = __shfl_xor(y1, h);
        const bool lo = (lane & h) == 0;
        y0 = lo ? y0 + p0 : p0 - y0;
        y1 = lo ? y1 + p1 : p1 - y1;
    }
    {
        const double u = y0, v = y1;
        y0 = u + v;
        y1 = u - v;
    }

    // ---- norm: S by the fixed tree s_j += s_{j+w}, w = 64, 32, ..., 1
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
    const uint16_t rho16 = f64_to_f16_rne(rho);
    double z0 = 0.0, z1 = 0.0;
    if (S > 0.0) {
        z0 = y0 / rho;
        z1 = y1 / rho;
    }

    // ---- nearest level; an exact midpoint goes to the inner level
    int m0 = 0, m1 = 0;
    for (int j = 0; j + 1 < M; ++j) {
        const double bj = T->bounds[j];
        if (bj >= 0.0) {
            m0 += z0 > bj;
            m1 += z1 > bj;
        } else {
            m0 += z0 >= bj;
            m1 += z1 >= bj;
        }
    }
    const int n0 = m0, n1 = m1;
    int R = wave_sum_i(T->cost[m0] + T->cost[m1]);

    const uint64_t lt_mask = (1ull << lane) - 1ull;
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
        // candidates: one level inward and strictly cheaper (section 4.3)
        const int i0 = T->inner[m0], i1 = T->inner[m1];
        const int dr0 = i0 >= 0 ? T->cost[m0] - T->cost[i0] : 0;
        const int dr1 = i1 >= 0 ? T->cost[m1] - T->cost[i1] : 0;
        const bool c0 = i0 >= 0 && dr0 > 0, c1 = i1 >= 0 && dr1 > 0;
        uint64_t k0 = 0, k1 = 0;
        if (c0) {
            const double a0 = z0 - T->recon[i0], b0 = z0 - T->recon[m0];
            const double dd = a0 * a0 - b0 * b0;
            k0 = order_key(dd / (double)dr0);
        }
        if (c1) {
            const double a1 = z1 - T->recon[i1], b1 = z1 - T->recon[m1];
            const double dd = a1 * a1 - b1 * b1;
            k1 = order_key(dd / (double)dr1);
        }
        // compact the candidates in channel order
        const uint64_t bal0 = __ballot(c0), bal1 = __ballot(c1);
        const int pos0 = __popcll(bal0 & lt_mask);
        const int pos1 = __popcll(bal0) + __popcll(bal1 & lt_mask);
        const int nc = __popcll(bal0) + __popcll(bal1);
        if (c0) { W.key[pos0] = k0; W.dr[pos0] = dr0; }
        if (c1) { W.key[pos1] = k1; W.dr[pos1] = dr1; }
        wave_sync();
        // rank and the rate removed by every candidate ahead of this one in (key, channel) order
        int rank0 = 0, rank1 = 0, cb0 = 0, cb1 = 0, tot = 0;
        for (int j = 0; j < nc; ++j) {
            const uint64_t kj = W.key[j];
            const int dj = W.dr[j];
            tot += dj;
            const bool a0 = kj < k0 || (kj == k0 && j < pos0);
            const bool a1 = kj < k1 || (kj == k1 && j < pos1);
            rank0 += a0;
            cb0 += a0 ? dj : 0;
            rank1 += a1;
            cb1 += a1 ? dj : 0;
        }
        wave_sync();
        const int need = R - budget;
        if (tot >= need) {
            int kmin = 0;
            if (need > 0) kmin = __popcll(__ballot(c0 && cb0 < need)) + __popcll(__ballot(c1 && cb1 < need));
            for (int k = kmin; k <= nc; ++k) {
                const int s0 = (c0 && rank0 < k) ? i0 : m0;
                const int s1 = (c1 && rank1 < k) ? i1 : m1;
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
            if (nc == 0) { failed = true; break; }
            // fallback round: every candidate moves, and drift starts again from there
            m0 = c0 ? i0 : m0;
            m1 = c1 ? i1 : m1;
            R = wave_sum_i(T->cost[m0] + T->cost[m1]);
        }
    }

    // ---- store: [state, 3 bytes LE][bytes in decode order][zeros]
    const int page = slot / a.page_size, po = slot - page * a.page_size;
    const size_t idx = ((size_t)page * a.num_kv_heads + head) * a.page_size + po;
    uint8_t* dst = a.cache[kv] + idx * C;
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
        a.norm[kv][idx] = rho16;
        if (a.drift_stats)
            a.drift_stats[((size_t)token * a.num_kv_heads + head) * 2 + kv] =
                (uint16_t)((changed & 255) | ((rounds > 255 ? 255 : rounds) << 8));
        if (failed && a.err_word) atomicOr(a.err_word, DQ_DEVERR_ENCODE);
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

}  // namespace

hipError_t launch_encode(const EncArgs& a, hipStream_t s) {
    const long streams = 2l * a.num_tokens * a.num_kv_heads;
    dim3 grid((unsigned)((streams + kWaves - 1) / kWaves));
    hipLaunchKernelGGL(encode_kernel, grid, dim3(64 * kWaves), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_selftest_fp64(const double* a, const double* b, int n, double* sq, double* dv, uint16_t* f16,
                                hipStream_t s) {
    hipLaunchKernelGGL(selftest_kernel, dim3((n + 255) / 256), dim3(256), 0, s, a, b, n, sq, dv, f16);
    return hipGetLastError();
}

}  // namespace dq
