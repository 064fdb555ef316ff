// Fused decode attention over fixed-size rANS containers (D-Quant section 4.5
// "Decoding"), its split-K log-sum-exp merge, and the symbol-decode test hook.
//
// Work decomposition (one work-group = 4 waves = one (sequence, KV head,
// token split)):
//   * each wave owns 64-token tiles of the split, interleaved with the other
//     waves; one lane decodes one token's stream, so all 64 lanes step through
//     channel i together;
//   * q.k: after every 8 decoded key channels a lane holds 8 fp16 levels of its
//     own token - exactly the B operand of v_mfma_f32_16x16x32_f16 for column
//     (lane % 16) and k-group (lane / 16). A block-diagonal A operand (query
//     head h in row 4*(lane/16) + h, non-zero only in k-group lane/16) makes
//     the 16x16 result land as the 4 head logits of the lane's own token, so
//     no transpose is needed and the affine map is folded in (levels enter
//     the contraction as they come out of the table, the per-token norm and
//     the grid step multiply the logit afterwards);
//   * p.v: the decoded value levels of 16 channels are written to LDS as a
//     [channel][token] tile and contracted over tokens with the softmax
//     weights by two MFMAs per 16 channels;
//   * online softmax in the log2 domain per wave; the 4 waves merge in LDS
//     and write one partial (m, l, acc[128]) per query head and split; a
//     second kernel merges the splits and rotates the result back.
#include "dq_device.h"

namespace dq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;
constexpr int kRowH = 72;                 // fp16 per LDS row of the level / weight tiles
constexpr int kRowB = kRowH * 2;          // bytes
constexpr int kPad = 256;                 // bytes after a container tile (a corrupt stream reads < 132 past its start)
constexpr uint32_t kOffTabK = 0;
constexpr uint32_t kOffTabV = 4096;
constexpr uint32_t kOffQt = 8192;         // [4][128] fp16 rotated queries
constexpr uint32_t kOffZero = 9216;       // 512 zero bytes: A operand of rows without a head
constexpr uint32_t kOffKappa = 9728;      // [4] floats
constexpr uint32_t kOffWaves = 9792;
constexpr float kLog2e = 1.4426950408889634f;

__host__ __device__ inline uint32_t align16(uint32_t v) { return (v + 15u) & ~15u; }

__host__ __device__ inline uint32_t wave_bytes(int ck, int cv) {
    return align16(kTile * ck + kPad) + align16(kTile * cv + kPad) + 16 * kRowB + 4 * kRowB;
}

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
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
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

// Copy the containers of 64 consecutive tokens (4 groups of 16, each group
// contiguous inside one page) of KV head g into LDS at `dst`, 16 bytes per
// lane and load. Groups that start at or past T are skipped.
__device__ __forceinline__ void stage_tile(uint8_t* lds, uint32_t dst, const uint8_t* __restrict__ cache,
                                           int C, const int32_t* __restrict__ bt_row, int log2p, int P,
                                           int hkv, int g, int t0, int T, int lane) {
    const int units = 4 * C;
    for (int u = lane; u < units; u += 64) {
        const int gi = (u >= C) + (u >= 2 * C) + (u >= 3 * C);
        const int off = u - gi * C;
        const int tok = t0 + 16 * gi;
        if (tok < T) {
            const int page = bt_row[tok >> log2p];
            const int o = tok & (P - 1);
            const uint8_t* src = cache + ((size_t)(page * hkv + g) * P + o) * C + (size_t)off * 16;
            const u32x4 v = *(const u32x4*)src;
            *(u32x4*)(lds + dst + (uint32_t)u * 16u) = v;
        }
    }
}

struct AttnLaunch {
    AttnArgs a;
    int log2p;
};

__global__ __launch_bounds__(kThreads) void attn_kernel(AttnLaunch L) {
    const AttnArgs& a = L.a;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = a.group;
    const int T = max(0, min(a.context_lens[b], a.max_pages_per_seq * a.page_size));
    const int start = split * a.split_len;
    const int end = min(T, start + a.split_len);
    const size_t head_stride = (size_t)a.num_splits * kPartStride;
    float* part = a.partials + (((size_t)b * a.num_q_heads + (size_t)g * G) * a.num_splits + split) * kPartStride;
    if (start >= end) {
        if (tid < G) {
            part[tid * head_stride + 0] = -INFINITY;
            part[tid * head_stride + 1] = 0.0f;
        }
        return;
    }

    const uint32_t kcB = align16(kTile * a.ck + kPad), vcB = align16(kTile * a.cv + kPad);
    const uint32_t oW = kOffWaves + (uint32_t)wave * wave_bytes(a.ck, a.cv);
    const uint32_t oKc = oW, oVc = oW + kcB, oVs = oVc + vcB, oWl = oVs + 16 * kRowB;

    // ---- prologue: tables, zero regions, rotated queries
    {
        const uint32_t* ent = a.entries;
        uint32_t* tab = (uint32_t*)lds;
        for (int i = tid; i < 2 * kTableSlots; i += kThreads) tab[i] = ent[i];
        uint32_t* z = (uint32_t*)(lds + kOffZero);
        if (tid < 128) z[tid] = 0u;
        uint32_t* vs = (uint32_t*)(lds + oVs);
        for (int i = lane; i < 16 * kRowB / 4; i += 64) vs[i] = 0u;   // low bytes of the level tile stay 0
    }
    if (wave < G) {
        const int h = g * G + wave;
        const size_t qo = ((size_t)b * a.num_q_heads + h) * kHeadDim;
        float v0, v1;
        if (a.q_dtype == DQ_DTYPE_BF16) {
            const uint16_t* q = (const uint16_t*)a.q + qo;
            v0 = bf16_to_f32(q[lane]);
            v1 = bf16_to_f32(q[lane + 64]);
        } else {
            const float* q = (const float*)a.q + qo;
            v0 = q[lane];
            v1 = q[lane + 64];
        }
        fwht128_f32(v0, v1, lane);
        const float mx = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
        // scale by a power of two so that the largest |q~| lies in [2^14, 2^15): fp16 keeps full precision
        const int e = mx > 0.0f ? f32_exponent(mx) - 14 : 0;
        _Float16* qt = (_Float16*)(lds + kOffQt) + wave * kHeadDim;
        qt[lane] = (_Float16)__builtin_amdgcn_ldexpf(v0, -e);
        qt[lane + 64] = (_Float16)__builtin_amdgcn_ldexpf(v1, -e);
        if (lane == 0)
            ((float*)(lds + kOffKappa))[wave] =
                __builtin_amdgcn_ldexpf(a.softmax_scale * kLog2e * a.step_k / (float)kHeadDim, e);
    }
    __syncthreads();

    const uint32_t* tabK = (const uint32_t*)(lds + kOffTabK);
    const uint32_t* tabV = (const uint32_t*)(lds + kOffTabV);
    const uint32_t maskK = (1u << a.pk) - 1u, maskV = (1u << a.pv) - 1u;
    const uint32_t pk = (uint32_t)a.pk, pv = (uint32_t)a.pv;
    float kap[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) kap[r] = r < G ? ((const float*)(lds + kOffKappa))[r] : 0.0f;

    // MFMA operand addresses (bytes into LDS)
    const int r16 = lane & 15, grp = lane >> 4;
    const uint32_t aq_off = (grp == (r16 >> 2) && (r16 & 3) < G) ? kOffQt + (uint32_t)(r16 & 3) * 256u : kOffZero;
    const uint32_t ap_off = r16 < G ? oWl + (uint32_t)r16 * kRowB + (uint32_t)grp * 16u : kOffZero;
    const uint32_t bp_off = oVs + (uint32_t)r16 * kRowB + (uint32_t)grp * 16u;

    const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages_per_seq;
    const int P = a.page_size, log2p = L.log2p, hkv = a.num_kv_heads;

    float m_run[4], l_lane[4];
    int e_run = -127;
    float4v acc[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) { m_run[r] = -INFINITY; l_lane[r] = 0.0f; }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = float4v{0.f, 0.f, 0.f, 0.f};
    uint32_t bad = 0;

    for (int t0 = start + wave * kTile; t0 < end; t0 += kWaves * kTile) {
        stage_tile(lds, oKc, a.k_cache, a.ck, bt_row, log2p, P, hkv, g, t0, T, lane);
        stage_tile(lds, oVc, a.v_cache, a.cv, bt_row, log2p, P, hkv, g, t0, T, lane);
        const int tok = t0 + lane;
        const bool valid = tok < T;
        float rk = 0.0f, rv = 0.0f;
        if (valid) {
            const int page = bt_row[tok >> log2p];
            const size_t ni = (size_t)(page * hkv + g) * P + (tok & (P - 1));
            rk = f16_to_f32(a.k_norm[ni]);
            rv = f16_to_f32(a.v_norm[ni]);
        }
        wave_lds_sync();

        // ---- keys: decode 128 channels, 16 MFMAs of 8 channels each
        float4v d = float4v{0.f, 0.f, 0.f, 0.f};
        {
            const uint32_t base = oKc + (uint32_t)lane * (uint32_t)a.ck;
            uint32_t x = (uint32_t)lds[base] | ((uint32_t)lds[base + 1] << 8) | ((uint32_t)lds[base + 2] << 16);
            uint32_t ptr = base + kStateBytes;
            bad |= (valid && x < kStateLow) ? 1u : 0u;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                uint32_t e[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) e[jj] = rans_dec_step(x, ptr, tabK, lds, maskK, pk);
                u32x4 bw;
                bw[0] = pack_levels(e[0], e[1]);
                bw[1] = pack_levels(e[2], e[3]);
                bw[2] = pack_levels(e[4], e[5]);
                bw[3] = pack_levels(e[6], e[7]);
                const half8 aq = *(const half8*)(lds + aq_off + 16u * j);
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, __builtin_bit_cast(half8, bw), d, 0, 0, 0);
            }
            bad |= (valid && (x != kStateLow || ptr - base > (uint32_t)a.ck)) ? 1u : 0u;
        }

        // ---- online softmax (log2 domain); lane = token, d[r] = raw logit of head r
        float w[4], alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float s = valid ? d[r] * rk * kap[r] : -INFINITY;
            const float mn = fmaxf(m_run[r], wave_max(s));
            alpha[r] = exp2f(m_run[r] - mn);
            m_run[r] = mn;
            w[r] = exp2f(s - mn);
            l_lane[r] = l_lane[r] * alpha[r] + w[r];
        }
        // value norms enter the p.v weights scaled by a running power of two so fp16 keeps them normal
        const int e_tile = wave_max_i(valid && rv > 0.0f ? f32_exponent(rv) : -127);
        const int e_new = max(e_run, e_tile);
        const float sc = __builtin_amdgcn_ldexpf(1.0f, e_run - e_new);
        e_run = e_new;
        const float rvs = __builtin_amdgcn_ldexpf(rv, -e_new);
        {
            _Float16* wl = (_Float16*)(lds + oWl);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (r < G) wl[r * kRowH + lane] = (_Float16)(valid ? w[r] * rvs : 0.0f);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][r] *= alpha[r] * sc;

        // ---- values: decode 16 channels into the [channel][token] level tile, then 2 MFMAs
        {
            const uint32_t base = oVc + (uint32_t)lane * (uint32_t)a.cv;
            uint32_t x = (uint32_t)lds[base] | ((uint32_t)lds[base + 1] << 8) | ((uint32_t)lds[base + 2] << 16);
            uint32_t ptr = base + kStateBytes;
            bad |= (valid && x < kStateLow) ? 1u : 0u;
            const uint32_t wbase = oVs + (uint32_t)lane * 2u + 1u;
#pragma unroll
            for (int blk = 0; blk < 8; ++blk) {
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const uint32_t e = rans_dec_step(x, ptr, tabV, lds, maskV, pv);
                    lds[wbase + (uint32_t)c * kRowB] = (uint8_t)e;
                }
                wave_lds_sync();
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const half8 av = *(const half8*)(lds + ap_off + 64u * hf);
                    const half8 bv = *(const half8*)(lds + bp_off + 64u * hf);
                    acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[blk], 0, 0, 0);
                }
                wave_lds_sync();
            }
            bad |= (valid && (x != kStateLow || ptr - base > (uint32_t)a.cv)) ? 1u : 0u;
        }
    }
    if (bad && a.err_word) atomicOr(a.err_word, DQ_DEVERR_DECODE);

    // ---- merge the 4 waves of this work-group
    float lsum[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lsum[r] = wave_sum(l_lane[r]);
    __syncthreads();   // every wave is done with its LDS tiles
    float* mg = (float*)(lds + oW);   // reuse this wave's own region: [0..3] m, [4..7] l, [8] e, [16..] acc[4][128]
    if (lane < 16) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) mg[16 + r * kHeadDim + i * 16 + lane] = acc[i][r];
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) { mg[r] = m_run[r]; mg[4 + r] = lsum[r]; }
        mg[8] = (float)e_run;
    }
    __syncthreads();
    const uint32_t wb = wave_bytes(a.ck, a.cv);
    for (int idx = tid; idx < G * kHeadDim; idx += kThreads) {
        const int h = idx >> 7, c = idx & 127;
        float M = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) M = fmaxf(M, ((const float*)(lds + kOffWaves + w2 * wb))[h]);
        float Lh = 0.0f, A = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) {
            const float* m2 = (const float*)(lds + kOffWaves + w2 * wb);
            if (m2[h] == -INFINITY) continue;
            const float f = exp2f(m2[h] - M);
            Lh += m2[4 + h] * f;
            A += __builtin_amdgcn_ldexpf(m2[16 + h * kHeadDim + c] * f, (int)m2[8]);
        }
        float* ph = part + (size_t)h * head_stride;
        if (c == 0) { ph[0] = M; ph[1] = Lh; }
        ph[4 + c] = A * a.step_v;
    }
}

// Merge the splits of one (sequence, query head) by log-sum-exp and rotate
// back: out = H (sum_s acc_s 2^(m_s - M)) / (128 * sum_s l_s 2^(m_s - M)).
__global__ __launch_bounds__(64) void merge_kernel(const float* __restrict__ partials, int splits,
                                                   float* __restrict__ out) {
    const int bh = blockIdx.x, lane = threadIdx.x;
    const float* p = partials + (size_t)bh * splits * kPartStride;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, p[(size_t)s * kPartStride]);
    float L = 0.0f, v0 = 0.0f, v1 = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < splits; ++s) {
            const float* ps = p + (size_t)s * kPartStride;
            if (ps[0] == -INFINITY) continue;
            const float f = exp2f(ps[0] - M);
            L += ps[1] * f;
            v0 += ps[4 + lane] * f;
            v1 += ps[4 + 64 + lane] * f;
        }
    }
    const float inv = L > 0.0f ? 1.0f / (L * (float)kHeadDim) : 0.0f;
    v0 *= inv;
    v1 *= inv;
    fwht128_f32(v0, v1, lane);
    out[(size_t)bh * kHeadDim + lane] = v0;
    out[(size_t)bh * kHeadDim + 64 + lane] = v1;
}

// Test hook: decode 64 contiguous containers per wave into symbol indices.
__global__ __launch_bounds__(kThreads) void decode_symbols_kernel(const uint32_t* __restrict__ ent, int p,
                                                                  int C, const uint8_t* __restrict__ in, int n,
                                                                  uint8_t* __restrict__ out,
                                                                  uint32_t* __restrict__ err) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t* tab = (uint32_t*)lds;
    for (int i = tid; i < kTableSlots; i += kThreads) tab[i] = ent[i];
    const uint32_t oT = 4096u + (uint32_t)wave * align16(kTile * C + kPad);
    const long s0 = ((long)blockIdx.x * kWaves + wave) * kTile;
    const long s1 = (long)n < s0 + kTile ? (long)n : s0 + kTile;
    const long nb = s0 < n ? (s1 - s0) * C : 0;
    const uint8_t* src = in + s0 * C;
    const long full = nb / 16;
    for (long u = lane; u < full; u += 64) *(u32x4*)(lds + oT + u * 16) = *(const u32x4*)(src + u * 16);
    for (long i = full * 16 + lane; i < nb; i += 64) lds[oT + i] = src[i];
    __syncthreads();
    const long s = s0 + lane;
    if (s >= n) return;
    const uint32_t base = oT + (uint32_t)lane * (uint32_t)C;
    uint32_t x = (uint32_t)lds[base] | ((uint32_t)lds[base + 1] << 8) | ((uint32_t)lds[base + 2] << 16);
    uint32_t ptr = base + kStateBytes;
    const bool bad_init = x < kStateLow;
    const uint32_t mask = (1u << p) - 1u;
    uint32_t* o = (uint32_t*)(out + s * kHeadDim);
    for (int i = 0; i < kHeadDim / 4; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) w |= (rans_dec_step(x, ptr, tab, lds, mask, (uint32_t)p) >> 28) << (8 * k);
        o[i] = w;
    }
    if ((bad_init || x != kStateLow || ptr - base > (uint32_t)C) && err) atomicOr(err, DQ_DEVERR_DECODE);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
    AttnLaunch L;
    L.a = a;
    L.log2p = 31 - __builtin_clz((unsigned)a.page_size);
    if ((1 << L.log2p) != a.page_size) return hipErrorInvalidValue;
    const size_t lds = kOffWaves + (size_t)kWaves * wave_bytes(a.ck, a.cv);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)attn_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid(a.num_splits, a.num_kv_heads, a.batch);
    hipLaunchKernelGGL(attn_kernel, grid, dim3(kThreads), lds, s, L);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(merge_kernel, dim3(a.batch * a.num_q_heads), dim3(64), 0, s, a.partials, a.num_splits,
                       a.out);
    return hipGetLastError();
}

hipError_t launch_decode_symbols(const uint32_t* entries, int prob_bits, int levels, int container,
                                 const uint8_t* containers, int n, uint8_t* out, uint32_t* err, hipStream_t s) {
    (void)levels;
    const size_t lds = 4096 + (size_t)kWaves * align16(kTile * container + kPad);
    const int streams_per_block = kWaves * kTile;
    dim3 grid((n + streams_per_block - 1) / streams_per_block);
    hipLaunchKernelGGL(decode_symbols_kernel, grid, dim3(kThreads), lds, s, entries, prob_bits, container,
                       containers, n, out, err);
    return hipGetLastError();
}

}  // namespace dq
