// Attention partial of the bf16 window of recent tokens, merged with the
// compressed partials by log-sum-exp.
#include "dq_device.h"
#include "dq_wave.h"

namespace dq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Attention partial of the uncompressed recent-token window (the paper keeps
// the most recent tokens in BF16, section 5.1). For each query head of KV head
// g: m = max logit, l = sum_t 2^(s_t - m) and acc = H (sum_t 2^(s_t - m) v_t),
// in the same log2 logit scale and rotated output domain as the compressed
// partials, written to slot `slot` so that merge_kernel combines them. Window
// rows are in the original domain. One work-group per (KV head, sequence); wave
// w takes window tokens [64w, 64w + 64) for all query heads of the group: lane
// t computes its token's logits from one K row; for p.v, lane (c, r) takes
// channels 8c..8c+7 of the wave's tokens r, r + 4, ... (16-byte row loads,
// all in flight at once). The lane groups are summed by shuffles, the waves'
// maxima, sums and accumulators in LDS. A kernel of its own: inlined into the decode kernel
// it costs that kernel's schedule more than it saves.
static_assert(kWindowMax == 64 * kWaves, "one window token per thread");
__global__ __launch_bounds__(kThreads) void window_kernel(AttnArgs a, int slot) {
    __shared__ float qs[4][kHeadDim];
    __shared__ float ps[4][kWindowMax];          // weights [head][token]
    __shared__ float wo[kWaves][4][kHeadDim];    // per-wave p.v accumulators
    __shared__ float wm[kWaves][4], wsum[kWaves][4];
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = a.group;
    const int W = max(0, min(a.win_lens[b], a.win_cap));
    const size_t hs = (size_t)a.slot_count * kPartStride;
    float* part = a.partials + (((size_t)b * a.num_q_heads + (size_t)g * G) * a.slot_count + slot) * kPartStride;
    if (W == 0) {
        if (tid < G) { part[tid * hs] = -INFINITY; part[tid * hs + 1] = 0.0f; }
        return;
    }
    for (int i = tid; i < G * kHeadDim; i += kThreads) {
        const size_t qo = ((size_t)b * a.num_q_heads + g * G + i / kHeadDim) * kHeadDim + i % kHeadDim;
        qs[i / kHeadDim][i % kHeadDim] =
            a.q_dtype == DQ_DTYPE_BF16 ? bf16_to_f32(((const uint16_t*)a.q)[qo]) : ((const float*)a.q)[qo];
    }
    __syncthreads();
    const size_t rows = ((size_t)b * a.num_kv_heads + g) * a.win_cap;
    const uint16_t* kr = a.win_k + rows * kHeadDim;
    const uint16_t* vr = a.win_v + rows * kHeadDim;
    const float sc = a.softmax_scale * kLog2e;
    const int t = 64 * wave + lane;
    float s[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (t < W) {
        const uint16_t* row = kr + (size_t)t * kHeadDim;
        u32x4 kw[kHeadDim / 8];   // the whole row in flight at once
#pragma unroll
        for (int i = 0; i < kHeadDim / 8; ++i) kw[i] = *(const u32x4*)(row + 8 * i);
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < kHeadDim / 8; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float k0 = __uint_as_float(kw[i][k] << 16), k1 = __uint_as_float(kw[i][k] & 0xFFFF0000u);
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    if (h < G) acc[h] += qs[h][8 * i + 2 * k] * k0 + qs[h][8 * i + 2 * k + 1] * k1;
            }
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) s[h] = acc[h] * sc;
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const float mw = wave_max(s[h]);
        if (lane == 0) wm[wave][h] = mw;
    }
    __syncthreads();
    float M[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        M[h] = fmaxf(fmaxf(wm[0][h], wm[1][h]), fmaxf(wm[2][h], wm[3][h]));
        const float p = (t < W && h < G) ? exp2f(s[h] - M[h]) : 0.0f;
        ps[h][t] = p;
        const float lw = wave_sum(p);
        if (lane == 0) wsum[wave][h] = lw;
    }
    wave_lds_sync();
    // p.v: lane (c, r) takes channels 8c..8c+7 of the wave's tokens 4k + r
    const int c8 = lane & 15, r = lane >> 4;
    float o[4][8];
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[h][j] = 0.0f;
    // tokens at or past W have weight 0; their loads read row W - 1 instead
    u32x4 w8[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int u = min(64 * wave + 4 * k + r, W - 1);
        w8[k] = *(const u32x4*)(vr + (size_t)u * kHeadDim + 8 * c8);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int u = 64 * wave + 4 * k + r;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float p = ps[h][u];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                o[h][2 * j] += p * __uint_as_float(w8[k][j] << 16);
                o[h][2 * j + 1] += p * __uint_as_float(w8[k][j] & 0xFFFF0000u);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            o[h][j] += __shfl_xor(o[h][j], 16);
            o[h][j] += __shfl_xor(o[h][j], 32);
        }
    if (r == 0) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) wo[wave][h][8 * c8 + j] = o[h][j];
    }
    __syncthreads();
    if (wave < G) {
        const int h = wave;
        float o0 = 0.0f, o1 = 0.0f, L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            o0 += wo[w][h][lane];
            o1 += wo[w][h][64 + lane];
            L += wsum[w][h];
        }
        fwht128_f32(o0, o1, lane);
        float* ph = part + (size_t)h * hs;
        if (lane == 0) { ph[0] = M[h]; ph[1] = L; }
        ph[4 + lane] = o0;
        ph[4 + 64 + lane] = o1;
    }
}

}  // namespace

hipError_t launch_window(const AttnArgs& a, int slot, hipStream_t s) {
    hipLaunchKernelGGL(window_kernel, dim3(a.num_kv_heads, a.batch), dim3(kThreads), 0, s, a, slot);
    return hipGetLastError();
}

}  // namespace dq
