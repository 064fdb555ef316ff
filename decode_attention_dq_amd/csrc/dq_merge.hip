// Split-K log-sum-exp merge of attention partials (m, l, acc[128]) per
// (sequence, query head), shared by the compressed and the bf16 kernels.
#include "dq_internal.h"
#include "dq_sched.h"
#include "dq_wave.h"

namespace dq {
namespace {

// Merge the splits of one (sequence, query head) by log-sum-exp and rotate
// back: out = H (sum_s acc_s 2^(m_s - M)) / (128 * sum_s l_s 2^(m_s - M)),
// or, for partials in the original domain (ROTATED false),
// out = (sum_s acc_s 2^(m_s - M)) / (sum_s l_s 2^(m_s - M)). The splits are
// the ceil(T_b / split_len) that hold tokens of sequence b, plus the window
// slot when there is one. W waves share them (wave w takes the w-th, the
// (w + W)-th, ...), each lane two channels; the loads of different splits are
// independent, so many are in flight at once. W = 4 waves per row, or 16 when
// there are few rows with many splits (a long single sequence), so that each
// wave walks fewer splits one after another.
template <bool ROTATED, int kMergeWaves>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(MergeArgs a) {
    __shared__ float red[kMergeWaves][132];
    const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* p = a.partials + (size_t)bh * a.slot_count * kPartStride;
    const int len = a.context_lens[bh / a.num_q_heads];
    const int T = covered_tokens(len, a.cap);
    if (tid == 0 && a.err_word && (len < 0 || len > a.cap)) atomicOr(a.err_word, DQ_DEVERR_CONTEXT);
    const int n = (T + a.split_len - 1) / a.split_len;
    const int slots = n + (a.window_slot >= 0 ? 1 : 0);
    auto slot = [&](int i) { return i < n ? i : a.window_slot; };
    float M = -INFINITY;
    for (int i = tid; i < slots; i += 64 * kMergeWaves) M = fmaxf(M, p[(size_t)slot(i) * kPartStride]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    if (lane == 0) red[wave][0] = M;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) M = fmaxf(M, red[w][0]);
    __syncthreads();
    float L = 0.0f, v0 = 0.0f, v1 = 0.0f;
    if (M != -INFINITY) {
#pragma unroll 4
        for (int i = wave; i < slots; i += kMergeWaves) {
            const float* ps = p + (size_t)slot(i) * kPartStride;
            const float ms = ps[0];
            if (ms == -INFINITY) continue;
            const float f = exp2f(ms - M);
            L += ps[1] * f;
            v0 += ps[4 + lane] * f;
            v1 += ps[4 + 64 + lane] * f;
        }
    }
    red[wave][lane] = v0;
    red[wave][64 + lane] = v1;
    if (lane == 0) red[wave][128] = L;
    __syncthreads();
    if (wave != 0) return;
    v0 = 0.0f;
    v1 = 0.0f;
    L = 0.0f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) {
        v0 += red[w][lane];
        v1 += red[w][64 + lane];
        L += red[w][128];
    }
    const float inv = L > 0.0f ? 1.0f / (ROTATED ? L * (float)kHeadDim : L) : 0.0f;
    v0 *= inv;
    v1 *= inv;
    if (ROTATED) fwht128_f32(v0, v1, lane);
    a.out[(size_t)bh * kHeadDim + lane] = v0;
    a.out[(size_t)bh * kHeadDim + 64 + lane] = v1;
}

// The same merge for few rows with up to 128 partials: 16 waves per row, wave
// w holding slots w, w + 16, ..., w + 112 in registers. Every load of a wave
// goes out at once, before the row's context length and maximum are known
// (one memory round trip); slots without tokens are dropped afterwards.
template <bool ROTATED>
__global__ __launch_bounds__(64 * 16) void merge_wide_kernel(MergeArgs a) {
    constexpr int kW = 16, kPer = 8;
    __shared__ float red[kW][132];
    const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const float* p = a.partials + (size_t)bh * a.slot_count * kPartStride;
    // the loads go out before the context length is known: slots i < min(slot_count,
    // 128) (the host picks this kernel when a row's partials fit; a slot past them
    // can only be the unused window slot); which hold tokens is settled after
    const int sc = min(a.slot_count, kW * kPer);
    float ms[kPer], ls[kPer], x0[kPer], x1[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        const int i = wave + c * kW;
        ms[c] = -INFINITY;
        ls[c] = x0[c] = x1[c] = 0.0f;
        if (i < sc) {
            const float* ps = p + (size_t)i * kPartStride;
            ms[c] = ps[0];
            ls[c] = ps[1];
            x0[c] = ps[4 + lane];
            x1[c] = ps[4 + 64 + lane];
        }
    }
    const int len = a.context_lens[bh / a.num_q_heads];
    const int T = covered_tokens(len, a.cap);
    if (tid == 0 && a.err_word && (len < 0 || len > a.cap)) atomicOr(a.err_word, DQ_DEVERR_CONTEXT);
    const int n = (T + a.split_len - 1) / a.split_len;
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        const int i = wave + c * kW;
        if (!(i < n || i == a.window_slot)) ms[c] = -INFINITY;   // a partial without tokens may hold anything
    }
    float M = ms[0];
#pragma unroll
    for (int c = 1; c < kPer; ++c) M = fmaxf(M, ms[c]);
    if (lane == 0) red[wave][0] = M;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kW; ++w) M = fmaxf(M, red[w][0]);
    __syncthreads();
    float L = 0.0f, v0 = 0.0f, v1 = 0.0f;
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        if (ms[c] != -INFINITY) {   // a partial without tokens may hold anything
            const float f = exp2f(ms[c] - M);
            L += ls[c] * f;
            v0 += x0[c] * f;
            v1 += x1[c] * f;
        }
    }
    red[wave][lane] = v0;
    red[wave][64 + lane] = v1;
    if (lane == 0) red[wave][128] = L;
    __syncthreads();
    if (wave != 0) return;
    v0 = 0.0f;
    v1 = 0.0f;
    L = 0.0f;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
        v0 += red[w][lane];
        v1 += red[w][64 + lane];
        L += red[w][128];
    }
    const float inv = L > 0.0f ? 1.0f / (ROTATED ? L * (float)kHeadDim : L) : 0.0f;
    v0 *= inv;
    v1 *= inv;
    if (ROTATED) fwht128_f32(v0, v1, lane);
    a.out[(size_t)bh * kHeadDim + lane] = v0;
    a.out[(size_t)bh * kHeadDim + 64 + lane] = v1;
}

// One wave per (sequence, query head) row, four rows per work-group, for rows
// with at most 64 partials: lane i holds (m, l) of partial i, the maxima and
// the weighted sums of l are wave reductions, and each partial's weight is
// read from its lane. Every load goes out at once, before the row's context
// length is known: the (m, l) of the partials, and the lane's two channels of
// the first kPre partials (later ones are read in the sum); which partials hold
// tokens (the first ceil(T_b / split_len), and the window slot, the last, when
// there is one) is settled when the loads are back. The partials are added in
// slot order, skipping those without weight.
template <bool ROTATED>
__global__ __launch_bounds__(256) void merge_rows_kernel(MergeArgs a, int rows) {
    constexpr int kPre = 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int bh = blockIdx.x * 4 + (tid >> 6);
    if (bh >= rows) return;
    const float* p = a.partials + (size_t)bh * a.slot_count * kPartStride;
    // slot_count <= 65; slot 64 can only be the unused window slot of a row without a window
    const int sc = min(a.slot_count, 64);
    float mi = -INFINITY, li = 0.0f;
    if (lane < sc) {
        mi = p[(size_t)lane * kPartStride];
        li = p[(size_t)lane * kPartStride + 1];
    }
    float x0[kPre], x1[kPre];
#pragma unroll
    for (int c = 0; c < kPre; ++c) {
        x0[c] = x1[c] = 0.0f;
        if (c < sc) {
            x0[c] = p[(size_t)c * kPartStride + 4 + lane];
            x1[c] = p[(size_t)c * kPartStride + 4 + 64 + lane];
        }
    }
    const int len = a.context_lens[bh / a.num_q_heads];
    const int T = covered_tokens(len, a.cap);
    if (lane == 0 && a.err_word && (len < 0 || len > a.cap)) atomicOr(a.err_word, DQ_DEVERR_CONTEXT);
    const int n = (T + a.split_len - 1) / a.split_len;
    if (!(lane < n || lane == a.window_slot)) {   // a partial without tokens may hold anything
        mi = -INFINITY;
        li = 0.0f;
    }
    float M = mi;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float fi = (mi == -INFINITY) ? 0.0f : exp2f(mi - M);
    float L = li * fi;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
    float v0 = 0.0f, v1 = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
        for (int c = 0; c < kPre; ++c) {
            const float f = __shfl(fi, c);
            if (c < sc && f != 0.0f) {
                v0 += x0[c] * f;
                v1 += x1[c] * f;
            }
        }
        for (int c = kPre; c < sc; ++c) {
            const float f = __shfl(fi, c);
            if (f != 0.0f) {
                const float* ps = p + (size_t)c * kPartStride;
                v0 += ps[4 + lane] * f;
                v1 += ps[4 + 64 + lane] * f;
            }
        }
    }
    const float inv = L > 0.0f ? 1.0f / (ROTATED ? L * (float)kHeadDim : L) : 0.0f;
    v0 *= inv;
    v1 *= inv;
    if (ROTATED) fwht128_f32(v0, v1, lane);
    a.out[(size_t)bh * kHeadDim + lane] = v0;
    a.out[(size_t)bh * kHeadDim + 64 + lane] = v1;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, int rows, bool rotated, hipStream_t s) {
    // partials a row can hold: the splits, plus the window's (slot_count also
    // counts a window slot when there is no window)
    const int slots = a.slot_count - 1 + (a.window_slot >= 0 ? 1 : 0);
    if (slots <= 64 && !(rows < 1024 && slots > 32)) {
        const dim3 grid((unsigned)((rows + 3) / 4));
        if (rotated)
            hipLaunchKernelGGL((merge_rows_kernel<true>), grid, dim3(256), 0, s, a, rows);
        else
            hipLaunchKernelGGL((merge_rows_kernel<false>), grid, dim3(256), 0, s, a, rows);
        return hipGetLastError();
    }
    const bool wide = rows < 1024 && slots > 32;
    if (wide && slots <= 128) {
        if (rotated)
            hipLaunchKernelGGL((merge_wide_kernel<true>), dim3(rows), dim3(64 * 16), 0, s, a);
        else
            hipLaunchKernelGGL((merge_wide_kernel<false>), dim3(rows), dim3(64 * 16), 0, s, a);
        return hipGetLastError();
    }
    if (wide) {
        if (rotated)
            hipLaunchKernelGGL((merge_kernel<true, 16>), dim3(rows), dim3(64 * 16), 0, s, a);
        else
            hipLaunchKernelGGL((merge_kernel<false, 16>), dim3(rows), dim3(64 * 16), 0, s, a);
    } else {
        if (rotated)
            hipLaunchKernelGGL((merge_kernel<true, 4>), dim3(rows), dim3(64 * 4), 0, s, a);
        else
            hipLaunchKernelGGL((merge_kernel<false, 4>), dim3(rows), dim3(64 * 4), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace dq
