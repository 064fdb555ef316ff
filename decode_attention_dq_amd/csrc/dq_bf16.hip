// Split-K decode attention over an uncompressed paged bf16 KV cache: the
// full-precision reference D-Quant is compared against (the paper's baseline
// is BF16 attention, section 5.1), on the same paged layout, GQA map, token
// splits and log-sum-exp merge as the compressed kernel, so the two can be
// timed side by side. It is HBM-bound: 512 bytes per (token, KV head).
//
// One work-group = 4 waves = one (sequence, KV head, token split); each wave
// takes 32-token tiles of the split in turn.
//   * q.k on MFMA: the 16 rows of one v_mfma_f32_16x16x32_bf16 are 16 tokens,
//     whose K rows are loaded straight from HBM as the A operand (lane i%16
//     reads channels 8*(i/16).. of its token); the B operand holds the G query
//     heads of the group as columns. Lane (head, r) then owns the logits of
//     tokens 4r..4r+3 of the block.
//   * online softmax in the log2 domain per head;
//   * p.v on the VALU: lane (c, r) owns channels 8c..8c+7 and the tokens
//     r, r+4, ...; the weights come from LDS, and the 4 lane groups and then
//     the 4 waves are summed at the end.
#include "dq_internal.h"
#include "dq_sched.h"

namespace dq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;                    // tokens per wave per step
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ __launch_bounds__(kThreads, 4) void bf16_attn_kernel(Bf16Args a) {
    __shared__ __attribute__((aligned(16))) float pl[kWaves][kTile][4];   // weights [token][head]
    __shared__ float red[kWaves][4 * kHeadDim + 8];                       // acc[4][128], m[4], l[4]
    // KV head fastest (an even share of every job class per XCD, as work-groups
    // reach the XCDs round-robin by linear index), jobs longest first.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x % a.num_kv_heads;
    int b, split;
    if (!pick_job(a.context_lens, a.batch, a.token_cap, a.split_len, blockIdx.x / a.num_kv_heads, lane, b, split))
        return;
    const int G = a.group;
    const int T = covered_tokens(a.context_lens[b], a.token_cap);
    const int start = split * a.split_len;
    const int end = min(T, start + a.split_len);
    const size_t head_stride = (size_t)a.slot_count * kPartStride;
    float* part = a.partials + (((size_t)b * a.num_q_heads + (size_t)g * G) * a.slot_count + split) * kPartStride;
    const int col = lane & 15, r = lane >> 4;   // MFMA column / lane group
    const int P = a.page_size, hkv = a.num_kv_heads;
    const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages_per_seq;
    const float sc = a.softmax_scale * kLog2e;

    // B operand: column col = query head g*G + col (zero past G), k-group r
    bf16x8 qb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (col < G) w = *(const u32x4*)(a.q + ((size_t)b * a.num_q_heads + g * G + col) * kHeadDim + 32 * j + 8 * r);
        qb[j] = __builtin_bit_cast(bf16x8, w);
    }

    float m_run = -INFINITY, l_part = 0.0f;   // head col (lanes col < G)
    float o[4][8];
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int c = 0; c < 8; ++c) o[h][c] = 0.0f;

    for (int t = start + wave * kTile; t < end; t += kWaves * kTile) {
        // rows of the tile's two 16-token groups (each inside one page)
        size_t row[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int tok = t + 16 * tb;
            if (tb == 0 || tok < T) {
                const int page = bt_row[tok >> a.log2p];
                row[tb] = ((size_t)page * hkv + g) * (size_t)P + (size_t)(tok & (P - 1));
            } else {
                row[tb] = row[0];
            }
        }
        // logits: A = 16 K rows per block, straight from HBM
        float4v s[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const uint16_t* kr = a.k_cache + (row[tb] + (size_t)col) * kHeadDim + 8 * r;
            bf16x8 ka[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) ka[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(kr + 32 * j));
            s[tb] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) s[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[j], qb[j], s[tb], 0, 0, 0);
        }
        // lane (col, r) holds tokens 16*tb + 4r + i of head col
        float mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = t + 16 * tb + 4 * r + i < T;
                s[tb][i] = ok ? s[tb][i] * sc : -INFINITY;
                mx = fmaxf(mx, s[tb][i]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - mn);   // 0 on the first tile
        m_run = mn;
        float ls = 0.0f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = exp2f(s[tb][i] - mn);
                ls += p;
                if (col < 4) pl[wave][16 * tb + 4 * r + i][col] = p;
            }
        l_part = l_part * alpha + ls;
        // every lane needs the rescale of all 4 heads: lanes 0..3 hold heads 0..3
        float al[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) al[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h));
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int c = 0; c < 8; ++c) o[h][c] *= al[h];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // p.v: lane (col, r) takes channels 8col..8col+7 of tokens 4k + r
#pragma unroll
        for (int k = 0; k < kTile / 4; ++k) {
            const int u = 4 * k + r;
            u32x4 w = *(const u32x4*)(a.v_cache + (row[u >> 4] + (size_t)(u & 15)) * kHeadDim + 8 * col);
            if (t + u >= T) w = u32x4{0u, 0u, 0u, 0u};   // rows past the end may hold anything
            const float4v pw = *(const float4v*)&pl[wave][u][0];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    o[h][2 * c] += pw[h] * lo_bf16(w[c]);
                    o[h][2 * c + 1] += pw[h] * hi_bf16(w[c]);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // sum the 4 lane groups (tokens r mod 4) and the head sums over r
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            o[h][c] += __shfl_xor(o[h][c], 16);
            o[h][c] += __shfl_xor(o[h][c], 32);
        }
    l_part += __shfl_xor(l_part, 16);
    l_part += __shfl_xor(l_part, 32);
    if (r == 0) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int c = 0; c < 8; ++c) red[wave][h * kHeadDim + 8 * col + c] = o[h][c];
    }
    if (lane < 4) {
        red[wave][4 * kHeadDim + lane] = m_run;
        red[wave][4 * kHeadDim + 4 + lane] = l_part;
    }
    __syncthreads();
    for (int idx = tid; idx < G * kHeadDim; idx += kThreads) {
        const int h = idx >> 7, c = idx & 127;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red[w][4 * kHeadDim + h]);
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = red[w][4 * kHeadDim + h];
            if (mw == -INFINITY) continue;
            const float f = exp2f(mw - M);
            L += red[w][4 * kHeadDim + 4 + h] * f;
            A += red[w][h * kHeadDim + c] * f;
        }
        float* ph = part + (size_t)h * head_stride;
        if (c == 0) { ph[0] = M; ph[1] = L; }
        ph[4 + c] = A;
    }
}

}  // namespace

hipError_t launch_bf16_attention(const Bf16Args& a, hipStream_t s) {
    dim3 grid((unsigned)(a.num_splits * a.num_kv_heads * a.batch));
    hipLaunchKernelGGL(bf16_attn_kernel, grid, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    MergeArgs m = {a.partials, a.slot_count, a.context_lens, a.token_cap, a.split_len, a.num_q_heads, -1, a.out,
                   nullptr};
    return launch_merge(m, a.batch * a.num_q_heads, false, s);
}

}  // namespace dq
