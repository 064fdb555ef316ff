// Decode attention over per-token streams (D-Quant section 4.5 "Decoding"):
// a work-group owns a token range of one sequence and decodes each token's K
// and V stream once; the levels of KV head g feed the query heads of group g
// while the stream moves on to head g + 1. The affine grid folds into both
// products (section 4.2): q~ . y_hat = o sum(q~) + s (q~ . m), and
// sum_t p_t y_hat_t = sum_t p_t o_t + sum_t (p_t s_t) m_t.
//
// Work decomposition: 4 waves; a wave takes 64-token tiles, one token per
// lane. Per tile it decodes K head 0, then for g = 0..7 updates the softmax
// of group g, decodes V head g together with K head g + 1 (two independent
// rANS chains per lane), moves the V levels through an LDS transpose, and
// accumulates p.v with each lane owning two channels of every query head.
// The transpose holds 64 channels: p.v runs after each half of V head g.
// The decode tables are in two-dword form (f_m and the level byte, then the
// bias), so a decode step extracts no fields.
// Containers sit in the cache dword-interleaved across the slots of a page
// (dword j of every slot in row j), so the 64 lanes of a wave read
// neighbouring dwords of the same few rows and every cache line is shared
// while it is resident. A lane reads its stream through a 4-byte window that
// is refilled every 4 steps from three dwords loaded at the previous refill
// (at most 4 bytes are consumed in between, so the window lies inside them);
// each refill issues the loads for the next one, clamped to the container's
// last row, so no read leaves the container.
#include "dq_device.h"
#include "dq_token.h"
#include "dq_sched.h"
#include "dq_wave.h"

#include <type_traits>

namespace dq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;           // tokens per wave tile, one per lane
constexpr int kGrp = 4;             // query heads per KV head held (GQA group <= 4)
constexpr int kVtRowDw = kTile + 4; // dwords per row of the V level transpose (16-byte rows, padded)

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The logits run on v_mfma_f32_16x16x32_f16: after 8 key channels a lane
// holds 8 fp16 levels of its own token, the B operand for column lane % 16
// and k-group lane / 16; a block-diagonal A operand (query head h of the
// group in row 4 (lane / 16) + h, non-zero only in k-group lane / 16) lands
// the 4 head logits of the lane's own token in its accumulator, so no
// transpose is needed. p.v runs on v_mfma_f32_4x4x4f16 (16 blocks of 4x4x4):
// block b of the MFMA takes channels 4b..4b+3 and 4 tokens, the same weights
// in every block, so lane l ends with the 4 query heads of channel l (and of
// l + 64 in a second accumulator). Levels enter centred,
// m - (M-1)/2, as fp16 whose high byte is the decode entry's level byte (the
// low byte is zero); the centre joins the offset, so the offset is near the
// values' mean and the products carry only the centred part.
struct TokShared {
    uint32_t tab[2][2 * kTableSlots];             // two-dword decode tables, K then V
    _Float16 qa[kTokHeads][kGrp][kHeadDim];       // rotated queries [KV head][head in group][channel]
    uint32_t zero[64];                            // A operand of the rows without a head (16 blocks of 16 bytes)
    float qsum[kTokHeads][kGrp];                  // their sums over the channels (fp32)
    union alignas(16) {
        struct {
            uint32_t vt[kHeadDim / 8][kVtRowDw];  // V level bytes of one 64-channel half: row k holds
                                                  // channels 4k..4k+3 of the half, column = token
            _Float16 w[kGrp][kTile];              // p * s_v per head and token
        } wave[kWaves];
        struct {
            float acc[kWaves][kGrp][kHeadDim];
            float m[kWaves][kGrp];
            float l[kWaves][kGrp];
        } red;
    } u;
};

typedef float float4_t __attribute__((ext_vector_type(4)));

// Wave-wide max and sum as wave-uniform values: the butterflies and row
// broadcasts of the DPP reduction each as one v_max/v_add with a DPP source
// (the compiler's forms add a move, and for the max a canonicalisation, per
// stage). Each stage reads the previous one's result, so two wait states
// precede it. Every lane must be active; the values are never NaN.
__device__ __forceinline__ float tok_wave_max(float v) {
    asm volatile(
        "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
        "s_nop 1"
        : "+v"(v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float tok_wave_sum(float v) {
    asm volatile(
        "s_nop 1\n\tv_add_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_add_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
        "s_nop 1\n\tv_add_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
        "s_nop 1"
        : "+v"(v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// The three container dwords from byte a (aligned) on: rows a/4 .. a/4 + 2,
// the next refill's source. Row r of a container is the dword at byte
// row0 + r * stride of the cache, read through a buffer resource with 32-bit
// byte offsets (a cache stays under 4 GiB), so a load costs one clamp and one
// 24-bit multiply-add. Rows past the container's last are read as the last
// row; a valid stream never consumes their bytes.
struct GWin {
    uint32_t a, d0, d1, d2;
};
struct GSrc {
    uint32_t row0;          // byte offset of the container's first dword
    uint32_t stride;        // bytes between rows (4 x the page size)
    uint32_t last;          // index of the container's last row (>= 3: containers have >= 16 bytes)
    uint32_t row2;          // row0 + 2 stride: the refill loads row r + 2 as min(r, last - 2) stride + row2
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t cache_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xFFFFFFFFu, 0x00020000);
}
__device__ __forceinline__ uint32_t row_load(__amdgpu_buffer_rsrc_t rs, const GSrc& src, uint32_t r) {
    return __builtin_amdgcn_raw_buffer_load_b32(rs, __umul24(min(r, src.last), src.stride) + src.row0,
                                                0, 0);
}
// Move the window past the consumed bytes. At most 4 bytes went since the
// last refill, so ptr - g.a is at most 7: the window's 4 bytes lie in rows
// a/4 + up and a/4 + up + 1, where up says whether the aligned start moved
// (to g.a + 4). Those two rows stay as the new first two; only the third is
// loaded, for the next refill.
__device__ __forceinline__ void grans_refill(RansLane& r, GWin& g, __amdgpu_buffer_rsrc_t rs, const GSrc& src) {
    r.ptr += r.sel - kSel0;
    const uint32_t na = r.ptr & ~3u;
    const bool up = na != g.a;
    const uint32_t lo = up ? g.d1 : g.d0, hi = up ? g.d2 : g.d1;
    r.win = __builtin_amdgcn_alignbyte(hi, lo, r.ptr);
    r.sel = kSel0;
    g.a = na;
    g.d0 = lo;
    g.d1 = hi;
    g.d2 = __builtin_amdgcn_raw_buffer_load_b32(rs, __umul24(min(r.ptr >> 2, src.last - 2u), src.stride) + src.row2,
                                                0, 0);
}
// Stream state from the 3-byte flush at the container's start, then the
// window at byte 3 (byte offsets count from the container's start).
__device__ __forceinline__ void grans_init(RansLane& r, GWin& g, __amdgpu_buffer_rsrc_t rs, const GSrc& src) {
    g.a = 0u;
    g.d0 = row_load(rs, src, 0u);
    g.d1 = row_load(rs, src, 1u);
    g.d2 = row_load(rs, src, 2u);
    r.ptr = 0u;
    r.x = g.d0 & 0xFFFFFFu;
    r.sel = kSel0 + (uint32_t)kStateBytes;
    grans_refill(r, g, rs, src);
}

__global__ __launch_bounds__(kThreads, 3) void token_attn_kernel(TokAttnArgs a) {
    __shared__ TokShared S;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int b, split;
    if (!pick_job(a.context_lens, a.batch, a.token_cap, a.split_len, blockIdx.x, lane, b, split)) return;
    const int G = a.group;
    const int T = covered_tokens(a.context_lens[b], a.token_cap);
    const int start = split * a.split_len;
    const int end = min(T, start + a.split_len);

    // ---- prologue: decode tables, rotated queries q~ = H q and their sums
    for (int i = tid; i < kTableSlots; i += kThreads) ((u32x4*)&S.tab[0][0])[i] = ((const u32x4*)a.wide)[i];
    for (int i = tid; i < kTokHeads * kGrp * kHeadDim / 2; i += kThreads) ((uint32_t*)&S.qa[0][0][0])[i] = 0u;
    if (tid < 64) S.zero[tid] = 0u;
    if (tid < kTokHeads * kGrp) (&S.qsum[0][0])[tid] = 0.0f;
    __syncthreads();
    for (int h = wave; h < a.num_q_heads; h += kWaves) {
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
        const int g = h / G, hh = h - g * G;
        S.qa[g][hh][lane] = (_Float16)v0;
        S.qa[g][hh][lane + 64] = (_Float16)v1;
        const float sum = wave_sum(v0 + v1);
        if (lane == 0) S.qsum[g][hh] = sum;
    }
    __syncthreads();

    const uint32_t tabK = (uint32_t)(size_t)(__attribute__((address_space(3))) uint32_t*)&S.tab[0][0];
    const uint32_t tabV = tabK + kTableSlots * 8u;
    const uint32_t maskK = (1u << a.pk) - 1u, maskV = (1u << a.pv) - 1u;
    const __amdgpu_buffer_rsrc_t kres = cache_rsrc(a.k_cache), vres = cache_rsrc(a.v_cache);
    const float cs = a.softmax_scale * kLog2e / (float)kHeadDim;
    // A operand of the logit MFMA: lane l supplies row l % 16 in k-group
    // l / 16, the query head (l % 16) & 3 of the group when l / 16 is
    // (l % 16) / 4, else zeros (16 blocks of 8 channels, 16 bytes each)
    const char* Sb = (const char*)&S;
    const int r16 = lane & 15;
    const bool qrow = (lane >> 4) == (r16 >> 2) && (r16 & 3) < G;
    const uint32_t qa0 = (uint32_t)((const char*)&S.qa[0][r16 & 3][0] - Sb);
    const uint32_t qz = (uint32_t)((const char*)&S.zero[0] - Sb);
    auto q_off = [&](int g) -> uint32_t { return qrow ? qa0 + (uint32_t)g * (kGrp * kHeadDim * 2u) : qz; };

    // acc[g][c][h]: query head h of group g at channel lane + 64 c
    float4_t acc[kTokHeads][2];
#pragma unroll
    for (int g = 0; g < kTokHeads; ++g) acc[g][0] = acc[g][1] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float mrun = -INFINITY, lrun = 0.0f;   // lane 4g + hh: running max and sum of head (g, hh)
    bool bad = false;
    auto& Wv = S.u.wave[wave];
    // p.v B operand: channel lane (lane + 64) is byte lane & 3 of row lane / 4
    // (16 + lane / 4) of the transpose; the selector puts that byte of two
    // tokens' dwords into the high bytes of an fp16 pair
    const uint32_t vb = (uint32_t)lane & 3u;
    const uint32_t vsel = 0x000C000Cu | (vb << 8) | ((vb + 4u) << 24);
    const uint32_t vrow = (uint32_t)lane >> 2;

    for (int t0 = start + wave * kTile; t0 < end; t0 += kWaves * kTile) {
        const int t = t0 + lane;
        const bool valid = t < end;
        const int tt = valid ? t : t0;   // lanes past the end decode a real stream and are masked
        const int page = a.block_table[(size_t)b * a.max_pages_per_seq + (tt >> a.log2p)];
        const uint32_t idx = (uint32_t)page * (uint32_t)a.page_size + (uint32_t)(tt & (a.page_size - 1));
        const uint32_t km = ((const uint32_t*)a.k_meta)[idx], vm = ((const uint32_t*)a.v_meta)[idx];
        // centred grid: y_hat = (o + s (M-1)/2) + s (m - (M-1)/2), the products take the centred levels
        const float sk = f16_to_f32((uint16_t)(km >> 16)), sv = f16_to_f32((uint16_t)(vm >> 16));
        const float ok = f16_to_f32((uint16_t)(km & 0xFFFFu)) + sk * a.half_k;
        const float ov = f16_to_f32((uint16_t)(vm & 0xFFFFu)) + sv * a.half_v;
        const uint32_t ck4 = ((uint32_t)a.ck + 3u) >> 2, cv4 = ((uint32_t)a.cv + 3u) >> 2;
        const uint32_t pg = (uint32_t)page * (uint32_t)a.page_size, po = idx - pg;
        const uint32_t stride = 4u * (uint32_t)a.page_size;
        const GSrc sk_ = {4u * (pg * ck4 + po), stride, ck4 - 1u, 4u * (pg * ck4 + po) + 2u * stride};
        const GSrc sv_ = {4u * (pg * cv4 + po), stride, cv4 - 1u, 4u * (pg * cv4 + po) + 2u * stride};
        // key block means: lane 4g + hh gets q~ . (q * s16) of query head
        // (g, hh) and the 128-token block the tile lies in
        float qmu = 0.0f;
        if (a.k_mean) {
            const int tb = t0 & ~(kMeanBlock - 1);
            const int mpage = a.block_table[(size_t)b * a.max_pages_per_seq + (tb >> a.log2p)];
            const int mg = lane >> 2, mh = lane & 3;
            if (lane < 4 * kTokHeads && mh < G) {
                const size_t row = ((size_t)mpage * kTokHeads + mg) * (size_t)mean_rows_per_page(a.page_size) +
                                   (size_t)((tb & (a.page_size - 1)) / kMeanBlock);
                const uint32_t* mr = (const uint32_t*)(a.k_mean + row * kHeadDim);
                float d = 0.0f;
                for (int c4 = 0; c4 < kHeadDim / 4; ++c4) {
                    const uint32_t w = mr[c4];
                    const half2_t m0 = {(_Float16)(int8_t)(w & 255u), (_Float16)(int8_t)((w >> 8) & 255u)};
                    const half2_t m1 = {(_Float16)(int8_t)((w >> 16) & 255u), (_Float16)(int8_t)(w >> 24)};
                    // the address is formed here (hoisted, the 32 addresses would take registers)
                    uint32_t qo = (uint32_t)((const char*)&S.qa[mg][mh][4 * c4] - Sb);
                    asm volatile("" : "+v"(qo));
                    const half2_t* qp = (const half2_t*)(Sb + qo);
                    d = __builtin_amdgcn_fdot2(qp[0], m0, d, false);
                    d = __builtin_amdgcn_fdot2(qp[1], m1, d, false);
                }
                qmu = d * f16_to_f32(a.k_mean_scale[row]);
            }
        }
        RansLane rk, rv;
        GWin gk, gv;
        grans_init(rk, gk, kres, sk_);
        grans_init(rv, gv, vres, sv_);

        // K head 0 alone; dk[h] ends as the raw logit of head h of the group
        float4_t dk = {0.0f, 0.0f, 0.0f, 0.0f};
        {
            const uint32_t qo = q_off(0);
#pragma unroll 1
            for (int c8 = 0; c8 < kHeadDim / 8; ++c8) {
                u32x4 kw;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    if (c8 | hf) grans_refill(rk, gk, kres, sk_);
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        const u32x2 e0 = rans_lookup_wide(rk, tabK, maskK);
                        rans_advance_wide(rk, e0, (uint32_t)a.pk);
                        const u32x2 e1 = rans_lookup_wide(rk, tabK, maskK);
                        rans_advance_wide(rk, e1, (uint32_t)a.pk);
                        kw[2 * hf + i / 2] = pack_levels_wide(e0.x, e1.x);
                    }
                }
                uint32_t qa = qo + 16u * (uint32_t)c8;
                asm volatile("" : "+v"(qa));
                const half8 aq = *(const half8*)(Sb + qa);
                dk = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, __builtin_bit_cast(half8, kw), dk, 0, 0, 0);
            }
        }
        grans_refill(rk, gk, kres, sk_);

        // KV heads in order: the softmax of group g, V head g (fused with K
        // head g + 1 while there is one), the group's p.v. acc[0] holds the
        // current group's accumulators and the array rotates by one group per
        // head, back to its order after the eighth. The loop is unrolled by
        // two, so every other rotation is only a renaming of registers; fully
        // unrolled, the kernel no longer fits the instruction cache.
#pragma unroll 2
        for (int g = 0; g < kTokHeads; ++g) {
            float4_t wv;
#pragma unroll
            for (int hh = 0; hh < kGrp; ++hh) {
                const int hl = 4 * g + hh;
                const float qm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qmu), hl));
                const float L = valid ? (ok * S.qsum[g][hh] + (sk * dk[hh] + qm)) * cs : -INFINITY;
                const float mo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mrun), hl));
                // the running maximum moves only when a logit of the tile exceeds
                // it (after the first tiles, rarely); otherwise the maximum
                // reduction is skipped, and the result is the same
                float mn = mo;
                if (__builtin_amdgcn_ballot_w64(L > mo)) mn = fmaxf(mo, tok_wave_max(L));
                // both arguments are <= 0 (or -inf): v_exp_f32 as it stands
                const float fac = __builtin_amdgcn_exp2f(mo - mn);
                const float p = valid ? __builtin_amdgcn_exp2f(L - mn) : 0.0f;
                const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lrun), hl));
                const float ln = lo * fac + tok_wave_sum(p);
                const float os = tok_wave_sum(p * ov);
                acc[0][0][hh] = acc[0][0][hh] * fac + os;
                acc[0][1][hh] = acc[0][1][hh] * fac + os;
                mrun = lane == hl ? mn : mrun;
                lrun = lane == hl ? ln : lrun;
                wv[hh] = p * sv;
            }
#pragma unroll
            for (int hh = 0; hh < kGrp; ++hh) Wv.w[hh][lane] = (_Float16)wv[hh];

            // p.v of one 64-channel half of V head g, 4 tokens per MFMA: the A
            // operand is head lane & 3's weights of the 4 tokens, the B operand
            // channel lane's levels of the same tokens (lane + 64's in the upper half)
            auto pv_half = [&](float4_t& accv) {
                wave_lds_sync();
#pragma unroll 4
                for (int j = 0; j < kTile; j += 4) {
                    const u32x4 d = *(const u32x4*)&Wv.vt[vrow][j];
                    const half4_t aw = *(const half4_t*)&Wv.w[lane & 3][j];
                    const u32x2 bb = {__builtin_amdgcn_perm(d[1], d[0], vsel), __builtin_amdgcn_perm(d[3], d[2], vsel)};
                    accv = __builtin_amdgcn_mfma_f32_4x4x4f16(aw, __builtin_bit_cast(half4_t, bb), accv, 0, 0, 0);
                }
                wave_lds_sync();
            };
            // the level bytes (bits 24..31 of dword 0 of an entry) of 4 channels
            // of the lane's token, channel 4k first
            auto vt_word = [](const uint32_t (&ev)[4]) {
                return __builtin_amdgcn_perm(__builtin_amdgcn_perm(ev[3], ev[2], 0x0C0C0703u),
                                             __builtin_amdgcn_perm(ev[1], ev[0], 0x0C0C0703u), 0x05040100u);
            };

            dk = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
            if (g + 1 < kTokHeads) {
                const uint32_t qo = q_off(g + 1);
#pragma unroll
                for (int half = 0; half < 2; ++half) {
#pragma unroll 1
                    for (int c8 = 0; c8 < kHeadDim / 16; ++c8) {
                        u32x4 kw;
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const int c4 = 2 * c8 + hf;   // row of the half's transpose
                            if (half | c4) {
                                grans_refill(rv, gv, vres, sv_);
                                grans_refill(rk, gk, kres, sk_);
                            }
                            uint32_t ev[4];
#pragma unroll
                            for (int i = 0; i < 4; i += 2) {
                                const u32x2 v0 = rans_lookup_wide(rv, tabV, maskV);
                                const u32x2 k0 = rans_lookup_wide(rk, tabK, maskK);
                                rans_advance_wide(rv, v0, (uint32_t)a.pv);
                                rans_advance_wide(rk, k0, (uint32_t)a.pk);
                                const u32x2 v1 = rans_lookup_wide(rv, tabV, maskV);
                                const u32x2 k1 = rans_lookup_wide(rk, tabK, maskK);
                                rans_advance_wide(rv, v1, (uint32_t)a.pv);
                                rans_advance_wide(rk, k1, (uint32_t)a.pk);
                                ev[i] = v0.x;
                                ev[i + 1] = v1.x;
                                kw[2 * hf + i / 2] = pack_levels_wide(k0.x, k1.x);
                            }
                            Wv.vt[c4][lane] = vt_word(ev);
                        }
                        uint32_t qa = qo + 16u * (uint32_t)(c8 + half * (kHeadDim / 16));
                        asm volatile("" : "+v"(qa));
                        const half8 aq = *(const half8*)(Sb + qa);
                        dk = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, __builtin_bit_cast(half8, kw), dk, 0, 0, 0);
                    }
                    pv_half(acc[0][half]);
                }
                grans_refill(rk, gk, kres, sk_);
            } else {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
#pragma unroll 1
                    for (int c4 = 0; c4 < kHeadDim / 8; ++c4) {
                        if (half | c4) grans_refill(rv, gv, vres, sv_);
                        uint32_t ev[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const u32x2 e = rans_lookup_wide(rv, tabV, maskV);
                            rans_advance_wide(rv, e, (uint32_t)a.pv);
                            ev[i] = e.x;
                        }
                        Wv.vt[c4][lane] = vt_word(ev);
                    }
                    pv_half(acc[0][half]);
                }
            }
            grans_refill(rv, gv, vres, sv_);

            // rotate: the next group's accumulators to the front
            const float4_t first0 = acc[0][0], first1 = acc[0][1];
#pragma unroll
            for (int gg = 0; gg + 1 < kTokHeads; ++gg) acc[gg][0] = acc[gg + 1][0], acc[gg][1] = acc[gg + 1][1];
            acc[kTokHeads - 1][0] = first0;
            acc[kTokHeads - 1][1] = first1;
        }
        // both streams must end in the initial state having read no byte past C
        const bool okk = rk.x == kStateLow && rk.ptr + (rk.sel - kSel0) <= (uint32_t)a.ck;
        const bool okv = rv.x == kStateLow && rv.ptr + (rv.sel - kSel0) <= (uint32_t)a.cv;
        bad = bad || (valid && !(okk && okv));
    }
    if (__any(bad) && lane == 0 && a.err_word) atomicOr(a.err_word, DQ_DEVERR_DECODE);

    // ---- combine the 4 waves' partials per KV head and write them
    __syncthreads();
    auto combine = [&](auto gtag, const float4_t (&ag)[2]) {
        constexpr int g = decltype(gtag)::value;
#pragma unroll
        for (int hh = 0; hh < kGrp; ++hh) {
            S.u.red.acc[wave][hh][lane] = ag[0][hh];
            S.u.red.acc[wave][hh][lane + 64] = ag[1][hh];
        }
        const float mg = __shfl(mrun, 4 * g + (lane & 3)), lg = __shfl(lrun, 4 * g + (lane & 3));
        if (lane < kGrp) {
            S.u.red.m[wave][lane] = mg;
            S.u.red.l[wave][lane] = lg;
        }
        __syncthreads();
        if (wave < G) {
            const int hh = wave, h = g * G + hh;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, S.u.red.m[w][hh]);
            float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float mw = S.u.red.m[w][hh];
                if (mw == -INFINITY) continue;
                const float f = exp2f(mw - M);
                L += S.u.red.l[w][hh] * f;
                o0 += S.u.red.acc[w][hh][lane] * f;
                o1 += S.u.red.acc[w][hh][lane + 64] * f;
            }
            float* part = a.partials + (((size_t)b * a.num_q_heads + h) * a.slot_count + split) * kPartStride;
            if (lane == 0) {
                part[0] = M;
                part[1] = L;
            }
            part[4 + lane] = o0;
            part[4 + 64 + lane] = o1;
        }
        __syncthreads();
    };
    combine(std::integral_constant<int, 0>{}, acc[0]);
    combine(std::integral_constant<int, 1>{}, acc[1]);
    combine(std::integral_constant<int, 2>{}, acc[2]);
    combine(std::integral_constant<int, 3>{}, acc[3]);
    combine(std::integral_constant<int, 4>{}, acc[4]);
    combine(std::integral_constant<int, 5>{}, acc[5]);
    combine(std::integral_constant<int, 6>{}, acc[6]);
    combine(std::integral_constant<int, 7>{}, acc[7]);
}

}  // namespace

hipError_t launch_token_attention(const TokAttnArgs& a, hipStream_t s) {
    if (a.win_k) {
        // the bf16 window's partial (the same kernel as for per-head caches; it
        // reads only the queries, the window and the partial layout)
        AttnArgs w = {};
        w.q = a.q;
        w.q_dtype = a.q_dtype;
        w.batch = a.batch;
        w.num_q_heads = a.num_q_heads;
        w.num_kv_heads = kTokHeads;
        w.group = a.group;
        w.slot_count = a.slot_count;
        w.win_k = a.win_k;
        w.win_v = a.win_v;
        w.win_lens = a.win_lens;
        w.win_cap = a.win_cap;
        w.softmax_scale = a.softmax_scale;
        w.partials = a.partials;
        hipError_t e = launch_window(w, a.num_splits, s);
        if (e != hipSuccess) return e;
    }
    dim3 grid((unsigned)(a.num_splits * a.batch));
    hipLaunchKernelGGL(token_attn_kernel, grid, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    MergeArgs m = {a.partials, a.slot_count, a.context_lens, a.token_cap, a.split_len, a.num_q_heads,
                   a.win_k ? a.num_splits : -1, a.out, a.err_word};
    return launch_merge(m, a.batch * a.num_q_heads, true, s);
}

}  // namespace dq
