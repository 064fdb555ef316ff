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
#include "dq_sched.h"
#include "dq_wave.h"

namespace dq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;
constexpr int kRowH = 72;                 // fp16 per LDS row of the level / weight tiles
constexpr int kRowB = kRowH * 2;          // bytes
constexpr int kPad = 144;                 // bytes after a container tile of the symbol-decode hook: lane 63 of a
                                          // corrupt tile reads < 63C + 132
constexpr int kVtRow = 16;                // bytes per token row of the V level tile (8 fp16 channels)
// LDS of attn_kernel. Both tables are held in two-dword form (8 KB each), so
// that neither chain's decode step needs a field extraction; with a value level
// tile of 8 channels a work-group stays at 40 KB, four per CU.
constexpr uint32_t kOffTabK = 0;          // [1024][2] two-dword key entries
constexpr uint32_t kOffTabV = 8192;       // [1024][2] two-dword value entries
constexpr uint32_t kOffQt = 16384;        // [4][128] fp16 rotated queries
constexpr uint32_t kOffZero = 17408;      // 256 zero bytes: A operand of rows without a head
constexpr uint32_t kOffKappa = 17664;     // [4] floats
constexpr uint32_t kOffLsum = 17680;      // [4 waves][4] floats: each wave's running sums of the weights per head
constexpr uint32_t kOffWaves = 17744;

__host__ __device__ inline uint32_t align16(uint32_t v) { return (v + 15u) & ~15u; }

// Per-wave LDS: the key container tile, the value container tile, then the
// value level tile, which also holds the fp16 p.v weights between passes (they
// are read into registers at the start of a pass, before its first level
// row is written). No padding separates the regions: the byte window of a
// corrupt stream can read up to 138 - C bytes past its tile, which stays
// inside the next region of the same wave (the value container tile, or the
// 1024-byte level tile).
// LDS stride of one token's container: C itself unless C is a multiple of 8,
// in which case C + 4 keeps the stride an odd number of dwords, so that the
// lanes' byte-window reads spread over the LDS banks (a stride of 8 dwords
// would put every fourth lane on the same bank).
__host__ __device__ inline uint32_t lds_stride(int c) { return (c & 7) ? (uint32_t)c : (uint32_t)c + 4u; }

__host__ __device__ inline uint32_t wave_bytes(int ck, int cv) {
    return align16(kTile * lds_stride(ck)) + align16(kTile * lds_stride(cv)) + kTile * kVtRow;
}
static_assert(4 * kRowB <= kTile * kVtRow, "the p.v weights fit in the value level tile");

// A 64-token tile is four 16-token groups; a page holds a multiple of 16
// tokens, so each group's containers are 16 * C contiguous bytes and its norms
// 16 contiguous halves, at row (page * Hkv + g) * P + slot of its first token.
// A group that starts at or past T takes group 0's row: its lanes are masked
// out of the softmax, and the copy stays inside pages of this sequence.
// Everything here is uniform over the wave.
//
// Page ids of the tile's 4 groups, loaded into VGPRs without waiting: issued
// a tile ahead, their latency hides behind a decode pass.
__device__ __forceinline__ void tile_pages(int* pg, const int32_t* __restrict__ bt_row, int log2p, int t0, int T) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
        const int tok = t0 + 16 * gi;
        pg[gi] = bt_row[(gi == 0 || tok < T ? tok : t0) >> log2p];
    }
}
// The same page ids held in one register: lane gi (gi < 4) loads group gi's;
// page_of(v, gi) reads it back as a scalar.
__device__ __forceinline__ int tile_pages_lane(const int32_t* __restrict__ bt_row, int log2p, int t0, int T, int lane) {
    asm volatile("" : "+v"(lane));   // recomputed here: hoisted, the offset would be held through the passes
    const int gi = lane & 3, tok = t0 + 16 * gi;
    return bt_row[(gi == 0 || tok < T ? tok : t0) >> log2p];
}
__device__ __forceinline__ int page_of(int v, int gi) { return __builtin_amdgcn_readlane(v, gi); }

// Row indices of the tile's 4 token groups from their page ids (uniform).
__device__ __forceinline__ void rows_from_pages(size_t* row, const int* pg, int P, int hkv, int g, int t0, int T) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
        const int tok = t0 + 16 * gi;
        const int page = __builtin_amdgcn_readfirstlane(pg[gi]);
        row[gi] = (gi == 0 || tok < T) ? ((size_t)page * (size_t)hkv + (size_t)g) * (size_t)P + (size_t)(tok & (P - 1))
                                       : row[0];
    }
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Copy the containers of the tile's 4 token groups into LDS at `dst`, token t
// at dst + t * lds_stride(C), straight from HBM into LDS (a direct-to-LDS load
// writes lane u's bytes at the uniform LDS address plus u times the unit size),
// with no register round trip and no wait here: the copy completes behind the
// following work and is waited for (vmcnt) before the tile is read.
// Unpadded layout: lane u (and u + 64 when C > 64) moves 16-byte unit u of
// every group.
// Padded layout (C a multiple of 8; stride S = C + 4, an odd dword count, so
// that the lanes' window reads fall in distinct banks): the S/4 words of each
// padded row come in 4-byte units. Word k of a group's padded rows is word
// k - t (S/4) of token t = k / (S/4) (t = (k * magic) >> 16, exact for these k
// with magic = ceil(2^16 / (S/4))); the row's last word, the padding, repeats
// the container's last dword. The loads go through a buffer resource over the
// group's 16 C bytes, so a lane's source is one 32-bit offset.
template <bool PADDED>
__device__ __forceinline__ void stage_tile(uint8_t* lds, uint32_t dst, const uint8_t* __restrict__ cache,
                                           int C, uint32_t magic, const size_t* row, int lane) {
    if (!PADDED) {
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            const uint8_t* gb = cache + row[gi] * (size_t)C;   // uniform
            lds_ptr d = (lds_ptr)(lds + dst + (uint32_t)gi * 16u * (uint32_t)C);
            if (lane < C) __builtin_amdgcn_global_load_lds((const void*)(gb + 16u * (uint32_t)lane), d, 16, 0, 0);
            if (C > 64 && lane + 64 < C)
                __builtin_amdgcn_global_load_lds((const void*)(gb + 16u * (uint32_t)(lane + 64)),
                                                 (lds_ptr)(lds + dst + (uint32_t)gi * 16u * (uint32_t)C + 1024u), 16, 0, 0);
        }
        return;
    }
    const uint32_t n = (uint32_t)C / 4u + 1u;   // words per padded row
    const uint32_t words = 16u * n;             // per group
    __amdgpu_buffer_rsrc_t rs[4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
        rs[gi] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(cache + row[gi] * (size_t)C), (short)0,
                                                   16 * C, 0x00020000);
    for (uint32_t i = 0; 64u * i < words; ++i) {
        uint32_t k = 64u * i + (uint32_t)lane;
        asm volatile("" : "+v"(k));   // recomputed per tile: hoisted, the offsets would stay live through the pass
        const uint32_t t = __umul24(k, magic) >> 16;
        const uint32_t j = min(k - __umul24(t, n), n - 2u);
        const uint32_t off = __umul24(t, (uint32_t)C) + 4u * j;
        if (k < words) {
#pragma unroll
            for (int gi = 0; gi < 4; ++gi)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs[gi], (lds_ptr)(lds + dst + (uint32_t)gi * 16u * (n * 4u) + 256u * i), 4, off, 0, 0, 0);
        }
    }
}

// Waits for this wave's outstanding global loads, the direct-to-LDS copies
// among them, before their tile is read.
__device__ __forceinline__ void stage_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

struct AttnLaunch {
    AttnArgs a;
    int log2p;
    uint32_t magic_k, magic_v;   // ceil(2^16 / (C / 4 + 1)) for the padded staging
    int prio;                    // step the issue priority down per tile (launches of at most two rounds)
};

// PAD_K / PAD_V: containers laid out at the padded LDS stride; MEANS: key
// block means are added to the logits (a separate instantiation, so that the
// kernels without them keep their own register allocation).
template <bool PAD_K, bool PAD_V, bool MEANS>
__global__ __launch_bounds__(kThreads, 4) void attn_kernel(AttnLaunch L) {
    // Decoder lanes with the carried window. The unpadded instantiation
    // without key means keeps all its values in registers only when the refill
    // holds no aligned start (one more VALU instruction per refill); the
    // others run faster holding it.
    using Lane = RansLaneCarry<PAD_K || PAD_V || MEANS>;
    const AttnArgs& a = L.a;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // Work-groups reach the eight XCDs round-robin by linear index; with the KV
    // head fastest every XCD gets an even share of each job class. Jobs go
    // longest first (pick_job); work-groups past the last job exit.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = blockIdx.x % a.num_kv_heads;
    int b, split;
    if (!pick_job(a.context_lens, a.batch, a.token_cap, a.split_len, blockIdx.x / a.num_kv_heads, lane, b, split))
        return;
    __attribute__((address_space(3))) uint8_t* lds_base = (__attribute__((address_space(3))) uint8_t*)lds;
    const int G = a.group;
    const int T = covered_tokens(a.context_lens[b], a.token_cap);
    const int start = split * a.split_len;
    const int end = min(T, start + a.split_len);
    const size_t head_stride = (size_t)a.slot_count * kPartStride;
    float* part = a.partials + (((size_t)b * a.num_q_heads + (size_t)g * G) * a.slot_count + split) * kPartStride;

    const uint32_t kcB = align16(kTile * lds_stride(a.ck)), vcB = align16(kTile * lds_stride(a.cv));
    const uint32_t oW = kOffWaves + (uint32_t)wave * wave_bytes(a.ck, a.cv);
    const uint32_t oKc = oW, oVc = oW + kcB, oVt = oVc + vcB, oWl = oVt;

    // Issue priority. A SIMD issues to its oldest ready wave first, so in a
    // launch of about one round the work-groups dispatched first run ahead and
    // each CU ends with its later ones at falling occupancy. In such launches
    // waves start at the highest priority and step down after each of their
    // first three tiles, so the waves that are behind take the issue slots. In
    // longer launches the later rounds already mix the phases, and the steps
    // cost time.
    if (L.prio) __builtin_amdgcn_s_setprio(3);

    // ---- prologue: tables, zero regions, rotated queries
    {
        // 1024 16-byte units straight into LDS (no registers): the two-dword key
        // table, then the two-dword value table, as they lie in memory; each
        // wave instruction fills 1 KB
        static_assert(kOffTabK == 0 && kOffTabV == 8192 && kThreads == 256, "table units map to LDS 16 u");
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int u = tid + k * kThreads;
            const uint8_t* src = (const uint8_t*)a.wide_k + 16 * u;
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(lds + 16 * (uint32_t)(k * kThreads + wave * 64)),
                                             16, 0, 0);
        }
        uint32_t* z = (uint32_t*)(lds + kOffZero);
        if (tid < 64) z[tid] = 0u;
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
    stage_wait();   // the table copies
    __syncthreads();

    const uint32_t lds0 = (uint32_t)(size_t)lds_base;      // absolute LDS address of the dynamic allocation
    const uint32_t tabK = lds0 + kOffTabK, tabV = lds0 + kOffTabV;
    const uint32_t maskK = (1u << a.pk) - 1u, maskV = (1u << a.pv) - 1u;
    const uint32_t pk = (uint32_t)a.pk, pv = (uint32_t)a.pv;
    float kap[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)   // uniform: kept in scalar registers
        kap[r] = r < G ? __int_as_float(__builtin_amdgcn_readfirstlane(((const int*)(lds + kOffKappa))[r])) : 0.0f;

    // MFMA operand addresses (bytes into LDS)
    const int r16 = lane & 15, grp = lane >> 4;
    const uint32_t aq_off = (grp == (r16 >> 2) && (r16 & 3) < G) ? kOffQt + (uint32_t)(r16 & 3) * 256u : kOffZero;
    // p.v A operand: the 16 rows are four groups of 4 heads, group 2c + h for
    // the value channels of half c of a 16-channel block and the tokens of half
    // h of the tile (row 4(2c + h) + r: head r's weights of tokens 32h + k);
    // ap_off addresses the lane's row for its group, ap_hi says which channel
    // half that group serves
    const bool ap_hi = (r16 >> 3) != 0;
    const uint32_t ap_off = (r16 & 3) < G ? oWl + (uint32_t)(r16 & 3) * kRowB + (uint32_t)((r16 >> 2) & 1) * 64u +
                                                (uint32_t)grp * 16u
                                          : kOffZero;

    const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages_per_seq;
    const int P = a.page_size, log2p = L.log2p, hkv = a.num_kv_heads;

    float m_run[4];   // per head, wave-uniform: the running maximum
    // the running sums of the weights per head, in LDS: a register for them
    // would be held through every pass
    float* l_run = (float*)(lds + kOffLsum) + 4 * wave;
    int e_run = -127;
    float4v acc[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.0f; }   // every lane writes the same value
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = float4v{0.f, 0.f, 0.f, 0.f};
    uint32_t bad = 0;

    // V level tile: 8 channels of fp16 (16 bytes) per token, token t in row t
    // for the first half of the tile and in row t ^ 8 for the second, so that
    // the two halves' rows read by one 16-lane group of a transposed load lie
    // 32 banks apart
    auto vt_row_of = [](int t) { return (uint32_t)(t < 32 ? t : t ^ 8); };
    const uint32_t vt_row = oVt + vt_row_of(lane) * kVtRow;
    // transpose-load sources for the p.v B operand, whose 16 columns are the
    // tile's 8 channels for the tokens of half 0 (columns 0..7) and of half 1
    // (8..15): lane s of a 16-lane group points at 4 channels (8 bytes, half
    // s & 1 of the row) of token 8*group + 32*((s & 3) >> 1) + s/4 (+4 tokens,
    // 4 rows, for the second load), so that result lane n gets channel n % 8 of
    // 4 tokens of half n / 8
    const uint32_t tr0 = oVt + vt_row_of(8 * grp + 32 * ((r16 & 3) >> 1) + (r16 >> 2)) * kVtRow +
                         8u * (uint32_t)(r16 & 1);

    // One pass over the 128 channels of a key tile (do_k) and/or a value tile
    // (do_v): two independent decode chains per lane, the q.k MFMA after each
    // 8 key channels, the p.v MFMAs after each 16 value channels.
    auto pass = [&](bool do_k, bool do_v, Lane& kr, Lane& vr, float4v& dk) {
        // the weights are the same A operand for every 16 channels of the tile:
        // for channel half c, the lane's row, or zeros when its group serves
        // the other half
        half8 av[2];
        if (do_v) {
            av[0] = *(const half8*)(lds + (ap_hi ? kOffZero : ap_off));
            av[1] = *(const half8*)(lds + (ap_hi ? ap_off : kOffZero));
        }
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                uint32_t ek[8], ev[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    if ((jj & 3) == 0) {
                        if (do_k) rans_refill(kr);
                        if (do_v) rans_refill(vr);
                    }
                    if (do_k && do_v) {
                        // both table reads in flight before either chain advances
                        const u32x2 wk = rans_lookup_wide(kr, tabK, maskK);
                        const u32x2 wv = rans_lookup_wide(vr, tabV, maskV);
                        __builtin_amdgcn_sched_barrier(0);
                        rans_advance_wide(kr, wk, pk);
                        ek[jj] = wk.x;
                        rans_advance_wide(vr, wv, pv);
                        ev[jj] = wv.x;
                    } else {
                        if (do_k) {
                            const u32x2 wk = rans_lookup_wide(kr, tabK, maskK);
                            rans_advance_wide(kr, wk, pk);
                            ek[jj] = wk.x;
                        }
                        if (do_v) {
                            const u32x2 wv = rans_lookup_wide(vr, tabV, maskV);
                            rans_advance_wide(vr, wv, pv);
                            ev[jj] = wv.x;
                        }
                    }
                }
                if (do_k) {
                    u32x4 bw;
                    bw[0] = pack_levels_wide(ek[0], ek[1]);
                    bw[1] = pack_levels_wide(ek[2], ek[3]);
                    bw[2] = pack_levels_wide(ek[4], ek[5]);
                    bw[3] = pack_levels_wide(ek[6], ek[7]);
                    // pinned here: hoisting all 16 query loads to the top of the pass costs 64 VGPRs
                    uint32_t qa = aq_off + 16u * (2 * blk + hh);
                    asm volatile("" : "+v"(qa));
                    const half8 aq = *(const half8*)(lds + qa);
                    dk = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, __builtin_bit_cast(half8, bw), dk, 0, 0, 0);
                }
                if (do_v) {
                    // the 8 channels of this half into the level tile; one MFMA
                    // per half covers all 64 tokens: B column n takes channel
                    // n % 8 of the tokens of half n / 8, and the rows of the
                    // groups of channel half hh pick the matching token half.
                    // Half 0's operand is read only after half 1's decode,
                    // just before half 1's levels overwrite the tile (a wave's
                    // LDS operations complete in order), and both MFMAs follow.
                    u32x4 vw;
                    vw[0] = pack_levels_wide(ev[0], ev[1]);
                    vw[1] = pack_levels_wide(ev[2], ev[3]);
                    vw[2] = pack_levels_wide(ev[4], ev[5]);
                    vw[3] = pack_levels_wide(ev[6], ev[7]);
                    if (hh == 0) {
                        *(u32x4*)(lds + vt_row) = vw;
                    } else {
                        wave_lds_sync();
                        const v4i16 lo0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_base + tr0));
                        const v4i16 hi0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_base + tr0 + 4u * kVtRow));
                        wave_lds_sync();
                        *(u32x4*)(lds + vt_row) = vw;
                        wave_lds_sync();
                        const v4i16 lo1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_base + tr0));
                        const v4i16 hi1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds_base + tr0 + 4u * kVtRow));
                        const half8 b0 = __builtin_bit_cast(half8, i16x8{lo0[0], lo0[1], lo0[2], lo0[3], hi0[0], hi0[1], hi0[2], hi0[3]});
                        const half8 b1 = __builtin_bit_cast(half8, i16x8{lo1[0], lo1[1], lo1[2], lo1[3], hi1[0], hi1[1], hi1[2], hi1[3]});
                        acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[0], b0, acc[blk], 0, 0, 0);
                        acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[1], b1, acc[blk], 0, 0, 0);
                        wave_lds_sync();
                    }
                }
            }
        }
    };

    // Online softmax (log2 domain) of a decoded key tile; lane = token, d[r] =
    // raw logit of head r. The running maximum m_run is only a reference
    // point: any value works as long as the weights 2^(s - m_run) stay in
    // range, so it is moved (and the accumulators rescaled) only when some
    // logit of the tile exceeds it by more than kSlack - after the first
    // tiles, rarely. Value norms enter the p.v weights scaled by a running
    // power of two 2^-e_run (moved on the same condition) so that the fp16
    // weights w * |v| 2^-e_run stay below 2^(kSlack + 1).
    auto softmax = [&](const float4v& d, bool valid, uint32_t nk, uint32_t nv, const float* cm) {
        constexpr float kSlack = 8.0f;
        const float rk = f16_to_f32((uint16_t)nk), rv = f16_to_f32((uint16_t)nv);
        float sv[4];
        bool up = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sv[r] = valid ? (MEANS ? d[r] * rk * kap[r] + cm[r] : d[r] * rk * kap[r]) : -INFINITY;
            up |= r < G && sv[r] > m_run[r] + kSlack;
        }
        const int ev = valid && rv > 0.0f ? f32_exponent(rv) : -127;
        if (__builtin_amdgcn_ballot_w64(up || ev > e_run)) {
            float alpha[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                alpha[r] = 1.0f;
                if (r < G) {
                    const float mn = fmaxf(m_run[r], wave_max_uniform(sv[r]));
                    alpha[r] = exp2f(m_run[r] - mn);
                    m_run[r] = mn;
                    l_run[r] *= alpha[r];
                }
            }
            const int e_new = max(e_run, wave_max_uniform_i(ev));
            const float sc = __builtin_amdgcn_ldexpf(1.0f, e_run - e_new);
            e_run = e_new;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][r] *= alpha[r] * sc;
        }
        const float rvs = __builtin_amdgcn_ldexpf(rv, -e_run);
        _Float16* wl = (_Float16*)(lds + oWl);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (r < G) {
                const float w = __builtin_amdgcn_exp2f(sv[r] - m_run[r]);   // 0 for a masked token
                l_run[r] += wave_sum_uniform(w);
                wl[r * kRowH + lane] = (_Float16)(w * rvs);
            }
        }
    };

    // The key block mean's share of the tile's logits (sections 3.2, 5): the
    // block's INT8 channel means times its scale, dotted with the rotated query,
    // in the log2 logit scale; uniform over the tile (a 64-token tile lies in
    // one 128-token block).
    // mean_load issues the loads (the lane's two INT8 means packed in one
    // register, and the block's scale) well before mean_finish uses them.
    // pg_t0 is the page id of token t0 (already loaded with the tile's pages):
    // with pages of 128 tokens or more the block lies in that page, so only
    // smaller pages read the block table here (a dependent load).
    auto mean_load = [&](int t0, int pg_t0, uint32_t& mq, float& s16) {
        mq = 0;
        s16 = 0.0f;
        if (!MEANS) return;
        const int tb = t0 & ~(kMeanBlock - 1);
        const int page = P >= kMeanBlock ? __builtin_amdgcn_readfirstlane(pg_t0) : bt_row[tb >> log2p];
        const size_t mrow = ((size_t)page * hkv + g) * (size_t)mean_rows_per_page(P) + (size_t)((tb & (P - 1)) >> 7);
        s16 = f16_to_f32(a.k_mean_scale[mrow]);
        const uint8_t* mb = (const uint8_t*)a.k_mean + mrow * kHeadDim;
        mq = (uint32_t)mb[lane] | ((uint32_t)mb[64 + lane] << 8);
    };
    auto mean_finish = [&](uint32_t mq, float s16, float* cm) {
#pragma unroll
        for (int r = 0; r < 4; ++r) cm[r] = 0.0f;
        if (!MEANS) return;
        const float m0 = (float)(int8_t)(mq & 255u), m1 = (float)(int8_t)(mq >> 8);
        const _Float16* qt = (const _Float16*)(lds + kOffQt);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (r < G)
                cm[r] = wave_sum_uniform((float)qt[r * kHeadDim + lane] * m0 + (float)qt[r * kHeadDim + 64 + lane] * m1) *
                        s16 * (kap[r] / a.step_k);
    };

    // norms of the lane's token (row of its 16-token group plus its place in
    // the group), kept as fp16 bits: converted only in the softmax after the
    // pass, so the loads are not waited on before it
    auto load_norms = [&](int t0, const size_t* row, uint32_t& nk, uint32_t& nv) {
        const int gl = lane >> 4;
        const size_t r = (gl == 0 ? row[0] : gl == 1 ? row[1] : gl == 2 ? row[2] : row[3]) + (size_t)(lane & 15);
        nk = 0;
        nv = 0;
        if (t0 + lane < T) {
            nk = a.k_norm[r];
            nv = a.v_norm[r];
        }
    };

    const int kStep = kWaves * kTile;
    const uint32_t kbase = oKc + (uint32_t)lane * lds_stride(a.ck);
    const uint32_t vbase = oVc + (uint32_t)lane * lds_stride(a.cv);
    const uint32_t kabs = lds0 + kbase, vabs = lds0 + vbase;   // absolute addresses for the decode steps
    // a stream's state bytes start at its tile row: the address is formed where it
    // is needed (computed once and held, it would be spilled)
    auto stream_base = [](uint32_t base) {
        asm volatile("" : "+v"(base));
        return base;
    };
    int t = start + wave * kTile;
    int pgn[4] = {0, 0, 0, 0};   // page ids of the next tile's groups (scalars), loaded a tile ahead
    if (t < end) {
        // prologue: keys of the first tile
        size_t row[4];
        int pg0[4];
        tile_pages(pg0, bt_row, log2p, t, T);
        rows_from_pages(row, pg0, P, hkv, g, t, T);
        stage_tile<PAD_K>(lds, oKc, a.k_cache, a.ck, L.magic_k, row, lane);
        stage_tile<PAD_V>(lds, oVc, a.v_cache, a.cv, L.magic_v, row, lane);
        stage_wait();
        if (t + kStep < end) tile_pages(pgn, bt_row, log2p, t + kStep, T);   // waited for below, before the pass
        float cm[4], ms;
        uint32_t mq, rk, rv;
        mean_load(t, pg0[0], mq, ms);
        load_norms(t, row, rk, rv);
        wave_lds_sync();
        const bool valid = t + lane < T;
        Lane kr;
        rans_init(kr, stream_base(kabs));
        bad |= (valid && kr.x < kStateLow) ? 1u : 0u;
        float4v dk = float4v{0.f, 0.f, 0.f, 0.f};
        // keys only, as a rolled loop: it touches no accumulator array, and keeping
        // it small keeps the kernel inside the instruction cache
#pragma unroll 1
        for (int j = 0; j < 16; ++j) {
            uint32_t ek[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                if ((jj & 3) == 0) rans_refill(kr);
                const u32x2 wk = rans_lookup_wide(kr, tabK, maskK);
                rans_advance_wide(kr, wk, pk);
                ek[jj] = wk.x;
            }
            u32x4 bw;
            bw[0] = pack_levels_wide(ek[0], ek[1]);
            bw[1] = pack_levels_wide(ek[2], ek[3]);
            bw[2] = pack_levels_wide(ek[4], ek[5]);
            bw[3] = pack_levels_wide(ek[6], ek[7]);
            uint32_t qa = aq_off + 16u * (uint32_t)j;
            asm volatile("" : "+v"(qa));
            const half8 aq = *(const half8*)(lds + qa);
            dk = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, __builtin_bit_cast(half8, bw), dk, 0, 0, 0);
        }
        bad |= (valid && (kr.x != kStateLow || rans_consumed(kr, kabs) > (uint32_t)a.ck)) ? 1u : 0u;
        mean_finish(mq, ms, cm);
        softmax(dk, valid, rk, rv, cm);
        wave_lds_sync();   // the pass is done with the key tile
        if (t + kStep < end) {
            rows_from_pages(row, pgn, P, hkv, g, t + kStep, T);
            stage_tile<PAD_K>(lds, oKc, a.k_cache, a.ck, L.magic_k, row, lane);
        }
    }
    // Tiles are staged right after the pass that frees their region, and waited
    // for just before the pass that decodes them.
    int done = 0;   // tiles finished by this wave (for the issue priority)
    for (; t < end; t += kStep) {
        // values of tile t, interleaved with the keys of tile t + kStep
        const int tn = t + kStep;
        const bool has_next = tn < end;
        const bool valid = t + lane < T, valid_n = tn + lane < T;
        float cm_n[4], ms_n = 0.0f;
        uint32_t mq_n = 0, rk_n = 0, rv_n = 0;
        int pgv = 0;   // the page ids of tile tn + kStep, one per lane (lanes 0..3)
        int pgnn[4] = {0, 0, 0, 0};
        stage_wait();   // this pass's key tile tn and value tile t
        if (has_next) {
            mean_load(tn, pgn[0], mq_n, ms_n);
            size_t row[4];
            rows_from_pages(row, pgn, P, hkv, g, tn, T);
            load_norms(tn, row, rk_n, rv_n);
            if (tn + kStep < end) pgv = tile_pages_lane(bt_row, log2p, tn + kStep, T, lane);
        }
        wave_lds_sync();
        Lane vr, kr;
        rans_init(vr, stream_base(vabs));
        kr = vr;
        bad |= (valid && vr.x < kStateLow) ? 1u : 0u;
        float4v dk = float4v{0.f, 0.f, 0.f, 0.f};
        if (has_next) {
            rans_init(kr, stream_base(kabs));
            bad |= (valid_n && kr.x < kStateLow) ? 1u : 0u;
            pass(true, true, kr, vr, dk);
            bad |= (valid_n && (kr.x != kStateLow || rans_consumed(kr, kabs) > (uint32_t)a.ck)) ? 1u : 0u;
        } else {
            pass(false, true, kr, vr, dk);
        }
        bad |= (valid && (vr.x != kStateLow || rans_consumed(vr, vabs) > (uint32_t)a.cv)) ? 1u : 0u;
        if (has_next) {
            mean_finish(mq_n, ms_n, cm_n);
            softmax(dk, valid_n, rk_n, rv_n, cm_n);
            wave_lds_sync();   // the pass is done with both container tiles
            // the prefetched page ids go to scalars before any copy is issued, so
            // that nothing waits for the copies until the next pass needs them
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) pgnn[gi] = page_of(pgv, gi);
            size_t row[4];   // from the page ids held through the pass
            rows_from_pages(row, pgn, P, hkv, g, tn, T);
            stage_tile<PAD_V>(lds, oVc, a.v_cache, a.cv, L.magic_v, row, lane);
            if (tn + kStep < end) {
                rows_from_pages(row, pgnn, P, hkv, g, tn + kStep, T);
                stage_tile<PAD_K>(lds, oKc, a.k_cache, a.ck, L.magic_k, row, lane);
            }
        }
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) pgn[gi] = pgnn[gi];
        ++done;
        if (L.prio) {
            if (done == 1) __builtin_amdgcn_s_setprio(2);
            else if (done == 2) __builtin_amdgcn_s_setprio(1);
            else if (done == 3) __builtin_amdgcn_s_setprio(0);
        }
    }
    stage_wait();   // no copy into this wave's region may still be in flight
    if (bad && a.err_word) atomicOr(a.err_word, DQ_DEVERR_DECODE);

    // ---- merge the 4 waves of this work-group
    float lsum[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lsum[r] = l_run[r];
    __syncthreads();   // every wave is done with its LDS tiles
    float* mg = (float*)(lds + oW);   // reuse this wave's own region: [0..3] m, [4..7] l, [8] e, [16..] acc[4][128]
    // acc[i][r] of lane l is row 4(l/16) + r, column l % 16 of block i's p.v
    // tile: group l/16 = 2c + h holds channel half c summed over the tokens of
    // half h, in the columns of that token half. Channel 16i + 8c + e is then
    // lane 32c + e (h = 0, column e) plus lane 32c + 24 + e (h = 1, column 8 + e).
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float o = __shfl(acc[i][r], (lane + 24) & 63);
            if ((lane & 31) < 8) mg[16 + r * kHeadDim + i * 16 + 8 * (lane >> 5) + (lane & 7)] = acc[i][r] + o;
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

// Test hook: decode 64 contiguous containers per wave into symbol indices.
__global__ __launch_bounds__(kThreads) void decode_symbols_kernel(const uint32_t* __restrict__ ent, int p,
                                                                  int C, const uint8_t* __restrict__ in, int n,
                                                                  uint8_t* __restrict__ out,
                                                                  uint32_t* __restrict__ err) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t* tab = (uint32_t*)lds;
    for (int i = tid; i < kTableSlots; i += kThreads) tab[i] = ent[i];
    const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)lds;
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
    const uint32_t base = lds0 + oT + (uint32_t)lane * (uint32_t)C;
    // the decoder lanes of the attention kernel, both forms of the carried
    // window refill (odd waves hold the aligned start, even waves do not)
    const uint32_t mask = (1u << p) - 1u;
    uint32_t* o = (uint32_t*)(out + s * kHeadDim);
    auto run = [&](auto& r) {
        rans_init(r, base);
        const bool bad_init = r.x < kStateLow;
        for (int i = 0; i < kHeadDim / 4; ++i) {
            rans_refill(r);
            uint32_t w = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) w |= (rans_dec_step(r, lds0, mask, (uint32_t)p) >> 28) << (8 * k);
            o[i] = w;
        }
        if ((bad_init || r.x != kStateLow || rans_consumed(r, base) > (uint32_t)C) && err)
            atomicOr(err, DQ_DEVERR_DECODE);
    };
    if (wave & 1) {
        RansLaneCarry<true> r;
        run(r);
    } else {
        RansLaneCarry<false> r;
        run(r);
    }
}

// Split partials of dq_decode_attention_noalloc, for callers that cannot
// allocate. Every device the library runs on holds its own copy until the
// process ends. In host code `scratch` is only a host-side stand-in for the
// symbol: its device address comes from scratch_device_address().
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

typedef void (*AttnKernel)(AttnLaunch);
const AttnKernel kAttnKernels[8] = {
    attn_kernel<false, false, false>, attn_kernel<false, true, false>, attn_kernel<true, false, false>,
    attn_kernel<true, true, false>,   attn_kernel<false, false, true>, attn_kernel<false, true, true>,
    attn_kernel<true, false, true>,   attn_kernel<true, true, true>};

}  // namespace

// Large containers need more than the default 64 KB of dynamic LDS. Set once
// per device when its tables are created (a set-up call), so that the launch
// path writes no shared state.
hipError_t prepare_attention_kernels() {
    for (const AttnKernel fn : kAttnKernels) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Address of the current device's copy of `scratch`; called once per device
// with that device current (by dq_tables_init), the result kept with the
// device's tables.
hipError_t scratch_device_address(void** out) {
    *out = nullptr;
    return hipGetSymbolAddress(out, HIP_SYMBOL(scratch));
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
    AttnLaunch L;
    L.a = a;
    L.log2p = 31 - __builtin_clz((unsigned)a.page_size);
    if ((1 << L.log2p) != a.page_size) return hipErrorInvalidValue;
    const size_t lds = kOffWaves + (size_t)kWaves * wave_bytes(a.ck, a.cv);
    L.magic_k = ((1u << 16) + (uint32_t)a.ck / 4u) / ((uint32_t)a.ck / 4u + 1u);
    L.magic_v = ((1u << 16) + (uint32_t)a.cv / 4u) / ((uint32_t)a.cv / 4u + 1u);
    const bool pk = lds_stride(a.ck) != (uint32_t)a.ck, pv = lds_stride(a.cv) != (uint32_t)a.cv;
    const bool mk = a.k_mean != nullptr;
    const int which = (mk ? 4 : 0) + (pk ? 2 : 0) + (pv ? 1 : 0);
    const AttnKernel fn = kAttnKernels[which];
    if (a.win_k) {
        hipError_t e = launch_window(a, a.num_splits, s);
        if (e != hipSuccess) return e;
    }
    const long wgs = (long)a.num_splits * a.num_kv_heads * a.batch;
    L.prio = wgs <= 2L * 1024 ? 1 : 0;   // 4 resident work-groups on each of 256 CUs per round
    dim3 grid((unsigned)wgs);
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, s, L);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    MergeArgs m = {a.partials, a.slot_count, a.context_lens, a.token_cap, a.split_len, a.num_q_heads,
                   a.win_k ? a.num_splits : -1, a.out, a.err_word};
    return launch_merge(m, a.batch * a.num_q_heads, true, s);
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
