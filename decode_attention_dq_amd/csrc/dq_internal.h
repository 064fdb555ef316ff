// Internal declarations shared by the host API and the kernels of libdq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dq.h"

namespace dq {

constexpr int kHeadDim = 128;
constexpr int kStateLowBits = 16;            // rANS state interval [2^16, 2^24)
constexpr uint32_t kStateLow = 1u << kStateLowBits;
constexpr int kStateBytes = 3;               // flush size; sigma = 24 bits
constexpr int kCostFracBits = 16;            // costs in units of 2^-16 bit
constexpr int kMaxLevels = 9;
constexpr int kMaxProbBits = 10;
constexpr int kTableSlots = 1 << kMaxProbBits;

// Decode-table entry, one per slot s of [0, 2^p):
//   bits  0.. 7  high byte of the fp16 value of the centred level m - (M-1)/2
//                (its low byte is zero for M <= 9)
//   bits  8..17  bias = s - c_m (so that Dec(x) = f_m * (x >> p) + bias)
//   bits 18..27  f_m
//   bits 28..31  m
__host__ __device__ inline uint32_t entry_pack(uint32_t lvl_hi, uint32_t bias, uint32_t f, uint32_t m) {
    return lvl_hi | (bias << 8) | (f << 18) | (m << 28);
}

// Two-dword form of the same entry, read with one 8-byte LDS load: dword 0 =
// f_m | lvl_hi << 24 (its low 24 bits are exactly the multiplicand of a 24-bit
// multiply-add), dword 1 = bias (the addend). The decode step then needs no
// field extraction.
__host__ __device__ inline void wide_entry_pack(uint32_t lvl_hi, uint32_t bias, uint32_t f, uint32_t* out) {
    out[0] = f | (lvl_hi << 24);
    out[1] = bias;
}

// Per-table constants the encoder needs (passed by value to kernels).
struct EncTable {
    int levels, container, prob_bits, pad0;
    int32_t budget_fx;            // (8C - 24) * 2^16
    int32_t cost[16];             // fixed-point symbol costs
    int32_t inner[16];            // adjacent level toward zero or -1
    uint32_t freq[16];
    uint32_t cum[16];
    uint32_t renorm_lim[16];      // 2^(24-p) * f: emit a byte while x >= this
    uint32_t div_magic[16];       // floor(x / f) = umulhi(x, magic) >> shift, x < 2^24
    uint32_t div_shift[16];
    double recon[16];             // level values (unit RMS)
    double bounds[16];            // decision boundaries
};

struct EncArgs {
    const void* k;
    const void* v;
    int dtype, num_tokens, num_kv_heads, page_size;
    const int32_t* slot_mapping;
    uint8_t* cache[2];
    uint16_t* norm[2];
    uint16_t* drift_stats;
    uint32_t* err_word;
    const EncTable* tables;       // device copy: [0] keys, [1] values
    int max_c;                    // the larger of the two container sizes
    // key channel-mean removal: tokens form blocks of 128 (block j = tokens
    // 128j .. 128j+127 of the call); null when off
    int8_t* k_mean;               // [pages][Hkv][mean_rows_per_page][128]
    uint16_t* k_mean_scale;       // [pages][Hkv][mean_rows_per_page], fp16 bits
};

constexpr int kMeanBlock = 128;   // tokens per key-mean block
// Mean rows per page: one per 128-token block a page holds, or one (owned by
// the page a block starts in) when a page holds fewer than 128 tokens.
__host__ __device__ inline int mean_rows_per_page(int page_size) {
    return page_size >= kMeanBlock ? page_size / kMeanBlock : 1;
}

struct AttnArgs {
    const void* q;
    int q_dtype;
    const uint8_t* k_cache;
    const uint8_t* v_cache;
    const uint16_t* k_norm;
    const uint16_t* v_norm;
    const int32_t* block_table;
    const int32_t* context_lens;
    int batch, num_q_heads, num_kv_heads, group, max_pages_per_seq, page_size;
    int num_splits, split_len;          // tokens per split (multiple of the work-group tile)
    int slot_count;                     // partial slots per (sequence, query head): splits + 1
    int token_cap;                      // tokens a sequence covers at most: max_context
    const uint16_t* win_k;              // optional bf16 window [batch][Hkv][win_cap][128]
    const uint16_t* win_v;
    const int32_t* win_lens;            // [batch]
    int win_cap;
    int ck, cv;                         // container bytes
    int pk, pv;                         // prob bits
    float step_k, step_v;
    float softmax_scale;
    const int8_t* k_mean;               // optional key block means (see EncArgs)
    const uint16_t* k_mean_scale;
    const uint32_t* entries;            // [2][kTableSlots] decode tables (K then V)
    const uint32_t* wide_k;             // [kTableSlots][2] the key table in two-dword form
    float* partials;                    // [batch][Hq][slot_count][kPartStride]
    float* out;
    uint32_t* err_word;
};

// Uncompressed bf16 reference: the same paged layout with 128 bf16 per
// (token, KV head) row instead of a container and a norm.
struct Bf16Args {
    const uint16_t* q;                  // bf16 [batch][Hq][128]
    const uint16_t* k_cache;            // bf16 [pages][Hkv][page_size][128]
    const uint16_t* v_cache;
    const int32_t* block_table;
    const int32_t* context_lens;
    int batch, num_q_heads, num_kv_heads, group, max_pages_per_seq, page_size, log2p;
    int num_splits, split_len, slot_count, token_cap;
    float softmax_scale;
    float* partials;
    float* out;
};

constexpr int kPartStride = 132;         // m, l, pad, pad, acc[128]
constexpr int kWindowMax = 256;          // largest bf16 window

// Launchers (defined next to their kernels).
hipError_t launch_encode(const EncArgs& a, hipStream_t s);   // runs the mean pass first when a.k_mean
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
hipError_t prepare_attention_kernels();   // per device, from dq_tables_init
// Fixed device scratch of dq_decode_attention_noalloc: the split partials of
// one call. Its device address on the current device (see dq_attn.hip).
constexpr size_t kScratchBytes = (size_t)32 << 20;
hipError_t scratch_device_address(void** out);
hipError_t launch_bf16_attention(const Bf16Args& a, hipStream_t s);
// Partial of the bf16 window, written to partial slot `slot`.
hipError_t launch_window(const AttnArgs& a, int slot, hipStream_t s);
// Log-sum-exp merge of the partials of each (sequence, query head) into out:
// the splits that hold tokens of the sequence, and the window slot if any.
struct MergeArgs {
    const float* partials;              // [batch][Hq][slot_count][kPartStride]
    int slot_count;
    const int32_t* context_lens;
    int cap;                            // tokens a sequence covers at most (max_context)
    int split_len, num_q_heads;
    int window_slot;                    // slot of the bf16 window partial, or -1
    float* out;
    uint32_t* err_word;                 // optional: DQ_DEVERR_CONTEXT for a length outside [0, cap]
};
// `rotated`: the partials are in the rotated domain (inverse rotation applied).
hipError_t launch_merge(const MergeArgs& a, int rows, bool rotated, hipStream_t s);
hipError_t launch_decode_symbols(const uint32_t* entries, int prob_bits, int levels, int container,
                                 const uint8_t* containers, int n, uint8_t* out, uint32_t* err,
                                 hipStream_t s);
hipError_t launch_selftest_fp64(const double* a, const double* b, int n, double* sq, double* dv,
                                uint16_t* f16, hipStream_t s);

// Split rule shared by dq_workspace_size and dq_decode_attention.
int choose_splits(int batch, int num_kv_heads, int max_context);
int split_tokens(int max_context, int splits);

}  // namespace dq

struct dq_tables {
    int device;
    int format;               // 0: per-head streams, 1: per-token streams
    dq_table_info info[2];
    dq::EncTable enc[2];
    uint32_t* d_entries;      // [2][kTableSlots] decode tables, the two EncTables, the two-dword key table
    dq::EncTable* d_enc;
    uint32_t* d_wide;         // [2][kTableSlots][2] decode tables in two-dword form, K then V (inside d_entries)
    void* d_scratch;          // this device's copy of the fixed attention scratch (not owned)
};
