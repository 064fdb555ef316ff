// Internal declarations of the per-token format (one stream of the 8 KV
// heads' 1024 rotated values per token, on a token-wise affine grid (o, s)
// stored as two fp16 values), shared by its host API and its kernels.
#pragma once

#include "dq_internal.h"

namespace dq {

constexpr int kTokHeads = 8;
constexpr int kTokN = kTokHeads * kHeadDim;   // symbols per stream
constexpr int kTokMinC = 16, kTokMaxC = 1024; // container bytes
constexpr int kTokMaxPage = 65536;            // largest page (the attention kernel's 24-bit row offsets)

struct TokEncArgs {
    const void* k;                      // [num_tokens][8][128], bf16 bits or fp32
    const void* v;
    int dtype, num_tokens, page_size;
    const int32_t* slot_mapping;        // [num_tokens], slot = page * page_size + offset; < 0: skip
    uint8_t* cache[2];                  // [pages][ceil(C/4)][page_size][4], dwords interleaved over slots
    uint16_t* meta[2];                  // [pages][page_size][2]: o16, s16
    uint32_t* drift_stats;              // optional [num_tokens][2]: changed | rounds << 16
    uint32_t* err_word;
    const EncTable* tables;             // device copy: [0] keys, [1] values
    int max_c;                          // the larger of the two container sizes (sizes the kernel's LDS)
    // key block means (blocks of 128 rows of the call, as for the per-head
    // format with 8 KV heads), written by a pass before the streams; null when off
    int8_t* k_mean;                     // [pages][8][mean_rows_per_page][128]
    uint16_t* k_mean_scale;             // [pages][8][mean_rows_per_page], fp16 bits
};

struct TokAttnArgs {
    const void* q;                      // [batch][Hq][128]
    int q_dtype;
    const uint8_t* k_cache;             // [pages][ceil(C_K/4)][page_size][4]
    const uint8_t* v_cache;
    const uint16_t* k_meta;             // [pages][page_size][2]
    const uint16_t* v_meta;
    const int32_t* block_table;
    const int32_t* context_lens;
    int batch, num_q_heads, group, max_pages_per_seq, page_size, log2p;
    int num_splits, split_len, slot_count, token_cap;
    int ck, cv, pk, pv;
    float half_k, half_v;               // (M - 1) / 2: the entries carry centred levels
    const uint16_t* win_k;              // optional bf16 window [batch][8][win_cap][128]
    const uint16_t* win_v;
    const int32_t* win_lens;            // [batch]
    int win_cap;
    const int8_t* k_mean;               // optional key block means (see TokEncArgs)
    const uint16_t* k_mean_scale;
    float softmax_scale;
    const uint32_t* wide;               // [2][kTableSlots][2] decode tables in two-dword form (K then V)
    float* partials;                    // [batch][Hq][slot_count][kPartStride]
    float* out;
    uint32_t* err_word;
};

// Launchers (defined next to their kernels). launch_token_encode runs the
// key-mean pass first when a.k_mean is set.
hipError_t launch_token_encode(const TokEncArgs& a, hipStream_t s);
hipError_t launch_token_attention(const TokAttnArgs& a, hipStream_t s);
hipError_t launch_token_decode_symbols(const EncTable* table, const uint8_t* containers, int n, uint8_t* out,
                                       uint32_t* err, hipStream_t s);

// Split rule shared by dq_token_workspace_size and the attention call.
int token_choose_splits(int batch, int max_context);

}  // namespace dq
