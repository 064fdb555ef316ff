/*
 * dq.h - C ABI of the D-Quant KV-cache codec and fused decode attention for
 * AMD Instinct MI355X (gfx950).
 *
 * Method: "D-Quant: Driftable Entropy Coding for KV Cache Quantization"
 * (Su, Liu, Yu, Zhu; arXiv 2609.19880). The paper compresses the key (or
 * value) vector of one token into a fixed-size container (section 4.1), so
 * that attention kernels can address compressed tokens at a fixed stride and
 * dequantize them in parallel (abstract; section 4.1). The cache write is:
 * Hadamard rotation and normalisation (section 3.2, section 4.1), quantisation
 * on an affine grid (section 4.2, grid equation), rANS coding with a static
 * table derived from the standard normal and sharpened by p' ~ p^alpha
 * (section 3.1 Enc/Dec equations; section 4.4 "Distribution sharpening"), and
 * drift: the length-constrained assignment of section 4.3 that moves a few
 * expensive symbols inward, each to the nearest strictly cheaper level toward
 * zero, until sum r(m_i) <= 8C - sigma (section 4.2 container equation). The
 * frequency quantisation keeps the strict outward order of the N(0,1) cell
 * masses, so for every table whose cells get less probable outward (all the
 * defaults) that target is the adjacent level and no symbol moves by more
 * than one level. Decoding feeds
 * the decoded levels straight
 * into the attention contraction with the affine map folded in (section 4.5
 * "Decoding").
 *
 * Stream format (fixed here; the paper leaves it open):
 *   - one stream = the 128 channels of one (token, KV head) of K or of V;
 *   - per-stream scale: rho = sqrt(sum_i y_i^2 / 128) for the rotated row
 *     y = H x (rho equals the L2 norm of x), stored as fp16 rounded once to
 *     nearest even from fp64; y / rho (exact rho, fp64) has unit RMS;
 *   - levels: a symmetric uniform grid, level m at step*(m - (M-1)/2) in
 *     unit-RMS units; the reconstruction of channel i of the rotated row is
 *     rho16 * step * (m_i - (M-1)/2), and the original row is H r / 128 with
 *     H the 128-point Sylvester Hadamard matrix (entries +-1, H H = 128 I);
 *   - rANS: probability precision 2^p, state interval [2^16, 2^24), byte-wise
 *     renormalisation (at most one byte per symbol because every frequency is
 *     at least 2^(p-8)), the final state flushed as 3 little-endian bytes at
 *     offset 0, then the renormalisation bytes in the order the decoder reads
 *     them, then zero padding up to C bytes. sigma = 24 bits. The decoder emits
 *     channel 0 first; after 128 symbols its state is again 2^16.
 *
 * Conventions for every call:
 *   - all array pointers are device memory owned by the caller unless stated;
 *     the library allocates device memory only in dq_tables_init (freed by
 *     dq_tables_destroy);
 *   - calls are asynchronous on the HIP stream passed as `stream` (a
 *     hipStream_t; NULL means the default stream) and never synchronise;
 *     calls on different streams may be made from several host threads at
 *     once (the launch path keeps no mutable shared state; dq_tables_init,
 *     a set-up call, prepares the kernels of its device);
 *   - return value 0 (DQ_OK) or one of the DQ_ERR_* codes below; no C++
 *     exception crosses this interface; dq_strerror() names a code and
 *     dq_last_hip_error() gives the text of the last HIP failure seen by the
 *     calling thread;
 *   - data-dependent device failures (a corrupt container) are not fatal: they
 *     set bits in *err_word when err_word is not NULL, and the affected
 *     outputs are then undefined.
 */
#ifndef DQ_H
#define DQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DQ_HEAD_DIM 128

enum {
    DQ_OK = 0,
    DQ_ERR_INVALID_ARG = 1,  /* null or misaligned pointer, bad size or shape */
    DQ_ERR_UNSUPPORTED = 2,  /* a parameter outside what the kernels implement */
    DQ_ERR_INFEASIBLE = 3,   /* table parameters admit no fitting stream */
    DQ_ERR_WORKSPACE = 4,    /* workspace too small */
    DQ_ERR_HIP = 5           /* a HIP runtime call failed */
};

enum { DQ_DTYPE_F32 = 0, DQ_DTYPE_BF16 = 1 };
enum { DQ_KEYS = 0, DQ_VALUES = 1 };

/* err_word bits set by the device */
#define DQ_DEVERR_DECODE 1u   /* a decoded stream did not return to state 2^16 or overran C */
#define DQ_DEVERR_ENCODE 2u   /* a stream could not be made to fit its container */
#define DQ_DEVERR_MEAN_SLOT 4u /* a key block's first slot is not where a 128-token block starts */
#define DQ_DEVERR_CONTEXT 8u   /* a context length is negative or above max_context: the sequence is
                                  attended over its length clamped to [0, max_context] */

/*
 * Parameters of one static entropy table (keys and values each have one).
 *   levels     M, number of reconstruction levels, 2..9 (the paper uses 8 for
 *              keys and 6 for values at 2.26 bits, section 1 and section 5.1)
 *   container  C, bytes per stream, 8..128
 *   step       grid step in unit-RMS units; 0 selects the default for (M, C):
 *              (8,37) 0.92, (6,37) 0.90, (8,32) 1.12, (6,32) 1.09,
 *              (8,41) 0.79, (6,27) 1.34 - the steps minimising the mean
 *              post-drift NMSE of i.i.d. N(0,1) streams; other (M, C) need
 *              an explicit step
 *   alpha      sharpening exponent, p'_m ~ p_m^alpha (section 4.4); 0 selects
 *              1.4 (section 5.1)
 *   prob_bits  p, 9..10; 0 selects 10
 */
typedef struct dq_table_params {
    int levels;
    int container;
    double step;
    double alpha;
    int prob_bits;
} dq_table_params;

/* Host view of one derived table (filled by dq_table_describe). */
typedef struct dq_table_info {
    int levels, container, prob_bits, feasible;
    double step, alpha;
    double recon[16];     /* level values, unit-RMS units */
    double bounds[16];    /* decision boundaries b_1..b_{M-1} (index 0..M-2) */
    double mass[16];      /* N(0,1) mass of each level's nearest-neighbour cell */
    uint32_t freq[16];    /* integer frequencies f_m, sum 2^p */
    uint32_t cum[17];     /* c_m = sum_{j<m} f_j */
    int64_t cost[16];     /* rint((p - log2 f_m) * 2^16): cost in 2^-16 bit units */
    int32_t inner[16];    /* drift target: nearest level toward zero with a lower cost, -1 if none */
    int64_t budget_fx;    /* (8C - 24) * 2^16 */
} dq_table_info;

typedef struct dq_tables dq_tables;   /* opaque */

/*
 * Derive one table on the host (no device work): N(0,1) cell masses of the
 * nearest-level cells (section 1, section 3.2: the model comes straight from
 * the standard normal), sharpening (section 4.4), integer frequencies (round
 * half even, floor 2^(p-8), one unit more than the outer neighbour where the
 * model makes a level strictly more probable, mirrored, residual to the
 * central level(s)), costs, drift targets, and the feasibility check: a
 * stream whose symbols all sit at the ends of their drift chains (the
 * central levels, for the default tables) must fit with one byte of slack.
 * Returns DQ_ERR_UNSUPPORTED / DQ_ERR_INFEASIBLE as dq_tables_init.
 */
int dq_table_describe(const dq_table_params* params, dq_table_info* out);

/*
 * Build the key and value tables and upload them to the current HIP device
 * (synchronously; this is set-up, not a hot-path call). *out receives a
 * handle owned by the caller and released with dq_tables_destroy. The handle
 * may be used from any stream on the device it was created on.
 */
int dq_tables_init(dq_tables** out, const dq_table_params* keys, const dq_table_params* values);
int dq_tables_destroy(dq_tables* tables);

/* Host copy of a table held by a handle (which = DQ_KEYS or DQ_VALUES). */
int dq_tables_info(const dq_tables* tables, int which, dq_table_info* out);

/*
 * Cache write (sections 4.1-4.3, 4.5 "Encoding"): encode K and V rows of
 * num_tokens new tokens into the paged compressed cache.
 *   k, v          [num_tokens][num_kv_heads][128], dtype DQ_DTYPE_F32 or
 *                 DQ_DTYPE_BF16 (bf16 as raw uint16 bits); finite values
 *   slot_mapping  int32 [num_tokens]: physical slot page * page_size + offset
 *                 of each token; a negative slot skips the token
 *   k_cache       uint8 [num_pages][num_kv_heads][page_size][C_K]
 *   v_cache       uint8 [num_pages][num_kv_heads][page_size][C_V]
 *   k_norm,v_norm uint16 (fp16 bits) [num_pages][num_kv_heads][page_size]
 *   drift_stats   optional (may be NULL) uint16 [num_tokens][num_kv_heads][2]
 *                 (K then V): low byte = symbols changed by drift, high byte =
 *                 drift rounds taken (0: none needed, 1: one round, >1: the
 *                 fallback that may move a symbol by more than one level)
 *   err_word      optional; DQ_DEVERR_ENCODE is set if a stream cannot fit
 * page_size must be a multiple of 16. The caller guarantees distinct slots.
 */
int dq_encode_kv(const dq_tables* tables, const void* k, const void* v, int dtype,
                 int num_tokens, int num_kv_heads, int page_size, const int32_t* slot_mapping,
                 uint8_t* k_cache, uint8_t* v_cache, uint16_t* k_norm, uint16_t* v_norm,
                 uint16_t* drift_stats, uint32_t* err_word, void* stream);

/*
 * Cache write with windowed key channel-mean removal (the paper removes the
 * channel-wise mean of the rotated keys, section 3.2 Table 1, with windowed
 * INT8 channel means, section 5): the call's tokens form num_blocks blocks of
 * 128 (block j = rows 128j .. 128j+127 of k and v, 128 consecutive positions
 * of one sequence starting at a multiple of 128). For every block and KV head
 * the rotated key rows' mean mu (token-order fp64 sum / 128) is stored as
 * INT8 with one fp16 scale s16 = fp16(max|mu| / 127), q = rint(mu / s16)
 * clamped to +-127; each key stream then codes its rotated row minus q * s16.
 * Values are coded as by dq_encode_kv. Arguments as for dq_encode_kv, plus:
 *   k_mean        int8 [num_pages][num_kv_heads][R][128], R = page_size / 128
 *                 when page_size >= 128, else 1: a block's row lives in the
 *                 page its first token occupies, at index (offset / 128)
 *   k_mean_scale  uint16 (fp16 bits) [num_pages][num_kv_heads][R]
 * page_size must be a power of two (DQ_ERR_UNSUPPORTED). A block whose first
 * slot is negative or not at offset 0 mod min(page_size, 128) of its page sets
 * DQ_DEVERR_MEAN_SLOT and its key streams are not written.
 */
int dq_encode_kv_blocks(const dq_tables* tables, const void* k, const void* v, int dtype,
                        int num_blocks, int num_kv_heads, int page_size, const int32_t* slot_mapping,
                        uint8_t* k_cache, uint8_t* v_cache, uint16_t* k_norm, uint16_t* v_norm,
                        int8_t* k_mean, uint16_t* k_mean_scale, uint16_t* drift_stats,
                        uint32_t* err_word, void* stream);

/*
 * Workspace bytes dq_decode_attention needs for these sizes; num_splits 0
 * means the split count the library picks itself (the same rule as
 * dq_decode_attention). Returns 0 for invalid sizes.
 */
size_t dq_workspace_size(int batch, int num_q_heads, int num_kv_heads, int max_context,
                         int num_splits);

/*
 * Fused decode attention over the compressed cache (section 4.5 "Decoding"):
 * for sequence b and query head h with KV head g = h / (Hq / Hkv),
 *     out[b][h] = sum_t softmax_t(scale * q[b][h] . k_hat_t) v_hat_t,
 * t over the first context_lens[b] tokens, k_hat / v_hat the reconstructed
 * rows in the original (unrotated) domain. Work runs in the rotated domain:
 * the query is rotated once, levels enter the contraction directly and the
 * output is rotated back.
 *   q             [batch][num_q_heads][128], DQ_DTYPE_F32 or DQ_DTYPE_BF16
 *   block_table   int32 [batch][max_pages_per_seq]: physical page of each
 *                 logical page; entries past the context are not read
 *   context_lens  int32 [batch], 0 <= len <= max_context (0 gives zeros); a
 *                 length outside that range is clamped to it and sets
 *                 DQ_DEVERR_CONTEXT in *err_word
 *   max_context   host-side upper bound of context_lens (sizes the split)
 *   softmax_scale <= 0 selects 1/sqrt(128)
 *   num_splits    0 = chosen by the library; otherwise the number of token
 *                 ranges each (sequence, KV head) is split into, merged by
 *                 log-sum-exp (flash-decoding)
 *   out           fp32 [batch][num_q_heads][128]
 *   workspace     device buffer of at least dq_workspace_size(...) bytes,
 *                 16-byte aligned
 * num_q_heads / num_kv_heads must be 1..4 (query heads per KV head) and
 * page_size a power of two of at least 16 (DQ_ERR_UNSUPPORTED otherwise);
 * caches and workspace 16-byte aligned (DQ_ERR_INVALID_ARG otherwise).
 */
int dq_decode_attention(const dq_tables* tables, const void* q, int q_dtype,
                        const uint8_t* k_cache, const uint8_t* v_cache,
                        const uint16_t* k_norm, const uint16_t* v_norm,
                        const int32_t* block_table, const int32_t* context_lens,
                        int batch, int num_q_heads, int num_kv_heads, int max_pages_per_seq,
                        int page_size, int max_context, float softmax_scale, int num_splits,
                        float* out, void* workspace, size_t workspace_bytes,
                        uint32_t* err_word, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * dq_decode_attention, same arguments and results, without the workspace
 * arguments. The split partials go to a fixed scratch of DQ_NOALLOC_SCRATCH
 * bytes that the library holds on each device until the process ends (its
 * address is resolved by dq_tables_init); the call allocates nothing. Returns
 * DQ_ERR_WORKSPACE when the sizes need more, i.e. when
 * dq_workspace_size(batch, num_q_heads, num_kv_heads, max_context, num_splits)
 * exceeds DQ_NOALLOC_SCRATCH. Every call on one device shares that scratch:
 * calls that overlap in time on one device (different streams, or different
 * host threads) race and give undefined results; calls ordered on one stream
 * are safe. No part of the scratch has to start at any particular value.
 */
#define DQ_NOALLOC_SCRATCH (32u << 20)
int dq_decode_attention_noalloc(const dq_tables* tables, const void* q, int q_dtype,
                                const uint8_t* k_cache, const uint8_t* v_cache,
                                const uint16_t* k_norm, const uint16_t* v_norm,
                                const int32_t* block_table, const int32_t* context_lens,
                                int batch, int num_q_heads, int num_kv_heads, int max_pages_per_seq,
                                int page_size, int max_context, float softmax_scale, int num_splits,
                                float* out, uint32_t* err_word, void* stream);

/*
 * Decode attention over the compressed cache plus an uncompressed window of
 * each sequence's most recent tokens (the paper keeps the latest tokens in
 * BF16 and compresses older ones, section 5.1). The two parts are combined by
 * log-sum-exp: out[b][h] attends over the context_lens[b] compressed tokens
 * and the window_lens[b] window tokens together. Arguments as for
 * dq_decode_attention, plus:
 *   window_k, window_v  bf16 bits [batch][num_kv_heads][window_cap][128],
 *                       original (unrotated) domain, 16-byte aligned; rows
 *                       [0, window_lens[b]) of each sequence are used
 *   window_lens         int32 [batch], 0 <= len <= window_cap
 *   window_cap          1..256
 * The workspace size is the same as for dq_decode_attention.
 */
int dq_decode_attention_window(const dq_tables* tables, const void* q, int q_dtype,
                               const uint8_t* k_cache, const uint8_t* v_cache,
                               const uint16_t* k_norm, const uint16_t* v_norm,
                               const int32_t* block_table, const int32_t* context_lens,
                               int batch, int num_q_heads, int num_kv_heads, int max_pages_per_seq,
                               int page_size, int max_context, float softmax_scale, int num_splits,
                               const uint16_t* window_k, const uint16_t* window_v,
                               const int32_t* window_lens, int window_cap,
                               float* out, void* workspace, size_t workspace_bytes,
                               uint32_t* err_word, void* stream);

/*
 * Uncompressed reference: split-K decode attention over a paged bf16 KV cache
 * (the paper's full-precision baseline is BF16 attention, section 5.1), with
 * the same paged layout, GQA map, split rule and workspace as
 * dq_decode_attention, for timing the two side by side.
 *   q                bf16 bits [batch][num_q_heads][128]
 *   k_cache, v_cache bf16 bits [num_pages][num_kv_heads][page_size][128],
 *                    16-byte aligned
 *   block_table, context_lens, batch .. num_splits, out, workspace as for
 *                    dq_decode_attention (workspace of dq_workspace_size(...))
 * out[b][h] = softmax(q.K^T * scale) V over the context_lens[b] tokens, fp32.
 * Rows past context_lens[b] inside a page may hold anything; they are ignored.
 * Returns DQ_ERR_INVALID_ARG / DQ_ERR_UNSUPPORTED / DQ_ERR_WORKSPACE as
 * dq_decode_attention does.
 */
int dq_bf16_decode_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                             const int32_t* block_table, const int32_t* context_lens,
                             int batch, int num_q_heads, int num_kv_heads, int max_pages_per_seq,
                             int page_size, int max_context, float softmax_scale, int num_splits,
                             float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Optional inputs of dq_decode_attention_ext; a NULL pointer leaves a part out.
 *   window_k, window_v, window_lens, window_cap   a bf16 window of recent
 *                 tokens, as for dq_decode_attention_window
 *   k_mean, k_mean_scale   the key block means written by dq_encode_kv_blocks
 *                 for every compressed token (context_lens counts whole
 *                 blocks then, except for a sequence's unfinished last block,
 *                 whose tokens use that block's row all the same)
 */
typedef struct {
    const uint16_t* window_k;
    const uint16_t* window_v;
    const int32_t* window_lens;
    int window_cap;
    const int8_t* k_mean;
    const uint16_t* k_mean_scale;
} dq_attention_extras;

/*
 * Decode attention with any of the optional parts of dq_attention_extras: a
 * bf16 window merged by log-sum-exp, and key block means (their share
 * q~ . (q * s16) / 128 is added to every logit of the block, sections 3.2 and
 * 5). extras may be NULL (then it is dq_decode_attention). Other arguments,
 * errors and workspace as for dq_decode_attention.
 */
int dq_decode_attention_ext(const dq_tables* tables, const void* q, int q_dtype,
                            const uint8_t* k_cache, const uint8_t* v_cache,
                            const uint16_t* k_norm, const uint16_t* v_norm,
                            const int32_t* block_table, const int32_t* context_lens,
                            int batch, int num_q_heads, int num_kv_heads, int max_pages_per_seq,
                            int page_size, int max_context, float softmax_scale, int num_splits,
                            const dq_attention_extras* extras, float* out, void* workspace,
                            size_t workspace_bytes, uint32_t* err_word, void* stream);

/*
 * Test hook: decode n_streams contiguous containers ([n_streams][C] bytes of
 * table `which`) into symbol indices uint8 [n_streams][128] with the same
 * device decode routine the attention kernel uses. Streams that fail the
 * integrity check (final state != 2^16 or more than C bytes read) set
 * DQ_DEVERR_DECODE in *err_word.
 */
int dq_decode_symbols(const dq_tables* tables, int which, const uint8_t* containers,
                      int n_streams, uint8_t* symbols_out, uint32_t* err_word, void* stream);

/*
 * Test hook for the fp64 primitives the encoder's bit-exactness rests on:
 * for each of n inputs a (finite, >= 0 for the square root),
 * sqrt_out = correctly rounded sqrt(a), div_out = correctly rounded a / b,
 * f16_out = a rounded once (nearest even) to fp16 bits.
 */
int dq_selftest_fp64(const double* a, const double* b, int n, double* sqrt_out,
                     double* div_out, uint16_t* f16_out, void* stream);

/* ------------------------------------------------------------------------
 * Per-token format (sections 4.2, 4.5 and 5.1 of the paper: each token is one
 * group of 1024 values, the 8 KV heads' rotated rows in head order, coded as a
 * single stream on a token-wise min-max affine grid x_hat = o + s*m, with the
 * least-squares refit of (o, s) stored as two fp16 values; 331 / 231-byte
 * key / value containers with 8 / 6 levels by default).
 * The KV head count is fixed at 8 (DQ_TOKEN_HEADS).
 * ------------------------------------------------------------------------ */
#define DQ_TOKEN_HEADS 8
#define DQ_TOKEN_VALUES 1024

/*
 * Tables of the per-token format. As dq_tables_init, with 1024 symbols per
 * stream and containers of 16..1024 bytes; params.step = 0 selects the
 * min-max grid of an average stream, 2 E[max of 1024 N(0,1)] / (M - 1).
 * The tables serve only the dq_*token* calls (the per-head calls return
 * DQ_ERR_INVALID_ARG for them, and the token calls for per-head tables).
 */
int dq_token_tables_init(dq_tables** out, const dq_table_params* keys, const dq_table_params* values);
int dq_token_table_describe(const dq_table_params* params, dq_table_info* out);

/*
 * Per-token cache write (sections 4.2, 4.3, 4.5 "Encoding"): per token and
 * tensor, y = H x for each of the 8 heads, the min-max grid o = min y,
 * s = (max y - min y)/(M-1), nearest levels, drift until the stream fits,
 * rANS, then the least-squares refit of (o, s).
 *   k, v          [num_tokens][8][128], DQ_DTYPE_F32 or DQ_DTYPE_BF16; finite
 *   slot_mapping  int32 [num_tokens]: slot = page * page_size + offset; < 0
 *                 skips the token
 *   k_cache       uint8 [pages][ceil(C_K/4)][page_size][4] (C_V for v_cache):
 *                 each container as dwords interleaved across the page's slots,
 *                 dword j of slot s at [page][j][s], zero-padded to whole
 *                 dwords; written at each slot, nothing else is touched
 *   k_meta        fp16 bits [pages][page_size][2]: (o16, s16) per slot
 *   drift_stats   optional uint32 [num_tokens][2] (K, V): symbols changed by
 *                 drift | rounds << 16
 *   err_word      optional; DQ_DEVERR_ENCODE if a stream cannot be fitted
 * Ownership: all buffers are the caller's device memory; asynchronous on
 * `stream`.
 */
int dq_encode_tokens(const dq_tables* tables, const void* k, const void* v, int dtype, int num_tokens,
                     int page_size, const int32_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                     uint16_t* k_meta, uint16_t* v_meta, uint32_t* drift_stats, uint32_t* err_word,
                     void* stream);

/*
 * Per-token cache write with windowed key channel-mean removal (section 3.2
 * Table 1, section 5 "windowed INT8 channel means"), the paper's full
 * per-token configuration: the call's tokens form num_blocks blocks of 128
 * (block j = rows 128j .. 128j+127 of k and v, 128 consecutive positions of
 * one sequence starting at a multiple of 128). For every block and each of
 * the 8 KV heads the mean mu of the rotated key rows H x (token-order fp64
 * sum / 128) is stored as INT8 with one fp16 scale, s16 = fp16(max|mu| / 127),
 * q = rint(mu / s16) clamped to +-127; each key stream then codes its rotated
 * values minus q * s16 of its head. Values are coded as by dq_encode_tokens.
 * Arguments as for dq_encode_tokens, plus:
 *   k_mean        int8 [num_pages][8][R][128], R = page_size / 128 when
 *                 page_size >= 128, else 1: a block's rows live in the page its
 *                 first token occupies, at index (offset / 128); 4-byte aligned
 *   k_mean_scale  uint16 (fp16 bits) [num_pages][8][R]
 * page_size must be a power of two (DQ_ERR_UNSUPPORTED). A block whose first
 * slot is negative or not at offset 0 mod min(page_size, 128) of its page sets
 * DQ_DEVERR_MEAN_SLOT and its key streams are not written.
 */
int dq_encode_tokens_blocks(const dq_tables* tables, const void* k, const void* v, int dtype, int num_blocks,
                            int page_size, const int32_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                            uint16_t* k_meta, uint16_t* v_meta, int8_t* k_mean, uint16_t* k_mean_scale,
                            uint32_t* drift_stats, uint32_t* err_word, void* stream);

/* Workspace bytes of dq_token_decode_attention (0 = library split rule). */
size_t dq_token_workspace_size(int batch, int num_q_heads, int max_context, int num_splits);

/*
 * Decode attention over the per-token format (section 4.5 "Decoding": each
 * stream is decoded once and feeds every query head of its KV heads).
 * out[b][h] = softmax(q . K^T * scale) V over the context_lens[b] tokens,
 * K and V the reconstructions H (o16 + s16 m) / 128 per head; query head h
 * uses KV head h / (Hq / 8).
 *   q             [batch][num_q_heads][128], F32 or BF16; num_q_heads = 8 * G,
 *                 G <= 4 (else DQ_ERR_UNSUPPORTED)
 *   k_cache, v_cache, k_meta, v_meta   as written by dq_encode_tokens; the
 *                 caches 16-byte aligned and under 4 GiB each, the metadata
 *                 4-byte aligned
 *   block_table   int32 [batch][max_pages_per_seq]; page_size a power of two
 *                 of at most 65536 (else DQ_ERR_UNSUPPORTED)
 *   context_lens  int32 [batch], 0 <= len <= max_context (0 gives zeros); a
 *                 length outside that range is clamped to it and sets
 *                 DQ_DEVERR_CONTEXT in *err_word
 *   workspace     dq_token_workspace_size bytes, 16-byte aligned
 *   err_word      optional; DQ_DEVERR_DECODE when a stream does not end in
 *                 the initial state or reads past its container
 * Returns DQ_ERR_WORKSPACE if the workspace is too small.
 */
int dq_token_decode_attention(const dq_tables* tables, const void* q, int q_dtype, const uint8_t* k_cache,
                              const uint8_t* v_cache, const uint16_t* k_meta, const uint16_t* v_meta,
                              const int32_t* block_table, const int32_t* context_lens, int batch,
                              int num_q_heads, int max_pages_per_seq, int page_size, int max_context,
                              float softmax_scale, int num_splits, float* out, void* workspace,
                              size_t workspace_bytes, uint32_t* err_word, void* stream);

/*
 * dq_token_decode_attention with the optional parts of dq_attention_extras
 * (sections 3.2, 5 and 5.1); extras may be NULL.
 *   window_k, window_v, window_lens, window_cap   a bf16 window of the most
 *                 recent tokens, [batch][8][window_cap][128] in the original
 *                 domain with window_lens [batch], merged by log-sum-exp as in
 *                 dq_decode_attention_ext
 *   k_mean, k_mean_scale   the key block means written by
 *                 dq_encode_tokens_blocks (k_mean 4-byte aligned): every
 *                 logit of token t and query head h gains q~_h . (q * s16) / 128
 *                 of t's block and KV head (a sequence's unfinished last block
 *                 uses that block's row all the same); one of the two without
 *                 the other is DQ_ERR_INVALID_ARG
 */
int dq_token_decode_attention_ext(const dq_tables* tables, const void* q, int q_dtype, const uint8_t* k_cache,
                                  const uint8_t* v_cache, const uint16_t* k_meta, const uint16_t* v_meta,
                                  const int32_t* block_table, const int32_t* context_lens, int batch,
                                  int num_q_heads, int max_pages_per_seq, int page_size, int max_context,
                                  float softmax_scale, int num_splits, const dq_attention_extras* extras,
                                  float* out, void* workspace, size_t workspace_bytes, uint32_t* err_word,
                                  void* stream);

/*
 * Test hook: decode n_streams contiguous per-token containers ([n][C] bytes
 * of table `which`) into symbols uint8 [n][1024] by a plain per-thread
 * decoder. Streams failing the integrity check set DQ_DEVERR_DECODE.
 */
int dq_token_decode_symbols(const dq_tables* tables, int which, const uint8_t* containers, int n_streams,
                            uint8_t* symbols_out, uint32_t* err_word, void* stream);

const char* dq_strerror(int code);
const char* dq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DQ_H */
