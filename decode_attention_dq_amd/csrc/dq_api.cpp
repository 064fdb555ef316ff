// Host side of libdq: table derivation, argument checks, split choice and
// launches. Every entry point is extern "C" and returns a status code.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <string>

#include "dq_token.h"

namespace {

thread_local std::string g_last_hip_error;

int hip_fail(hipError_t e) {
    g_last_hip_error = hipGetErrorString(e);
    return DQ_ERR_HIP;
}

// fp64 -> fp16 bits, one rounding to nearest even (host copy; only used for
// the small exact level values stored in the decode table).
uint16_t host_f64_to_f16(double d) {
    uint64_t b;
    memcpy(&b, &d, 8);
    uint32_t sign = (uint32_t)(b >> 63) << 15;
    int exp = (int)((b >> 52) & 0x7FF);
    uint64_t mant = b & ((1ull << 52) - 1);
    if (exp == 0x7FF) return (uint16_t)(sign | 0x7C00 | (mant ? 0x200 : 0));
    if (exp == 0) return (uint16_t)sign;   // fp64 subnormals are far below fp16's range
    int e = exp - 1023;
    uint64_t m53 = mant | (1ull << 52);
    int shift;            // bits dropped from m53
    uint32_t base;        // exponent field contribution
    if (e >= -14) {
        shift = 42;
        base = (uint32_t)(e + 15) << 10;
        m53 &= (1ull << 52) - 1;   // implicit bit handled through `base`
    } else {
        shift = 28 - e;   // subnormal: value / 2^-24
        base = 0;
        if (shift > 62) return (uint16_t)sign;
    }
    uint64_t q = m53 >> shift;
    uint64_t rem = m53 & ((1ull << shift) - 1);
    uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) q++;
    uint32_t r = base + (uint32_t)q;   // a mantissa carry bumps the exponent
    if (r >= 0x7C00) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | r);
}

double std_normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

double default_step(int levels, int container) {
    if (container == 37 && levels == 8) return 0.92;
    if (container == 37 && levels == 6) return 0.90;
    if (container == 32 && levels == 8) return 1.12;
    if (container == 32 && levels == 6) return 1.09;
    if (container == 41 && levels == 8) return 0.79;
    if (container == 27 && levels == 6) return 1.34;
    return 0.0;
}

// E[max of n i.i.d. N(0,1)] = integral of x n phi(x) Phi(x)^(n-1) dx by the
// composite Simpson rule on [-12, 12] with 40000 intervals.
double expected_max(int n) {
    const int steps = 40000;
    const double lo = -12.0, hi = 12.0, h = (hi - lo) / steps;
    double total = 0.0;
    for (int i = 0; i <= steps; ++i) {
        const double x = lo + i * h;
        const double phi = exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
        const double cdf = 0.5 * erfc(-x / sqrt(2.0));
        const double f = x * n * phi * pow(cdf, n - 1);
        const double w = (i == 0 || i == steps) ? 1.0 : (i % 2 ? 4.0 : 2.0);
        total += w * f;
    }
    return total * h / 3.0;
}

// Default grid step of the per-token format: the min-max grid of an average
// stream of 1024 N(0,1) values, 2 E[max] / (M - 1), in N(0,1) units.
double token_step(int levels) { return 2.0 * expected_max(dq::kTokN) / (levels - 1); }

// Table derivation. The probability model is the N(0,1) mass of each
// level's nearest-neighbour cell (the paper derives its model directly from
// the standard normal: section 1, section 3.2), sharpened by p^alpha and
// renormalised (section 4.4), then quantised to integer frequencies summing
// to 2^p for the rANS pair of section 3.1.
// `token`: a table of the per-token format (1024 symbols per stream).
int describe(const dq_table_params* in, dq_table_info* t, bool token = false) {
    if (!in || !t) return DQ_ERR_INVALID_ARG;
    memset(t, 0, sizeof(*t));
    const int M = in->levels, C = in->container;
    const int p = in->prob_bits ? in->prob_bits : 10;
    const double alpha = in->alpha > 0 ? in->alpha : 1.4;
    const int n = token ? dq::kTokN : dq::kHeadDim;
    const int c_lo = token ? dq::kTokMinC : 8, c_hi = token ? dq::kTokMaxC : 128;
    if (M < 2 || M > dq::kMaxLevels || p < 9 || p > dq::kMaxProbBits || C < c_lo || C > c_hi)
        return DQ_ERR_UNSUPPORTED;
    double step = in->step > 0 ? in->step : (token ? token_step(M) : default_step(M, C));
    if (!(step > 0) || !(alpha > 0) || !isfinite(step) || !isfinite(alpha)) return DQ_ERR_INVALID_ARG;
    t->levels = M;
    t->container = C;
    t->prob_bits = p;
    t->step = step;
    t->alpha = alpha;
    const uint32_t total = 1u << p;
    const uint32_t f_min = 1u << (p - 8);

    const double half = (M - 1) / 2.0;
    for (int m = 0; m < M; ++m) t->recon[m] = step * ((double)m - half);
    for (int j = 1; j < M; ++j) t->bounds[j - 1] = (t->recon[j - 1] + t->recon[j]) / 2.0;

    // cell masses, lower half from the CDF (accurate tail), mirrored
    for (int m = 0; m < M / 2; ++m) {
        double lo = (m == 0) ? 0.0 : std_normal_cdf(t->bounds[m - 1]);
        double hi = (M % 2 == 0 && m == M / 2 - 1) ? 0.5 : std_normal_cdf(t->bounds[m]);
        t->mass[m] = hi - lo;
        t->mass[M - 1 - m] = t->mass[m];
    }
    if (M % 2 == 1) {
        int c = M / 2;
        t->mass[c] = erf(-t->bounds[c - 1] / sqrt(2.0));
    }

    // sharpening, normalised by a left-to-right sum
    double w[16], s = 0.0;
    for (int m = 0; m < M; ++m) w[m] = pow(t->mass[m], alpha);
    for (int m = 0; m < M; ++m) s += w[m];

    // Rounding and the floor keep the model's order: going inward, a level
    // whose cell is strictly more probable than its outer neighbour's gets at
    // least one more unit, so its cost is strictly lower.
    int64_t sum = 0;
    for (int m = 0; m < M / 2; ++m) {
        double r = nearbyint((w[m] / s) * (double)total);   // round half to even
        int64_t f = (int64_t)r;
        if (f < (int64_t)f_min) f = f_min;
        if (m > 0 && t->mass[m] > t->mass[m - 1] && f <= (int64_t)t->freq[m - 1]) f = (int64_t)t->freq[m - 1] + 1;
        t->freq[m] = (uint32_t)f;
        t->freq[M - 1 - m] = (uint32_t)f;
        sum += 2 * f;
    }
    bool ok = true;
    if (M % 2 == 0) {
        int64_t resid = (int64_t)total - sum;      // even
        int64_t a = t->freq[M / 2 - 1] + resid / 2;
        int64_t b = t->freq[M / 2] + resid / 2;
        if (a < (int64_t)f_min || b < (int64_t)f_min) ok = false;
        t->freq[M / 2 - 1] = (uint32_t)(a < 0 ? 0 : a);
        t->freq[M / 2] = (uint32_t)(b < 0 ? 0 : b);
    } else {
        int64_t c = (int64_t)total - sum;
        if (c < (int64_t)f_min) ok = false;
        t->freq[M / 2] = (uint32_t)(c < 0 ? 0 : c);
    }
    t->cum[0] = 0;
    for (int m = 0; m < M; ++m) t->cum[m + 1] = t->cum[m] + t->freq[m];
    if (t->cum[M] != total) ok = false;

    for (int m = 0; m < M; ++m) {
        if (t->freq[m] == 0) { ok = false; continue; }
        t->cost[m] = (int64_t)nearbyint(((double)p - log2((double)t->freq[m])) * (double)(1 << dq::kCostFracBits));
    }
    // drift target: the nearest level toward zero with a strictly lower cost
    // (expensive symbols drift to nearby cheaper ones, section 4.3); with the
    // model's order kept above this is the adjacent inner level wherever the
    // cells get less probable outward; the walk ends after the first level at
    // or across zero
    for (int m = 0; m < M; ++m) {
        t->inner[m] = -1;
        const int d = t->recon[m] > 0 ? -1 : (t->recon[m] < 0 ? 1 : 0);
        for (int j = m + d; d != 0 && j >= 0 && j < M; j += d) {
            if (t->cost[j] < t->cost[m]) { t->inner[m] = j; break; }
            if (t->recon[j] * t->recon[m] <= 0) break;
        }
    }
    t->budget_fx = (int64_t)(8 * C - 8 * dq::kStateBytes) << dq::kCostFracBits;
    // Drift moves a symbol only to its strictly cheaper drift target, so from
    // level m it ends at most at the end of that chain; a stream made only of
    // such terminal levels must fit with a byte of rANS slack.
    int64_t worst = 0;
    for (int m = 0; ok && m < M; ++m) {
        int cur = m;
        while (t->inner[cur] >= 0) cur = t->inner[cur];
        if (t->cost[cur] > worst) worst = t->cost[cur];
    }
    if (ok && (int64_t)n * worst + (8ll << dq::kCostFracBits) > t->budget_fx) ok = false;
    t->feasible = ok ? 1 : 0;
    return ok ? DQ_OK : DQ_ERR_INFEASIBLE;
}

void fill_enc_table(const dq_table_info& t, dq::EncTable* e) {
    memset(e, 0, sizeof(*e));
    e->levels = t.levels;
    e->container = t.container;
    e->prob_bits = t.prob_bits;
    e->budget_fx = (int32_t)t.budget_fx;
    for (int m = 0; m < t.levels; ++m) {
        const uint32_t f = t.freq[m];
        e->cost[m] = (int32_t)t.cost[m];
        e->inner[m] = t.inner[m];
        e->freq[m] = f;
        e->cum[m] = t.cum[m];
        e->renorm_lim[m] = f << (24 - t.prob_bits);
        // floor(x / f) = (x * magic) >> (31 + s) for x < 2^24, s = floor(log2 f)
        // (f >= 2), with magic = ceil(2^(31+s) / f) raised by less than 32 so that
        // its low 5 bits equal the shift s - 1 applied after the high product
        // (a kernel can shift by the magic itself). Exact: magic = 2^(31+s) / f + d
        // with 0 <= d < 32, and x d / 2^(31+s) < 2^(24+5-31-s) = 2^-(2+s) < 1/(2f)
        // because f < 2^(s+1); so x magic / 2^(31+s) stays below floor(x/f) + 1.
        // magic < 2^32: 2^(31+s) / f <= 2^31 and d < 32.
        int s = 31 - __builtin_clz(f);
        unsigned __int128 num = ((unsigned __int128)1) << (31 + s);
        uint64_t magic = (uint64_t)((num + f - 1) / f);
        magic += (uint64_t)(((uint32_t)(s - 1) - (uint32_t)magic) & 31u);
        e->div_magic[m] = (uint32_t)magic;
        e->div_shift[m] = (uint32_t)(s - 1);
        e->recon[m] = t.recon[m];
    }
    for (int j = 0; j + 1 < t.levels; ++j) e->bounds[j] = t.bounds[j];
}

// Decode entries; bits 0..7 hold the fp16 high byte of the centred level
// m - (M-1)/2 (its low byte is zero for M <= 9). The per-token kernel folds
// the centre into the grid offset: o + s m = (o + s (M-1)/2) + s (m - (M-1)/2).
void fill_entries(const dq_table_info& t, uint32_t* ent, uint32_t* wide) {
    const uint32_t total = 1u << t.prob_bits;
    for (int m = 0; m < t.levels; ++m) {
        uint16_t h = host_f64_to_f16((double)m - (t.levels - 1) / 2.0);
        for (uint32_t s = t.cum[m]; s < t.cum[m + 1]; ++s) {
            ent[s] = dq::entry_pack(h >> 8, s - t.cum[m], t.freq[m], (uint32_t)m);
            if (wide) dq::wide_entry_pack(h >> 8, s - t.cum[m], t.freq[m], wide + 2 * s);
        }
    }
    for (uint32_t s = total; s < (uint32_t)dq::kTableSlots; ++s) {
        ent[s] = 0;
        if (wide) wide[2 * s] = wide[2 * s + 1] = 0;
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static_assert(DQ_NOALLOC_SCRATCH == dq::kScratchBytes, "the header states the scratch size");
static_assert((2 * sizeof(dq::EncTable)) % 16 == 0, "the two-dword key table starts 16-byte aligned");

}  // namespace

namespace dq {

// Split rule. Work-groups are taken longest job first, so a launch ends well
// when its last jobs are short ones: 1536-token splits (whose last split per
// sequence is shorter) when they give at least four work-groups per slot (4
// resident work-groups on each of 256 CUs). Otherwise 2048-token splits fill
// every slot with equal jobs; when those make fewer than two rounds, 1024-token
// splits instead (two rounds of 4-tile waves finish sooner than one of 8-tile
// waves, whose key-only first and value-only last passes all run at once); and
// shorter splits, down to one 256-token tile, when even 2048-token splits would
// leave fewer than 1024 work-groups.
int choose_splits(int batch, int num_kv_heads, int max_context) {
    const long units = (long)batch * num_kv_heads;
    const int tile = 256, slots = 1024;
    const int max_by_len = (max_context + tile - 1) / tile;
    long s = (max_context + 1535) / 1536;
    if (units * s < 4L * slots) {
        s = (max_context + 2047) / 2048;
        if (units * s < slots)
            s = (slots + units - 1) / units;
        else if (units * s < 2L * slots)
            s = (max_context + 1023) / 1024;
    }
    if (s > max_by_len) s = max_by_len;
    if (s < 1) s = 1;
    return (int)s;
}

// Per-token split rule: 2048-token splits, or shorter ones (down to one
// 256-token tile) until there are 1536 work-groups, two rounds of the 768 that
// are resident at once (3 per CU). On the Qwen3-8B layer (128 x 8192) that is
// 11 jobs of 768 tokens per sequence; 16 of 512 took 1% longer, 6 of 1536
// (one round, the last job of each sequence short) 9% longer.
int token_choose_splits(int batch, int max_context) {
    const int tile = 256, target = 1536;
    const int max_by_len = (max_context + tile - 1) / tile;
    long s = (max_context + 2047) / 2048;
    if ((long)batch * s < target) s = (target + batch - 1) / batch;
    if (s > max_by_len) s = max_by_len;
    if (s < 1) s = 1;
    return (int)s;
}

int split_tokens(int max_context, int splits) {
    const int tile = 256;
    int per = (max_context + splits - 1) / splits;
    per = (per + tile - 1) / tile * tile;
    return per < tile ? tile : per;
}

}  // namespace dq

extern "C" {

const char* dq_strerror(int code) {
    switch (code) {
        case DQ_OK: return "ok";
        case DQ_ERR_INVALID_ARG: return "invalid argument";
        case DQ_ERR_UNSUPPORTED: return "unsupported parameter";
        case DQ_ERR_INFEASIBLE: return "table parameters admit no fitting stream";
        case DQ_ERR_WORKSPACE: return "workspace too small";
        case DQ_ERR_HIP: return "HIP runtime error";
        default: return "unknown error";
    }
}

const char* dq_last_hip_error(void) { return g_last_hip_error.c_str(); }

int dq_table_describe(const dq_table_params* params, dq_table_info* out) {
    return describe(params, out);
}

static int tables_init(dq_tables** out, const dq_table_params* keys, const dq_table_params* values, bool token) {
    if (!out || !keys || !values) return DQ_ERR_INVALID_ARG;
    *out = nullptr;
    dq_tables* t = new (std::nothrow) dq_tables();
    if (!t) return DQ_ERR_INVALID_ARG;
    t->format = token ? 1 : 0;
    int rc = describe(keys, &t->info[0], token);
    if (rc == DQ_OK) rc = describe(values, &t->info[1], token);
    if (rc != DQ_OK) { delete t; return rc; }
    fill_enc_table(t->info[0], &t->enc[0]);
    fill_enc_table(t->info[1], &t->enc[1]);
    // two-dword entries, K then V ([2][kTableSlots][2])
    uint32_t host[2 * dq::kTableSlots], wide[4 * dq::kTableSlots];
    fill_entries(t->info[0], host, wide);
    fill_entries(t->info[1], host + dq::kTableSlots, wide + 2 * dq::kTableSlots);
    hipError_t e = hipGetDevice(&t->device);
    if (e == hipSuccess) e = dq::prepare_attention_kernels();
    if (e == hipSuccess) e = dq::scratch_device_address(&t->d_scratch);
    if (e != hipSuccess) { delete t; return hip_fail(e); }
    const size_t ent_bytes = sizeof(uint32_t) * 2 * dq::kTableSlots;
    const size_t wide_off = ent_bytes + sizeof(dq::EncTable) * 2;   // a multiple of 16 bytes
    const size_t total = wide_off + sizeof(wide);
    void* d = nullptr;
    e = hipMalloc(&d, total);
    if (e != hipSuccess) { delete t; return hip_fail(e); }
    e = hipMemcpy(d, host, ent_bytes, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy((char*)d + ent_bytes, t->enc, sizeof(dq::EncTable) * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy((char*)d + wide_off, wide, sizeof(wide), hipMemcpyHostToDevice);
    if (e != hipSuccess) { (void)hipFree(d); delete t; return hip_fail(e); }
    t->d_entries = (uint32_t*)d;
    t->d_enc = (dq::EncTable*)((char*)d + ent_bytes);
    t->d_wide = (uint32_t*)((char*)d + wide_off);
    *out = t;
    return DQ_OK;
}

int dq_tables_init(dq_tables** out, const dq_table_params* keys, const dq_table_params* values) {
    return tables_init(out, keys, values, false);
}

int dq_token_tables_init(dq_tables** out, const dq_table_params* keys, const dq_table_params* values) {
    return tables_init(out, keys, values, true);
}

int dq_token_table_describe(const dq_table_params* params, dq_table_info* out) {
    return describe(params, out, true);
}

int dq_tables_destroy(dq_tables* t) {
    if (!t) return DQ_OK;
    hipError_t e = hipSuccess;
    if (t->d_entries) e = hipFree(t->d_entries);
    delete t;
    return e == hipSuccess ? DQ_OK : hip_fail(e);
}

int dq_tables_info(const dq_tables* t, int which, dq_table_info* out) {
    if (!t || !out || (which != DQ_KEYS && which != DQ_VALUES)) return DQ_ERR_INVALID_ARG;
    *out = t->info[which];
    return DQ_OK;
}

namespace {
int encode_impl(const dq_tables* t, const void* k, const void* v, int dtype, int num_tokens, int num_kv_heads,
                int page_size, const int32_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache, uint16_t* k_norm,
                uint16_t* v_norm, int8_t* k_mean, uint16_t* k_mean_scale, uint16_t* drift_stats, uint32_t* err_word,
                void* stream) {
    if (!t || t->format != 0 || num_tokens < 0 || num_kv_heads <= 0 || page_size <= 0 || page_size % 16)
        return DQ_ERR_INVALID_ARG;
    if (dtype != DQ_DTYPE_F32 && dtype != DQ_DTYPE_BF16) return DQ_ERR_INVALID_ARG;
    if (num_tokens == 0) return DQ_OK;
    if (!k || !v || !slot_mapping || !k_cache || !v_cache || !k_norm || !v_norm)
        return DQ_ERR_INVALID_ARG;
    if ((long)num_tokens * num_kv_heads * 2 > (long)INT32_MAX / 2) return DQ_ERR_INVALID_ARG;
    dq::EncArgs a;
    a.k = k;
    a.v = v;
    a.dtype = dtype;
    a.num_tokens = num_tokens;
    a.num_kv_heads = num_kv_heads;
    a.page_size = page_size;
    a.slot_mapping = slot_mapping;
    a.cache[0] = k_cache;
    a.cache[1] = v_cache;
    a.norm[0] = k_norm;
    a.norm[1] = v_norm;
    a.drift_stats = drift_stats;
    a.err_word = err_word;
    a.tables = t->d_enc;
    a.max_c = std::max(t->info[0].container, t->info[1].container);
    a.k_mean = k_mean;
    a.k_mean_scale = k_mean_scale;
    hipError_t e = dq::launch_encode(a, (hipStream_t)stream);
    return e == hipSuccess ? DQ_OK : hip_fail(e);
}
}  // namespace

int dq_encode_kv(const dq_tables* t, const void* k, const void* v, int dtype, int num_tokens,
                 int num_kv_heads, int page_size, const int32_t* slot_mapping, uint8_t* k_cache,
                 uint8_t* v_cache, uint16_t* k_norm, uint16_t* v_norm, uint16_t* drift_stats,
                 uint32_t* err_word, void* stream) {
    return encode_impl(t, k, v, dtype, num_tokens, num_kv_heads, page_size, slot_mapping, k_cache, v_cache, k_norm,
                       v_norm, nullptr, nullptr, drift_stats, err_word, stream);
}

int dq_encode_kv_blocks(const dq_tables* t, const void* k, const void* v, int dtype, int num_blocks,
                        int num_kv_heads, int page_size, const int32_t* slot_mapping, uint8_t* k_cache,
                        uint8_t* v_cache, uint16_t* k_norm, uint16_t* v_norm, int8_t* k_mean,
                        uint16_t* k_mean_scale, uint16_t* drift_stats, uint32_t* err_word, void* stream) {
    if (!k_mean || !k_mean_scale || num_blocks < 0 || (long)num_blocks * dq::kMeanBlock > INT32_MAX)
        return DQ_ERR_INVALID_ARG;
    if (page_size > 0 && (page_size & (page_size - 1))) return DQ_ERR_UNSUPPORTED;
    return encode_impl(t, k, v, dtype, num_blocks * dq::kMeanBlock, num_kv_heads, page_size, slot_mapping, k_cache,
                       v_cache, k_norm, v_norm, k_mean, k_mean_scale, drift_stats, err_word, stream);
}

size_t dq_workspace_size(int batch, int num_q_heads, int num_kv_heads, int max_context, int num_splits) {
    if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context < 0 || num_splits < 0)
        return 0;
    int s = num_splits ? num_splits : dq::choose_splits(batch, num_kv_heads, max_context);
    // one partial per split, plus one slot for an optional bf16 window
    return (size_t)batch * num_q_heads * (s + 1) * dq::kPartStride * sizeof(float);
}

static int decode_attention_impl(const dq_tables* t, const void* q, int q_dtype, const uint8_t* k_cache,
                                 const uint8_t* v_cache, const uint16_t* k_norm, const uint16_t* v_norm,
                                 const int32_t* block_table, const int32_t* context_lens, int batch,
                                 int num_q_heads, int num_kv_heads, int max_pages_per_seq, int page_size,
                                 int max_context, float softmax_scale, int num_splits, const uint16_t* window_k,
                                 const uint16_t* window_v, const int32_t* window_lens, int window_cap,
                                 const int8_t* k_mean, const uint16_t* k_mean_scale, float* out,
                                 void* workspace, size_t workspace_bytes, uint32_t* err_word, void* stream) {
    if (!t || t->format != 0 || !q || !k_cache || !v_cache || !k_norm || !v_norm || !block_table || !context_lens ||
        !out || !workspace)
        return DQ_ERR_INVALID_ARG;
    if (q_dtype != DQ_DTYPE_F32 && q_dtype != DQ_DTYPE_BF16) return DQ_ERR_INVALID_ARG;
    if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
        max_pages_per_seq <= 0 || page_size <= 0 || page_size % 16 || max_context < 0 ||
        num_splits < 0 || (long)max_pages_per_seq * page_size < max_context)
        return DQ_ERR_INVALID_ARG;
    if (num_q_heads / num_kv_heads > 4 || (page_size & (page_size - 1))) return DQ_ERR_UNSUPPORTED;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace)) return DQ_ERR_INVALID_ARG;
    const bool win = window_k != nullptr;
    if (win) {
        if (!window_v || !window_lens || window_cap <= 0 || !aligned16(window_k) || !aligned16(window_v))
            return DQ_ERR_INVALID_ARG;
        if (window_cap > dq::kWindowMax) return DQ_ERR_UNSUPPORTED;
    }
    if ((k_mean == nullptr) != (k_mean_scale == nullptr)) return DQ_ERR_INVALID_ARG;
    int splits = num_splits ? num_splits : dq::choose_splits(batch, num_kv_heads, max_context);
    if (workspace_bytes < dq_workspace_size(batch, num_q_heads, num_kv_heads, max_context, splits))
        return DQ_ERR_WORKSPACE;
    if ((long)batch * num_kv_heads * splits > (long)INT32_MAX / 4) return DQ_ERR_INVALID_ARG;
    dq::AttnArgs a;
    a.q = q;
    a.q_dtype = q_dtype;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_norm = k_norm;
    a.v_norm = v_norm;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.batch = batch;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.max_pages_per_seq = max_pages_per_seq;
    a.page_size = page_size;
    a.num_splits = splits;
    a.split_len = dq::split_tokens(max_context, splits);
    a.slot_count = splits + 1;
    a.token_cap = max_context;   // within the pages and the splits (checked above / by construction)
    a.win_k = window_k;
    a.win_v = window_v;
    a.win_lens = window_lens;
    a.win_cap = win ? window_cap : 0;
    a.k_mean = k_mean;
    a.k_mean_scale = k_mean_scale;
    a.ck = t->info[0].container;
    a.cv = t->info[1].container;
    a.pk = t->info[0].prob_bits;
    a.pv = t->info[1].prob_bits;
    a.step_k = (float)t->info[0].step;
    a.step_v = (float)t->info[1].step;
    a.softmax_scale = softmax_scale > 0 ? softmax_scale : 1.0f / sqrtf((float)dq::kHeadDim);
    a.entries = t->d_entries;
    a.wide_k = t->d_wide;
    a.partials = (float*)workspace;
    a.out = out;
    a.err_word = err_word;
    hipError_t e = dq::launch_attention(a, (hipStream_t)stream);
    return e == hipSuccess ? DQ_OK : hip_fail(e);
}

int dq_decode_attention(const dq_tables* t, const void* q, int q_dtype, const uint8_t* k_cache,
                        const uint8_t* v_cache, const uint16_t* k_norm, const uint16_t* v_norm,
                        const int32_t* block_table, const int32_t* context_lens, int batch,
                        int num_q_heads, int num_kv_heads, int max_pages_per_seq, int page_size,
                        int max_context, float softmax_scale, int num_splits, float* out,
                        void* workspace, size_t workspace_bytes, uint32_t* err_word, void* stream) {
    return decode_attention_impl(t, q, q_dtype, k_cache, v_cache, k_norm, v_norm, block_table, context_lens,
                                 batch, num_q_heads, num_kv_heads, max_pages_per_seq, page_size, max_context,
                                 softmax_scale, num_splits, nullptr, nullptr, nullptr, 0, nullptr, nullptr, out,
                                 workspace, workspace_bytes, err_word, stream);
}

int dq_decode_attention_noalloc(const dq_tables* t, const void* q, int q_dtype, const uint8_t* k_cache,
                                const uint8_t* v_cache, const uint16_t* k_norm, const uint16_t* v_norm,
                                const int32_t* block_table, const int32_t* context_lens, int batch,
                                int num_q_heads, int num_kv_heads, int max_pages_per_seq, int page_size,
                                int max_context, float softmax_scale, int num_splits, float* out,
                                uint32_t* err_word, void* stream) {
    if (!t || !t->d_scratch) return DQ_ERR_INVALID_ARG;
    return decode_attention_impl(t, q, q_dtype, k_cache, v_cache, k_norm, v_norm, block_table, context_lens,
                                 batch, num_q_heads, num_kv_heads, max_pages_per_seq, page_size, max_context,
                                 softmax_scale, num_splits, nullptr, nullptr, nullptr, 0, nullptr, nullptr, out,
                                 t->d_scratch, dq::kScratchBytes, err_word, stream);
}

int dq_bf16_decode_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                             const int32_t* block_table, const int32_t* context_lens, int batch,
                             int num_q_heads, int num_kv_heads, int max_pages_per_seq, int page_size,
                             int max_context, float softmax_scale, int num_splits, float* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out || !workspace)
        return DQ_ERR_INVALID_ARG;
    if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
        max_pages_per_seq <= 0 || page_size <= 0 || page_size % 16 || max_context < 0 ||
        num_splits < 0 || (long)max_pages_per_seq * page_size < max_context)
        return DQ_ERR_INVALID_ARG;
    if (num_q_heads / num_kv_heads > 4 || (page_size & (page_size - 1))) return DQ_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace))
        return DQ_ERR_INVALID_ARG;
    const int splits = num_splits ? num_splits : dq::choose_splits(batch, num_kv_heads, max_context);
    if (workspace_bytes < dq_workspace_size(batch, num_q_heads, num_kv_heads, max_context, splits))
        return DQ_ERR_WORKSPACE;
    if ((long)batch * num_kv_heads * splits > (long)INT32_MAX / 4) return DQ_ERR_INVALID_ARG;
    dq::Bf16Args a;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.batch = batch;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.max_pages_per_seq = max_pages_per_seq;
    a.page_size = page_size;
    a.log2p = 31 - __builtin_clz((unsigned)page_size);
    a.num_splits = splits;
    a.split_len = dq::split_tokens(max_context, splits);
    a.slot_count = splits + 1;
    a.token_cap = max_context;   // within the pages and the splits (checked above / by construction)
    a.softmax_scale = softmax_scale > 0 ? softmax_scale : 1.0f / sqrtf((float)dq::kHeadDim);
    a.partials = (float*)workspace;
    a.out = out;
    hipError_t e = dq::launch_bf16_attention(a, (hipStream_t)stream);
    return e == hipSuccess ? DQ_OK : hip_fail(e);
}

int dq_decode_attention_window(const dq_tables* t, const void* q, int q_dtype, const uint8_t* k_cache,
                               const uint8_t* v_cache, const uint16_t* k_norm, const uint16_t* v_norm,
                               const int32_t* block_table, const int32_t* context_lens, int batch,
                               int num_q_heads, int num_kv_heads, int max_pages_per_seq, int page_size,
                               int max_context, float softmax_scale, int num_splits, const uint16_t* window_k,
                               const uint16_t* window_v, const int32_t* window_lens, int window_cap, float* out,
                               void* workspace, size_t workspace_bytes, uint32_t* err_word, void* stream) {
    if (!window_k) return DQ_ERR_INVALID_ARG;
    return decode_attention_impl(t, q, q_dtype, k_cache, v_cache, k_norm, v_norm, block_table, context_lens,
                                 batch, num_q_heads, num_kv_heads, max_pages_per_seq, page_size, max_context,
                                 softmax_scale, num_splits, window_k, window_v, window_lens, window_cap, nullptr,
                                 nullptr, out, workspace, workspace_bytes, err_word, stream);
}

int dq_decode_attention_ext(const dq_tables* t, const void* q, int q_dtype, const uint8_t* k_cache,
                            const uint8_t* v_cache, const uint16_t* k_norm, const uint16_t* v_norm,
                            const int32_t* block_table, const int32_t* context_lens, int batch,
                            int num_q_heads, int num_kv_heads, int max_pages_per_seq, int page_size,
                            int max_context, float softmax_scale, int num_splits, const dq_attention_extras* ex,
                            float* out, void* workspace, size_t workspace_bytes, uint32_t* err_word,
                            void* stream) {
    dq_attention_extras none;
    memset(&none, 0, sizeof(none));
    if (!ex) ex = &none;
    if (ex->window_k && !ex->window_v) return DQ_ERR_INVALID_ARG;
    return decode_attention_impl(t, q, q_dtype, k_cache, v_cache, k_norm, v_norm, block_table, context_lens,
                                 batch, num_q_heads, num_kv_heads, max_pages_per_seq, page_size, max_context,
                                 softmax_scale, num_splits, ex->window_k, ex->window_v, ex->window_lens,
                                 ex->window_cap, ex->k_mean, ex->k_mean_scale, out, workspace, workspace_bytes,
                                 err_word, stream);
}

int dq_decode_symbols(const dq_tables* t, int which, const uint8_t* containers, int n_streams,
                      uint8_t* symbols_out, uint32_t* err_word, void* stream) {
    if (!t || t->format != 0 || (which != DQ_KEYS && which != DQ_VALUES) || n_streams < 0)
        return DQ_ERR_INVALID_ARG;
    if (n_streams == 0) return DQ_OK;
    if (!containers || !symbols_out || !aligned16(containers) || !aligned16(symbols_out))
        return DQ_ERR_INVALID_ARG;
    const dq_table_info& ti = t->info[which];
    hipError_t e = dq::launch_decode_symbols(t->d_entries + which * dq::kTableSlots, ti.prob_bits,
                                             ti.levels, ti.container, containers, n_streams,
                                             symbols_out, err_word, (hipStream_t)stream);
    return e == hipSuccess ? DQ_OK : hip_fail(e);
}

size_t dq_token_workspace_size(int batch, int num_q_heads, int max_context, int num_splits) {
    if (batch <= 0 || num_q_heads <= 0 || max_context < 0 || num_splits < 0) return 0;
    const int s = num_splits ? num_splits : dq::token_choose_splits(batch, max_context);
    return (size_t)batch * num_q_heads * (s + 1) * dq::kPartStride * sizeof(float);
}

int dq_token_decode_attention_ext(const dq_tables* t, const void* q, int q_dtype, const uint8_t* k_cache,
                                  const uint8_t* v_cache, const uint16_t* k_meta, const uint16_t* v_meta,
                                  const int32_t* block_table, const int32_t* context_lens, int batch,
                                  int num_q_heads, int max_pages_per_seq, int page_size, int max_context,
                                  float softmax_scale, int num_splits, const dq_attention_extras* ex, float* out,
                                  void* workspace, size_t workspace_bytes, uint32_t* err_word, void* stream) {
    if (!t || t->format != 1 || !q || !k_cache || !v_cache || !k_meta || !v_meta || !block_table ||
        !context_lens || !out || !workspace)
        return DQ_ERR_INVALID_ARG;
    if (q_dtype != DQ_DTYPE_F32 && q_dtype != DQ_DTYPE_BF16) return DQ_ERR_INVALID_ARG;
    if (batch <= 0 || num_q_heads <= 0 || max_pages_per_seq <= 0 || page_size <= 0 || max_context < 0 ||
        num_splits < 0 || (long)max_pages_per_seq * page_size < max_context)
        return DQ_ERR_INVALID_ARG;
    if (num_q_heads % dq::kTokHeads || num_q_heads / dq::kTokHeads > 4 || (page_size & (page_size - 1)) ||
        page_size > dq::kTokMaxPage)
        return DQ_ERR_UNSUPPORTED;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace) || ((uintptr_t)k_meta & 3u) ||
        ((uintptr_t)v_meta & 3u))
        return DQ_ERR_INVALID_ARG;
    const bool win = ex && ex->window_k;
    const bool mk = ex && ex->k_mean;
    if (ex && !ex->k_mean != !ex->k_mean_scale) return DQ_ERR_INVALID_ARG;
    if (mk && ((uintptr_t)ex->k_mean & 3u)) return DQ_ERR_INVALID_ARG;
    if (win) {
        if (!ex->window_v || !ex->window_lens || ex->window_cap <= 0 || !aligned16(ex->window_k) ||
            !aligned16(ex->window_v))
            return DQ_ERR_INVALID_ARG;
        if (ex->window_cap > dq::kWindowMax) return DQ_ERR_UNSUPPORTED;
    }
    const int splits = num_splits ? num_splits : dq::token_choose_splits(batch, max_context);
    if (workspace_bytes < dq_token_workspace_size(batch, num_q_heads, max_context, splits)) return DQ_ERR_WORKSPACE;
    if ((long)batch * splits > (long)INT32_MAX / 4) return DQ_ERR_INVALID_ARG;
    dq::TokAttnArgs a;
    a.q = q;
    a.q_dtype = q_dtype;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.k_meta = k_meta;
    a.v_meta = v_meta;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.batch = batch;
    a.num_q_heads = num_q_heads;
    a.group = num_q_heads / dq::kTokHeads;
    a.max_pages_per_seq = max_pages_per_seq;
    a.page_size = page_size;
    a.log2p = 31 - __builtin_clz((unsigned)page_size);
    a.num_splits = splits;
    a.split_len = dq::split_tokens(max_context, splits);
    a.slot_count = splits + 1;
    a.token_cap = max_context;   // within the pages and the splits (checked above / by construction)
    a.ck = t->info[0].container;
    a.cv = t->info[1].container;
    a.pk = t->info[0].prob_bits;
    a.pv = t->info[1].prob_bits;
    a.half_k = 0.5f * (float)(t->info[0].levels - 1);
    a.half_v = 0.5f * (float)(t->info[1].levels - 1);
    a.win_k = win ? ex->window_k : nullptr;
    a.win_v = win ? ex->window_v : nullptr;
    a.win_lens = win ? ex->window_lens : nullptr;
    a.win_cap = win ? ex->window_cap : 0;
    a.k_mean = mk ? ex->k_mean : nullptr;
    a.k_mean_scale = mk ? ex->k_mean_scale : nullptr;
    a.softmax_scale = softmax_scale > 0 ? softmax_scale : 1.0f / sqrtf((float)dq::kHeadDim);
    a.wide = t->d_wide;
    a.partials = (float*)workspace;
    a.out = out;
    a.err_word = err_word;
    hipError_t e = dq::launch_token_attention(a, (hipStream_t)stream);
    return e == hipSuccess ? DQ_OK : hip_fail(e);
}

int dq_token_decode_attention(const dq_tables* t, const void* q, int q_dtype, const uint8_t* k_cache,
                              const uint8_t* v_cache, const uint16_t* k_meta, const uint16_t* v_meta,
                              const int32_t* block_table, const int32_t* context_lens, int batch, int num_q_heads,
                              int max_pages_per_seq, int page_size, int max_context, float softmax_scale,
                              int num_splits, float* out, void* workspace, size_t workspace_bytes,
                              uint32_t* err_word, void* stream) {
    return dq_token_decode_attention_ext(t, q, q_dtype, k_cache, v_cache, k_meta, v_meta, block_table, context_lens,
                                         batch, num_q_heads, max_pages_per_seq, page_size, max_context,
                                         softmax_scale, num_splits, nullptr, out, workspace, workspace_bytes,
                                         err_word, stream);
}

namespace {
int token_encode_impl(const dq_tables* t, const void* k, const void* v, int dtype, int num_tokens, int page_size,
                      const int32_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache, uint16_t* k_meta,
                      uint16_t* v_meta, int8_t* k_mean, uint16_t* k_mean_scale, uint32_t* drift_stats,
                      uint32_t* err_word, void* stream) {
    if (!t || t->format != 1 || num_tokens < 0 || page_size <= 0) return DQ_ERR_INVALID_ARG;
    if (dtype != DQ_DTYPE_F32 && dtype != DQ_DTYPE_BF16) return DQ_ERR_INVALID_ARG;
    if (num_tokens == 0) return DQ_OK;
    if (!k || !v || !slot_mapping || !k_cache || !v_cache || !k_meta || !v_meta) return DQ_ERR_INVALID_ARG;
    if ((long)num_tokens * 2 > (long)INT32_MAX / 2) return DQ_ERR_INVALID_ARG;
    dq::TokEncArgs a;
    a.k = k;
    a.v = v;
    a.dtype = dtype;
    a.num_tokens = num_tokens;
    a.page_size = page_size;
    a.slot_mapping = slot_mapping;
    a.cache[0] = k_cache;
    a.cache[1] = v_cache;
    a.meta[0] = k_meta;
    a.meta[1] = v_meta;
    a.drift_stats = drift_stats;
    a.err_word = err_word;
    a.tables = t->d_enc;
    a.max_c = std::max(t->enc[0].container, t->enc[1].container);
    a.k_mean = k_mean;
    a.k_mean_scale = k_mean_scale;
    hipError_t e = dq::launch_token_encode(a, (hipStream_t)stream);
    return e == hipSuccess ? DQ_OK : hip_fail(e);
}
}  // namespace

int dq_encode_tokens(const dq_tables* t, const void* k, const void* v, int dtype, int num_tokens,
                     int page_size, const int32_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                     uint16_t* k_meta, uint16_t* v_meta, uint32_t* drift_stats, uint32_t* err_word, void* stream) {
    return token_encode_impl(t, k, v, dtype, num_tokens, page_size, slot_mapping, k_cache, v_cache, k_meta, v_meta,
                             nullptr, nullptr, drift_stats, err_word, stream);
}

int dq_encode_tokens_blocks(const dq_tables* t, const void* k, const void* v, int dtype, int num_blocks,
                            int page_size, const int32_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                            uint16_t* k_meta, uint16_t* v_meta, int8_t* k_mean, uint16_t* k_mean_scale,
                            uint32_t* drift_stats, uint32_t* err_word, void* stream) {
    if (!k_mean || !k_mean_scale || num_blocks < 0 || (long)num_blocks * dq::kMeanBlock > INT32_MAX)
        return DQ_ERR_INVALID_ARG;
    if (page_size > 0 && (page_size & (page_size - 1))) return DQ_ERR_UNSUPPORTED;
    return token_encode_impl(t, k, v, dtype, num_blocks * dq::kMeanBlock, page_size, slot_mapping, k_cache, v_cache,
                             k_meta, v_meta, k_mean, k_mean_scale, drift_stats, err_word, stream);
}

int dq_token_decode_symbols(const dq_tables* t, int which, const uint8_t* containers, int n_streams,
                            uint8_t* symbols_out, uint32_t* err_word, void* stream) {
    if (!t || t->format != 1 || (which != DQ_KEYS && which != DQ_VALUES) || n_streams < 0)
        return DQ_ERR_INVALID_ARG;
    if (n_streams == 0) return DQ_OK;
    if (!containers || !symbols_out) return DQ_ERR_INVALID_ARG;
    hipError_t e = dq::launch_token_decode_symbols(t->d_enc + which, containers, n_streams, symbols_out, err_word,
                                                   (hipStream_t)stream);
    return e == hipSuccess ? DQ_OK : hip_fail(e);
}

int dq_selftest_fp64(const double* a, const double* b, int n, double* sqrt_out, double* div_out,
                     uint16_t* f16_out, void* stream) {
    if (n < 0) return DQ_ERR_INVALID_ARG;
    if (n == 0) return DQ_OK;
    if (!a || !b || !sqrt_out || !div_out || !f16_out) return DQ_ERR_INVALID_ARG;
    hipError_t e = dq::launch_selftest_fp64(a, b, n, sqrt_out, div_out, f16_out, (hipStream_t)stream);
    return e == hipSuccess ? DQ_OK : hip_fail(e);
}

}  // extern "C"
