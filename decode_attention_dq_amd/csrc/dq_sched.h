// Longest-job-first order of the split-K work of a decode-attention call.
//
// A job is one split of one sequence (for one KV head): the tokens
// [split * split_len, min(T_b, (split + 1) * split_len)). Its cost is the
// number of 256-token tiles it covers, from split_len / 256 for a full split
// down to 1. Jobs are numbered from the most tiles to the fewest:
//   class K (K = split_len / 256): for each sequence in order, its full
//     splits, then its last split if that one also covers K tiles;
//   class k = K-1 .. 1: the sequences whose last split covers k tiles, in
//     order.
// Work-group w takes job w / Hkv for KV head w % Hkv, so work-groups are
// dispatched longest job first; the short last splits of a ragged batch fill
// in the end of the launch instead of prolonging it, and work-groups past the
// last job exit at once. The merge reads the ceil(T_b / split_len) splits that
// exist for each sequence, so no partial slot has to be written for the rest.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dq {

constexpr int kJobTile = 256;

// Tokens of sequence b that the call covers: its length clamped to
// [0, max_context] (max_context fits the pages and the splits; the merge
// flags a length outside that range).
__host__ __device__ inline int covered_tokens(int len, int cap) { return len < 0 ? 0 : (len < cap ? len : cap); }

// Inclusive prefix sum over the wave (every lane active).
__device__ __forceinline__ int wave_scan_incl(int v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

// The job with number `job` in the order above: its sequence and split, both
// wave-uniform. Returns false when `job` is past the last job. Every lane of
// the wave must be active; lens is read B times per call (it stays in cache).
__device__ __forceinline__ bool pick_job(const int32_t* lens, int B, int cap, int split_len, int job, int lane,
                                         int& b_out, int& split_out) {
    const int K = split_len / kJobTile;
    int j = job;
    // class K: full splits, plus last splits of K tiles
    for (int c0 = 0; c0 < B; c0 += 64) {
        const int i = c0 + lane;
        const int T = i < B ? covered_tokens(lens[i], cap) : 0;
        const int full = T / split_len, rem = T - full * split_len;
        const int cls = (rem + kJobTile - 1) / kJobTile;
        const int cnt = full + (cls == K ? 1 : 0);
        const int incl = wave_scan_incl(cnt, lane);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (j < total) {
            const uint64_t hit = __ballot(incl > j && incl - cnt <= j);
            const int l = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
            b_out = c0 + l;
            split_out = j - __builtin_amdgcn_readlane(incl - cnt, l);
            return true;
        }
        j -= total;
    }
    // classes K-1 .. 1: one last split per sequence, in sequence order
    for (int k = K - 1; k >= 1; --k) {
        for (int c0 = 0; c0 < B; c0 += 64) {
            const int i = c0 + lane;
            const int T = i < B ? covered_tokens(lens[i], cap) : 0;
            const int full = T / split_len, rem = T - full * split_len;
            const bool in = i < B && (rem + kJobTile - 1) / kJobTile == k;
            const uint64_t m = __ballot(in);
            const int n = __popcll(m);
            if (j < n) {
                const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                const uint64_t hit = __ballot(in && below == j);
                const int l = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
                b_out = c0 + l;
                split_out = __builtin_amdgcn_readlane(full, l);
                return true;
            }
            j -= n;
        }
    }
    return false;
}

}  // namespace dq
