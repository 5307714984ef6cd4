// sampling.h -- stochastic (rejection-sampling) verification on the GPU.
//
// The target's logits of the K+1 verified positions of every sequence are in
// an fp32 buffer [T][V] (row t = b (K+1) + j).  Three kernels turn them into
// the step's outcome:
//
//   sample_stats_kernel     per (row, 4096-entry vocabulary tile): the running
//                           maximum and sum of exp(z - max) of z = logit / tau,
//                           and the largest Gumbel key z_v + g_v (a draw from
//                           softmax(z) restricted to the tile)
//   sample_residual_kernel  per (sequence, draft position j < K, tile): the
//                           largest key log(max(0, p_j(v) - q_{j+1}(v))) + g_v,
//                           a draw from the residual distribution, computed
//                           for every position ahead of the acceptance
//   sample_accept_kernel    per sequence: log-sum-exp of every row from the
//                           tile statistics, the acceptance test
//                           u_i q_i(d_i) < p_{i-1}(d_i) left to right, and the
//                           final draw (residual at the first rejected
//                           position, else the bonus draw from p_K)
//
// Method: speculative sampling as in Leviathan et al. (2023) and Chen et al.
// (2023): each draft is kept with probability min(1, p/q); the first rejected
// one is replaced by a draw from max(0, p - q) normalised; when every draft
// is kept a bonus token is drawn from the target.  "Architecture and
// acceleration of an end-to-end OCR expert model", section 6.1, states the
// property this keeps: the output is distributed exactly as the target's own
// decoding.
//
// Draws use the Gumbel-max construction: the index of the largest
// log-weight + standard Gumbel noise is distributed as the normalised
// weights, so a draw over 129k entries is an order-independent argmax that
// splits over tiles like the greedy argmax.  The noise of (sequence b,
// position j, entry v) comes from Philox4x32-10 (Salmon et al., SC 2011):
// key = the 64-bit seed, counter = (v / 4, j, b, offset), word v % 4; a
// word w becomes the uniform ((w >> 9) + 0.5) 2^-23 (exact in fp32, inside
// (0, 1)) and the noise is -log(-log(uniform)).  Ties go to the lower index
// (the argmax key of common.h).  A residual with no positive entry (only
// through rounding, when p_j and q_{j+1} agree) falls back to the draw from
// p_j with the same noise.
#pragma once
#include "common.h"

constexpr int SAMPLE_TILE = 4096;       // vocabulary entries per workgroup (256 lanes x 16)
constexpr int SAMPLE_MAX_TILES = 64;    // one statistics entry per lane in the reductions

struct SampleArgs {
    const float* logits;            // [T][V] target logits (before the temperature)
    const int* drafts;              // [B][K]
    const float* q;                 // [B][K][V] draft distributions
    const float* u;                 // [B][K] acceptance uniforms
    float inv_tau;
    uint32_t key0, key1, offset;    // generator key (seed low, high word) and counter word 3
    int V, T, K1, ntile;
    float2* stats;                  // [T][ntile] (max, sum of exp(z - max)); max = NaN if a NaN was seen
    unsigned long long* pkeys;      // [T][ntile] draw keys from p
    unsigned long long* rkeys;      // [B K][ntile] draw keys from the residual of position j
    const int* ctx_in;
    int* ctx_out;
    int* accepted;
    int* next_tok;
    const int* seq_err;             // optional [B]: errors found by the forward pass
    unsigned* err_word;
};

// Philox4x32 with 10 rounds: two 32x32 -> 64-bit products per round, the key
// bumped by the Weyl constants between rounds.
SV_DEV uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; r++) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
        const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    }
    return c;
}

SV_DEV float gumbel_from_word(uint32_t w)
{
    const float u = ((float)(w >> 9) + 0.5f) * 0x1p-23f;
    return -logf(-logf(u));
}

// Gumbel noise of the four consecutive entries v0 .. v0+3 (v0 % 4 == 0).
SV_DEV float4 gumbel4(const SampleArgs& a, int b, int j, int v0)
{
    const uint4 w = philox4x32_10(make_uint4((uint32_t)v0 >> 2, (uint32_t)j, (uint32_t)b, a.offset),
                                  a.key0, a.key1);
    return make_float4(gumbel_from_word(w.x), gumbel_from_word(w.y), gumbel_from_word(w.z),
                       gumbel_from_word(w.w));
}

// log-sum-exp of row t from its tile statistics (ntile <= 64, one per lane);
// every lane gets the result.  nan_out: a NaN was seen in the row.
SV_DEV float row_lse(const SampleArgs& a, int t, bool& nan_out)
{
    const int lane = threadIdx.x & 63;
    float2 st = make_float2(-INFINITY, 0.f);
    if (lane < a.ntile) st = a.stats[(size_t)t * a.ntile + lane];
    nan_out = __any(st.x != st.x);
    const float M = wave_max(st.x);
    const float s = st.y > 0.f ? st.y * expf(st.x - M) : 0.f;
    return M + logf(wave_sum(s));
}

// Grid (ntile, T), 256 threads: each thread owns four float4 groups of the
// tile, lanes side by side.
__global__ __launch_bounds__(256) void sample_stats_kernel(SampleArgs a)
{
    __shared__ float red_m[4], red_s[4];
    __shared__ unsigned long long red_k[4];
    __shared__ int red_nan[4];
    const int tile = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
    const int b = t / a.K1, j = t - b * a.K1;
    const float* __restrict__ row = a.logits + (size_t)t * a.V;
    float4 z[4];
    int v0[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {    // loads first, clamped to the row
        v0[i] = tile * SAMPLE_TILE + 1024 * i + 4 * tid;
        z[i] = *reinterpret_cast<const float4*>(row + min(v0[i], a.V - 4));
    }
    float m = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        z[i].x *= a.inv_tau;
        z[i].y *= a.inv_tau;
        z[i].z *= a.inv_tau;
        z[i].w *= a.inv_tau;
        if (v0[i] < a.V) {
            m = fmaxf(m, fmaxf(fmaxf(z[i].x, z[i].y), fmaxf(z[i].z, z[i].w)));
            nan |= z[i].x != z[i].x || z[i].y != z[i].y || z[i].z != z[i].z || z[i].w != z[i].w;
        }
    }
    float s = 0.f;
    unsigned long long best = 0ull;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (v0[i] >= a.V) continue;
        s += expf(z[i].x - m);
        s += expf(z[i].y - m);
        s += expf(z[i].z - m);
        s += expf(z[i].w - m);
        const float4 g = gumbel4(a, b, j, v0[i]);
        best = umax64(best, argmax_key(z[i].x + g.x, (uint32_t)v0[i]));
        best = umax64(best, argmax_key(z[i].y + g.y, (uint32_t)v0[i] + 1));
        best = umax64(best, argmax_key(z[i].z + g.z, (uint32_t)v0[i] + 2));
        best = umax64(best, argmax_key(z[i].w + g.w, (uint32_t)v0[i] + 3));
    }
    // fixed-order combination: wave maximum, sums rescaled to it, then the
    // four waves in order
    const float M = wave_max(m);
    const float sw = wave_sum(s > 0.f ? s * expf(m - M) : 0.f);
    best = wave_max_u64(best);
    const bool nan_w = __any(nan);
    const int w = tid >> 6;
    if ((tid & 63) == 0) {
        red_m[w] = M;
        red_s[w] = sw;
        red_k[w] = best;
        red_nan[w] = nan_w;
    }
    __syncthreads();
    if (tid == 0) {
        float MM = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
        float SS = 0.f;
        unsigned long long kk = 0ull;
        bool any_nan = false;
        for (int i = 0; i < 4; i++) {
            if (red_s[i] > 0.f) SS += red_s[i] * expf(red_m[i] - MM);
            kk = umax64(kk, red_k[i]);
            any_nan |= red_nan[i] != 0;
        }
        if (any_nan) MM = __int_as_float(0x7fc00000);
        a.stats[(size_t)t * a.ntile + tile] = make_float2(MM, SS);
        a.pkeys[(size_t)t * a.ntile + tile] = kk;
    }
}

// Grid (ntile, B K), 256 threads: row y = b K + j (draft position j < K).
__global__ __launch_bounds__(256) void sample_residual_kernel(SampleArgs a)
{
    __shared__ unsigned long long red_k[4];
    const int tile = blockIdx.x, y = blockIdx.y, tid = threadIdx.x;
    const int K = a.K1 - 1, b = y / K, j = y - b * K, t = b * a.K1 + j;
    const float* __restrict__ row = a.logits + (size_t)t * a.V;
    const float* __restrict__ qrow = a.q + (size_t)y * a.V;
    float4 z[4], qv[4];
    int v0[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v0[i] = tile * SAMPLE_TILE + 1024 * i + 4 * tid;
        const int vc = min(v0[i], a.V - 4);
        z[i] = *reinterpret_cast<const float4*>(row + vc);
        qv[i] = *reinterpret_cast<const float4*>(qrow + vc);
    }
    bool nan_row;
    const float lse = row_lse(a, t, nan_row);
    unsigned long long best = 0ull;   // 0: no positive residual entry in this thread's share
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (v0[i] >= a.V) continue;
        const float4 g = gumbel4(a, b, j, v0[i]);
        const float r0 = expf(z[i].x * a.inv_tau - lse) - qv[i].x;
        const float r1 = expf(z[i].y * a.inv_tau - lse) - qv[i].y;
        const float r2 = expf(z[i].z * a.inv_tau - lse) - qv[i].z;
        const float r3 = expf(z[i].w * a.inv_tau - lse) - qv[i].w;
        if (r0 > 0.f) best = umax64(best, argmax_key(logf(r0) + g.x, (uint32_t)v0[i]));
        if (r1 > 0.f) best = umax64(best, argmax_key(logf(r1) + g.y, (uint32_t)v0[i] + 1));
        if (r2 > 0.f) best = umax64(best, argmax_key(logf(r2) + g.z, (uint32_t)v0[i] + 2));
        if (r3 > 0.f) best = umax64(best, argmax_key(logf(r3) + g.w, (uint32_t)v0[i] + 3));
    }
    best = wave_max_u64(best);
    if ((tid & 63) == 0) red_k[tid >> 6] = best;
    __syncthreads();
    if (tid == 0)
        a.rkeys[(size_t)y * a.ntile + tile] =
            umax64(umax64(red_k[0], red_k[1]), umax64(red_k[2], red_k[3]));
}

// Largest of the ntile keys of one row (one per lane), in every lane.
SV_DEV unsigned long long row_best(const unsigned long long* keys, int ntile)
{
    const int lane = threadIdx.x & 63;
    unsigned long long k = lane < ntile ? keys[lane] : 0ull;
    return wave_max_u64(k);
}

// One wave per sequence.
__global__ __launch_bounds__(64) void sample_accept_kernel(SampleArgs a)
{
    const int b = blockIdx.x, lane = threadIdx.x, K1 = a.K1, K = K1 - 1;
    const int t0 = b * K1;
    // the acceptance inputs of draft lane + 1 (loaded first; clamped indices)
    const int il = min(lane, K - 1);
    const int d = a.drafts[(size_t)b * K + il];
    const bool bad_tok = lane < K && (d < 0 || d >= a.V);
    const int dc = min(max(d, 0), a.V - 1);
    const float zd = a.logits[(size_t)(t0 + il) * a.V + dc] * a.inv_tau;
    const float qd = a.q[((size_t)b * K + il) * a.V + dc];
    const float ud = a.u[(size_t)b * K + il];
    // log-sum-exp of every row; lane j keeps row j's (K1 <= 64)
    float lse_mine = 0.f;
    bool nan_any = false;
    for (int j = 0; j < K1; j++) {
        bool nan_j;
        const float l = row_lse(a, t0 + j, nan_j);
        nan_any |= nan_j;
        if (lane == j) lse_mine = l;
    }
    const float p = expf(zd - lse_mine);
    const unsigned long long rej = __ballot(lane < K && !(ud * qd < p));
    const int n = rej ? (__ffsll((long long)rej) - 1) : K;
    unsigned long long best;
    if (n < K) {
        best = row_best(a.rkeys + ((size_t)b * K + n) * a.ntile, a.ntile);
        if (best == 0ull) best = row_best(a.pkeys + (size_t)(t0 + n) * a.ntile, a.ntile);
    } else {
        best = row_best(a.pkeys + (size_t)(t0 + K) * a.ntile, a.ntile);
    }
    const int tok = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
    const bool bad_any = __any(bad_tok);
    if (lane == 0) {
        unsigned e = a.seq_err ? (unsigned)a.seq_err[b] : 0u;
        unsigned mine = 0u;
        if (nan_any || best == ~0ull) mine |= SV_DEV_NAN_LOGIT;
        if (bad_any) mine |= SV_DEV_BAD_TOKEN;
        const int c = a.ctx_in[b];
        if (e | mine) {
            if (mine) atomicOr(a.err_word, mine);
            a.accepted[b] = -1;
            a.next_tok[b] = -1;
            a.ctx_out[b] = c;
        } else {
            a.accepted[b] = n;
            a.next_tok[b] = tok;
            a.ctx_out[b] = c + n + 1;
        }
    }
}
