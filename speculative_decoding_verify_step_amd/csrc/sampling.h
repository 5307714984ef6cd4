// sampling.h -- stochastic (rejection-sampling) verification on the GPU.
//
// The target's logits of the K+1 verified positions of every sequence are in
// an fp32 buffer [T][V] (row t = b (K+1) + j).  Three kernels turn them into
// the step's outcome:
//
//   sample_stats_kernel   per (row, 4096-entry vocabulary tile): the maximum
//                         of z = logit / tau and the sum of exp(z - max)
//   sample_draw_kernel    per (sequence, tile): every workgroup of a sequence
//                         takes the same acceptance decision from the
//                         statistics (log-sum-exp of each row, then the test
//                         u_i q_i(d_i) < p_{i-1}(d_i) left to right), then
//                         draws over its tile of the one row that needs a
//                         draw: the residual max(0, p_a - q_{a+1}) at the
//                         first rejected position a, else p_K (the bonus)
//   sample_finish_kernel  per sequence: the largest draw key over the tiles,
//                         the outputs and the commit
// Only one row per sequence is read by the draw, so the cost beyond the
// statistics pass does not grow with K.
//
// Method: speculative sampling as in Leviathan et al. (2023) and Chen et al.
// (2023): each draft is kept with probability min(1, p/q); the first rejected
// one is replaced by a draw from max(0, p - q) normalised; when every draft
// is kept a bonus token is drawn from the target.  "Architecture and
// acceleration of an end-to-end OCR expert model", section 6.1, states the
// property this keeps: the output is distributed exactly as the target's own
// decoding.
//
// Draws use the exponential-race form of the Gumbel-max construction: with
// independent E_v ~ Exp(1), the index of the largest w_v / E_v is distributed
// as the normalised weights w (it is the largest log w_v + Gumbel noise
// -log E_v), so a draw over 129k entries is an order-independent argmax that
// splits over tiles like the greedy argmax.  E_v of (sequence b, position j,
// entry v) comes from Philox4x32-10 (Salmon et al., SC 2011): key = the
// 64-bit seed, counter = (v / 4, j, b, offset), word v % 4; a word w becomes
// the uniform ((w >> 9) + 0.5) 2^-23 (exact in fp32, inside (0, 1)) and
// E = -log(uniform).  Ties go to the lower index (the argmax key of
// common.h).  A residual with no positive entry (only through rounding, when
// p_a and q_{a+1} agree) falls back to the draw from p_a with the same noise.
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
    unsigned long long* dkeys;      // [B][ntile] draw keys (residual, or p_K for the bonus)
    unsigned long long* fkeys;      // [B][ntile] draw keys from p_a (the residual's fallback)
    int* decision;                  // [B] accepted count | error bits << 8 (written by tile 0)
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

SV_DEV float exp1_from_word(uint32_t w)
{
    const float u = ((float)(w >> 9) + 0.5f) * 0x1p-23f;
    return -logf(u);
}

// Exp(1) variables of the four consecutive entries v0 .. v0+3 (v0 % 4 == 0).
SV_DEV float4 exp1x4(const SampleArgs& a, int b, int j, int v0)
{
    const uint4 w = philox4x32_10(make_uint4((uint32_t)v0 >> 2, (uint32_t)j, (uint32_t)b, a.offset),
                                  a.key0, a.key1);
    return make_float4(exp1_from_word(w.x), exp1_from_word(w.y), exp1_from_word(w.z),
                       exp1_from_word(w.w));
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
    __shared__ int red_nan[4];
    const int tile = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
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
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (v0[i] >= a.V) continue;
        s += expf(z[i].x - m);
        s += expf(z[i].y - m);
        s += expf(z[i].z - m);
        s += expf(z[i].w - m);
    }
    // fixed-order combination: wave maximum, sums rescaled to it, then the
    // four waves in order
    const float M = wave_max(m);
    const float sw = wave_sum(s > 0.f ? s * expf(m - M) : 0.f);
    const bool nan_w = __any(nan);
    const int w = tid >> 6;
    if ((tid & 63) == 0) {
        red_m[w] = M;
        red_s[w] = sw;
        red_nan[w] = nan_w;
    }
    __syncthreads();
    if (tid == 0) {
        float MM = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
        float SS = 0.f;
        bool any_nan = false;
        for (int i = 0; i < 4; i++) {
            if (red_s[i] > 0.f) SS += red_s[i] * expf(red_m[i] - MM);
            any_nan |= red_nan[i] != 0;
        }
        if (any_nan) MM = __int_as_float(0x7fc00000);
        a.stats[(size_t)t * a.ntile + tile] = make_float2(MM, SS);
    }
}

// Grid (ntile, B), 256 threads.
__global__ __launch_bounds__(256) void sample_draw_kernel(SampleArgs a)
{
    __shared__ float lse[64];
    __shared__ int nan_row[64];
    __shared__ int dec_s;
    __shared__ unsigned long long red_d[4], red_f[4];
    const int tile = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int K1 = a.K1, K = K1 - 1, t0 = b * K1;
    // the acceptance inputs of draft lane + 1 (wave 0; clamped indices)
    const int il = min(lane, K - 1);
    int d = 0;
    float zd = 0.f, qd = 0.f, ud = 0.f;
    if (w == 0) {
        d = a.drafts[(size_t)b * K + il];
        const int dc = min(max(d, 0), a.V - 1);
        zd = a.logits[(size_t)(t0 + il) * a.V + dc] * a.inv_tau;
        qd = a.q[((size_t)b * K + il) * a.V + dc];
        ud = a.u[(size_t)b * K + il];
    }
    // log-sum-exp of every row: wave w takes rows w, w + 4, ...
    for (int j = w; j < K1; j += 4) {
        bool nj;
        const float l = row_lse(a, t0 + j, nj);
        if (lane == 0) {
            lse[j] = l;
            nan_row[j] = nj;
        }
    }
    __syncthreads();
    if (w == 0) {
        const bool bad_tok = lane < K && (d < 0 || d >= a.V);
        const float p = expf(zd - lse[il]);
        const unsigned long long rej = __ballot(lane < K && !(ud * qd < p));
        const int n = rej ? (__ffsll((long long)rej) - 1) : K;
        const bool nan_any = __any(lane < K1 && nan_row[min(lane, K1 - 1)] != 0);
        const bool bad_any = __any(bad_tok);
        if (lane == 0)
            dec_s = n | (nan_any ? (int)SV_DEV_NAN_LOGIT << 8 : 0) |
                    (bad_any ? (int)SV_DEV_BAD_TOKEN << 8 : 0);
    }
    __syncthreads();
    const int dec = dec_s, n = dec & 0xff;
    if (tile == 0 && tid == 0) a.decision[b] = dec;
    // the draw over this tile of row n: residual weights max(0, p_n - q_{n+1})
    // (n < K) or p_K, each over an Exp(1) variable; p_n / E for the fallback
    const float* __restrict__ row = a.logits + (size_t)(t0 + n) * a.V;
    const float* __restrict__ qrow = a.q + ((size_t)b * K + min(n, K - 1)) * a.V;
    const bool resid = n < K;
    const float ln = lse[n];
    float4 z[4], qv[4];
    int v0[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v0[i] = tile * SAMPLE_TILE + 1024 * i + 4 * tid;
        const int vc = min(v0[i], a.V - 4);
        z[i] = *reinterpret_cast<const float4*>(row + vc);
        qv[i] = resid ? *reinterpret_cast<const float4*>(qrow + vc) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    unsigned long long bd = 0ull, bf = 0ull;   // 0: no entry with a positive weight
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (v0[i] >= a.V) continue;
        const float4 e = exp1x4(a, b, n, v0[i]);
        const float zz[4] = {z[i].x, z[i].y, z[i].z, z[i].w};
        const float qq[4] = {qv[i].x, qv[i].y, qv[i].z, qv[i].w};
        const float ee[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const float p = expf(zz[c] * a.inv_tau - ln);
            const float r = p - qq[c];
            const uint32_t v = (uint32_t)v0[i] + c;
            if (r > 0.f) bd = umax64(bd, argmax_key(r / ee[c], v));
            if (p > 0.f) bf = umax64(bf, argmax_key(p / ee[c], v));
        }
    }
    bd = wave_max_u64(bd);
    bf = wave_max_u64(bf);
    if (lane == 0) {
        red_d[w] = bd;
        red_f[w] = bf;
    }
    __syncthreads();
    if (tid == 0) {
        a.dkeys[(size_t)b * a.ntile + tile] = umax64(umax64(red_d[0], red_d[1]), umax64(red_d[2], red_d[3]));
        a.fkeys[(size_t)b * a.ntile + tile] = umax64(umax64(red_f[0], red_f[1]), umax64(red_f[2], red_f[3]));
    }
}

// Largest of the ntile keys of one sequence (one per lane), in every lane.
SV_DEV unsigned long long tiles_best(const unsigned long long* keys, int ntile)
{
    const int lane = threadIdx.x & 63;
    unsigned long long k = lane < ntile ? keys[lane] : 0ull;
    return wave_max_u64(k);
}

// One wave per sequence.
__global__ __launch_bounds__(64) void sample_finish_kernel(SampleArgs a)
{
    const int b = blockIdx.x, lane = threadIdx.x;
    const int dec = a.decision[b], n = dec & 0xff;
    unsigned long long best = tiles_best(a.dkeys + (size_t)b * a.ntile, a.ntile);
    const unsigned long long fb = tiles_best(a.fkeys + (size_t)b * a.ntile, a.ntile);
    if (best == 0ull) best = fb;     // residual with no positive entry: draw from p_n
    const int tok = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
    if (lane == 0) {
        const unsigned e = a.seq_err ? (unsigned)a.seq_err[b] : 0u;
        unsigned mine = (unsigned)dec >> 8;
        if (best == 0ull || best == ~0ull) mine |= SV_DEV_NAN_LOGIT;
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
