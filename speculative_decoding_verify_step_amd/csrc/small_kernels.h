// small_kernels.h -- the row-wise and bookkeeping kernels of the verify step:
// token block + embedding + first RMSNorm, rotary + KV append, residual
// update + RMSNorm (after the attention projection, after the FFN), MoE
// routing (softmax, top-k, stable permutation and tile list), and
// longest-prefix acceptance + commit.
#pragma once
#include "common.h"

template <bool BF> struct Act;
template <> struct Act<true> {
    typedef uint16_t T;
    static SV_DEV float ld(const T* p, size_t i) { return bf16_bits_to_f32(p[i]); }
    static SV_DEV void st(T* p, size_t i, float v) { p[i] = (uint16_t)f32_to_bf16_bits(v); }
};
template <> struct Act<false> {
    typedef float T;
    static SV_DEV float ld(const T* p, size_t i) { return p[i]; }
    static SV_DEV void st(T* p, size_t i, float v) { p[i] = v; }
};

// Block-wide sum over 256 threads (deterministic: fixed butterfly, then a
// fixed-order sum of the four wave totals).
SV_DEV float block_sum256(float v, float* sh4)
{
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh4[w] = v;
    __syncthreads();
    float s = (sh4[0] + sh4[1]) + (sh4[2] + sh4[3]);
    __syncthreads();
    return s;
}

// x[H] (fp32 in `xs`, shared) -> h = x / sqrt(mean(x^2) + eps) * g, stored as act
template <bool BF>
SV_DEV void rms_store(const float* xs, int H, const float* g, float eps, typename Act<BF>::T* h,
                      float* sh4)
{
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += 256) ss += xs[i] * xs[i];
    ss = block_sum256(ss, sh4);
    float r = rsqrtf(ss / (float)H + eps);
    for (int i = threadIdx.x; i < H; i += 256) Act<BF>::st(h, i, xs[i] * r * g[i]);
}

struct RowArgs {
    int H, K1, V, cap, E, topk, n_shared, T, nsplit;
    float eps;
    const int* committed;       // [B]
    const int* drafts;          // [B][K]
    const int* ctx_in;          // [B]
    int* seq_err;               // [B]
    unsigned* err_word;         // sticky
    const void* embed;          // [V][H]
    float* x;                   // [T][H] residual
    void* h;                    // [T][H] normalised activations
    const float* gain;          // [H] gain of the norm that follows
    const float* parts;         // [nsplit][T][H] partial sums to add (or null)
    const float* y;             // MoE expert outputs [rows][H]
    const float* gate;          // [T][topk]
    const int* slot;            // [T][topk]
    float* dbg_hidden;          // optional [T][H] copy of x after the update
};

// token block + embedding gather + RMSNorm (one workgroup per row)
template <bool BF>
__global__ __launch_bounds__(256) void embed_norm_kernel(RowArgs a)
{
    __shared__ float xs[8192];
    __shared__ float sh4[4];
    const int t = blockIdx.x, K1 = a.K1, K = K1 - 1;
    const int b = t / K1, j = t % K1;
    int tok = (j == 0) ? a.committed[b] : a.drafts[(size_t)b * K + j - 1];
    bool bad = tok < 0 || tok >= a.V;
    if (j == 0 && threadIdx.x == 0) {
        unsigned e = 0;
        for (int i = 0; i < K1; i++) {
            int ti = (i == 0) ? a.committed[b] : a.drafts[(size_t)b * K + i - 1];
            if (ti < 0 || ti >= a.V) e |= SV_DEV_BAD_TOKEN;
        }
        int c = a.ctx_in[b];
        if (c < 0 || c + K1 > a.cap) e |= SV_DEV_CAPACITY;
        a.seq_err[b] = (int)e;
        if (e) atomicOr(a.err_word, e);
    }
    if (bad) tok = 0;
    const typename Act<BF>::T* er = (const typename Act<BF>::T*)a.embed + (size_t)tok * a.H;
    for (int i = threadIdx.x; i < a.H; i += 256) {
        float v = Act<BF>::ld(er, i);
        xs[i] = v;
        a.x[(size_t)t * a.H + i] = v;
    }
    __syncthreads();
    rms_store<BF>(xs, a.H, a.gain, a.eps, (typename Act<BF>::T*)a.h + (size_t)t * a.H, sh4);
}

// Sum of `n` fp32 values `stride` apart, loads issued together.
SV_DEV float sum_strided(const float* __restrict__ p, int n, size_t stride)
{
    float acc = 0.f;
#pragma unroll 8
    for (int s = 0; s < n; s++) acc += p[(size_t)s * stride];
    return acc;
}

// Block-wide sum over RT threads (deterministic: butterfly within waves, then
// the wave totals in wave order).
template <int RT>
SV_DEV float block_sum(float v, float* shw)
{
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) shw[w] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < RT / 64; i++) s += shw[i];
    __syncthreads();
    return s;
}

// x += (sum of K-split partials) or (sum over ranks of gate * expert output +
// shared-expert outputs); then RMSNorm into h.  One 1024-thread workgroup per
// row, so a thread owns one or two columns and issues all of a column's loads
// (every split, or every rank and shared expert) before consuming any.
template <bool BF, bool MOE>
__global__ __launch_bounds__(1024) void residual_norm_kernel(RowArgs a)
{
    constexpr int RT = 1024;
    __shared__ float xs[8192];
    __shared__ float shw[RT / 64];
    const int t = blockIdx.x, H = a.H, T = a.T;
    float* __restrict__ xr = a.x + (size_t)t * H;
    const float* __restrict__ y = a.y;
    int slot[8];
    float gate[8];
    if constexpr (MOE) {
#pragma unroll
        for (int r = 0; r < 8; r++) {
            slot[r] = r < a.topk ? a.slot[t * a.topk + r] : 0;
            gate[r] = r < a.topk ? a.gate[t * a.topk + r] : 0.f;
        }
    }
    float ss = 0.f;
    for (int i = threadIdx.x; i < H; i += RT) {
        float d = 0.f;
        if constexpr (MOE) {
            float v[8];
#pragma unroll
            for (int r = 0; r < 8; r++) v[r] = r < a.topk ? y[(size_t)slot[r] * H + i] : 0.f;
#pragma unroll
            for (int r = 0; r < 8; r++) d += gate[r] * v[r];
            d += sum_strided(y + ((size_t)T * a.topk + t) * H + i, a.n_shared, (size_t)T * H);
        } else {
            d = sum_strided(a.parts + (size_t)t * H + i, a.nsplit, (size_t)T * H);
        }
        float v = xr[i] + d;
        xr[i] = v;
        xs[i] = v;
        ss += v * v;
        if (a.dbg_hidden) a.dbg_hidden[(size_t)t * H + i] = v;
    }
    ss = block_sum<RT>(ss, shw);
    const float r = rsqrtf(ss / (float)H + a.eps);
    typename Act<BF>::T* h = (typename Act<BF>::T*)a.h + (size_t)t * H;
    for (int i = threadIdx.x; i < H; i += RT) Act<BF>::st(h, i, xs[i] * r * a.gain[i]);
}

struct RopeArgs {
    const float* qkv;           // [nsplit][T][(n_q + 2 n_kv) D] partial sums
    int nsplit, T, K1, n_q, n_kv, D, L, layer, cap;
    const int* ctx_in;
    const int* seq_err;
    const float2* rope;         // [cap][D/2] (cos, sin)
    void* q;                    // [T][n_q][D] act
    void* kc;                   // K cache
    void* vc;                   // V cache (channel-major)
};

// Element offsets of (pos, d) inside one (sequence, layer, KV head) region of
// the tiled caches (layout documented with the C ABI).
template <bool BF>
SV_DEV size_t k_cache_index(int pos, int d, int D)
{
    constexpr int KL = BF ? 8 : 4, KT = 4 * KL, NB = KL / 4;
    const int DS = D / (4 * KL);
    const int t = pos / KT, r = pos % KT;
    const int rem = r % KL;
    const int slot = 4 * (r / KL) + (rem & 3), blk = rem >> 2;
    const int s = d / (4 * KL), g = (d % (4 * KL)) / KL, e = d % KL;
    return ((((size_t)t * NB + blk) * DS + s) * 64 + slot + 16 * g) * KL + e;
}

template <bool BF>
SV_DEV size_t v_cache_index(int pos, int d, int D)
{
    constexpr int KL = BF ? 8 : 4, KT = 4 * KL;
    const int t = pos / KT, r = pos % KT;
    const int g = r / KL, e = r % KL;
    return (((size_t)t * (D / 16) + d / 16) * 64 + (d % 16) + 16 * g) * KL + e;
}

// rotary on q and k (pair (i, i + D/2) turned by pos * theta^(-2i/D)), then q
// to the attention input and k, v to the caches at position ctx + j.  One
// wave per (row, head); grid (T, n_q + 2 n_kv).
template <bool BF>
__global__ __launch_bounds__(64) void rope_append_kernel(RopeArgs a)
{
    const int t = blockIdx.x, hh = blockIdx.y, lane = threadIdx.x;
    const int K1 = a.K1, D = a.D, half = D / 2;
    const int b = t / K1, j = t % K1;
    const int QKV = (a.n_q + 2 * a.n_kv) * D;
    const bool write_cache = a.seq_err[b] == 0;
    const int pos = min(max(a.ctx_in[b], 0), a.cap - K1) + j;
    typedef typename Act<BF>::T AT;
    const float* __restrict__ src = a.qkv + (size_t)t * QKV + (size_t)hh * D;
    const size_t sstride = (size_t)a.T * QKV;
    if (hh < a.n_q + a.n_kv) {
        for (int i = lane; i < half; i += 64) {
            float2 cs = a.rope[(size_t)pos * half + i];
            float x0 = sum_strided(src + i, a.nsplit, sstride);
            float x1 = sum_strided(src + i + half, a.nsplit, sstride);
            float r0 = x0 * cs.x - x1 * cs.y;
            float r1 = x1 * cs.x + x0 * cs.y;
            if (hh < a.n_q) {
                AT* qo = (AT*)a.q + ((size_t)t * a.n_q + hh) * D;
                Act<BF>::st(qo, i, r0);
                Act<BF>::st(qo, i + half, r1);
            } else if (write_cache) {
                int kh = hh - a.n_q;
                AT* kp = (AT*)a.kc + (((size_t)b * a.L + a.layer) * a.n_kv + kh) * (size_t)a.cap * D;
                Act<BF>::st(kp, k_cache_index<BF>(pos, i, D), r0);
                Act<BF>::st(kp, k_cache_index<BF>(pos, i + half, D), r1);
            }
        }
    } else if (write_cache) {
        int vh = hh - a.n_q - a.n_kv;
        AT* vp = (AT*)a.vc + (((size_t)b * a.L + a.layer) * a.n_kv + vh) * (size_t)a.cap * D;
        for (int d = lane; d < D; d += 64) {
            float v = sum_strided(src + d, a.nsplit, sstride);
            Act<BF>::st(vp, v_cache_index<BF>(pos, d, D), v);
        }
    }
}

struct RouteArgs {
    const float* logits;        // [nsplit][T][E] partial router logits
    int nsplit, T, E, topk, n_shared, renorm, BM, max_tiles;
    float* probs;               // [T][E] workspace: routing probabilities
    int* sel;                   // [T][topk]
    float* gate;                // [T][topk]
    int* slot;                  // [T][topk] row of (t, rank) in the permuted order
    int* perm_tok;              // [T*topk + n_shared*T] token of every permuted row
    int* tiles;                 // [max_tiles][3]
    int* n_tiles;               // [1]
    int* dbg_sel;               // optional copy of sel
};

// Router, part 1: softmax over the E router logits of every row (fp32), top-k
// by probability with the lower expert index first on ties, gates = the
// selected probabilities (optionally renormalised).  One wave per row; lane l
// holds experts l, l+64, l+128, l+192.
__global__ __launch_bounds__(256) void route_topk_kernel(RouteArgs a)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;
    const int E = a.E, k = a.topk, T = a.T;
    float p[4];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        int e = lane + 64 * q;
        p[q] = e < E ? sum_strided(a.logits + (size_t)t * E + e, a.nsplit, (size_t)T * E) : -INFINITY;
        m = fmaxf(m, p[q]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        p[q] = (lane + 64 * q < E) ? __expf(p[q] - m) : 0.f;
        sum += p[q];
    }
    sum = wave_sum(sum);
    const float inv = 1.f / sum;
#pragma unroll
    for (int q = 0; q < 4; q++) p[q] *= inv;
    bool taken[4] = {false, false, false, false};
    float gsum = 0.f, chosen_p[8];
    int chosen[8];
    for (int r = 0; r < k; r++) {
        unsigned long long best = 0ull;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            int e = lane + 64 * q;
            if (e < E && !taken[q]) best = umax64(best, argmax_key(p[q], (uint32_t)e));
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) best = umax64(best, shfl_xor_u64(best, o));
        int e = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
        const int qq = e >> 6;   // expert e lives in register qq of lane e % 64
#pragma unroll
        for (int q = 0; q < 4; q++)
            if ((e & 63) == lane && q == qq) taken[q] = true;
        float v0 = __shfl(p[0], e & 63, 64), v1 = __shfl(p[1], e & 63, 64);
        float v2 = __shfl(p[2], e & 63, 64), v3 = __shfl(p[3], e & 63, 64);
        float pe = qq == 0 ? v0 : (qq == 1 ? v1 : (qq == 2 ? v2 : v3));
        chosen[r] = e;
        chosen_p[r] = pe;
        gsum += pe;
    }
    if (lane < k) {
        float pe = 0.f;
        int e = 0;
        for (int r = 0; r < k; r++)
            if (r == lane) { pe = chosen_p[r]; e = chosen[r]; }
        a.sel[t * k + lane] = e;
        if (a.dbg_sel) a.dbg_sel[t * k + lane] = e;
        a.gate[t * k + lane] = a.renorm ? pe / gsum : pe;
    }
}

// Router, part 2: a stable counting sort of the T*topk assignments by expert
// -- assignment (t, r) of expert e goes to offset[e] + (number of rows t' < t
// that also chose e) -- followed by the shared-expert rows (every token, in
// order), and the list of BM-row tiles per group for the grouped GEMMs.  One
// workgroup; deterministic.
__global__ __launch_bounds__(256) void route_permute_kernel(RouteArgs a)
{
    extern __shared__ unsigned short cnt[];          // [T][E], then sel [T][topk] as shorts
    __shared__ int total[256], offset[257];
    const int T = a.T, E = a.E, k = a.topk;
    unsigned short* sel = cnt + (size_t)T * E;
    for (int i = threadIdx.x; i < T * E; i += 256) cnt[i] = 0;
    for (int i = threadIdx.x; i < T * k; i += 256) sel[i] = (unsigned short)a.sel[i];
    __syncthreads();
    for (int t = threadIdx.x; t < T; t += 256)
        for (int r = 0; r < k; r++) cnt[t * E + sel[t * k + r]] = 1;
    __syncthreads();
    // exclusive scan over tokens, one expert per thread
    for (int e = threadIdx.x; e < E; e += 256) {
        int run = 0;
        for (int t = 0; t < T; t++) {
            int c = cnt[t * E + e];
            cnt[t * E + e] = (unsigned short)run;
            run += c;
        }
        total[e] = run;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int off = 0, nt = 0;
        for (int e = 0; e < E; e++) {
            offset[e] = off;
            for (int r0 = 0; r0 < total[e]; r0 += a.BM) {
                if (nt < a.max_tiles) {
                    a.tiles[3 * nt] = e;
                    a.tiles[3 * nt + 1] = off + r0;
                    a.tiles[3 * nt + 2] = min(a.BM, total[e] - r0);
                }
                nt++;
            }
            off += total[e];
        }
        offset[E] = off;
        for (int sx = 0; sx < a.n_shared; sx++) {
            for (int r0 = 0; r0 < T; r0 += a.BM) {
                if (nt < a.max_tiles) {
                    a.tiles[3 * nt] = E + sx;
                    a.tiles[3 * nt + 1] = T * k + sx * T + r0;
                    a.tiles[3 * nt + 2] = min(a.BM, T - r0);
                }
                nt++;
            }
        }
        *a.n_tiles = min(nt, a.max_tiles);
    }
    __syncthreads();
    for (int t = threadIdx.x; t < T; t += 256) {
        for (int r = 0; r < k; r++) {
            int e = sel[t * k + r];
            int sl = offset[e] + cnt[t * E + e];
            a.slot[t * k + r] = sl;
            a.perm_tok[sl] = t;
        }
        for (int sx = 0; sx < a.n_shared; sx++) a.perm_tok[T * k + sx * T + t] = t;
    }
}

struct AcceptArgs {
    const unsigned long long* keys;   // [NT][T]
    int NT, T, K1;
    const int* drafts;                // [B][K]
    const int* ctx_in;
    int* ctx_out;
    int* accepted;
    int* next_tok;
    int* target;                      // optional [B][K1]
    const int* seq_err;               // optional [B]
    unsigned* err_word;
};

// Greedy token per position (max over the column-tile keys), then the longest
// prefix of drafts equal to the target's tokens, the bonus token, and the new
// context length.  One workgroup of 4 waves per sequence; wave w reduces the
// positions j = w, w+4, ...
__global__ __launch_bounds__(256) void accept_kernel(AcceptArgs a)
{
    __shared__ int g[64];
    __shared__ int nan_seen[64];
    const int b = blockIdx.x, K1 = a.K1, K = K1 - 1;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int j = w; j < K1; j += 4) {
        const int t = b * K1 + j;
        const unsigned long long* __restrict__ kp = a.keys + t;
        unsigned long long part[8] = {0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull};
        int n = lane;
        for (; n + 7 * 64 < a.NT; n += 8 * 64) {
#pragma unroll
            for (int u = 0; u < 8; u++) part[u] = umax64(part[u], kp[(size_t)(n + u * 64) * a.T]);
        }
        for (; n < a.NT; n += 64) part[0] = umax64(part[0], kp[(size_t)n * a.T]);
        unsigned long long best = part[0];
#pragma unroll
        for (int u = 1; u < 8; u++) best = umax64(best, part[u]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) best = umax64(best, shfl_xor_u64(best, m));
        if (lane == 0) {
            nan_seen[j] = best == ~0ull;
            g[j] = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned e = a.seq_err ? (unsigned)a.seq_err[b] : 0u;
        int nan_any = 0;
        for (int j = 0; j < K1; j++) nan_any |= nan_seen[j];
        if (nan_any) e |= SV_DEV_NAN_LOGIT;
        int c = a.ctx_in[b];
        if (e) {
            if (a.seq_err == nullptr || nan_any) atomicOr(a.err_word, e);
            a.accepted[b] = -1;
            a.next_tok[b] = -1;
            a.ctx_out[b] = c;
        } else {
            int n = 0;
            while (n < K && a.drafts[(size_t)b * K + n] == g[n]) n++;
            a.accepted[b] = n;
            a.next_tok[b] = g[n];
            a.ctx_out[b] = c + n + 1;
        }
    }
    if (a.target)
        for (int j = threadIdx.x; j < K1; j += 256) a.target[(size_t)b * K1 + j] = g[j];
}

// fp32 logits [T][V] -> per-(column tile, row) argmax keys, for acceptance
// from given logits.  Grid (NT, T); 256 threads scan a 1024-column tile.
__global__ __launch_bounds__(256) void logits_keys_kernel(const float* logits, int V, int T,
                                                          unsigned long long* keys)
{
    __shared__ unsigned long long red[4];
    const int nt = blockIdx.x, t = blockIdx.y;
    unsigned long long best = 0ull;
    for (int n = nt * 1024 + threadIdx.x; n < min(V, (nt + 1) * 1024); n += 256)
        best = umax64(best, argmax_key(logits[(size_t)t * V + n], (uint32_t)n));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) best = umax64(best, shfl_xor_u64(best, m));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0)
        keys[(size_t)nt * T + t] = umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
}

// Row-major [rows][cols] -> 16-row blocks stored step-major (one KiB per block
// and reduction step, lane l's 16 bytes = row l%16, slice l/16 of the step).
// One thread per 16-byte slice; padding rows are written as zeros.
__global__ __launch_bounds__(256) void pack_tiled16_kernel(const char* __restrict__ src,
                                                           char* __restrict__ dst, long rows,
                                                           int cols, int esize)
{
    const int KL = 16 / esize, S = 4 * KL;
    const long steps = cols / S;
    const long nblk = (rows + 15) / 16;
    const long total = nblk * steps * 64;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int l = (int)(i & 63);
        const long bs = i >> 6;              // block * steps + step
        const long rb = bs / steps, st = bs % steps;
        const long row = rb * 16 + (l & 15);
        const long col = st * S + (long)(l >> 4) * KL;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < rows) v = *reinterpret_cast<const uint4*>(src + (row * cols + col) * esize);
        *reinterpret_cast<uint4*>(dst + i * 16) = v;
    }
}
