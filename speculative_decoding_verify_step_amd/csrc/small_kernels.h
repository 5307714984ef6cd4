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

// x += (sum of K-split partials) or (sum over ranks of gate * expert output +
// shared-expert outputs); then RMSNorm into h.  One workgroup per row.
template <bool BF, bool MOE>
__global__ __launch_bounds__(256) void residual_norm_kernel(RowArgs a)
{
    __shared__ float xs[8192];
    __shared__ float sh4[4];
    const int t = blockIdx.x, H = a.H, T = a.T;
    float* xr = a.x + (size_t)t * H;
    for (int i = threadIdx.x; i < H; i += 256) {
        float d = 0.f;
        if constexpr (MOE) {
            for (int r = 0; r < a.topk; r++)
                d += a.gate[t * a.topk + r] * a.y[(size_t)a.slot[t * a.topk + r] * H + i];
            for (int s = 0; s < a.n_shared; s++)
                d += a.y[((size_t)T * a.topk + (size_t)s * T + t) * H + i];
        } else {
            for (int s = 0; s < a.nsplit; s++) d += a.parts[((size_t)s * T + t) * H + i];
        }
        float v = xr[i] + d;
        xr[i] = v;
        xs[i] = v;
        if (a.dbg_hidden) a.dbg_hidden[(size_t)t * H + i] = v;
    }
    __syncthreads();
    rms_store<BF>(xs, H, a.gain, a.eps, (typename Act<BF>::T*)a.h + (size_t)t * H, sh4);
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

// rotary on q and k (pair (i, i + D/2) turned by pos * theta^(-2i/D)), then q
// to the attention input and k, v to the caches at position ctx + j.
template <bool BF>
__global__ __launch_bounds__(256) void rope_append_kernel(RopeArgs a)
{
    const int t = blockIdx.x, K1 = a.K1, D = a.D, half = D / 2;
    const int b = t / K1, j = t % K1;
    const int QKV = (a.n_q + 2 * a.n_kv) * D;
    const bool write_cache = a.seq_err[b] == 0;
    const int pos = min(max(a.ctx_in[b], 0), a.cap - K1) + j;
    typedef typename Act<BF>::T AT;
    auto val = [&](int c) {
        float s = 0.f;
        for (int p = 0; p < a.nsplit; p++) s += a.qkv[((size_t)p * a.T + t) * QKV + c];
        return s;
    };
    const int nh = a.n_q + a.n_kv;
    for (int idx = threadIdx.x; idx < nh * half; idx += 256) {
        int hh = idx / half, i = idx % half;
        float2 cs = a.rope[(size_t)pos * half + i];
        float x0 = val(hh * D + i), x1 = val(hh * D + i + half);
        float r0 = x0 * cs.x - x1 * cs.y;
        float r1 = x1 * cs.x + x0 * cs.y;
        if (hh < a.n_q) {
            AT* qo = (AT*)a.q + ((size_t)t * a.n_q + hh) * D;
            Act<BF>::st(qo, i, r0);
            Act<BF>::st(qo, i + half, r1);
        } else if (write_cache) {
            int kh = hh - a.n_q;
            size_t base = (((size_t)b * a.L + a.layer) * a.n_kv + kh) * (size_t)a.cap;
            AT* kp = (AT*)a.kc + (base + pos) * D;
            Act<BF>::st(kp, i, r0);
            Act<BF>::st(kp, i + half, r1);
        }
    }
    if (write_cache) {
        for (int idx = threadIdx.x; idx < a.n_kv * D; idx += 256) {
            int vh = idx / D, d = idx % D;
            float v = val((a.n_q + a.n_kv + vh) * D + d);
            size_t base = ((((size_t)b * a.L + a.layer) * a.n_kv + vh) * D + d) * (size_t)a.cap;
            Act<BF>::st((AT*)a.vc, base + pos, v);
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

// Router: softmax over the E logits of every row (fp32), top-k by probability
// (lower index first on ties), gates = the selected probabilities (optionally
// renormalised).  Then a stable counting sort of the T*topk assignments by
// expert -- assignment (t, r) of expert e goes to offset[e] + (number of rows
// t' < t that also chose e) -- followed by the shared-expert rows (every token,
// in order), and the list of BM-row tiles per group for the grouped GEMMs.
// One workgroup; deterministic.
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a)
{
    extern __shared__ unsigned short cnt[];          // [T][E]
    __shared__ int total[256], offset[257];
    const int T = a.T, E = a.E, k = a.topk;
    for (int i = threadIdx.x; i < T * E; i += 256) cnt[i] = 0;
    __syncthreads();
    for (int t = threadIdx.x; t < T; t += 256) {
        float* p = a.probs + (size_t)t * E;
        float m = -INFINITY;
        for (int e = 0; e < E; e++) {
            float s = 0.f;
            for (int q = 0; q < a.nsplit; q++) s += a.logits[((size_t)q * T + t) * E + e];
            p[e] = s;
            m = fmaxf(m, s);
        }
        float sum = 0.f;
        for (int e = 0; e < E; e++) { float v = __expf(p[e] - m); p[e] = v; sum += v; }
        float inv = 1.f / sum;
        for (int e = 0; e < E; e++) p[e] *= inv;
        float gsum = 0.f;
        int chosen[8];
        for (int r = 0; r < k; r++) {
            int best = -1;
            float bv = 0.f;
            for (int e = 0; e < E; e++) {
                bool taken = false;
                for (int q = 0; q < r; q++) taken |= (chosen[q] == e);
                if (taken) continue;
                float v = p[e];
                if (best < 0 || v > bv) { best = e; bv = v; }
            }
            chosen[r] = best;
            gsum += bv;
        }
        for (int r = 0; r < k; r++) {
            int e = chosen[r];
            a.sel[t * k + r] = e;
            if (a.dbg_sel) a.dbg_sel[t * k + r] = e;
            a.gate[t * k + r] = a.renorm ? p[e] / gsum : p[e];
            cnt[t * E + e] = 1;
        }
    }
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
        for (int s = 0; s < a.n_shared; s++) {
            for (int r0 = 0; r0 < T; r0 += a.BM) {
                if (nt < a.max_tiles) {
                    a.tiles[3 * nt] = E + s;
                    a.tiles[3 * nt + 1] = T * k + s * T + r0;
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
            int e = a.sel[t * k + r];
            int s = offset[e] + cnt[t * E + e];
            a.slot[t * k + r] = s;
            a.perm_tok[s] = t;
        }
        for (int s = 0; s < a.n_shared; s++) a.perm_tok[T * k + s * T + t] = t;
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
// context length.  One wave per sequence.
__global__ __launch_bounds__(64) void accept_kernel(AcceptArgs a)
{
    __shared__ int g[64];
    __shared__ int nan_seen;
    const int b = blockIdx.x, K1 = a.K1, K = K1 - 1, lane = threadIdx.x;
    if (lane == 0) nan_seen = 0;
    __syncthreads();
    for (int j = 0; j < K1; j++) {
        const int t = b * K1 + j;
        unsigned long long best = 0ull;
        for (int n = lane; n < a.NT; n += 64) best = umax64(best, a.keys[(size_t)n * a.T + t]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) best = umax64(best, shfl_xor_u64(best, m));
        if (lane == 0) {
            if (best == ~0ull) nan_seen = 1;
            g[j] = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
        }
    }
    __syncthreads();
    if (lane == 0) {
        unsigned e = a.seq_err ? (unsigned)a.seq_err[b] : 0u;
        if (nan_seen) e |= SV_DEV_NAN_LOGIT;
        int c = a.ctx_in[b];
        if (e) {
            if (a.seq_err == nullptr || nan_seen) atomicOr(a.err_word, e);
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
        for (int j = lane; j < K1; j += 64) a.target[(size_t)b * K1 + j] = g[j];
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
