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
    // router fused into the norm (MoE, after attention): W_r [E][H] row-major
    const void* w_router;
    const float* s_router;      // fp8 per-row scales
    int wdtype;
    int renorm;
    int* sel;                   // [T][topk] out
    float* gate_out;            // [T][topk] out
    int* dbg_sel;               // optional copy of sel
};

// token block + embedding gather + RMSNorm (one workgroup per row)
template <bool BF>
__global__ __launch_bounds__(256) void embed_norm_kernel(RowArgs a)
{
    __shared__ __align__(16) float xs[8192];
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
// Router of one token (after the attention half's norm): logits r = W_r h
// over the stored (activation-typed) h, softmax over all E in fp32, top-k by
// probability with the lower expert index first on ties, gates = the selected
// probabilities (optionally renormalised).  Waves take experts round-robin;
// wave 0 then does the softmax and selection.
template <bool BF>
SV_DEV void route_row(const RowArgs& a, int t, const float* hs)
{
    __shared__ float logit[256];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, NW = blockDim.x >> 6;
    const int E = a.E, H = a.H, k = a.topk;
    // lane l covers elements [EPL l + 64 EPL j, + EPL) of a row (EPL = elements
    // per 16-byte load); four experts per pass keep four rows of loads in flight
    const int EPL = a.wdtype == SV_F32 ? 4 : (a.wdtype == SV_BF16 ? 8 : 16);
    const int esz = 16 / EPL;
    for (int e0 = w; e0 < E; e0 += 4 * NW) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        // up to 4 row chunks x 4 experts of loads issued before any is used
        for (int i00 = EPL * lane; i00 < H; i00 += 4 * 64 * EPL) {
            uint4 wv[4][4];
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int i0 = i00 + c * 64 * EPL;
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    int e = min(e0 + u * NW, E - 1);
                    wv[c][u] = i0 < H ? ldg16((const char*)a.w_router + ((size_t)e * H + i0) * esz)
                                      : make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int i0 = i00 + c * 64 * EPL;
                if (i0 >= H) break;
                // this lane's EPL activation values, read once (16-byte LDS reads)
                float hv[16];
                const float4* h4 = reinterpret_cast<const float4*>(hs + i0);
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    if (q * 4 < EPL) {
                        float4 t = h4[q];
                        hv[4 * q] = t.x; hv[4 * q + 1] = t.y; hv[4 * q + 2] = t.z; hv[4 * q + 3] = t.w;
                    }
                }
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const uint32_t wd[4] = {wv[c][u].x, wv[c][u].y, wv[c][u].z, wv[c][u].w};
                    if (a.wdtype == SV_F32) {
#pragma unroll
                        for (int q = 0; q < 4; q++) acc[u] += __uint_as_float(wd[q]) * hv[q];
                    } else if (a.wdtype == SV_BF16) {
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            acc[u] += bf16_bits_to_f32(wd[q] & 0xffffu) * hv[2 * q];
                            acc[u] += bf16_bits_to_f32(wd[q] >> 16) * hv[2 * q + 1];
                        }
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; q++)
#pragma unroll
                            for (int bb = 0; bb < 4; bb++)
                                acc[u] += e4m3_to_f32((wd[q] >> (8 * bb)) & 0xffu) * hv[4 * q + bb];
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            int e = e0 + u * NW;
            float v = wave_sum(acc[u]);
            if (e < E && lane == 0) logit[e] = (a.wdtype == SV_FP8) ? v * a.s_router[e] : v;
        }
    }
    __syncthreads();
    if (w != 0) return;
    float p[4];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        int e = lane + 64 * q;
        p[q] = e < E ? logit[e] : -INFINITY;
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
    for (int rr = 0; rr < k; rr++) {
        unsigned long long best = 0ull;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            int e = lane + 64 * q;
            if (e < E && !taken[q]) best = umax64(best, argmax_key(p[q], (uint32_t)e));
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) best = umax64(best, shfl_xor_u64(best, o));
        const int e = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
        const int qq = e >> 6;   // expert e lives in register qq of lane e % 64
#pragma unroll
        for (int q = 0; q < 4; q++)
            if ((e & 63) == lane && q == qq) taken[q] = true;
        float v0 = __shfl(p[0], e & 63, 64), v1 = __shfl(p[1], e & 63, 64);
        float v2 = __shfl(p[2], e & 63, 64), v3 = __shfl(p[3], e & 63, 64);
        float pe = qq == 0 ? v0 : (qq == 1 ? v1 : (qq == 2 ? v2 : v3));
        chosen[rr] = e;
        chosen_p[rr] = pe;
        gsum += pe;
    }
    if (lane < k) {
        float pe = 0.f;
        int e = 0;
        for (int rr = 0; rr < k; rr++)
            if (rr == lane) { pe = chosen_p[rr]; e = chosen[rr]; }
        a.sel[t * k + lane] = e;
        if (a.dbg_sel) a.dbg_sel[t * k + lane] = e;
        a.gate_out[t * k + lane] = a.renorm ? pe / gsum : pe;
    }
}

template <bool BF, bool MOE, bool ROUTE = false>
__global__ __launch_bounds__(1024) void residual_norm_kernel(RowArgs a)
{
    constexpr int RT = 1024;
    __shared__ __align__(16) float xs[8192];
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
    for (int i = threadIdx.x; i < H; i += RT) {
        float v = xs[i] * r * a.gain[i];
        Act<BF>::st(h, i, v);
        if constexpr (ROUTE) xs[i] = Act<BF>::ld(h, i);   // the value the experts will read
    }
    if constexpr (ROUTE) {
        __syncthreads();
        route_row<BF>(a, t, xs);
    }
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

// Router permutation: a stable counting sort of the T*topk assignments by
// expert -- assignment (t, r) of expert e goes to offset[e] + (number of rows
// t' < t that also chose e) -- followed by the shared-expert rows (every
// token, in order), and the list of BM-row tiles per group for the grouped
// GEMMs.  One 256-thread workgroup, deterministic:
//   * flags[t][e] = 1 if row t chose e;
//   * 4 threads per expert each scan a quarter of the rows, then add the
//     totals of the earlier quarters (exclusive ranks within the expert);
//   * one wave scans the per-group tile counts; each group writes its tiles.
__global__ __launch_bounds__(256) void route_permute_kernel(RouteArgs a)
{
    extern __shared__ unsigned short cnt[];          // [T][E] flags -> ranks, then sel [T][topk]
    __shared__ int total[256 * 4], offset[257], tile0[257 + 8];
    const int T = a.T, E = a.E, k = a.topk, tid = threadIdx.x;
    unsigned short* sel = cnt + (size_t)T * E;
    for (int i = tid; i < T * E; i += 256) cnt[i] = 0;
    for (int i = tid; i < T * k; i += 256) sel[i] = (unsigned short)a.sel[i];
    __syncthreads();
    for (int i = tid; i < T * k; i += 256) cnt[(i / k) * E + sel[i]] = 1;
    __syncthreads();
    // ranks: thread (e, quarter) scans rows [quarter * T/4, ...) of expert e
    const int QT = (T + 3) / 4;
    for (int job = tid; job < E * 4; job += 256) {
        const int e = job >> 2, qtr = job & 3;
        int run = 0;
        const int t1 = min(T, (qtr + 1) * QT);
        for (int t = qtr * QT; t < t1; t++) {
            int c = cnt[t * E + e];
            cnt[t * E + e] = (unsigned short)run;
            run += c;
        }
        total[job] = run;
    }
    __syncthreads();
    for (int job = tid; job < E * 4; job += 256) {
        const int e = job >> 2, qtr = job & 3;
        int add = 0;
        for (int q = 0; q < qtr; q++) add += total[e * 4 + q];
        if (add) {
            const int t1 = min(T, (qtr + 1) * QT);
            for (int t = qtr * QT; t < t1; t++) cnt[t * E + e] = (unsigned short)(cnt[t * E + e] + add);
        }
    }
    __syncthreads();
    // per-group rows and tiles (groups: E routed experts, then n_shared shared)
    const int G = E + a.n_shared;
    if (tid < 64) {
        int run_rows = 0, run_tiles = 0;
        for (int g0 = 0; g0 < G; g0 += 64) {
            const int g = g0 + tid;
            int rows = 0;
            if (g < E) rows = total[g * 4] + total[g * 4 + 1] + total[g * 4 + 2] + total[g * 4 + 3];
            else if (g < G) rows = T;
            int tiles = (rows + a.BM - 1) / a.BM;
            // inclusive wave scans of rows (routed only) and tiles
            int sr = g < E ? rows : 0, st = tiles;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                int vr = __shfl_up(sr, o, 64), vt = __shfl_up(st, o, 64);
                if (tid >= o) { sr += vr; st += vt; }
            }
            if (g < G) {
                if (g < E) offset[g] = run_rows + sr - rows;
                tile0[g] = run_tiles + st - tiles;
            }
            run_rows += __shfl(sr, 63, 64);
            run_tiles += __shfl(st, 63, 64);
        }
        if (tid == 0) {
            offset[E] = run_rows;
            tile0[G] = run_tiles;
            *a.n_tiles = min(run_tiles, a.max_tiles);
        }
    }
    __syncthreads();
    for (int g = tid; g < G; g += 256) {
        const int rows = g < E ? offset[g + 1 < E ? g + 1 : E] - offset[g] : T;
        const int first = g < E ? offset[g] : T * k + (g - E) * T;
        for (int r0 = 0, ti = tile0[g]; r0 < rows; r0 += a.BM, ti++) {
            if (ti < a.max_tiles) {
                a.tiles[3 * ti] = g;
                a.tiles[3 * ti + 1] = first + r0;
                a.tiles[3 * ti + 2] = min(a.BM, rows - r0);
            }
        }
    }
    for (int t = tid; t < T; t += 256) {
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
