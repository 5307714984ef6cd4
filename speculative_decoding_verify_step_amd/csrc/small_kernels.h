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
    static SV_DEV float round(float v) { return bf16_bits_to_f32((uint16_t)f32_to_bf16_bits(v)); }
};
template <> struct Act<false> {
    typedef float T;
    static SV_DEV float ld(const T* p, size_t i) { return p[i]; }
    static SV_DEV void st(T* p, size_t i, float v) { p[i] = v; }
    static SV_DEV float round(float v) { return v; }
};

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

struct RowArgs {
    int H, K1, V, cap, E, topk, n_shared, T, nsplit;
    float eps;
    const int* committed;       // [B]
    const int* drafts;          // [B][K]
    const int* ctx_in;          // [B]
    int* seq_err;               // [B]
    unsigned* err_word;         // sticky
    const void* embed;          // [V][H]
    const float* x;             // [T][H] residual read
    float* x_out;               // [T][H] residual written (may equal x when one workgroup owns a row)
    void* h;                    // [T][H] normalised activations
    const float* gain;          // [H] gain of the norm that follows
    const float* parts;         // [nsplit][T][H] partial sums to add (or null)
    const float* y;             // MoE expert outputs [rows][H]
    const float* gate;          // [T][topk]
    const int* slot;            // [T][topk] expert-output row of (t, rank)
    float* dbg_hidden;          // optional [T][H] copy of x after the update
    // router after the attention half's norm: W_r [E][H] row-major
    const void* w_router;
    const float* s_router;      // fp8 per-row scales
    int wdtype;
    int renorm;
    int* sel;                   // [T][topk] out
    float* gate_out;            // [T][topk] out
    int* dbg_sel;               // optional copy of sel
    float* dbg_rlogits;         // optional [T][E] copy of the router logits (ROUTE)
    // the router's experts shared out over S workgroups per row
    int S;
    float* logits_g;            // [T][E] router logits (S > 1)
    // permutation (stable counting sort by expert) and expert tile list
    int BM, max_tiles;
    int* slot_out;              // [T][topk] row of (t, rank) in the permuted order
    int* perm_tok;              // [T*topk + n_shared*T] token of every permuted row
    int* tiles;                 // [max_tiles][3] = (group, first row, rows)
    int* n_tiles;               // [1]
    int implied;                // combine: slots implied by `sel` (few assignments, see implied_slot)
};

// token block + embedding gather + RMSNorm (one 1024-thread workgroup per
// row; a thread owns up to 8 columns and issues all of their loads -- embedding
// and gain -- before using any)
template <bool BF>
__global__ __launch_bounds__(1024) void embed_norm_kernel(RowArgs a)
{
    constexpr int RT = 1024, EPT = 8;      // H <= 8192
    __shared__ float shw[RT / 64];
    const int t = blockIdx.x, K1 = a.K1, K = K1 - 1, tid = threadIdx.x;
    const int b = t / K1, j = t % K1;
    int tok = (j == 0) ? a.committed[b] : a.drafts[(size_t)b * K + j - 1];
    if (j == 0 && tid < 64) {
        // one lane per token of the block (K1 <= 64), flags combined by a wave vote
        int ti = 0;
        if (tid < K1) ti = (tid == 0) ? a.committed[b] : a.drafts[(size_t)b * K + tid - 1];
        const int c = a.ctx_in[b];
        unsigned e = 0;
        if (__any(tid < K1 && (ti < 0 || ti >= a.V))) e |= SV_DEV_BAD_TOKEN;
        if (c < 0 || c + K1 > a.cap) e |= SV_DEV_CAPACITY;
        if (tid == 0) {
            a.seq_err[b] = (int)e;
            if (e) atomicOr(a.err_word, e);
        }
    }
    if (tok < 0 || tok >= a.V) tok = 0;
    const typename Act<BF>::T* er = (const typename Act<BF>::T*)a.embed + (size_t)tok * a.H;
    float v[EPT], g[EPT];
#pragma unroll
    for (int u = 0; u < EPT; u++) {
        const int i = min(tid + u * RT, a.H - 1);
        v[u] = Act<BF>::ld(er, i);
        g[u] = a.gain[i];
    }
#pragma unroll
    for (int u = 0; u < EPT; u++) v[u] = tid + u * RT < a.H ? v[u] : 0.f;
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < EPT; u++) {
        const int i = tid + u * RT;
        if (i < a.H) a.x_out[(size_t)t * a.H + i] = v[u];
        ss += v[u] * v[u];
    }
    ss = block_sum<RT>(ss, shw);
    const float r = rsqrtf(ss / (float)a.H + a.eps);
    typename Act<BF>::T* h = (typename Act<BF>::T*)a.h + (size_t)t * a.H;
#pragma unroll
    for (int u = 0; u < EPT; u++) {
        const int i = tid + u * RT;
        if (i < a.H) Act<BF>::st(h, i, v[u] * r * g[u]);
    }
}

// Loads that must be in flight together are written without conditions:
// indices are clamped into range and the unwanted values replaced afterwards.
// (A load inside a branch lets the compiler move its first use into the
// branch, which puts a wait on it before the next load issues.)
//
// n (<= NMAX) fp32 values `stride` apart into v[] (slots past n read as 0);
// p must be readable even when n == 0.
template <int NMAX>
SV_DEV void load_strided(const float* __restrict__ p, int n, size_t stride, float (&v)[NMAX])
{
    const int last = max(n, 1) - 1;
#pragma unroll
    for (int s = 0; s < NMAX; s++) v[s] = p[(size_t)min(s, last) * stride];
#pragma unroll
    for (int s = 0; s < NMAX; s++) v[s] = s < n ? v[s] : 0.f;
}

// fp32 at a wave-uniform base plus a 32-bit byte offset (one offset register
// serves every load that shares it; the base stays in scalar registers)
SV_DEV float ld_at(const float* base, unsigned byte_off)
{
    return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) + byte_off);
}

template <int NMAX>
SV_DEV float sum_in_order(const float (&v)[NMAX])
{
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < NMAX; s++) acc += v[s];
    return acc;
}

// Router weight slices of one pass: wave w, pass (e0, i00) covers experts
// e0 + 16 u (u < UPW, clamped below eend) and row chunks i00 + 64 EPL c (c < 4)
// of 16 bytes per lane.
SV_DEV int router_epl(int wdtype) { return wdtype == SV_F32 ? 4 : (wdtype == SV_BF16 ? 8 : 16); }

// e0 is wave-uniform; the row bases are formed as uniform pointers so that each
// load is (uniform base + 32-bit lane offset)
template <int UPW>
SV_DEV void router_loads(const RowArgs& a, int e0, int i00, int eend, uint4 (&wv)[4][UPW])
{
    const int EPL = router_epl(a.wdtype), esz = 16 / EPL;
    e0 = __builtin_amdgcn_readfirstlane(e0);
#pragma unroll
    for (int u = 0; u < UPW; u++) {
        const int e = min(e0 + u * 16, eend - 1);
        const char* row = (const char*)a.w_router + (size_t)e * a.H * esz;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            // columns past H re-read the row's last slice; the consumer skips them
            const unsigned i0 = (unsigned)min(i00 + c * 64 * EPL, a.H - EPL);
            wv[c][u] = ldg16(row + i0 * esz);
        }
    }
}

// Router logits r[e] = W_r[e] . h for experts [ebeg, eend) over the stored
// (activation-typed) row h in shared memory: the 16 waves take experts
// round-robin, UPW at a time; `wv` arrives holding the first pass's weight
// slices (loaded at kernel entry).  Results go to logit[e].
template <int UPW>
SV_DEV void router_logits(const RowArgs& a, const float* hs, uint4 (&wv)[4][UPW], int ebeg, int eend,
                          float* logit)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int H = a.H, EPL = router_epl(a.wdtype);
    bool first = true;
    for (int e0 = ebeg + w; e0 < eend; e0 += 16 * UPW) {
        float acc[UPW];
#pragma unroll
        for (int u = 0; u < UPW; u++) acc[u] = 0.f;
        for (int i00 = EPL * lane; i00 < H; i00 += 4 * 64 * EPL) {
            if (!first) router_loads<UPW>(a, e0, i00, eend, wv);   // later passes reuse the registers
            first = false;
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
                for (int u = 0; u < UPW; u++) {
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
        for (int u = 0; u < UPW; u++) {
            const int e = e0 + u * 16;
            const float v = wave_sum(acc[u]);
            if (e < eend && lane == 0) logit[e] = (a.wdtype == SV_FP8) ? v * a.s_router[e] : v;
        }
    }
}

// Selection of row t for the routing kernels (router_select_to).
SV_DEV void router_select(const RowArgs& a, int t, float (&p)[4], unsigned short* sel_lds = nullptr)
{
    router_select_to(a.E, a.topk, a.renorm != 0, t, p, a.sel, a.gate_out, a.dbg_sel, sel_lds);
}

// Router permutation over all T rows (the selections already in shared
// memory, `lds` layout below): a stable counting sort of the T*topk
// assignments by expert -- assignment (t, r) of expert e goes to offset[e] +
// (number of rows t' < t that also chose e) -- followed by the shared-expert
// rows (every token, in order), and the list of BM-row tiles per group for
// the grouped GEMMs.  Run by one workgroup, deterministic:
//   * each wave takes whole experts and ranks their tokens with a wave vote
//     over 64 tokens at a time (no serial scans);
//   * one wave scans the per-group row and tile counts; each group writes its tiles.
// `lds`: T (E + topk) 2 bytes (16-aligned) + 6.2 KB of shared memory.
SV_DEV unsigned short* perm_sel_lds(const RowArgs& a, char* lds)
{
    return reinterpret_cast<unsigned short*>(lds) + (size_t)a.T * a.E;
}

SV_DEV void permute_rows(const RowArgs& a, char* lds)
{
    const int T = a.T, E = a.E, k = a.topk, tid = threadIdx.x, NT = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, NW = NT >> 6;
    unsigned short* rank = reinterpret_cast<unsigned short*>(lds);   // [T][k] rank inside the expert
    unsigned short* sel = perm_sel_lds(a, lds);                       // [T][k], filled by the caller
    int* total = reinterpret_cast<int*>(lds + (((size_t)T * (E + k) * 2 + 15) & ~(size_t)15));   // [E]
    int* offset = total + 1024;                                       // [E + 1]
    int* tile0 = offset + 260;                                        // [E + n_shared + 1]
    // ranks: wave w takes experts w, w + NW, ...; a token chooses an expert
    // at most once, so the rank of (t, e) is the number of tokens before t
    // that chose e: a wave vote over 64 tokens at a time
    for (int e = wave; e < E; e += NW) {
        int run = 0;
        for (int t0 = 0; t0 < T; t0 += 64) {
            const int t = t0 + lane;
            int rsel = -1;
            if (t < T)
                for (int r = 0; r < k; r++)
                    if (sel[t * k + r] == e) rsel = r;
            const unsigned long long m = __ballot(rsel >= 0);
            if (rsel >= 0) rank[t * k + rsel] = (unsigned short)(run + __popcll(m & ((1ull << lane) - 1ull)));
            run += __popcll(m);
        }
        if (lane == 0) total[e] = run;
    }
    __syncthreads();
    // per-group rows and tiles (groups: E routed experts, then n_shared shared)
    const int G = E + a.n_shared;
    if (tid < 64) {
        int run_rows = 0, run_tiles = 0;
        for (int g0 = 0; g0 < G; g0 += 64) {
            const int g = g0 + tid;
            int rows = 0;
            if (g < E) rows = total[g];
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
    for (int g = tid; g < G; g += NT) {
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
    for (int i = tid; i < T * k; i += NT) {
        const int sl = offset[sel[i]] + rank[i];
        a.slot_out[i] = sl;
        a.perm_tok[sl] = i / k;
    }
    for (int i = tid; i < a.n_shared * T; i += NT) a.perm_tok[T * k + i] = i % T;
}

// x_out = x + (sum of K-split partials) or x + (sum over ranks of gate * expert
// output + shared-expert outputs); then RMSNorm into h.  One 1024-thread
// workgroup per row; a thread owns up to two columns per pass and issues every
// load of the pass -- residual, gain and all splits (or ranks and shared
// experts) of both columns -- before consuming any, so a pass costs one memory
// round trip.  ROUTE (MoE, after attention): S workgroups per row each
// recompute the update and the norm (workgroup 0 writes them) and take E/S of
// the router's experts; with S > 1 they write the logits for the selection in
// route_finish_kernel, with S = 1 the row selects its experts here.  NSP
// bounds the K-splits (or, MoE, the shared experts, at most 8) that a column
// loads: the launch picks the smallest power of two that covers them, so
// that no load repeats a partial.
template <bool BF, bool MOE, bool ROUTE = false, int UPW = 4, int NSP = 16>
__global__ __launch_bounds__(1024) void residual_norm_kernel(RowArgs a)
{
    constexpr int RT = 1024, EPT = 2, NS = ROUTE ? 4 : NSP, NSH = NSP < 8 ? NSP : 8;
    __shared__ __align__(16) float smem[2 * 8192];   // row update, gains
    __shared__ float shw[RT / 64];
    __shared__ float logit[256];
    float* xs = smem;
    float* gs = smem + 8192;
    const int t = blockIdx.x, H = a.H, T = a.T, tid = threadIdx.x;
    const int sidx = ROUTE ? blockIdx.y : 0;
    const bool writer = sidx == 0;
    const float* xr = a.x + (size_t)t * H;
    float* xo = a.x_out + (size_t)t * H;
    const float* __restrict__ y = a.y;
    int slot[8];
    float gate[8];
    if constexpr (MOE) {
        if (a.implied) {
            const int A = T * a.topk;
            const int sv = min(max(a.sel[min(tid & 63, A - 1)], 0), a.E - 1);
#pragma unroll
            for (int r = 0; r < 8; r++) slot[r] = implied_slot(sv, A, t * a.topk + min(r, a.topk - 1));
        } else {
#pragma unroll
            for (int r = 0; r < 8; r++) slot[r] = a.slot[t * a.topk + min(r, a.topk - 1)];
        }
#pragma unroll
        for (int r = 0; r < 8; r++) gate[r] = a.gate[t * a.topk + min(r, a.topk - 1)];
#pragma unroll
        for (int r = 0; r < 8; r++) gate[r] = r < a.topk ? gate[r] : 0.f;
    }
    // uniform row bases; every load below is (uniform base + 32-bit byte offset)
    const float* __restrict__ prow = a.parts + (size_t)t * H;
    const size_t pstride = (size_t)T * H;
    const float* __restrict__ shrow =
        (MOE && a.n_shared > 0) ? y + ((size_t)T * a.topk + t) * H : y;
    const int nlast = MOE ? max(a.n_shared, 1) - 1 : max(a.nsplit, 1) - 1;
    float xv[EPT], gv[EPT], pv[EPT][MOE ? 8 + NSH : NS];
    auto loads = [&](int i0) {
#pragma unroll
        for (int u = 0; u < EPT; u++) {
            const unsigned off = 4u * (unsigned)min(i0 + u * RT, H - 1);
            xv[u] = ld_at(xr, off);
            gv[u] = ld_at(a.gain, off);
            if constexpr (MOE) {
#pragma unroll
                for (int r = 0; r < 8; r++) pv[u][r] = ld_at(y + (size_t)slot[r] * H, off);
#pragma unroll
                for (int sx = 0; sx < NSH; sx++)
                    pv[u][8 + sx] = ld_at(shrow + (size_t)min(sx, nlast) * pstride, off);
            } else {
#pragma unroll
                for (int sp = 0; sp < NS; sp++) pv[u][sp] = ld_at(prow + (size_t)min(sp, nlast) * pstride, off);
            }
        }
    };
    float ss = 0.f;
    auto consume = [&](int i0) {
#pragma unroll
        for (int u = 0; u < EPT; u++) {
            const int i = i0 + u * RT;
            float d = 0.f;
            if constexpr (MOE) {     // clamped re-reads are dropped here
#pragma unroll
                for (int r = 0; r < 8; r++) d += gate[r] * (r < a.topk ? pv[u][r] : 0.f);
                float sh = 0.f;
#pragma unroll
                for (int sx = 0; sx < NSH; sx++) sh += sx < a.n_shared ? pv[u][8 + sx] : 0.f;
                d += sh;
            } else {
#pragma unroll
                for (int sp = 0; sp < NS; sp++) d += sp < a.nsplit ? pv[u][sp] : 0.f;
            }
            if (i >= H) continue;
            const float v = xv[u] + d;
            if (writer) {
                xo[i] = v;
                if (a.dbg_hidden) a.dbg_hidden[(size_t)t * H + i] = v;
            }
            xs[i] = v;
            gs[i] = gv[u];
            ss += v * v;
        }
    };
    // first pass: its loads, then the router's first weight slices (still in
    // flight while the residual is summed and normalised), then the rest
    const int EP = ROUTE ? a.E / a.S : 0, ebeg = sidx * EP, eend = ebeg + EP;
    loads(tid);
    uint4 wv[4][UPW];
    if constexpr (ROUTE) router_loads<UPW>(a, ebeg + (tid >> 6), router_epl(a.wdtype) * (tid & 63), eend, wv);
    consume(tid);
    for (int i0 = tid + EPT * RT; i0 < H; i0 += EPT * RT) {
        loads(i0);
        consume(i0);
    }
    ss = block_sum<RT>(ss, shw);
    const float r = rsqrtf(ss / (float)H + a.eps);
    typename Act<BF>::T* h = (typename Act<BF>::T*)a.h + (size_t)t * H;
    for (int i = tid; i < H; i += RT) {   // each thread rereads only the columns it wrote
        float v = xs[i] * r * gs[i];
        if (writer) Act<BF>::st(h, i, v);
        if constexpr (ROUTE) xs[i] = Act<BF>::round(v);   // the value the experts will read
    }
    if constexpr (ROUTE) {
        __syncthreads();
        router_logits<UPW>(a, xs, wv, ebeg, eend, logit);
        __syncthreads();
        if (a.dbg_rlogits && tid >= 64 && tid - 64 < eend - ebeg)
            a.dbg_rlogits[(size_t)t * a.E + ebeg + tid - 64] = logit[ebeg + tid - 64];
        if (tid < 64) {
            const int lane = tid, E = a.E;
            if (a.S > 1) {
                // this workgroup's share of the row's logits; selection follows
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int e = lane + 64 * q;
                    if (e >= ebeg && e < eend) a.logits_g[(size_t)t * E + e] = logit[e];
                }
            } else {
                float p[4];
#pragma unroll
                for (int q = 0; q < 4; q++)
                    p[q] = lane + 64 * q < E ? logit[min(lane + 64 * q, E - 1)] : -INFINITY;
                // the row buffer is free after the logits: wave 0's key scratch
                router_select(a, t, p);
            }
        }
    }
}

// Permutation for few assignments (T*topk <= 64, T <= BM: every expert's rows
// fit one tile), by one wave without barriers; the same result as
// permute_rows.  Lane i holds assignment i = (t = i / k, rank): its expert's
// offset is the number of assignments with a lower expert, its rank inside the
// expert the number of earlier assignments with the same expert (row order);
// the expert's tile index is the number of distinct lower experts (a bitmask
// of the experts present).  The assignments are read from shared memory four
// at a time (register compares, no cross-lane round trips).
SV_DEV void permute_rows_wave(const RowArgs& a, const unsigned short* sel, unsigned* mask)
{
    const int lane = threadIdx.x & 63, T = a.T, k = a.topk, A = T * k;
    if (lane < 8) mask[lane] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const bool act = lane < A;
    const int e = act ? sel[lane] : 0x7fffffff;
    if (act) atomicOr(&mask[e >> 5], 1u << (e & 31));
    int off = 0, rank = 0, cnt = 0;
#pragma unroll 4
    for (int j0 = 0; j0 < A; j0 += 4) {
        const uint2 q = *reinterpret_cast<const uint2*>(sel + j0);
        const int ej[4] = {(int)(q.x & 0xffffu), (int)(q.x >> 16), (int)(q.y & 0xffffu), (int)(q.y >> 16)};
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int j = j0 + u;
            if (j < A) {
                off += ej[u] < e;
                rank += (ej[u] == e) & (j < lane);
                cnt += ej[u] == e;
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const bool first = act && rank == 0;
    int tile = 0, distinct = 0;
#pragma unroll
    for (int w = 0; w < 8; w++) {
        const unsigned mw = mask[w];
        distinct += __popc(mw);
        if (act) tile += w < (e >> 5) ? __popc(mw) : (w == (e >> 5) ? __popc(mw & ((1u << (e & 31)) - 1u)) : 0);
    }
    if (act) {
        const int slot = off + rank;
        a.slot_out[lane] = slot;
        a.perm_tok[slot] = lane / k;
    }
    if (first && tile < a.max_tiles) {
        a.tiles[3 * tile] = e;
        a.tiles[3 * tile + 1] = off;
        a.tiles[3 * tile + 2] = cnt;
    }
    // shared experts: every token, one tile each (T <= BM)
    for (int i = lane; i < a.n_shared * T; i += 64) a.perm_tok[A + i] = i % T;
    if (lane < a.n_shared) {
        const int ti = distinct + lane;
        if (ti < a.max_tiles) {
            a.tiles[3 * ti] = a.E + lane;
            a.tiles[3 * ti + 1] = A + lane * T;
            a.tiles[3 * ti + 2] = T;
        }
    }
    if (lane == 0) *a.n_tiles = min(distinct + a.n_shared, a.max_tiles);
}

// Routing, second half (one 1024-thread workgroup): when the router was
// shared out (S > 1), each wave selects the experts of rows w, w + 16, ...
// from the published logits; otherwise the rows' selections are read back.
// Then the permutation and tile list of every row (by one wave when the
// assignments are few), unless the consumers derive them from the selections.
__global__ __launch_bounds__(1024) void route_finish_kernel(RowArgs a)
{
    __shared__ __align__(16) char lds[81920];
    const int T = a.T, E = a.E, k = a.topk, tid = threadIdx.x, lane = tid & 63;
    unsigned short* sel = perm_sel_lds(a, lds);
    if (a.S > 1) {
        for (int row = tid >> 6; row < T; row += 16) {
            float p[4];
#pragma unroll
            for (int q = 0; q < 4; q++) p[q] = a.logits_g[(size_t)row * E + min(lane + 64 * q, E - 1)];
#pragma unroll
            for (int q = 0; q < 4; q++) p[q] = lane + 64 * q < E ? p[q] : -INFINITY;
            router_select(a, row, p, sel);
        }
    } else {
        for (int i = tid; i < T * k; i += 1024) sel[i] = (unsigned short)a.sel[i];
    }
    if (a.implied) return;   // the consumers derive tiles and slots from the selections
    __syncthreads();
    if (T * k <= 64 && T <= a.BM) {
        // the mask lives in the space permute_rows would use for its totals
        unsigned* mask = reinterpret_cast<unsigned*>(lds + (((size_t)T * (E + k) * 2 + 15) & ~(size_t)15));
        if (tid < 64) permute_rows_wave(a, sel, mask);
        return;
    }
    permute_rows(a, lds);
}

struct RopeArgs {
    const float* qkv;           // [nsplit][T][(n_q + 2 n_kv) D] partial sums
    int nsplit, T, K1, n_q, n_kv, D, L, layer, cap;
    const int* ctx_in;
    const int* seq_err;
    const float2* rope;         // [cap][D/2] (cos, sin)
    void* q;                    // [T][n_q][D] act
    void* kc;                   // K cache (a page pool when kvp.table is set)
    void* vc;                   // V cache
    KvPages kvp;
    unsigned* err_word;
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
// wave per (row, head); grid (T, n_q + 2 n_kv).  A lane owns one rotary pair
// (q, k heads) or two channels (v heads) and issues the loads of every K-split
// partial of them at once (NS >= nsplit loads per channel: the launch picks
// the smallest power of two, so that no load repeats a partial); the rotary
// table read waits only for ctx.
template <bool BF, int NS>
__global__ __launch_bounds__(64) void rope_append_kernel(RopeArgs a)
{
    const int t = blockIdx.x, hh = blockIdx.y, lane = threadIdx.x;
    const int K1 = a.K1, D = a.D, half = D / 2;     // D in {64, 128}: half <= 64
    const int b = t / K1, j = t % K1;
    const int QKV = (a.n_q + 2 * a.n_kv) * D;
    typedef typename Act<BF>::T AT;
    const float* __restrict__ src = a.qkv + (size_t)t * QKV + (size_t)hh * D;
    const size_t sstride = (size_t)a.T * QKV;
    float p0[NS], p1[NS];
    const bool rot = hh < a.n_q + a.n_kv;
    // rotary heads: channels lane and lane + half; value heads: lane and lane + 64
    const int i0 = lane, i1 = rot ? lane + half : lane + 64;
    const bool ok0 = rot ? lane < half : lane < D, ok1 = rot ? lane < half : lane + 64 < D;
    load_strided<NS>(src + (ok0 ? i0 : 0), ok0 ? a.nsplit : 0, sstride, p0);
    load_strided<NS>(src + (ok1 ? i1 : 0), ok1 ? a.nsplit : 0, sstride, p1);
    const int ctx = a.ctx_in[b];
    const bool write_cache = a.seq_err[b] == 0;
    const int pos = min(max(ctx, 0), a.cap - K1) + j;
    int pin, span;
    bool kv_bad = false;
    const size_t kvb = kv_block(a.kvp, b, a.L, a.layer, a.n_kv, a.cap, D, pos, pin, span, kv_bad);
    if (kv_bad && lane == 0 && write_cache) atomicOr(a.err_word, SV_DEV_CAPACITY);
    const float x0 = sum_in_order(p0), x1 = sum_in_order(p1);
    if (rot) {
        if (!ok0) return;
        const float2 cs = a.rope[(size_t)pos * half + lane];
        const float r0 = x0 * cs.x - x1 * cs.y;
        const float r1 = x1 * cs.x + x0 * cs.y;
        if (hh < a.n_q) {
            AT* qo = (AT*)a.q + ((size_t)t * a.n_q + hh) * D;
            Act<BF>::st(qo, lane, r0);
            Act<BF>::st(qo, lane + half, r1);
        } else if (write_cache) {
            const int kh = hh - a.n_q;
            AT* kp = (AT*)a.kc + kvb + (size_t)kh * span * D;
            Act<BF>::st(kp, k_cache_index<BF>(pin, lane, D), r0);
            Act<BF>::st(kp, k_cache_index<BF>(pin, lane + half, D), r1);
        }
    } else if (write_cache) {
        const int vh = hh - a.n_q - a.n_kv;
        AT* vp = (AT*)a.vc + kvb + (size_t)vh * span * D;
        if (ok0) Act<BF>::st(vp, v_cache_index<BF>(pin, i0, D), x0);
        if (ok1) Act<BF>::st(vp, v_cache_index<BF>(pin, i1, D), x1);
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
// context length.  One 1024-thread workgroup per sequence: the 16 waves are
// shared out over the K+1 positions (WPP waves per position when K+1 <= 16,
// else positions round-robin), every lane keeps 16 key loads in flight, and
// the drafts are staged in shared memory alongside; the first mismatch is
// found with a wave vote.
__global__ __launch_bounds__(1024) void accept_kernel(AcceptArgs a)
{
    constexpr int NW = 16, KB = 16;
    __shared__ unsigned long long part[64][NW];     // [position][wave part], K1 <= 64
    __shared__ int dr[64];
    __shared__ int g[64];
    const int b = blockIdx.x, K1 = a.K1, K = K1 - 1, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    // this sequence's drafts: loaded now, stored to shared memory after the key loads
    const int dv = a.drafts[(size_t)b * K + min(tid, K - 1)];
    const int WPP = K1 >= NW ? 1 : NW / K1;          // waves per position
    const int NG = NW / WPP;                         // position groups
    const int gi = w / WPP, pi = w % WPP;
    if (gi < NG) {
        for (int j = gi; j < K1; j += NG) {
            const unsigned long long* __restrict__ kp = a.keys + (size_t)b * K1 + j;
            unsigned long long best = 0ull;
            for (int n0 = pi * 64 + lane; n0 < a.NT; n0 += KB * 64 * WPP) {
                unsigned long long v[KB];
#pragma unroll
                for (int u = 0; u < KB; u++) {   // clamped: a repeated key leaves the maximum
                    const int n = min(n0 + u * 64 * WPP, a.NT - 1);
                    v[u] = kp[(size_t)n * a.T];
                }
#pragma unroll
                for (int u = 0; u < KB; u++) best = umax64(best, v[u]);
            }
            best = wave_max_u64(best);
            if (lane == 0) part[j][pi] = best;
        }
    }
    if (tid < K) dr[tid] = dv;
    __syncthreads();
    if (w != 0) return;
    // wave 0: lane j < K1 finishes position j
    unsigned long long best = 0ull;
    if (lane < K1)
        for (int p = 0; p < WPP; p++) best = umax64(best, part[lane][p]);
    const bool nan_here = lane < K1 && best == ~0ull;
    const int gj = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
    if (lane < K1) g[lane] = gj;
    const bool nan_any = __any(nan_here);
    const unsigned long long miss = __ballot(lane < K && dr[lane] != gj);
    const int n = miss ? (__ffsll((long long)miss) - 1) : K;
    const int gn = __shfl(gj, n, 64);
    if (a.target && lane < K1) a.target[(size_t)b * K1 + lane] = gj;
    if (lane == 0) {
        unsigned e = a.seq_err ? (unsigned)a.seq_err[b] : 0u;
        if (nan_any) e |= SV_DEV_NAN_LOGIT;
        const int c = a.ctx_in[b];
        if (e) {
            if (a.seq_err == nullptr || nan_any) atomicOr(a.err_word, e);
            a.accepted[b] = -1;
            a.next_tok[b] = -1;
            a.ctx_out[b] = c;
        } else {
            a.accepted[b] = n;
            a.next_tok[b] = gn;
            a.ctx_out[b] = c + n + 1;
        }
    }
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
    best = wave_max_u64(best);
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

// MXFP4 block scales, row-major [rows][cols/32] bytes -> the tiled form the
// GEMM kernels read: per 16-row block and group of 16 reduction steps (128
// columns each), 64 lanes x 16 bytes, lane l = r + 16 g holding the scales of
// row r, column blocks 4 s + g for the group's steps s (one 16-byte load per
// lane covers 16 steps).  Bytes past the row's blocks and rows past `rows`
// are written as 127 (scale 1).  One thread per 16-byte lane slice.
__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint8_t* __restrict__ src,
                                                             uint8_t* __restrict__ dst, long rows,
                                                             int cols)
{
    const int nb = cols / 32, steps = cols / 128, nchunk = (steps + 15) / 16;
    const long nblk = (rows + 15) / 16;
    const long total = nblk * nchunk * 64;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int l = (int)(i & 63);
        const long bc = i >> 6;             // block * nchunk + chunk
        const long rb = bc / nchunk;
        const int c = (int)(bc % nchunk);
        const long row = rb * 16 + (l & 15);
        const int g = l >> 4;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            uint32_t v = 0;
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const int st = 16 * c + 4 * q + b, blk = 4 * st + g;
                const uint32_t byte = (row < rows && st < steps) ? src[row * nb + blk] : 127u;
                v |= byte << (8 * b);
            }
            w[q] = v;
        }
        *reinterpret_cast<uint4*>(dst + i * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}
