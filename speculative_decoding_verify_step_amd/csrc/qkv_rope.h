// qkv_rope.h -- the attention input of the verify step for few rows (the
// small-row path), in one kernel:
//   * first layer: the token block (committed token + drafts of every
//     sequence), embedding gather and RMSNorm, done in the prologue (each
//     workgroup normalises the rows it multiplies; the first column tile also
//     writes the residual stream and the per-sequence error flags);
//   * QKV = X W_qkv^T with MFMA -- a workgroup owns the column pair
//     (i, i + D/2) of 16 channels of one head and its W waves split the
//     reduction (wave 0 adds the others' partial sums in wave order);
//   * rotary on q and k (pair (i, i + D/2) turned by pos * theta^(-2i/D)), q to
//     the attention input, k and v appended to the caches at position ctx + j.
// The MFMA output layout puts channels i and i + D/2 of a row in the same lane,
// which is what makes the rotary a per-lane epilogue.
#pragma once
#include "common.h"
#include "gemm.h"
#include "small_kernels.h"

struct QkvArgs {
    const void* X;              // normalised rows [T][H] (layers after the first)
    const void* embed;          // [V][H] (first layer)
    const float* gain;          // attention-norm gain [H] (first layer)
    const int* committed;       // [B]
    const int* drafts;          // [B][K]
    const int* ctx_in;          // [B]
    int* seq_err;               // [B]: written by the first layer, read after
    unsigned* err_word;
    float* x_out;               // residual stream [T][H] (first layer)
    const void* W;              // W_qkv [(n_q + 2 n_kv) D][H]
    const float* ws;            // fp8 per-row scales
    const float2* rope;         // [cap][D/2] (cos, sin)
    void* q;                    // [T][n_q][D]
    void* kc;                   // K cache (tiled; a page pool when kvp.table is set)
    void* vc;                   // V cache (tiled)
    KvPages kvp;
    int V, cap, K1, T, H, n_q, n_kv, D, L, layer, MT, NT;
    float eps;
};

template <int WT, int MF, int W, int U, bool PACKED, bool EMBED>
__global__ __launch_bounds__(64 * W) void qkv_rope_kernel(QkvArgs a)
{
    using Tr = WTraits<WT>;
    constexpr int KL = Tr::KL, SK = Tr::SK, XU = Tr::XU, WESZ = Tr::ESZ;
    constexpr int AESZ = ATraits<WT>::ESZ;
    constexpr bool BF = WT != SV_F32;
    typedef typename Act<BF>::T AT;
    constexpr int BM = 16 * MF, NTH = 64 * W;
    constexpr int TPR = NTH / BM;                 // threads per row in the prologue
    static_assert(TPR >= 1 && TPR <= 64 && (64 % TPR) == 0, "prologue thread layout");
    __shared__ float rs[BM];                      // 1 / rms of each row
    __shared__ unsigned rflag[BM];                // error flags of each row's sequence
    __shared__ __align__(16) float gs[EMBED ? 8192 : 4];
    __shared__ f32x4_t part[W > 1 ? W - 1 : 1][MF][2][64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int id = blockIdx.x, xcd = id & 7, qd = id >> 3;
    const int mt = qd % a.MT, nt = (qd / a.MT) * 8 + xcd;
    if (nt >= a.NT) return;
    const int row0 = mt * BM, nrows = min(BM, a.T - row0);
    if (nrows <= 0) return;
    const int D = a.D, half = D >> 1, tpp = half >> 4;   // column-pair tiles per head
    const int hh = nt / tpp, a16 = nt % tpp;
    const int c0 = hh * D + 16 * a16;                     // first fragment; the second at c0 + half
    const int H = a.H, K1 = a.K1, K = K1 - 1;

    // this wave's reduction range (explicitly uniform: scalar loop bounds)
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int steps = H / SK;
    const int kb = wu * steps / W * SK, ke = (wu + 1) * steps / W * SK;

    const char* wrow[2];
#pragma unroll
    for (int f = 0; f < 2; f++) {
        const int n0 = c0 + f * half;
        if constexpr (PACKED) wrow[f] = (const char*)a.W + (size_t)(n0 >> 4) * H * 16 * WESZ + (size_t)lane * 16;
        else wrow[f] = (const char*)a.W + ((size_t)(n0 + l16) * H + (size_t)lg * KL) * WESZ;
    }
    uint4 wA[U][2], wB[U][2];
    auto wload = [&](int k, uint4 (&w)[U][2]) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int kk = k + u * SK;
            if (kk < ke) {
#pragma unroll
                for (int f = 0; f < 2; f++) {
                    if constexpr (PACKED) w[u][f] = ldg16_stream(wrow[f] + (size_t)(kk / SK) * 1024);
                    else w[u][f] = ldg16_stream(wrow[f] + (size_t)kk * WESZ);
                }
            }
        }
    };
    // the first weight stage is in flight during the prologue
    if (kb < ke) wload(kb, wA);

    // token of a row of this tile (invalid ids read embedding row 0)
    auto row_token = [&](int t) {
        const int b = t / K1, j = t % K1;
        const int tok = j == 0 ? a.committed[b] : a.drafts[(size_t)b * K + j - 1];
        return (tok < 0 || tok >= a.V) ? 0 : tok;
    };

    // activation rows of this lane (one per row fragment) and the epilogue
    // inputs: position and rotary (cos, sin) of each of the lane's rows for
    // channels i0 .. i0 + 3.  All of these loads, the embedding loads of the
    // normalisation pass and the first activation stage are issued before
    // anything waits, so the prologue costs two memory round trips (token,
    // embedding row) and one barrier.
    const char* xrow[MF];
    const int i0 = 16 * a16 + 4 * lg;
    const bool rot = hh < a.n_q + a.n_kv;
    int pos[MF], pin[MF], span[MF];
    size_t kvb[MF];             // cache block of the row's position (paged or contiguous)
    bool kv_bad = false;
    float4 csa[MF], csb[MF];
#pragma unroll
    for (int m = 0; m < MF; m++) {
        const int r = min(16 * m + l16, nrows - 1), t = row0 + r, b = t / K1, j = t % K1;
        if constexpr (EMBED) xrow[m] = (const char*)a.embed + ((size_t)row_token(t) * H + (size_t)lg * KL) * AESZ;
        else xrow[m] = (const char*)a.X + ((size_t)t * H + (size_t)lg * KL) * AESZ;
        pos[m] = min(max(a.ctx_in[b], 0), a.cap - K1) + j;
        kvb[m] = kv_block(a.kvp, b, a.L, a.layer, a.n_kv, a.cap, a.D, pos[m], pin[m], span[m], kv_bad);
        const float4* cp = reinterpret_cast<const float4*>(a.rope + (size_t)pos[m] * half + (rot ? i0 : 0));
        csa[m] = cp[0];
        csb[m] = cp[1];
    }
    if (kv_bad) atomicOr(a.err_word, SV_DEV_CAPACITY);   // a page index outside the pool
    float rsd[MF];   // 1 / rms of the lane's rows (first layer; set after the prologue)
#pragma unroll
    for (int m = 0; m < MF; m++) rsd[m] = 1.f;
    uint4 xA[U][MF][XU], xB[U][MF][XU];
    auto xload = [&](int k, uint4 (&x)[U][MF][XU]) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int kk = k + u * SK;
            if (kk < ke) {
#pragma unroll
                for (int m = 0; m < MF; m++)
#pragma unroll
                    for (int v = 0; v < XU; v++) x[u][m][v] = ldg16(xrow[m] + ((size_t)kk + 8 * v) * AESZ);
            }
        }
    };
    // first layer: x * (1/rms) * gain, rounded to the activation type, as the
    // separate normalisation would have stored it
    auto normed = [&](uint4 v, int k0, float r) -> uint4 {
        if constexpr (!EMBED) {
            return v;
        } else if constexpr (BF) {
            const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const float lo = bf16_bits_to_f32(wd[q] & 0xffffu) * r * gs[k0 + 2 * q];
                const float hi = bf16_bits_to_f32(wd[q] >> 16) * r * gs[k0 + 2 * q + 1];
                o[q] = pack_bf16x2(lo, hi);
            }
            return make_uint4(o[0], o[1], o[2], o[3]);
        } else {
            return make_uint4(__float_as_uint(__uint_as_float(v.x) * r * gs[k0]),
                              __float_as_uint(__uint_as_float(v.y) * r * gs[k0 + 1]),
                              __float_as_uint(__uint_as_float(v.z) * r * gs[k0 + 2]),
                              __float_as_uint(__uint_as_float(v.w) * r * gs[k0 + 3]));
        }
    };

    f32x4_t acc[MF][2];
#pragma unroll
    for (int m = 0; m < MF; m++)
#pragma unroll
        for (int f = 0; f < 2; f++) acc[m][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int k, uint4 (&w)[U][2], uint4 (&x)[U][MF][XU]) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int kk = k + u * SK;
            if (kk < ke) {
                uint4 xo[MF][XU];
#pragma unroll
                for (int m = 0; m < MF; m++)
#pragma unroll
                    for (int v = 0; v < XU; v++) xo[m][v] = normed(x[u][m][v], kk + lg * KL + 8 * v, rsd[m]);
#pragma unroll
                for (int f = 0; f < 2; f++) {
                    const WOp<WT> wo = wprep<WT>(w[u][f]);
#pragma unroll
                    for (int m = 0; m < MF; m++) acc[m][f] = mma_op<WT>(wo, xo[m], acc[m][f]);
                }
            }
        }
    };
    constexpr int STAGE = U * SK;
    if (kb < ke) xload(kb, xA);

    if constexpr (EMBED) {
        // per row r (TPR threads each): the sequence's validity (this thread's
        // share of its K1 tokens, and the context length), the sum of squares
        // over 16-byte slices in a fixed assignment, then butterflies inside
        // the TPR lanes; the gain is copied to shared memory meanwhile
        constexpr int EPC = 16 / AESZ, NB = 8, GPT = 8192 / NTH;
        const int r = tid / TPR, sl = tid % TPR;
        const bool rv = r < nrows;
        const int t = row0 + (rv ? r : 0), b = t / K1;
        unsigned e = 0u;
        if (sl == 0) {
            const int c = a.ctx_in[b];
            if (c < 0 || c + K1 > a.cap) e |= SV_DEV_CAPACITY;
        }
        for (int i = sl; i < K1; i += TPR) {
            const int ti = i == 0 ? a.committed[b] : a.drafts[(size_t)b * K + i - 1];
            if (ti < 0 || ti >= a.V) e |= SV_DEV_BAD_TOKEN;
        }
        float gv[GPT];
#pragma unroll
        for (int i = 0; i < GPT; i++) gv[i] = a.gain[min(tid + NTH * i, H - 1)];
        float ss = 0.f;
        if (rv) {
            const char* er = (const char*)a.embed + (size_t)row_token(t) * H * AESZ;
            float* xo = a.x_out + (size_t)t * H;
            for (int c00 = sl * EPC; c00 < H; c00 += TPR * EPC * NB) {
                uint4 v[NB];
#pragma unroll
                for (int u = 0; u < NB; u++) v[u] = ldg16(er + (size_t)min(c00 + u * TPR * EPC, H - EPC) * AESZ);
#pragma unroll
                for (int u = 0; u < NB; u++) {
                    const int c = c00 + u * TPR * EPC;
                    if (c >= H) break;
                    float f[8];
                    const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                    if constexpr (BF) {
#pragma unroll
                        for (int q = 0; q < 4; q++) { f[2 * q] = bf16_bits_to_f32(wd[q] & 0xffffu); f[2 * q + 1] = bf16_bits_to_f32(wd[q] >> 16); }
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; q++) f[q] = __uint_as_float(wd[q]);
                    }
#pragma unroll
                    for (int q = 0; q < EPC; q++) ss += f[q] * f[q];
                    if (nt == 0) {   // the residual stream, once per row
#pragma unroll
                        for (int q = 0; q < EPC; q += 4)
                            *reinterpret_cast<float4*>(xo + c + q) = make_float4(f[q], f[q + 1], f[q + 2], f[q + 3]);
                    }
                }
            }
        }
#pragma unroll
        for (int o = TPR / 2; o >= 1; o >>= 1) {
            ss += __shfl_xor(ss, o, 64);
            e |= (unsigned)__shfl_xor((int)e, o, 64);
        }
#pragma unroll
        for (int i = 0; i < GPT; i++)
            if (tid + NTH * i < H) gs[tid + NTH * i] = gv[i];
        if (rv && sl == 0) {
            rs[r] = rsqrtf(ss / (float)H + a.eps);
            rflag[r] = e;
            if (nt == 0 && t % K1 == 0) {   // the sequence's flags, once
                a.seq_err[b] = (int)e;
                if (e) atomicOr(a.err_word, e);
            }
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < MF; m++) rsd[m] = rs[min(16 * m + l16, nrows - 1)];
    }
    for (int k = kb; k < ke; k += 2 * STAGE) {
        if (k + STAGE < ke) { wload(k + STAGE, wB); xload(k + STAGE, xB); }
        compute(k, wA, xA);
        if (k + 2 * STAGE < ke) { wload(k + 2 * STAGE, wA); xload(k + 2 * STAGE, xA); }
        if (k + STAGE < ke) compute(k + STAGE, wB, xB);
    }

    // partial sums of waves 1.. through shared memory, added by wave 0 in wave order
    if (wave > 0) {
#pragma unroll
        for (int m = 0; m < MF; m++)
#pragma unroll
            for (int f = 0; f < 2; f++) part[wave - 1][m][f][lane] = acc[m][f];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < W - 1; w++)
#pragma unroll
        for (int m = 0; m < MF; m++)
#pragma unroll
            for (int f = 0; f < 2; f++) acc[m][f] += part[w][m][f][lane];

    // epilogue: channels i = i0 + e and i + D/2 of row 16 m + l16
    float s0[4] = {1.f, 1.f, 1.f, 1.f}, s1[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (WT == SV_FP8) {
#pragma unroll
        for (int e = 0; e < 4; e++) { s0[e] = a.ws[c0 + 4 * lg + e]; s1[e] = a.ws[c0 + half + 4 * lg + e]; }
    }
#pragma unroll
    for (int m = 0; m < MF; m++) {
        const int r = 16 * m + l16;
        if (r >= nrows) continue;
        const int t = row0 + r, b = t / K1;
        const bool write_cache = EMBED ? rflag[r] == 0u : a.seq_err[b] == 0;
        float x0[4], x1[4];
#pragma unroll
        for (int e = 0; e < 4; e++) { x0[e] = acc[m][0][e] * s0[e]; x1[e] = acc[m][1][e] * s1[e]; }
        if (rot) {
            const float cs[8] = {csa[m].x, csa[m].y, csa[m].z, csa[m].w, csb[m].x, csb[m].y, csb[m].z, csb[m].w};
            float r0[4], r1[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                r0[e] = x0[e] * cs[2 * e] - x1[e] * cs[2 * e + 1];
                r1[e] = x1[e] * cs[2 * e] + x0[e] * cs[2 * e + 1];
            }
            if (hh < a.n_q) {
                AT* qo = (AT*)a.q + ((size_t)t * a.n_q + hh) * D;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    Act<BF>::st(qo, i0 + e, r0[e]);
                    Act<BF>::st(qo, i0 + half + e, r1[e]);
                }
            } else if (write_cache) {
                const int kh = hh - a.n_q;
                AT* kp = (AT*)a.kc + kvb[m] + (size_t)kh * span[m] * D;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    Act<BF>::st(kp, k_cache_index<BF>(pin[m], i0 + e, D), r0[e]);
                    Act<BF>::st(kp, k_cache_index<BF>(pin[m], i0 + half + e, D), r1[e]);
                }
            }
        } else if (write_cache) {
            const int vh = hh - a.n_q - a.n_kv;
            AT* vp = (AT*)a.vc + kvb[m] + (size_t)vh * span[m] * D;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                Act<BF>::st(vp, v_cache_index<BF>(pin[m], i0 + e, D), x0[e]);
                Act<BF>::st(vp, v_cache_index<BF>(pin[m], i0 + half + e, D), x1[e]);
            }
        }
    }
}
