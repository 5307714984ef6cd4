// gemm_lds.h -- dense GEMMs with up to 256 activation rows on bf16 matrix
// cores, both operands staged in LDS by direct global -> LDS loads.
//
// A workgroup of RG x 4 waves owns a tile of RG*MR*32 activation rows x
// 128*NF weight rows (output columns; SwiGLU: 128 gate + the 128 matching up
// rows, 128 outputs).  Every reduction step of the tiled16 layout (SK elements) is
// one pipeline stage: the workgroup copies the step's 16 weight pieces (one
// 1 KiB piece per 16-row block, already in MFMA operand order) and its
// activation operands (64 lanes x 16 bytes each, gathered from the row-major
// activations in the order the matrix instruction reads them) straight into
// LDS, S stages deep; no register staging.  Wave (rg, cg) multiplies its MR
// activation fragments by its NF weight fragments (32x32x16 products, fp32
// accumulation) for every stage, so each weight byte is read from HBM once
// and each activation byte once per workgroup.
//
// Reduction mapping: as in gemm_wide_kernel -- operand (u, h) of lane l
// carries elements KL*(2u + l/32) + 8h .. +7 of the step, for the weight
// fragment (row l%32) and for the activation fragment (row l%32) alike.
//
// Used for the bf16 LM head at 65 .. 256 rows (batch 64: 136 -> 115 us per
// launch, same box; 128-row tiles up to 128 rows).  What bounds it is the copy into LDS, not the products:
// with the products skipped the same launch took 105 us (about 6.2 TB/s of
// operands moved into LDS, the 256 activation rows re-read for every
// 256-column tile); the fp8 LM head and the SwiGLU and K-split projections
// measured slower here than on gemm_wide_kernel and stay there.
#pragma once
#include "gemm.h"
#include "lds_dma.h"

template <int WT, int MODE, int RG, int MR, int S, int NF = 2>
__global__ __launch_bounds__(256 * RG) void gemm_lds_kernel(GemmArgs a)
{
    static_assert(WT == SV_BF16 || WT == SV_FP8, "bf16 or fp8 weights");
    static_assert(MODE != GM_SWIGLU || NF == 2, "SwiGLU tiles: 128 gate + 128 up columns");
    constexpr int CG = 4, WAVES = RG * CG;
    constexpr int WESZ = (WT == SV_FP8) ? 1 : 2;
    constexpr int KL = 16 / WESZ, SK = 4 * KL, XU = (WT == SV_FP8) ? 2 : 1;
    constexpr int BM = 32 * MR * RG;                 // activation rows per tile
    constexpr int WPC = 8 * NF;                      // weight pieces per stage (128 NF weight rows)
    constexpr int XPC = (BM / 32) * 2 * XU;          // activation operand pieces per stage
    constexpr int PPS = WPC + XPC;
    static_assert(PPS % WAVES == 0, "pieces per wave");
    constexpr int LPW = PPS / WAVES;                 // global -> LDS loads per wave per stage
    static_assert(LPW * (S - 1) < 64, "vmcnt range");
    __shared__ __align__(16) uint4 lds[S][PPS][64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, lh = lane >> 5;
    const int rg = wave / CG, cg = wave % CG;
    int mt, nt;
    if (!xcd_item(blockIdx.x, a.NT, a.MT, nt, mt)) return;
    const int row0 = mt * BM, nrows = min(BM, a.M - row0);
    if (nrows <= 0) return;
    const int K = a.K, kspan = K / a.ksplit, kb = blockIdx.y * kspan, nst = kspan / SK;
    const int nrb = a.N / 16;                        // 16-row weight blocks (SwiGLU: gate part)
    // output columns of the tile: 256 (store, argmax) or 128 gate columns (SwiGLU)
    constexpr int TN = (MODE == GM_SWIGLU) ? 128 : 128 * NF;
    const int n_tile0 = nt * TN;

    // this wave's global -> LDS loads: piece p = wave * LPW + i
    const char* src[LPW];
    bool wpiece[LPW];
#pragma unroll
    for (int i = 0; i < LPW; i++) {
        const int p = wave * LPW + i;
        if (p < WPC) {
            // weight block of piece p; blocks past the matrix read its last block
            int rb;
            if constexpr (MODE == GM_SWIGLU) rb = min(n_tile0 / 16 + (p & 7), nrb - 1) + (p >= 8 ? a.dual_off / 16 : 0);
            else rb = min(n_tile0 / 16 + p, nrb - 1);
            src[i] = (const char*)a.W + ((size_t)rb * (K / SK) + kb / SK) * 1024 + (size_t)lane * 16;
            wpiece[i] = true;
        } else {
            const int q = p - WPC, h = q % XU, u = (q / XU) % 2, m = q / (2 * XU);
            const int r = row0 + min(32 * m + l32, nrows - 1);
            src[i] = (const char*)a.X + ((size_t)r * a.ldx + kb + KL * (2 * u + lh) + 8 * h) * 2;
            wpiece[i] = false;
        }
    }
    auto issue = [&](int st) {   // stage st of this split into ring slot st % S
        const int buf = st % S;
#pragma unroll
        for (int i = 0; i < LPW; i++) {
            const int p = wave * LPW + i;
            const char* g = src[i] + (wpiece[i] ? (size_t)st * 1024 : (size_t)st * SK * 2);
            copy_to_lds(g, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4*)&lds[buf][p][0]);
        }
    };

    f32x16_t acc[MR][NF];
#pragma unroll
    for (int m = 0; m < MR; m++)
#pragma unroll
        for (int f = 0; f < NF; f++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[m][f][r] = 0.f;

    // weight fragment f of this wave: local 16-row blocks wb[f], wb[f] + 1
    int wb[NF];
#pragma unroll
    for (int f = 0; f < NF; f++) wb[f] = (MODE == GM_SWIGLU) ? 8 * f + 2 * cg : 2 * (cg * NF + f);

#pragma unroll
    for (int st = 0; st < S - 1; st++)
        if (st < nst) issue(st);
    for (int st = 0; st < nst; st++) {
        // this wave's loads of stage st are done once at most the later
        // stages' loads are outstanding; the barrier then covers every wave's
        // loads of stage st and every wave's reads of the slot refilled below
        const int later = min(S - 2, nst - 1 - st);
        if constexpr (S == 3) {
            if (later >= 1) wait_vmcnt<LPW>();
            else wait_vmcnt<0>();
        } else {
            if (later >= 2) wait_vmcnt<2 * LPW>();
            else if (later == 1) wait_vmcnt<LPW>();
            else wait_vmcnt<0>();
        }
        lds_barrier();
        if (st + S - 1 < nst) issue(st + S - 1);
        const uint4 (*buf)[64] = lds[st % S];
#pragma unroll
        for (int u = 0; u < 2; u++) {
            WOp<WT> wo[NF];
#pragma unroll
            for (int f = 0; f < NF; f++)
                wo[f] = wprep<WT>(buf[wb[f] + (l32 >> 4)][32 * u + 16 * lh + (l32 & 15)]);
#pragma unroll
            for (int h = 0; h < XU; h++)
#pragma unroll
                for (int m = 0; m < MR; m++) {
                    const uint4 xf = buf[WPC + (((rg * MR + m) * 2 + u) * XU) + h][lane];
#pragma unroll
                    for (int f = 0; f < NF; f++) acc[m][f] = mma32_bf16(wo[f].v[h], xf, acc[m][f]);
                }
        }
    }

    // epilogue: lane holds rows row0 + 32 (rg MR + m) + l32 and, per fragment,
    // output columns (fragment base) + 8 j + 4 lh + e in register 4 j + e
    const float* sc = a.ws;
    if constexpr (MODE == GM_STORE) {
        float* out = (float*)a.out + (size_t)blockIdx.y * a.split_stride;
#pragma unroll
        for (int f = 0; f < NF; f++) {
            const int nb = n_tile0 + 32 * (cg * NF + f);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int n = nb + 8 * j + 4 * lh;
                if (n >= a.N) continue;
                float s4[4] = {1.f, 1.f, 1.f, 1.f};
                if constexpr (WT == SV_FP8) {
#pragma unroll
                    for (int e = 0; e < 4; e++) s4[e] = sc[n + e];
                }
#pragma unroll
                for (int m = 0; m < MR; m++) {
                    const int r = 32 * (rg * MR + m) + l32;
                    if (r >= nrows) continue;
                    *reinterpret_cast<float4*>(out + (size_t)(row0 + r) * a.ldo + n) =
                        make_float4(acc[m][f][4 * j] * s4[0], acc[m][f][4 * j + 1] * s4[1],
                                    acc[m][f][4 * j + 2] * s4[2], acc[m][f][4 * j + 3] * s4[3]);
                }
            }
        }
    } else if constexpr (MODE == GM_SWIGLU) {
        const int nb = n_tile0 + 32 * cg;   // gate columns of this wave (fragment 0), up: fragment 1
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int n = nb + 8 * j + 4 * lh;
            if (n >= a.N) continue;
            float gs[4] = {1.f, 1.f, 1.f, 1.f}, us[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (WT == SV_FP8) {
#pragma unroll
                for (int e = 0; e < 4; e++) { gs[e] = sc[n + e]; us[e] = sc[a.dual_off + n + e]; }
            }
#pragma unroll
            for (int m = 0; m < MR; m++) {
                const int r = 32 * (rg * MR + m) + l32;
                if (r >= nrows) continue;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; e++)
                    v[e] = silu_f32(acc[m][0][4 * j + e] * gs[e]) * (acc[m][1][4 * j + e] * us[e]);
                *reinterpret_cast<uint2*>((uint16_t*)a.out + (size_t)(row0 + r) * a.ldo + n) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
        }
    } else {   // GM_ARGMAX: per row, the largest key over the tile's 256 columns
        __syncthreads();   // every wave is done with the staged operands
        unsigned long long* red = reinterpret_cast<unsigned long long*>(&lds[0][0][0]);
        static_assert(sizeof(lds) >= CG * BM * sizeof(unsigned long long), "reduction space");
#pragma unroll
        for (int m = 0; m < MR; m++) {
            const int r = 32 * (rg * MR + m) + l32;
            unsigned long long best = 0ull;
#pragma unroll
            for (int f = 0; f < NF; f++) {
                const int nb = n_tile0 + 32 * (cg * NF + f);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int n = nb + 8 * j + 4 * lh;
                    if (n >= a.N) continue;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        v[e] = acc[m][f][4 * j + e];
                        if constexpr (WT == SV_FP8) v[e] *= sc[n + e];
                        best = umax64(best, argmax_key(v[e], (uint32_t)(n + e)));
                    }
                    if (a.dbg && r < nrows)
                        *reinterpret_cast<float4*>(a.dbg + (size_t)(row0 + r) * a.dbg_ld + n) =
                            make_float4(v[0], v[1], v[2], v[3]);
                }
            }
            best = umax64(best, shfl_xor_u64(best, 32));
            if (lh == 0) red[cg * BM + r] = best;
        }
        __syncthreads();
        for (int r = tid; r < nrows; r += 64 * WAVES) {
            unsigned long long b = red[r];
#pragma unroll
            for (int c2 = 1; c2 < CG; c2++) b = umax64(b, red[c2 * BM + r]);
            a.keys[(size_t)nt * a.key_ld + row0 + r] = b;
        }
    }
}
