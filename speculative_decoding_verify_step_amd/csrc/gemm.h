// gemm.h -- weight-streaming MFMA GEMM for the verify step:
//   Y[m][n] = sum_k X[m][k] * W[n][k]     (W row-major [N][K], one row per output)
// with the epilogue chosen at compile time:
//   GM_STORE   fp32 partial sums (one slab per K split) for a consumer kernel
//   GM_SWIGLU  gate rows n and up rows n + dual_off in the same wave; writes
//              silu(gate) * up in the activation type
//   GM_ARGMAX  per-row (value, index) maximum over the workgroup's columns as
//              an order-preserving 64-bit key, plus optional fp32 logits
//
// Shapes on the verify path are "few rows, many weights": M = B (K+1) rows of
// activations (4 .. 256) against weight matrices of 0.2 - 390 MB, so the
// kernel streams each weight element from HBM once and keeps the activations
// in cache.  Operand roles: the weight fragment is the MFMA A operand (16
// output columns), the activation fragment is the B operand (16 rows); a wave
// owns 16*NF output columns and 16*MF rows, and four waves side by side make
// a 64*NF-column workgroup tile.  Every lane loads 16 contiguous bytes of a
// weight row per step (the 16 rows of a fragment are 16 separate 64-byte
// runs, and consecutive steps walk along the rows).
//
// Grouped mode (mixture of experts): a device-built tile list names, per
// grid row, (group, first row, row count) over the permuted assignment rows;
// the group selects the expert's weights (groups >= G1 use the second weight
// set: shared experts), and `gather` maps a permuted row to its token's
// activation row.  The grid is sized for the largest possible list and
// workgroups past the device-side count exit at once (graph-safe, no host
// round trip).
//
// Launch mapping is XCD-aware: workgroup ids are dealt to the 8 XCDs round
// robin, so the tiles that share one weight slab (same column tile, different
// row tiles) are given ids 8 apart and land on the same XCD's L2.
#pragma once
#include "common.h"

enum { GM_STORE = 0, GM_SWIGLU = 1, GM_ARGMAX = 2 };

struct GemmArgs {
    const void* X;          // activations [rows][ldx] (fp32 or bf16)
    long ldx;
    const int* gather;      // grouped: permuted row -> activation row (or null)
    int M;                  // dense: rows
    int N;                  // output columns, a multiple of 4 (SWIGLU: columns of gate = of up)
    int K;                  // full reduction length
    int ksplit;             // K splits (grid.y); K / ksplit is a multiple of the step
    const void* W;          // weights of groups 0 .. G1-1
    const float* ws;        // fp8 per-row scales of W
    long w_gstride;         // elements between groups of W
    long s_gstride;         // scales between groups
    const void* W2;         // weights of groups G1 ..
    const float* ws2;
    long w2_gstride, s2_gstride;
    int G1;
    int dual_off;           // SWIGLU: row offset of the "up" rows
    const int* tiles;       // grouped: [max_tiles][3] = (group, row0, nrows); null = dense
    const int* n_tiles;     // grouped: device count of valid tiles
    const int* sel;         // grouped, few rows: tiles implied by the selections [T][topk]
                            // (then tiles/n_tiles/gather are unused; see implied_tile)
    int sel_T, sel_k, sel_E, sel_S;
    // selections made here (SwiGLU): with sel_logits set (router logits
    // [T][E], T <= 4, E <= 64) every workgroup selects the experts itself
    // (router_select_to) instead of reading `sel`, and workgroup 0 publishes
    // them for the kernels that follow (sel_out, gate_out, dbg_sel_out: [T][topk])
    const float* sel_logits;
    int sel_renorm;
    int* sel_out;
    float* gate_out;
    int* dbg_sel_out;
    int MT;                 // row tiles in the grid (dense: ceil(M / BM); grouped: max tiles)
    int NT;                 // column tiles (16*NF*WAVES columns each)
    void* out;              // STORE: fp32 [ksplit][rows][ldo]; SWIGLU: act [rows][ldo]
    long ldo;
    long split_stride;      // STORE: elements between K-split slabs
    unsigned long long* keys;   // ARGMAX: [NT][key_ld]
    long key_ld;
    float* dbg;             // ARGMAX: optional fp32 logits [rows][dbg_ld]
    long dbg_ld;
};

// Whether the group (expert) of tile mt of a device-built tile list has other
// row tiles (its tiles are consecutive in the list): those tiles read the
// same weights, so the loads keep them in L2 for the others instead of
// streaming them past it.
SV_DEV bool group_has_siblings(const int* tiles, int mt, int ntiles, int group)
{
    const int prev = tiles[3 * max(mt - 1, 0)];
    const int next = tiles[3 * min(mt + 1, ntiles - 1)];
    return (mt > 0 && prev == group) || (mt + 1 < ntiles && next == group);
}

// Work item (column tile nt, row tile mt) of workgroup `id` among NT x MT
// items, row tiles fastest.  Workgroup ids are dealt to the 8 XCDs round
// robin; each XCD takes one contiguous range of equal length of the items, so
// every XCD streams the same share of the weights (with column tiles dealt
// out by id modulo 8, NT = 14 gave six XCDs two slabs and two XCDs one), and
// the row tiles of one column slab stay together on one XCD's L2.  False for
// a workgroup past the items (the grid is sized for an upper bound).
SV_DEV bool xcd_item(int id, int NT, int MT, int& nt, int& mt)
{
    const int x = id & 7, q = id >> 3, total = NT * MT, per = (total + 7) >> 3, u = x * per + q;
    if (q >= per || u >= total) return false;
    nt = u / MT;
    mt = u % MT;
    return true;
}

// per weight storage type: elements per 16-byte lane slice, reduction step
template <int WT> struct WTraits;
template <> struct WTraits<SV_F32> { static constexpr int KL = 4, SK = 16, XU = 1, ESZ = 4; };
template <> struct WTraits<SV_BF16> { static constexpr int KL = 8, SK = 32, XU = 1, ESZ = 2; };
template <> struct WTraits<SV_FP8> { static constexpr int KL = 16, SK = 64, XU = 2, ESZ = 1; };
// MXFP4 (tiled16 layout only): 32 E2M1 codes per 16-byte lane slice, one E8M0
// scale byte per slice (tiled scales: 16 steps per 16-byte lane slice, K <=
// 2048); ESZ is not used (a code is half a byte)
template <> struct WTraits<SV_MXFP4> { static constexpr int KL = 32, SK = 128, XU = 4, ESZ = 1; };

// weight element size in half-bytes (byte offsets of packed 4-bit codes)
template <int WT> constexpr int w_half_bytes() { return WT == SV_F32 ? 8 : (WT == SV_BF16 ? 4 : (WT == SV_FP8 ? 2 : 1)); }

// activation element size: fp32 with fp32 weights, bf16 otherwise
template <int WT> struct ATraits { static constexpr int ESZ = (WT == SV_F32) ? 4 : 2; };

// A weight slice in MFMA operand form: one 16-byte operand (fp32, bf16) or
// two bf16 operands widened from 16 e4m3 codes (fp8) -- converted once per
// fragment and reused for every row fragment.
template <int WT> struct WOp { uint4 v[WT == SV_FP8 ? 2 : (WT == SV_MXFP4 ? 4 : 1)]; };

// E8M0 scale byte -> 2^(s - 127) (0 -> 2^-127, a subnormal; 0xFF -> NaN)
SV_DEV float e8m0_to_f32(uint32_t s)
{
    return s == 0u ? __uint_as_float(0x00400000u)
                   : (s == 255u ? __uint_as_float(0x7fc00000u) : __uint_as_float(s << 23));
}

// 8 E2M1 codes (one 32-bit word, element 2i in the low half of byte i) times
// the block scale -> 8 bf16 in MFMA operand order: gfx950 converts two codes
// per instruction, exactly (a code times a power of two is a bf16 value)
SV_DEV uint4 e2m1x8_to_bf16(uint32_t w, float s)
{
    return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3)));
}

// MXFP4 scale of reduction step st (< 16) from a lane's tiled 16-byte scale
// slice (byte st: the block of the lane's 32 codes at that step)
SV_DEV uint32_t mx_scale_byte(uint4 v, int st)
{
    const int q = st >> 2;
    const uint32_t w = q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
    return (w >> (8 * (st & 3))) & 0xffu;
}

// a 16-byte MXFP4 lane slice (32 codes, one block) -> four bf16 operands
SV_DEV WOp<SV_MXFP4> wprep_mx(uint4 w, uint32_t sb)
{
    const float s = e8m0_to_f32(sb);
    WOp<SV_MXFP4> o;
    o.v[0] = e2m1x8_to_bf16(w.x, s);
    o.v[1] = e2m1x8_to_bf16(w.y, s);
    o.v[2] = e2m1x8_to_bf16(w.z, s);
    o.v[3] = e2m1x8_to_bf16(w.w, s);
    return o;
}

template <int WT>
SV_DEV WOp<WT> wprep(uint4 w)
{
    WOp<WT> o;
    if constexpr (WT == SV_FP8) e4m3x16_to_bf16(w, o.v[0], o.v[1]);
    else o.v[0] = w;
    return o;
}

template <int WT>
SV_DEV f32x4_t mma_op(const WOp<WT>& w, const uint4* x, f32x4_t c)
{
    if constexpr (WT == SV_F32) {
        return mma_f32x4(w.v[0], x[0], c);
    } else if constexpr (WT == SV_BF16) {
        return mma_bf16(w.v[0], x[0], c);
    } else if constexpr (WT == SV_MXFP4) {
        c = mma_bf16(w.v[0], x[0], c);
        c = mma_bf16(w.v[1], x[1], c);
        c = mma_bf16(w.v[2], x[2], c);
        return mma_bf16(w.v[3], x[3], c);
    } else {
        c = mma_bf16(w.v[0], x[0], c);
        return mma_bf16(w.v[1], x[1], c);
    }
}

template <int WT>
SV_DEV f32x4_t mma_step(uint4 w, const uint4* x, f32x4_t c)
{
    if constexpr (WT == SV_F32) {
        return mma_f32x4(w, x[0], c);
    } else if constexpr (WT == SV_BF16) {
        return mma_bf16(w, x[0], c);
    } else {
        uint4 lo, hi;
        e4m3x16_to_bf16(w, lo, hi);
        c = mma_bf16(lo, x[0], c);
        return mma_bf16(hi, x[1], c);
    }
}

// Epilogue shared by the GEMM kernels.  The lane holds columns
// ncol0 + 16 f + 4 lg + e (e = 0..3) of rows row0 + 16 m + l16; `red` is
// WAVES * 16 MF keys of shared memory (argmax mode only).
template <int WT, int MF, int NF, int MODE, int WAVES>
SV_DEV void gemm_epilogue(const GemmArgs& a, f32x4_t (&acc)[MF][(MODE == GM_SWIGLU) ? 2 * NF : NF],
                          int row0, int nrows, int ncol0, int nt, const float* sc,
                          const bool (&fvalid)[NF], unsigned long long* red)
{
    constexpr int AESZ = ATraits<WT>::ESZ;
    constexpr int BM = 16 * MF;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    if constexpr (MODE == GM_STORE) {
        float* out = (float*)a.out + (size_t)blockIdx.y * a.split_stride;
#pragma unroll
        for (int f = 0; f < NF; f++) {
            int n = ncol0 + 16 * f + 4 * lg;
            if (!fvalid[f] || n >= a.N) continue;
            float s0 = 1.f, s1 = 1.f, s2 = 1.f, s3 = 1.f;
            if constexpr (WT == SV_FP8) { s0 = sc[n]; s1 = sc[n + 1]; s2 = sc[n + 2]; s3 = sc[n + 3]; }
#pragma unroll
            for (int m = 0; m < MF; m++) {
                int r = 16 * m + l16;
                if (r >= nrows) continue;
                float4 v = make_float4(acc[m][f][0] * s0, acc[m][f][1] * s1, acc[m][f][2] * s2,
                                       acc[m][f][3] * s3);
                *reinterpret_cast<float4*>(out + (size_t)(row0 + r) * a.ldo + n) = v;
            }
        }
    } else if constexpr (MODE == GM_SWIGLU) {
#pragma unroll
        for (int f = 0; f < NF; f++) {
            int n = ncol0 + 16 * f + 4 * lg;
            if (!fvalid[f] || n >= a.N) continue;
            float gs[4] = {1.f, 1.f, 1.f, 1.f}, us[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (WT == SV_FP8) {
#pragma unroll
                for (int r = 0; r < 4; r++) { gs[r] = sc[n + r]; us[r] = sc[a.dual_off + n + r]; }
            }
#pragma unroll
            for (int m = 0; m < MF; m++) {
                int r = 16 * m + l16;
                if (r >= nrows) continue;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; e++)
                    v[e] = silu_f32(acc[m][f][e] * gs[e]) * (acc[m][NF + f][e] * us[e]);
                size_t o = (size_t)(row0 + r) * a.ldo + n;
                if constexpr (AESZ == 2) {
                    uint2 p = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                    *reinterpret_cast<uint2*>((uint16_t*)a.out + o) = p;
                } else {
                    *reinterpret_cast<float4*>((float*)a.out + o) = make_float4(v[0], v[1], v[2], v[3]);
                }
            }
        }
    } else {   // GM_ARGMAX
#pragma unroll
        for (int m = 0; m < MF; m++) {
            unsigned long long best = 0ull;
            int r = 16 * m + l16;
#pragma unroll
            for (int f = 0; f < NF; f++) {
                int n = ncol0 + 16 * f + 4 * lg;
                if (!fvalid[f] || n >= a.N) continue;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    v[e] = acc[m][f][e];
                    if constexpr (WT == SV_FP8) v[e] *= sc[n + e];
                    best = umax64(best, argmax_key(v[e], (uint32_t)(n + e)));
                }
                if (a.dbg && r < nrows)
                    *reinterpret_cast<float4*>(a.dbg + (size_t)(row0 + r) * a.dbg_ld + n) =
                        make_float4(v[0], v[1], v[2], v[3]);
            }
            best = umax64(best, shfl_xor_u64(best, 16));
            best = umax64(best, shfl_xor_u64(best, 32));
            if (lg == 0) red[wave * BM + r] = best;
        }
        __syncthreads();
        for (int r = threadIdx.x; r < nrows; r += 64 * WAVES) {
            unsigned long long b = red[r];
#pragma unroll
            for (int w2 = 1; w2 < WAVES; w2++) b = umax64(b, red[w2 * BM + r]);
            a.keys[(size_t)nt * a.key_ld + row0 + r] = b;
        }
    }
}

// WAVES waves per workgroup side by side (a 16*NF*WAVES-column tile), or with
// KW the WAVES waves share one 16*NF-column tile and each takes a contiguous
// share of the reduction steps (more loads in flight per column tile; wave 0
// adds the other waves' partial sums from shared memory in wave order, then
// runs the epilogue; STORE and SWIGLU only).  UU reduction steps per prefetch
// stage (0: by row count).
template <int WT, int MF, int NF, int MODE, int WAVES = 4, int UU = 0, bool PACKED = false, bool KW = false>
__global__ __launch_bounds__(64 * WAVES) void gemm_kernel(GemmArgs a)
{
    static_assert(!KW || MODE != GM_ARGMAX, "K-split waves: STORE and SWIGLU epilogues only");
    constexpr bool MX = WT == SV_MXFP4;
    static_assert(!MX || PACKED, "MXFP4 weights: tiled16 layout only");
    using Tr = WTraits<WT>;
    constexpr int KL = Tr::KL, SK = Tr::SK, XU = Tr::XU, WESZ = Tr::ESZ;
    constexpr int EH = w_half_bytes<WT>();
    constexpr int AESZ = ATraits<WT>::ESZ;
    constexpr int NFT = (MODE == GM_SWIGLU) ? 2 * NF : NF;   // weight fragments per wave
    constexpr int BM = 16 * MF;
    // reduction steps per stage (by row count unless given; an MXFP4 step
    // carries four bf16 steps of activations, so half as many by default)
    constexpr int U0 = (MF >= 4) ? 2 : (MF == 2 ? 4 : 8);
    constexpr int U = UU ? UU : (MX ? U0 / 2 : U0);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l16 = lane & 15;
    const int lg = lane >> 4;

    // XCD-aware tile mapping (tiles implied by the selections: the column
    // tile by id modulo 8, its row tiles 8 ids apart; otherwise balanced, the
    // device-built tile count in grouped mode)
    const int id = blockIdx.x;
    int mt, nt;
    if (a.sel) {
        mt = (id >> 3) % a.MT;
        nt = ((id >> 3) / a.MT) * 8 + (id & 7);
        if (nt >= a.NT) return;
    } else if (!xcd_item(id, a.NT, a.tiles ? *a.n_tiles : a.MT, nt, mt)) {
        return;
    }

    int group = 0, row0, nrows;
    bool keep = false;   // weights also read by sibling row tiles: normal (cached) loads
    int xtok = -1;   // implied tiles: activation row of this lane's row l16 (MF == 1)
    if (a.sel) {
        const int A = a.sel_T * a.sel_k;
        int sraw = 0;
        bool selected = false;
        // shared-expert tiles need no selection (workgroup 0 still makes and
        // publishes it)
        const bool shared_tile = mt < a.sel_S;
        if constexpr (MODE == GM_SWIGLU) {
            if (a.sel_logits && (!shared_tile || (blockIdx.x == 0 && blockIdx.y == 0))) {
                // the routing's selection of every row (T <= 4, E <= 64): all
                // rows' logits in one round trip, then the selections in this wave
                __shared__ int ssel[WAVES][64];
                __shared__ float sgate[WAVES][64];
                const int E = a.sel_E;
                float lv[4];
#pragma unroll
                for (int t = 0; t < 4; t++) lv[t] = a.sel_logits[(size_t)min(t, a.sel_T - 1) * E + min(lane, E - 1)];
                router_select_rows4(E, a.sel_k, a.sel_renorm != 0, a.sel_T, lv, ssel[wave], sgate[wave]);
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                sraw = ssel[wave][min(lane, A - 1)];
                if (blockIdx.x == 0 && blockIdx.y == 0 && wave == 0 && lane < A) {
                    a.sel_out[lane] = sraw;
                    a.gate_out[lane] = sgate[0][lane];
                    if (a.dbg_sel_out) a.dbg_sel_out[lane] = sraw;
                }
                selected = true;
            }
        }
        if (!selected && !shared_tile) sraw = a.sel[min(lane, A - 1)];
        const int sv = min(max(sraw, 0), a.sel_E - 1);
        const ImpliedTile it = implied_tile(sv, A, a.sel_T, a.sel_E, a.sel_S, mt);
        group = it.group;
        row0 = it.row0;
        nrows = it.nrows;
        if (group < a.sel_E) {
            // row i of an expert tile is its i-th member assignment: send each
            // member's token to lane i (non-members to lane 63, never a row)
            const bool mem = (it.members >> lane) & 1ull;
            const int dst = mem ? __popcll(it.members & ((1ull << lane) - 1ull)) : 63;
            xtok = __builtin_amdgcn_ds_permute(4 * dst, lane / a.sel_k);
        } else {
            xtok = l16;   // shared expert: row i is token i
        }
    } else if (a.tiles) {
        group = a.tiles[3 * mt];
        row0 = a.tiles[3 * mt + 1];
        nrows = a.tiles[3 * mt + 2];
        keep = group_has_siblings(a.tiles, mt, *a.n_tiles, group);
    } else {
        row0 = mt * BM;
        nrows = min(BM, a.M - row0);
    }
    if (nrows <= 0) return;

    const char* Wb;
    const float* sc;
    const uint8_t* scb = nullptr;   // MXFP4: the group's E8M0 block scales [rows][K/32]
    if (group < a.G1) {
        Wb = (const char*)a.W + (size_t)group * a.w_gstride * EH / 2;
        sc = a.ws ? a.ws + (size_t)group * a.s_gstride : nullptr;
        if constexpr (MX) scb = (const uint8_t*)a.ws + (size_t)group * a.s_gstride;
    } else {
        Wb = (const char*)a.W2 + (size_t)(group - a.G1) * a.w2_gstride * EH / 2;
        sc = a.ws2 ? a.ws2 + (size_t)(group - a.G1) * a.s2_gstride : nullptr;
        if constexpr (MX) scb = (const uint8_t*)a.ws2 + (size_t)(group - a.G1) * a.s2_gstride;
    }

    const int ncol0 = KW ? nt * 16 * NF : (nt * WAVES + wave) * 16 * NF;   // this wave's first column
    const int K = a.K;
    const int kspan = K / a.ksplit;
    int kb = blockIdx.y * kspan;
    int ke = kb + kspan;
    if constexpr (KW) {   // wave w: reduction steps [w S / WAVES, (w + 1) S / WAVES) of the split
        // (the wave index made explicitly uniform: scalar loop bounds, as in the
        // one-wave case; derived from the lane id the loop became exec-masked and
        // its sums came out wrong)
        const int wu = __builtin_amdgcn_readfirstlane(wave);
        const int steps = kspan / SK;
        ke = kb + (wu + 1) * steps / WAVES * SK;
        kb = kb + wu * steps / WAVES * SK;
    }

    // weight rows of this lane, one per fragment (invalid fragments read row 0)
    const char* wrow[NFT];
    uint4 sslice[MX ? NFT : 1];   // MXFP4: this lane's scale bytes of steps 0..15 (K <= 2048)
    bool fvalid[NF];
#pragma unroll
    for (int f = 0; f < NF; f++) {
        int n0 = ncol0 + 16 * f;
        fvalid[f] = n0 < a.N;
        int r = fvalid[f] ? min(n0 + l16, a.N - 1) : 0;   // rows past N read row N-1
        if constexpr (PACKED) {
            // 16-row blocks stored step-major: block rb, step s at ((rb * K/SK) + s) KiB,
            // lane l's 16 bytes at l * 16; the k offset below is in elements of SK per KiB
            int rb = fvalid[f] ? n0 / 16 : 0;
            wrow[f] = Wb + (size_t)rb * K * 8 * EH + (size_t)lane * 16;
            if constexpr (MODE == GM_SWIGLU)
                wrow[NF + f] = Wb + (size_t)(rb + a.dual_off / 16) * K * 8 * EH + (size_t)lane * 16;
            if constexpr (MX) {
                // tiled scales: one 16-byte slice per lane and row block (16 steps)
                sslice[f] = ldg16(scb + ((size_t)rb * 64 + lane) * 16);
                if constexpr (MODE == GM_SWIGLU)
                    sslice[NF + f] = ldg16(scb + ((size_t)(rb + a.dual_off / 16) * 64 + lane) * 16);
            }
        } else {
            wrow[f] = Wb + ((size_t)r * K + (size_t)lg * KL) * WESZ;
            if constexpr (MODE == GM_SWIGLU)
                wrow[NF + f] = Wb + ((size_t)(r + a.dual_off) * K + (size_t)lg * KL) * WESZ;
        }
    }
    // activation rows of this lane, one per row fragment
    const char* xrow[MF];
#pragma unroll
    for (int m = 0; m < MF; m++) {
        int r = 16 * m + l16;
        r = (r < nrows) ? row0 + r : row0;
        int xr;
        if (a.sel) xr = a.gather ? __shfl(xtok, min(16 * m + l16, nrows - 1), 64) : r;   // (MF == 1)
        else xr = a.gather ? a.gather[r] : r;
        xrow[m] = (const char*)a.X + ((size_t)xr * a.ldx + (size_t)lg * KL) * AESZ;
    }

    f32x4_t acc[MF][NFT];
#pragma unroll
    for (int m = 0; m < MF; m++)
#pragma unroll
        for (int f = 0; f < NFT; f++) acc[m][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 wA[U][NFT], wB[U][NFT];
    uint4 xA[U][MF][XU], xB[U][MF][XU];
    uint32_t sA[U][MX ? NFT : 1], sB[U][MX ? NFT : 1];   // MXFP4 scale bytes

    auto load = [&](int k, uint4 (&w)[U][NFT], uint4 (&x)[U][MF][XU],
                    uint32_t (&sb)[U][MX ? NFT : 1]) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            int kk = k + u * SK;
            if (kk < ke) {
                auto wl = [&](auto ld) {
#pragma unroll
                    for (int f = 0; f < NFT; f++) {
                        if constexpr (PACKED) w[u][f] = ld(wrow[f] + (size_t)(kk / SK) * 1024);
                        else w[u][f] = ld(wrow[f] + (size_t)kk * WESZ);
                        if constexpr (MX) sb[u][f] = mx_scale_byte(sslice[f], kk / SK);
                    }
                };
                if (keep) wl([](const void* p) { return ldg16(p); });
                else wl([](const void* p) { return ldg16_stream(p); });
#pragma unroll
                for (int m = 0; m < MF; m++)
#pragma unroll
                    for (int v = 0; v < XU; v++)
                        x[u][m][v] = ldg16(xrow[m] + ((size_t)kk + 8 * v) * AESZ);
            }
        }
    };
    auto compute = [&](int k, uint4 (&w)[U][NFT], uint4 (&x)[U][MF][XU],
                       uint32_t (&sb)[U][MX ? NFT : 1]) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (k + u * SK < ke) {
#pragma unroll
                for (int f = 0; f < NFT; f++) {
                    WOp<WT> wo;
                    if constexpr (MX) wo = wprep_mx(w[u][f], sb[u][f]);
                    else wo = wprep<WT>(w[u][f]);
#pragma unroll
                    for (int m = 0; m < MF; m++) acc[m][f] = mma_op<WT>(wo, x[u][m], acc[m][f]);
                }
            }
        }
    };

    constexpr int STAGE = U * SK;
    if (kb < ke) load(kb, wA, xA, sA);
    for (int k = kb; k < ke; k += 2 * STAGE) {
        if (k + STAGE < ke) load(k + STAGE, wB, xB, sB);
        compute(k, wA, xA, sA);
        if (k + 2 * STAGE < ke) load(k + 2 * STAGE, wA, xA, sA);
        if (k + STAGE < ke) compute(k + STAGE, wB, xB, sB);
    }
    if constexpr (KW) {
        // partial sums of waves 1.. through shared memory, added by wave 0 in wave order
        __shared__ f32x4_t part[WAVES > 1 ? WAVES - 1 : 1][MF][NFT][64];
        if (wave > 0) {
#pragma unroll
            for (int m = 0; m < MF; m++)
#pragma unroll
                for (int f = 0; f < NFT; f++) part[wave - 1][m][f][lane] = acc[m][f];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 0; w < WAVES - 1; w++)
#pragma unroll
            for (int m = 0; m < MF; m++)
#pragma unroll
                for (int f = 0; f < NFT; f++) acc[m][f] += part[w][m][f][lane];
        gemm_epilogue<WT, MF, NF, MODE, 1>(a, acc, row0, nrows, ncol0, nt, sc, fvalid, nullptr);
        return;
    }

    // ------------------------------------------------------------ epilogue
    if constexpr (MODE == GM_ARGMAX) {
        __shared__ unsigned long long red[WAVES * BM];
        gemm_epilogue<WT, MF, NF, MODE, WAVES>(a, acc, row0, nrows, ncol0, nt, sc, fvalid, red);
    } else {
        gemm_epilogue<WT, MF, NF, MODE, WAVES>(a, acc, row0, nrows, ncol0, nt, sc, fvalid, nullptr);
    }
}

// ---------------------------------------------------------------------------
// MXFP4 weights, up to 16 rows, K <= 128 MAXS (the LM head at few rows).  A
// quarter of the bf16 bytes per reduction step leaves the small-row kernel
// above latency-bound (a wave's weights arrive in several dependent stages,
// four activation registers per weight load).  Here each wave issues every
// weight load of its NF column fragments at once (the whole reduction in
// registers), while the workgroup copies the activations straight into LDS
// (global_load_lds: no registers) in MFMA operand order; after one wait the
// steps run from registers and LDS.  Grid and tiles as gemm_kernel (dense,
// 16-row tiles, 4 waves of NF fragments side by side).
template <int NF, int MAXS, int MODE>
__global__ __launch_bounds__(256) void gemm_mx_lds_kernel(GemmArgs a)
{
    constexpr int WAVES = 4, MF = 1, BM = 16;
    __shared__ uint4 xs[MAXS][4][64];   // [step][8-element unit][lane]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int id = blockIdx.x, xcd = id & 7, q = id >> 3;
    const int mt = q % a.MT;
    const int nt = (q / a.MT) * 8 + xcd;
    if (nt >= a.NT) return;
    const int row0 = mt * BM, nrows = min(BM, a.M - row0);
    if (nrows <= 0) return;
    const int K = a.K, nsteps = K / 128;
    const int ncol0 = (nt * WAVES + wave) * 16 * NF;

    const char* wrow[NF];
    uint4 sslice[NF];
    bool fvalid[NF];
#pragma unroll
    for (int f = 0; f < NF; f++) {
        const int n0 = ncol0 + 16 * f;
        fvalid[f] = n0 < a.N;
        const int rb = fvalid[f] ? n0 / 16 : 0;
        wrow[f] = (const char*)a.W + (size_t)rb * K * 8 + (size_t)lane * 16;
        sslice[f] = ldg16((const uint8_t*)a.ws + ((size_t)rb * 64 + lane) * 16);   // K <= 2048
    }
    uint4 w[MAXS][NF];
#pragma unroll
    for (int s = 0; s < MAXS; s++)
        if (s < nsteps)
#pragma unroll
            for (int f = 0; f < NF; f++) w[s][f] = ldg16_stream(wrow[f] + (size_t)s * 1024);
    // activations: wave v stages steps v, v + 4, ...; lane (l16, lg) of unit u
    // of step s holds row l16, columns 128 s + 32 lg + 8 u .. + 7
    {
        const int xr = row0 + min(l16, nrows - 1);
        const char* xsrc = (const char*)a.X + ((size_t)xr * a.ldx + (size_t)lg * 32) * 2;
        for (int s = wave; s < nsteps; s += WAVES)
#pragma unroll
            for (int u = 0; u < 4; u++)
                __builtin_amdgcn_global_load_lds((const void*)(xsrc + ((size_t)s * 128 + 8 * u) * 2),
                                                 (__attribute__((address_space(3))) void*)&xs[s][u][0],
                                                 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    f32x4_t acc[MF][NF];
#pragma unroll
    for (int f = 0; f < NF; f++) acc[0][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < MAXS; s++) {
        if (s < nsteps) {
            uint4 xf[4];
#pragma unroll
            for (int u = 0; u < 4; u++) xf[u] = xs[s][u][lane];
#pragma unroll
            for (int f = 0; f < NF; f++) {
                const WOp<SV_MXFP4> wo = wprep_mx(w[s][f], mx_scale_byte(sslice[f], s));
                acc[0][f] = mma_op<SV_MXFP4>(wo, xf, acc[0][f]);
            }
        }
    }
    if constexpr (MODE == GM_ARGMAX) {
        __shared__ unsigned long long red[WAVES * BM];
        gemm_epilogue<SV_MXFP4, MF, NF, MODE, WAVES>(a, acc, row0, nrows, ncol0, nt, nullptr, fvalid, red);
    } else {
        gemm_epilogue<SV_MXFP4, MF, NF, MODE, WAVES>(a, acc, row0, nrows, ncol0, nt, nullptr, fvalid, nullptr);
    }
}

// ---------------------------------------------------------------------------
// Large-row variant (dense mode with 64 .. 256 rows, or grouped mode).  The small-row kernel above
// re-reads every activation fragment from cache for each 16x16 product; with
// 16 row fragments per wave that traffic exceeds what the vector cache can
// deliver.  Here the workgroup stages a K-chunk of all its rows in LDS once,
// in operand order (row block, step, lane: one 1 KiB piece per fragment, read
// back with one conflict-free 16-byte access per lane), double-buffered with
// one barrier per chunk; each wave streams NF (x2 for SwiGLU) distinct weight
// fragments from HBM one chunk ahead and applies every activation fragment to
// all of them.
template <int WT, int MF, int NF, int MODE, bool PACKED>
__global__ __launch_bounds__(256) void gemm_bigm_kernel(GemmArgs a)
{
    constexpr bool MX = WT == SV_MXFP4;
    static_assert(!MX || PACKED, "MXFP4 weights: tiled16 layout only");
    using Tr = WTraits<WT>;
    constexpr int KL = Tr::KL, SK = Tr::SK, XU = Tr::XU, WESZ = Tr::ESZ;
    constexpr int EH = w_half_bytes<WT>();
    constexpr int AESZ = ATraits<WT>::ESZ;
    constexpr int NFT = (MODE == GM_SWIGLU) ? 2 * NF : NF;
    constexpr int BM = 16 * MF;
    constexpr int CS = MX ? 1 : 2;               // reduction steps per chunk (an MXFP4 step is 128 long)
    constexpr int KC = CS * SK;                  // chunk length
    constexpr int PIECES = MF * CS * XU;         // 1 KiB activation pieces per chunk
    constexpr int PPW = (PIECES + 3) / 4;        // pieces each wave stages (the last may idle)
    __shared__ uint4 xs[2][PIECES < 4 ? 4 : PIECES][64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    int mt, nt;
    const int ntiles = a.tiles ? *a.n_tiles : a.MT;
    if (!xcd_item(blockIdx.x, a.NT, ntiles, nt, mt)) return;
    int group = 0, row0, nrows;
    bool keep = false;
    if (a.tiles) {
        group = a.tiles[3 * mt];
        row0 = a.tiles[3 * mt + 1];
        nrows = a.tiles[3 * mt + 2];
        keep = group_has_siblings(a.tiles, mt, ntiles, group);
    } else {
        row0 = mt * BM;
        nrows = min(BM, a.M - row0);
    }
    if (nrows <= 0) return;
    const char* Wb;
    const float* sc;
    const uint8_t* scb = nullptr;   // MXFP4: the group's tiled E8M0 scales
    if (group < a.G1) {
        Wb = (const char*)a.W + (size_t)group * a.w_gstride * EH / 2;
        sc = a.ws ? a.ws + (size_t)group * a.s_gstride : nullptr;
        if constexpr (MX) scb = (const uint8_t*)a.ws + (size_t)group * a.s_gstride;
    } else {
        Wb = (const char*)a.W2 + (size_t)(group - a.G1) * a.w2_gstride * EH / 2;
        sc = a.ws2 ? a.ws2 + (size_t)(group - a.G1) * a.s2_gstride : nullptr;
        if constexpr (MX) scb = (const uint8_t*)a.ws2 + (size_t)(group - a.G1) * a.s2_gstride;
    }
    const int ncol0 = (nt * 4 + wave) * 16 * NF;
    const int K = a.K;
    const int kspan = K / a.ksplit;
    const int kb = blockIdx.y * kspan;
    const int nchunk = kspan / KC;

    const char* wrow[NFT];
    uint4 sslice[MX ? NFT : 1];   // MXFP4: the lane's scale bytes of steps 0..15 (K <= 2048)
    bool fvalid[NF];
#pragma unroll
    for (int f = 0; f < NF; f++) {
        int n0 = ncol0 + 16 * f;
        fvalid[f] = n0 < a.N;
        int r = fvalid[f] ? min(n0 + l16, a.N - 1) : 0;
        if constexpr (PACKED) {
            int rb = fvalid[f] ? n0 / 16 : 0;
            wrow[f] = Wb + (size_t)rb * K * 8 * EH + (size_t)lane * 16;
            if constexpr (MODE == GM_SWIGLU)
                wrow[NF + f] = Wb + (size_t)(rb + a.dual_off / 16) * K * 8 * EH + (size_t)lane * 16;
            if constexpr (MX) {
                sslice[f] = ldg16(scb + ((size_t)rb * 64 + lane) * 16);
                if constexpr (MODE == GM_SWIGLU)
                    sslice[NF + f] = ldg16(scb + ((size_t)(rb + a.dual_off / 16) * 64 + lane) * 16);
            }
        } else {
            wrow[f] = Wb + ((size_t)r * K + (size_t)lg * KL) * WESZ;
            if constexpr (MODE == GM_SWIGLU)
                wrow[NF + f] = Wb + ((size_t)(r + a.dual_off) * K + (size_t)lg * KL) * WESZ;
        }
    }
    // activation pieces this wave stages: piece p = (m * CS + s) * XU + v
    const char* xsrc[PPW];
#pragma unroll
    for (int i = 0; i < PPW; i++) {
        int p = min(wave * PPW + i, PIECES - 1);
        int v = p % XU, s = (p / XU) % CS, m = p / (XU * CS);
        int r = 16 * m + l16;
        r = (r < nrows) ? row0 + r : row0;
        int xr = a.gather ? a.gather[r] : r;
        xsrc[i] = (const char*)a.X + ((size_t)xr * a.ldx + (size_t)s * SK + (size_t)lg * KL + 8 * v) * AESZ;
    }
    auto staged = [&](int i) { return wave * PPW + i < PIECES; };
    auto wload = [&](int k, uint4 (&w)[CS][NFT]) {
        auto one = [&](auto ld) {
#pragma unroll
            for (int s = 0; s < CS; s++)
#pragma unroll
                for (int f = 0; f < NFT; f++) {
                    int kk = k + s * SK;
                    if constexpr (PACKED) w[s][f] = ld(wrow[f] + (size_t)(kk / SK) * 1024);
                    else w[s][f] = ld(wrow[f] + (size_t)kk * WESZ);
                }
        };
        if (keep) one([](const void* p) { return ldg16(p); });
        else one([](const void* p) { return ldg16_stream(p); });
    };
    auto xload = [&](int k, uint4 (&st)[PPW]) {
#pragma unroll
        for (int i = 0; i < PPW; i++)
            if (staged(i)) st[i] = ldg16(xsrc[i] + (size_t)k * AESZ);
    };

    f32x4_t acc[MF][NFT];
#pragma unroll
    for (int m = 0; m < MF; m++)
#pragma unroll
        for (int f = 0; f < NFT; f++) acc[m][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 wcur[CS][NFT], wnext[CS][NFT], stage[PPW];
    // weights first: the wait for the staged activations then also covers
    // them, so no load is still counted when the loop starts (a pending load
    // on entry would make every iteration wait for the next chunk's loads)
    wload(kb, wcur);
    xload(kb, stage);
#pragma unroll
    for (int i = 0; i < PPW; i++)
        if (staged(i)) xs[0][wave * PPW + i][lane] = stage[i];
    __syncthreads();
    for (int c = 0; c < nchunk; c++) {
        const int buf = c & 1;
        const int kn = kb + (c + 1) * KC;
        const bool more = c + 1 < nchunk;
        if (more) {
            xload(kn, stage);
            wload(kn, wnext);
        }
#pragma unroll
        for (int s = 0; s < CS; s++) {
            WOp<WT> wo[NFT];
#pragma unroll
            for (int f = 0; f < NFT; f++) {
                if constexpr (MX) wo[f] = wprep_mx(wcur[s][f], mx_scale_byte(sslice[f], (kb + c * KC) / SK + s));
                else wo[f] = wprep<WT>(wcur[s][f]);
            }
#pragma unroll
            for (int m = 0; m < MF; m++) {
                uint4 xf[XU];
#pragma unroll
                for (int v = 0; v < XU; v++) xf[v] = xs[buf][(m * CS + s) * XU + v][lane];
#pragma unroll
                for (int f = 0; f < NFT; f++) acc[m][f] = mma_op<WT>(wo[f], xf, acc[m][f]);
            }
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < PPW; i++)
                if (staged(i)) xs[buf ^ 1][wave * PPW + i][lane] = stage[i];
#pragma unroll
            for (int s = 0; s < CS; s++)
#pragma unroll
                for (int f = 0; f < NFT; f++) wcur[s][f] = wnext[s][f];
        }
        __syncthreads();
    }

    if constexpr (MODE == GM_ARGMAX) {
        // the activation buffers are no longer needed: reuse them for the reduction
        unsigned long long* red = reinterpret_cast<unsigned long long*>(&xs[0][0][0]);
        static_assert(sizeof(xs) >= 4 * BM * sizeof(unsigned long long), "reduction space");
        gemm_epilogue<WT, MF, NF, MODE, 4>(a, acc, row0, nrows, ncol0, nt, sc, fvalid, red);
    } else {
        gemm_epilogue<WT, MF, NF, MODE, 4>(a, acc, row0, nrows, ncol0, nt, sc, fvalid, nullptr);
    }
}

// ---------------------------------------------------------------------------
// Wide large-row variant: dense GEMMs with 64 .. 256 rows and bf16 or fp8
// weights in the tiled16 layout, on 32x32x16 MFMA tiles.  The activation
// chunk read from shared memory per product is what limits the large-row
// kernel above (one 1 KiB fragment per 16 columns); here a wave owns 32*MW
// rows x 32*NW columns, so every activation fragment read from LDS feeds NW
// 32-column products (half the LDS bytes per flop of a 32-column wave), and
// the WAVES waves of a workgroup sit side by side in columns sharing one
// staged chunk.  SwiGLU: the first NW/2 fragments are gate columns, the
// others the matching up columns.
//
// Reduction mapping.  A tiled16 piece holds 16 weight rows x SK elements as
// 64 16-byte slots (slot 16*g + r: row r, elements KL*g ..); one 16-byte
// load per lane takes row l%32 of a 32-row fragment from the piece pair of
// its two 16-row blocks, slot group g = 2u + l/32 (u = 0, 1), and yields XU
// MFMA operands (fp8: two, widened).  Operand (u, h) of lane l therefore
// carries elements KL*(2u + l/32) + 8h .. +7 of the step, and the activation
// operand staged for it carries the same elements of row l%32: every
// reduction index is used exactly once, in a fixed order.
//
// Staging: each thread loads 16-byte segments of activation rows and stores
// each where its operand lane reads it; chunks of CS steps are double-buffered
// with one barrier per chunk, weights are loaded one chunk ahead into
// registers.
template <int WT, int MW, int NW, int MODE, int WAVES, int CS = 2>
__global__ __launch_bounds__(64 * WAVES) void gemm_wide_kernel(GemmArgs a)
{
    static_assert(WT == SV_BF16 || WT == SV_FP8, "bf16 or fp8 weights");
    static_assert(MODE != GM_SWIGLU || NW % 2 == 0, "gate/up fragment pairs");
    constexpr int WESZ = (WT == SV_FP8) ? 1 : 2;
    constexpr int KL = 16 / WESZ;                // weight elements per 16-byte slot
    constexpr int SK = 4 * KL;                   // elements per tiled16 piece
    constexpr int XU = (WT == SV_FP8) ? 2 : 1;   // operands per 16-byte weight load
    constexpr int KC = CS * SK;                  // chunk length (CS steps)
    constexpr int BM = 32 * MW;
    constexpr int NWO = (MODE == GM_SWIGLU) ? NW / 2 : NW;   // output column fragments
    constexpr int PIECES = MW * CS * 2 * XU;     // 1 KiB activation operands per chunk
    constexpr int RSEG = KC / 8;                 // 16-byte segments of a row per chunk
    constexpr int SPT = BM * RSEG / (64 * WAVES);
    static_assert(SPT * 64 * WAVES == BM * RSEG, "staging split");
    __shared__ uint4 xs[2][PIECES][64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, lh = lane >> 5;
    int mt, nt;
    if (!xcd_item(blockIdx.x, a.NT, a.MT, nt, mt)) return;
    const int row0 = mt * BM;
    const int nrows = min(BM, a.M - row0);
    if (nrows <= 0) return;
    const char* Wb = (const char*)a.W;
    const float* sc = a.ws;
    const int K = a.K;
    const int kspan = K / a.ksplit;
    const int kb = blockIdx.y * kspan;
    const int nchunk = kspan / KC;
    const int ncol0 = (nt * WAVES + wave) * 32 * NWO;
    const int nrb = a.N / 16;                    // 16-row weight blocks

    // weight fragment bases: lane row l32 of the fragment, slot group lh
    const char* wrow[NW];
    bool fvalid[NWO];
#pragma unroll
    for (int f = 0; f < NW; f++) {
        const int fo = (MODE == GM_SWIGLU) ? f % NWO : f;
        const int n0 = ncol0 + 32 * fo;
        const bool ok = n0 < a.N;
        if (f < NWO) fvalid[f] = ok;
        int rb = ok ? min(n0 / 16 + (l32 >> 4), nrb - 1) : 0;
        if (MODE == GM_SWIGLU && f >= NWO) rb += a.dual_off / 16;
        wrow[f] = Wb + (size_t)rb * K * 16 * WESZ + (size_t)(16 * lh + (l32 & 15)) * 16;
    }
    // activation segments this thread stages: segment it = tid + 64 WAVES j
    const char* xsrc[SPT];
    int xdst[SPT];
#pragma unroll
    for (int j = 0; j < SPT; j++) {
        // a wave covers 16 rows x 4 segments: each 16-lane write phase then
        // stores 16 rows (distinct LDS banks), each row read is 64 bytes
        const int it = tid + 64 * WAVES * j, wi = it >> 6, li = it & 63;
        const int m = 16 * (wi / (RSEG / 4)) + (li & 15), qs = 4 * (wi % (RSEG / 4)) + (li >> 4);
        const int s = qs / (SK / 8), qq = qs % (SK / 8);
        const int sl = qq / XU, h = qq % XU;      // slot of the step, operand half
        const int u = sl >> 1, g = sl & 1;
        const int piece = (((m >> 5) * CS + s) * 2 + u) * XU + h;
        xdst[j] = piece * 64 + 32 * g + (m & 31);
        const int r = row0 + min(m, nrows - 1);
        xsrc[j] = (const char*)a.X + ((size_t)r * a.ldx + (size_t)s * SK + (size_t)qq * 8) * 2;
    }
    uint4* xsf = &xs[0][0][0];
    auto xload = [&](int k, uint4 (&st)[SPT]) {
#pragma unroll
        for (int j = 0; j < SPT; j++) st[j] = ldg16(xsrc[j] + (size_t)k * 2);
    };
    auto xstore = [&](int buf, const uint4 (&st)[SPT]) {
#pragma unroll
        for (int j = 0; j < SPT; j++) xsf[buf * PIECES * 64 + xdst[j]] = st[j];
    };
    auto wload = [&](int k, uint4 (&w)[CS][NW][2]) {
#pragma unroll
        for (int s = 0; s < CS; s++)
#pragma unroll
            for (int f = 0; f < NW; f++)
#pragma unroll
                for (int u = 0; u < 2; u++)
                    w[s][f][u] = ldg16(wrow[f] + (size_t)((k + s * SK) / SK) * 1024 + u * 512);
    };

    f32x16_t acc[MW][NW];
#pragma unroll
    for (int m = 0; m < MW; m++)
#pragma unroll
        for (int f = 0; f < NW; f++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[m][f][r] = 0.f;

    uint4 wcur[CS][NW][2], wnext[CS][NW][2], stage[SPT];
    wload(kb, wcur);         // weights first (see the large-row kernel)
    xload(kb, stage);
    xstore(0, stage);
    __syncthreads();
    for (int c = 0; c < nchunk; c++) {
        const int buf = c & 1;
        const bool more = c + 1 < nchunk;
        if (more) {
            const int kn = kb + (c + 1) * KC;
            xload(kn, stage);
            wload(kn, wnext);
        }
        const uint4* xb = xsf + buf * PIECES * 64 + lane;
#pragma unroll
        for (int s = 0; s < CS; s++)
#pragma unroll
            for (int u = 0; u < 2; u++) {
                WOp<WT> wo[NW];
#pragma unroll
                for (int f = 0; f < NW; f++) wo[f] = wprep<WT>(wcur[s][f][u]);
#pragma unroll
                for (int h = 0; h < XU; h++)
#pragma unroll
                    for (int m = 0; m < MW; m++) {
                        const uint4 xf = xb[((((m * CS + s) * 2 + u) * XU) + h) * 64];
#pragma unroll
                        for (int f = 0; f < NW; f++) acc[m][f] = mma32_bf16(wo[f].v[h], xf, acc[m][f]);
                    }
            }
        if (more) {
            xstore(buf ^ 1, stage);
#pragma unroll
            for (int s = 0; s < CS; s++)
#pragma unroll
                for (int f = 0; f < NW; f++)
#pragma unroll
                    for (int u = 0; u < 2; u++) wcur[s][f][u] = wnext[s][f][u];
        }
        __syncthreads();
    }

    // epilogue: lane holds rows row0 + 32 m + l32, columns n0 + 8 j + 4 lh + e
    // (register 4 j + e) of each fragment
    if constexpr (MODE == GM_STORE) {
        float* out = (float*)a.out + (size_t)blockIdx.y * a.split_stride;
#pragma unroll
        for (int f = 0; f < NW; f++) {
            if (!fvalid[f]) continue;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int n = ncol0 + 32 * f + 8 * j + 4 * lh;
                if (n >= a.N) continue;
                float s4[4] = {1.f, 1.f, 1.f, 1.f};
                if constexpr (WT == SV_FP8) {
#pragma unroll
                    for (int e = 0; e < 4; e++) s4[e] = sc[n + e];
                }
#pragma unroll
                for (int m = 0; m < MW; m++) {
                    const int r = 32 * m + l32;
                    if (r >= nrows) continue;
                    *reinterpret_cast<float4*>(out + (size_t)(row0 + r) * a.ldo + n) =
                        make_float4(acc[m][f][4 * j] * s4[0], acc[m][f][4 * j + 1] * s4[1],
                                    acc[m][f][4 * j + 2] * s4[2], acc[m][f][4 * j + 3] * s4[3]);
                }
            }
        }
    } else if constexpr (MODE == GM_SWIGLU) {
#pragma unroll
        for (int f = 0; f < NWO; f++) {
            if (!fvalid[f]) continue;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int n = ncol0 + 32 * f + 8 * j + 4 * lh;
                if (n >= a.N) continue;
                float gs[4] = {1.f, 1.f, 1.f, 1.f}, us[4] = {1.f, 1.f, 1.f, 1.f};
                if constexpr (WT == SV_FP8) {
#pragma unroll
                    for (int e = 0; e < 4; e++) { gs[e] = sc[n + e]; us[e] = sc[a.dual_off + n + e]; }
                }
#pragma unroll
                for (int m = 0; m < MW; m++) {
                    const int r = 32 * m + l32;
                    if (r >= nrows) continue;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        v[e] = silu_f32(acc[m][f][4 * j + e] * gs[e]) * (acc[m][NWO + f][4 * j + e] * us[e]);
                    *reinterpret_cast<uint2*>((uint16_t*)a.out + (size_t)(row0 + r) * a.ldo + n) =
                        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
            }
        }
    } else {   // GM_ARGMAX: per row, the largest key over the workgroup's columns
        unsigned long long* red = reinterpret_cast<unsigned long long*>(xsf);
        static_assert(sizeof(xs) >= WAVES * BM * sizeof(unsigned long long), "reduction space");
#pragma unroll
        for (int m = 0; m < MW; m++) {
            const int r = 32 * m + l32;
            unsigned long long best = 0ull;
#pragma unroll
            for (int f = 0; f < NW; f++) {
                if (!fvalid[f]) continue;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int n = ncol0 + 32 * f + 8 * j + 4 * lh;
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
            if (lh == 0) red[wave * BM + r] = best;
        }
        __syncthreads();
        for (int r = tid; r < nrows; r += 64 * WAVES) {
            unsigned long long b = red[r];
#pragma unroll
            for (int w2 = 1; w2 < WAVES; w2++) b = umax64(b, red[w2 * BM + r]);
            a.keys[(size_t)nt * a.key_ld + row0 + r] = b;
        }
    }
}
