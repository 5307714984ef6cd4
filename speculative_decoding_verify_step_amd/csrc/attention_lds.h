// attention_lds.h -- split-KV verify attention for many query rows per KV
// head (grouped-query heads times block positions, R = (K+1) G >= 17), with
// the K/V tiles staged in LDS.
//
// One workgroup takes one (sequence, KV head, chunk of CH keys) for all R
// rows of the KV head: NW waves, wave w owning the FPW 16-row query
// fragments 16 FPW w ..  Every 4 KL-key tile of the chunk is one pipeline
// stage: the workgroup copies the tile's K and V operand pieces (1 KiB each,
// stored in MFMA operand order by the cache layout) straight from the cache
// into an S-deep LDS ring (no register staging, S - 1 tiles in flight), and
// each wave reads the pieces from LDS for its fragments.  So every K/V byte is
// read from HBM once per step, however many query rows use it, and the
// workgroup's waves keep the tile loads of later stages in flight while they
// multiply.  The per-tile math (scores, masking, online softmax, output
// product) and the chunk partials are those of attn_split_kernel; the merge
// kernel is shared.
#pragma once
#include "attention.h"
#include "lds_dma.h"

template <int DH, int FPW, int NW, int S>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void attn_lds_kernel(AttnArgs a)
{
    constexpr int ESZ = 2, KL = 8, KT = 4 * KL;        // bf16: 32 keys per tile
    constexpr int DS = DH / (4 * KL), DF = DH / 16, NB = KL / 4;
    constexpr int KP = NB * DS;                        // K pieces per tile
    constexpr int PPT = KP + DF;                       // K + V pieces per tile
    static_assert(PPT % NW == 0, "pieces per wave");
    constexpr int PPW = PPT / NW;                      // copies per wave per stage
    static_assert(S >= 2 && S <= 4 && PPW * (S - 1) < 64, "ring depth");
    constexpr size_t TILE = (size_t)KT * DH * ESZ;     // bytes per key tile of K (and of V)
    __shared__ __align__(16) uint4 lds[S][PPT][64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int chunk = blockIdx.x, hkv = blockIdx.y, b = blockIdx.z;
    const int K1 = a.K1, G = a.n_q / a.n_kv, R = K1 * G;
    const int c0 = chunk * a.CH;
    // paged caches: lane i holds the physical page of this chunk's i-th page
    const bool paged = a.kvp.table != nullptr;
    const int pg0 = paged ? c0 / a.kvp.page : 0;
    int my_page = 0;
    if (paged) my_page = a.kvp.table[(size_t)b * a.kvp.max_pages + min(pg0 + lane, a.kvp.max_pages - 1)];
    const int ctx = min(max(a.ctx_in[b], 0), a.cap - K1);
    const int total = ctx + K1;
    if (c0 >= total) return;
    const int c1 = min(c0 + a.CH, total);
    const int nst = (c1 - c0 + KT - 1) / KT;

    const size_t head = ((size_t)b * a.L + a.layer) * a.n_kv + hkv;
    const char* kbase = (const char*)a.kc + head * (size_t)a.cap * DH * ESZ + lane * 16;
    const char* vbase = (const char*)a.vc + head * (size_t)a.cap * DH * ESZ + lane * 16;
    if (paged) {
        const bool bad = pg0 + lane <= (c1 - 1) / a.kvp.page && (my_page < 0 || my_page >= a.kvp.n_pages);
        if (__any(bad) && lane == 0) atomicOr(a.err_word, SV_DEV_CAPACITY);
        my_page = min(max(my_page, 0), a.kvp.n_pages - 1);
    }
    const size_t page_bytes = paged ? (size_t)a.kvp.page * DH * ESZ : 0;

    // stage st = key tile c0 + KT st into ring slot st % S; this wave copies
    // pieces PPW wave .. PPW wave + PPW - 1 of the tile's K pieces, then V pieces
    auto issue = [&](int st) {
        const int kt = c0 + st * KT;
        const char* tk;
        const char* tv;
        if (paged) {
            const int pg = __shfl(my_page, kt / a.kvp.page - pg0, 64);
            const size_t off = (((size_t)pg * a.L + a.layer) * a.n_kv + hkv) * page_bytes +
                               (size_t)((kt % a.kvp.page) / KT) * TILE + lane * 16;
            tk = (const char*)a.kc + off;
            tv = (const char*)a.vc + off;
        } else {
            const size_t toff = (size_t)(kt / KT) * TILE;
            tk = kbase + toff;
            tv = vbase + toff;
        }
#pragma unroll
        for (int i = 0; i < PPW; i++) {
            const int p = wave * PPW + i;
            const char* g = p < KP ? tk + (size_t)p * 1024 : tv + (size_t)(p - KP) * 1024;
            copy_to_lds(g, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4*)&lds[st % S][p][0]);
        }
    };

    float m_run[FPW];
    f32x4_t lsum[FPW], o[FPW][DF];
#pragma unroll
    for (int i = 0; i < FPW; i++) {
        m_run[i] = -INFINITY;
        lsum[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < DF; d++) o[i][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

#pragma unroll
    for (int st = 0; st < S - 1; st++)
        if (st < nst) issue(st);
    // query fragments (B operand), loaded while the first copies are in
    // flight.  The compiler does not see the copies; waiting for the query
    // loads with its own s_waitcnt (vmcnt 0, which also covers the copies
    // issued before them) leaves no load it tracks pending in the loop, where
    // it would otherwise wait for all loads, the copies in flight included,
    // at the first use of the fragments in every iteration.
    uint4 qf[FPW][DS];
    int limit[FPW];
#pragma unroll
    for (int i = 0; i < FPW; i++) {
        const int r = (wave * FPW + i) * 16 + l16;
        const bool ok = r < R;
        const int j = ok ? r / G : 0;
        const int hq = hkv * G + (ok ? r % G : 0);
        limit[i] = ok ? ctx + j : -1;
        const char* qp = (const char*)a.q + (((size_t)b * K1 + j) * a.n_q + hq) * DH * ESZ;
#pragma unroll
        for (int st = 0; st < DS; st++)
            qf[i][st] = ok ? ldg16(qp + (size_t)(st * 4 * KL + lg * KL) * ESZ) : make_uint4(0, 0, 0, 0);
    }

    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));   // vmcnt(0)
    for (int st = 0; st < nst; st++) {
        // this wave's copies of stage st are done once at most those of the
        // later stages in flight remain; the barrier then covers every wave's
        // copies of stage st and every wave's reads of the slot refilled below
        const int later = min(S - 2, nst - 1 - st);
        if (later >= 2) wait_vmcnt<2 * PPW>();
        else if (later == 1) wait_vmcnt<PPW>();
        else wait_vmcnt<0>();
        lds_read_barrier();
        if (st + S - 1 < nst) issue(st + S - 1);
        const uint4 (*buf)[64] = lds[st % S];
        const int kt = c0 + st * KT;
        uint4 kf[NB][DS];
#pragma unroll
        for (int blk = 0; blk < NB; blk++)
#pragma unroll
            for (int s2 = 0; s2 < DS; s2++) kf[blk][s2] = buf[blk * DS + s2][lane];
        uint4 vf[DF];
#pragma unroll
        for (int d = 0; d < DF; d++) vf[d] = buf[KP + d][lane];
        if (kt + KT > total) attn_clear_dead<true, DF>(vf, kt, lg, total);
        // every key of the tile at or before the context end: visible to every
        // row (rows past R are never written)
        const bool before_ctx = kt + KT - 1 <= ctx;
#pragma unroll
        for (int i = 0; i < FPW; i++)
            attn_tile_lazy<DH>(kf, vf, qf[i], kt, lg, limit[i], before_ctx, a.scale_log2, m_run[i], lsum[i], o[i]);
    }

#pragma unroll
    for (int i = 0; i < FPW; i++)
        // every lane group holds the whole row sum: a quarter each, which the
        // writer's sum over the four lane groups restores exactly
        attn_write_partial<DH>(a, b, hkv, chunk, wave * FPW + i, l16, lg, m_run[i], 0.25f * lsum[i][0], o[i]);
}
