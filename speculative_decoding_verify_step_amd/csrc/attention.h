// attention.h -- split-KV verify attention with MFMA tiles (gfx950).
//
// For every sequence b and KV head h the verify step has R = (K+1) * G query
// rows (K+1 positions times the G = n_q / n_kv query heads that read this KV
// head; row r is position r / G, query head h*G + r % G).  Row r attends to
// cache positions 0 .. ctx_b + r/G: the cached context, then the block's own
// new positions up to itself (causal).
//
// The key range of a sequence is cut into chunks of CH keys; one wave takes
// one chunk for QPW 16-row query fragments and keeps a flash-style running
// (max, sum, output) per row, then writes the unnormalised partial.  A second
// kernel merges the partials of all chunks in chunk order.
//
// Tile shapes (KL = elements per 16-byte slice: 8 for bf16, 4 for fp32):
//   scores   S^T[key][row] = K[key][:] . Q[row][:]  -- key tile = A operand,
//            query fragment = B operand (held in registers for the chunk);
//   output   O^T[d][row] += V^T[d][keys] . P^T[keys][row] -- the probabilities
//            a lane produced by the score product are exactly its B slice:
// a 4*KL-key tile is computed as KL/4 score blocks of 16 keys whose slot s
// maps to key KL*(s/4) + 4*blk + s%4, so that lane group g ends up holding
// keys KL*g .. KL*g + KL-1 for its row.  The cache stores every tile as the
// 1 KiB operand pieces of exactly these instructions (layout documented with
// the C ABI), so each fragment load is 64 lanes x 16 contiguous bytes.
#pragma once
#include "common.h"

struct AttnArgs {
    const void* q;            // [T][n_q][D] activations (rotary applied)
    const void* kc;           // K cache, tiled (see the C ABI; a page pool when kvp.table is set)
    const void* vc;           // V cache, tiled
    KvPages kvp;
    unsigned* err_word;
    const int* ctx_in;        // [B]
    const int* seq_err;       // [B]
    int layer, L, n_q, n_kv, D, K1, cap, CH, maxch, QG;
    int B;                    // sequences in the step
    float scale_log2;         // log2(e) / sqrt(D)
    float* opart;             // [B][n_q][K1][maxch][D]
    float* mlpart;            // [B][n_q][K1][maxch][2]  (max in log2 units, sum)
};

// STREAM: the K/V tiles are read by this workgroup only (one query group per
// KV head) and are loaded with streaming (nontemporal) loads; with several
// query groups the later readers of a tile hit in L2, so normal loads stay.
// Softmax weights 2^(s - max) <= 1 with the hardware exp2 alone (v_exp_f32;
// the library exp2f adds a rescaling for results below the normal range,
// i.e. weights under 2^-126 of the row maximum).
SV_DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// The last tile of a sequence reaches past its newest written position:
// those slots were never written (or hold an older step's data) and may be
// any bit pattern.  Their probabilities are 0, but 0 * NaN or 0 * Inf in the
// output product would still poison the row, so their values are cleared
// (lane group lg holds keys kt + KL lg + e of every value fragment).
template <bool BF, int DF>
SV_DEV void attn_clear_dead(uint4 (&vf)[DF], int kt, int lg, int total)
{
    constexpr int KL = BF ? 8 : 4;
    const int nv = total - (kt + KL * lg);
    uint32_t m[4];
#pragma unroll
    for (int w = 0; w < 4; w++) {
        if constexpr (BF) m[w] = (2 * w < nv ? 0xffffu : 0u) | (2 * w + 1 < nv ? 0xffff0000u : 0u);
        else m[w] = w < nv ? 0xffffffffu : 0u;
    }
#pragma unroll
    for (int d = 0; d < DF; d++) {
        vf[d].x &= m[0];
        vf[d].y &= m[1];
        vf[d].z &= m[2];
        vf[d].w &= m[3];
    }
}

// One key tile (16 keys) of an fp32 cache for one 16-row query fragment: the
// scores, the running (max, sum) of each row and the output product.  Row
// l16's keys past `limit` (causal end; -1 for a padding row) are masked.
// (bf16 caches use attn_tile_lazy below.)
template <int DH>
SV_DEV void attn_tile_f32(const uint4 (&kf)[1][DH / 16], const uint4 (&vf)[DH / 16],
                          const uint4 (&qf)[DH / 16], int kt, int lg, int limit, float scale_log2,
                          float& m_run, float& l_run, f32x4_t (&o)[DH / 16])
{
    constexpr int KL = 4, DS = DH / 16, DF = DH / 16;
    float s[KL];
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < DS; st++) acc = mma_f32x4(kf[0][st], qf[st], acc);
#pragma unroll
    for (int r = 0; r < 4; r++) s[r] = acc[r];
    // lane (lg, l16) holds keys kt + KL*lg + e for row l16 of the fragment
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < KL; e++) {
        int key = kt + KL * lg + e;
        s[e] = (key <= limit) ? s[e] * scale_log2 : -INFINITY;
        mt = fmaxf(mt, s[e]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    float mnew = fmaxf(m_run, mt);
    float muse = (mnew == -INFINITY) ? 0.f : mnew;
    float alpha = exp2_fast(m_run - muse);
    m_run = mnew;
    float p[KL], ps = 0.f;
#pragma unroll
    for (int e = 0; e < KL; e++) { p[e] = exp2_fast(s[e] - muse); ps += p[e]; }
    l_run = l_run * alpha + ps;
    const uint4 pb = make_uint4(__float_as_uint(p[0]), __float_as_uint(p[1]), __float_as_uint(p[2]),
                                __float_as_uint(p[3]));
#pragma unroll
    for (int d = 0; d < DF; d++) {
        o[d] = o[d] * alpha;
        o[d] = mma_f32x4(vf[d], pb, o[d]);
    }
}

// Maximum over the four 16-lane rows' lanes l, l ^ 16, l ^ 32, l ^ 48 (lane
// groups lg of one query row) with the gfx950 row swaps: VALU only, no LDS
// round trip.
SV_DEV float max_over_lane_groups(float v)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}

// bf16 1.0 in every element: the A operand whose product with the weights
// gives each query row's weight sum
constexpr uint32_t BF16_ONE_X2 = 0x3f803f80u;

// One 32-key bf16 tile for one 16-row query fragment, as attn_tile_f32, with
// less vector-ALU work per score (the scores per tile are as many as the
// products' multiply-adds per 256, so the ALU is what bounds many-row tiles):
//  * the causal mask is applied only to tiles that reach past the context
//    (`nomask`: every key of the tile is visible to every row);
//  * the running maximum is a base that moves only when a row's tile maximum
//    exceeds it by more than 2^8 (lazy rescaling: weights 2^(s - base) stay
//    below 2^8, exact in bf16's range and fp32 sums); the output and sum are
//    rescaled only then, for the rows whose base moved;
//  * the 1/sqrt(D) scale folds into the exponent's fused multiply-add;
//  * the weight sum is one more matrix product, of the bf16 weights with a
//    fragment of ones (`lsum`: every lane of query row l16 holds the row's
//    sum), so the sum adds up exactly the rounded weights the output
//    product uses;
//  * maxima are plain float max instructions.
// The partial (base, sum, output) means the same as attn_tile_f32's.
template <int DH>
SV_DEV void attn_tile_lazy(const uint4 (&kf)[2][DH / 32], const uint4 (&vf)[DH / 16],
                           const uint4 (&qf)[DH / 32], int kt, int lg, int limit, bool nomask,
                           float scale_log2, float& m_run, f32x4_t& lsum, f32x4_t (&o)[DH / 16])
{
    constexpr int KL = 8, DS = DH / 32, DF = DH / 16, NB = 2;
    constexpr float TAU = 8.f;
    float s[KL];
#pragma unroll
    for (int blk = 0; blk < NB; blk++) {
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < DS; st++) acc = mma_bf16(kf[blk][st], qf[st], acc);
#pragma unroll
        for (int r = 0; r < 4; r++) s[4 * blk + r] = acc[r];
    }
    if (!nomask) {
        const int rel = limit - (kt + KL * lg);   // score e is visible when e <= rel
#pragma unroll
        for (int e = 0; e < KL; e++) s[e] = (e <= rel) ? s[e] : -INFINITY;
    }
    float mt = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mt = max_over_lane_groups(mt) * scale_log2;      // the scale is positive
    const bool grow = mt > m_run + TAU;              // also from an empty (-inf) base
    if (__any(grow)) {
        const float mnew = grow ? mt : m_run;
        const float alpha = grow ? exp2_fast(m_run - mnew) : 1.f;
        m_run = mnew;
        lsum = lsum * alpha;
#pragma unroll
        for (int d = 0; d < DF; d++) o[d] = o[d] * alpha;
    }
    const float nbase = (m_run == -INFINITY) ? 0.f : -m_run;
    float p[KL];
#pragma unroll
    for (int e = 0; e < KL; e++) p[e] = exp2_fast(fmaf(s[e], scale_log2, nbase));
    const uint4 pb = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
    lsum = mma_bf16(make_uint4(BF16_ONE_X2, BF16_ONE_X2, BF16_ONE_X2, BF16_ONE_X2), pb, lsum);
#pragma unroll
    for (int d = 0; d < DF; d++) o[d] = mma_bf16(vf[d], pb, o[d]);
}

// Partial of one chunk for one 16-row query fragment (row r = 16 f + l16 of
// the KV head's R rows): O^T[d = 16 df + 4 lg + i][row l16] and (max, sum).
template <int DH>
SV_DEV void attn_write_partial(const AttnArgs& a, int b, int hkv, int chunk, int f, int l16, int lg,
                               float m_run, float l_run, const f32x4_t (&o)[DH / 16])
{
    constexpr int DF = DH / 16;
    const int K1 = a.K1, G = a.n_q / a.n_kv, R = K1 * G;
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int r = f * 16 + l16;
    if (r >= R) return;
    const int j = r / G, hq = hkv * G + r % G;
    const size_t slot = (((size_t)b * a.n_q + hq) * K1 + j) * a.maxch + chunk;
    float* op = a.opart + slot * DH;
#pragma unroll
    for (int d = 0; d < DF; d++)
        *reinterpret_cast<float4*>(op + 16 * d + 4 * lg) = make_float4(o[d][0], o[d][1], o[d][2], o[d][3]);
    if (lg == 0) *reinterpret_cast<float2*>(a.mlpart + slot * 2) = make_float2(m_run, l);
}

// With streaming loads (one reader per tile, caches far beyond the Infinity
// Cache) at most two waves per SIMD: more concurrent streams measured slower
// (batch 64: 254 us per layer at two, 283 us at three).
template <bool BF, int QPW, int DH, bool STREAM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, STREAM ? 2 : 8))) void attn_split_kernel(AttnArgs a)
{
    constexpr int ESZ = BF ? 2 : 4;
    constexpr int KL = BF ? 8 : 4;          // elements per 16-byte slice
    constexpr int KT = 4 * KL;              // keys per tile
    constexpr int DS = DH / (4 * KL);       // reduction steps over the head dimension
    constexpr int DF = DH / 16;             // output fragments over the head dimension
    constexpr int NB = KL / 4;              // 16-key score blocks per tile

    const int lane = threadIdx.x, l16 = lane & 15, lg = lane >> 4;
    // grid: with one query group per KV head (chunk, KV head, sequence).  With
    // QG > 1 groups a 1-D grid: the work items u = (sequence, KV head, chunk)
    // in blocks of 8, x = (u / 8, query group, u % 8), so that the groups
    // reading one K/V tile are 8 workgroups apart -- on the same XCD
    // (workgroups go to the 8 XCDs round-robin), where the later readers find
    // the tile in that XCD's L2 instead of fetching it from HBM again -- and
    // every XCD gets the same share of the work items
    int chunk, qgi, hkv, b;
    if (a.QG > 1) {
        const int x = blockIdx.x;
        const int u = (x / (8 * a.QG)) * 8 + (x & 7);
        if (u >= a.B * a.n_kv * a.maxch) return;   // padding of the last block of 8
        qgi = (x >> 3) % a.QG;
        chunk = u % a.maxch;
        hkv = (u / a.maxch) % a.n_kv;
        b = u / (a.maxch * a.n_kv);
    } else {
        chunk = blockIdx.x;
        qgi = 0;
        hkv = blockIdx.y;
        b = blockIdx.z;
    }
    const int K1 = a.K1, G = a.n_q / a.n_kv, R = K1 * G;
    const int c0 = chunk * a.CH;
    // paged caches: lane i holds the physical page of this chunk's i-th page,
    // loaded once (its index needs only the chunk, so the load overlaps the
    // context-length load); each tile takes its page with a cross-lane read
    const bool paged = a.kvp.table != nullptr;
    const int pg0 = paged ? c0 / a.kvp.page : 0;
    int my_page = 0;
    if (paged) my_page = a.kvp.table[(size_t)b * a.kvp.max_pages + min(pg0 + lane, a.kvp.max_pages - 1)];
    const int ctx = min(max(a.ctx_in[b], 0), a.cap - K1);
    const int total = ctx + K1;
    if (c0 >= total) return;
    const int c1 = min(c0 + a.CH, total);

    const size_t head = ((size_t)b * a.L + a.layer) * a.n_kv + hkv;
    const char* kbase = (const char*)a.kc + head * (size_t)a.cap * DH * ESZ + lane * 16;
    const char* vbase = (const char*)a.vc + head * (size_t)a.cap * DH * ESZ + lane * 16;
    constexpr size_t TILE = (size_t)KT * DH * ESZ;     // bytes per key tile
    if (paged) {
        const bool bad = pg0 + lane <= (c1 - 1) / a.kvp.page && (my_page < 0 || my_page >= a.kvp.n_pages);
        if (__any(bad) && lane == 0) atomicOr(a.err_word, SV_DEV_CAPACITY);
        my_page = min(max(my_page, 0), a.kvp.n_pages - 1);
    }
    const size_t page_bytes = paged ? (size_t)a.kvp.page * DH * ESZ : 0;

    // query fragments (B operand): lane supplies row l16, slice lg of each step
    uint4 qf[QPW][DS];
    int limit[QPW];
#pragma unroll
    for (int f = 0; f < QPW; f++) {
        int r = (qgi * QPW + f) * 16 + l16;
        bool ok = r < R;
        int j = ok ? r / G : 0;
        int hq = hkv * G + (ok ? r % G : 0);
        limit[f] = ok ? ctx + j : -1;
        const char* qp = (const char*)a.q + (((size_t)b * K1 + j) * a.n_q + hq) * DH * ESZ;
#pragma unroll
        for (int s = 0; s < DS; s++) {
            qf[f][s] = ok ? ldg16(qp + (size_t)(s * 4 * KL + lg * KL) * ESZ) : make_uint4(0, 0, 0, 0);
        }
    }

    float m_run[QPW], l_run[QPW];
    f32x4_t lsum[QPW], o[QPW][DF];   // bf16: row sums as products (lsum), fp32: l_run
#pragma unroll
    for (int f = 0; f < QPW; f++) {
        m_run[f] = -INFINITY;
        l_run[f] = 0.f;
        lsum[f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < DF; d++) o[f][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    auto kvload = [&](const char* p) {
        if constexpr (STREAM) return ldg16_stream(p);
        else return ldg16(p);
    };
    for (int kt = c0; kt < c1; kt += KT) {
        const char* kt_k;
        const char* kt_v;
        if (paged) {
            const int pg = __shfl(my_page, kt / a.kvp.page - pg0, 64);
            const size_t off = (((size_t)pg * a.L + a.layer) * a.n_kv + hkv) * page_bytes +
                               (size_t)((kt % a.kvp.page) / KT) * TILE + lane * 16;
            kt_k = (const char*)a.kc + off;
            kt_v = (const char*)a.vc + off;
        } else {
            const size_t toff = (size_t)(kt / KT) * TILE;
            kt_k = kbase + toff;
            kt_v = vbase + toff;
        }
        // key tile (A operand of the score product): lane (slot l16, slice lg)
        uint4 kf[NB][DS];
#pragma unroll
        for (int blk = 0; blk < NB; blk++)
#pragma unroll
            for (int s = 0; s < DS; s++) kf[blk][s] = kvload(kt_k + (size_t)(blk * DS + s) * 1024);
        // value tile (A operand of the output product): lane (channel 16 df + l16, keys KL lg ..)
        uint4 vf[DF];
#pragma unroll
        for (int d = 0; d < DF; d++) vf[d] = kvload(kt_v + (size_t)d * 1024);
        if (kt + KT > total) attn_clear_dead<BF, DF>(vf, kt, lg, total);
        // every key of the tile at or before the context end: visible to every
        // row of the block (rows past R are never written)
        const bool before_ctx = kt + KT - 1 <= ctx;
#pragma unroll
        for (int f = 0; f < QPW; f++) {
            if constexpr (BF)
                attn_tile_lazy<DH>(kf, vf, qf[f], kt, lg, limit[f], before_ctx, a.scale_log2, m_run[f], lsum[f], o[f]);
            else
                attn_tile_f32<DH>(kf, vf, qf[f], kt, lg, limit[f], a.scale_log2, m_run[f], l_run[f], o[f]);
        }
    }

#pragma unroll
    for (int f = 0; f < QPW; f++)
        attn_write_partial<DH>(a, b, hkv, chunk, qgi * QPW + f, l16, lg, m_run[f],
                               BF ? 0.25f * lsum[f][0] : l_run[f], o[f]);
}

// Merge the chunk partials of one (sequence, query head, position) row in
// chunk order and write the attention output row in the activation type.
// One wave merges two rows, a half-wave each; lane i of a half owns channels
// 4i .. 4i+3 (D/4 lanes) and chunk weights i, i + 32, ...  The partial
// outputs of the first CB chunks (16-byte loads, indices clamped so that the
// loads carry no conditions) are issued together with the chunk (max, sum)
// pairs, so one memory round trip follows the context-length read.  CB and
// NI (= ceil(maxch / 32)) are chosen from the chunk count at launch.
SV_DEV float half_max(float v)
{
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

SV_DEV float half_sum(float v)
{
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);   // fixed pairing order
    return v;
}

template <bool BF, int CB, int NI>
__global__ __launch_bounds__(64) void attn_merge_kernel(AttnArgs a, void* out /* [T][n_q*D] */, int rows)
{
    __shared__ float wgt[2][32 * NI];
    const int lane = threadIdx.x, half = lane >> 5, l32 = lane & 31;
    const int row = min(blockIdx.x * 2 + half, rows - 1);   // ((b * n_q + hq) * K1 + j)
    const bool live = blockIdx.x * 2 + half < rows;
    const int K1 = a.K1, D = a.D;
    const int j = row % K1;
    const int hq = (row / K1) % a.n_q;
    const int b = row / (K1 * a.n_q);
    const int ctx = min(max(a.ctx_in[b], 0), a.cap - K1);
    const int nch = (ctx + K1 + a.CH - 1) / a.CH;   // 1 .. maxch <= 32 NI
    const float2* __restrict__ ml = reinterpret_cast<const float2*>(a.mlpart) + (size_t)row * a.maxch;
    const float* __restrict__ op = a.opart + (size_t)row * a.maxch * D;
    const int cg = min(l32, D / 4 - 1);             // channel group (lanes past D/4 repeat the last)
    float4 ov[CB];
#pragma unroll
    for (int c = 0; c < CB; c++)
        ov[c] = *reinterpret_cast<const float4*>(op + (size_t)min(c, nch - 1) * D + 4 * cg);
    float2 mv[NI];
#pragma unroll
    for (int i = 0; i < NI; i++) mv[i] = ml[min(l32 + 32 * i, nch - 1)];
#pragma unroll
    for (int i = 0; i < NI; i++) mv[i] = l32 + 32 * i < nch ? mv[i] : make_float2(-INFINITY, 0.f);
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < NI; i++) M = fmaxf(M, mv[i].x);
    M = half_max(M);
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < NI; i++) {
        const float wc = (mv[i].x == -INFINITY) ? 0.f : exp2_fast(mv[i].x - M);
        wgt[half][l32 + 32 * i] = wc;
        L += wc * mv[i].y;
    }
    L = half_sum(L);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const float* w = wgt[half];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int c = 0; c < CB; c++) {
        const float wc = c < nch ? w[c] : 0.f;
        acc.x += wc * ov[c].x; acc.y += wc * ov[c].y; acc.z += wc * ov[c].z; acc.w += wc * ov[c].w;
    }
    for (int c0 = CB; c0 < nch; c0 += CB) {
#pragma unroll
        for (int c = 0; c < CB; c++)
            ov[c] = *reinterpret_cast<const float4*>(op + (size_t)min(c0 + c, nch - 1) * D + 4 * cg);
#pragma unroll
        for (int c = 0; c < CB; c++) {
            const float wc = c0 + c < nch ? w[c0 + c] : 0.f;
            acc.x += wc * ov[c].x; acc.y += wc * ov[c].y; acc.z += wc * ov[c].z; acc.w += wc * ov[c].w;
        }
    }
    if (!live || l32 >= D / 4) return;
    const float inv = 1.f / L;
    const size_t t = (size_t)b * K1 + j;
    const size_t o = t * (size_t)a.n_q * D + (size_t)hq * D + 4 * cg;
    if constexpr (BF) {
        *reinterpret_cast<uint2*>((uint16_t*)out + o) =
            make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
    } else {
        *reinterpret_cast<float4*>((float*)out + o) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
}
