// common.h -- device helpers shared by the verify-step kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#define SV_DEV __device__ __forceinline__

// ----------------------------------------------------------------- formats
SV_DEV float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
// fp32 -> bf16, round to nearest even (one v_cvt_pk_bf16_f32 per pair on
// gfx950); NaN stays NaN.
SV_DEV uint32_t f32_to_bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

SV_DEV uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    const bf16x2_v v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// One OCP e4m3fn byte -> the fp32 with the same value.  The 7 magnitude bits
// are placed at the bottom of the fp32 exponent field and the top of its
// mantissa, which reads as 2^(e-127) * 1.mmm (or 2^-126 * 0.mmm when e = 0);
// multiplying by 2^120 rebases the exponent from bias 127 to bias 7.  Exact;
// the two NaN codes (magnitude 0x7f) give NaN.
SV_DEV float e4m3_to_f32(uint32_t c)
{
    float f = __uint_as_float(((c & 0x7fu) << 20) | ((c & 0x80u) << 24));
    return (c & 0x7fu) == 0x7fu ? __builtin_nanf("") : f * 0x1p120f;
}

// Two e4m3fn bytes (bits 0-7 and 8-15 of w, or 16-31 with HI) -> two packed
// bf16.  gfx950 converts OCP fp8 in one instruction; with a unit scale the
// result is exact (every e4m3fn value has at most 4 significant bits) and the
// NaN codes stay NaN.
template <bool HI>
SV_DEV uint32_t e4m3x2_to_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// 16 e4m3fn bytes -> 16 bf16 as two 16-byte operands (elements 0-7, 8-15).
SV_DEV void e4m3x16_to_bf16(uint4 w, uint4& lo, uint4& hi)
{
    lo.x = e4m3x2_to_bf16x2<false>(w.x);
    lo.y = e4m3x2_to_bf16x2<true>(w.x);
    lo.z = e4m3x2_to_bf16x2<false>(w.y);
    lo.w = e4m3x2_to_bf16x2<true>(w.y);
    hi.x = e4m3x2_to_bf16x2<false>(w.z);
    hi.y = e4m3x2_to_bf16x2<true>(w.z);
    hi.z = e4m3x2_to_bf16x2<false>(w.w);
    hi.w = e4m3x2_to_bf16x2<true>(w.w);
}

// ------------------------------------------------------------------- MFMA
// 16x16 output tiles, fp32 accumulate.  Lane l holds output rows
// 4*(l/16) .. +3 of column l%16.  Operand lanes: lane l supplies row l%16
// of A (column l%16 of B) and a slice of the reduction index chosen by l/16;
// A and B always use the same slice mapping, so the reduction covers every
// index exactly once.
SV_DEV f32x4_t mma_bf16(uint4 a, uint4 b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 32x32 output tiles (16-step reduction), fp32 accumulate.  Operand lane l
// supplies row l%32 of A (column l%32 of B) and reduction elements
// 8*(l/32) .. +7 of its 16-byte slice; register r of lane l holds output row
// 8*(r/4) + 4*(l/32) + r%4 of column l%32.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
SV_DEV f32x16_t mma32_bf16(uint4 a, uint4 b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// four 16x16x4 fp32 products, element e of each lane's 16-byte slice in step e
SV_DEV f32x4_t mma_f32x4(uint4 a, uint4 b, f32x4_t c)
{
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
}

SV_DEV uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// streamed once: keep weights from displacing reusable lines
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
SV_DEV uint4 ldg16_stream(const void* p)
{
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- argmax
// Order-preserving key of (value, index): larger value wins, then the lower
// index; a NaN value maps to the all-ones key so it wins every comparison
// and is detected after the reduction.
SV_DEV unsigned long long argmax_key(float v, uint32_t idx)
{
    if (v != v) return ~0ull;
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)u << 32) | (unsigned long long)(0xffffffffu - idx);
}

SV_DEV unsigned long long umax64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

SV_DEV unsigned long long shfl_xor_u64(unsigned long long v, int m)
{
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = __shfl_xor(lo, m, 64);
    hi = __shfl_xor(hi, m, 64);
    return ((unsigned long long)hi << 32) | lo;
}

// Wave-wide reductions with DPP (row_shr 1, 2, 4, 8 inside each 16-lane row,
// then row_bcast15 / row_bcast31 across rows, then a read of lane 63): no LDS
// round trips (a __shfl_xor butterfly compiles to one ds_bpermute per step).
// Fixed order, so deterministic; the result is returned in every lane.
template <int CTRL, int RM>
SV_DEV float dpp_f32(float old, float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, RM, 0xf, false));
}

template <int CTRL, int RM>
SV_DEV uint32_t dpp_u32(uint32_t old, uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, RM, 0xf, false);
}

enum { DPP_SHR1 = 0x111, DPP_SHR2 = 0x112, DPP_SHR4 = 0x114, DPP_SHR8 = 0x118,
       DPP_BCAST15 = 0x142, DPP_BCAST31 = 0x143 };

SV_DEV float lane63(float v) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63)); }

SV_DEV float wave_sum(float v)
{
    v += dpp_f32<DPP_SHR1, 0xf>(0.f, v);
    v += dpp_f32<DPP_SHR2, 0xf>(0.f, v);
    v += dpp_f32<DPP_SHR4, 0xf>(0.f, v);
    v += dpp_f32<DPP_SHR8, 0xf>(0.f, v);
    v += dpp_f32<DPP_BCAST15, 0xa>(0.f, v);
    v += dpp_f32<DPP_BCAST31, 0xc>(0.f, v);
    return lane63(v);
}

SV_DEV float wave_max(float v)
{
    v = fmaxf(v, dpp_f32<DPP_SHR1, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<DPP_SHR2, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<DPP_SHR4, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<DPP_SHR8, 0xf>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<DPP_BCAST15, 0xa>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<DPP_BCAST31, 0xc>(-INFINITY, v));
    return lane63(v);
}

template <int CTRL, int RM>
SV_DEV unsigned long long dpp_max_u64(unsigned long long v)
{
    const uint32_t lo = dpp_u32<CTRL, RM>(0u, (uint32_t)v), hi = dpp_u32<CTRL, RM>(0u, (uint32_t)(v >> 32));
    return umax64(v, ((unsigned long long)hi << 32) | lo);
}

SV_DEV unsigned long long wave_max_u64(unsigned long long v)
{
    v = dpp_max_u64<DPP_SHR1, 0xf>(v);
    v = dpp_max_u64<DPP_SHR2, 0xf>(v);
    v = dpp_max_u64<DPP_SHR4, 0xf>(v);
    v = dpp_max_u64<DPP_SHR8, 0xf>(v);
    v = dpp_max_u64<DPP_BCAST15, 0xa>(v);
    v = dpp_max_u64<DPP_BCAST31, 0xc>(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((unsigned long long)hi << 32) | lo;
}

template <int CTRL, int RM>
SV_DEV unsigned long long dpp_or_u64(unsigned long long v)
{
    const uint32_t lo = dpp_u32<CTRL, RM>(0u, (uint32_t)v), hi = dpp_u32<CTRL, RM>(0u, (uint32_t)(v >> 32));
    return v | (((unsigned long long)hi << 32) | lo);
}

SV_DEV unsigned long long wave_or_u64(unsigned long long v)
{
    v = dpp_or_u64<DPP_SHR1, 0xf>(v);
    v = dpp_or_u64<DPP_SHR2, 0xf>(v);
    v = dpp_or_u64<DPP_SHR4, 0xf>(v);
    v = dpp_or_u64<DPP_SHR8, 0xf>(v);
    v = dpp_or_u64<DPP_BCAST15, 0xa>(v);
    v = dpp_or_u64<DPP_BCAST31, 0xc>(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((unsigned long long)hi << 32) | lo;
}

// Routing implied by the selections (few assignments: A = T * topk <= 64,
// E <= 64), without a permutation pass.  The permuted order is the stable
// counting sort of the assignments by expert: assignment j with expert e sits
// at slot (number of assignments with a smaller expert) + (number of earlier
// assignments with expert e).  Tiles 0 .. n_shared - 1 are the shared experts,
// each over all T rows (they need no selection, so their workgroups start
// loading weights at once); tile n_shared + i is the i-th expert present in
// ascending order.  `sv` is lane l's selection (any value for l >= A; not
// used for a shared tile).
struct ImpliedTile { int group, row0, nrows; unsigned long long members; };

SV_DEV ImpliedTile implied_tile(int sv, int A, int T, int E, int n_shared, int tile)
{
    const int lane = threadIdx.x & 63;
    const bool act = lane < A;
    ImpliedTile r{0, 0, 0, 0ull};
    if (tile < n_shared) {
        r.group = E + tile;
        r.row0 = A + tile * T;
        r.nrows = T;
        return r;
    }
    tile -= n_shared;
    const unsigned long long present = wave_or_u64(act ? 1ull << sv : 0ull);
    const int distinct = __popcll(present);
    if (tile < distinct) {
        const bool bit = (present >> lane) & 1ull;
        const int pre = __popcll(present & ((1ull << lane) - 1ull));
        const int e = __builtin_ctzll(__ballot(bit && pre == tile));
        r.group = e;
        r.row0 = __popcll(__ballot(act && sv < e));
        r.members = __ballot(act && sv == e);
        r.nrows = __popcll(r.members);
    }
    return r;
}

// slot of assignment j (uniform) given every lane's selection
SV_DEV int implied_slot(int sv, int A, int j)
{
    const int lane = threadIdx.x & 63;
    const bool act = lane < A;
    const int e = __builtin_amdgcn_readlane(sv, j);
    return __popcll(__ballot(act && sv < e)) + __popcll(__ballot(act && sv == e && lane < j));
}

SV_DEV float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// Selection order of the routing: larger probability first, then the lower
// expert index (a NaN probability above every number).  The probability part
// is an order-preserving 32-bit key (0 for an empty slot); ties are broken by
// the lowest index with a wave vote.
SV_DEV uint32_t route_hi(float v)
{
    if (v != v) return 0xffffffffu;
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The probability a key was made from (exact; NaN for NaN).
SV_DEV float route_hi_value(uint32_t hi)
{
    if (hi == 0xffffffffu) return __uint_as_float(0x7fc00000u);
    return __uint_as_float((hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi);
}

template <int CTRL, int RM>
SV_DEV uint32_t dpp_max_u32(uint32_t v)
{
    const uint32_t o = dpp_u32<CTRL, RM>(0u, v);
    return o > v ? o : v;
}

SV_DEV uint32_t wave_max_u32(uint32_t v)
{
    v = dpp_max_u32<DPP_SHR1, 0xf>(v);
    v = dpp_max_u32<DPP_SHR2, 0xf>(v);
    v = dpp_max_u32<DPP_SHR4, 0xf>(v);
    v = dpp_max_u32<DPP_SHR8, 0xf>(v);
    v = dpp_max_u32<DPP_BCAST15, 0xa>(v);
    v = dpp_max_u32<DPP_BCAST31, 0xc>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Softmax over the E logits of row t (lane l holds experts l + 64 q) in fp32,
// top-k by probability with the lower expert index first on ties, gates = the
// selected probabilities (optionally renormalised, summed in rank order).  One
// wave, k <= 8.  The r-th choice is the largest remaining probability key
// (a DPP maximum over the wave), the lowest expert holding it (a wave vote),
// which then drops out: k rounds.  Outputs sel and gate_out [T][k] (dbg_sel,
// sel_lds if given).
SV_DEV void router_select_to(int E, int k, bool renorm, int t, float (&p)[4], int* sel, float* gate_out,
                             int* dbg_sel, unsigned short* sel_lds)
{
    const int lane = threadIdx.x & 63;
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; q++) m = fmaxf(m, p[q]);
    m = wave_max(m);
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        p[q] = (lane + 64 * q < E) ? __expf(p[q] - m) : 0.f;
        sum += p[q];
    }
    sum = wave_sum(sum);
    const float inv = 1.f / sum;
    uint32_t hi[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        p[q] *= inv;
        hi[q] = lane + 64 * q < E ? route_hi(p[q]) : 0u;
    }
    float pr[8];
#pragma unroll
    for (int r = 0; r < 8; r++) {
        pr[r] = 0.f;
        if (r < k) {
            uint32_t mx = hi[0] > hi[1] ? hi[0] : hi[1];
            const uint32_t m23 = hi[2] > hi[3] ? hi[2] : hi[3];
            mx = wave_max_u32(mx > m23 ? mx : m23);
            // the lowest expert e = lane + 64 q holding the maximum
            int e = 0x7fffffff;
#pragma unroll
            for (int q = 3; q >= 0; q--) {
                const unsigned long long b = __ballot(hi[q] == mx);
                if (b) e = 64 * q + __builtin_ctzll(b);
            }
            pr[r] = route_hi_value(mx);
#pragma unroll
            for (int q = 0; q < 4; q++) hi[q] = lane + 64 * q == e ? 0u : hi[q];
            if (lane == 0) {
                sel[t * k + r] = e;
                if (sel_lds) sel_lds[t * k + r] = (unsigned short)e;
                if (dbg_sel) dbg_sel[t * k + r] = e;
            }
        }
    }
    if (lane < k) {
        float gsum = 0.f;
#pragma unroll
        for (int rr = 0; rr < 8; rr++) gsum += rr < k ? pr[rr] : 0.f;   // in rank order
        float pe = pr[0];
#pragma unroll
        for (int rr = 1; rr < 8; rr++) pe = lane == rr ? pr[rr] : pe;
        gate_out[t * k + lane] = renorm ? pe / gsum : pe;
    }
}

// The selections of up to four rows at once when E <= 64 (lane e holds
// expert e of every row): router_select_to's arithmetic for each row, the
// four rows' dependent reductions interleaved (independent DPP chains).
SV_DEV void router_select_rows4(int E, int k, bool renorm, int T, const float (&lv)[4], int* sel,
                                float* gate_out)
{
    const int lane = threadIdx.x & 63;
    float m[4], e[4];
#pragma unroll
    for (int t = 0; t < 4; t++) m[t] = fmaxf(-INFINITY, lane < E ? lv[t] : -INFINITY);   // as router_select_to
#define SV_ROWS4_MAX(CTRL, RM)                                                              \
    _Pragma("unroll") for (int t = 0; t < 4; t++) m[t] = fmaxf(m[t], dpp_f32<CTRL, RM>(-INFINITY, m[t]));
    SV_ROWS4_MAX(DPP_SHR1, 0xf) SV_ROWS4_MAX(DPP_SHR2, 0xf) SV_ROWS4_MAX(DPP_SHR4, 0xf)
    SV_ROWS4_MAX(DPP_SHR8, 0xf) SV_ROWS4_MAX(DPP_BCAST15, 0xa) SV_ROWS4_MAX(DPP_BCAST31, 0xc)
#undef SV_ROWS4_MAX
#pragma unroll
    for (int t = 0; t < 4; t++) {
        m[t] = lane63(m[t]);
        e[t] = lane < E ? __expf(lv[t] - m[t]) : 0.f;
    }
    float sum[4];
#pragma unroll
    for (int t = 0; t < 4; t++) sum[t] = 0.f + e[t];
#define SV_ROWS4_SUM(CTRL, RM)                                                              \
    _Pragma("unroll") for (int t = 0; t < 4; t++) sum[t] += dpp_f32<CTRL, RM>(0.f, sum[t]);
    SV_ROWS4_SUM(DPP_SHR1, 0xf) SV_ROWS4_SUM(DPP_SHR2, 0xf) SV_ROWS4_SUM(DPP_SHR4, 0xf)
    SV_ROWS4_SUM(DPP_SHR8, 0xf) SV_ROWS4_SUM(DPP_BCAST15, 0xa) SV_ROWS4_SUM(DPP_BCAST31, 0xc)
#undef SV_ROWS4_SUM
    uint32_t hi[4];
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const float inv = 1.f / lane63(sum[t]);
        hi[t] = lane < E ? route_hi(e[t] * inv) : 0u;
    }
    float pr[4][8];
#pragma unroll
    for (int r = 0; r < 8; r++) {
        if (r < k) {
            uint32_t mx[4];
#pragma unroll
            for (int t = 0; t < 4; t++) mx[t] = hi[t];
#define SV_ROWS4_UMAX(CTRL, RM)                                                             \
            _Pragma("unroll") for (int t = 0; t < 4; t++) mx[t] = dpp_max_u32<CTRL, RM>(mx[t]);
            SV_ROWS4_UMAX(DPP_SHR1, 0xf) SV_ROWS4_UMAX(DPP_SHR2, 0xf) SV_ROWS4_UMAX(DPP_SHR4, 0xf)
            SV_ROWS4_UMAX(DPP_SHR8, 0xf) SV_ROWS4_UMAX(DPP_BCAST15, 0xa) SV_ROWS4_UMAX(DPP_BCAST31, 0xc)
#undef SV_ROWS4_UMAX
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)mx[t], 63);
                const int ew = __builtin_ctzll(__ballot(hi[t] == b));   // the lowest expert holding it
                pr[t][r] = route_hi_value(b);
                hi[t] = lane == ew ? 0u : hi[t];
                if (lane == 0 && t < T) sel[t * k + r] = ew;
            }
        } else {
#pragma unroll
            for (int t = 0; t < 4; t++) pr[t][r] = 0.f;
        }
    }
    if (lane < k) {
#pragma unroll
        for (int t = 0; t < 4; t++) {
            if (t >= T) break;
            float gsum = 0.f;
#pragma unroll
            for (int rr = 0; rr < 8; rr++) gsum += rr < k ? pr[t][rr] : 0.f;   // in rank order
            float pe = pr[t][0];
#pragma unroll
            for (int rr = 1; rr < 8; rr++) pe = lane == rr ? pr[t][rr] : pe;
            gate_out[t * k + lane] = renorm ? pe / gsum : pe;
        }
    }
}

// ---------------------------------------------------------------- paged KV
// With a page table the cache of (sequence b, layer l, KV head h) is split in
// pages of `page` positions: table [B][max_pages] holds physical page indices
// into a pool [n_pages][L][n_kv][page][D], every (page, layer, head) block
// tiled like a contiguous region of `page` positions.  Without a table the
// region of (b, l, h) holds `cap` positions.  An index outside the pool is
// clamped (no access leaves the pool) and reported through `bad`.
struct KvPages {
    const int* table;     // [B][max_pages], or nullptr: contiguous regions
    int page, max_pages, n_pages;
};

// Element offset of the (page or region, layer l, head 0) block that holds
// position pos of sequence b, and the position inside it (`pin`); the head's
// block is at + h * span * D with span = page (paged) or cap.
SV_DEV size_t kv_block(const KvPages& p, int b, int L, int l, int n_kv, int cap, int D, int pos,
                       int& pin, int& span, bool& bad)
{
    if (!p.table) {
        pin = pos;
        span = cap;
        return ((size_t)b * L + l) * n_kv * (size_t)cap * D;
    }
    const int pi = min(max(pos / p.page, 0), p.max_pages - 1);
    int pg = p.table[(size_t)b * p.max_pages + pi];
    bad = bad || pg < 0 || pg >= p.n_pages;
    pg = min(max(pg, 0), p.n_pages - 1);
    pin = pos - pi * p.page;
    span = p.page;
    return ((size_t)pg * L + l) * n_kv * (size_t)p.page * D;
}
