// draft.h -- FastMTP drafting (Jina-OCR-v1 paper, section 3.1) on the GPU.
//
// One shared dense block B is applied recursively for K depths:
//   z(k) = P [N_e(e(next token)); N_h(a(k))],  u(k) = N_o(B(z(k); pos)),
//   draft k = argmax of W_lm u(k),
// with a(1) the target's post-norm state (the LM head's input) of a committed
// position and a(k) = u(k-1).  The embedding, N_o and W_lm are the target's.
//
// Every depth runs as one pass of the verify-shaped forward (K+1 rows per
// sequence) over a one-layer dense model whose input rows are z instead of
// an embedding:
//   depth 1: row j of sequence b is committed position ctx+j (state: the
//            verify step's row j; next token d_{j+1} for j < a, the bonus
//            token for j = a), so the block's cache receives every committed
//            position; the draft comes from row a;
//   depth k: row 0 is position ctx+a+k-1 (state u(k-1), token draft k-1);
//            rows 1..K repeat it one position further on: their cache slots
//            lie past the committed length and are rewritten by the next
//            depth-1 pass (rollback by length), so they cost time only.
// mtp_input_kernel builds the concatenated normalised rows, the projection P
// is the ordinary GEMM, and draft_pick_kernel takes the draft and the state
// of the next depth from the pass's argmax keys and final-normed rows.
#pragma once
#include "small_kernels.h"

struct DraftArgs {
    int H, K1, V, cap, k, T;      // k: the depth of this pass (1..K)
    float eps;
    const void* embed;            // [V][H] activation type
    const void* vstate;           // depth 1: the verify step's final-normed rows [T][H]
    void* ustate;                 // [B][H] u of the previous depth (written by the pick)
    const float* g_e;             // N_e gain [H]
    const float* g_h;             // N_h gain [H]
    const int* accepted;          // [B] the verify step's (-1: that step failed)
    const int* next_tok;          // [B]
    const int* drafts_in;         // [B][K] the verify step's drafts
    int* drafts_out;              // [B][K]
    const int* ctx_in;            // [B] the verify step's context lengths before it
    int* pos;                     // [B] position of row 0 of this pass (written)
    void* cat;                    // [T][2H] activation type
    int* seq_err;                 // [B]
    unsigned* err_word;
    const unsigned long long* keys;   // [NT][T] argmax keys of the pass
    int NT;
    const void* h;                // [T][H] final-normed rows of the pass
};

// A sequence left out of drafting for a reason already reported elsewhere
// (its verify step failed, or an earlier depth did): no error bits.
constexpr unsigned DRAFT_SKIP = 0x100u;

// Sequence b's error bits for depth k (token range, capacity; DRAFT_SKIP)
// and its row-0 position.
SV_DEV unsigned draft_seq_check(const DraftArgs& a, int b, int& p)
{
    const int K = a.K1 - 1, acc = a.accepted[b];
    unsigned e = 0u;
    if (acc < 0 || acc > K) {
        p = 0;
        return DRAFT_SKIP;
    }
    p = a.k == 1 ? a.ctx_in[b] : a.ctx_in[b] + acc + a.k - 1;
    if (p < 0 || (long)p + a.K1 > a.cap) e |= SV_DEV_CAPACITY;
    if (a.k == 1) {
        const int nt = a.next_tok[b];
        if (nt < 0 || nt >= a.V) e |= SV_DEV_BAD_TOKEN;
        for (int j = 0; j < acc; j++) {
            const int d = a.drafts_in[(size_t)b * K + j];
            if (d < 0 || d >= a.V) e |= SV_DEV_BAD_TOKEN;
        }
    } else {
        const int d = a.drafts_out[(size_t)b * K + a.k - 2];
        if (d < 0) e |= DRAFT_SKIP;
        else if (d >= a.V) e |= SV_DEV_BAD_TOKEN;
    }
    return e;
}

// One 256-thread workgroup per row: cat = [rms(e) g_e ; rms(state) g_h].
template <bool BF>
__global__ __launch_bounds__(256) void mtp_input_kernel(DraftArgs a)
{
    using A = Act<BF>;
    __shared__ float shw[4];
    const int t = blockIdx.x, H = a.H, K = a.K1 - 1;
    const int b = t / a.K1, j = t - b * a.K1;
    int p;
    const unsigned err = draft_seq_check(a, b, p);
    const int acc = min(max(a.accepted[b], 0), K);
    int tok;
    const typename A::T* st;
    if (a.k == 1) {
        tok = j < acc ? a.drafts_in[(size_t)b * K + j] : a.next_tok[b];
        st = (const typename A::T*)a.vstate + (size_t)t * H;
    } else {
        tok = a.drafts_out[(size_t)b * K + a.k - 2];
        st = (const typename A::T*)a.ustate + (size_t)b * H;
    }
    tok = min(max(tok, 0), a.V - 1);   // an invalid token is flagged, its row is not used
    const typename A::T* er = (const typename A::T*)a.embed + (size_t)tok * H;
    float se = 0.f, ss = 0.f;
    for (int i = threadIdx.x; i < H; i += 256) {
        const float ev = A::ld(er, i), sv = A::ld(st, i);
        se += ev * ev;
        ss += sv * sv;
    }
    se = block_sum<256>(se, shw);
    ss = block_sum<256>(ss, shw);
    const float re = rsqrtf(se / (float)H + a.eps), rs = rsqrtf(ss / (float)H + a.eps);
    typename A::T* out = (typename A::T*)a.cat + (size_t)t * 2 * H;
    for (int i = threadIdx.x; i < H; i += 256) {
        A::st(out, i, A::ld(er, i) * re * a.g_e[i]);
        A::st(out, H + i, A::ld(st, i) * rs * a.g_h[i]);
    }
    if (j == 0 && threadIdx.x == 0) {
        a.pos[b] = p;
        a.seq_err[b] = (int)err;
    }
}

// One 256-thread workgroup per sequence: the draft of depth k (the greedy
// token of row a of depth 1, row 0 of deeper depths) and that row's
// final-normed state.  Every thread issues its key loads (8 at a time,
// clamped indices) before reducing them.
template <bool BF>
__global__ __launch_bounds__(256) void draft_pick_kernel(DraftArgs a)
{
    using A = Act<BF>;
    constexpr int KB = 8;
    __shared__ unsigned long long red[4];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, K = a.K1 - 1;
    const int r = a.k == 1 ? min(max(a.accepted[b], 0), K) : 0;
    const int t = b * a.K1 + r;
    unsigned long long best = 0ull;
    for (int n0 = tid; n0 < a.NT; n0 += 256 * KB) {
        unsigned long long v[KB];
#pragma unroll
        for (int u = 0; u < KB; u++) v[u] = a.keys[(size_t)min(n0 + 256 * u, a.NT - 1) * a.T + t];
#pragma unroll
        for (int u = 0; u < KB; u++) best = umax64(best, v[u]);
    }
    best = wave_max_u64(best);
    if (lane == 0) red[tid >> 6] = best;
    __syncthreads();
    best = umax64(umax64(red[0], red[1]), umax64(red[2], red[3]));
    const bool nan = best == ~0ull;
    const bool bad = a.seq_err[b] != 0 || nan;
    const int tok = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
    if (tid == 0) {
        a.drafts_out[(size_t)b * K + a.k - 1] = bad ? -1 : tok;
        const unsigned e = ((unsigned)a.seq_err[b] & 0xffu) | (nan ? SV_DEV_NAN_LOGIT : 0u);
        if (e) atomicOr(a.err_word, e);
        if (a.k == 1 && bad) {   // the whole draft block of a failed sequence is -1
            for (int i = 1; i < K; i++) a.drafts_out[(size_t)b * K + i] = -1;
        }
    }
    const typename A::T* src = (const typename A::T*)a.h + (size_t)t * a.H;
    typename A::T* dst = (typename A::T*)a.ustate + (size_t)b * a.H;
    for (int i = tid; i < a.H; i += 256) dst[i] = src[i];
}
