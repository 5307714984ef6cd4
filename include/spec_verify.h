/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) speculative-decoding verify
 * step: greedy, and sampled (rejection sampling, spec_verify_step_sampled).
 *
 * One call runs the target decoder over the K+1 positions of every sequence
 * of a batch (the last committed token plus K draft tokens) against the
 * sequence's KV cache, takes the target's greedy token at every position,
 * keeps the longest prefix of drafts that agrees with them plus one token of
 * the target's own, and commits the new context length.
 *
 * Where the operation is defined:
 *   - Jina-OCR-v1 paper, abstract and section 3: a DeepSeekMoE decoder
 *     verifies K=3 drafts; greedy verification is lossless.
 *   - jina-ocr-v1 tweet digest, FastMTP paragraph: greedy verification keeps
 *     the longest matching prefix and the output equals ordinary greedy
 *     autoregressive decoding; 64 routed + 2 shared experts, top-6 routing.
 *   - Jina-OCR-v1 release article, L4 paragraph: tokens per verify counts the
 *     bonus token that verification brings out.
 *   - "Architecture and acceleration of an end-to-end OCR expert model",
 *     section 6.1 (verification is one teacher-forced parallel forward; accept
 *     left to right up to the first disagreement, where the target supplies
 *     the token) and section 7 (the draft / verify / accept loop).
 * The pages give no layer-level formulas; the decoder layer is the plain
 * pre-norm block: RMSNorm (eps from the config), rotary embedding with
 * rotate-half pairing (i, i + D/2) and angle pos * theta^(-2i/D), causal
 * softmax attention with scale 1/sqrt(D) where query head h reads KV head
 * floor(h * n_kv / n_q), residual add, RMSNorm, then a top-k softmax-routed
 * SwiGLU mixture of experts (gate = the selected softmax probability) plus
 * always-on shared experts, or a dense SwiGLU, residual add.  A final RMSNorm,
 * the LM head and an argmax (lowest index on ties, compared in fp32) give the
 * greedy token.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller and only
 *     borrowed for the duration of the call, except where "host" is written.
 *   - Work is enqueued on the given HIP stream (NULL = the default stream) and
 *     the call returns before the GPU finishes; outputs are valid once the
 *     caller has synchronised that stream.  No entry point synchronises the
 *     device except spec_verify_error_word and spec_verify_kernel_time.
 *   - Return value: SV_OK (0) or a negative status (see below); no exception
 *     or abort crosses the ABI.  Problems only the device can see (a token id
 *     outside the vocabulary, a context that does not leave room for K+1 new
 *     positions, a NaN logit) are reported per sequence -- accepted_len and
 *     next_tok are set to -1 and ctx_lens_out = ctx_lens_in -- and in a sticky
 *     error word read with spec_verify_error_word.
 *   - Calls that share one context must not overlap in time (they share its
 *     workspace); distinct contexts are independent.
 *
 * Storage formats:
 *   SV_F32   IEEE binary32.
 *   SV_BF16  bfloat16 (the upper 16 bits of a binary32).
 *   SV_FP8   OCP 8-bit float E4M3FN (bias 7, max 448, no infinities), with one
 *            fp32 scale per output row of every matrix: W[n][k] = code * s[n].
 *   SV_MXFP4 OCP Microscaling MXFP4 (OCP MX formats v1.0): E2M1 codes (1 sign,
 *            2 exponent bits with bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3,
 *            4, 6), two per byte (the even column in the low 4 bits), and one
 *            E8M0 scale byte 2^(s - 127) per 32 consecutive elements of a row.
 * Supported combinations: weights, embedding, activations and KV cache all
 * SV_F32; or weights SV_BF16 or SV_FP8 with embedding and KV cache SV_BF16
 * (activations bf16, accumulation fp32).  With mx_dtype = SV_MXFP4 (bf16
 * models, hidden and expert_inter multiples of 128 and at most 2048, tiled16
 * layout) the weight-streaming matrices -- MoE: w_gate_up, w_down,
 * w_sh_gate_up, w_sh_down; every model: lm_head -- are MXFP4: each
 * is the byte matrix [rows][cols/2] of codes, packed with
 * spec_verify_pack_tiled16 as an SV_FP8 matrix of cols/2 columns, and its s_x
 * pointer (lm_scale for the LM head) points to its E8M0 bytes
 * [rows][cols/32] packed with spec_verify_pack_mx_scales (an expert stack is
 * packed as one tall matrix).  The codes are widened exactly to bf16 (gfx950
 * v_cvt_scalef32_pk_bf16_fp4) and multiplied on the bf16 matrix cores.
 *
 * Weight layouts (row-major, [out][in] per matrix, contiguous):
 *   embed        [V][H]                       embedding storage type
 *   attn_norm, ffn_norm, final_norm  [H]     fp32 gains
 *   w_qkv        [(n_q + 2 n_kv) D][H]        q rows, then k rows, then v rows
 *   w_o          [H][n_q D]
 *   MoE:  w_router [E][H], w_gate_up [E][2I][H] (rows 0..I-1 gate, I..2I-1 up),
 *         w_down [E][H][I], w_sh_gate_up [S][2I][H], w_sh_down [S][H][I]
 *   dense: w_gate_up [2 I_d][H], w_down [H][I_d]
 *   lm_head      [V][H]
 *   fp8 scales: s_x has one fp32 per row of w_x, laid out like w_x without
 *   its last dimension (e.g. s_gate_up [E][2I]).
 *
 * Two layouts are accepted for the matrices that feed a matrix product
 * (w_qkv, w_o, w_gate_up, w_down, w_sh_gate_up, w_sh_down, lm_head), chosen
 * by spec_verify_weights.layout (the router w_router is always row-major: it
 * is applied inside the normalisation kernel, one row of logits per token):
 *   SV_LAYOUT_ROW_MAJOR  as above;
 *   SV_LAYOUT_TILED16    rows grouped in blocks of 16, each block stored step
 *                        by step along the reduction dimension (exact format
 *                        at spec_verify_pack_tiled16).  Every 64-lane load of a
 *                        weight fragment is then one contiguous KiB, which is
 *                        what lets the weight stream run near the HBM peak.
 * The embedding is always row-major (it is gathered by row, not multiplied).
 *
 * KV-cache layout (storage = kv dtype).  Each (sequence b, layer l, KV head h)
 * owns one contiguous region of capacity * D elements at offset
 * ((b * L + l) * n_kv + h) * capacity * D, for both the K and the V cache;
 * sequence b's regions are contiguous.  Inside a region, positions are grouped
 * in tiles of KT keys (KL = 16 / element size: 8 for bf16, 4 for fp32;
 * KT = 4 KL) and every tile is KT * D contiguous elements, made of 1 KiB
 * pieces of 64 lanes x KL elements, the exact operands of the attention's
 * matrix instructions:
 *   K: piece (blk, s) of tile t (blk < KL/4, s < D/(4 KL)) is at element
 *      ((t * KL/4 + blk) * D/(4 KL) + s) * 64 KL; lane l = q4 + 16 g (q4 < 16,
 *      g < 4) holds K[pos][d] for pos = t KT + KL (q4 / 4) + 4 blk + q4 % 4 and
 *      d = s 4 KL + g KL + e, e < KL.
 *   V: piece f of tile t (f < D/16) is at element (t * D/16 + f) * 64 KL; lane
 *      l = c + 16 g holds V[pos][d] for pos = t KT + g KL + e (e < KL) and
 *      d = 16 f + c.
 * A cache built in the natural order [pos][d] per region can be converted
 * with a pure permutation (the Python binding provides one).  Positions
 * 0 .. ctx_lens_in[b]-1 hold the cached context.  The step writes positions
 * ctx .. ctx+K; after the commit, slots at or past ctx_lens_out[b] are dead
 * and are overwritten by the next step (rollback is by length).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_VERIFY_ABI_VERSION 5

/* status codes */
#define SV_OK 0
#define SV_ERR_INVALID_ARG (-1)   /* null pointer, bad size, batch out of range */
#define SV_ERR_UNSUPPORTED (-2)   /* shape or dtype combination not supported */
#define SV_ERR_HIP (-3)           /* a HIP runtime call failed (message kept) */
#define SV_ERR_NO_DEVICE (-4)     /* no usable gfx950 device */
#define SV_ERR_NOT_SET (-5)       /* requested data was never produced */

/* storage types */
#define SV_F32 0
#define SV_BF16 1
#define SV_FP8 2
#define SV_MXFP4 3                /* expert and LM-head weights only (spec_verify_config.mx_dtype) */

/* feed-forward kinds */
#define SV_FFN_MOE 0
#define SV_FFN_DENSE 1

/* bits of the sticky device error word and of per-sequence errors */
#define SV_DEV_BAD_TOKEN 1u       /* a committed or draft token outside [0, V) */
#define SV_DEV_CAPACITY 2u        /* ctx < 0 or ctx + K + 1 > capacity */
#define SV_DEV_NAN_LOGIT 4u       /* a NaN among a position's logits */

/* weight layouts */
#define SV_LAYOUT_ROW_MAJOR 0
#define SV_LAYOUT_TILED16 1

/* kernel classes for spec_verify_kernel_time */
#define SV_KC_LM_HEAD 0           /* final norm output x LM head + argmax partials */
#define SV_KC_ATTENTION 1         /* split-KV verify attention (not the merge) */
#define SV_KC_EXPERT_GATE_UP 2    /* grouped expert gate/up + SwiGLU (MoE) or dense gate/up */
#define SV_KC_EXPERT_DOWN 3       /* grouped expert down projection (MoE) or dense down */
#define SV_KC_QKV 4               /* QKV projection */
#define SV_KC_SAMPLING 5          /* sampled verification: statistics, decision + draw, commit
                                     (three launches per step) */
#define SV_KC_COUNT 6

typedef struct spec_verify_ctx spec_verify_ctx;   /* opaque; owns only its workspace */

typedef struct {
    int n_layers;       /* L >= 1 */
    int hidden;         /* H, multiple of 64 */
    int n_q_heads;      /* n_q */
    int n_kv_heads;     /* n_kv, divides n_q */
    int head_dim;       /* D: 64 or 128 */
    int ffn_kind;       /* SV_FFN_MOE or SV_FFN_DENSE */
    int n_experts;      /* E (MoE), multiple of 4, <= 256 */
    int expert_inter;   /* I (MoE), multiple of 64 */
    int top_k;          /* k (MoE), 1 <= k <= min(E, 8) */
    int n_shared;       /* shared experts (MoE), 0..8 */
    int renorm_topk;    /* 1: gates renormalised to sum 1 over the selected experts */
    int dense_inter;    /* I_d (dense), multiple of 64 */
    int vocab;          /* V, multiple of 16 */
    int max_batch;      /* B_max: largest batch a step may be called with */
    int k_draft;        /* K >= 1 drafts per sequence */
    int kv_capacity;    /* slots per (sequence, layer, KV head), multiple of 64 */
    float rope_theta;   /* rotary base */
    float rms_eps;      /* RMSNorm epsilon */
    int weight_dtype;   /* SV_F32 / SV_BF16 / SV_FP8 */
    int embed_dtype;    /* SV_F32 / SV_BF16 */
    int kv_dtype;       /* SV_F32 / SV_BF16 */
    int mx_dtype;       /* 0, or SV_MXFP4: expert matrices and LM head in OCP MXFP4 (below) */
    int kv_page_size;   /* 0: contiguous KV regions; else positions per page (multiple of 64,
                           dividing kv_capacity): paged caches, see spec_verify_set_kv_pages */
    int kv_pool_pages;  /* paged caches: physical pages in the K (and the V) pool */
} spec_verify_config;

typedef struct {
    const float* attn_norm;
    const void* w_qkv;        const float* s_qkv;
    const void* w_o;          const float* s_o;
    const float* ffn_norm;
    const void* w_router;     const float* s_router;
    const void* w_gate_up;    const float* s_gate_up;
    const void* w_down;       const float* s_down;
    const void* w_sh_gate_up; const float* s_sh_gate_up;
    const void* w_sh_down;    const float* s_sh_down;
} spec_verify_layer;          /* s_* are used only for SV_FP8 weights (NULL otherwise) */

typedef struct {
    const void* embed;
    const spec_verify_layer* layers;   /* HOST array of n_layers entries */
    const float* final_norm;
    const void* lm_head;
    const float* lm_scale;             /* SV_FP8 only */
    int layout;                        /* SV_LAYOUT_ROW_MAJOR or SV_LAYOUT_TILED16 */
} spec_verify_weights;

/* Validate `cfg` (host), pick the kernel plan, allocate the workspace for
 * max_batch sequences and upload the rotary table (cos/sin of pos *
 * theta^(-2i/D), computed in double on the host, stored fp32) for positions
 * 0 .. kv_capacity-1.  *out receives the context.  Uses the current HIP
 * device. */
int spec_verify_init(const spec_verify_config* cfg, spec_verify_ctx** out);

/* Free the workspace.  NULL is allowed. */
void spec_verify_destroy(spec_verify_ctx* ctx);

/*
 * One verify step for sequences 0 .. batch-1 (1 <= batch <= max_batch).
 *   committed_tok [batch]       int32, the last committed token of each sequence
 *   draft_toks    [batch][K]    int32 drafts
 *   ctx_lens_in   [batch]       int32 tokens already cached
 *   ctx_lens_out  [batch]       int32 <- ctx_lens_in + accepted_len + 1 (may alias
 *                               ctx_lens_in)
 *   accepted_len  [batch]       int32 <- drafts kept, 0..K
 *   next_tok      [batch]       int32 <- the target's token after the kept drafts
 *                               (the bonus); the caller feeds it back as the next
 *                               committed token
 *   k_cache, v_cache            the caches (layout above); positions ctx..ctx+K of
 *                               every layer are written
 * The step reads and updates context lengths on the device only, so it needs no
 * host synchronisation and may be captured into a HIP graph.
 */
int spec_verify_step(spec_verify_ctx* ctx, const spec_verify_weights* w, void* k_cache,
                     void* v_cache, const int32_t* committed_tok, const int32_t* draft_toks,
                     const int32_t* ctx_lens_in, int32_t* ctx_lens_out, int batch,
                     int32_t* accepted_len, int32_t* next_tok, void* stream);

/*
 * The greedy verify step for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It needs no context: it plans the step from `cfg` and takes
 * its workspace from a static device array of the library (64 MiB, one per
 * GPU, held until the process ends); it calls no hipMalloc, hipFree or
 * allocating library routine.
 *   cfg           the model (as for spec_verify_init; kv_page_size must be 0);
 *                 max_batch picks the attention plan, as it does for a context,
 *                 so a context with the same cfg gives the same results
 *   error_word    device uint32 that receives the SV_DEV_* bits of the call
 *                 (OR-ed in; the caller clears it), or NULL
 * Other arguments, outputs and per-sequence errors as in spec_verify_step.
 * SV_ERR_UNSUPPORTED (nothing launched) when the step's workspace for this
 * batch exceeds the array, e.g. 12 layers at batch 64 with long contexts.
 * Every call on a GPU shares that GPU's array: calls that overlap in time on
 * one GPU race.  Each call rewrites the rotary table and clears its error
 * word in the array with kernels (no memset), so it may be captured into a
 * HIP graph; a replay uses the array as the captured launches left it.
 */
int spec_verify_step_noalloc(const spec_verify_config* cfg, const spec_verify_weights* w,
                             void* k_cache, void* v_cache, const int32_t* committed_tok,
                             const int32_t* draft_toks, const int32_t* ctx_lens_in,
                             int32_t* ctx_lens_out, int batch, int32_t* accepted_len,
                             int32_t* next_tok, uint32_t* error_word, void* stream);

/*
 * Paged KV caches (kv_page_size = P > 0).  Defined by: OCRia-1 technical-
 * report digest, third item of its list of things worth copying (the
 * inference stack reuses a shared prompt prefix); "Architecture and
 * acceleration of an end-to-end OCR expert model", section 9 (long contexts
 * need KV-cache management).  The k_cache / v_cache arguments of
 * the steps are then pools of kv_pool_pages physical pages: page g holds, for
 * every layer l and KV head h, P positions at element offset
 * ((g * L + l) * n_kv + h) * P * D, tiled exactly like a contiguous region of
 * P positions (the KV-cache layout above with capacity P).  `table`
 * [max_batch][kv_capacity / P] int32 (device, caller-owned, read by every
 * following step until replaced) maps logical page i of sequence b -- its
 * positions i P .. i P + P - 1 -- to a physical page.  Sequences may share
 * physical pages for a common prefix (the pages are only read); the pages
 * that receive a step's new positions ctx .. ctx+K must be the sequence's
 * own.  An entry outside [0, kv_pool_pages) that a step touches is clamped
 * into the pool and raises SV_DEV_CAPACITY in the error word (that
 * sequence's results are then meaningless).  SV_ERR_UNSUPPORTED for a
 * context without paged caches.
 */
int spec_verify_set_kv_pages(spec_verify_ctx* ctx, const int32_t* table);

/*
 * Debug outputs for the following steps (any pointer may be NULL; all NULL
 * turns them off).  logits [batch][K+1][V] fp32 (scaled logits of every
 * verified position), hidden [L][batch (K+1)][H] fp32 (residual stream after
 * each layer), target_tok [batch][K+1] int32 (greedy token of every position),
 * routing [L][batch (K+1)][top_k] int32 (MoE only: the experts each position
 * was routed to, in rank order).  Writing logits costs an extra pass of
 * V*T*4 bytes.
 */
int spec_verify_set_debug(spec_verify_ctx* ctx, float* logits, float* hidden,
                          int32_t* target_tok, int32_t* routing);

/*
 * Router debug output for the following steps (MoE models; NULL turns it
 * off): router_logits [L][batch (K+1)][E] fp32, the router's logits W_r h of
 * every position and layer (fp8 row scale applied) -- the values the top-k
 * selection of the jina-ocr-v1 tweet digest's "64 routed experts, top-6"
 * router is taken on.  SV_ERR_UNSUPPORTED for a dense model.
 */
int spec_verify_set_debug_router(spec_verify_ctx* ctx, float* router_logits);

/*
 * Acceptance and commit alone, from given fp32 logits [batch][K+1][V]
 * (device): argmax per position (lowest index on ties, NaN -> error) and the
 * same acceptance / commit as spec_verify_step.  target_tok may be NULL.
 */
int spec_verify_accept_from_logits(spec_verify_ctx* ctx, const float* logits,
                                   const int32_t* draft_toks, const int32_t* ctx_lens_in,
                                   int32_t* ctx_lens_out, int batch, int32_t* accepted_len,
                                   int32_t* next_tok, int32_t* target_tok, void* stream);

/*
 * Sampled (stochastic) verification: the same forward pass, then speculative
 * sampling instead of the greedy comparison.  "Architecture and acceleration
 * of an end-to-end OCR expert model", section 6.1, names the property:
 * verification by rejection sampling leaves the output distributed exactly
 * as the target's own decoding; section 7 gives the loop (keep the agreeing
 * prefix, the target resamples at the first disagreement).  The rule is the
 * standard one (Leviathan et al. 2023; Chen et al. 2023):
 *   p_j = softmax(logits_j / temperature), j = 0..K, the target after
 *   position j; q_i the distribution draft d_i was drawn from (i = 1..K).
 *   Draft d_i is kept while accept_u[i-1] * q_i(d_i) < p_{i-1}(d_i) (fp32),
 *   i.e. with probability min(1, p/q).  At the first failure (accepted_len =
 *   a < K) next_tok is drawn from max(0, p_a - q_{a+1}) normalised (from p_a
 *   if rounding leaves no positive entry); with every draft kept (a = K)
 *   next_tok is drawn from p_K.  ctx_lens_out = ctx_lens_in + a + 1.
 * Draws: the exponential race (Gumbel-max): the entry with the largest fp32
 * weight / E_v, the lower index on ties, where E_v = -log(uniform) and the
 * uniform comes from Philox4x32-10 (Salmon et al., SC 2011): key = seed (low
 * 32 bits first), counter = (v / 4, position j, sequence b, offset), output
 * word v % 4 -> uniform ((w >> 9) + 0.5) * 2^-23.  This is the largest
 * log-weight + Gumbel noise -log(E_v).  Pass a fresh (seed, offset) every
 * step.
 *   draft_probs  [batch][K][V] fp32, q_i of every draft position (device)
 *   accept_u     [batch][K]    fp32 uniforms in [0, 1) (device)
 *   temperature  > 0, applied to the target's logits only
 * Other arguments, outputs and per-sequence errors as in spec_verify_step
 * (a NaN logit, or a draft outside [0, V), sets the sequence's outputs to -1).
 * The LM head writes fp32 logits [batch (K+1)][V] into the context's
 * workspace (or into the debug logits buffer when one is set); the debug
 * target_tok buffer is not written.  Needs vocab <= 262144 (SV_ERR_UNSUPPORTED
 * otherwise); a temperature that is not positive and finite, or whose
 * inverse overflows, is SV_ERR_INVALID_ARG.
 */
int spec_verify_step_sampled(spec_verify_ctx* ctx, const spec_verify_weights* w, void* k_cache,
                             void* v_cache, const int32_t* committed_tok,
                             const int32_t* draft_toks, const float* draft_probs,
                             const float* accept_u, float temperature, uint64_t seed,
                             uint32_t offset, const int32_t* ctx_lens_in, int32_t* ctx_lens_out,
                             int batch, int32_t* accepted_len, int32_t* next_tok, void* stream);

/*
 * The sampled acceptance and commit alone, from given target logits
 * [batch][K+1][V] fp32 (device, before the temperature); arguments and
 * outputs as in spec_verify_step_sampled.
 */
int spec_verify_sample_from_logits(spec_verify_ctx* ctx, const float* logits,
                                   const int32_t* draft_toks, const float* draft_probs,
                                   const float* accept_u, float temperature, uint64_t seed,
                                   uint32_t offset, const int32_t* ctx_lens_in,
                                   int32_t* ctx_lens_out, int batch, int32_t* accepted_len,
                                   int32_t* next_tok, void* stream);

/*
 * FastMTP drafting (Jina-OCR-v1 paper, section 3.1; the jina-ocr-v1 tweet
 * digest: one shared dense draft block run recursively K times).  After a
 * verify step on `verify_ctx`, proposes the next step's K drafts of every
 * sequence:
 *   a(1) = the target's post-norm state (LM-head input) of a committed
 *   position, a(k) = u(k-1); z(k) = P [N_e(e(next token)); N_h(a(k))];
 *   u(k) = N_o(B(z(k); pos)); draft k = argmax_v (W_lm u(k))[v] (lowest
 *   index on ties), where N_e / N_h are RMSNorms with gains enorm / hnorm,
 *   P = eh_proj [H][2H] (column block 0 multiplies N_e(e)), B the draft
 *   block, and the embedding, N_o (the final norm) and W_lm the target's.
 * Depth 1 runs the block over the committed positions ctx .. ctx+a of the
 * verify step (a = accepted_len; next token d_{j+1} for j < a and next_tok
 * at j = a), writing the block's cache there; depth k > 1 runs at position
 * ctx+a+k-1 on the previous depth's u and draft.
 *   draft_ctx     a context made for the draft block: n_layers = 1,
 *                 SV_FFN_DENSE (dense_inter = the block's FFN width), the
 *                 target's hidden, heads, vocab, K, dtypes and mx_dtype (the
 *                 tied LM head keeps its storage); kv_capacity >=
 *                 the largest ctx + 3 (K+1) (deeper depths also fill K
 *                 slots past their position, which the next depth-1 pass
 *                 rewrites)
 *   w             the draft block as a one-layer model: layers[0] = the
 *                 block (attn_norm, w_qkv, w_o, ffn_norm, w_gate_up, w_down),
 *                 embed / final_norm / lm_head (+ lm_scale) the target's;
 *                 layout as for spec_verify_step
 *   mtp           enorm, hnorm [H] fp32; eh_proj [H][2H] in the weight
 *                 storage type and layout (+ s_eh_proj for SV_FP8)
 *   k_cache, v_cache  the block's own KV cache (layout as for the target's,
 *                 one layer)
 *   verify_ctx    the context of the verify step just run: its final-normed
 *                 rows are the states a(1) (call before its next step)
 *   ctx_in, accepted_len, next_tok, draft_toks  that verify step's inputs
 *                 and outputs ([batch] / [batch][K], device)
 *   drafts_out    [batch][K] int32 <- the next step's drafts; all -1 for a
 *                 sequence whose verify step failed (accepted_len < 0; no new
 *                 error bit) or whose tokens are out of range, and -1 from the
 *                 first depth whose K+1 rows would pass the capacity or that
 *                 meets a NaN logit (those set SV_DEV_* bits in draft_ctx's
 *                 error word); a skipped pass does not write the block cache
 * Every pass is enqueued on `stream` with no host synchronisation.
 */
typedef struct {
    const float* enorm;       /* N_e gain [H] */
    const float* hnorm;       /* N_h gain [H] */
    const void* eh_proj;      /* P [H][2H] */
    const float* s_eh_proj;   /* fp8 row scales of P [H] (SV_FP8 only) */
} spec_mtp_weights;

int spec_draft_step(spec_verify_ctx* draft_ctx, const spec_verify_weights* w,
                    const spec_mtp_weights* mtp, void* k_cache, void* v_cache,
                    const spec_verify_ctx* verify_ctx, const int32_t* ctx_in,
                    const int32_t* accepted_len, const int32_t* next_tok,
                    const int32_t* draft_toks, int batch, int32_t* drafts_out, void* stream);

/*
 * Repack one row-major matrix W[rows][cols] (device, storage `dtype`) into
 * the SV_LAYOUT_TILED16 layout at `dst` (device, caller-owned, at least
 * spec_verify_tiled16_bytes(rows, cols, dtype) bytes, not overlapping src).
 * Layout: let esize be the element size (4, 2 or 1), KL = 16 / esize and
 * S = 4 KL (the reduction step: 16, 32 or 64 elements).  Rows are padded with
 * zeros to a multiple of 16.  Row block r (rows 16r .. 16r+15) and step s
 * (columns sS .. sS+S-1) occupy the 1024 bytes at offset
 * (r * cols / S + s) * 1024; inside them, the 16 bytes at offset 16 l
 * (l = 0..63) hold W[16r + l%16][sS + (l/16) KL .. + KL-1].  cols must be a
 * multiple of S.  A stack of equally shaped matrices (experts) may be packed
 * as one tall matrix when each matrix's row count is a multiple of 16.
 * Enqueued on `stream`.
 */
int spec_verify_pack_tiled16(const void* src, void* dst, long rows, int cols, int dtype,
                             void* stream);

/* Bytes of a matrix in the SV_LAYOUT_TILED16 layout (rows padded to 16). */
long spec_verify_tiled16_bytes(long rows, int cols, int dtype);

/*
 * Repack the E8M0 block scales of an MXFP4 matrix with `cols` columns
 * (row-major bytes [rows][cols/32], device) into the form the kernels read
 * (at `dst`, device, caller-owned, spec_verify_mx_scales_bytes bytes): per
 * 16-row block and group of 16 reduction steps of 128 columns, 1024 bytes of
 * 64 lanes x 16 bytes, at offset ((block * G + group) * 64 + l) * 16 with
 * G = ceil(cols / 2048); byte j of lane l = r + 16 g is the scale of row
 * 16 block + r, column block 4 (16 group + j) + g.  Padding bytes are 127.
 * cols must be a positive multiple of 128.  Enqueued on `stream`.
 */
int spec_verify_pack_mx_scales(const void* src, void* dst, long rows, int cols, void* stream);

/* Bytes of packed MXFP4 scales for a [rows][cols] matrix (-1 if invalid). */
long spec_verify_mx_scales_bytes(long rows, int cols);

/* Read (host) the sticky device error word (SV_DEV_* bits) accumulated since
 * the last clear; synchronises `stream` first.  clear != 0 resets it. */
int spec_verify_error_word(spec_verify_ctx* ctx, uint32_t* out, int clear, void* stream);

/*
 * Kernel timing with HIP events on the launch stream.  enable = 1 starts
 * recording events around every launch of class `kclass` (SV_KC_*) and resets
 * the totals, enable = 0 stops recording, any other value leaves the state
 * as it is.  With out pointers given (before the state changes), synchronises
 * the recorded events and returns (host) the summed duration in milliseconds
 * and the number of launches timed since the last reset.  At most 8192
 * launches are recorded per reset.
 */
int spec_verify_kernel_time(spec_verify_ctx* ctx, int kclass, int enable, double* total_ms,
                            int* launches);

/* Copy (host) the message of the most recent failed call in this process
 * (validation or HIP error) into buf, NUL-terminated and truncated to len
 * bytes; returns its full length. */
int spec_verify_last_error(char* buf, int len);

/* Static description of a status code. */
const char* spec_verify_status_string(int status);

/* SPEC_VERIFY_ABI_VERSION of the built library. */
int spec_verify_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
