// spec_verify.hip -- host runtime and C ABI of the verify step (see
// include/spec_verify.h for the contract).  The runtime validates arguments,
// owns one workspace per context, plans split factors and tile shapes from the
// batch size, and enqueues the kernels of one step on the caller's stream:
//
//   embed + norm
//   per layer: QKV GEMM -> rotary + KV append -> split-KV attention -> merge
//              -> O GEMM -> residual + norm
//              -> MoE: router GEMM -> routing -> grouped gate/up (SwiGLU)
//                      -> grouped down -> combine + residual + norm
//              -> dense: gate/up (SwiGLU) -> down -> residual + norm
//   LM-head GEMM with argmax epilogue -> acceptance + commit
//   (sampled verification: the LM head also writes fp32 logits, then tile
//   statistics -> acceptance decision + draw -> commit, sampling.h)
//
// Nothing here reads device memory back: context lengths, routing and
// acceptance stay on the device, so a step can be captured in a HIP graph.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "attention.h"
#include "common.h"
#include "gemm.h"
#include "gemm_lds.h"
#include "attention_lds.h"
#include "small_kernels.h"
#include "qkv_rope.h"
#include "sampling.h"
#include "draft.h"

namespace {

std::mutex g_err_mu;
std::string g_err;

int fail(int code, const std::string& msg)
{
    std::lock_guard<std::mutex> lk(g_err_mu);
    g_err = msg;
    return code;
}

#define HIP_TRY(expr)                                                                      \
    do {                                                                                   \
        hipError_t e_ = (expr);                                                            \
        if (e_ != hipSuccess)                                                              \
            return fail(SV_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));   \
    } while (0)

constexpr int KS_MAX = 16;           // largest K split
constexpr int ATT_MAXCH_CAP = 1024;  // chunks per sequence (merge kernel weights in LDS)

inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

int wsteps(int wt)
{
    return wt == SV_F32 ? 16 : (wt == SV_BF16 ? 32 : (wt == SV_FP8 ? 64 : 128));
}

struct EventPair {
    hipEvent_t a, b;
};

// Events of the launch being timed (set by ProfScope).  A timed kernel is
// launched with hipExtLaunchKernelGGL, which stamps the start and end of the
// kernel itself into the events as part of its dispatch, so timing adds no
// packets (and no gaps) to the stream.
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;

template <typename... KArgs, typename... Args>
void launch(void (*k)(KArgs...), dim3 grid, dim3 block, size_t shm, hipStream_t s, Args... args)
{
    if (g_ev_start) hipExtLaunchKernelGGL(k, grid, block, (uint32_t)shm, s, g_ev_start, g_ev_stop, 0, args...);
    else hipLaunchKernelGGL(k, grid, block, shm, s, args...);
}

}  // namespace

struct spec_verify_ctx {
    spec_verify_config c;
    int device = 0;
    int T_max = 0, K1 = 0, QKV = 0, QD = 0;
    bool bf = true;
    int att_CH = 256, att_maxch = 1, att_QPW = 1, att_QG = 1;
    bool att_stream = false;
    int att_lds_nw = 0;   // > 0: attn_lds_kernel with this many waves per workgroup
    // workspace
    std::vector<void*> allocs;
    float* x = nullptr;
    float* x2 = nullptr;        // residual after the attention half (MoE: written by the router kernel)
    void* h = nullptr;
    float* parts = nullptr;
    size_t parts_elems = 0;
    void* q = nullptr;
    void* o = nullptr;
    float* opart = nullptr;
    float* mlpart = nullptr;
    float2* rope = nullptr;
    float* logits_g = nullptr;  // router logits shared between a row's workgroups
    int* sel = nullptr;
    float* gate = nullptr;
    int* slot = nullptr;
    int* perm_tok = nullptr;
    int* tiles = nullptr;
    int* n_tiles = nullptr;
    void* act = nullptr;
    float* y = nullptr;
    unsigned long long* keys = nullptr;
    size_t keys_elems = 0;
    int* seq_err = nullptr;
    unsigned* err_word = nullptr;
    // sampled verification (sampling.h); s_ntile = 0: vocabulary too large for it
    int s_ntile = 0;
    float* slogits = nullptr;
    float2* sstats = nullptr;
    unsigned long long* sdkeys = nullptr;
    unsigned long long* sfkeys = nullptr;
    int* sdecision = nullptr;
    // FastMTP drafting (draft.h): concatenated input rows, a zero residual,
    // row-0 positions of a pass, the state carried between depths
    void* dcat = nullptr;
    float* dzero = nullptr;
    int* dpos = nullptr;
    void* dstate = nullptr;
    // paged KV caches: page table [max_batch][kv_capacity / kv_page_size] (device)
    const int* kv_table = nullptr;
    // debug outputs
    float* dbg_logits = nullptr;
    float* dbg_hidden = nullptr;
    int* dbg_target = nullptr;
    int* dbg_routing = nullptr;
    float* dbg_rlogits = nullptr;
    // kernel timing
    int prof_class = -1;
    std::vector<EventPair> prof_events;
    size_t prof_used = 0;
};

namespace {

template <typename T>
int dalloc(spec_verify_ctx* c, T** p, size_t elems)
{
    void* v = nullptr;
    size_t bytes = std::max<size_t>(elems * sizeof(T), 256);
    HIP_TRY(hipMalloc(&v, bytes));
    c->allocs.push_back(v);
    *p = (T*)v;
    return SV_OK;
}

int validate_config(const spec_verify_config& c)
{
    auto bad = [](const char* m) { return fail(SV_ERR_UNSUPPORTED, m); };
    if (c.n_layers < 1 || c.hidden < 64 || c.hidden % 64 || c.hidden > 8192)
        return bad("hidden must be a multiple of 64 in [64, 8192] and n_layers >= 1");
    if (c.n_q_heads < 1 || c.n_kv_heads < 1 || c.n_q_heads % c.n_kv_heads)
        return bad("n_kv_heads must divide n_q_heads");
    if (c.head_dim != 64 && c.head_dim != 128) return bad("head_dim must be 64 or 128");
    if (c.vocab < 16 || c.vocab % 16) return bad("vocab must be a positive multiple of 16");
    if (c.k_draft < 1 || c.k_draft + 1 > 64) return bad("k_draft must be in [1, 63]");
    if (c.max_batch < 1) return bad("max_batch must be >= 1");
    if (c.kv_capacity < c.k_draft + 1 || c.kv_capacity % 64)
        return bad("kv_capacity must be a multiple of 64 and >= K+1");
    bool f32 = c.weight_dtype == SV_F32;
    if (f32) {
        if (c.embed_dtype != SV_F32 || c.kv_dtype != SV_F32)
            return bad("fp32 weights need fp32 embedding and KV cache");
    } else if (c.weight_dtype == SV_BF16 || c.weight_dtype == SV_FP8) {
        if (c.embed_dtype != SV_BF16 || c.kv_dtype != SV_BF16)
            return bad("bf16/fp8 weights need bf16 embedding and KV cache");
    } else {
        return bad("unknown weight dtype");
    }
    int step = wsteps(c.weight_dtype);
    if (c.hidden % step || (c.n_q_heads * c.head_dim) % step)
        return bad("hidden and n_q*head_dim must be multiples of the weight step");
    if (c.ffn_kind == SV_FFN_MOE) {
        if (c.n_experts < 1 || c.n_experts > 256) return bad("n_experts must be in [1, 256]");
        if (c.top_k < 1 || c.top_k > 8 || c.top_k > c.n_experts) return bad("bad top_k");
        if (c.expert_inter < 64 || c.expert_inter % 64 || c.expert_inter % step)
            return bad("expert_inter must be a multiple of 64");
        if (c.n_shared < 0 || c.n_shared > 8) return bad("n_shared must be in [0, 8]");
        if (c.n_experts % 4) return bad("n_experts must be a multiple of 4");
        long T = (long)c.max_batch * (c.k_draft + 1);
        if (T * c.n_experts > 32768) return bad("max_batch*(K+1)*n_experts must be <= 32768");
        // the permutation's shared memory: T (E + top_k) 2 bytes + 6.2 KB <= 80 KB
        if (((T * (c.n_experts + c.top_k) * 2 + 15) & ~15L) + 1024 * 4 + 525 * 4 > 81920)
            return bad("max_batch*(K+1)*(n_experts+top_k) too large for the routing permutation");
    } else if (c.ffn_kind == SV_FFN_DENSE) {
        if (c.dense_inter < 64 || c.dense_inter % 64 || c.dense_inter % step)
            return bad("dense_inter must be a multiple of 64");
    } else {
        return bad("unknown ffn_kind");
    }
    if (c.kv_page_size != 0) {
        if (c.kv_page_size < 64 || c.kv_page_size % 64 || c.kv_capacity % c.kv_page_size)
            return bad("kv_page_size must be a multiple of 64 that divides kv_capacity");
        if (c.kv_pool_pages < 1) return bad("kv_pool_pages must be >= 1");
    }
    if (c.mx_dtype != 0) {
        if (c.mx_dtype != SV_MXFP4) return bad("mx_dtype must be 0 or SV_MXFP4");
        if (c.weight_dtype != SV_BF16)
            return bad("MXFP4 expert and LM-head weights need a bf16 model");
        const bool moe = c.ffn_kind == SV_FFN_MOE;
        if (c.hidden % 128 || c.hidden > 2048 || (moe && (c.expert_inter % 128 || c.expert_inter > 2048)))
            return bad("MXFP4 weights need hidden and expert_inter multiples of 128, at most 2048");
    }
    return SV_OK;
}

// ------------------------------------------------------------- GEMM launch
template <int WT, int MODE, bool PK>
void launch_gemm_t(int MF, const GemmArgs& a, dim3 grid, hipStream_t s)
{
    if (a.tiles) {
        // grouped (experts): one 16-column tile per workgroup; gate/up one wave,
        // down (K = expert_inter, shorter rows) its reduction shared by 2 waves
        if constexpr (MODE == GM_SWIGLU) {
            switch (MF) {
            case 1: launch(gemm_kernel<WT, 1, 1, MODE, 1, 0, PK>, grid, dim3(64), 0, s, a); break;
            case 2: launch(gemm_kernel<WT, 2, 1, MODE, 1, 0, PK>, grid, dim3(64), 0, s, a); break;
            default: launch(gemm_kernel<WT, 4, 1, MODE, 1, 0, PK>, grid, dim3(64), 0, s, a); break;
            }
        } else if constexpr (MODE == GM_STORE) {
            switch (MF) {
            case 1: launch(gemm_kernel<WT, 1, 1, MODE, 2, 8, PK, true>, grid, dim3(128), 0, s, a); break;
            case 2: launch(gemm_kernel<WT, 2, 1, MODE, 2, 4, PK, true>, grid, dim3(128), 0, s, a); break;
            default: launch(gemm_kernel<WT, 4, 1, MODE, 2, 2, PK, true>, grid, dim3(128), 0, s, a); break;
            }
        }
        return;
    }
    switch (MF) {
    case 1: launch(gemm_kernel<WT, 1, 1, MODE, 4, 0, PK>, grid, dim3(256), 0, s, a); break;
    case 2: launch(gemm_kernel<WT, 2, 1, MODE, 4, 0, PK>, grid, dim3(256), 0, s, a); break;
    default: launch(gemm_kernel<WT, 4, 1, MODE, 4, 0, PK>, grid, dim3(256), 0, s, a); break;
    }
}

// MXFP4 weights (a quarter of the bf16 bytes per column): wider wave tiles so
// that a wave still streams enough bytes.  LM head: 2 column fragments per
// wave (128-column workgroup tiles; same-box step 81.4 us with 4, 79.8 with
// 2, 88.0 with 8), 2 steps per stage on the general kernel.
// Grouped experts: gate/up one column fragment per wave as with bf16 (at
// batch 1 wider tiles leave too few waves: 11.7 -> 13.2 us with two), down 4
// (its 2 waves split the reduction; 9.2 -> 8.6 us), 2 steps per stage.
constexpr int MX_LM_NF = 2, MX_LM_U = 2, MX_GU_NF = 1, MX_DN_NF = 4;
constexpr int MX_LDS_MAXS = 10;   // reduction steps (128 columns each) the LDS kernel holds

int small_col_tile(int wt, int mode) { return (wt == SV_MXFP4 && mode == GM_ARGMAX) ? 64 * MX_LM_NF : 64; }

// columns of one grouped-expert workgroup tile on the small-row kernel
int grouped_col_tile(int wt, int mode)
{
    if (wt != SV_MXFP4) return 16;
    return 16 * (mode == GM_SWIGLU ? MX_GU_NF : MX_DN_NF);
}

template <int MODE>
void launch_gemm_mx(int MF, const GemmArgs& a, dim3 grid, hipStream_t s)
{
    constexpr int WT = SV_MXFP4;
    if (a.tiles || a.sel) {   // grouped experts: the bf16 variants' shapes (2 steps per stage)
        if constexpr (MODE == GM_SWIGLU) {
            switch (MF) {
            case 1: launch(gemm_kernel<WT, 1, MX_GU_NF, MODE, 1, 0, true>, grid, dim3(64), 0, s, a); break;
            case 2: launch(gemm_kernel<WT, 2, MX_GU_NF, MODE, 1, 0, true>, grid, dim3(64), 0, s, a); break;
            default: launch(gemm_kernel<WT, 4, MX_GU_NF, MODE, 1, 0, true>, grid, dim3(64), 0, s, a); break;
            }
        } else if constexpr (MODE == GM_STORE) {
            switch (MF) {
            case 1: launch(gemm_kernel<WT, 1, MX_DN_NF, MODE, 2, 2, true, true>, grid, dim3(128), 0, s, a); break;
            case 2: launch(gemm_kernel<WT, 2, MX_DN_NF, MODE, 2, 1, true, true>, grid, dim3(128), 0, s, a); break;
            default: launch(gemm_kernel<WT, 4, MX_DN_NF, MODE, 2, 1, true, true>, grid, dim3(128), 0, s, a); break;
            }
        }
        return;
    }
    if constexpr (MODE == GM_ARGMAX) {
        // up to 16 rows and K <= 1280: whole reduction in flight, activations in LDS
        if (MF == 1 && a.K <= 128 * MX_LDS_MAXS) {
            launch(gemm_mx_lds_kernel<MX_LM_NF, MX_LDS_MAXS, MODE>, grid, dim3(256), 0, s, a);
            return;
        }
        switch (MF) {
        case 1: launch(gemm_kernel<WT, 1, MX_LM_NF, MODE, 4, MX_LM_U, true>, grid, dim3(256), 0, s, a); break;
        case 2: launch(gemm_kernel<WT, 2, MX_LM_NF, MODE, 4, 1, true>, grid, dim3(256), 0, s, a); break;
        default: launch(gemm_kernel<WT, 4, MX_LM_NF, MODE, 4, 1, true>, grid, dim3(256), 0, s, a); break;
        }
    }
}

template <int MODE, bool PK>
void launch_gemm_m(int wt, int MF, const GemmArgs& a, dim3 grid, hipStream_t s)
{
    if (wt == SV_F32) launch_gemm_t<SV_F32, MODE, PK>(MF, a, grid, s);
    else if (wt == SV_BF16) launch_gemm_t<SV_BF16, MODE, PK>(MF, a, grid, s);
    else if (wt == SV_FP8) launch_gemm_t<SV_FP8, MODE, PK>(MF, a, grid, s);
    else if constexpr (PK) launch_gemm_mx<MODE>(MF, a, grid, s);   // tiled16 only
}

template <bool PK>
void launch_gemm_l(int wt, int mode, int MF, const GemmArgs& a, dim3 grid, hipStream_t s)
{
    if (mode == GM_STORE) launch_gemm_m<GM_STORE, PK>(wt, MF, a, grid, s);
    else if (mode == GM_SWIGLU) launch_gemm_m<GM_SWIGLU, PK>(wt, MF, a, grid, s);
    else launch_gemm_m<GM_ARGMAX, PK>(wt, MF, a, grid, s);
}

void launch_gemm(int wt, int mode, int MF, bool packed, GemmArgs& a, hipStream_t s)
{
    dim3 grid((unsigned)(cdiv(a.NT, 8) * 8 * a.MT), (unsigned)a.ksplit, 1);
    if (packed) launch_gemm_l<true>(wt, mode, MF, a, grid, s);
    else launch_gemm_l<false>(wt, mode, MF, a, grid, s);
}

// Large-row path: 128-row workgroup tiles (MF 8) of 128 columns (NF 2); the
// projections (STORE: QKV, O, down, N of a few thousand) take 64-column
// tiles, twice the workgroups (batch 32: 2,334 -> 2,315 us per step, the O
// projection having had 40 workgroups).
constexpr int BIG_MF = 8, BIG_NF = 2, BIG_CHUNK_STEPS = 2;
constexpr int big_nf(int mode) { return mode == GM_STORE ? 1 : BIG_NF; }

template <int MODE, bool PK>
void launch_big_m(int wt, const GemmArgs& a, dim3 grid, hipStream_t s)
{
    // (fp32 weights never take the large-row path: it needs bf16 or fp8 weights)
    constexpr int NF = big_nf(MODE);
    if (wt == SV_BF16) launch(gemm_bigm_kernel<SV_BF16, BIG_MF, NF, MODE, PK>, grid, dim3(256), 0, s, a);
    else if (wt == SV_FP8) launch(gemm_bigm_kernel<SV_FP8, BIG_MF, NF, MODE, PK>, grid, dim3(256), 0, s, a);
    else if constexpr (PK) {
        if (wt == SV_MXFP4) launch(gemm_bigm_kernel<SV_MXFP4, BIG_MF, NF, MODE, PK>, grid, dim3(256), 0, s, a);
    }
}

// Grouped (expert) GEMMs on the large-row kernel: MF row fragments per tile,
// one column fragment per wave (64-column workgroup tiles: twice the
// workgroups of the dense tiles, measured 7-8% faster at 12-row experts).
constexpr int GROUPED_NF = 1;

template <int MODE, bool PK, int MF>
void launch_grouped_mf(int wt, const GemmArgs& a, dim3 grid, hipStream_t s)
{
    if (wt == SV_BF16) launch(gemm_bigm_kernel<SV_BF16, MF, GROUPED_NF, MODE, PK>, grid, dim3(256), 0, s, a);
    else if (wt == SV_FP8) launch(gemm_bigm_kernel<SV_FP8, MF, GROUPED_NF, MODE, PK>, grid, dim3(256), 0, s, a);
    else if constexpr (PK) launch(gemm_bigm_kernel<SV_MXFP4, MF, GROUPED_NF, MODE, PK>, grid, dim3(256), 0, s, a);
}

template <int MODE, bool PK>
void launch_grouped_m(int wt, int MF, const GemmArgs& a, dim3 grid, hipStream_t s)
{
    if (MF == 1) launch_grouped_mf<MODE, PK, 1>(wt, a, grid, s);
    else if (MF == 2) launch_grouped_mf<MODE, PK, 2>(wt, a, grid, s);
    else launch_grouped_mf<MODE, PK, 4>(wt, a, grid, s);
}

void launch_grouped_big(int wt, int mode, int MF, bool packed, GemmArgs& a, hipStream_t s)
{
    dim3 grid((unsigned)(cdiv(a.NT, 8) * 8 * a.MT), 1, 1);
    if (packed) {
        if (mode == GM_SWIGLU) launch_grouped_m<GM_SWIGLU, true>(wt, MF, a, grid, s);
        else launch_grouped_m<GM_STORE, true>(wt, MF, a, grid, s);
    } else {
        if (mode == GM_SWIGLU) launch_grouped_m<GM_SWIGLU, false>(wt, MF, a, grid, s);
        else launch_grouped_m<GM_STORE, false>(wt, MF, a, grid, s);
    }
}

void launch_gemm_big(int wt, int mode, bool packed, GemmArgs& a, hipStream_t s)
{
    dim3 grid((unsigned)(cdiv(a.NT, 8) * 8 * a.MT), (unsigned)a.ksplit, 1);
    if (packed) {
        if (mode == GM_STORE) launch_big_m<GM_STORE, true>(wt, a, grid, s);
        else if (mode == GM_SWIGLU) launch_big_m<GM_SWIGLU, true>(wt, a, grid, s);
        else launch_big_m<GM_ARGMAX, true>(wt, a, grid, s);
    } else {
        if (mode == GM_STORE) launch_big_m<GM_STORE, false>(wt, a, grid, s);
        else if (mode == GM_SWIGLU) launch_big_m<GM_SWIGLU, false>(wt, a, grid, s);
        else launch_big_m<GM_ARGMAX, false>(wt, a, grid, s);
    }
}

// Dense large-row GEMMs with packed weights (fp8, or bf16 above 128 rows): 32x32 MFMA tiles, a
// wave owns 64 rows x 64 columns (SwiGLU: 32 gate + the 32 matching up
// columns), four waves side by side.  Measured at 256 rows against the
// 128-row tiles above: fp8 gate/up 75 -> 51 us, LM head 314 -> 266 us; bf16
// LM head 152 -> 126 us.
constexpr int WIDE_MW = 2, WIDE_NW = 2, WIDE_WAVES = 4;

int wide_col_tile(int mode) { return 32 * WIDE_WAVES * (mode == GM_SWIGLU ? WIDE_NW / 2 : WIDE_NW); }

// Steps per staged chunk: 2, except the fp8 LM head with 1 (three waves per
// SIMD instead of two: 273 -> 262 us per launch at 256 rows, same box).
// fp8 projections whose K split holds 16 or more 64-long reduction steps
// (the planner then takes the most such splits within 512 workgroups: dense
// fp8 QKV 2 x 20, O 4 x 16, down 8 x 19 steps) run the same 64 x 256 tiles on
// the LDS-staged kernel with 3 stages (two steps in flight per workgroup
// without registers): dense fp8 K = 31, down 41.3 -> 32.1 us per layer (step
// 1,904 -> 1,833 us, same box).  Splits of 8 steps, the fp8 SwiGLU (47.5 ->
// 52.1 us per layer), the fp8 LM head (265 -> 272 us) and bf16 at 256 rows
// (QKV and O of batch 64: 208 -> 220 us per step) measured no faster there.
constexpr int WIDE_LDS_MIN_STEPS = 16;

template <int WT>
void launch_wide_t(int mode, const GemmArgs& a, dim3 grid, hipStream_t s)
{
    const dim3 blk(64 * WIDE_WAVES);
    if (mode == GM_STORE) {
        if constexpr (WT == SV_FP8) {
            const int span = a.K / a.ksplit;
            if (span >= WIDE_LDS_MIN_STEPS * WTraits<WT>::SK && span % WTraits<WT>::SK == 0) {
                launch(gemm_lds_kernel<WT, GM_STORE, 1, WIDE_MW, 3, WIDE_NW>, grid, blk, 0, s, a);
                return;
            }
        }
        launch(gemm_wide_kernel<WT, WIDE_MW, WIDE_NW, GM_STORE, WIDE_WAVES, 2>, grid, blk, 0, s, a);
    } else if (mode == GM_SWIGLU) {
        launch(gemm_wide_kernel<WT, WIDE_MW, WIDE_NW, GM_SWIGLU, WIDE_WAVES, 2>, grid, blk, 0, s, a);
    } else {
        // LM head: fp8 one reduction step per chunk, bf16 two
        constexpr int CS = WT == SV_FP8 ? 1 : 2;
        launch(gemm_wide_kernel<WT, WIDE_MW, WIDE_NW, GM_ARGMAX, WIDE_WAVES, CS>, grid, blk, 0, s, a);
    }
}

void launch_gemm_wide(int wt, int mode, GemmArgs& a, hipStream_t s)
{
    dim3 grid((unsigned)(cdiv(a.NT, 8) * 8 * a.MT), (unsigned)a.ksplit, 1);
    if (wt == SV_BF16) launch_wide_t<SV_BF16>(mode, a, grid, s);
    else launch_wide_t<SV_FP8>(mode, a, grid, s);
}

// bf16 LM head at 65 .. 256 rows: both operands staged in LDS, tiles of 8
// waves (gemm_lds.h).  129 .. 256 rows: 256 x 256 tiles, 4 stages.  65 .. 128
// rows: 128 x 512 tiles, 3 stages (120 KB), so each activation row is copied
// once per 512 columns (batch 32: LM head 86.6 -> 72.5 us per launch, step
// 2,301.7 -> 2,283.5 us against the register-staged 128 x 128 tiles, same box)
int lm_head_lds_cols(int T) { return T <= 128 ? 512 : 256; }

void launch_lm_head_lds(const GemmArgs& a, hipStream_t s)
{
    dim3 grid((unsigned)(cdiv(a.NT * a.MT, 8) * 8), 1, 1), blk(512);
    if (a.M <= 128) launch(gemm_lds_kernel<SV_BF16, GM_ARGMAX, 2, 2, 3, 4>, grid, blk, 0, s, a);
    else launch(gemm_lds_kernel<SV_BF16, GM_ARGMAX, 2, 4, 4>, grid, blk, 0, s, a);
}

// merge: CB partials per load batch, NI = ceil(maxch / 32) chunk weights per lane
template <bool BF>
void launch_merge_t(int maxch, const AttnArgs& at, void* out, int rows, hipStream_t s)
{
    dim3 grid((unsigned)cdiv(rows, 2)), blk(64);
    if (maxch <= 8) launch(attn_merge_kernel<BF, 8, 1>, grid, blk, 0, s, at, out, rows);
    else if (maxch <= 16) launch(attn_merge_kernel<BF, 16, 1>, grid, blk, 0, s, at, out, rows);
    else if (maxch <= 32) launch(attn_merge_kernel<BF, 32, 1>, grid, blk, 0, s, at, out, rows);
    else if (maxch <= 64) launch(attn_merge_kernel<BF, 32, 2>, grid, blk, 0, s, at, out, rows);
    else if (maxch <= 256) launch(attn_merge_kernel<BF, 32, 8>, grid, blk, 0, s, at, out, rows);
    else launch(attn_merge_kernel<BF, 32, 32>, grid, blk, 0, s, at, out, rows);
}

void launch_merge(bool bf, int maxch, const AttnArgs& at, void* out, int rows, hipStream_t s)
{
    if (bf) launch_merge_t<true>(maxch, at, out, rows, s);
    else launch_merge_t<false>(maxch, at, out, rows, s);
}

int rows_mf(int rows) { return rows <= 16 ? 1 : (rows <= 32 ? 2 : 4); }

void launch_attention_lds(int D, int NW, dim3 grid, const AttnArgs& at, hipStream_t s)
{
    constexpr int FPW = 2, S = 4;
#define ATT_LDS(DH)                                                                                   \
    switch (NW) {                                                                                     \
    case 1: launch(attn_lds_kernel<DH, FPW, 1, S>, grid, dim3(64), 0, s, at); break;                  \
    case 2: launch(attn_lds_kernel<DH, FPW, 2, S>, grid, dim3(128), 0, s, at); break;                 \
    case 4: launch(attn_lds_kernel<DH, FPW, 4, S>, grid, dim3(256), 0, s, at); break;                 \
    default: launch(attn_lds_kernel<DH, FPW, 8, S>, grid, dim3(512), 0, s, at); break;                \
    }
    if (D == 128) { ATT_LDS(128) } else { ATT_LDS(64) }
#undef ATT_LDS
}

template <bool BF, int DH, bool ST>
void launch_attention_t(int QPW, dim3 grid, const AttnArgs& at, hipStream_t s)
{
    if constexpr (BF) {
        // bf16 caches with 17 .. 256 rows per KV head take the LDS-ring kernel,
        // so the split kernel sees one fragment per wave, or four above 256
        // rows (several query groups, never streamed); the plan checks this
        if constexpr (!ST) {
            if (QPW == 4) {
                launch(attn_split_kernel<BF, 4, DH, false>, grid, dim3(64), 0, s, at);
                return;
            }
        }
        launch(attn_split_kernel<BF, 1, DH, ST>, grid, dim3(64), 0, s, at);
    } else {
        if (QPW == 4) launch(attn_split_kernel<BF, 4, DH, ST>, grid, dim3(64), 0, s, at);
        else if (QPW == 2) launch(attn_split_kernel<BF, 2, DH, ST>, grid, dim3(64), 0, s, at);
        else launch(attn_split_kernel<BF, 1, DH, ST>, grid, dim3(64), 0, s, at);
    }
}

// split-KV attention; streaming K/V loads when each tile has one reader
void launch_attention(bool bf, int D, int QPW, bool stream, dim3 grid, const AttnArgs& at, hipStream_t s)
{
#define ATT_CASE(BF, DH)                                                     \
    if (stream) launch_attention_t<BF, DH, true>(QPW, grid, at, s);          \
    else launch_attention_t<BF, DH, false>(QPW, grid, at, s);
    if (bf) {
        if (D == 128) { ATT_CASE(true, 128) } else { ATT_CASE(true, 64) }
    } else {
        if (D == 128) { ATT_CASE(false, 128) } else { ATT_CASE(false, 64) }
    }
#undef ATT_CASE
}

// Fused attention input (few rows): 8 waves split each column pair's
// reduction; 5 steps per prefetch stage for one row fragment (one stage at
// hidden 1280 bf16), fewer stages and, for four fragments, 4 waves (registers).
constexpr int QKV_W = 8;

template <int WT, bool PK, bool EMB>
void launch_qkv_rope_t(int MF, const QkvArgs& a, dim3 grid, hipStream_t s)
{
    switch (MF) {
    case 1: launch(qkv_rope_kernel<WT, 1, QKV_W, 5, PK, EMB>, grid, dim3(64 * QKV_W), 0, s, a); break;
    case 2: launch(qkv_rope_kernel<WT, 2, QKV_W, 3, PK, EMB>, grid, dim3(64 * QKV_W), 0, s, a); break;
    default: launch(qkv_rope_kernel<WT, 4, 4, 2, PK, EMB>, grid, dim3(256), 0, s, a); break;   // registers
    }
}

void launch_qkv_rope(int wt, int MF, bool packed, bool embed, const QkvArgs& a, hipStream_t s)
{
    dim3 grid((unsigned)(cdiv(a.NT, 8) * 8 * a.MT));
#define QKV_CASE(WT)                                                              \
    if (packed) {                                                                 \
        if (embed) launch_qkv_rope_t<WT, true, true>(MF, a, grid, s);             \
        else launch_qkv_rope_t<WT, true, false>(MF, a, grid, s);                  \
    } else {                                                                      \
        if (embed) launch_qkv_rope_t<WT, false, true>(MF, a, grid, s);            \
        else launch_qkv_rope_t<WT, false, false>(MF, a, grid, s);                 \
    }
    if (wt == SV_F32) { QKV_CASE(SV_F32) }
    else if (wt == SV_BF16) { QKV_CASE(SV_BF16) }
    else { QKV_CASE(SV_FP8) }
#undef QKV_CASE
}

// Rotary + cache append over the K-split partials of the QKV projection: the
// kernel instance with the fewest loads per channel that covers the splits
template <bool BF>
void launch_rope_append(dim3 grid, hipStream_t s, const RopeArgs& rp)
{
    if (rp.nsplit <= 1) rope_append_kernel<BF, 1><<<grid, 64, 0, s>>>(rp);
    else if (rp.nsplit <= 2) rope_append_kernel<BF, 2><<<grid, 64, 0, s>>>(rp);
    else if (rp.nsplit <= 4) rope_append_kernel<BF, 4><<<grid, 64, 0, s>>>(rp);
    else if (rp.nsplit <= 8) rope_append_kernel<BF, 8><<<grid, 64, 0, s>>>(rp);
    else rope_append_kernel<BF, 16><<<grid, 64, 0, s>>>(rp);
}

// Residual update + RMSNorm of every row: the kernel instance with the fewest
// loads per column that covers the K-split partials (dense) or the shared
// experts' outputs (MoE combine)
template <bool BF, bool MOE>
void launch_residual_norm(int T, hipStream_t s, const RowArgs& ra)
{
    const int n = MOE ? ra.n_shared : ra.nsplit;   // shared experts <= 8, splits <= 16
    if (n <= 1) residual_norm_kernel<BF, MOE, false, 4, 1><<<T, 1024, 0, s>>>(ra);
    else if (n <= 2) residual_norm_kernel<BF, MOE, false, 4, 2><<<T, 1024, 0, s>>>(ra);
    else if (n <= 4) residual_norm_kernel<BF, MOE, false, 4, 4><<<T, 1024, 0, s>>>(ra);
    else if (MOE || n <= 8) residual_norm_kernel<BF, MOE, false, 4, 8><<<T, 1024, 0, s>>>(ra);
    else if constexpr (!MOE) residual_norm_kernel<BF, MOE, false, 4, 16><<<T, 1024, 0, s>>>(ra);
}

// K split: enough waves to cover the GPU, each split at least 4 reduction steps
int pick_ksplit(long waves, int K, int step, int smax = KS_MAX)
{
    int steps = K / step, best = 1;
    for (int s = 1; s <= smax; s++) {
        if (steps % s) continue;
        if (steps / s < 4) break;
        best = s;
        if (waves * s >= 2048) break;
    }
    return best;
}

GemmArgs dense_args(const void* X, long ldx, int M, int N, int K, const void* W, const float* ws)
{
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.X = X;
    a.ldx = ldx;
    a.M = M;
    a.N = N;
    a.K = K;
    a.ksplit = 1;
    a.W = W;
    a.ws = ws;
    a.G1 = 1;
    return a;
}

// event-timed launch scope
// Times the one kernel launched inside the scope if its class is recorded.
struct ProfScope {
    ProfScope(spec_verify_ctx* c, int kc, hipStream_t)
    {
        if (c->prof_class == kc && c->prof_used < c->prof_events.size()) {
            size_t idx = c->prof_used++;
            g_ev_start = c->prof_events[idx].a;
            g_ev_stop = c->prof_events[idx].b;
        }
    }
    ~ProfScope() { g_ev_start = g_ev_stop = nullptr; }
};

// One depth of FastMTP drafting run through the step (draft.h).
struct DraftPass {
    DraftArgs args;           // pass-invariant fields; k, keys, h, NT, T set per pass
    const void* P;            // eh_proj [H][2H]
    const float* sP;          // its fp8 row scales
};

struct SampleIn {
    const float* q;
    const float* u;
    float inv_tau;
    uint64_t seed;
    uint32_t offset;
};

int sample_in(const spec_verify_ctx* c, const float* q, const float* u, float temperature,
              uint64_t seed, uint32_t offset, SampleIn* out)
{
    if (!c) return fail(SV_ERR_INVALID_ARG, "null context");
    if (c->s_ntile == 0)
        return fail(SV_ERR_UNSUPPORTED, "sampled verification needs vocab <= " +
                                            std::to_string(SAMPLE_MAX_TILES * SAMPLE_TILE));
    if (!q || !u) return fail(SV_ERR_INVALID_ARG, "null draft distribution or uniforms");
    if (!(temperature > 0.f) || !std::isfinite(temperature) || !std::isfinite(1.0f / temperature))
        return fail(SV_ERR_INVALID_ARG, "temperature must be positive and finite, with a finite inverse");
    out->q = q;
    out->u = u;
    out->inv_tau = 1.0f / temperature;
    out->seed = seed;
    out->offset = offset;
    return SV_OK;
}

// Tile statistics, acceptance decision + draw, commit (sampling.h).
int launch_sampling(spec_verify_ctx* c, const SampleIn& smp, const float* logits,
                    const int32_t* drafts, const int32_t* ctx_in, int32_t* ctx_out, int B,
                    int32_t* accepted, int32_t* next_tok, const int* seq_err, hipStream_t s)
{
    const int K1 = c->K1, T = B * K1, nt = c->s_ntile;
    SampleArgs a;
    memset(&a, 0, sizeof(a));
    a.logits = logits;
    a.drafts = drafts;
    a.q = smp.q;
    a.u = smp.u;
    a.inv_tau = smp.inv_tau;
    a.key0 = (uint32_t)smp.seed;
    a.key1 = (uint32_t)(smp.seed >> 32);
    a.offset = smp.offset;
    a.V = c->c.vocab;
    a.T = T;
    a.K1 = K1;
    a.ntile = nt;
    a.stats = c->sstats;
    a.dkeys = c->sdkeys;
    a.fkeys = c->sfkeys;
    a.decision = c->sdecision;
    a.ctx_in = ctx_in;
    a.ctx_out = ctx_out;
    a.accepted = accepted;
    a.next_tok = next_tok;
    a.seq_err = seq_err;
    a.err_word = c->err_word;
    {
        ProfScope ps(c, SV_KC_SAMPLING, s);
        launch(sample_stats_kernel, dim3(nt, T), dim3(256), 0, s, a);
    }
    {
        ProfScope ps(c, SV_KC_SAMPLING, s);
        launch(sample_draw_kernel, dim3(nt, B), dim3(256), 0, s, a);
    }
    {
        ProfScope ps(c, SV_KC_SAMPLING, s);
        launch(sample_finish_kernel, dim3(B), dim3(64), 0, s, a);
    }
    HIP_TRY(hipGetLastError());
    return SV_OK;
}

// The current device, which must be a gfx950.
int check_device(int* dev)
{
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1)
        return fail(SV_ERR_NO_DEVICE, "no HIP device visible");
    HIP_TRY(hipGetDevice(dev));
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, *dev));
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(SV_ERR_NO_DEVICE, std::string("device is ") + prop.gcnArchName + ", not gfx950");
    return SV_OK;
}

// Shapes and the attention plan of a context for `cfg` (no memory).
int plan_context(spec_verify_ctx* c, const spec_verify_config& cfg, int dev)
{
    c->c = cfg;
    c->device = dev;
    const spec_verify_config& k = c->c;
    c->K1 = k.k_draft + 1;
    c->T_max = k.max_batch * c->K1;
    c->QD = k.n_q_heads * k.head_dim;
    c->QKV = (k.n_q_heads + 2 * k.n_kv_heads) * k.head_dim;
    c->bf = k.weight_dtype != SV_F32;
    // attention plan: rows per KV head and chunking
    int G = k.n_q_heads / k.n_kv_heads;
    int R = c->K1 * G;
    int QF = cdiv(R, 16);
    // more query fragments per wave reuse each loaded K/V tile more often:
    // dense GQA verify (128 rows per KV head) 78 -> 62 us per layer with four
    c->att_QPW = QF >= 4 ? 4 : (QF >= 2 ? 2 : 1);
    c->att_QG = cdiv(QF, c->att_QPW);
    // bf16 caches with 17 .. 256 rows per KV head: one workgroup per (sequence,
    // KV head, chunk) for all rows, K/V tiles staged in LDS (two fragments per
    // wave, 1 .. 8 waves)
    c->att_lds_nw = 0;
    if (c->bf && QF >= 2 && QF <= 16 && (k.head_dim == 64 || k.head_dim == 128)) {
        int nw = 1;
        while (nw * 2 < QF) nw *= 2;
        c->att_lds_nw = nw;
    }
    if (c->att_lds_nw > 0) {
        // about two workgroups per CU over the largest batch, chunks of at
        // most 512 keys (the chunk partials of all R rows are written per chunk)
        const long work = (long)k.max_batch * k.n_kv_heads * k.kv_capacity;
        int ch = 64;
        while (ch < 512 && work / ch > 512) ch *= 2;
        c->att_CH = ch;
        c->att_maxch = cdiv(k.kv_capacity, ch);
        if (c->att_maxch > ATT_MAXCH_CAP)
            return fail(SV_ERR_UNSUPPORTED, "kv_capacity too large for the attention plan");
    } else {
        // streaming K/V loads only when every tile has one reader (one query
        // group per KV head) and the caches are far larger than the 256 MB
        // Infinity Cache; a smaller cache stays resident from step to step
        const double kv_bytes = 2.0 * k.max_batch * k.n_layers * k.n_kv_heads * (double)k.kv_capacity *
                                k.head_dim * (k.kv_dtype == SV_F32 ? 4 : 2);
        c->att_stream = c->att_QG == 1 && kv_bytes > 1024.0 * 1024 * 1024;
        // the bf16 split kernel exists with one fragment per wave, and with
        // four for several query groups (launch_attention_t)
        if (c->bf && !(c->att_QPW == 1 || (c->att_QPW == 4 && !c->att_stream)))
            return fail(SV_ERR_UNSUPPORTED, "no split-KV attention instance for this shape");
        long work = (long)k.max_batch * k.n_kv_heads * c->att_QG * k.kv_capacity;
        int ch = 64;
        const long waves_target = c->att_QPW >= 4 ? 2048 : 2 * 2048;   // busier waves: fewer of them
        // streamed chunks at most 512 keys: batch 64 with long contexts,
        // 271 -> 258 us per layer against 1,024-key chunks (same box)
        const int ch_max = c->att_stream ? 512 : 1024;
        while (ch < ch_max && work / ch > waves_target) ch *= 2;
        c->att_CH = ch;
        c->att_maxch = cdiv(k.kv_capacity, ch);
        if (c->att_maxch > ATT_MAXCH_CAP)
            return fail(SV_ERR_UNSUPPORTED, "kv_capacity too large for the attention plan");
    }

    return SV_OK;
}

// The workspace of a context for up to B sequences, taken piece by piece
// from `take(bytes)` (nullptr: out of memory).  `extras`: also the buffers of
// sampled verification and of FastMTP drafting.
template <class Take>
int carve_workspace(spec_verify_ctx* c, int B, bool extras, Take take)
{
    const spec_verify_config& k = c->c;
    const int T = B * c->K1, H = k.hidden;
    const size_t AES = c->bf ? 2 : 4;
    int E = k.n_experts, tk = k.top_k, S = k.n_shared;
    long moe_rows = (long)T * tk + (long)S * T;
    int NT_lm = cdiv(k.vocab, 64);
    int NT_lg = cdiv(k.vocab, 1024);
    size_t part_cols = std::max<size_t>({(size_t)c->QKV, (size_t)H, (size_t)(E > 0 ? E : 1)});
    c->parts_elems = (size_t)KS_MAX * T * part_cols;
    c->keys_elems = (size_t)std::max(NT_lm, NT_lg) * T;
    bool ok = true;
    auto get = [&](auto*& p, size_t elems) {
        using E_ = std::remove_reference_t<decltype(*p)>;
        void* v = ok ? take(std::max<size_t>(elems * sizeof(E_), 1)) : nullptr;
        ok = ok && v;
        p = (E_*)v;
    };
    char* hbuf = nullptr;
    char* qbuf = nullptr;
    char* obuf = nullptr;
    get(c->x, (size_t)T * H);
    get(c->x2, (size_t)T * H);
    get(hbuf, (size_t)T * H * AES);
    c->h = hbuf;
    get(c->parts, c->parts_elems);
    get(qbuf, (size_t)T * c->QD * AES);
    c->q = qbuf;
    get(obuf, (size_t)T * c->QD * AES);
    c->o = obuf;
    size_t prow = (size_t)B * k.n_q_heads * c->K1 * c->att_maxch;
    get(c->opart, prow * k.head_dim);
    get(c->mlpart, prow * 2);
    get(c->rope, (size_t)k.kv_capacity * (k.head_dim / 2));
    get(c->keys, c->keys_elems);
    get(c->seq_err, (size_t)B);
    get(c->err_word, 1);
    if (extras) {
        char* dc = nullptr;
        char* ds = nullptr;
        get(dc, (size_t)T * 2 * H * AES);
        c->dcat = dc;
        get(c->dzero, (size_t)T * H);
        get(c->dpos, (size_t)B);
        get(ds, (size_t)B * H * AES);
        c->dstate = ds;
        if (k.vocab <= SAMPLE_MAX_TILES * SAMPLE_TILE) {
            c->s_ntile = cdiv(k.vocab, SAMPLE_TILE);
            get(c->slogits, (size_t)T * k.vocab);
            get(c->sstats, (size_t)T * c->s_ntile);
            get(c->sdkeys, (size_t)B * c->s_ntile);
            get(c->sfkeys, (size_t)B * c->s_ntile);
            get(c->sdecision, (size_t)B);
        }
    }
    if (k.ffn_kind == SV_FFN_MOE) {
        char* abuf = nullptr;
        get(c->logits_g, (size_t)T * E);
        get(c->sel, (size_t)T * tk);
        get(c->gate, (size_t)T * tk);
        get(c->slot, (size_t)T * tk);
        get(c->perm_tok, (size_t)moe_rows);
        get(c->tiles, (size_t)3 * (E + moe_rows + 8));
        get(c->n_tiles, 1);
        get(abuf, (size_t)moe_rows * k.expert_inter * AES);
        c->act = abuf;
        get(c->y, (size_t)moe_rows * H);
    } else {
        char* abuf = nullptr;
        get(abuf, (size_t)T * k.dense_inter * AES);
        c->act = abuf;
    }
    if (!ok) return fail(SV_ERR_HIP, "workspace allocation failed");
    return SV_OK;
}

}  // namespace

// ====================================================================== ABI
extern "C" {

int spec_verify_abi_version(void) { return SPEC_VERIFY_ABI_VERSION; }

const char* spec_verify_status_string(int s)
{
    switch (s) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARG: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SV_ERR_HIP: return "HIP runtime error";
    case SV_ERR_NO_DEVICE: return "no usable gfx950 device";
    case SV_ERR_NOT_SET: return "requested data was never produced";
    default: return "unknown status";
    }
}

int spec_verify_last_error(char* buf, int len)
{
    std::lock_guard<std::mutex> lk(g_err_mu);
    if (buf && len > 0) {
        size_t n = std::min<size_t>(g_err.size(), (size_t)len - 1);
        memcpy(buf, g_err.data(), n);
        buf[n] = 0;
    }
    return (int)g_err.size();
}

void spec_verify_destroy(spec_verify_ctx* c)
{
    if (!c) return;
    (void)hipSetDevice(c->device);
    for (auto& e : c->prof_events) {
        (void)hipEventDestroy(e.a);
        (void)hipEventDestroy(e.b);
    }
    for (void* p : c->allocs) (void)hipFree(p);
    delete c;
}

int spec_verify_init(const spec_verify_config* cfg, spec_verify_ctx** out)
{
    if (!cfg || !out) return fail(SV_ERR_INVALID_ARG, "null config or output pointer");
    *out = nullptr;
    int rc = validate_config(*cfg);
    if (rc) return rc;
    int dev = 0;
    rc = check_device(&dev);
    if (rc) return rc;

    spec_verify_ctx* c = new spec_verify_ctx();
    rc = plan_context(c, *cfg, dev);
    if (rc) {
        delete c;
        return rc;
    }
    rc = carve_workspace(c, cfg->max_batch, true, [c](size_t bytes) -> void* {
        void* v = nullptr;
        if (hipMalloc(&v, std::max<size_t>(bytes, 256)) != hipSuccess) return nullptr;
        c->allocs.push_back(v);
        return v;
    });
    if (rc) {
        spec_verify_destroy(c);
        return rc;
    }
    const spec_verify_config& k = c->c;
    // rotary table: angle pos * theta^(-2i/D) in double, stored as fp32 (cos, sin)
    {
        int half = k.head_dim / 2;
        std::vector<float2> tab((size_t)k.kv_capacity * half);
        for (int p = 0; p < k.kv_capacity; p++)
            for (int i = 0; i < half; i++) {
                double ang = (double)p * std::pow((double)k.rope_theta, -2.0 * i / k.head_dim);
                tab[(size_t)p * half + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
            }
        hipError_t e = hipMemcpy(c->rope, tab.data(), tab.size() * sizeof(float2),
                                 hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            spec_verify_destroy(c);
            return fail(SV_ERR_HIP, std::string("rope upload: ") + hipGetErrorString(e));
        }
    }
    hipError_t e = hipMemset(c->err_word, 0, sizeof(unsigned));
    if (e == hipSuccess) e = hipMemset(c->dzero, 0, (size_t)c->T_max * k.hidden * sizeof(float));
    if (e != hipSuccess) {
        spec_verify_destroy(c);
        return fail(SV_ERR_HIP, std::string("workspace reset: ") + hipGetErrorString(e));
    }
    *out = c;
    return SV_OK;
}

int spec_verify_set_kv_pages(spec_verify_ctx* c, const int32_t* table)
{
    if (!c) return fail(SV_ERR_INVALID_ARG, "null context");
    if (!c->c.kv_page_size) return fail(SV_ERR_UNSUPPORTED, "the context's caches are not paged");
    if (!table) return fail(SV_ERR_INVALID_ARG, "null page table");
    c->kv_table = table;
    return SV_OK;
}

int spec_verify_set_debug(spec_verify_ctx* c, float* logits, float* hidden, int32_t* target,
                          int32_t* routing)
{
    if (!c) return fail(SV_ERR_INVALID_ARG, "null context");
    c->dbg_logits = logits;
    c->dbg_hidden = hidden;
    c->dbg_target = target;
    c->dbg_routing = routing;
    return SV_OK;
}

int spec_verify_set_debug_router(spec_verify_ctx* c, float* router_logits)
{
    if (!c) return fail(SV_ERR_INVALID_ARG, "null context");
    if (router_logits && c->c.ffn_kind != SV_FFN_MOE)
        return fail(SV_ERR_UNSUPPORTED, "router logits exist for MoE models only");
    c->dbg_rlogits = router_logits;
    return SV_OK;
}

// The forward pass and the greedy acceptance, or (smp != nullptr) the sampled
// acceptance on the logits the LM head writes alongside its argmax keys.
static int step_impl(spec_verify_ctx* c, const spec_verify_weights* w, void* k_cache,
                     void* v_cache, const int32_t* committed, const int32_t* drafts,
                     const int32_t* ctx_in, int32_t* ctx_out, int B, int32_t* accepted,
                     int32_t* next_tok, void* stream, const SampleIn* smp,
                     DraftPass* dp = nullptr)
{
    if (!c || !w) return fail(SV_ERR_INVALID_ARG, "null context or weights");
    if (B < 1 || B > c->c.max_batch) return fail(SV_ERR_INVALID_ARG, "batch outside [1, max_batch]");
    if (!k_cache || !v_cache || !ctx_in ||
        (!dp && (!committed || !drafts || !ctx_out || !accepted || !next_tok)))
        return fail(SV_ERR_INVALID_ARG, "null buffer pointer");
    const spec_verify_config& k = c->c;
    if (!w->embed || !w->layers || !w->final_norm || !w->lm_head)
        return fail(SV_ERR_INVALID_ARG, "null weight pointer");
    const bool fp8 = k.weight_dtype == SV_FP8;
    if (fp8 && !w->lm_scale) return fail(SV_ERR_INVALID_ARG, "fp8 weights need lm_scale");
    for (int l = 0; l < k.n_layers; l++) {
        const spec_verify_layer& L = w->layers[l];
        bool ok = L.attn_norm && L.ffn_norm && L.w_qkv && L.w_o && L.w_gate_up && L.w_down;
        if (k.ffn_kind == SV_FFN_MOE) ok = ok && L.w_router && (k.n_shared == 0 || (L.w_sh_gate_up && L.w_sh_down));
        if (fp8) {
            ok = ok && L.s_qkv && L.s_o && L.s_gate_up && L.s_down;
            if (k.ffn_kind == SV_FFN_MOE)
                ok = ok && L.s_router && (k.n_shared == 0 || (L.s_sh_gate_up && L.s_sh_down));
        }
        if (!ok) return fail(SV_ERR_INVALID_ARG, "null pointer in layer " + std::to_string(l));
    }
    if (w->layout != SV_LAYOUT_ROW_MAJOR && w->layout != SV_LAYOUT_TILED16)
        return fail(SV_ERR_INVALID_ARG, "unknown weight layout");
    const bool packed = w->layout == SV_LAYOUT_TILED16;
    if (k.kv_page_size && !c->kv_table)
        return fail(SV_ERR_NOT_SET, "paged KV caches need a page table (spec_verify_set_kv_pages)");
    const bool mx = k.mx_dtype == SV_MXFP4;
    if (mx) {
        if (!packed) return fail(SV_ERR_UNSUPPORTED, "MXFP4 weights need the tiled16 layout");
        if (!w->lm_scale) return fail(SV_ERR_INVALID_ARG, "MXFP4 LM head needs lm_scale");
        for (int l = 0; l < k.n_layers && k.ffn_kind == SV_FFN_MOE; l++) {
            const spec_verify_layer& L = w->layers[l];
            if (!L.s_gate_up || !L.s_down || (k.n_shared > 0 && (!L.s_sh_gate_up || !L.s_sh_down)))
                return fail(SV_ERR_INVALID_ARG, "MXFP4 expert matrices need their block scales");
        }
    }
    HIP_TRY(hipSetDevice(c->device));
    hipStream_t s = (hipStream_t)stream;
    const int wt = k.weight_dtype, step = wsteps(wt);
    const int wt_mx = mx ? SV_MXFP4 : wt;   // experts and LM head
    const int K1 = c->K1, T = B * K1, H = k.hidden, L = k.n_layers, QKV = c->QKV, QD = c->QD;
    const bool bf = c->bf;
    const size_t AES = bf ? 2 : 4;
    (void)AES;

    RowArgs ra;
    memset(&ra, 0, sizeof(ra));
    ra.H = H;
    ra.K1 = K1;
    ra.V = k.vocab;
    ra.cap = k.kv_capacity;
    ra.E = k.n_experts;
    ra.topk = k.top_k;
    ra.n_shared = k.n_shared;
    ra.T = T;
    ra.eps = k.rms_eps;
    ra.committed = committed;
    ra.drafts = drafts;
    ra.ctx_in = ctx_in;
    ra.seq_err = c->seq_err;
    ra.err_word = c->err_word;
    ra.embed = w->embed;
    ra.x = c->x;
    ra.x_out = c->x;
    ra.h = c->h;
    ra.gain = w->layers[0].attn_norm;
    const int MFd = rows_mf(T);
    const int MTd = cdiv(T, 16 * MFd);
    // rows >= 64: the large-row kernel (activation chunks staged in LDS);
    // fewer rows: the attention input (embedding + norm for the first layer,
    // QKV, rotary, cache append) is one kernel
    const bool big = T >= 64 && wt != SV_F32;
    if (big && !dp) {
        embed_norm_kernel<true><<<T, 1024, 0, s>>>(ra);   // large rows: bf16 activations
    }
    QkvArgs qa;
    memset(&qa, 0, sizeof(qa));
    qa.X = c->h;
    qa.embed = w->embed;
    qa.gain = w->layers[0].attn_norm;
    qa.committed = committed;
    qa.drafts = drafts;
    qa.ctx_in = ctx_in;
    qa.seq_err = c->seq_err;
    qa.err_word = c->err_word;
    qa.x_out = c->x;
    qa.rope = c->rope;
    qa.q = c->q;
    KvPages kvp;
    kvp.table = k.kv_page_size ? c->kv_table : nullptr;
    kvp.page = k.kv_page_size;
    kvp.max_pages = k.kv_page_size ? k.kv_capacity / k.kv_page_size : 0;
    kvp.n_pages = k.kv_pool_pages;
    qa.kc = k_cache;
    qa.vc = v_cache;
    qa.kvp = kvp;
    qa.V = k.vocab;
    qa.cap = k.kv_capacity;
    qa.K1 = K1;
    qa.T = T;
    qa.H = H;
    qa.n_q = k.n_q_heads;
    qa.n_kv = k.n_kv_heads;
    qa.D = k.head_dim;
    qa.L = L;
    qa.MT = MTd;
    qa.NT = (k.n_q_heads + 2 * k.n_kv_heads) * (k.head_dim / 32);
    qa.eps = k.rms_eps;
    const int MTb = cdiv(T, 16 * BIG_MF);
    // dense GEMM (or the dense SwiGLU / argmax variants); returns the K split used
    // allow_split: largest K split the consumer accepts (0 or 1: none)
    int last_nt = 0;   // column tiles of the last dense GEMM (argmax key columns)
    // fp32 logits written by the LM head: the debug buffer, and for sampled
    // verification the sampling input (the debug buffer when one is set)
    float* lm_logits = smp ? (c->dbg_logits ? c->dbg_logits : c->slogits) : c->dbg_logits;
    auto dense_gemm = [&](int mode, const void* X, long ldx, int N, int Kd, const void* W,
                          const float* ws, void* out, long ldo, int allow_split,
                          int wdt = -1) -> int {
        const int wtd = wdt >= 0 ? wdt : wt;
        GemmArgs a = dense_args(X, ldx, T, N, Kd, W, ws);
        a.out = out;
        a.ldo = ldo;
        a.split_stride = (long)T * ldo;
        a.keys = c->keys;
        a.key_ld = T;
        a.dbg = lm_logits;
        a.dbg_ld = k.vocab;
        if (mode == GM_SWIGLU) a.dual_off = N;
        // MXFP4 (LM head): one 128-long step per chunk, and the 128-row tiles
        const int chunk = wtd == SV_MXFP4 ? wsteps(wtd) : BIG_CHUNK_STEPS * step;
        // bf16 at up to 128 rows: one 128-row tile reads each weight once, which
        // the HBM-bound shapes prefer (LM head at 128 rows: 6% faster)
        const bool wide = big && packed && Kd % chunk == 0 && wtd != SV_MXFP4 &&
                          (wt == SV_FP8 || T > 128);
        if (big && packed && mode == GM_ARGMAX && wtd == SV_BF16 && T > 64 && T <= 256 &&
            Kd % wsteps(SV_BF16) == 0) {
            a.MT = 1;
            a.NT = cdiv(N, lm_head_lds_cols(T));
            a.ksplit = 1;
            launch_lm_head_lds(a, s);
            last_nt = a.NT;
            return 1;
        }
        if (big && Kd % chunk == 0) {
            a.MT = wide ? cdiv(T, 32 * WIDE_MW) : MTb;
            a.NT = wide ? cdiv(N, wide_col_tile(mode)) : cdiv(N, 16 * 4 * big_nf(mode));
            long wgs = (long)a.NT * a.MT;
            a.ksplit = 1;
            if (allow_split > 1) {   // enough workgroups for the 256 CUs, each split >= 4 chunks
                int steps = Kd / chunk;
                for (int sp = 2; sp <= allow_split; sp++) {
                    if (steps % sp || steps / sp < 4) continue;
                    if (wgs * a.ksplit >= 512) break;
                    a.ksplit = sp;
                }
            }
            // fp8 projections: the most K splits of 16 or more 64-long steps
            // within 512 workgroups, which run on the LDS-staged kernel (see
            // launch_wide_t; QKV of the dense fp8 model: 2 splits of 20 steps
            // instead of 5 of 8 on the register-staged kernel, 23.2 -> 22.5 us
            // per layer; down: 8 splits of 19 steps)
            if (wide && wtd == SV_FP8 && mode == GM_STORE && allow_split > 1) {
                const int steps64 = Kd / 64;
                for (int sp = 2; sp <= allow_split; sp++) {
                    if (steps64 % sp || steps64 / sp < WIDE_LDS_MIN_STEPS) continue;
                    if (wgs * sp > 512) break;
                    a.ksplit = sp;
                }
            }
            if (wide) launch_gemm_wide(wt, mode, a, s);
            else launch_gemm_big(wtd, mode, packed, a, s);
            last_nt = a.NT;
            return a.ksplit;
        }
        a.MT = MTd;
        a.NT = cdiv(N, small_col_tile(wtd, mode));
        long waves = (long)a.NT * a.MT * 4;
        a.ksplit = allow_split > 1 ? pick_ksplit(waves, Kd, step, allow_split) : 1;
        launch_gemm(wtd, mode, MFd, packed, a, s);
        last_nt = a.NT;
        return a.ksplit;
    };

    AttnArgs at;
    memset(&at, 0, sizeof(at));
    at.q = c->q;
    at.kc = k_cache;
    at.vc = v_cache;
    at.kvp = kvp;
    at.err_word = c->err_word;
    at.ctx_in = ctx_in;
    at.seq_err = c->seq_err;
    at.L = L;
    at.n_q = k.n_q_heads;
    at.n_kv = k.n_kv_heads;
    at.D = k.head_dim;
    at.K1 = K1;
    at.cap = k.kv_capacity;
    at.CH = c->att_CH;
    at.maxch = c->att_maxch;
    at.QG = c->att_QG;
    at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)k.head_dim));
    at.opart = c->opart;
    at.mlpart = c->mlpart;

    if (dp) {
        // drafting: the block's input rows z = P [N_e(e); N_h(state)] instead
        // of an embedding, then the block's first norm
        DraftArgs& da = dp->args;
        da.T = T;
        da.cat = c->dcat;
        da.pos = c->dpos;
        da.seq_err = c->seq_err;
        da.ustate = c->dstate;
        if (bf) mtp_input_kernel<true><<<T, 256, 0, s>>>(da);
        else mtp_input_kernel<false><<<T, 256, 0, s>>>(da);
        const int ks = dense_gemm(GM_STORE, c->dcat, 2L * H, H, 2 * H, dp->P, dp->sP, c->parts, H,
                                  KS_MAX);
        ra.x = c->dzero;
        ra.x_out = c->x;
        ra.parts = c->parts;
        ra.nsplit = ks;
        ra.gain = w->layers[0].attn_norm;
        ra.dbg_hidden = nullptr;
        if (bf) launch_residual_norm<true, false>(T, s, ra);
        else launch_residual_norm<false, false>(T, s, ra);
    }
    for (int l = 0; l < L; l++) {
        const spec_verify_layer& Lw = w->layers[l];
        // ---- attention half
        int ks;
        if (!big) {
            qa.W = Lw.w_qkv;
            qa.ws = Lw.s_qkv;
            qa.layer = l;
            ProfScope ps(c, SV_KC_QKV, s);
            launch_qkv_rope(wt, MFd, packed, l == 0 && !dp, qa, s);
        } else {
            {
                ProfScope ps(c, SV_KC_QKV, s);
                ks = dense_gemm(GM_STORE, c->h, H, QKV, H, Lw.w_qkv, Lw.s_qkv, c->parts, QKV, KS_MAX);
            }
            RopeArgs rp;
            rp.qkv = c->parts;
            rp.nsplit = ks;
            rp.T = T;
            rp.K1 = K1;
            rp.n_q = k.n_q_heads;
            rp.n_kv = k.n_kv_heads;
            rp.D = k.head_dim;
            rp.L = L;
            rp.layer = l;
            rp.cap = k.kv_capacity;
            rp.ctx_in = ctx_in;
            rp.seq_err = c->seq_err;
            rp.rope = c->rope;
            rp.q = c->q;
            rp.kc = k_cache;
            rp.vc = v_cache;
            rp.kvp = kvp;
            rp.err_word = c->err_word;
            dim3 grid(T, k.n_q_heads + 2 * k.n_kv_heads);
            launch_rope_append<true>(grid, s, rp);   // large rows: bf16 activations
        }

        at.layer = l;
        {
            ProfScope ps(c, SV_KC_ATTENTION, s);
            at.B = B;
            if (c->att_lds_nw > 0) {
                launch_attention_lds(k.head_dim, c->att_lds_nw, dim3(c->att_maxch, k.n_kv_heads, B), at, s);
            } else {
                const dim3 grid = c->att_QG > 1
                    ? dim3((unsigned)(cdiv(B * k.n_kv_heads * c->att_maxch, 8) * 8 * c->att_QG), 1, 1)
                    : dim3(c->att_maxch, k.n_kv_heads, B);
                launch_attention(bf, k.head_dim, c->att_QPW, c->att_stream, grid, at, s);
            }
        }
        launch_merge(bf, c->att_maxch, at, c->o, B * k.n_q_heads * K1, s);
        // the MoE consumer (residual + norm + router) takes at most 4 splits
        ks = dense_gemm(GM_STORE, c->o, QD, H, QD, Lw.w_o, Lw.s_o, c->parts, H,
                        k.ffn_kind == SV_FFN_MOE ? 4 : KS_MAX);
        ra.parts = c->parts;
        ra.nsplit = ks;
        ra.gain = Lw.ffn_norm;
        ra.dbg_hidden = nullptr;
        ra.x = c->x;
        // few rows (batch 1): the router's logits are selected inside the
        // gate/up GEMM (every workgroup selects; workgroup 0 publishes)
        const bool sel_in_gemm = k.ffn_kind == SV_FFN_MOE && !big && T <= 4 && k.n_experts <= 64 &&
                                 k.n_experts % 16 == 0 && k.n_experts >= 32 && T * k.top_k <= 64;
        if (k.ffn_kind == SV_FFN_MOE) {
            // residual + norm + router (experts shared out over S workgroups per
            // row when rows are few; the updated residual goes to x2 since a
            // row's workgroups all read x), then selection + permutation
            const int E = k.n_experts, tk = k.top_k;
            // few assignments: the grouped GEMMs and the combine derive tiles and
            // slots from the selections (no permutation pass)
            const bool implied = !big && T <= 16 && T * tk <= 64 && E <= 64;
            const int S = (E % 16 == 0 && E >= 32 && T <= 64) ? E / 16 : 1;
            const int avg_rows = std::max(1, T * tk / E);
            const int BMe = 16 * rows_mf(avg_rows);
            ra.x_out = c->x2;
            ra.w_router = Lw.w_router;
            ra.s_router = Lw.s_router;
            ra.wdtype = wt;
            ra.renorm = k.renorm_topk;
            ra.sel = c->sel;
            ra.gate_out = c->gate;
            ra.dbg_sel = c->dbg_routing ? c->dbg_routing + (size_t)l * T * k.top_k : nullptr;
            ra.dbg_rlogits = c->dbg_rlogits ? c->dbg_rlogits + (size_t)l * T * E : nullptr;
            ra.S = S;
            ra.logits_g = c->logits_g;
            ra.BM = BMe;
            ra.max_tiles = std::min(E, T * tk) + (T * tk) / BMe + k.n_shared * cdiv(T, BMe) + 1;
            ra.slot_out = c->slot;
            ra.perm_tok = c->perm_tok;
            ra.tiles = c->tiles;
            ra.n_tiles = c->n_tiles;
            dim3 grid(T, S);
            if (S > 1) {
                if (bf) residual_norm_kernel<true, false, true, 1><<<grid, 1024, 0, s>>>(ra);
                else residual_norm_kernel<false, false, true, 1><<<grid, 1024, 0, s>>>(ra);
            } else {
                if (bf) residual_norm_kernel<true, false, true, 4><<<grid, 1024, 0, s>>>(ra);
                else residual_norm_kernel<false, false, true, 4><<<grid, 1024, 0, s>>>(ra);
            }
            ra.implied = implied;
            // with at most 4 rows the gate/up GEMM selects the experts itself
            // (one launch fewer; batch 1 115.5 -> 115.2 us per step, same box:
            // the four rows' selections add about 3 us to every gate/up
            // workgroup); otherwise the selection (implied tiles) or selection
            // + permutation run here
            if (!implied || (S > 1 && !sel_in_gemm)) route_finish_kernel<<<1, 1024, 0, s>>>(ra);
        } else {
            ra.x_out = c->x;
            if (bf) launch_residual_norm<true, false>(T, s, ra);
            else launch_residual_norm<false, false>(T, s, ra);
        }

        // ---- feed-forward half
        const float* next_gain = (l + 1 < L) ? w->layers[l + 1].attn_norm : w->final_norm;
        float* dbg_h = c->dbg_hidden ? c->dbg_hidden + (size_t)l * T * H : nullptr;
        if (k.ffn_kind == SV_FFN_MOE) {
            const int E = k.n_experts, tk = k.top_k, S = k.n_shared, I = k.expert_inter;
            const bool implied = !big && T <= 16 && T * tk <= 64 && E <= 64;   // as in the routing
            const int avg_rows = std::max(1, T * tk / E);
            const int MFe = implied ? 1 : rows_mf(avg_rows);
            const int BMe = 16 * MFe;
            const int max_tiles = std::min(E, T * tk) + (T * tk) / BMe + S * cdiv(T, BMe) + 1;

            GemmArgs g;
            memset(&g, 0, sizeof(g));
            g.X = c->h;
            g.ldx = H;
            g.gather = c->perm_tok;
            g.N = I;
            g.K = H;
            g.ksplit = 1;
            g.W = Lw.w_gate_up;
            g.ws = Lw.s_gate_up;
            g.w_gstride = (long)2 * I * H;
            g.s_gstride = mx ? spec_verify_mx_scales_bytes(2L * I, H) : 2L * I;   // MXFP4: bytes per expert
            g.W2 = Lw.w_sh_gate_up;
            g.ws2 = Lw.s_sh_gate_up;
            g.w2_gstride = (long)2 * I * H;
            g.s2_gstride = g.s_gstride;
            g.G1 = E;
            g.dual_off = I;
            g.tiles = c->tiles;
            g.n_tiles = c->n_tiles;
            g.sel = implied ? c->sel : nullptr;
            g.sel_T = T;
            g.sel_k = tk;
            g.sel_E = E;
            g.sel_S = S;
            if (sel_in_gemm) {
                g.sel_logits = c->logits_g;
                g.sel_renorm = k.renorm_topk;
                g.sel_out = c->sel;
                g.gate_out = c->gate;
                g.dbg_sel_out = c->dbg_routing ? c->dbg_routing + (size_t)l * T * k.top_k : nullptr;
            }
            g.MT = max_tiles;
            // many rows (T >= 64): 4-wave tiles sharing an LDS activation tile;
            // few rows: one-wave tiles streaming weights (finer balance)
            const bool big_e = big && H % (BIG_CHUNK_STEPS * step) == 0 &&
                               I % (BIG_CHUNK_STEPS * step) == 0;
            g.NT = big_e ? cdiv(I, 16 * 4 * GROUPED_NF) : cdiv(I, grouped_col_tile(wt_mx, GM_SWIGLU));
            g.out = c->act;
            g.ldo = I;
            {
                ProfScope ps(c, SV_KC_EXPERT_GATE_UP, s);
                if (big_e) launch_grouped_big(wt_mx, GM_SWIGLU, MFe, packed, g, s);
                else launch_gemm(wt_mx, GM_SWIGLU, MFe, packed, g, s);
            }
            GemmArgs d = g;
            d.sel_logits = nullptr;   // the selections published by the gate/up GEMM
            d.X = c->act;
            d.ldx = I;
            d.gather = nullptr;
            d.N = H;
            d.K = I;
            d.W = Lw.w_down;
            d.ws = Lw.s_down;
            d.w_gstride = (long)H * I;
            d.s_gstride = mx ? spec_verify_mx_scales_bytes(H, I) : H;
            d.W2 = Lw.w_sh_down;
            d.ws2 = Lw.s_sh_down;
            d.w2_gstride = (long)H * I;
            d.s2_gstride = d.s_gstride;
            d.dual_off = 0;
            d.NT = big_e ? cdiv(H, 16 * 4 * GROUPED_NF) : cdiv(H, grouped_col_tile(wt_mx, GM_STORE));
            d.out = c->y;
            d.ldo = H;
            d.split_stride = 0;
            {
                ProfScope ps(c, SV_KC_EXPERT_DOWN, s);
                if (big_e) launch_grouped_big(wt_mx, GM_STORE, MFe, packed, d, s);
                else launch_gemm(wt_mx, GM_STORE, MFe, packed, d, s);
            }
            ra.y = c->y;
            ra.gate = c->gate;
            ra.slot = c->slot;
            ra.gain = next_gain;
            ra.dbg_hidden = dbg_h;
            ra.x = c->x2;
            ra.x_out = c->x;
            if (bf) launch_residual_norm<true, true>(T, s, ra);
            else launch_residual_norm<false, true>(T, s, ra);
        } else {
            const int I = k.dense_inter;
            {
                ProfScope ps(c, SV_KC_EXPERT_GATE_UP, s);
                dense_gemm(GM_SWIGLU, c->h, H, I, H, Lw.w_gate_up, Lw.s_gate_up, c->act, I, 0);
            }
            {
                ProfScope ps(c, SV_KC_EXPERT_DOWN, s);
                ks = dense_gemm(GM_STORE, c->act, I, H, I, Lw.w_down, Lw.s_down, c->parts, H, KS_MAX);
            }
            ra.parts = c->parts;
            ra.nsplit = ks;
            ra.gain = next_gain;
            ra.dbg_hidden = dbg_h;
            ra.x = c->x;
            ra.x_out = c->x;
            if (bf) launch_residual_norm<true, false>(T, s, ra);
            else launch_residual_norm<false, false>(T, s, ra);
        }
    }

    // ---- LM head + argmax, acceptance
    {
        ProfScope ps(c, SV_KC_LM_HEAD, s);
        dense_gemm(GM_ARGMAX, c->h, H, k.vocab, H, w->lm_head, w->lm_scale, nullptr, 0, 0, wt_mx);
    }
    if (dp) {
        DraftArgs& da = dp->args;
        da.keys = c->keys;
        da.NT = last_nt;
        da.h = c->h;
        if (bf) draft_pick_kernel<true><<<B, 256, 0, s>>>(da);
        else draft_pick_kernel<false><<<B, 256, 0, s>>>(da);
        HIP_TRY(hipGetLastError());
        return SV_OK;
    }
    if (smp) return launch_sampling(c, *smp, lm_logits, drafts, ctx_in, ctx_out, B, accepted,
                                    next_tok, c->seq_err, s);
    const int NT_lm = last_nt;   // argmax key columns written by the LM head
    AcceptArgs ac;
    ac.keys = c->keys;
    ac.NT = NT_lm;
    ac.T = T;
    ac.K1 = K1;
    ac.drafts = drafts;
    ac.ctx_in = ctx_in;
    ac.ctx_out = ctx_out;
    ac.accepted = accepted;
    ac.next_tok = next_tok;
    ac.target = c->dbg_target;
    ac.seq_err = c->seq_err;
    ac.err_word = c->err_word;
    accept_kernel<<<B, 1024, 0, s>>>(ac);
    HIP_TRY(hipGetLastError());
    return SV_OK;
}

int spec_verify_step(spec_verify_ctx* c, const spec_verify_weights* w, void* k_cache,
                     void* v_cache, const int32_t* committed, const int32_t* drafts,
                     const int32_t* ctx_in, int32_t* ctx_out, int B, int32_t* accepted,
                     int32_t* next_tok, void* stream)
{
    return step_impl(c, w, k_cache, v_cache, committed, drafts, ctx_in, ctx_out, B, accepted,
                     next_tok, stream, nullptr);
}

int spec_verify_step_sampled(spec_verify_ctx* c, const spec_verify_weights* w, void* k_cache,
                             void* v_cache, const int32_t* committed, const int32_t* drafts,
                             const float* draft_probs, const float* accept_u, float temperature,
                             uint64_t seed, uint32_t offset, const int32_t* ctx_in,
                             int32_t* ctx_out, int B, int32_t* accepted, int32_t* next_tok,
                             void* stream)
{
    SampleIn smp;
    int rc = sample_in(c, draft_probs, accept_u, temperature, seed, offset, &smp);
    if (rc) return rc;
    return step_impl(c, w, k_cache, v_cache, committed, drafts, ctx_in, ctx_out, B, accepted,
                     next_tok, stream, &smp);
}

int spec_draft_step(spec_verify_ctx* c, const spec_verify_weights* w, const spec_mtp_weights* m,
                    void* k_cache, void* v_cache, const spec_verify_ctx* vc, const int32_t* ctx_in,
                    const int32_t* accepted, const int32_t* next_tok, const int32_t* drafts_in,
                    int B, int32_t* drafts_out, void* stream)
{
    if (!c || !w || !m || !vc) return fail(SV_ERR_INVALID_ARG, "null context or weights");
    const spec_verify_config& k = c->c;
    if (k.n_layers != 1 || k.ffn_kind != SV_FFN_DENSE || k.mx_dtype != vc->c.mx_dtype)
        return fail(SV_ERR_UNSUPPORTED, "the draft context must be a one-layer dense model "
                                         "with the target's LM-head storage");
    if (vc->c.hidden != k.hidden || vc->c.k_draft != k.k_draft || vc->c.vocab != k.vocab ||
        vc->bf != c->bf || B > vc->c.max_batch)
        return fail(SV_ERR_INVALID_ARG, "draft and verify contexts differ in hidden, K, vocab, "
                                        "activation type or batch");
    if (!ctx_in || !accepted || !next_tok || !drafts_in || !drafts_out)
        return fail(SV_ERR_INVALID_ARG, "null buffer pointer");
    if (!m->enorm || !m->hnorm || !m->eh_proj || (k.weight_dtype == SV_FP8 && !m->s_eh_proj))
        return fail(SV_ERR_INVALID_ARG, "null draft-head weight");
    DraftPass dp;
    memset(&dp, 0, sizeof(dp));
    DraftArgs& da = dp.args;
    da.H = k.hidden;
    da.K1 = c->K1;
    da.V = k.vocab;
    da.cap = k.kv_capacity;
    da.eps = k.rms_eps;
    da.embed = w->embed;
    da.vstate = vc->h;
    da.g_e = m->enorm;
    da.g_h = m->hnorm;
    da.accepted = accepted;
    da.next_tok = next_tok;
    da.drafts_in = drafts_in;
    da.drafts_out = drafts_out;
    da.ctx_in = ctx_in;
    da.err_word = c->err_word;
    dp.P = m->eh_proj;
    dp.sP = m->s_eh_proj;
    for (int d = 1; d <= k.k_draft; d++) {
        da.k = d;
        int rc = step_impl(c, w, k_cache, v_cache, nullptr, nullptr, c->dpos, nullptr, B, nullptr,
                           nullptr, stream, nullptr, &dp);
        if (rc) return rc;
    }
    return SV_OK;
}

int spec_verify_sample_from_logits(spec_verify_ctx* c, const float* logits,
                                   const int32_t* drafts, const float* draft_probs,
                                   const float* accept_u, float temperature, uint64_t seed,
                                   uint32_t offset, const int32_t* ctx_in, int32_t* ctx_out,
                                   int B, int32_t* accepted, int32_t* next_tok, void* stream)
{
    SampleIn smp;
    int rc = sample_in(c, draft_probs, accept_u, temperature, seed, offset, &smp);
    if (rc) return rc;
    if (B < 1 || B > c->c.max_batch) return fail(SV_ERR_INVALID_ARG, "batch outside [1, max_batch]");
    if (!logits || !drafts || !ctx_in || !ctx_out || !accepted || !next_tok)
        return fail(SV_ERR_INVALID_ARG, "null buffer pointer");
    HIP_TRY(hipSetDevice(c->device));
    return launch_sampling(c, smp, logits, drafts, ctx_in, ctx_out, B, accepted, next_tok,
                           nullptr, (hipStream_t)stream);
}

int spec_verify_accept_from_logits(spec_verify_ctx* c, const float* logits, const int32_t* drafts,
                                   const int32_t* ctx_in, int32_t* ctx_out, int B,
                                   int32_t* accepted, int32_t* next_tok, int32_t* target,
                                   void* stream)
{
    if (!c) return fail(SV_ERR_INVALID_ARG, "null context");
    if (B < 1 || B > c->c.max_batch) return fail(SV_ERR_INVALID_ARG, "batch outside [1, max_batch]");
    if (!logits || !drafts || !ctx_in || !ctx_out || !accepted || !next_tok)
        return fail(SV_ERR_INVALID_ARG, "null buffer pointer");
    HIP_TRY(hipSetDevice(c->device));
    hipStream_t s = (hipStream_t)stream;
    const int T = B * c->K1, V = c->c.vocab;
    const int NT = cdiv(V, 1024);
    logits_keys_kernel<<<dim3(NT, T), 256, 0, s>>>(logits, V, T, c->keys);
    AcceptArgs ac;
    ac.keys = c->keys;
    ac.NT = NT;
    ac.T = T;
    ac.K1 = c->K1;
    ac.drafts = drafts;
    ac.ctx_in = ctx_in;
    ac.ctx_out = ctx_out;
    ac.accepted = accepted;
    ac.next_tok = next_tok;
    ac.target = target;
    ac.seq_err = nullptr;
    ac.err_word = c->err_word;
    accept_kernel<<<B, 1024, 0, s>>>(ac);
    HIP_TRY(hipGetLastError());
    return SV_OK;
}

long spec_verify_mx_scales_bytes(long rows, int cols)
{
    if (rows < 1 || cols < 128 || cols % 128) return -1;
    return (rows + 15) / 16 * (long)((cols / 128 + 15) / 16) * 1024;
}

int spec_verify_pack_mx_scales(const void* src, void* dst, long rows, int cols, void* stream)
{
    if (!src || !dst) return fail(SV_ERR_INVALID_ARG, "null scale pointer");
    if (rows < 1 || cols < 128 || cols % 128)
        return fail(SV_ERR_INVALID_ARG, "MXFP4 scales: cols must be a positive multiple of 128");
    hipStream_t s = (hipStream_t)stream;
    long slices = spec_verify_mx_scales_bytes(rows, cols) / 16;
    long blocks = std::min<long>((slices + 255) / 256, 65536);
    pack_mx_scales_kernel<<<(unsigned)blocks, 256, 0, s>>>((const uint8_t*)src, (uint8_t*)dst, rows, cols);
    HIP_TRY(hipGetLastError());
    return SV_OK;
}

long spec_verify_tiled16_bytes(long rows, int cols, int dtype)
{
    if (rows < 1 || cols < 1 || dtype < SV_F32 || dtype > SV_FP8) return -1;
    long es = dtype == SV_F32 ? 4 : (dtype == SV_BF16 ? 2 : 1);
    return (rows + 15) / 16 * 16 * (long)cols * es;
}

int spec_verify_pack_tiled16(const void* src, void* dst, long rows, int cols, int dtype,
                             void* stream)
{
    if (!src || !dst) return fail(SV_ERR_INVALID_ARG, "null matrix pointer");
    if (rows < 1 || cols < 1 || dtype < SV_F32 || dtype > SV_FP8)
        return fail(SV_ERR_INVALID_ARG, "bad matrix shape or dtype");
    int es = dtype == SV_F32 ? 4 : (dtype == SV_BF16 ? 2 : 1);
    int S = 4 * (16 / es);
    if (cols % S) return fail(SV_ERR_UNSUPPORTED, "cols must be a multiple of the reduction step");
    hipStream_t s = (hipStream_t)stream;
    long chunks = (rows + 15) / 16 * (cols / S) * 64;
    long blocks = std::min<long>((chunks + 255) / 256, 65536);
    pack_tiled16_kernel<<<(unsigned)blocks, 256, 0, s>>>((const char*)src, (char*)dst, rows, cols, es);
    HIP_TRY(hipGetLastError());
    return SV_OK;
}

int spec_verify_error_word(spec_verify_ctx* c, uint32_t* out, int clear, void* stream)
{
    if (!c || !out) return fail(SV_ERR_INVALID_ARG, "null argument");
    HIP_TRY(hipSetDevice(c->device));
    hipStream_t s = (hipStream_t)stream;
    HIP_TRY(hipStreamSynchronize(s));
    unsigned v = 0;
    HIP_TRY(hipMemcpy(&v, c->err_word, sizeof(v), hipMemcpyDeviceToHost));
    *out = v;
    if (clear) HIP_TRY(hipMemset(c->err_word, 0, sizeof(unsigned)));
    return SV_OK;
}

int spec_verify_kernel_time(spec_verify_ctx* c, int kclass, int enable, double* total_ms,
                            int* launches)
{
    if (!c) return fail(SV_ERR_INVALID_ARG, "null context");
    if (kclass < 0 || kclass >= SV_KC_COUNT) return fail(SV_ERR_INVALID_ARG, "bad kernel class");
    HIP_TRY(hipSetDevice(c->device));
    if (total_ms || launches) {
        if (c->prof_class != kclass && c->prof_used == 0) return fail(SV_ERR_NOT_SET, "not recording");
        double tot = 0;
        for (size_t i = 0; i < c->prof_used; i++) {
            HIP_TRY(hipEventSynchronize(c->prof_events[i].b));
            float ms = 0;
            HIP_TRY(hipEventElapsedTime(&ms, c->prof_events[i].a, c->prof_events[i].b));
            tot += ms;
        }
        if (total_ms) *total_ms = tot;
        if (launches) *launches = (int)c->prof_used;
    }
    if (enable == 1) {
        if (c->prof_events.empty()) {
            c->prof_events.resize(8192);
            for (auto& e : c->prof_events) {
                HIP_TRY(hipEventCreate(&e.a));
                HIP_TRY(hipEventCreate(&e.b));
            }
        }
        c->prof_class = kclass;
        c->prof_used = 0;
    } else if (enable == 0) {
        c->prof_class = -1;
    }
    return SV_OK;
}

}  // extern "C"

#include "noalloc.h"
