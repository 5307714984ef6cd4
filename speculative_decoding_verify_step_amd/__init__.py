"""Python binding of the MI355X greedy speculative-decoding verify step.

A thin ctypes layer over libspecverify.so (include/spec_verify.h): the
functions carry the C ABI's names and only marshal arguments -- every step of
the verify path runs in the library's HIP kernels.  PyTorch is used for device
memory and streams only.  If the library has not been built the import fails
loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int, c_uint32, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_OK, SV_ERR_INVALID_ARG, SV_ERR_UNSUPPORTED, SV_ERR_HIP, SV_ERR_NO_DEVICE, SV_ERR_NOT_SET = (
    0, -1, -2, -3, -4, -5)
SV_F32, SV_BF16, SV_FP8, SV_MXFP4 = 0, 1, 2, 3
SV_FFN_MOE, SV_FFN_DENSE = 0, 1
SV_DEV_BAD_TOKEN, SV_DEV_CAPACITY, SV_DEV_NAN_LOGIT = 1, 2, 4
(SV_KC_LM_HEAD, SV_KC_ATTENTION, SV_KC_EXPERT_GATE_UP, SV_KC_EXPERT_DOWN, SV_KC_QKV,
 SV_KC_SAMPLING) = range(6)
SV_LAYOUT_ROW_MAJOR, SV_LAYOUT_TILED16 = 0, 1
_LAYOUTS = {"row_major": SV_LAYOUT_ROW_MAJOR, "tiled16": SV_LAYOUT_TILED16}
# matrices that feed a matrix product (packed in the tiled16 layout)
GEMM_MATRICES = ("w_qkv", "w_o", "w_gate_up", "w_down", "w_sh_gate_up", "w_sh_down")
KERNEL_CLASSES = {"lm_head": 0, "attention": 1, "expert_gate_up": 2, "expert_down": 3, "qkv": 4,
                  "sampling": 5}
_DT = {"f32": SV_F32, "bf16": SV_BF16, "fp8": SV_FP8}

# every function include/spec_verify.h declares
EXPORTS = ("spec_verify_init", "spec_verify_destroy", "spec_verify_step", "spec_verify_set_debug",
           "spec_verify_accept_from_logits", "spec_verify_error_word", "spec_verify_kernel_time",
           "spec_verify_last_error", "spec_verify_status_string", "spec_verify_abi_version",
           "spec_verify_pack_tiled16", "spec_verify_tiled16_bytes", "spec_verify_step_sampled",
           "spec_verify_sample_from_logits", "spec_verify_pack_mx_scales",
           "spec_verify_mx_scales_bytes", "spec_draft_step", "spec_verify_set_kv_pages",
           "spec_verify_set_debug_router", "spec_verify_step_noalloc")


class SpecVerifyConfig(ctypes.Structure):
    _fields_ = [("n_layers", c_int), ("hidden", c_int), ("n_q_heads", c_int),
                ("n_kv_heads", c_int), ("head_dim", c_int), ("ffn_kind", c_int),
                ("n_experts", c_int), ("expert_inter", c_int), ("top_k", c_int),
                ("n_shared", c_int), ("renorm_topk", c_int), ("dense_inter", c_int),
                ("vocab", c_int), ("max_batch", c_int), ("k_draft", c_int),
                ("kv_capacity", c_int), ("rope_theta", c_float), ("rms_eps", c_float),
                ("weight_dtype", c_int), ("embed_dtype", c_int), ("kv_dtype", c_int),
                ("mx_dtype", c_int), ("kv_page_size", c_int), ("kv_pool_pages", c_int)]


class SpecVerifyLayer(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "attn_norm", "w_qkv", "s_qkv", "w_o", "s_o", "ffn_norm", "w_router", "s_router",
        "w_gate_up", "s_gate_up", "w_down", "s_down", "w_sh_gate_up", "s_sh_gate_up",
        "w_sh_down", "s_sh_down")]


class SpecVerifyWeights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("layers", POINTER(SpecVerifyLayer)),
                ("final_norm", c_void_p), ("lm_head", c_void_p), ("lm_scale", c_void_p),
                ("layout", c_int)]


class SpecMtpWeights(ctypes.Structure):
    _fields_ = [("enorm", c_void_p), ("hnorm", c_void_p), ("eh_proj", c_void_p),
                ("s_eh_proj", c_void_p)]


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {spec_verify_status_string(status)} ({status}): "
                         f"{spec_verify_last_error()}")


_lib = None


def load_library() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              f"`python -m speculative_decoding_verify_step_amd._build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = c_void_p
        lib.spec_verify_init.argtypes = [P, P]
        lib.spec_verify_destroy.argtypes = [P]
        lib.spec_verify_destroy.restype = None
        lib.spec_verify_step.argtypes = [P, P, P, P, P, P, P, P, c_int, P, P, P]
        lib.spec_verify_set_debug.argtypes = [P, P, P, P, P]
        lib.spec_verify_set_debug_router.argtypes = [P, P]
        lib.spec_verify_step_noalloc.argtypes = [P, P, P, P, P, P, P, P, c_int, P, P, P, P]
        lib.spec_verify_accept_from_logits.argtypes = [P, P, P, P, P, c_int, P, P, P, P]
        U64, U32 = ctypes.c_uint64, ctypes.c_uint32
        lib.spec_verify_step_sampled.argtypes = [P, P, P, P, P, P, P, P, c_float, U64, U32, P, P,
                                                 c_int, P, P, P]
        lib.spec_verify_sample_from_logits.argtypes = [P, P, P, P, P, c_float, U64, U32, P, P,
                                                       c_int, P, P, P]
        lib.spec_verify_error_word.argtypes = [P, P, c_int, P]
        lib.spec_verify_kernel_time.argtypes = [P, c_int, c_int, P, P]
        lib.spec_verify_last_error.argtypes = [c_char_p, c_int]
        lib.spec_verify_status_string.argtypes = [c_int]
        lib.spec_verify_status_string.restype = c_char_p
        lib.spec_verify_abi_version.argtypes = []
        lib.spec_verify_pack_tiled16.argtypes = [P, P, ctypes.c_long, c_int, c_int, P]
        lib.spec_verify_tiled16_bytes.argtypes = [ctypes.c_long, c_int, c_int]
        lib.spec_verify_pack_mx_scales.argtypes = [P, P, ctypes.c_long, c_int, P]
        lib.spec_draft_step.argtypes = [P, P, P, P, P, P, P, P, P, P, c_int, P, P]
        lib.spec_verify_set_kv_pages.argtypes = [P, P]
        lib.spec_verify_mx_scales_bytes.argtypes = [ctypes.c_long, c_int]
        for f in EXPORTS:
            if f not in ("spec_verify_destroy", "spec_verify_status_string"):
                getattr(lib, f).restype = c_int
        lib.spec_verify_tiled16_bytes.restype = ctypes.c_long
        lib.spec_verify_mx_scales_bytes.restype = ctypes.c_long
        _lib = lib
    return _lib


def _check(rc: int, where: str):
    if rc != SV_OK:
        raise SpecVerifyError(rc, where)


def _p(t):
    """Device (or host) address of a tensor, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


# ----------------------------------------------------------- ABI functions
def spec_verify_abi_version() -> int:
    return load_library().spec_verify_abi_version()


def spec_verify_status_string(status: int) -> str:
    return load_library().spec_verify_status_string(status).decode()


def spec_verify_last_error() -> str:
    buf = ctypes.create_string_buffer(1024)
    load_library().spec_verify_last_error(buf, 1024)
    return buf.value.decode(errors="replace")


def make_config(cfg, max_batch: int, kv_capacity: int, kv_page_size: int = 0,
                kv_pool_pages: int = 0) -> SpecVerifyConfig:
    """Config struct from any object with the workload fields (paged KV caches
    when kv_page_size > 0)."""
    c = SpecVerifyConfig()
    c.n_layers, c.hidden, c.n_q_heads, c.n_kv_heads = cfg.n_layers, cfg.hidden, cfg.n_q, cfg.n_kv
    c.head_dim = cfg.head_dim
    c.ffn_kind = SV_FFN_MOE if cfg.ffn == "moe" else SV_FFN_DENSE
    c.n_experts, c.expert_inter, c.top_k = cfg.n_experts, cfg.expert_inter, cfg.top_k
    c.n_shared, c.renorm_topk, c.dense_inter = cfg.n_shared, cfg.renorm_topk, cfg.dense_inter
    c.vocab, c.max_batch, c.k_draft, c.kv_capacity = cfg.vocab, max_batch, cfg.k_draft, kv_capacity
    c.rope_theta, c.rms_eps = cfg.rope_theta, cfg.rms_eps
    c.weight_dtype, c.embed_dtype, c.kv_dtype = _DT[cfg.wdtype], _DT[cfg.embdtype], _DT[cfg.kvdtype]
    c.mx_dtype = SV_MXFP4 if getattr(cfg, "mx", "") == "mxfp4" else 0
    c.kv_page_size, c.kv_pool_pages = kv_page_size, kv_pool_pages
    return c


def spec_verify_init(config: SpecVerifyConfig) -> int:
    """Returns the opaque context handle (an address)."""
    h = c_void_p()
    _check(load_library().spec_verify_init(ctypes.byref(config), ctypes.byref(h)),
           "spec_verify_init")
    return h.value


def spec_verify_destroy(ctx: int) -> None:
    load_library().spec_verify_destroy(ctx)


def spec_verify_tiled16_bytes(rows: int, cols: int, dtype: int) -> int:
    return load_library().spec_verify_tiled16_bytes(rows, cols, dtype)


def spec_verify_pack_tiled16(src, dst, rows: int, cols: int, dtype: int, stream=None) -> None:
    _check(load_library().spec_verify_pack_tiled16(_p(src), _p(dst), rows, cols, dtype,
                                                   _stream(stream)), "spec_verify_pack_tiled16")


def spec_verify_mx_scales_bytes(rows: int, cols: int) -> int:
    return load_library().spec_verify_mx_scales_bytes(rows, cols)


def spec_verify_pack_mx_scales(src, dst, rows: int, cols: int, stream=None) -> None:
    _check(load_library().spec_verify_pack_mx_scales(_p(src), _p(dst), rows, cols,
                                                     _stream(stream)), "spec_verify_pack_mx_scales")


def pack_mx_scales(t, stream=None):
    """E8M0 scale bytes [..., cols/32] (row-major, stacked matrices flattened
    into one tall matrix) repacked by the library; returns a new uint8 tensor."""
    import torch
    cols = t.shape[-1] * 32
    rows = t.numel() // t.shape[-1]
    dst = torch.empty(spec_verify_mx_scales_bytes(rows, cols), dtype=torch.uint8, device=t.device)
    spec_verify_pack_mx_scales(t.contiguous(), dst, rows, cols, stream)
    return dst


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: SV_F32, torch.bfloat16: SV_BF16, torch.uint8: SV_FP8,
            torch.float8_e4m3fn: SV_FP8}[t.dtype]


def pack_matrix(t, stream=None):
    """A device tensor [..., cols] (row-major, stacked matrices flattened into
    one tall matrix) repacked by the library into the tiled16 layout; returns
    a new uint8 tensor of spec_verify_tiled16_bytes bytes."""
    import torch
    cols = t.shape[-1]
    rows = t.numel() // cols
    dt = _dtype_code(t)
    dst = torch.empty(spec_verify_tiled16_bytes(rows, cols, dt), dtype=torch.uint8,
                      device=t.device)
    spec_verify_pack_tiled16(t.contiguous(), dst, rows, cols, dt, stream)
    return dst


MX_MATRICES = ("w_gate_up", "w_down", "w_sh_gate_up", "w_sh_down")


def pack_weights(weights: dict, stream=None, mx: str = "") -> dict:
    """A copy of a weight dict with every matrix-product weight in the
    tiled16 layout (norm gains, fp8 scales and the embedding unchanged); with
    mx = "mxfp4" the block scales of the MXFP4 matrices (experts, LM head)
    are repacked too."""
    out = dict(weights)
    out["layers"] = []
    for L in weights["layers"]:
        L2 = dict(L)
        for name in GEMM_MATRICES:
            if L.get(name) is not None:
                # an empty stack (no shared experts) stays empty: nothing to pack
                L2[name] = pack_matrix(L[name], stream) if L[name].numel() else L[name]
        if mx == "mxfp4":
            for name in MX_MATRICES:
                sk = "s" + name[1:]
                if L.get(sk) is not None and L[sk].numel():
                    L2[sk] = pack_mx_scales(L[sk], stream)
        out["layers"].append(L2)
    out["lm_head"] = pack_matrix(weights["lm_head"], stream)
    if mx == "mxfp4":
        out["lm_scale"] = pack_mx_scales(weights["lm_scale"], stream)
    out["layout"] = "tiled16"
    return out


def make_weights(weights: dict, n_layers: int):
    """Weights struct from a dict of device tensors laid out as the header
    documents (key "layout": "row_major" (default) or "tiled16"); returns
    (struct, keep-alive list)."""
    keep = []
    layers = (SpecVerifyLayer * n_layers)()
    for l, L in enumerate(weights["layers"]):
        lay = layers[l]
        for name, _ in SpecVerifyLayer._fields_:
            t = L.get(name)
            if t is not None:
                keep.append(t)
                setattr(lay, name, t.data_ptr())
    w = SpecVerifyWeights()
    w.embed = weights["embed"].data_ptr()
    w.layers = ctypes.cast(layers, POINTER(SpecVerifyLayer))
    w.final_norm = weights["final_norm"].data_ptr()
    w.lm_head = weights["lm_head"].data_ptr()
    sc = weights.get("lm_scale")
    w.lm_scale = sc.data_ptr() if sc is not None else None
    w.layout = _LAYOUTS[weights.get("layout", "row_major")]
    keep += [layers, weights]
    return w, keep


def spec_verify_step(ctx: int, weights: SpecVerifyWeights, k_cache, v_cache, committed_tok,
                     draft_toks, ctx_lens_in, ctx_lens_out, batch: int, accepted_len, next_tok,
                     stream=None) -> None:
    _check(load_library().spec_verify_step(
        ctx, ctypes.byref(weights), _p(k_cache), _p(v_cache), _p(committed_tok), _p(draft_toks),
        _p(ctx_lens_in), _p(ctx_lens_out), int(batch), _p(accepted_len), _p(next_tok),
        _stream(stream)), "spec_verify_step")


def spec_verify_step_noalloc(config: SpecVerifyConfig, weights: SpecVerifyWeights, k_cache, v_cache,
                             committed_tok, draft_toks, ctx_lens_in, ctx_lens_out, batch: int,
                             accepted_len, next_tok, error_word=None, stream=None) -> None:
    _check(load_library().spec_verify_step_noalloc(
        ctypes.byref(config), ctypes.byref(weights), _p(k_cache), _p(v_cache), _p(committed_tok),
        _p(draft_toks), _p(ctx_lens_in), _p(ctx_lens_out), int(batch), _p(accepted_len),
        _p(next_tok), _p(error_word), _stream(stream)), "spec_verify_step_noalloc")


def spec_verify_set_debug(ctx: int, logits=None, hidden=None, target_tok=None,
                          routing=None) -> None:
    _check(load_library().spec_verify_set_debug(ctx, _p(logits), _p(hidden), _p(target_tok),
                                                _p(routing)), "spec_verify_set_debug")


def spec_verify_set_debug_router(ctx: int, router_logits=None) -> None:
    _check(load_library().spec_verify_set_debug_router(ctx, _p(router_logits)),
           "spec_verify_set_debug_router")


def spec_verify_set_kv_pages(ctx: int, table) -> None:
    _check(load_library().spec_verify_set_kv_pages(ctx, _p(table)), "spec_verify_set_kv_pages")


def kv_paged_from_library(k_cache, v_cache, page: int, order=None):
    """Contiguous tiled caches [B][L][n_kv][cap][D] (the library layout) ->
    page pools [B*cap/page][L][n_kv][page][D] and a page table [B][cap/page]
    (int32): logical page i of sequence b is stored in physical page
    order[b*cap/page + i] (default: the identity).  A pure data movement."""
    import torch
    B, L, H, cap, D = k_cache.shape
    npg = cap // page

    def pool(t):
        p = t.reshape(B, L, H, npg, page, D).permute(0, 3, 1, 2, 4, 5).reshape(B * npg, L, H, page, D)
        if order is None:
            return p.contiguous()
        # a fresh contiguous pool (empty_like would keep a permuted view's strides)
        out = torch.empty(p.shape, dtype=p.dtype, device=p.device)
        out[torch.as_tensor(order, device=t.device)] = p
        return out

    ident = torch.arange(B * npg, dtype=torch.int32, device=k_cache.device)
    table = ident if order is None else torch.as_tensor(order, dtype=torch.int32, device=k_cache.device)
    return pool(k_cache), pool(v_cache), table.reshape(B, npg).contiguous()


def spec_verify_accept_from_logits(ctx: int, logits, draft_toks, ctx_lens_in, ctx_lens_out,
                                   batch: int, accepted_len, next_tok, target_tok=None,
                                   stream=None) -> None:
    _check(load_library().spec_verify_accept_from_logits(
        ctx, _p(logits), _p(draft_toks), _p(ctx_lens_in), _p(ctx_lens_out), int(batch),
        _p(accepted_len), _p(next_tok), _p(target_tok), _stream(stream)),
        "spec_verify_accept_from_logits")


def spec_verify_step_sampled(ctx: int, weights: SpecVerifyWeights, k_cache, v_cache,
                             committed_tok, draft_toks, draft_probs, accept_u, temperature: float,
                             seed: int, offset: int, ctx_lens_in, ctx_lens_out, batch: int,
                             accepted_len, next_tok, stream=None) -> None:
    _check(load_library().spec_verify_step_sampled(
        ctx, ctypes.byref(weights), _p(k_cache), _p(v_cache), _p(committed_tok), _p(draft_toks),
        _p(draft_probs), _p(accept_u), float(temperature), int(seed) & (2 ** 64 - 1),
        int(offset) & 0xFFFFFFFF, _p(ctx_lens_in), _p(ctx_lens_out), int(batch),
        _p(accepted_len), _p(next_tok), _stream(stream)), "spec_verify_step_sampled")


def spec_verify_sample_from_logits(ctx: int, logits, draft_toks, draft_probs, accept_u,
                                   temperature: float, seed: int, offset: int, ctx_lens_in,
                                   ctx_lens_out, batch: int, accepted_len, next_tok,
                                   stream=None) -> None:
    _check(load_library().spec_verify_sample_from_logits(
        ctx, _p(logits), _p(draft_toks), _p(draft_probs), _p(accept_u), float(temperature),
        int(seed) & (2 ** 64 - 1), int(offset) & 0xFFFFFFFF, _p(ctx_lens_in), _p(ctx_lens_out),
        int(batch), _p(accepted_len), _p(next_tok), _stream(stream)),
        "spec_verify_sample_from_logits")


def spec_draft_step(ctx: int, weights: SpecVerifyWeights, mtp: SpecMtpWeights, k_cache, v_cache,
                    verify_ctx: int, ctx_in, accepted_len, next_tok, draft_toks, batch: int,
                    drafts_out, stream=None) -> None:
    _check(load_library().spec_draft_step(
        ctx, ctypes.byref(weights), ctypes.byref(mtp), _p(k_cache), _p(v_cache), verify_ctx,
        _p(ctx_in), _p(accepted_len), _p(next_tok), _p(draft_toks), int(batch), _p(drafts_out),
        _stream(stream)), "spec_draft_step")


def spec_verify_error_word(ctx: int, clear: bool = False, stream=None) -> int:
    v = c_uint32()
    _check(load_library().spec_verify_error_word(ctx, ctypes.byref(v), int(clear),
                                                 _stream(stream)), "spec_verify_error_word")
    return v.value


def spec_verify_kernel_time(ctx: int, kclass: int, enable: int = -1, query: bool = True):
    """enable 1: start/reset recording class `kclass`; 0: stop; -1: keep.
    Returns (total_ms, launches) when query is true."""
    ms, n = c_double(), c_int()
    args = (ctypes.byref(ms), ctypes.byref(n)) if query else (None, None)
    _check(load_library().spec_verify_kernel_time(ctx, kclass, enable, *args),
           "spec_verify_kernel_time")
    return (ms.value, n.value) if query else None


# --------------------------------------------------------------- helpers
def _kv_shape(t):
    esize = t.element_size()
    KL = 16 // esize
    B, L, H, cap, D = t.shape
    if cap % (4 * KL) or D % (4 * KL):
        raise ValueError("capacity and head_dim must be multiples of the key tile")
    return B, L, H, cap, D, KL, KL // 4, D // (4 * KL), cap // (4 * KL)


def kv_to_library(k_cache, v_cache):
    """Caches in the natural order [B][L][n_kv][capacity][D] -> the library's
    tiled layout (a pure permutation; see include/spec_verify.h)."""
    B, L, H, cap, D, KL, NB, DS, NT = _kv_shape(k_cache)
    # K: key r = q*4NB + blk*4 + m, channel d = s*4KL + g*KL + e
    k = k_cache.reshape(B, L, H, NT, 4, NB, 4, DS, 4, KL).permute(0, 1, 2, 3, 5, 7, 8, 4, 6, 9)
    # V: key r = g*KL + e, channel d = 16f + c
    v = v_cache.reshape(B, L, H, NT, 4, KL, D // 16, 16).permute(0, 1, 2, 3, 6, 4, 7, 5)
    return (k.contiguous().reshape(B, L, H, cap, D), v.contiguous().reshape(B, L, H, cap, D))


def kv_from_library(k_cache, v_cache):
    """Inverse of kv_to_library."""
    B, L, H, cap, D, KL, NB, DS, NT = _kv_shape(k_cache)
    k = k_cache.reshape(B, L, H, NT, NB, DS, 4, 4, 4, KL).permute(0, 1, 2, 3, 7, 4, 8, 5, 6, 9)
    v = v_cache.reshape(B, L, H, NT, D // 16, 4, 16, KL).permute(0, 1, 2, 3, 5, 7, 4, 6)
    return (k.contiguous().reshape(B, L, H, cap, D), v.contiguous().reshape(B, L, H, cap, D))


class VerifyContext:
    """Owns one library context; wraps spec_verify_step for torch tensors."""

    def __init__(self, cfg, max_batch: int, kv_capacity: int, weights: dict,
                 layout: str = "tiled16", kv_page_size: int = 0, kv_pool_pages: int = 0):
        """`weights`: row-major device tensors (the workload dict).  With
        layout "tiled16" the matrix-product weights are repacked once by the
        library into a copy owned by this object."""
        self.cfg = cfg
        self.max_batch = max_batch
        self.kv_capacity = kv_capacity
        self._config = make_config(cfg, max_batch, kv_capacity, kv_page_size, kv_pool_pages)
        self.handle = spec_verify_init(self._config)
        if layout == "tiled16" and weights.get("layout", "row_major") == "row_major":
            weights = pack_weights(weights, mx=getattr(cfg, "mx", ""))
        self.weights = weights
        self._w, self._keep = make_weights(weights, cfg.n_layers)

    def step(self, k_cache, v_cache, committed, drafts, ctx_in, ctx_out, accepted, next_tok,
             batch=None, stream=None):
        B = committed.shape[0] if batch is None else batch
        spec_verify_step(self.handle, self._w, k_cache, v_cache, committed, drafts, ctx_in,
                         ctx_out, B, accepted, next_tok, stream)

    def set_kv_pages(self, table):
        self._kv_table = table
        spec_verify_set_kv_pages(self.handle, table)

    def set_debug(self, logits=None, hidden=None, target_tok=None, routing=None):
        self._dbg = (logits, hidden, target_tok, routing)
        spec_verify_set_debug(self.handle, logits, hidden, target_tok, routing)

    def set_debug_router(self, router_logits=None):
        self._dbg_router = router_logits
        spec_verify_set_debug_router(self.handle, router_logits)

    def accept_from_logits(self, logits, drafts, ctx_in, ctx_out, accepted, next_tok,
                           target_tok=None, stream=None):
        spec_verify_accept_from_logits(self.handle, logits, drafts, ctx_in, ctx_out,
                                       drafts.shape[0], accepted, next_tok, target_tok, stream)

    def step_sampled(self, k_cache, v_cache, committed, drafts, draft_probs, accept_u,
                     temperature, seed, offset, ctx_in, ctx_out, accepted, next_tok,
                     batch=None, stream=None):
        B = committed.shape[0] if batch is None else batch
        spec_verify_step_sampled(self.handle, self._w, k_cache, v_cache, committed, drafts,
                                 draft_probs, accept_u, temperature, seed, offset, ctx_in,
                                 ctx_out, B, accepted, next_tok, stream)

    def sample_from_logits(self, logits, drafts, draft_probs, accept_u, temperature, seed,
                           offset, ctx_in, ctx_out, accepted, next_tok, stream=None):
        spec_verify_sample_from_logits(self.handle, logits, drafts, draft_probs, accept_u,
                                       temperature, seed, offset, ctx_in, ctx_out,
                                       drafts.shape[0], accepted, next_tok, stream)

    def error_word(self, clear=False, stream=None) -> int:
        return spec_verify_error_word(self.handle, clear, stream)

    def kernel_time(self, kclass, enable=-1, query=True):
        return spec_verify_kernel_time(self.handle, kclass, enable, query)

    def close(self):
        if self.handle:
            spec_verify_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DraftContext:
    """Owns a library context for the FastMTP draft block; wraps
    spec_draft_step.  `cfg` is the block's one-layer dense shape, `target`
    the target's weight dict (its embedding, final norm and LM head are
    used; already tiled16-packed ones are taken as they are), `mtp` the draft
    head's weights (enorm, hnorm, eh_proj (+ s_eh_proj), block)."""

    def __init__(self, cfg, max_batch: int, kv_capacity: int, target: dict, mtp: dict,
                 layout: str = "tiled16"):
        self.cfg = cfg
        self.handle = spec_verify_init(make_config(cfg, max_batch, kv_capacity))
        block = dict(mtp["block"])
        P = mtp["eh_proj"]
        tl = target.get("layout", "row_major")
        if layout == "tiled16":
            for name in GEMM_MATRICES:
                if block.get(name) is not None:
                    block[name] = pack_matrix(block[name])
            P = pack_matrix(P)
            if tl == "row_major":
                target = pack_weights(target)
        elif tl != "row_major":
            raise ValueError("row-major draft weights need a row-major target")
        self.weights = {"embed": target["embed"], "layers": [block],
                        "final_norm": target["final_norm"], "lm_head": target["lm_head"],
                        "lm_scale": target.get("lm_scale"), "layout": layout}
        self._w, self._keep = make_weights(self.weights, 1)
        self._mtp = SpecMtpWeights()
        self._mtp.enorm = mtp["enorm"].data_ptr()
        self._mtp.hnorm = mtp["hnorm"].data_ptr()
        self._mtp.eh_proj = P.data_ptr()
        s = mtp.get("s_eh_proj")
        self._mtp.s_eh_proj = s.data_ptr() if s is not None else None
        self._keep += [mtp, P]

    def draft(self, k_cache, v_cache, verify_ctx, ctx_in, accepted, next_tok, drafts_in,
              drafts_out, batch=None, stream=None):
        B = accepted.shape[0] if batch is None else batch
        vh = verify_ctx.handle if hasattr(verify_ctx, "handle") else verify_ctx
        spec_draft_step(self.handle, self._w, self._mtp, k_cache, v_cache, vh, ctx_in, accepted,
                        next_tok, drafts_in, B, drafts_out, stream)

    def error_word(self, clear=False, stream=None) -> int:
        return spec_verify_error_word(self.handle, clear, stream)

    def close(self):
        if self.handle:
            spec_verify_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
