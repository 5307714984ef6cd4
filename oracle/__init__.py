"""CPU oracle of the greedy speculative-decoding verify step -- TEST INFRASTRUCTURE.

A thin ctypes wrapper around oracle.c (plain fp64 loops).  Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import this package;
the HIP library and its binding never do.  Parity claims rest on this code
being independent of the GPU path: it shares no source with it.

Inputs are numpy arrays or CPU torch tensors as produced by the `workloads`
package: fp32 arrays, bf16 tensors (passed as their uint16 bit patterns),
fp8 e4m3fn codes (uint8) with fp32 per-row scales.  KV caches use the natural
layout [B][L][n_kv][capacity][D].
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from ctypes import POINTER, c_double, c_int, c_long, c_ubyte, c_void_p

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_SANITIZE=1 loads a build instrumented with AddressSanitizer and
# UndefinedBehaviorSanitizer (host code only; run Python with the ASan runtime
# preloaded, see build())
_SANITIZE = os.environ.get("ORACLE_SANITIZE", "") == "1"
_LIB = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")

F32, BF16, FP8, MXFP4 = 0, 1, 2, 3
_DT = {"f32": F32, "bf16": BF16, "fp8": FP8, "mxfp4": MXFP4}
# matrices stored in the workload's `mx` format when it names one (the
# weight-streaming ones: the LM head, and a MoE model's experts)
MX_MATRICES = ("w_gate_up", "w_down", "w_sh_gate_up", "w_sh_down", "lm_head")
BAD_TOKEN, CAPACITY, NAN_LOGIT = 1, 2, 4


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, OpenMP, no
    fast-math, no floating-point contraction).  With ORACLE_SANITIZE=1 the
    library is liboracle_san.so, built with -fsanitize=address,undefined
    (aborting on the first report); load it with the ASan runtime preloaded:
      ORACLE_SANITIZE=1 ASAN_OPTIONS=detect_leaks=0 \
      LD_PRELOAD=$(gcc -print-file-name=libasan.so) python -m pytest tests/test_oracle_pins.py"""
    if force or not os.path.exists(_LIB):
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-fno-omit-frame-pointer", "-g"] if _SANITIZE else []
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", *san, "-shared",
               "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("n_layers", c_int), ("hidden", c_int), ("n_q", c_int), ("n_kv", c_int),
                ("head_dim", c_int), ("ffn_kind", c_int), ("n_experts", c_int),
                ("expert_inter", c_int), ("top_k", c_int), ("n_shared", c_int),
                ("renorm_topk", c_int), ("dense_inter", c_int), ("vocab", c_int),
                ("k_draft", c_int), ("capacity", c_int), ("rope_theta", c_double),
                ("rms_eps", c_double), ("wdtype", c_int), ("embdtype", c_int),
                ("kvdtype", c_int)]


class _Mat(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("scale", c_void_p), ("dtype", c_int)]


class _Layer(ctypes.Structure):
    _fields_ = [("attn_norm", c_void_p), ("w_qkv", _Mat), ("w_o", _Mat), ("ffn_norm", c_void_p),
                ("w_router", _Mat), ("w_gate_up", _Mat), ("w_down", _Mat),
                ("w_sh_gate_up", _Mat), ("w_sh_down", _Mat), ("w_dense_gate_up", _Mat),
                ("w_dense_down", _Mat)]


class _RouteIO(ctypes.Structure):
    _fields_ = [("force", c_void_p), ("sel_out", c_void_p), ("rlogits_out", c_void_p)]


class _Weights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("layers", POINTER(_Layer)), ("final_norm", c_void_p),
                ("lm_head", _Mat)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = c_void_p
        lib.or_verify_step.argtypes = [P, P, P, P, c_int, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.or_verify_step.restype = None
        lib.or_decode_one.argtypes = [P, P, P, P, c_long, c_long, c_int, P, P]
        lib.or_decode_one.restype = c_int
        lib.or_make_drafts.argtypes = [P, P, P, P, c_long, c_long, c_int, P, P, P]
        lib.or_make_drafts.restype = None
        lib.or_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.or_bf16_to_double.restype = c_double
        lib.or_e4m3_to_double.argtypes = [c_ubyte]
        lib.or_e4m3_to_double.restype = c_double
        lib.or_e2m1_to_double.argtypes = [c_ubyte]
        lib.or_e2m1_to_double.restype = c_double
        lib.or_e8m0_to_double.argtypes = [c_ubyte]
        lib.or_e8m0_to_double.restype = c_double
        lib.or_round_bf16.argtypes = [c_double]
        lib.or_round_bf16.restype = c_double
        lib.or_matvec.argtypes = [P, P, c_int, c_long, c_int, c_int, P, P]
        lib.or_rmsnorm.argtypes = [P, P, c_int, c_double, P]
        lib.or_rope.argtypes = [P, c_int, c_long, c_double]
        lib.or_attend.argtypes = [P, P, P, c_int, c_int, c_long, P, P]
        lib.or_softmax.argtypes = [P, c_int, P]
        lib.or_topk.argtypes = [P, c_int, c_int, P]
        lib.or_silu.argtypes = [c_double]
        lib.or_silu.restype = c_double
        lib.or_ffn.argtypes = [P, P, P, P, P, P, P]
        lib.or_argmax.argtypes = [P, c_long]
        lib.or_argmax.restype = c_int
        lib.or_accept.argtypes = [c_int, P, P, P, P]
        lib.or_forward_rows.argtypes = [P, P, P, P, c_long, c_long, c_int, P, P, P, P]
        lib.or_forward_rows.restype = None
        lib.or_mtp_draft.argtypes = [P, P, P, P, P, P, P, c_long, c_long, c_int, P, c_int, P, P, P]
        lib.or_mtp_draft.restype = None
        lib.or_num_threads.argtypes = []
        lib.or_num_threads.restype = c_int
        for f in ("or_matvec", "or_rmsnorm", "or_rope", "or_attend", "or_softmax", "or_topk",
                  "or_ffn", "or_accept"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def lib():
    return _load()


def as_np(t) -> np.ndarray:
    """Contiguous numpy view of a CPU tensor / array; bf16 becomes its uint16
    bit pattern, fp8 codes stay uint8."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return np.ascontiguousarray(t)
    if isinstance(t, (list, tuple, int)):
        return np.asarray(t)
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(c_void_p)


class Oracle:
    """The verify step for one weight set.  `cfg` is any object with the
    workload fields (n_layers, hidden, n_q, n_kv, head_dim, ffn, n_experts,
    expert_inter, top_k, n_shared, renorm_topk, dense_inter, vocab, k_draft,
    rope_theta, rms_eps, wdtype, embdtype, kvdtype)."""

    def __init__(self, cfg, weights: dict, capacity: int):
        self.cfg = cfg
        self.capacity = int(capacity)
        self._keep = []
        c = _Cfg()
        c.n_layers, c.hidden, c.n_q, c.n_kv = cfg.n_layers, cfg.hidden, cfg.n_q, cfg.n_kv
        c.head_dim = cfg.head_dim
        c.ffn_kind = 0 if cfg.ffn == "moe" else 1
        c.n_experts, c.expert_inter, c.top_k = cfg.n_experts, cfg.expert_inter, cfg.top_k
        c.n_shared, c.renorm_topk, c.dense_inter = cfg.n_shared, cfg.renorm_topk, cfg.dense_inter
        c.vocab, c.k_draft, c.capacity = cfg.vocab, cfg.k_draft, self.capacity
        c.rope_theta, c.rms_eps = cfg.rope_theta, cfg.rms_eps
        c.wdtype, c.embdtype, c.kvdtype = _DT[cfg.wdtype], _DT[cfg.embdtype], _DT[cfg.kvdtype]
        self._c = c
        layers = (_Layer * cfg.n_layers)()
        for l, L in enumerate(weights["layers"]):
            lay = layers[l]
            lay.attn_norm = self._p(L["attn_norm"], np.float32)
            lay.ffn_norm = self._p(L["ffn_norm"], np.float32)
            lay.w_qkv = self._m(L, "w_qkv", "s_qkv")
            lay.w_o = self._m(L, "w_o", "s_o")
            if cfg.ffn == "moe":
                lay.w_router = self._m(L, "w_router", "s_router")
                lay.w_gate_up = self._m(L, "w_gate_up", "s_gate_up")
                lay.w_down = self._m(L, "w_down", "s_down")
                lay.w_sh_gate_up = self._m(L, "w_sh_gate_up", "s_sh_gate_up")
                lay.w_sh_down = self._m(L, "w_sh_down", "s_sh_down")
            else:
                lay.w_dense_gate_up = self._m(L, "w_gate_up", "s_gate_up")
                lay.w_dense_down = self._m(L, "w_down", "s_down")
        self._layers = layers
        w = _Weights()
        w.embed = self._p(weights["embed"])
        w.layers = ctypes.cast(layers, POINTER(_Layer))
        w.final_norm = self._p(weights["final_norm"], np.float32)
        w.lm_head = self._m(weights, "lm_head", "lm_scale")
        self._w = w

    def _p(self, t, dtype=None):
        a = as_np(t)
        if dtype is not None:
            a = np.ascontiguousarray(a, dtype=dtype)
        self._keep.append(a)
        return _ptr(a)

    def _m(self, d, wkey, skey):
        m = _Mat()
        m.data = self._p(d[wkey])
        s = d.get(skey)
        mx = getattr(self.cfg, "mx", "") == "mxfp4" and (
            wkey == "lm_head" or (self.cfg.ffn == "moe" and wkey in MX_MATRICES))
        m.dtype = MXFP4 if mx else -1
        if s is None:
            m.scale = None
        else:
            m.scale = self._p(s, np.uint8) if mx else self._p(s, np.float32)
        return m

    # ------------------------------------------------------------------ API
    def kv_np(self, k_cache, v_cache):
        """Writable numpy copies of the caches (natural layout)."""
        return np.array(as_np(k_cache), copy=True), np.array(as_np(v_cache), copy=True)

    def verify_step(self, k_cache: np.ndarray, v_cache: np.ndarray, committed, drafts, ctx_in,
                    want_logits=False, want_hidden=False, want_layer_hidden=False,
                    force_sel=None, want_routing=False) -> dict:
        """One verify step; caches (numpy, natural layout) are updated in place.
        force_sel [B][L][K+1][top_k] replaces the experts' top-k choice (test
        hook); want_routing returns the selections used ("sel") and the
        router logits ("router_logits")."""
        cfg = self.cfg
        K = cfg.k_draft
        com = np.ascontiguousarray(as_np(committed), dtype=np.int32).reshape(-1)
        B = com.shape[0]
        dr = np.ascontiguousarray(as_np(drafts), dtype=np.int32).reshape(B, K)
        ci = np.ascontiguousarray(as_np(ctx_in), dtype=np.int32).reshape(B)
        out = {k: np.zeros(B, np.int32) for k in ("ctx_out", "accepted", "next_tok", "status")}
        out["target"] = np.zeros((B, K + 1), np.int32)
        logits = np.zeros((B, K + 1, cfg.vocab)) if want_logits else None
        hidden = np.zeros((B, K + 1, cfg.hidden)) if want_hidden else None
        lh = np.zeros((B, cfg.n_layers, K + 1, cfg.hidden)) if want_layer_hidden else None
        self._check_kv(k_cache, v_cache, B)
        rio = _RouteIO()
        moe = cfg.ffn == "moe"
        fs = sel = rl = None
        if moe and force_sel is not None:
            fs = np.ascontiguousarray(force_sel, dtype=np.int32).reshape(
                B, cfg.n_layers, K + 1, cfg.top_k)
            if fs.min() < 0 or fs.max() >= cfg.n_experts:
                raise ValueError("forced expert out of range")
            rio.force = _ptr(fs)
        if moe and want_routing:
            sel = np.zeros((B, cfg.n_layers, K + 1, cfg.top_k), np.int32)
            rl = np.zeros((B, cfg.n_layers, K + 1, cfg.n_experts))
            rio.sel_out, rio.rlogits_out = _ptr(sel), _ptr(rl)
        _load().or_verify_step(ctypes.byref(self._c), ctypes.byref(self._w), _ptr(k_cache),
                               _ptr(v_cache), B, _ptr(com), _ptr(dr), _ptr(ci),
                               _ptr(out["ctx_out"]), _ptr(out["accepted"]),
                               _ptr(out["next_tok"]), _ptr(out["status"]), _ptr(out["target"]),
                               _ptr(logits), _ptr(hidden), _ptr(lh), ctypes.byref(rio))
        if sel is not None:
            out["sel"], out["router_logits"] = sel, rl
        if want_logits:
            out["logits"] = logits
        if want_hidden:
            out["hidden"] = hidden
        if want_layer_hidden:
            out["layer_hidden"] = lh
        return out

    def decode_one(self, k_cache, v_cache, b: int, pos: int, tok: int, want_logits=False):
        """Plain single-token greedy decode; returns (token, logits or None, hidden)."""
        logits = np.zeros(self.cfg.vocab) if want_logits else None
        hidden = np.zeros(self.cfg.hidden)
        g = _load().or_decode_one(ctypes.byref(self._c), ctypes.byref(self._w), _ptr(k_cache),
                                  _ptr(v_cache), b, pos, int(tok), _ptr(logits), _ptr(hidden))
        return g, logits, hidden

    def make_drafts(self, k_cache, v_cache, b: int, ctx: int, committed: int, coins, rand_tok):
        K = self.cfg.k_draft
        co = np.ascontiguousarray(as_np(coins), dtype=np.uint8).reshape(K)
        rt = np.ascontiguousarray(as_np(rand_tok), dtype=np.int32).reshape(K)
        out = np.zeros(K, np.int32)
        _load().or_make_drafts(ctypes.byref(self._c), ctypes.byref(self._w), _ptr(k_cache),
                               _ptr(v_cache), b, ctx, int(committed), _ptr(co), _ptr(rt),
                               _ptr(out))
        return out

    def forward_rows(self, k_cache, v_cache, b: int, ctx: int, x_in, want_logits=False):
        """The decoder on given residual rows x_in [n][H] at positions ctx ..
        ctx+n-1 of sequence b (caches updated); returns (final-normed rows
        [n][H], logits [n][V] or None, greedy tokens [n])."""
        x = np.ascontiguousarray(x_in, dtype=np.float64)
        n = x.shape[0]
        f = np.zeros((n, self.cfg.hidden))
        lg = np.zeros((n, self.cfg.vocab)) if want_logits else None
        am = np.zeros(n, np.int32)
        _load().or_forward_rows(ctypes.byref(self._c), ctypes.byref(self._w), _ptr(k_cache),
                                _ptr(v_cache), b, ctx, n, _ptr(x), _ptr(f), _ptr(lg), _ptr(am))
        return f, lg, am

    def mtp_draft(self, mtp: dict, k_cache, v_cache, b: int, ctx: int, accepted: int, drafts,
                  next_tok: int, bstate):
        """FastMTP drafting after a verify step (Jina-OCR-v1 paper, section
        3.1), with this oracle's model as the shared draft block: `mtp` holds
        enorm [H], hnorm [H] (fp32 gains) and eh_proj [H][2H] (+ s_eh_proj for
        fp8); bstate [accepted+1][H] are the target's post-norm rows of
        positions ctx .. ctx+accepted.  Returns (drafts [K], gaps [K])."""
        K = self.cfg.k_draft
        a = int(accepted)
        m = self._m(mtp, "eh_proj", "s_eh_proj")
        ge = np.ascontiguousarray(as_np(mtp["enorm"]), dtype=np.float32)
        gh = np.ascontiguousarray(as_np(mtp["hnorm"]), dtype=np.float32)
        dr = np.ascontiguousarray(as_np(drafts), dtype=np.int32).reshape(K)
        bs = np.ascontiguousarray(bstate, dtype=np.float64).reshape(a + 1, self.cfg.hidden)
        out = np.zeros(K, np.int32)
        gaps = np.zeros(K)
        _load().or_mtp_draft(ctypes.byref(self._c), ctypes.byref(self._w), _ptr(ge), _ptr(gh),
                             ctypes.byref(m), _ptr(k_cache), _ptr(v_cache), b, ctx, a, _ptr(dr),
                             int(next_tok), _ptr(bs), _ptr(out), _ptr(gaps))
        return out, gaps

    def _check_kv(self, k, v, B):
        cfg = self.cfg
        shape = (cfg.n_layers, cfg.n_kv, self.capacity, cfg.head_dim)
        for a in (k, v):
            if not isinstance(a, np.ndarray) or not a.flags.c_contiguous:
                raise TypeError("caches must be C-contiguous numpy arrays")
            if tuple(a.shape[1:]) != shape or a.shape[0] < B:
                raise ValueError(f"cache shape {a.shape} does not hold [B>={B}]{shape}")
            want = np.float32 if cfg.kvdtype == "f32" else np.uint16
            if a.dtype != want:
                raise TypeError(f"cache dtype {a.dtype}, expected {want}")


# ------------------------------------------------------------- primitives
def _d(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def rmsnorm(x, g, eps):
    x, g = _d(x), np.ascontiguousarray(g, dtype=np.float32)
    y = np.zeros_like(x)
    _load().or_rmsnorm(_ptr(x), _ptr(g), x.shape[0], eps, _ptr(y))
    return y


def rope(v, pos, theta):
    v = np.array(v, dtype=np.float64, copy=True)
    _load().or_rope(_ptr(v), v.shape[0], pos, theta)
    return v


def attend(q, keys, values, kvdtype="f32"):
    """q [D]; keys/values [n][D] (fp32, or bf16 bit patterns)."""
    q = _d(q)
    dt = np.float32 if kvdtype == "f32" else np.uint16
    keys, values = np.ascontiguousarray(keys, dtype=dt), np.ascontiguousarray(values, dtype=dt)
    n, D = keys.shape
    out, scratch = np.zeros(D), np.zeros(n)
    _load().or_attend(_ptr(q), _ptr(keys), _ptr(values), _DT[kvdtype], D, n, _ptr(out),
                      _ptr(scratch))
    return out


def softmax(r):
    r = _d(r)
    p = np.zeros_like(r)
    _load().or_softmax(_ptr(r), r.shape[0], _ptr(p))
    return p


def topk(v, k):
    v = _d(v)
    idx = np.zeros(k, np.int32)
    _load().or_topk(_ptr(v), v.shape[0], k, _ptr(idx))
    return idx


def silu(z):
    return _load().or_silu(float(z))


def matvec(W, x, dtype="f32", scale=None):
    """y = W x.  mxfp4: W is the packed code matrix [N][K/2] (uint8) and
    scale the E8M0 block scales [N][K/32] (uint8)."""
    Wn = as_np(W)
    x = _d(x)
    N = Wn.shape[0]
    K = Wn.shape[1] * (2 if dtype == "mxfp4" else 1)
    y = np.zeros(N)
    sdt = np.uint8 if dtype == "mxfp4" else np.float32
    sc = None if scale is None else np.ascontiguousarray(as_np(scale), dtype=sdt)
    _load().or_matvec(_ptr(Wn), _ptr(sc), _DT[dtype], 0, N, K, _ptr(x), _ptr(y))
    return y


def argmax(logits):
    lg = _d(logits)
    return _load().or_argmax(_ptr(lg), lg.shape[0])


def accept(g, d):
    g = np.ascontiguousarray(g, dtype=np.int32)
    d = np.ascontiguousarray(d, dtype=np.int32)
    a, n = c_int(), c_int()
    _load().or_accept(d.shape[0], _ptr(g), _ptr(d), ctypes.byref(a), ctypes.byref(n))
    return a.value, n.value


def bf16_to_double(bits: int) -> float:
    return _load().or_bf16_to_double(bits)


def e4m3_to_double(code: int) -> float:
    return _load().or_e4m3_to_double(code)


def e2m1_to_double(code: int) -> float:
    return _load().or_e2m1_to_double(code)


def e8m0_to_double(code: int) -> float:
    return _load().or_e8m0_to_double(code)


def round_bf16(x: float) -> float:
    return _load().or_round_bf16(x)


def ffn(orc: Oracle, layer: int, h):
    """Feed-forward half of layer `layer` on the normalised input h[H];
    returns (y, selected experts or None)."""
    h = _d(h)
    y = np.zeros_like(h)
    k = max(orc.cfg.top_k, 1)
    sel = np.zeros(k, np.int32)
    lay = ctypes.byref(orc._layers[layer])
    _load().or_ffn(ctypes.byref(orc._c), lay, _ptr(h), _ptr(y), None, _ptr(sel), None)
    return y, (sel if orc.cfg.ffn == "moe" else None)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return _load().or_num_threads()
