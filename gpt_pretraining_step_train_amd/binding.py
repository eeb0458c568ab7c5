"""Thin ctypes binding of libgptmi.so (argument marshalling only).

Every step of the training step runs in the HIP library; torch is used for
device memory (the arena and token buffers) and for the current stream.  The
binding raises if the library is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# GPTMI_LIB selects another build of the same library (the host-sanitizer build of the CPU tests)
LIB_PATH = os.environ.get("GPTMI_LIB") or os.path.join(HERE, "libgptmi.so")

GPT_FP32, GPT_BF16, GPT_FP8 = 0, 1, 2
PREC = {"fp32": GPT_FP32, "bf16": GPT_BF16, "fp8": GPT_FP8}


class GptCfg(ctypes.Structure):
    _fields_ = [
        ("depth", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_head", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("seq_len", ctypes.c_int32), ("batch", ctypes.c_int32), ("precision", ctypes.c_int32),
        ("init_std", ctypes.c_float), ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float),
        ("muon_momentum", ctypes.c_float), ("ns_steps", ctypes.c_int32),
        ("ns_coeffs", (ctypes.c_float * 3) * 5), ("num_steps", ctypes.c_int64),
        ("ns_split_steps", ctypes.c_int32), ("fp8_gemms", ctypes.c_int32), ("attn_window", ctypes.c_int32),
        ("n_kv_head", ctypes.c_int32), ("extras", ctypes.c_int32), ("normuon_beta2", ctypes.c_float),
    ]

    def coeffs(self):
        return [tuple(self.ns_coeffs[i][j] for j in range(3)) for i in range(5)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_long
_SZ = ctypes.c_size_t
_F = ctypes.c_float

_SIGS = {
    "gpt_cfg_from_depth": (_I, [ctypes.c_int32, ctypes.POINTER(GptCfg)]),
    "gpt_cfg_validate": (_I, [ctypes.POINTER(GptCfg)]),
    "gpt_state_bytes": (_SZ, [ctypes.POINTER(GptCfg)]),
    "gpt_init": (_I, [ctypes.POINTER(GptCfg), ctypes.c_uint64, _P, _SZ, _P, ctypes.POINTER(_P)]),
    "gpt_step": (_F, [_P, _P, _P, ctypes.POINTER(GptCfg), _P]),
    "gpt_step_accumulate": (_F, [_P, _P, _P, ctypes.POINTER(GptCfg), _I, _F, _P]),
    "gpt_step_async": (_I, [_P, _P, _P, ctypes.POINTER(GptCfg), _I, _F, _P]),
    "gpt_step_result": (_F, [_P, _P]),
    "gpt_grads": (_I, [_P, ctypes.c_int32, _P, _SZ, _P]),
    "muon_update": (_I, [_P, _F, _P]),
    "adamw_update": (_I, [_P, _F, _F, _F, _F, _F, _P]),
    "gpt_argmax": (_I, [_P, _P, _P]),
    "gpt_row_loss": (_I, [_P, _P, _P]),
    "gpt_get_params": (_I, [_P, ctypes.c_int32, _P, _SZ, _P]),
    "gpt_set_params": (_I, [_P, ctypes.c_int32, _P, _SZ, _P]),
    "gpt_set_grads": (_I, [_P, ctypes.c_int32, _P, _SZ, _P]),
    "gpt_get_momentum": (_I, [_P, ctypes.c_int32, _P, _SZ, _P]),
    "gpt_set_momentum": (_I, [_P, ctypes.c_int32, _P, _SZ, _P]),
    "gpt_tensor_count": (_I, [ctypes.POINTER(GptCfg)]),
    "gpt_cfg_bytes": (_SZ, []),
    "gpt_tensor_shape": (_I, [ctypes.POINTER(GptCfg), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                              ctypes.POINTER(ctypes.c_int32)]),
    "gpt_last_status": (_I, [_P]),
    "gpt_status_str": (ctypes.c_char_p, [_I]),
    "gpt_free": (None, [_P]),
    "gpt_prof_enable": (_I, [_P, ctypes.c_char_p]),
    "gpt_prof_read": (_I, [_P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double),
                           ctypes.POINTER(ctypes.c_double)]),
    "gpt_capture_bytes": (_SZ, [ctypes.POINTER(GptCfg), ctypes.c_int32]),
    "gpt_capture": (_I, [_P, ctypes.c_int32, _P, _SZ]),
    "gptk_gemm_auto_splits": (_I, [_I, _I, _I, _I, _I, _I, _I]),
    "gptk_gemm": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _L, _L, _P, _L, _L, _P, _L, _L, _I, _I, _P, _SZ, _P]),
    "gptk_gemm_split": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _L, _L, _P, _P, _L, _L, _P, _L, _L, _P]),
    "gptk_ns_ws_bytes": (_SZ, [_I, _I]),
    "gptk_newton_schulz": (_I, [_I, _P, _I, _I, _P, _I, _P, _P, _SZ, _P]),
    "gptk_quant_e4m3": (_I, [_I, _P, _I, _I, _L, _P, _P, _P, _P, _P]),
    "gptk_gemm_fp8": (_I, [_I, _I, _I, _P, _L, _P, _L, _P, _P, _P, _L, _I, _P, _SZ, _P]),
    "gpt_gemm_kernel_name": (ctypes.c_char_p, [_I, _I, _I, _I, _I, _I, _I]),
    "gptk_attn_variant": (_I, [_I, _I]),
    "gptk_ce_variant": (_I, [_I]),
    "gptk_fp8_fused_amax": (_I, [_I]),
    "gptk_side_stream": (_I, [_I]),
    "gptk_attn_fwd": (_I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "gptk_attn_fwd_qknorm": (_I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "gptk_attn_bwd": (_I, [_I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "gptk_attn_bwd_noalloc": (_I, [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "gptk_rmsnorm_fwd": (_I, [_I, _P, _P, _P, _I, _I, _F, _P]),
    "gptk_rmsnorm_bwd": (_I, [_I, _P, _P, _P, _P, _P, _P, _I, _I, _P]),
    "gptk_rope_qknorm_fwd": (_I, [_I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _P]),
    "gptk_rope_qknorm_bwd": (_I, [_I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "gptk_cross_entropy": (_I, [_I, _P, _P, _P, _P, _P, _I, _I, _F, _P, _P]),
    "gptk_embed_gather": (_I, [_P, _P, _P, _I, _I, _I, _P, _P]),
    "gptk_embed_ws_bytes": (_SZ, [_I, _I, _I]),
    "gptk_embed_scatter": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P]),
}

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class GptError(RuntimeError):
    pass


def check(rc: int, what: str = ""):
    if rc != 0:
        raise GptError(f"{what}: {lib().gpt_status_str(rc).decode()} ({rc})")


def make_cfg(c: dict) -> GptCfg:
    """Build a gpt_cfg from a config dict (shapes + optional overrides)."""
    cfg = GptCfg()
    check(lib().gpt_cfg_from_depth(int(c["depth"]), ctypes.byref(cfg)), "gpt_cfg_from_depth")
    for k in ("d_model", "n_head", "head_dim", "d_ff", "vocab", "seq_len", "batch"):
        setattr(cfg, k, int(c[k]))
    p = c.get("precision", "bf16")
    cfg.precision = PREC[p] if isinstance(p, str) else int(p)
    for k in ("init_std", "rope_base", "norm_eps", "muon_momentum"):
        if k in c:
            setattr(cfg, k, float(c[k]))
    if "ns_steps" in c:
        cfg.ns_steps = int(c["ns_steps"])
    if "ns_split_steps" in c:
        cfg.ns_split_steps = int(c["ns_split_steps"])
    if "fp8_gemms" in c:
        cfg.fp8_gemms = int(c["fp8_gemms"])
    if "attn_window" in c:
        cfg.attn_window = int(c["attn_window"])
    if "n_kv_head" in c:
        cfg.n_kv_head = int(c["n_kv_head"])
    if "extras" in c:
        cfg.extras = int(c["extras"])
    if "normuon_beta2" in c:
        cfg.normuon_beta2 = float(c["normuon_beta2"])
    if "ns_coeffs" in c:
        for i, abc in enumerate(c["ns_coeffs"]):
            for j in range(3):
                cfg.ns_coeffs[i][j] = float(abc[j])
    return cfg


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


class Model:
    """One GPT training state in a caller-owned (torch) device arena."""

    def __init__(self, c: dict, seed: int = 0, device: str = "cuda"):
        import torch
        self.c = dict(c)
        self.cfg = make_cfg(c)
        check(lib().gpt_cfg_validate(ctypes.byref(self.cfg)), "gpt_cfg_validate")
        nbytes = lib().gpt_state_bytes(ctypes.byref(self.cfg))
        self.arena = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        base = self.arena.data_ptr()
        off = (-base) % 256
        self._h = ctypes.c_void_p()
        check(lib().gpt_init(ctypes.byref(self.cfg), seed, ctypes.c_void_p(base + off), nbytes, _stream(),
                             ctypes.byref(self._h)), "gpt_init")
        self.ntensors = lib().gpt_tensor_count(ctypes.byref(self.cfg))

    def __del__(self):
        try:
            if self._h:
                lib().gpt_free(self._h)
                self._h = ctypes.c_void_p()
        except Exception:
            pass

    def shape(self, tid: int) -> tuple[int, int]:
        r, c = ctypes.c_int32(), ctypes.c_int32()
        check(lib().gpt_tensor_shape(ctypes.byref(self.cfg), tid, ctypes.byref(r), ctypes.byref(c)),
              "gpt_tensor_shape")
        return r.value, c.value

    def step(self, tokens, targets, accumulate: bool = False, grad_scale: float = 1.0) -> float:
        """tokens/targets: int32 device tensors [batch, seq_len].  With the defaults this
        is gpt_step; otherwise gpt_step_accumulate."""
        if not accumulate and grad_scale == 1.0:
            loss = lib().gpt_step(self._h, _ptr(tokens), _ptr(targets), ctypes.byref(self.cfg), _stream())
            what = "gpt_step"
        else:
            loss = lib().gpt_step_accumulate(self._h, _ptr(tokens), _ptr(targets), ctypes.byref(self.cfg),
                                             int(bool(accumulate)), float(grad_scale), _stream())
            what = "gpt_step_accumulate"
        st = lib().gpt_last_status(self._h)
        if st != 0:
            raise GptError(f"{what}: {lib().gpt_status_str(st).decode()} ({st})")
        return loss

    def step_async(self, tokens, targets, accumulate: bool = False, grad_scale: float = 1.0):
        """gpt_step_async: enqueue the step on the current stream (no synchronisation)."""
        check(lib().gpt_step_async(self._h, _ptr(tokens), _ptr(targets), ctypes.byref(self.cfg),
                                   int(bool(accumulate)), float(grad_scale), _stream()), "gpt_step_async")

    def step_result(self) -> float:
        """gpt_step_result: synchronise and return the last enqueued step's loss."""
        loss = lib().gpt_step_result(self._h, _stream())
        st = lib().gpt_last_status(self._h)
        if st != 0:
            raise GptError(f"gpt_step_result: {lib().gpt_status_str(st).decode()} ({st})")
        return loss

    def muon_update(self, lr: float):
        check(lib().muon_update(self._h, float(lr), _stream()), "muon_update")

    def adamw_update(self, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float):
        check(lib().adamw_update(self._h, float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                                 _stream()), "adamw_update")

    def _host_io(self, fn, tid, arr=None):
        r, c = self.shape(tid)
        if arr is None:
            out = np.empty((r, c), dtype=np.float32)
            check(fn(self._h, tid, out.ctypes.data_as(ctypes.c_void_p), out.size, _stream()), fn.__name__)
            return out
        a = np.ascontiguousarray(arr, dtype=np.float32).reshape(r, c)
        check(fn(self._h, tid, a.ctypes.data_as(ctypes.c_void_p), a.size, _stream()), fn.__name__)
        return None

    def grads(self, tid):
        return self._host_io(lib().gpt_grads, tid)

    def get_params(self, tid):
        return self._host_io(lib().gpt_get_params, tid)

    def set_params(self, tid, arr):
        self._host_io(lib().gpt_set_params, tid, arr)

    def set_grads(self, tid, arr):
        self._host_io(lib().gpt_set_grads, tid, arr)

    def get_momentum(self, tid):
        return self._host_io(lib().gpt_get_momentum, tid)

    def set_momentum(self, tid, arr):
        self._host_io(lib().gpt_set_momentum, tid, arr)

    def set_all_params(self, params):
        for i, w in enumerate(params):
            self.set_params(i, w)

    def argmax(self):
        import torch
        out = torch.empty(self.cfg.batch * self.cfg.seq_len, dtype=torch.int32, device=self.arena.device)
        check(lib().gpt_argmax(self._h, _ptr(out), _stream()), "gpt_argmax")
        return out

    def row_loss(self):
        import torch
        out = torch.empty(self.cfg.batch * self.cfg.seq_len, dtype=torch.float32, device=self.arena.device)
        check(lib().gpt_row_loss(self._h, _ptr(out), _stream()), "gpt_row_loss")
        return out

    # names and element types of gpt_capture's items, in buffer order
    CAPTURE_BLOCK = [("a", "act", "d"), ("qkv", "act", "QD"), ("x", "f32", "d"), ("o", "act", "d"),
                     ("h1", "f32", "d"), ("m", "act", "d"), ("g", "act", "F"), ("h2", "f32", "d"),
                     ("dh", "act", "d"), ("du", "act", "F"), ("dm", "f32", "d"), ("dh1", "act", "d"),
                     ("do", "act", "d"), ("dqkv", "act", "QD"), ("da", "f32", "d")]
    CAPTURE_HEAD = [("r", "act", "d"), ("logits", "f32", "V"), ("dlogits", "act", "V"), ("dr", "f32", "d")]

    def capture_step(self, layer, tokens, targets):
        """Run gpt_step with gpt_capture on `layer` (depth = the LM head) and return
        (loss, {name: float64 numpy array [N][cols]}) of the captured items."""
        import torch
        nbytes = lib().gpt_capture_bytes(ctypes.byref(self.cfg), layer)
        if nbytes == 0:
            raise GptError(f"gpt_capture_bytes: invalid layer {layer}")
        buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.arena.device)
        off = (-buf.data_ptr()) % 256
        check(lib().gpt_capture(self._h, layer, ctypes.c_void_p(buf.data_ptr() + off), nbytes), "gpt_capture")
        try:
            loss = self.step(tokens, targets)
            torch.cuda.synchronize()
        finally:
            check(lib().gpt_capture(self._h, 0, None, 0), "gpt_capture")
        c = self.cfg
        N = c.batch * c.seq_len
        kv = (c.n_kv_head or c.n_head) * c.head_dim
        width = {"d": c.d_model, "F": c.d_ff, "V": c.vocab, "QD": c.d_model + 2 * kv}
        act16 = c.precision != GPT_FP32
        out, pos = {}, off
        for name, kind, w in (self.CAPTURE_HEAD if layer == c.depth else self.CAPTURE_BLOCK):
            n = N * width[w]
            es = 2 if (kind == "act" and act16) else 4
            raw = buf[pos:pos + n * es]
            t = raw.view(torch.bfloat16) if es == 2 else raw.view(torch.float32)
            out[name] = t.float().cpu().numpy().astype(np.float64).reshape(N, width[w])
            pos += (n * es + 255) // 256 * 256
        return loss, out

    def prof_enable(self, name):
        check(lib().gpt_prof_enable(self._h, name.encode() if name else None), "gpt_prof_enable")

    def prof_read(self):
        n, ms, fl = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
        check(lib().gpt_prof_read(self._h, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl)), "gpt_prof_read")
        return n.value, ms.value, fl.value


# ----------------------------------------------------------------------------
# kernel-level calls (device tensors)


def gemm(dtype, a_kmaj, b_kmaj, M, N, K, A, lda, B, ldb, C, ldc, batch=1, sA=0, sB=0, sC=0, tile=0,
         splits=1, ws=None):
    ws_p = _ptr(ws) if ws is not None else ctypes.c_void_p()
    ws_b = ws.numel() * ws.element_size() if ws is not None else 0
    check(lib().gptk_gemm(dtype, int(a_kmaj), int(b_kmaj), M, N, K, batch, _ptr(A), lda, sA, _ptr(B), ldb, sB,
                          _ptr(C), ldc, sC, tile, splits, ws_p, ws_b, _stream()), "gptk_gemm")


def gemm_split(a_kmaj, b_kmaj, M, N, K, Ah, Al, lda, Bh, Bl, ldb, C, ldc, batch=1, sA=0, sB=0, sC=0):
    check(lib().gptk_gemm_split(int(a_kmaj), int(b_kmaj), M, N, K, batch, _ptr(Ah), _ptr(Al), lda, sA, _ptr(Bh),
                                _ptr(Bl), ldb, sB, _ptr(C), ldc, sC, _stream()), "gptk_gemm_split")


def newton_schulz(dtype, G, rows, cols, coeffs, steps, X):
    """gptk_newton_schulz on device tensors G, X (fp32 [rows][cols]); coeffs: (a, b, c) rows."""
    import torch
    nbytes = lib().gptk_ns_ws_bytes(rows, cols)
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=G.device)
    off = (-ws.data_ptr()) % 256
    cf = (ctypes.c_float * 15)(*[float(v) for abc in coeffs for v in abc][:15])
    check(lib().gptk_newton_schulz(dtype, _ptr(G), rows, cols, cf, steps, _ptr(X),
                                   ctypes.c_void_p(ws.data_ptr() + off), nbytes, _stream()), "gptk_newton_schulz")
    torch.cuda.synchronize()  # the workspace is released when this returns


def quant_e4m3(dtype, x, rows, cols, ld, amax_slot, q, qt, inv_scale):
    nul = ctypes.c_void_p()
    check(lib().gptk_quant_e4m3(dtype, _ptr(x), rows, cols, ld, _ptr(amax_slot), _ptr(q) if q is not None else nul,
                                _ptr(qt) if qt is not None else nul, _ptr(inv_scale), _stream()), "gptk_quant_e4m3")


def gemm_fp8(M, N, K, A, lda, B, ldb, dq_a, dq_b, C, ldc, splits=1, ws=None):
    ws_p = _ptr(ws) if ws is not None else ctypes.c_void_p()
    ws_b = ws.numel() * ws.element_size() if ws is not None else 0
    check(lib().gptk_gemm_fp8(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(dq_a), _ptr(dq_b), _ptr(C), ldc, splits, ws_p,
                              ws_b, _stream()), "gptk_gemm_fp8")


def gemm_auto_splits(dtype, M, N, K, batch=1, a_kmaj=1, b_kmaj=1) -> int:
    return lib().gptk_gemm_auto_splits(dtype, int(a_kmaj), int(b_kmaj), M, N, K, batch)


def gemm_kernel_name(dtype, M, N, K, batch=1, a_kmaj=1, b_kmaj=1) -> str:
    return lib().gpt_gemm_kernel_name(dtype, a_kmaj, b_kmaj, M, N, K, batch).decode()


def attn_variant(pass_, variant):
    check(lib().gptk_attn_variant(pass_, variant), "gptk_attn_variant")


def ce_variant(variant):
    check(lib().gptk_ce_variant(variant), "gptk_ce_variant")


def side_stream(on: int = -1) -> int:
    """gptk_side_stream: set (0 never, 1 where it fills idle CUs, 2 always) or query (-1);
    returns the previous setting."""
    return lib().gptk_side_stream(int(on))


def fp8_fused_amax(on: int = -1) -> int:
    """gptk_fp8_fused_amax: set (0/1) or query (-1); returns the previous setting."""
    return lib().gptk_fp8_fused_amax(int(on))


def attn_fwd(dtype, qkv, o, lse, B, T, H, hd, window=0, n_kv=None):
    """n_kv: key/value heads (None: H)."""
    hk = H if n_kv is None else n_kv
    check(lib().gptk_attn_fwd(dtype, _ptr(qkv), _ptr(o), _ptr(lse), B, T, H, hk, hd, window, _stream()),
          "gptk_attn_fwd")


def attn_fwd_qknorm(dtype, qkv, o, lse, B, T, H, hd, window=0, n_kv=None):
    """gptk_attn_fwd_qknorm: q and k rows must be RMS-normalised per head."""
    hk = H if n_kv is None else n_kv
    check(lib().gptk_attn_fwd_qknorm(dtype, _ptr(qkv), _ptr(o), _ptr(lse), B, T, H, hk, hd, window, _stream()),
          "gptk_attn_fwd_qknorm")


def attn_bwd(dtype, qkv, o, dO, lse, D, dqkv, B, T, H, hd, window=0, n_kv=None):
    hk = H if n_kv is None else n_kv
    check(lib().gptk_attn_bwd(dtype, _ptr(qkv), _ptr(o), _ptr(dO), _ptr(lse), _ptr(D), _ptr(dqkv), B, T, H, hk, hd,
                              window, _stream()), "gptk_attn_bwd")


def attn_bwd_noalloc(dtype, qkv, o, dO, lse, dqkv, B, T, H, hd, window=0, n_kv=None):
    """attn_bwd with the library's own device scratch for rowsum(dO*O) (no D argument)."""
    hk = H if n_kv is None else n_kv
    check(lib().gptk_attn_bwd_noalloc(dtype, _ptr(qkv), _ptr(o), _ptr(dO), _ptr(lse), _ptr(dqkv), B, T, H, hk, hd,
                                      window, _stream()), "gptk_attn_bwd_noalloc")


def rmsnorm_fwd(dtype, x, y, rstd, N, d, eps):
    check(lib().gptk_rmsnorm_fwd(dtype, _ptr(x), _ptr(y), _ptr(rstd), N, d, eps, _stream()), "gptk_rmsnorm_fwd")


def rmsnorm_bwd(dtype, dy, x, rstd, dres, dx, dx_act, N, d):
    nul = ctypes.c_void_p()
    check(lib().gptk_rmsnorm_bwd(dtype, _ptr(dy), _ptr(x), _ptr(rstd), _ptr(dres) if dres is not None else nul,
                                 _ptr(dx), _ptr(dx_act) if dx_act is not None else nul, N, d, _stream()),
          "gptk_rmsnorm_bwd")


def rope_qknorm_fwd(dtype, qkv, cs, rq, rk, B, T, H, hd, base, eps, n_kv=None):
    hk = H if n_kv is None else n_kv
    check(lib().gptk_rope_qknorm_fwd(dtype, _ptr(qkv), _ptr(cs), _ptr(rq), _ptr(rk), B, T, H, hk, hd, base, eps,
                                     _stream()), "gptk_rope_qknorm_fwd")


def rope_qknorm_bwd(dtype, dqkv, qkv, cs, rq, rk, B, T, H, hd, base, n_kv=None):
    hk = H if n_kv is None else n_kv
    check(lib().gptk_rope_qknorm_bwd(dtype, _ptr(dqkv), _ptr(qkv), _ptr(cs), _ptr(rq), _ptr(rk), B, T, H, hk, hd,
                                     base, _stream()), "gptk_rope_qknorm_bwd")


def cross_entropy(dtype, logits, targets, dlogits, row_loss, argmax, N, V, inv_n, err):
    check(lib().gptk_cross_entropy(dtype, _ptr(logits), _ptr(targets), _ptr(dlogits), _ptr(row_loss), _ptr(argmax),
                                   N, V, inv_n, _ptr(err), _stream()), "gptk_cross_entropy")


def embed_gather(tokens, E, h, N, d, V, err):
    check(lib().gptk_embed_gather(_ptr(tokens), _ptr(E), _ptr(h), N, d, V, _ptr(err), _stream()),
          "gptk_embed_gather")


def embed_ws_bytes(N, V, d) -> int:
    return lib().gptk_embed_ws_bytes(N, V, d)


def embed_scatter(tokens, dh, dE, N, V, d, ws, sorted_out):
    check(lib().gptk_embed_scatter(_ptr(tokens), _ptr(dh), _ptr(dE), N, V, d, _ptr(ws), _ptr(sorted_out),
                                   _stream()), "gptk_embed_scatter")
