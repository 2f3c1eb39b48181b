"""ctypes binding of libspec (include/spec.h): argument marshalling only.

Every computation runs in the HIP kernels of libspec.so; torch is used only
to own device memory (tensor.data_ptr()) and streams.  If the library is not
built, importing the functions raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Mapping, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SPEC_LIBSPEC: another build of the same sources (the host-sanitizer build)
LIBPATH = os.environ.get("SPEC_LIBSPEC") or os.path.join(_HERE, "libspec.so")

SPEC_OK = 0
SPEC_ERR_ARG = -1
SPEC_ERR_CAPACITY = -2
SPEC_ERR_STATE = -3
SPEC_ERR_OOM = -4
SPEC_ERR_HIP = -5
SPEC_K_MAX = 7
SPEC_AR_K_MAX = 63

_p = C.c_void_p
_i32 = C.c_int32
_u64 = C.c_uint64


class SpecError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libspec error {code}: {msg}")
        self.code = code


class SpecModelDesc(C.Structure):
    _fields_ = [
        ("n_layers", _i32), ("d_model", _i32), ("n_heads", _i32), ("n_kv_heads", _i32),
        ("head_dim", _i32), ("d_ffn", _i32), ("vocab", _i32),
        ("rope_theta", C.c_float), ("rms_eps", C.c_float),
        ("embed", _p), ("attn_norm", _p), ("wq", _p), ("wk", _p), ("wv", _p), ("wo", _p),
        ("ffn_norm", _p), ("wg", _p), ("wu", _p), ("wd", _p), ("final_norm", _p), ("lm_head", _p),
    ]


class SpecInitParams(C.Structure):
    _fields_ = [
        ("target", SpecModelDesc), ("draft", SpecModelDesc),
        ("k_max", _i32), ("max_seq", _i32), ("greedy", _i32), ("use_graphs", _i32),
        ("profile_kernels", _i32), ("stream_id", _u64), ("hip_stream", _p),
    ]


class SpecBatchParams(C.Structure):
    _fields_ = [
        ("target", SpecModelDesc), ("n_seq", _i32), ("k_max", _i32), ("max_seq", _i32),
        ("greedy", _i32), ("use_graphs", _i32), ("stream_id", _u64), ("hip_stream", _p),
    ]


SPEC_BATCH_MAX_SEQ = 32

K_BINS = 8  # SPEC_K_MAX + 1


class SpecState(C.Structure):
    _fields_ = [("target_len", _i32), ("draft_len", _i32), ("pending", _i32),
                ("device_error", _i32), ("accept_counts", (_i32 * K_BINS) * K_BINS)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBPATH):
            raise ImportError(f"{LIBPATH} is not built; run __graft_entry__.build() first")
        L = C.CDLL(LIBPATH)
        L.spec_init.argtypes = [C.POINTER(SpecInitParams), _p, _i32, C.POINTER(_p)]
        L.spec_draft.argtypes = [_p, _i32, _u64, _p, _p]
        L.spec_verify.argtypes = [_p, _i32, _u64, _p, _p, _p, _p, _p, _p]
        L.spec_draft_ngram.argtypes = [_p, _i32, _i32, _p, _p]
        L.spec_heads_init.argtypes = [_p, _p, _i32]
        L.spec_draft_heads.argtypes = [_p, _i32, _u64, _p, _p]
        L.spec_mat_create.argtypes = [_p, _i32, _i32, C.POINTER(_p)]
        L.spec_mat_mul.argtypes = [_p, _p, _i32, _p, _p]
        L.spec_mat_destroy.argtypes = [_p]
        L.spec_expected_tokens.argtypes = [C.c_double, _i32]
        L.spec_expected_tokens.restype = C.c_double
        L.spec_alpha_from_tokens.argtypes = [C.c_double, _i32]
        L.spec_alpha_from_tokens.restype = C.c_double
        L.spec_choose_k.argtypes = [C.c_double, C.c_double, C.c_double, _i32]
        L.spec_choose_k.restype = _i32
        L.spec_commit.argtypes = [_p, _p, _p]
        L.spec_destroy.argtypes = [_p]
        L.spec_last_error.argtypes = [_p]
        L.spec_last_error.restype = C.c_char_p
        L.spec_sync.argtypes = [_p]
        L.spec_stream.argtypes = [_p]
        L.spec_stream.restype = _p
        L.spec_get_state.argtypes = [_p, C.POINTER(SpecState)]
        L.spec_get_history.argtypes = [_p, _p, _i32]
        L.spec_kernel_times.argtypes = [_p, _p, _i32, C.POINTER(_i32)]
        L.spec_set_profiling.argtypes = [_p, _i32]
        L.spec_head_time.argtypes = [_p, C.POINTER(C.c_float)]
        L.spec_accept_reject.argtypes = [_p, _p, _p, _i32, _i32, _i32, _u64, _p, _u64, _i32, _p,
                                         _p, _p]
        L.spec_accept_reject_noalloc.argtypes = [_p, _p, _p, _i32, _i32, _i32, _u64, _p, _u64, _i32,
                                                 _p, _p, _p]
        L.spec_read_ceiling.argtypes = [_p, _u64, _i32, _p, C.POINTER(C.c_double)]
        L.spec_batch_init.argtypes = [C.POINTER(SpecBatchParams), _p, _i32, C.POINTER(_p)]
        L.spec_batch_draft_ngram.argtypes = [_p, _i32, _i32, _p, _p]
        L.spec_batch_verify.argtypes = [_p, _i32, _u64, _p, _p, _p, _p, _p, _p]
        L.spec_batch_commit.argtypes = [_p, _p, _p]
        L.spec_batch_sync.argtypes = [_p]
        L.spec_batch_get_state.argtypes = [_p, _p, _p]
        L.spec_batch_get_history.argtypes = [_p, _i32, _p, _i32]
        L.spec_batch_last_error.argtypes = [_p]
        L.spec_batch_last_error.restype = C.c_char_p
        L.spec_batch_destroy.argtypes = [_p]
        _lib = L
    return _lib


EXPORTED = ("spec_init", "spec_draft", "spec_draft_ngram", "spec_heads_init", "spec_draft_heads",
            "spec_verify", "spec_commit", "spec_destroy",
            "spec_last_error", "spec_sync", "spec_stream", "spec_get_state", "spec_get_history",
            "spec_kernel_times", "spec_set_profiling", "spec_head_time", "spec_accept_reject",
            "spec_accept_reject_noalloc", "spec_expected_tokens",
            "spec_alpha_from_tokens", "spec_choose_k", "spec_mat_create", "spec_mat_mul",
            "spec_mat_destroy", "spec_read_ceiling", "spec_batch_init", "spec_batch_draft_ngram",
            "spec_batch_verify", "spec_batch_commit", "spec_batch_sync", "spec_batch_get_state",
            "spec_batch_get_history", "spec_batch_last_error", "spec_batch_destroy")


def _check(rc: int, ctx=None):
    if rc != SPEC_OK:
        raise SpecError(rc, spec_last_error(ctx))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


WEIGHT_NAMES = ("embed", "attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd",
                "final_norm", "lm_head")


def model_desc(cfg, weights: Mapping[str, "object"]) -> SpecModelDesc:
    """cfg: any object with n_layers, d_model, n_heads, n_kv_heads, head_dim,
    d_ffn, vocab, rope_theta, rms_eps; weights: contiguous bf16 device tensors."""
    import torch
    m = SpecModelDesc()
    m.n_layers = cfg.n_layers; m.d_model = cfg.d_model; m.n_heads = cfg.n_heads
    m.n_kv_heads = cfg.n_kv_heads; m.head_dim = cfg.head_dim; m.d_ffn = cfg.d_ffn
    m.vocab = cfg.vocab; m.rope_theta = float(cfg.rope_theta); m.rms_eps = float(cfg.rms_eps)
    for k in WEIGHT_NAMES:
        t = weights[k]
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"weight {k} must be a contiguous bf16 device tensor")
        setattr(m, k, t.data_ptr())
    return m


class Ctx:
    """Owns a spec_ctx* handle."""

    def __init__(self, handle: int):
        self.handle = handle

    def __del__(self):
        if getattr(self, "handle", None):
            lib().spec_destroy(self.handle)
            self.handle = None


def spec_init(target_cfg, target_w, draft_cfg, draft_w, prompt, *, k_max: int, max_seq: int,
              greedy: bool, use_graphs: bool = True, profile_kernels: bool = False,
              stream_id: int = 0, stream: int = 0) -> Ctx:
    p = SpecInitParams()
    p.target = model_desc(target_cfg, target_w)
    p.draft = model_desc(draft_cfg, draft_w)
    p.k_max = k_max; p.max_seq = max_seq; p.greedy = int(bool(greedy))
    p.use_graphs = int(bool(use_graphs)); p.profile_kernels = int(bool(profile_kernels))
    p.stream_id = stream_id; p.hip_stream = stream or None
    pr = np.ascontiguousarray(prompt, dtype=np.int32)
    h = _p()
    rc = lib().spec_init(C.byref(p), pr.ctypes.data, len(pr), C.byref(h))
    _check(rc)
    return Ctx(h.value)


def spec_draft(ctx: Ctx, K: int, seed: int, d, D) -> None:
    _check(lib().spec_draft(ctx.handle, K, seed, _ptr(d), _ptr(D)), ctx)


def spec_draft_ngram(ctx: Ctx, K: int, n_max: int, d, D=None) -> None:
    _check(lib().spec_draft_ngram(ctx.handle, K, n_max, _ptr(d), _ptr(D)), ctx)


def spec_heads_init(ctx: Ctx, W, n_heads: int) -> None:
    """W: bf16 device tensor [n_heads][d_model][d_model] of the target's width."""
    _check(lib().spec_heads_init(ctx.handle, _ptr(W), n_heads), ctx)


def spec_draft_heads(ctx: Ctx, K: int, seed: int, d, D) -> None:
    _check(lib().spec_draft_heads(ctx.handle, K, seed, _ptr(d), _ptr(D)), ctx)


def spec_mat_create(W) -> int:
    """Packs a contiguous 2-D bf16 device tensor W [N][K]; returns the handle."""
    import torch
    if W.dtype != torch.bfloat16 or not W.is_cuda or not W.is_contiguous() or W.dim() != 2:
        raise ValueError("W must be a contiguous 2-D bf16 device tensor")
    h = _p()
    _check(lib().spec_mat_create(W.data_ptr(), W.shape[0], W.shape[1], C.byref(h)))
    return h.value


def spec_mat_mul(handle: int, X, Y, stream: int = 0) -> None:
    _check(lib().spec_mat_mul(handle, _ptr(X), X.shape[0], _ptr(Y), stream))


def spec_mat_destroy(handle: int) -> None:
    _check(lib().spec_mat_destroy(handle))


class Mat:
    """A packed weight matrix (spec_mat) for batched-row products."""

    def __init__(self, W):
        self.handle = spec_mat_create(W)
        self.N, self.K = W.shape

    def mul(self, X, Y, stream: int = 0) -> None:
        spec_mat_mul(self.handle, X, Y, stream)

    def __del__(self):
        if getattr(self, "handle", None):
            spec_mat_destroy(self.handle)
            self.handle = None


def spec_expected_tokens(alpha: float, K: int) -> float:
    return float(lib().spec_expected_tokens(alpha, K))


def spec_alpha_from_tokens(tokens_per_round: float, K: int) -> float:
    return float(lib().spec_alpha_from_tokens(tokens_per_round, K))


def spec_choose_k(alpha: float, t_draft_step: float, t_verify: float, k_max: int) -> int:
    k = lib().spec_choose_k(alpha, t_draft_step, t_verify, k_max)
    _check(0 if k > 0 else k)
    return int(k)


def spec_verify(ctx: Ctx, K: int, seed: int, d, D, out, n_acc, T=None, logits=None) -> None:
    _check(lib().spec_verify(ctx.handle, K, seed, _ptr(d), _ptr(D), _ptr(out), _ptr(n_acc),
                             _ptr(T), _ptr(logits)), ctx)


def spec_commit(ctx: Ctx, out, n_acc) -> None:
    _check(lib().spec_commit(ctx.handle, _ptr(out), _ptr(n_acc)), ctx)


def spec_destroy(ctx: Ctx) -> None:
    if ctx.handle:
        lib().spec_destroy(ctx.handle)
        ctx.handle = None


def spec_last_error(ctx: Optional[Ctx] = None) -> str:
    h = ctx.handle if isinstance(ctx, Ctx) else None
    return lib().spec_last_error(h).decode(errors="replace")


def spec_sync(ctx: Ctx) -> None:
    _check(lib().spec_sync(ctx.handle), ctx)


def spec_stream(ctx: Ctx) -> int:
    return int(lib().spec_stream(ctx.handle) or 0)


def spec_get_state(ctx: Ctx) -> dict:
    s = SpecState()
    _check(lib().spec_get_state(ctx.handle, C.byref(s)), ctx)
    counts = np.array([[s.accept_counts[k][n] for n in range(K_BINS)] for k in range(K_BINS)],
                      np.int64)
    return {"target_len": s.target_len, "draft_len": s.draft_len, "pending": s.pending,
            "device_error": s.device_error, "accept_counts": counts}


def spec_get_history(ctx: Ctx, n: int) -> np.ndarray:
    out = np.zeros(n, np.int32)
    _check(lib().spec_get_history(ctx.handle, out.ctypes.data, n), ctx)
    return out


def spec_kernel_times(ctx: Ctx, cap: int = 4096) -> np.ndarray:
    buf = np.zeros(cap, np.float32)
    n = _i32()
    _check(lib().spec_kernel_times(ctx.handle, buf.ctypes.data, cap, C.byref(n)), ctx)
    return buf[: n.value].copy()


def spec_head_time(ctx: Ctx) -> float:
    """LM-head duration (ms) of the last profiled spec_verify, or -1."""
    ms = C.c_float(-1.0)
    _check(lib().spec_head_time(ctx.handle, C.byref(ms)), ctx)
    return float(ms.value)


def spec_set_profiling(ctx: Ctx, enable: bool) -> None:
    _check(lib().spec_set_profiling(ctx.handle, int(bool(enable))), ctx)


def spec_read_ceiling(buf, reps: int = 3, stream: int = 0) -> float:
    """Streaming-read rate (GB/s) over the device tensor buf (measurement
    helper: the HBM ceiling the verify pass is set against)."""
    gbs = C.c_double(0.0)
    _check(lib().spec_read_ceiling(_ptr(buf), buf.numel() * buf.element_size(), reps,
                                   stream or None, C.byref(gbs)))
    return gbs.value


def spec_accept_reject(T, D, d, seed: int, pos, stream_id: int, greedy: bool, out, n_acc,
                       stream: int = 0) -> None:
    """T [B][K+1][V] f32, D [B][K][V] f32, d [B][K] i32, pos [B] i64 (read as
    uint64), out [B][K+1] i32, n_acc [B] i32: all device tensors."""
    B, K1, V = T.shape
    _check(lib().spec_accept_reject(_ptr(T), _ptr(D), _ptr(d), B, K1 - 1, V, seed, _ptr(pos),
                                    stream_id, int(bool(greedy)), _ptr(out), _ptr(n_acc),
                                    stream or None))



def spec_accept_reject_noalloc(T, D, d, seed: int, pos, stream_id: int, greedy: bool, out, n_acc,
                               stream: int = 0) -> None:
    """spec_accept_reject with the library's fixed scratch array instead of an
    allocated workspace (same arguments and results)."""
    B, K1, V = T.shape
    _check(lib().spec_accept_reject_noalloc(_ptr(T), _ptr(D), _ptr(d), B, K1 - 1, V, seed,
                                            _ptr(pos), stream_id, int(bool(greedy)), _ptr(out),
                                            _ptr(n_acc), stream or None))

# ------------------------------------------------------- batched verify --
class Batch:
    """Owns a spec_batch* handle (B sequences verified together)."""

    def __init__(self, handle: int, n_seq: int):
        self.handle = handle
        self.n_seq = n_seq

    def __del__(self):
        if getattr(self, "handle", None):
            lib().spec_batch_destroy(self.handle)
            self.handle = None


def _bcheck(rc: int, bc: Optional[Batch] = None):
    if rc != SPEC_OK:
        h = bc.handle if isinstance(bc, Batch) else None
        raise SpecError(rc, lib().spec_batch_last_error(h).decode(errors="replace"))


def spec_batch_init(target_cfg, target_w, prompts, *, k_max: int, max_seq: int, greedy: bool,
                    use_graphs: bool = True, stream_id: int = 0, stream: int = 0) -> Batch:
    """prompts: int [n_seq][n_prompt] (one row per sequence)."""
    pr = np.ascontiguousarray(prompts, dtype=np.int32)
    if pr.ndim != 2:
        raise ValueError("prompts must be [n_seq][n_prompt]")
    p = SpecBatchParams()
    p.target = model_desc(target_cfg, target_w)
    p.n_seq = pr.shape[0]; p.k_max = k_max; p.max_seq = max_seq; p.greedy = int(bool(greedy))
    p.use_graphs = int(bool(use_graphs)); p.stream_id = stream_id; p.hip_stream = stream or None
    h = _p()
    _bcheck(lib().spec_batch_init(C.byref(p), pr.ctypes.data, pr.shape[1], C.byref(h)))
    return Batch(h.value, pr.shape[0])


def spec_batch_draft_ngram(bc: Batch, K: int, n_max: int, d, D=None) -> None:
    _bcheck(lib().spec_batch_draft_ngram(bc.handle, K, n_max, _ptr(d), _ptr(D)), bc)


def spec_batch_verify(bc: Batch, K: int, seed: int, d, D, out, n_acc, T=None, logits=None) -> None:
    _bcheck(lib().spec_batch_verify(bc.handle, K, seed, _ptr(d), _ptr(D), _ptr(out), _ptr(n_acc),
                                    _ptr(T), _ptr(logits)), bc)


def spec_batch_commit(bc: Batch, out, n_acc) -> None:
    _bcheck(lib().spec_batch_commit(bc.handle, _ptr(out), _ptr(n_acc)), bc)


def spec_batch_sync(bc: Batch) -> None:
    _bcheck(lib().spec_batch_sync(bc.handle), bc)


def spec_batch_get_state(bc: Batch) -> dict:
    ln = np.zeros(bc.n_seq, np.int32)
    err = np.zeros(bc.n_seq, np.int32)
    _bcheck(lib().spec_batch_get_state(bc.handle, ln.ctypes.data, err.ctypes.data), bc)
    return {"len": ln, "device_error": err}


def spec_batch_get_history(bc: Batch, b: int, n: int) -> np.ndarray:
    out = np.zeros(n, np.int32)
    _bcheck(lib().spec_batch_get_history(bc.handle, b, out.ctypes.data, n), bc)
    return out


def spec_batch_last_error(bc: Optional[Batch] = None) -> str:
    h = bc.handle if isinstance(bc, Batch) else None
    return lib().spec_batch_last_error(h).decode(errors="replace")


def spec_batch_destroy(bc: Batch) -> None:
    if bc.handle:
        lib().spec_batch_destroy(bc.handle)
        bc.handle = None
