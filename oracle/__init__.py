"""ctypes binding of the plain-C oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  It shares no code with
the GPU library.  Argument marshalling only; every computation is in oracle.c,
except the closed-form measurement-model helpers at the bottom.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Mapping, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SPEC_ORACLE_LIB: another build of the same source (the sanitizer build)
_LIBPATH = os.environ.get("SPEC_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

OK, EARG, EBADPROB, ENOMEM, ECAPACITY = 0, -1, -2, -3, -4

_u64 = C.c_uint64
_i32 = C.c_int32
_p = C.c_void_p


class _Model(C.Structure):
    _fields_ = [
        ("n_layers", _i32), ("d_model", _i32), ("n_heads", _i32), ("n_kv_heads", _i32),
        ("head_dim", _i32), ("d_ffn", _i32), ("vocab", _i32),
        ("rope_theta", C.c_double), ("rms_eps", C.c_double),
        ("embed", _p), ("attn_norm", _p), ("wq", _p), ("wk", _p), ("wv", _p), ("wo", _p),
        ("ffn_norm", _p), ("wg", _p), ("wu", _p), ("wd", _p), ("final_norm", _p), ("lm_head", _p),
    ]


class _Stats(C.Structure):
    _fields_ = [("rounds", _i32), ("target_passes", _i32), ("draft_passes", _i32),
                ("accepted", C.c_int64), ("emitted", C.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIBPATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIBPATH)
        L.orc_philox4x64_10.argtypes = [_p, _p, _p]
        L.orc_uniform_words.argtypes = [_u64, _u64, _u64, _u64, _p]
        L.orc_u24.argtypes = [_u64]
        L.orc_u24.restype = C.c_uint32
        L.orc_fix.argtypes = [C.c_float, _p]
        L.orc_sample_icdf.argtypes = [_p, _i32, C.c_uint32]
        L.orc_sample_icdf.restype = _i32
        L.orc_argmax_low.argtypes = [_p, _i32]
        L.orc_argmax_low.restype = _i32
        L.orc_accept.argtypes = [C.c_float, C.c_float, C.c_float]
        L.orc_verify_sample.argtypes = [_p, _p, _p, _i32, _i32, _u64, _u64, _u64, _u64, _p, _p]
        L.orc_verify_sample_u.argtypes = [_p, _p, _p, _i32, _i32, _p, C.c_uint32, _p, _p]
        L.orc_verify_greedy.argtypes = [_p, _p, _i32, _i32, _p, _p]
        L.orc_accept_reject_batch.argtypes = [_p, _p, _p, _i32, _i32, _i32, _u64, _p, _u64, _i32,
                                              _p, _p]
        L.orc_draft_sample.argtypes = [_p, _i32, _u64, _u64, _u64, _u64, _i32]
        L.orc_draft_sample.restype = _i32
        L.orc_icdf_histogram.argtypes = [_p, _i32, _p]
        L.orc_accept_count.argtypes = [C.c_float, C.c_float]
        L.orc_accept_count.restype = _u64
        L.orc_kv_new.argtypes = [_p, _i32]
        L.orc_kv_new.restype = _p
        L.orc_kv_free.argtypes = [_p]
        L.orc_forward.argtypes = [_p, _p, _p, _i32, _i32, _p]
        L.orc_forward_hidden.argtypes = [_p, _p, _p, _i32, _i32, _p, _p]
        L.orc_softmax_f32.argtypes = [_p, _i32, _p]
        L.orc_heads_draft.argtypes = [_p, _p, _i32, _p, _i32, _i32, _u64, _u64, _u64, _p, _p]
        L.orc_spec_generate_heads.argtypes = [_p, _p, _i32, _p, _i32, _i32, _i32, _i32, _u64,
                                              _u64, _p, _p, _p, _p]
        L.orc_generate.argtypes = [_p, _p, _i32, _i32, _i32, _u64, _u64, _p]
        L.orc_spec_generate.argtypes = [_p, _p, _p, _i32, _i32, _i32, _i32, _u64, _u64, _p, _p, _p]
        L.orc_num_threads.restype = _i32
        L.orc_rope.argtypes = [_p, _i32, _i32, C.c_double]
        L.orc_rmsnorm.argtypes = [_p, _i32, _p, C.c_double, _p]
        L.orc_attend.argtypes = [_p, _p, _p, _i32, _i32, _p]
        L.orc_draft_sample_batch.argtypes = [_p, _i32, _i32, _u64, _p, _u64, _i32, _p]
        L.orc_ngram_draft.argtypes = [_p, _i32, _i32, _i32, _p]
        L.orc_ngram_draft.restype = _i32
        L.orc_expected_tokens.argtypes = [C.c_double, _i32]
        L.orc_expected_tokens.restype = C.c_double
        L.orc_choose_k.argtypes = [C.c_double, C.c_double, C.c_double, _i32]
        L.orc_choose_k.restype = _i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- uniforms --
def philox4x64_10(ctr: Sequence[int], key: Sequence[int]) -> list[int]:
    c = _c(ctr, np.uint64)
    k = _c(key, np.uint64)
    o = np.zeros(4, np.uint64)
    lib().orc_philox4x64_10(_ptr(c), _ptr(k), _ptr(o))
    return [int(x) for x in o]


def uniform_words(seed: int, p: int, s: int = 0, c: int = 0) -> list[int]:
    o = np.zeros(4, np.uint64)
    lib().orc_uniform_words(seed, p, s, c, _ptr(o))
    return [int(x) for x in o]


def u24(w: int) -> int:
    return int(lib().orc_u24(w))


# ---------------------------------------------------------------- sampler --
def fix(x: float) -> int:
    o = np.zeros(1, np.uint64)
    rc = lib().orc_fix(float(np.float32(x)), _ptr(o))
    if rc != OK:
        raise ValueError(f"invalid probability {x!r}")
    return int(o[0])


def sample_icdf(q, u: int) -> int:
    qa = _c(q, np.uint64)
    return int(lib().orc_sample_icdf(_ptr(qa), len(qa), u))


def argmax_low(x) -> int:
    xa = _c(x, np.float32)
    return int(lib().orc_argmax_low(_ptr(xa), len(xa)))


def accept(r: float, T: float, D: float) -> bool:
    return bool(lib().orc_accept(float(np.float32(r)), float(np.float32(T)), float(np.float32(D))))


def verify_sample(T, D, d, seed: int, s: int, c: int, P: int):
    T = _c(T, np.float32); D = _c(D, np.float32); d = _c(d, np.int32)
    K = len(d); V = T.shape[-1]
    assert T.shape == (K + 1, V) and D.shape == (K, V)
    out = np.full(K + 1, -1, np.int32); n = np.zeros(1, np.int32)
    rc = lib().orc_verify_sample(_ptr(T), _ptr(D), _ptr(d), K, V, seed, s, c, P, _ptr(out), _ptr(n))
    return rc, int(n[0]), out


def verify_sample_u(T, D, d, u_acc, u_smp: int):
    T = _c(T, np.float32); D = _c(D, np.float32); d = _c(d, np.int32)
    ua = _c(u_acc, np.uint32)
    K = len(d); V = T.shape[-1]
    out = np.full(K + 1, -1, np.int32); n = np.zeros(1, np.int32)
    rc = lib().orc_verify_sample_u(_ptr(T), _ptr(D), _ptr(d), K, V, _ptr(ua), u_smp, _ptr(out), _ptr(n))
    return rc, int(n[0]), out


def verify_greedy(T, d):
    T = _c(T, np.float32); d = _c(d, np.int32)
    K = len(d); V = T.shape[-1]
    out = np.full(K + 1, -1, np.int32); n = np.zeros(1, np.int32)
    rc = lib().orc_verify_greedy(_ptr(T), _ptr(d), K, V, _ptr(out), _ptr(n))
    return rc, int(n[0]), out


def accept_reject_batch(T, D, d, seed: int, pos, stream_id: int, greedy: bool):
    """T [B][K+1][V], D [B][K][V], d [B][K], pos [B] -> (out [B][K+1], n_acc [B])."""
    T = _c(T, np.float32); D = _c(D, np.float32); d = _c(d, np.int32)
    pos = _c(pos, np.uint64)
    B, K1, V = T.shape
    K = K1 - 1
    out = np.full((B, K + 1), -1, np.int32); n = np.zeros(B, np.int32)
    rc = lib().orc_accept_reject_batch(_ptr(T), _ptr(D), _ptr(d), B, K, V, seed, _ptr(pos),
                                       stream_id, int(bool(greedy)), _ptr(out), _ptr(n))
    if rc != OK:
        raise ValueError(f"orc_accept_reject_batch rc={rc}")
    return out, n


def draft_sample(Drow, seed: int, p: int, s: int = 0, c: int = 0, greedy: bool = False) -> int:
    Da = _c(Drow, np.float32)
    return int(lib().orc_draft_sample(_ptr(Da), len(Da), seed, p, s, c, int(bool(greedy))))


def draft_sample_batch(D, seed: int, pos, c: int = 0, greedy: bool = False) -> np.ndarray:
    """D [B][V] -> tokens [B]; row b uses s = b and position pos[b]."""
    Da = _c(D, np.float32)
    B, V = Da.shape
    pa = _c(np.broadcast_to(np.asarray(pos, np.uint64), (B,)), np.uint64)
    out = np.zeros(B, np.int32)
    lib().orc_draft_sample_batch(_ptr(Da), B, V, seed, _ptr(pa), c, int(bool(greedy)), _ptr(out))
    return out


def ngram_draft(hist, L: int, K: int, n_max: int):
    """(draft tokens [K], match length) from orc_ngram_draft on hist[0..L]."""
    h = _c(hist, np.int32)
    if not 0 <= L < len(h):
        raise ValueError("L outside the history")
    d = np.zeros(K, np.int32)
    n = lib().orc_ngram_draft(_ptr(h), L, K, n_max, _ptr(d))
    if n < 0:
        raise ValueError(f"orc_ngram_draft error {n}")
    return d, int(n)


def expected_tokens(alpha: float, K: int) -> float:
    """orc_expected_tokens: 1 + a + ... + a^K ([en] Floor 6)."""
    return float(lib().orc_expected_tokens(alpha, K))


def choose_k(alpha: float, t_draft: float, t_verify: float, k_max: int) -> int:
    """orc_choose_k: the K in 1..k_max with the most tokens per unit time."""
    k = lib().orc_choose_k(alpha, t_draft, t_verify, k_max)
    if k < 0:
        raise ValueError(f"orc_choose_k error {k}")
    return int(k)


def icdf_histogram(q) -> np.ndarray:
    qa = _c(q, np.uint64)
    counts = np.zeros(len(qa), np.uint64)
    lib().orc_icdf_histogram(_ptr(qa), len(qa), _ptr(counts))
    return counts


def accept_count(T: float, D: float) -> int:
    return int(lib().orc_accept_count(float(np.float32(T)), float(np.float32(D))))


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ------------------------------------------------------------- primitives --
def rope(v, pos: int, theta: float) -> np.ndarray:
    a = np.array(v, dtype=np.float64)
    lib().orc_rope(_ptr(a), len(a), pos, float(theta))
    return a


def rmsnorm(x, g_bits, eps: float) -> np.ndarray:
    xa = _c(x, np.float64)
    ga = _c(g_bits, np.uint16)
    h = np.zeros(len(xa), np.float64)
    lib().orc_rmsnorm(_ptr(xa), len(xa), _ptr(ga), float(eps), _ptr(h))
    return h


def attend(q, k, v) -> np.ndarray:
    """One query head over keys k [n][hd] and values v [n][hd]."""
    qa = _c(q, np.float64); ka = _c(k, np.float64); va = _c(v, np.float64)
    n, hd = ka.shape
    o = np.zeros(hd, np.float64)
    lib().orc_attend(_ptr(qa), _ptr(ka), _ptr(va), n, hd, _ptr(o))
    return o


# ------------------------------------------------------------------ model --
WEIGHT_NAMES = ("embed", "attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd",
                "final_norm", "lm_head")


class Model:
    """Wraps a dict of bf16 weight arrays (uint16 bit patterns, stacked over
    layers) and the model dimensions; keeps the arrays alive for the C side."""

    def __init__(self, cfg, weights: Mapping[str, np.ndarray]):
        self.cfg = cfg
        self._w = {k: np.ascontiguousarray(weights[k], dtype=np.uint16) for k in WEIGHT_NAMES}
        m = _Model()
        m.n_layers = cfg.n_layers; m.d_model = cfg.d_model; m.n_heads = cfg.n_heads
        m.n_kv_heads = cfg.n_kv_heads; m.head_dim = cfg.head_dim; m.d_ffn = cfg.d_ffn
        m.vocab = cfg.vocab; m.rope_theta = float(cfg.rope_theta); m.rms_eps = float(cfg.rms_eps)
        for k in WEIGHT_NAMES:
            setattr(m, k, self._w[k].ctypes.data)
        self._m = m

    @property
    def vocab(self) -> int:
        return self.cfg.vocab

    def ref(self):
        return C.byref(self._m)


class KV:
    def __init__(self, model: Model, max_seq: int):
        self._h = lib().orc_kv_new(model.ref(), max_seq)
        if not self._h:
            raise MemoryError("orc_kv_new")
        self.model = model

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _lib is not None:
            try:
                _lib.orc_kv_free(h)
            except Exception:  # interpreter shutdown
                pass


def forward(model: Model, kv: KV, tokens, pos0: int, want_logits: bool = True):
    t = _c(tokens, np.int32)
    n = len(t)
    lg = np.zeros((n, model.vocab), np.float64) if want_logits else None
    rc = lib().orc_forward(model.ref(), kv._h, _ptr(t), n, pos0, _ptr(lg) if want_logits else None)
    if rc != OK:
        raise ValueError(f"orc_forward rc={rc}")
    return lg


def forward_hidden(model: Model, kv: KV, tokens, pos0: int, want_logits: bool = True):
    """(logits [n][V] or None, final normed states [n][d]) of orc_forward_hidden."""
    t = _c(tokens, np.int32)
    n = len(t)
    lg = np.zeros((n, model.vocab), np.float64) if want_logits else None
    hid = np.zeros((n, model.cfg.d_model), np.float64)
    rc = lib().orc_forward_hidden(model.ref(), kv._h, _ptr(t), n, pos0,
                                  _ptr(lg) if want_logits else None, _ptr(hid))
    if rc != OK:
        raise ValueError(f"orc_forward_hidden rc={rc}")
    return lg, hid


def heads_draft(model: Model, W_heads, h, K: int, greedy: bool, seed: int, P: int, c: int = 0):
    """orc_heads_draft: (D [K][V] fp32, drafts [K]) from the final normed
    state h [d] and head matrices W_heads [n_heads][d][d] (bf16 bits)."""
    W = _c(W_heads, np.uint16)
    ha = _c(h, np.float64)
    n_heads = W.shape[0]
    D = np.zeros((K, model.vocab), np.float32)
    d = np.zeros(K, np.int32)
    rc = lib().orc_heads_draft(model.ref(), _ptr(W), n_heads, _ptr(ha), K, int(bool(greedy)),
                               seed, P, c, _ptr(D), _ptr(d))
    if rc != OK:
        raise ValueError(f"orc_heads_draft rc={rc}")
    return D, d


def spec_generate_heads(target: Model, W_heads, prompt, n_new: int, K: int, greedy: bool,
                        seed: int = 0, c: int = 0):
    """(tokens [n_new], n_acc per round, drafts per round [rounds][K], stats)."""
    W = _c(W_heads, np.uint16)
    pr = _c(prompt, np.int32)
    out = np.zeros(n_new, np.int32)
    nacc = np.full(max(n_new, 1), -1, np.int32)
    drafts = np.full((max(n_new, 1), K), -1, np.int32)
    st = _Stats()
    rc = lib().orc_spec_generate_heads(target.ref(), _ptr(W), W.shape[0], _ptr(pr), len(pr), n_new,
                                       K, int(bool(greedy)), seed, c, _ptr(out), _ptr(nacc),
                                       _ptr(drafts), C.byref(st))
    if rc != OK:
        raise ValueError(f"orc_spec_generate_heads rc={rc}")
    stats = {"rounds": st.rounds, "target_passes": st.target_passes,
             "draft_passes": st.draft_passes, "accepted": st.accepted, "emitted": st.emitted}
    return out, nacc[: st.rounds], drafts[: st.rounds], stats


def softmax_f32(logits) -> np.ndarray:
    la = _c(logits, np.float64)
    p = np.zeros(len(la), np.float32)
    lib().orc_softmax_f32(_ptr(la), len(la), _ptr(p))
    return p


def generate(model: Model, prompt, n_new: int, greedy: bool, seed: int = 0, c: int = 0):
    pr = _c(prompt, np.int32)
    out = np.zeros(n_new, np.int32)
    rc = lib().orc_generate(model.ref(), _ptr(pr), len(pr), n_new, int(bool(greedy)), seed, c, _ptr(out))
    if rc != OK:
        raise ValueError(f"orc_generate rc={rc}")
    return out


def spec_generate(target: Model, draft: Model, prompt, n_new: int, K: int, greedy: bool,
                  seed: int = 0, c: int = 0):
    pr = _c(prompt, np.int32)
    out = np.zeros(n_new, np.int32)
    nacc = np.full(max(n_new, 1), -1, np.int32)
    st = _Stats()
    rc = lib().orc_spec_generate(target.ref(), draft.ref(), _ptr(pr), len(pr), n_new, K,
                                 int(bool(greedy)), seed, c, _ptr(out), _ptr(nacc), C.byref(st))
    if rc != OK:
        raise ValueError(f"orc_spec_generate rc={rc}")
    stats = {"rounds": st.rounds, "target_passes": st.target_passes,
             "draft_passes": st.draft_passes, "accepted": st.accepted, "emitted": st.emitted}
    return out, nacc[: st.rounds], stats


# -------------------------------------------- measurement-model helpers ----
def expected_tokens_per_round(alpha: float, k: int) -> float:
    """Mean tokens per round when every draft passes independently with
    probability alpha: (1 - alpha^(k+1)) / (1 - alpha) ([en] Floor 6)."""
    if alpha == 1.0:
        return float(k + 1)
    return (1.0 - alpha ** (k + 1)) / (1.0 - alpha)


def expected_accepted(betas: Sequence[float]) -> float:
    """E[n_acc] = sum_j prod_{i<=j} beta_i for per-position acceptance
    probabilities beta_i = sum_v min(T_i(v), D_i(v)) (each draft is reached
    only if all earlier ones passed)."""
    tot, run = 0.0, 1.0
    for b in betas:
        run *= b
        tot += run
    return tot
