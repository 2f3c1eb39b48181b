"""Seeded synthetic inputs shared by the tests, bench.py, the oracle side and
the GPU side.

This module holds none of the speculative-decoding arithmetic: it only draws
random numbers (model weights, prompts, logit rows) and rounds them to the
storage types.  Model shapes are the random-init Llama-style pairs the
workloads describe; weights are N(0, 0.02) rounded to bf16 once, norm gains
are 1, every tensor has its own seed derived from (seed, tensor name).
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, Optional, Tuple

import numpy as np

SEED_WEIGHTS = 1001
SEED_PROMPT = 1002
SEED_PHILOX = 1003
SEED_LOGITS = 1004
SEED_DIRICHLET = 1005
SEED_HEADS = 1006

WEIGHT_NAMES = ("embed", "attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd",
                "final_norm", "lm_head")


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    rope_theta: float = 10000.0
    rms_eps: float = 1e-5
    tied_head: bool = False      # lm_head is the embedding matrix

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def shapes(self) -> Dict[str, Tuple[int, ...]]:
        L, d, F, V = self.n_layers, self.d_model, self.d_ffn, self.vocab
        return {
            "embed": (V, d), "attn_norm": (L, d), "wq": (L, self.q_dim, d),
            "wk": (L, self.kv_dim, d), "wv": (L, self.kv_dim, d), "wo": (L, d, self.q_dim),
            "ffn_norm": (L, d), "wg": (L, F, d), "wu": (L, F, d), "wd": (L, d, F),
            "final_norm": (d,), "lm_head": (V, d),
        }

    def weight_bytes(self) -> int:
        """bf16 bytes of every matrix a forward pass streams (embedding rows
        excluded: a pass reads only a few of them)."""
        s = self.shapes()
        n = sum(int(np.prod(s[k])) for k in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm",
                                             "wg", "wu", "wd", "final_norm", "lm_head"))
        return 2 * n

    def replace(self, **kw) -> "ModelConfig":
        return dataclasses.replace(self, **kw)


# --- the workloads' model pairs ------------------------------------------
TOY = ModelConfig("toy-2L-d64", 2, 64, 4, 4, 16, 256, 256)
TOY_DRAFT = TOY.replace(name="toy-draft-layer0", n_layers=1)   # target layer 0 + shared head

L13B = ModelConfig("llama-1.3b-shape", 24, 2048, 16, 16, 128, 5504, 32000)
L13B_DRAFT = L13B.replace(name="llama-1.3b-draft-4L", n_layers=4)  # shares embed + head

L8B = ModelConfig("llama-8b-shape", 32, 4096, 32, 8, 128, 14336, 128256, rope_theta=500000.0)
L8B_DRAFT = ModelConfig("llama-1b-shape-draft", 16, 2048, 32, 8, 64, 8192, 128256,
                        rope_theta=500000.0, tied_head=True)

G31B = ModelConfig("31b-shape", 60, 5376, 32, 16, 168, 21504, 262144)
G31B_DRAFT = ModelConfig("4b-shape-draft", 34, 2560, 20, 4, 128, 10240, 262144, tied_head=True)

PAIRS = {
    "toy": (TOY, TOY_DRAFT),
    "1.3b": (L13B, L13B_DRAFT),
    "8b": (L8B, L8B_DRAFT),
    "31b": (G31B, G31B_DRAFT),
}


def _sub_seed(seed: int, name: str) -> list:
    return [int(seed), zlib.crc32(name.encode())]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns
    (storage conversion of generated inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


ONE_BF16 = 0x3F80


def weights_np(cfg: ModelConfig, seed: int = SEED_WEIGHTS, std: float = 0.02,
               names=WEIGHT_NAMES) -> Dict[str, np.ndarray]:
    """Host weights as bf16 bit patterns (uint16), stacked over layers."""
    out = {}
    for k, shp in cfg.shapes().items():
        if k not in names:
            continue
        if k in ("attn_norm", "ffn_norm", "final_norm"):
            out[k] = np.full(shp, ONE_BF16, np.uint16)
        elif k == "lm_head" and cfg.tied_head:
            continue
        else:
            rng = np.random.default_rng(_sub_seed(seed, cfg.name + "/" + k))
            out[k] = f32_to_bf16_bits(rng.standard_normal(shp, dtype=np.float32) * np.float32(std))
    if cfg.tied_head and "lm_head" in names:
        out["lm_head"] = out["embed"]
    return out


def weights_torch(cfg: ModelConfig, seed: int = SEED_WEIGHTS, device="cuda", std: float = 0.02,
                  share_from: Optional[Dict[str, "object"]] = None, share=()):
    """Device weights as torch.bfloat16 tensors (torch's generator on the
    device, then round-to-nearest-even to bf16).  Tensors named in `share`
    are taken from `share_from` (e.g. a draft sharing the target's embedding
    and LM head)."""
    import torch
    out = {}
    for k, shp in cfg.shapes().items():
        if share_from is not None and k in share:
            out[k] = share_from[k]
            continue
        if k in ("attn_norm", "ffn_norm", "final_norm"):
            out[k] = torch.ones(shp, dtype=torch.bfloat16, device=device)
        elif k == "lm_head" and cfg.tied_head:
            continue
        else:
            g = torch.Generator(device=device)
            g.manual_seed(zlib.crc32(f"{seed}/{cfg.name}/{k}".encode()))
            t = torch.empty(shp, dtype=torch.bfloat16, device=device)
            # generate in chunks to bound the fp32 temporary
            flat = t.view(-1)
            step = 1 << 26
            for i in range(0, flat.numel(), step):
                n = min(step, flat.numel() - i)
                flat[i:i + n].copy_(torch.randn(n, generator=g, device=device,
                                                dtype=torch.float32) * std)
            out[k] = t
    if cfg.tied_head:
        out["lm_head"] = out["embed"]
    return out


def heads_np(cfg: ModelConfig, n_heads: int, seed: int = SEED_HEADS, std: float = 0.02) -> np.ndarray:
    """Drafting-head matrices [n_heads][d][d] as bf16 bit patterns, N(0, std)."""
    rng = np.random.default_rng(_sub_seed(seed, f"{cfg.name}/heads/{n_heads}"))
    shp = (n_heads, cfg.d_model, cfg.d_model)
    return f32_to_bf16_bits(rng.standard_normal(shp, dtype=np.float32) * np.float32(std))


def heads_torch(cfg: ModelConfig, n_heads: int, seed: int = SEED_HEADS, device="cuda",
                std: float = 0.02):
    """Drafting-head matrices [n_heads][d][d] as a torch.bfloat16 device tensor."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(zlib.crc32(f"{seed}/{cfg.name}/heads/{n_heads}".encode()))
    t = torch.randn((n_heads, cfg.d_model, cfg.d_model), generator=g, device=device,
                    dtype=torch.float32) * std
    return t.to(torch.bfloat16)


def torch_to_bits(weights) -> Dict[str, np.ndarray]:
    """Host copies (uint16 bit patterns) of device bf16 weights."""
    import torch
    return {k: v.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            for k, v in weights.items()}


def self_draft_np(target_w: Dict[str, np.ndarray], n_layers: int = 1) -> Dict[str, np.ndarray]:
    """Draft made of the target's first `n_layers` layers plus the target's
    embedding, final norm and LM head (self-speculative)."""
    out = {}
    for k, v in target_w.items():
        if k in ("embed", "final_norm", "lm_head"):
            out[k] = v
        else:
            out[k] = np.ascontiguousarray(v[:n_layers])
    return out


def prompt(vocab: int, n: int, seed: int = SEED_PROMPT) -> np.ndarray:
    """iid uniform token ids."""
    return np.random.default_rng([seed, vocab, n]).integers(0, vocab, size=n, dtype=np.int32)


def _softmax64(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def logit_pair(B: int, K: int, V: int, sigma: float, seed: int = SEED_LOGITS,
               std: float = 2.0) -> Tuple[np.ndarray, np.ndarray]:
    """Isolated accept/reject inputs: per (sequence, row) independent target
    logits ~ N(0, std); draft logits = target logits + N(0, sigma).  Returns
    fp32 probability rows T [B][K+1][V] and D [B][K][V]."""
    rng = np.random.default_rng([seed, B, K, V, int(round(sigma * 1000))])
    zt = rng.standard_normal((B, K + 1, V)) * std
    zd = zt[:, :K, :] + rng.standard_normal((B, K, V)) * sigma
    return _softmax64(zt).astype(np.float32), _softmax64(zd).astype(np.float32)


def drafts_from_rows(D: np.ndarray, seed: int = SEED_LOGITS) -> np.ndarray:
    """Draft tokens for the isolated rule's inputs: one categorical draw per
    row of D [B][K][V] with numpy's generator (an input recipe only; the
    library's own drafters draw differently)."""
    rng = np.random.default_rng([seed, *D.shape])
    c = np.cumsum(D.astype(np.float64), axis=-1)
    u = rng.random(D.shape[:-1]) * c[..., -1]
    idx = (c < u[..., None]).sum(axis=-1)
    return np.minimum(idx, D.shape[-1] - 1).astype(np.int32)


def dirichlet_pair(V: int, seed: int = SEED_DIRICHLET) -> Tuple[np.ndarray, np.ndarray]:
    """T, D ~ Dirichlet(1) over V entries (normalized Exp(1)), fp32."""
    rng = np.random.default_rng([seed, V])
    t = rng.dirichlet(np.ones(V)).astype(np.float32)
    d = rng.dirichlet(np.ones(V)).astype(np.float32)
    return t, d
