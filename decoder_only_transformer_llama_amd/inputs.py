"""Seeded synthetic inputs for the LLaMA block / model workloads.

This module only draws random numbers and describes workload shapes. It holds
none of the method's arithmetic (no norm, projection, rotation, attention or
activation), so both the HIP path and the CPU oracle can take their inputs
from it without sharing any computation.

Every tensor comes from its own torch.Generator seeded from
(workload id, layer, tensor id). Values are drawn as float32 N(0, 1), scaled
and shifted in float32, then rounded to the workload dtype with torch's
round-to-nearest-even conversion. On a CUDA device the draw uses torch's
Philox generator; on the CPU, torch's CPU generator. A test that compares the
GPU path with the oracle draws on one device and hands the oracle a host copy
of the very same bits.

Workload shapes follow the LLaMA size table (paperfordummies.in LLaMA page,
"6.7B parameters, 1T tokens: the arithmetic"; zhongzhoutan-coder LLaMA note,
"Token Scaling for Inference Budgets" table).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

# Tensor ids inside one (workload, layer) seed space.
T_X, T_ATTN_NORM, T_WQ, T_WK, T_WV, T_WO = 0, 1, 2, 3, 4, 5
T_FFN_NORM, T_W_GATE, T_W_UP, T_W_DOWN = 6, 7, 8, 9
T_TOK_EMB, T_FINAL_NORM, T_OUTPUT, T_K_CACHE, T_V_CACHE, T_TOKENS = 10, 11, 12, 13, 14, 15
T_Q, T_K, T_V, T_POS = 16, 17, 18, 19
T_BUMP = 20

WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic workload."""
    wid: int
    name: str
    dim: int
    n_heads: int
    hidden: int
    batch: int
    seq: int
    dtype: str                 # "f32" or "bf16"
    gain_std: float = 0.0      # norm gains are 1 + N(0, gain_std); 0 -> exactly 1
    eps: float = 1e-6
    theta: float = 10000.0
    n_layers: int = 1
    vocab: int = 0
    max_seq: int = 0
    decode_pos: int = -1       # >= 0: a decode step at this position (cache holds 0..pos-1)
    n_kv_heads: int = 0        # key/value heads (0: n_heads; fewer: grouped-query attention)
    fan_in_init: bool = False  # weights N(0, 1/fan_in) instead of N(0, WEIGHT_STD^2)

    @property
    def head_dim(self) -> int:
        return self.dim // self.n_heads

    @property
    def kv_heads(self) -> int:
        return self.n_kv_heads or self.n_heads

    @property
    def kv_dim(self) -> int:
        return self.kv_heads * self.head_dim

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS: Dict[int, Workload] = {
    # tiny fp32 block
    0: Workload(0, "tiny-block-f32", dim=256, n_heads=4, hidden=768, batch=1, seq=128, dtype="f32"),
    # LLaMA-7B-shape block prefill
    1: Workload(1, "7b-block-prefill-s2048", dim=4096, n_heads=32, hidden=11008, batch=1, seq=2048,
                dtype="bf16", gain_std=0.1),
    # LLaMA-13B-shape block prefill, 4 sequences
    2: Workload(2, "13b-block-prefill-b4-s2048", dim=5120, n_heads=40, hidden=13824, batch=4, seq=2048,
                dtype="bf16"),
    # LLaMA-65B-shape block prefill, 2 sequences
    3: Workload(3, "65b-block-prefill-b2-s2048", dim=8192, n_heads=64, hidden=22016, batch=2, seq=2048,
                dtype="bf16"),
    # LLaMA-7B-shape full-model decode step, batch 32, cache of 2047 positions
    4: Workload(4, "7b-model-decode-b32-kv2047", dim=4096, n_heads=32, hidden=11008, batch=32, seq=1,
                dtype="bf16", n_layers=32, vocab=32000, max_seq=2048, decode_pos=2047),
    # norm placement study: a stack of 32 small blocks (d 64, one head, SwiGLU
    # hidden 256), one sequence of 16 tokens, fp32, weights N(0, 1/fan_in), gains 1
    7: Workload(7, "norm-placement-d64-l32-s16", dim=64, n_heads=1, hidden=256, batch=1, seq=16, dtype="f32",
                eps=1e-5, n_layers=32, fan_in_init=True),
    # fp32 training step at a size where the kernels, not the launches, set the
    # time: d 1024 (8 heads of 128), SwiGLU hidden 2816, one sequence of 1024
    8: Workload(8, "train-block-f32-d1024-s1024", dim=1024, n_heads=8, hidden=2816, batch=1, seq=1024,
                dtype="f32", gain_std=0.1),
    # the same model with grouped-query attention: 8 key/value heads (groups of 4)
    5: Workload(5, "7b-gqa8-model-decode-b32-kv2047", dim=4096, n_heads=32, hidden=11008, batch=32, seq=1,
                dtype="bf16", n_layers=32, vocab=32000, max_seq=2048, decode_pos=2047, n_kv_heads=8),
}

# Small workloads used only by tests (same recipes, shapes that run in seconds
# on the CPU and still span several GEMM / attention tiles and a ragged tail).
TEST_WORKLOADS: Dict[int, Workload] = {
    100: Workload(100, "test-block-bf16-ragged", dim=512, n_heads=4, hidden=1536, batch=2, seq=200,
                  dtype="bf16", gain_std=0.1),
    101: Workload(101, "test-model-bf16", dim=256, n_heads=2, hidden=768, batch=3, seq=40, dtype="bf16",
                  n_layers=2, vocab=1000, max_seq=64, gain_std=0.1),
    102: Workload(102, "test-model-f32", dim=256, n_heads=4, hidden=768, batch=2, seq=24, dtype="f32",
                  n_layers=2, vocab=300, max_seq=32),
    103: Workload(103, "test-block-bf16-hd64", dim=256, n_heads=4, hidden=768, batch=1, seq=129,
                  dtype="bf16"),
    # grouped-query attention: 8 query heads on 2 key/value heads (head_dim 64), ragged seq
    104: Workload(104, "test-block-bf16-gqa", dim=512, n_heads=8, hidden=1536, batch=2, seq=200, dtype="bf16",
                  gain_std=0.1, n_kv_heads=2),
    # grouped-query model, head_dim 128, groups of 4
    105: Workload(105, "test-model-bf16-gqa", dim=1024, n_heads=8, hidden=2816, batch=3, seq=40, dtype="bf16",
                  n_layers=2, vocab=1000, max_seq=64, gain_std=0.1, n_kv_heads=2),
    # fp32 training block: head_dim 128, two sequences of a ragged length
    107: Workload(107, "test-train-block-f32", dim=256, n_heads=2, hidden=768, batch=2, seq=37, dtype="f32",
                  gain_std=0.1),
    # one layer at the LLaMA-7B widths with the 32000-wide head: the model
    # path (embedding, split-K down projection, fp16 head) at full width
    108: Workload(108, "test-model-7b-dims-1layer", dim=4096, n_heads=32, hidden=11008, batch=1, seq=256,
                  dtype="bf16", n_layers=1, vocab=32000, max_seq=512, gain_std=0.1),
    # multi-query model (one key/value head), head_dim 128, groups of 4
    106: Workload(106, "test-model-bf16-mqa", dim=512, n_heads=4, hidden=1536, batch=2, seq=24, dtype="bf16",
                  n_layers=2, vocab=500, max_seq=48, n_kv_heads=1),
    # grouped-query models at head_dim 128 with groups of 2 and of 8 (one
    # key/value head), prompts past one 32-key decode chunk
    109: Workload(109, "test-model-bf16-gqa2", dim=1024, n_heads=8, hidden=2816, batch=2, seq=70, dtype="bf16",
                  n_layers=2, vocab=500, max_seq=96, gain_std=0.1, n_kv_heads=4),
    110: Workload(110, "test-model-bf16-gqa8", dim=1024, n_heads=8, hidden=2816, batch=3, seq=45, dtype="bf16",
                  n_layers=2, vocab=500, max_seq=64, gain_std=0.1, n_kv_heads=1),
}


def workload(wid: int) -> Workload:
    if wid in WORKLOADS:
        return WORKLOADS[wid]
    return TEST_WORKLOADS[wid]


def seed_of(wid: int, layer: int, tensor: int) -> int:
    """Seed of the stream for (workload, layer, tensor)."""
    return ((1000 + wid) << 32) | ((layer & 0xFFFF) << 16) | (tensor & 0xFFFF)


def generator(wid: int, layer: int, tensor: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(wid, layer, tensor))
    return g


def normal(shape, wid: int, layer: int, tensor: int, *, std: float = 1.0, mean: float = 0.0,
           dtype: torch.dtype = torch.float32, device="cpu") -> torch.Tensor:
    """N(mean, std^2) drawn in float32, rounded (RNE) to `dtype`."""
    g = generator(wid, layer, tensor, device)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def uniform_int(shape, high: int, wid: int, layer: int, tensor: int, device="cpu") -> torch.Tensor:
    g = generator(wid, layer, tensor, device)
    return torch.randint(0, high, shape, generator=g, device=device, dtype=torch.int64).to(torch.int32)


def gain(w: Workload, layer: int, tensor: int, device="cpu") -> torch.Tensor:
    if w.gain_std == 0.0:
        return torch.ones(w.dim, dtype=w.torch_dtype, device=device)
    return normal((w.dim,), w.wid, layer, tensor, std=w.gain_std, mean=1.0, dtype=w.torch_dtype,
                  device=device)


def block_weights(w: Workload, layer: int = 0, device="cpu") -> Dict[str, torch.Tensor]:
    """Weights of one block, [out, in] row-major (y = x W^T): N(0, 0.02^2), or
    N(0, 1/in) with `fan_in_init`."""
    d, h, dt = w.dim, w.hidden, w.torch_dtype
    wid = w.wid
    sd = (lambda fan_in: fan_in ** -0.5) if w.fan_in_init else (lambda fan_in: WEIGHT_STD)
    return {
        "attn_norm": gain(w, layer, T_ATTN_NORM, device),
        "wq": normal((d, d), wid, layer, T_WQ, std=sd(d), dtype=dt, device=device),
        "wk": normal((w.kv_dim, d), wid, layer, T_WK, std=sd(d), dtype=dt, device=device),
        "wv": normal((w.kv_dim, d), wid, layer, T_WV, std=sd(d), dtype=dt, device=device),
        "wo": normal((d, d), wid, layer, T_WO, std=sd(d), dtype=dt, device=device),
        "ffn_norm": gain(w, layer, T_FFN_NORM, device),
        "w_gate": normal((h, d), wid, layer, T_W_GATE, std=sd(d), dtype=dt, device=device),
        "w_up": normal((h, d), wid, layer, T_W_UP, std=sd(d), dtype=dt, device=device),
        "w_down": normal((d, h), wid, layer, T_W_DOWN, std=sd(h), dtype=dt, device=device),
    }


def bump_direction(w: Workload, device="cpu") -> torch.Tensor:
    """Unit-Frobenius-norm direction [tokens, dim] (fp32) for the
    finite-difference probe of a block stack."""
    u = normal((w.tokens, w.dim), w.wid, 0, T_BUMP, device=device)
    return u / torch.linalg.vector_norm(u)


def block_input(w: Workload, device="cpu") -> torch.Tensor:
    """Block input x [batch*seq, dim] ~ N(0, 1) in the workload dtype."""
    return normal((w.tokens, w.dim), w.wid, 0, T_X, dtype=w.torch_dtype, device=device)


def qkv_inputs(w: Workload, device="cpu"):
    """Standalone attention inputs q, k, v [batch*seq, dim] ~ N(0, 1)."""
    shape = (w.tokens, w.dim)
    return tuple(normal(shape, w.wid, 0, t, dtype=w.torch_dtype, device=device)
                 for t in (T_Q, T_K, T_V))


def model_globals(w: Workload, device="cpu") -> Dict[str, torch.Tensor]:
    """Embedding table, final norm gain and output head of a model workload."""
    dt = w.torch_dtype
    L = w.n_layers
    return {
        "tok_embeddings": normal((w.vocab, w.dim), w.wid, L, T_TOK_EMB, std=WEIGHT_STD, dtype=dt,
                                 device=device),
        "final_norm": gain(w, L, T_FINAL_NORM, device),
        "output": normal((w.vocab, w.dim), w.wid, L, T_OUTPUT, std=WEIGHT_STD, dtype=dt, device=device),
    }


def tokens(w: Workload, shape, device="cpu", stream: int = 0) -> torch.Tensor:
    return uniform_int(shape, w.vocab, w.wid, w.n_layers + stream, T_TOKENS, device)


def kv_cache_layer(w: Workload, layer: int, filled: int, device="cpu",
                   out: Optional[torch.Tensor] = None, batch_slice=None):
    """One layer's seeded K and V cache, [batch, n_heads, max_seq, head_dim].

    Positions [0, filled) hold N(0, 1) values (taken as already-rotated keys);
    the rest are zero. `batch_slice` returns only those sequences (the draw is
    still the full batch, so the bits match the full cache)."""
    shape = (w.batch, w.kv_heads, filled, w.head_dim)
    res = []
    for t in (T_K_CACHE, T_V_CACHE):
        full = normal(shape, w.wid, layer, t, dtype=w.torch_dtype, device=device)
        if batch_slice is not None:
            full = full[batch_slice]
        c = torch.zeros((full.shape[0], w.kv_heads, w.max_seq, w.head_dim), dtype=w.torch_dtype,
                        device=device)
        c[:, :, :filled] = full
        res.append(c)
    return res[0], res[1]
