"""Device-resident synthetic workloads built from the seeded generator
(inputs.py) and wrapped for the library: a block-prefill workload and the
whole-model decode workload with its pre-filled KV cache."""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import torch

from . import inputs as I
from . import ops


@dataclasses.dataclass
class BlockWorkload:
    w: I.Workload
    weights: Dict[str, torch.Tensor]
    x: torch.Tensor
    block: "ops.Block"


def block_workload(wid: int, device="cuda", numerics: int = 0, weights_f16: bool = False) -> BlockWorkload:
    """A block's seeded weights, input and callable. With `weights_f16`, the
    projections with fp16 operands get their weights converted to fp16 once,
    here (LLAMA_NUM_W_F16: the same bits the in-register conversion gives)."""
    w = I.workload(wid)
    wt = I.block_weights(w, device=device)
    x = I.block_input(w, device=device)
    if weights_f16:
        numerics, wt = ops.with_f16_weights(numerics, wt)
    cfg = ops.config(w.dim, w.n_heads, w.hidden, dtype=w.torch_dtype, eps=w.eps, theta=w.theta,
                     numerics=numerics, n_kv_heads=w.n_kv_heads)
    return BlockWorkload(w, wt, x, ops.Block(cfg, wt, w.batch, w.seq))


@dataclasses.dataclass
class DecodeWorkload:
    w: I.Workload
    layers: List[Dict[str, torch.Tensor]]
    globals: Dict[str, torch.Tensor]
    model: "ops.Model"
    tokens: torch.Tensor       # [B] int32
    pos: torch.Tensor          # [B] int32
    k_cache: torch.Tensor      # [L, B, H, max_seq, hd]
    v_cache: torch.Tensor


def decode_workload(wid: int, device="cuda", pack: bool = True) -> DecodeWorkload:
    """Model decode step: every sequence at position decode_pos with cache slots
    0..decode_pos-1 pre-filled with seeded N(0, 1) keys and values. With
    `pack`, the projections are also repacked into tile order for decode (a
    load-time copy of the weights)."""
    w = I.workload(wid)
    layers = [I.block_weights(w, l, device=device) for l in range(w.n_layers)]
    gl = I.model_globals(w, device=device)
    cfg = ops.config(w.dim, w.n_heads, w.hidden, dtype=w.torch_dtype, n_layers=w.n_layers, vocab=w.vocab,
                     max_seq=w.max_seq, eps=w.eps, theta=w.theta, n_kv_heads=w.n_kv_heads)
    m = ops.Model(cfg, layers, gl["tok_embeddings"], gl["final_norm"], gl["output"])
    shape = (w.n_layers, w.batch, w.kv_heads, w.max_seq, w.head_dim)
    kc = torch.empty(shape, dtype=w.torch_dtype, device=device)
    vc = torch.empty(shape, dtype=w.torch_dtype, device=device)
    for l in range(w.n_layers):
        k, v = I.kv_cache_layer(w, l, w.decode_pos, device=device)
        kc[l].copy_(k)
        vc[l].copy_(v)
        del k, v
    if pack:
        m.pack_for_decode()
    toks = I.tokens(w, (w.batch,), device=device)
    pos = torch.full((w.batch,), w.decode_pos, dtype=torch.int32, device=device)
    return DecodeWorkload(w, layers, gl, m, toks, pos, kc, vc)
