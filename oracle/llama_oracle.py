"""CPU fp64 oracle of the LLaMA pre-norm decoder block, final norm, output head
and KV-cache decode step.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module. The product path (the HIP
library and its Python binding) never does; it shares no code, table or
constant with this file.

Everything is plain NumPy float64 with no intermediate rounding, written from
the definitions on the pages:

  [P1] paperfordummies.in, "LLaMA: Open and Efficient Foundation Language
       Models" (the "explained as a diff" page), sections "The one formula",
       "RMSNorm: LayerNorm minus the mean", "SwiGLU: a gate in the FFN ...",
       "RoPE: rotate Q and K, leave V alone", "6.7B parameters, 1T tokens: the
       arithmetic" and "The code".
  [P4] chenyuan1125.github.io, "LLaMA: No Architecture Revolution, Yet It
       Became the Open-Model Foundation", section "An Architecture Recipe
       Without an Invention Myth" (RMSNorm-with-gain, SwiGLU and RoPE
       equations) and "GQA Was Not an Original LLaMA Feature" (KV cache).
  [P3] zhongzhoutan-coder.github.io, the LLaMA training note, section
       "Efficient Training Implementation" (manual backward, FlashAttention-
       style attention backward, checkpointing of linear outputs).

Readings where the pages leave a step open (softmax scale, mask, head split,
weight layout, per-head RoPE frequencies) are listed in the repository's design
notes; each function below states the one it takes.

Layouts: activations are [tokens, dim] with token = b*seq + s; head h owns
columns [h*hd, (h+1)*hd). Weights are [out, in], so linear(x, W) = x W^T (the
[P1] code writes x @ W with W [in, out]: the same map).
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Tuple

import numpy as np


def f64(a) -> np.ndarray:
    """Widen a host array (or a CPU torch tensor of any float dtype) to fp64 exactly."""
    if hasattr(a, "detach"):
        import torch  # only for the dtype widening of torch inputs
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- sizes
def llama_hidden(dim: int, multiple_of: int = 256) -> int:
    """SwiGLU hidden width ([P1] "SwiGLU: a gate in the FFN"): the vanilla
    FFN's 4*dim cut to two thirds, then rounded up to a multiple of
    `multiple_of` (256), the smallest such multiple at or above 8*dim/3,
    found here in exact integer arithmetic. For multiples of 8 this agrees
    with truncating 8*dim/3 first: 8*dim is then never one or two above a
    multiple of 3*multiple_of."""
    units = -(-(8 * dim) // (3 * multiple_of))   # ceil(8 dim / (3 multiple_of))
    return units * multiple_of


def count_params(dim: int, n_layers: int, hidden: int, vocab: int = 32000, bias: bool = False) -> int:
    """Parameter count of the model ([P1] "6.7B parameters ... the arithmetic").

    Per layer: four dim x dim attention matrices, three dim x hidden FFN
    matrices and two norm gains; plus an embedding table and an untied output
    head (vocab x dim each) and the final norm gain. With bias=True every block
    linear gets an output bias (q, k, v, o: 4*dim; gate, up: 2*hidden; down:
    dim) and each of the two block norms a shift (2*dim); this reading
    reproduces the page's +1,622,016 at 7B."""
    per_layer = 4 * dim * dim + 3 * dim * hidden + 2 * dim
    if bias:
        per_layer += 4 * dim + 2 * hidden + dim + 2 * dim
    return n_layers * per_layer + 2 * vocab * dim + dim


# --------------------------------------------------------------------------- primitives
def rmsnorm(x: np.ndarray, g: np.ndarray | None, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis ([P1] `rms_norm`; [P4]
    RMSNorm equation with gain g). eps sits inside the square root."""
    x = f64(x)
    rms = np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    y = x / rms
    if g is not None:
        y = y * f64(g)
    return y


def layernorm(x: np.ndarray, eps: float = 0.0) -> np.ndarray:
    """LayerNorm without affine terms, only used to pin rmsnorm on a centred vector
    ([P1] "RMSNorm: LayerNorm minus the mean")."""
    x = f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def silu(x: np.ndarray) -> np.ndarray:
    """x / (1 + e^-x) ([P1] `silu`). Written with exp of -|x| so large |x| gives
    no overflow warning; mathematically the same function."""
    x = f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, x / (1.0 + e), x * e / (1.0 + e))


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[t, o] = sum_k x[t, k] * W[o, k] (weights stored [out, in])."""
    return f64(x) @ f64(w).T


def rope(x: np.ndarray, positions: np.ndarray, head_dim: int, theta: float = 10000.0) -> np.ndarray:
    """Rotary position embedding, applied per head ([P4] RoPE equation; [P1]
    "RoPE: rotate Q and K, leave V alone").

    Channels (2i, 2i+1) of a head are one point of the plane, read as the
    complex number x[2i] + j x[2i+1]; RoPE turns it by the angle
    pos * theta^(-2i/hd), i.e. multiplies it by exp(j pos theta^(-2i/hd)),
    with hd the head dimension (reading: the frequencies run over one head's
    pairs). The pairs are adjacent channels, the interleaved layout of [P1]."""
    x = f64(x)
    t, width = x.shape
    assert width % head_dim == 0 and head_dim % 2 == 0
    pairs = x.reshape(t, width // head_dim, head_dim // 2, 2)
    z = pairs[..., 0] + 1j * pairs[..., 1]                                    # (t, heads, hd/2)
    i = np.arange(head_dim // 2, dtype=np.float64)
    freq = np.power(float(theta), -2.0 * i / head_dim)                        # per-pair frequency
    turn = np.exp(1j * np.asarray(positions, dtype=np.float64)[:, None, None] * freq[None, None, :])
    w = z * turn
    return np.stack([w.real, w.imag], axis=-1).reshape(t, width)


def causal_attention(q, k, v, batch: int, seq: int, n_heads: int) -> np.ndarray:
    """Scaled dot-product attention with a causal mask, per (sequence, head).

    Readings: scores are q.k / sqrt(hd); key j is visible to query i iff j <= i
    (diagonal included) and masked keys get exactly zero weight; head h owns
    columns [h*hd, (h+1)*hd) and heads are concatenated back in that order
    ([P1] "LLaMA is a pull request ...": the 2017 attention with a causal mask,
    untouched).

    k and v may hold fewer heads than q (grouped-query attention, [P4] "GQA
    Was Not an Original LLaMA Feature": a group of query heads shares one
    key-value head). Reading: the groups are consecutive, query head h uses
    key-value head h // (n_heads / n_kv_heads); equal head counts are plain
    multi-head attention."""
    q, k, v = f64(q), f64(k), f64(v)
    d = q.shape[1]
    hd = d // n_heads
    group = n_heads // (k.shape[1] // hd)
    out = np.empty_like(q)
    mask = np.triu(np.ones((seq, seq), dtype=bool), 1)        # True above the diagonal
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for h in range(n_heads):
            cols = slice(h * hd, (h + 1) * hd)
            kv = slice((h // group) * hd, (h // group + 1) * hd)
            s = q[rows, cols] @ k[rows, kv].T / math.sqrt(hd)
            s[mask] = -np.inf
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[rows, cols] = p @ v[rows, kv]
    return out


def attention_over_cache(q, k_cache, v_cache, q_pos, n_heads: int) -> np.ndarray:
    """Attention of one query row per sequence over that sequence's cached keys
    0..q_pos[b] (inclusive). q [B, dim]; caches [B, n_kv_heads, max_seq, hd]
    (query head h reads key-value head h // (n_heads / n_kv_heads))."""
    q = f64(q)
    B, d = q.shape
    hd = d // n_heads
    group = n_heads // k_cache.shape[1]
    out = np.empty_like(q)
    for b in range(B):
        p_end = int(q_pos[b]) + 1
        for h in range(n_heads):
            kk = f64(k_cache[b, h // group, :p_end])
            vv = f64(v_cache[b, h // group, :p_end])
            s = kk @ q[b, h * hd:(h + 1) * hd] / math.sqrt(hd)
            s = s - s.max()
            p = np.exp(s)
            p /= p.sum()
            out[b, h * hd:(h + 1) * hd] = p @ vv
    return out


def swiglu_ffn(z, w_gate, w_up, w_down) -> np.ndarray:
    """(silu(z Wg^T) * (z Wu^T)) Wd^T ([P1] `swiglu_ffn`; [P4] SwiGLU)."""
    return linear(silu(linear(z, w_gate)) * linear(z, w_up), w_down)


# --------------------------------------------------------------------------- block
def block_forward(x, w: Dict[str, np.ndarray], batch: int, seq: int, n_heads: int,
                  eps: float, theta: float = 10000.0, return_parts: bool = False):
    """One pre-norm LLaMA block ([P1] "The one formula" and `pre_norm_block`):

        h = x + Wo . CausalAttn(RoPE(Wq z), RoPE(Wk z), Wv z),  z  = RMSNorm(x; g1)
        y = h + Wdown (SiLU(Wgate z2) * Wup z2),                 z2 = RMSNorm(h; g2)

    No biases. RoPE positions are 0..seq-1 within every sequence; V is not
    rotated ([P1] "RoPE: rotate Q and K, leave V alone")."""
    x = f64(x)
    d = x.shape[1]
    hd = d // n_heads
    pos = np.tile(np.arange(seq, dtype=np.float64), batch)
    z = rmsnorm(x, w["attn_norm"], eps)
    q = rope(linear(z, w["wq"]), pos, hd, theta)
    k = rope(linear(z, w["wk"]), pos, hd, theta)
    v = linear(z, w["wv"])
    a = causal_attention(q, k, v, batch, seq, n_heads)
    h = x + linear(a, w["wo"])
    z2 = rmsnorm(h, w["ffn_norm"], eps)
    y = h + swiglu_ffn(z2, w["w_gate"], w["w_up"], w["w_down"])
    if return_parts:
        return y, {"z": z, "q": q, "k": k, "v": v, "attn": a, "h": h, "z2": z2}
    return y


# --------------------------------------------------------------------------- norm placement
def attn_sublayer(z, w: Dict[str, np.ndarray], batch: int, seq: int, n_heads: int,
                  theta: float = 10000.0) -> np.ndarray:
    """Wo . CausalAttn(RoPE(Wq z), RoPE(Wk z), Wv z): the attention branch of a
    block applied to whatever the placement feeds it."""
    z = f64(z)
    hd = z.shape[1] // n_heads
    pos = np.tile(np.arange(seq, dtype=np.float64), batch)
    q = rope(linear(z, w["wq"]), pos, hd, theta)
    k = rope(linear(z, w["wk"]), pos, hd, theta)
    return linear(causal_attention(q, k, linear(z, w["wv"]), batch, seq, n_heads), w["wo"])


def post_norm_block_forward(x, w: Dict[str, np.ndarray], batch: int, seq: int, n_heads: int,
                            eps: float, theta: float = 10000.0) -> np.ndarray:
    """The 2017 ordering, norm on the trunk after each residual add ([P1]
    "Pre-norm: the norm goes on the branch, not the trunk"):

        h = RMSNorm(x + Attn(x); g1),   y = RMSNorm(h + FFN(h); g2)

    with the same attention and SwiGLU branches as the LLaMA block. Reading:
    the block's two gains (attn_norm, ffn_norm) scale the two trunk norms; with
    g = 1 and eps = 0 every output row has norm sqrt(dim) exactly, the page's
    "pins the trunk at sqrt(d)"."""
    x = f64(x)
    h = rmsnorm(x + attn_sublayer(x, w, batch, seq, n_heads, theta), w["attn_norm"], eps)
    return rmsnorm(h + swiglu_ffn(h, w["w_gate"], w["w_up"], w["w_down"]), w["ffn_norm"], eps)


def no_norm_block_forward(x, w: Dict[str, np.ndarray], batch: int, seq: int, n_heads: int,
                          eps: float = 0.0, theta: float = 10000.0) -> np.ndarray:
    """The pre-norm block with both RMSNorm calls deleted ([P1] "Now break it":
    the no-norm block): h = x + Attn(x), y = h + FFN(h). The gains and eps are
    unused."""
    x = f64(x)
    h = x + attn_sublayer(x, w, batch, seq, n_heads, theta)
    return h + swiglu_ffn(h, w["w_gate"], w["w_up"], w["w_down"])


PLACEMENTS = {"pre": block_forward, "post": post_norm_block_forward, "none": no_norm_block_forward}


def stack_forward(x, blocks, batch: int, seq: int, n_heads: int, eps: float, placement: str = "pre",
                  theta: float = 10000.0):
    """Blocks applied one after another (a model without embedding and head).
    Returns the output and the trunk norm after every block: the mean over
    tokens of each token's L2 norm ([P1] "Pre-norm ...": "residual-stream norm
    per token"). Overflow is left to IEEE arithmetic (inf, then NaN), as in the
    page's no-norm run."""
    f = PLACEMENTS[placement]
    x = f64(x)
    norms = []
    with np.errstate(over="ignore", invalid="ignore"):
        for w in blocks:
            x = f(x, w, batch, seq, n_heads, eps, theta)
            norms.append(float(np.mean(np.sqrt(np.sum(x * x, axis=1)))))
    return x, norms


def amplification(x, direction, delta: float, blocks, batch: int, seq: int, n_heads: int, eps: float,
                  placement: str = "pre", theta: float = 10000.0) -> float:
    """Finite-difference probe of [P1] "Pre-norm ...": bump the stack's input
    by delta along `direction`, run both inputs through the blocks, and divide
    how far the output moved by how far the input moved:
        ||F(x + delta u) - F(x)|| / ||delta u||   (Frobenius norms).
    Reading: the page does not print the bump's shape; here it is one
    direction over all tokens and channels, and the ratio is the directional
    derivative's gain for small delta."""
    x, u = f64(x), f64(direction)
    y0, _ = stack_forward(x, blocks, batch, seq, n_heads, eps, placement, theta)
    y1, _ = stack_forward(x + delta * u, blocks, batch, seq, n_heads, eps, placement, theta)
    return float(np.linalg.norm(y1 - y0) / np.linalg.norm(delta * u))


def block_step_with_cache(x, w, pos, k_cache, v_cache, n_heads: int, eps: float,
                          theta: float = 10000.0) -> np.ndarray:
    """One block applied to a single new token per sequence (decode).

    x [B, dim] (fp64 residual). The rotated key and the value of the new token
    are written into cache slot pos[b] of each sequence (k_cache, v_cache are
    fp64 [B, H, max_seq, hd] and are modified in place), then the token attends
    over slots 0..pos[b] ([P4] "GQA Was Not an Original LLaMA Feature": the
    cache keeps keys and values of every previous token; LLaMA-1 is plain
    multi-head attention, one KV head per query head; with fewer key-value
    heads (Wk, Wv of n_kv_heads * hd rows) the caches hold n_kv_heads heads)."""
    x = f64(x)
    B, d = x.shape
    hd = d // n_heads
    z = rmsnorm(x, w["attn_norm"], eps)
    q = rope(linear(z, w["wq"]), pos, hd, theta)
    k = rope(linear(z, w["wk"]), pos, hd, theta)
    v = linear(z, w["wv"])
    n_kv = k.shape[1] // hd
    for b in range(B):
        p = int(pos[b])
        k_cache[b, :, p, :] = k[b].reshape(n_kv, hd)
        v_cache[b, :, p, :] = v[b].reshape(n_kv, hd)
    a = attention_over_cache(q, k_cache, v_cache, pos, n_heads)
    h = x + linear(a, w["wo"])
    z2 = rmsnorm(h, w["ffn_norm"], eps)
    return h + swiglu_ffn(z2, w["w_gate"], w["w_up"], w["w_down"])


# --------------------------------------------------------------------------- backward
# The manual backward of the pre-norm block ([P3] "Efficient Training
# Implementation": manual backward for the transformer layers, FlashAttention-
# style attention backward, checkpointing of the linear outputs). Each function
# is the chain rule of its forward written out; the tests pin every one with
# the finite-difference trick of [P1] "Pre-norm ..." (bump an input, measure how
# far the output moves, divide).
def rmsnorm_backward(x, g, eps: float, dy):
    """Gradients of y = x / sqrt(mean(x^2) + eps) * g per row: returns (dx, dg).
    With n = x * r, r = 1/sqrt(mean(x^2) + eps) and dn = dy * g:
    dx = r * (dn - n * mean(dn * n)), dg = sum over rows of dy * n."""
    x, dy = f64(x), f64(dy)
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    n = x * r
    dn = dy * (f64(g) if g is not None else 1.0)
    dx = r * (dn - n * (dn * n).mean(axis=-1, keepdims=True))
    dg = (dy * n).sum(axis=0)
    return dx, dg


def rope_backward(dy, positions, head_dim: int, theta: float = 10000.0):
    """RoPE is a rotation per pair, so its transpose is the rotation by minus
    the same angle: the gradient of rope(x) is rope(dy) at negated positions."""
    return rope(dy, -np.asarray(positions, dtype=np.float64), head_dim, theta)


def causal_attention_backward(q, k, v, do, batch: int, seq: int, n_heads: int):
    """Gradients (dq, dk, dv) of causal_attention given d(out) = do. Per
    (sequence, head), with S = q k^T / sqrt(hd) (masked) and P = softmax(S):
    dv = P^T do, dP = do v^T, dS = P * (dP - rowsum(dP * P)),
    dq = dS k / sqrt(hd), dk = dS^T q / sqrt(hd)."""
    q, k, v, do = f64(q), f64(k), f64(v), f64(do)
    d = q.shape[1]
    hd = d // n_heads
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    mask = np.triu(np.ones((seq, seq), dtype=bool), 1)
    for b in range(batch):
        rows = slice(b * seq, (b + 1) * seq)
        for h in range(n_heads):
            c = slice(h * hd, (h + 1) * hd)
            s = q[rows, c] @ k[rows, c].T / math.sqrt(hd)
            s[mask] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            g_o = do[rows, c]
            dv[rows, c] = p.T @ g_o
            dp = g_o @ v[rows, c].T
            ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
            dq[rows, c] = ds @ k[rows, c] / math.sqrt(hd)
            dk[rows, c] = ds.T @ q[rows, c] / math.sqrt(hd)
    return dq, dk, dv


def swiglu_backward(gate, up, du):
    """Gradients of u = SiLU(gate) * up: d_gate = du * up * SiLU'(gate) with
    SiLU'(t) = s(t) (1 + t (1 - s(t))), s the logistic function; d_up = du * SiLU(gate)."""
    gate, up, du = f64(gate), f64(up), f64(du)
    sg = 0.5 * (1.0 + np.tanh(0.5 * gate))      # logistic, without overflow
    return du * up * sg * (1.0 + gate * (1.0 - sg)), du * silu(gate)


def block_backward(x, w: Dict[str, np.ndarray], dy, batch: int, seq: int, n_heads: int, eps: float,
                   theta: float = 10000.0):
    """Backward of block_forward for the upstream gradient dy: returns dx and
    a dict of weight gradients with the keys of `w`. The forward's linear
    outputs (q, k, v after RoPE, the attention output, gate, up) and h are
    kept; the norms and SiLU(gate) * up are recomputed from them."""
    x, dy = f64(x), f64(dy)
    hd = x.shape[1] // n_heads
    pos = np.tile(np.arange(seq, dtype=np.float64), batch)
    z = rmsnorm(x, w["attn_norm"], eps)
    q = rope(linear(z, w["wq"]), pos, hd, theta)
    k = rope(linear(z, w["wk"]), pos, hd, theta)
    v = linear(z, w["wv"])
    a = causal_attention(q, k, v, batch, seq, n_heads)
    h = x + linear(a, w["wo"])
    z2 = rmsnorm(h, w["ffn_norm"], eps)
    gate, up = linear(z2, w["w_gate"]), linear(z2, w["w_up"])
    u = silu(gate) * up
    g = {}
    # y = h + u Wd^T
    g["w_down"] = dy.T @ u
    du = dy @ f64(w["w_down"])
    d_gate, d_up = swiglu_backward(gate, up, du)
    g["w_gate"], g["w_up"] = d_gate.T @ z2, d_up.T @ z2
    dz2 = d_gate @ f64(w["w_gate"]) + d_up @ f64(w["w_up"])
    dh_n, g["ffn_norm"] = rmsnorm_backward(h, w["ffn_norm"], eps, dz2)
    dh = dy + dh_n
    # h = x + a Wo^T
    g["wo"] = dh.T @ a
    dq, dk, dv = causal_attention_backward(q, k, v, dh @ f64(w["wo"]), batch, seq, n_heads)
    dq_lin, dk_lin = rope_backward(dq, pos, hd, theta), rope_backward(dk, pos, hd, theta)
    g["wq"], g["wk"], g["wv"] = dq_lin.T @ z, dk_lin.T @ z, dv.T @ z
    dz = dq_lin @ f64(w["wq"]) + dk_lin @ f64(w["wk"]) + dv @ f64(w["wv"])
    dx_n, g["attn_norm"] = rmsnorm_backward(x, w["attn_norm"], eps, dz)
    return dh + dx_n, g


def head(x, final_norm, output, eps: float) -> np.ndarray:
    """One final RMSNorm, then the untied vocab-wide output head ([P1] "The one
    formula": after the last block). Returns logits, no softmax."""
    return linear(rmsnorm(x, final_norm, eps), output)


# --------------------------------------------------------------------------- model
LayerFn = Callable[[int], Tuple[Dict[str, np.ndarray], np.ndarray, np.ndarray]]


def model_decode(tokens, pos, emb, get_layer: LayerFn, n_layers: int, final_norm, output,
                 n_heads: int, eps: float, theta: float = 10000.0) -> np.ndarray:
    """One decode step of the whole model: embedding rows of `tokens` [B], then
    every block with its cache, then final norm and head -> logits [B, vocab].

    `get_layer(l)` returns (weights, k_cache, v_cache) of layer l as fp64
    arrays; the caches are written in place at slot pos[b]. Streaming the
    layers through a callable keeps host memory at one layer."""
    x = f64(emb)[np.asarray(tokens, dtype=np.int64)]
    for l in range(n_layers):
        w, kc, vc = get_layer(l)
        x = block_step_with_cache(x, w, pos, kc, vc, n_heads, eps, theta)
    return head(x, final_norm, output, eps)


def model_forward(tokens, emb, get_layer: LayerFn, n_layers: int, final_norm, output,
                  n_heads: int, eps: float, theta: float = 10000.0) -> np.ndarray:
    """Prefill of the whole model over tokens [B, T] from position 0: the
    embedding rows, every block (writing each layer's rotated keys and values
    into cache slots 0..T-1), final norm and head -> logits [B, T, vocab]."""
    tokens = np.asarray(tokens, dtype=np.int64)
    B, T = tokens.shape
    x = f64(emb)[tokens.reshape(-1)]
    d = x.shape[1]
    hd = d // n_heads
    for l in range(n_layers):
        w, kc, vc = get_layer(l)
        y, parts = block_forward(x, w, B, T, n_heads, eps, theta, return_parts=True)
        n_kv = parts["k"].shape[1] // hd
        kc[:, :, :T, :] = parts["k"].reshape(B, T, n_kv, hd).transpose(0, 2, 1, 3)
        vc[:, :, :T, :] = parts["v"].reshape(B, T, n_kv, hd).transpose(0, 2, 1, 3)
        x = y
    return head(x, final_norm, output, eps).reshape(B, T, -1)


def greedy_generate(prompt, n_new: int, emb, get_layer: LayerFn, n_layers: int, final_norm, output,
                    n_heads: int, eps: float, theta: float = 10000.0, forced=None):
    """Greedy generation: prefill the prompt [B, T], then n_new tokens, each the
    index of the largest logit of the previous step (the first index among
    equal maxima, as numpy.argmax gives), fed back through one decode step at
    the next position. Returns (tokens [B, n_new], logits [n_new, B, vocab]).

    `forced` [B, n_new], when given, is fed back instead of the chosen tokens
    (to follow another implementation's choices and compare logits step by
    step). The caches of `get_layer` start empty and are filled in place."""
    prompt = np.asarray(prompt, dtype=np.int64)
    B, T = prompt.shape
    logits = model_forward(prompt, emb, get_layer, n_layers, final_norm, output, n_heads, eps, theta)[:, -1]
    toks, steps = [], []
    for i in range(n_new):
        steps.append(logits)
        tok = np.argmax(logits, axis=-1)
        toks.append(tok)
        if i + 1 == n_new:
            break
        feed = tok if forced is None else np.asarray(forced, dtype=np.int64)[:, i]
        pos = np.full(B, T + i, dtype=np.int64)
        logits = model_decode(feed, pos, emb, get_layer, n_layers, final_norm, output, n_heads, eps, theta)
    return np.stack(toks, axis=1), np.stack(steps)

