"""Plausible mistakes planted in (copies of) the oracle, on the CPU, must be
caught by the pins: this checks that the pins have teeth."""
import math

import numpy as np
import pytest

from oracle import llama_oracle as O
from tests import brute_force as BF
from tests.test_oracle_pins import _rand, _tiny_block

_rope, _attn, _attn_bwd = O.rope, O.causal_attention, O.causal_attention_backward


def rope_wrong_sign(x, positions, head_dim, theta=10000.0):
    return _rope(x, -np.asarray(positions, float), head_dim, theta)


def rope_half_split(x, positions, head_dim, theta=10000.0):
    # rotate (i, i + hd/2) pairs instead of the interleaved (2i, 2i+1) pairs
    t, w = x.shape
    perm = np.concatenate([np.arange(0, head_dim, 2), np.arange(1, head_dim, 2)])
    inv = np.argsort(perm)
    xp = x.reshape(t, -1, head_dim)[..., inv].reshape(t, w)
    return _rope(xp, positions, head_dim, theta).reshape(t, -1, head_dim)[..., perm].reshape(t, w)


def rope_full_width_freq(x, positions, head_dim, theta=10000.0):
    # frequencies over the whole model width instead of per head
    return _rope(x, positions, x.shape[1], theta)


def attn_no_scale(q, k, v, batch, seq, n_heads):
    hd = q.shape[1] // n_heads
    return _attn(np.asarray(q) * math.sqrt(hd), k, v, batch, seq, n_heads)


def attn_strict_mask(q, k, v, batch, seq, n_heads):
    out = _attn(q, k, v, batch, seq, n_heads)
    # excludes the diagonal: query i sees keys < i (row 0 falls back to key 0)
    res = np.array(out)
    for b in range(batch):
        for i in range(1, seq):
            qq = np.asarray(q)[b * seq:(b + 1) * seq]
            kk = np.asarray(k)[b * seq:(b + 1) * seq].copy()
            vv = np.asarray(v)[b * seq:(b + 1) * seq].copy()
            kk[i] = kk[i - 1]
            vv[i] = vv[i - 1]
            sub = _attn(qq[:i + 1], kk[:i + 1], vv[:i + 1], 1, i + 1, n_heads)
            res[b * seq + i] = sub[i]
    return res


def rmsnorm_eps_outside(x, g, eps):
    x = np.asarray(x, float)
    y = x / (np.sqrt((x * x).mean(axis=-1, keepdims=True)) + eps)
    return y if g is None else y * g


def _block_case():
    B, S, d, H = 1, 5, 16, 2
    w = _tiny_block(50, d, H)
    x = _rand((B * S, d), 51)
    want = np.array(BF.block(x.tolist(), {k: v.tolist() for k, v in w.items()}, B, S, H, 1e-2, 1e4))
    return x, w, B, S, H, want


@pytest.mark.parametrize("name,patch", [
    ("rope", rope_wrong_sign), ("rope", rope_half_split), ("rope", rope_full_width_freq),
    ("causal_attention", attn_no_scale), ("causal_attention", attn_strict_mask),
    ("rmsnorm", rmsnorm_eps_outside),
])
def test_planted_mistake_is_caught_by_brute_force(monkeypatch, name, patch):
    x, w, B, S, H, want = _block_case()
    np.testing.assert_allclose(O.block_forward(x, w, B, S, H, 1e-2, 1e4), want, rtol=1e-10, atol=1e-11)
    monkeypatch.setattr(O, name, patch)
    got = O.block_forward(x, w, B, S, H, 1e-2, 1e4)
    assert np.max(np.abs(got - want)) > 1e-6, f"planted mistake in {name} not caught"


def test_planted_ffn_norm_on_trunk_input_is_caught(monkeypatch):
    x, w, B, S, H, want = _block_case()
    real = O.rmsnorm
    calls = []

    def first_arg_memory(xx, g, eps):
        calls.append(np.array(xx))
        # second call (FFN norm) wrongly normalises the block input x instead of h
        return real(calls[0] if len(calls) == 2 else xx, g, eps)

    monkeypatch.setattr(O, "rmsnorm", first_arg_memory)
    got = O.block_forward(x, w, B, S, H, 1e-2, 1e4)
    assert np.max(np.abs(got - want)) > 1e-6


def _post_norm_norm_before_add(x, w, batch, seq, n_heads, eps, theta=10000.0):
    # 2017 ordering read wrongly: normalise the branch output, then add
    h = x + O.rmsnorm(O.attn_sublayer(x, w, batch, seq, n_heads, theta), w["attn_norm"], eps)
    return h + O.rmsnorm(O.swiglu_ffn(h, w["w_gate"], w["w_up"], w["w_down"]), w["ffn_norm"], eps)


def _no_norm_keeps_ffn_norm(x, w, batch, seq, n_heads, eps=0.0, theta=10000.0):
    # only the first norm deleted
    h = x + O.attn_sublayer(x, w, batch, seq, n_heads, theta)
    return h + O.swiglu_ffn(O.rmsnorm(h, w["ffn_norm"], 1e-6), w["w_gate"], w["w_up"], w["w_down"])


@pytest.mark.parametrize("which,patch", [("post", _post_norm_norm_before_add), ("none", _no_norm_keeps_ffn_norm)])
def test_planted_norm_placement_mistake_is_caught(which, patch):
    B, S, d, H = 2, 4, 16, 2
    w = _tiny_block(52, d, H)
    x = _rand((B * S, d), 53)
    wl = {k: v.tolist() for k, v in w.items()}
    if which == "post":
        want = np.array(BF.post_norm_block(x.tolist(), wl, B, S, H, 1e-6, 1e4))
    else:
        want = np.array(BF.no_norm_block(x.tolist(), wl, B, S, H, 1e4))
    assert np.max(np.abs(patch(x, w, B, S, H, 1e-6, 1e4) - want)) > 1e-6


def _rmsnorm_backward_no_mean(x, g, eps, dy):
    x, dy = np.asarray(x, float), np.asarray(dy, float)
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return r * dy * g, (dy * x * r).sum(axis=0)


def _attention_backward_no_rowsum(q, k, v, do, batch, seq, n_heads):
    dq, dk, dv = _attn_bwd(q, k, v, do, batch, seq, n_heads)
    return dq * 1.01, dk, dv   # a slightly wrong softmax Jacobian, as a dropped term would give


@pytest.mark.parametrize("name,patch", [("rmsnorm_backward", _rmsnorm_backward_no_mean),
                                        ("causal_attention_backward", _attention_backward_no_rowsum)])
def test_planted_backward_mistake_is_caught_by_finite_differences(monkeypatch, name, patch):
    from tests.test_oracle_pins import _fd_grad
    B, S, d, H = 1, 4, 16, 2
    w = _tiny_block(54, d, H)
    x, dy = _rand((B * S, d), 55), _rand((B * S, d), 56)
    monkeypatch.setattr(O, name, patch)
    dx, _ = O.block_backward(x, w, dy, B, S, H, 1e-5)
    f = lambda: float(np.sum(O.block_forward(x, w, B, S, H, 1e-5) * dy))
    worst = max(abs(_fd_grad(f, x, (i, j)) - dx[i, j]) for i in range(B * S) for j in range(0, d, 3))
    assert worst > 1e-4 * np.max(np.abs(dx))
