"""llama_model_decode_static: the decode step with its scratch in the
library's own device array (no workspace argument, no allocation), against
llama_model_decode with a caller workspace. Same kernels, same launch
sequence, so logits and cache writes must be bitwise equal; two calls in a
row, the second with a smaller batch, so a stale array from the first call
would show."""
import ctypes

import pytest
import torch

from decoder_only_transformer_llama_amd import _lib as L
from decoder_only_transformer_llama_amd import inputs as I

pytestmark = pytest.mark.gpu


def _model(wid):
    from decoder_only_transformer_llama_amd import ops
    w = I.workload(wid)
    layers = [I.block_weights(w, l, device="cuda") for l in range(w.n_layers)]
    gl = I.model_globals(w, device="cuda")
    cfg = ops.config(w.dim, w.n_heads, w.hidden, dtype=w.torch_dtype, n_layers=w.n_layers, vocab=w.vocab,
                     max_seq=w.max_seq, eps=w.eps, theta=w.theta, n_kv_heads=w.n_kv_heads)
    return w, ops.Model(cfg, layers, gl["tok_embeddings"], gl["final_norm"], gl["output"])


def _static_decode(m, tokens, pos, kc, vc, logits):
    st = L.load().llama_model_decode_static(ctypes.byref(m.cfg), ctypes.byref(m.wstruct), tokens.data_ptr(),
                                            pos.data_ptr(), tokens.shape[0], kc.data_ptr(), vc.data_ptr(),
                                            logits.data_ptr(), torch.cuda.current_stream().cuda_stream)
    L.check(st, "llama_model_decode_static")


@pytest.mark.parametrize("wid", [105, 108])
def test_decode_static_scratch_equals_workspace_decode(wid):
    w, m = _model(wid)
    for call, (B, T) in enumerate(((w.batch, 20), (max(1, w.batch - 1), 9))):
        toks = I.tokens(w, (B, T + 1), device="cuda", stream=call)
        kc, vc = m.new_cache(B, "cuda"), m.new_cache(B, "cuda")
        m.forward(toks[:, :T].contiguous(), kc, vc)
        kc2, vc2 = kc.clone(), vc.clone()
        pos = torch.tensor([T - i % 3 for i in range(B)], dtype=torch.int32, device="cuda")
        tok = toks[:, T].contiguous()
        ref = m.decode(tok, pos, kc, vc).clone()
        got = torch.full_like(ref, float("nan"))
        _static_decode(m, tok, pos, kc2, vc2, got)
        torch.cuda.synchronize()
        assert torch.isfinite(ref).all()
        assert torch.equal(got, ref), (wid, call, B)
        assert torch.equal(kc, kc2) and torch.equal(vc, vc2), (wid, call, B)
        print(f"{w.name}: call {call} (batch {B}, {T} cached tokens) static-scratch decode bitwise equal")


def test_decode_static_rejects_oversized_step():
    """A step whose scratch exceeds the array is refused before any launch."""
    w, m = _model(105)
    from decoder_only_transformer_llama_amd import ops
    c = m.cfg
    big = ops.config(c.dim, c.n_heads, c.hidden, n_layers=c.n_layers, vocab=400000, max_seq=c.max_seq,
                     n_kv_heads=c.n_kv_heads)
    assert ops.workspace_bytes(big, L.OP_MODEL_DECODE, 32, 1) > (64 << 20)
    fake = 0x1000
    st = L.load().llama_model_decode_static(ctypes.byref(big), ctypes.byref(m.wstruct), fake, fake, 32, fake, fake,
                                            fake, None)
    assert st == L.LLAMA_ERR_WORKSPACE
    assert b"static scratch" in L.load().llama_last_error()
