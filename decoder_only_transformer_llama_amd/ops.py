"""Torch-facing wrappers over the C ABI: they check tensors, allocate outputs
and workspaces with torch (device memory only), pass raw pointers and the
current HIP stream, and raise on a non-OK status. Every computation happens in
libllama_mi355x.so's kernels.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional, Sequence

import torch

from . import _lib as L

_DT = {torch.float32: L.LLAMA_F32, torch.bfloat16: L.LLAMA_BF16}
_TORCH = {L.LLAMA_F32: torch.float32, L.LLAMA_BF16: torch.bfloat16}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _need(t: torch.Tensor, name: str, shape, dtype) -> None:
    """Shape and dtype check before any launch: a wrong size would make the
    kernels read or write outside the tensor, a wrong dtype reinterpret it."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def config(dim: int, n_heads: int, hidden: int, *, dtype: torch.dtype = torch.bfloat16, n_layers: int = 1,
           vocab: int = 0, max_seq: int = 0, eps: float = 1e-6, theta: float = 10000.0,
           numerics: int = L.NUM_DEFAULT, n_kv_heads: int = 0,
           norm_placement: int = L.NORM_PRE) -> L.LlamaConfig:
    return L.LlamaConfig(dim, n_heads, hidden, n_layers, vocab, max_seq, eps, theta, _DT[dtype], numerics,
                         n_kv_heads, norm_placement)


def workspace_bytes(cfg: L.LlamaConfig, op: int, batch: int, seq: int) -> int:
    lib = L.load()
    n = ctypes.c_size_t(0)
    L.check(lib.llama_workspace_size(ctypes.byref(cfg), op, batch, seq, ctypes.byref(n)),
            "llama_workspace_size")
    return n.value


def hidden_dim(dim: int, multiple_of: int = 256) -> int:
    return L.load().llama_hidden_dim(dim, multiple_of)


def rmsnorm(x: torch.Tensor, g: Optional[torch.Tensor], eps: float,
            out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    _dev(x, g)
    dim = x.shape[-1]
    y = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    if g is not None and g.dtype != x.dtype:
        raise TypeError("gain dtype must match x")
    L.check(L.load().llama_rmsnorm(_dt(x), _dt(y), _p(x), _p(g), _p(y), x.numel() // dim, dim, eps, _stream()),
            "llama_rmsnorm")
    return y


def rope(x: torch.Tensor, positions: torch.Tensor, n_heads: int, theta: float = 10000.0,
         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _dev(x, positions)
    if positions.dtype != torch.int32:
        raise TypeError("positions must be int32")
    tokens = x.shape[0]
    head_dim = x.shape[-1] // n_heads
    y = torch.empty_like(x) if out is None else out
    L.check(L.load().llama_rope(_dt(x), _p(x), _p(y), _p(positions), tokens, n_heads, head_dim, theta,
                                _stream()), "llama_rope")
    return y


def linear(x: torch.Tensor, w: torch.Tensor, out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    _dev(x, w)
    rows, k = x.shape
    n = w.shape[0]
    y = torch.empty((rows, n), dtype=out_dtype, device=x.device)
    L.check(L.load().llama_linear(_dt(x), _dt(w), _DT[out_dtype], _p(x), _p(w), _p(y), rows, n, k, _stream()),
            "llama_linear")
    return y


def causal_attn(q, k, v, batch: int, seq: int, n_heads: int,
                out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    _dev(q, k, v)
    d = q.shape[-1]
    hd = d // n_heads
    o = torch.empty((batch * seq, d), dtype=out_dtype, device=q.device)
    cfg = config(d, n_heads, 1, dtype=q.dtype)
    ws = _ws(workspace_bytes(cfg, L.OP_CAUSAL_ATTN, batch, seq), q.device)
    L.check(L.load().llama_causal_attn(_dt(q), _DT[out_dtype], _p(q), _p(k), _p(v), _p(o), batch, seq, n_heads,
                                       hd, _p(ws), ws.numel(), _stream()), "llama_causal_attn")
    return o


def causal_attn_backward(q, k, v, dout, batch: int, seq: int, n_heads: int):
    """(dq, dk, dv) of causal_attn for the output gradient dout (fp32)."""
    _dev(q, k, v, dout)
    d = q.shape[-1]
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    cfg = config(d, n_heads, 1, dtype=q.dtype)
    ws = _ws(workspace_bytes(cfg, L.OP_CAUSAL_ATTN_BACKWARD, batch, seq), q.device)
    L.check(L.load().llama_causal_attn_backward(_dt(q), _p(q), _p(k), _p(v), _p(dout), _p(dq), _p(dk), _p(dv), batch,
                                                seq, n_heads, d // n_heads, _p(ws), ws.numel(), _stream()),
            "llama_causal_attn_backward")
    return dq, dk, dv


def swiglu_ffn(z, w_gate, w_up, w_down, out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    _dev(z, w_gate, w_up, w_down)
    tokens, dim = z.shape
    hidden = w_gate.shape[0]
    y = torch.empty((tokens, dim), dtype=out_dtype, device=z.device)
    cfg = config(dim, 1, hidden, dtype=z.dtype)
    ws = _ws(workspace_bytes(cfg, L.OP_SWIGLU_FFN, tokens, 1), z.device)
    L.check(L.load().llama_swiglu_ffn(_dt(z), _DT[out_dtype], _p(z), _p(w_gate), _p(w_up), _p(w_down), _p(y),
                                      tokens, dim, hidden, _p(ws), ws.numel(), _stream()), "llama_swiglu_ffn")
    return y


def argmax(logits: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Greedy token per row of logits [..., vocab] (lowest index on ties, -1 for a NaN row)."""
    _dev(logits)
    if logits.dtype != torch.float32:
        raise TypeError("logits must be float32")
    vocab = logits.shape[-1]
    rows = logits.numel() // vocab
    if out is None:
        out = torch.empty(logits.shape[:-1], dtype=torch.int32, device=logits.device)
    L.check(L.load().llama_argmax(_p(logits), rows, vocab, _p(out), _stream()), "llama_argmax")
    return out


BLOCK_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


def block_weights_struct(w: Dict[str, torch.Tensor]) -> L.BlockWeights:
    _dev(*[w[k] for k in BLOCK_KEYS])
    return L.BlockWeights(*[w[k].data_ptr() for k in BLOCK_KEYS])


class Block:
    """A block's weights and config with a reusable workspace (no allocation per call)."""

    def __init__(self, cfg: L.LlamaConfig, weights: Dict[str, torch.Tensor], batch: int, seq: int):
        self.cfg, self.weights, self.batch, self.seq = cfg, weights, batch, seq
        self.wstruct = block_weights_struct(weights)
        dev = weights["wq"].device
        self.ws = _ws(workspace_bytes(cfg, L.OP_BLOCK_FORWARD, batch, seq), dev)
        self.y = torch.empty((batch * seq, cfg.dim), dtype=torch.float32, device=dev)

    def __call__(self, x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
        y = self.y if y is None else y
        _dev(x, y)
        n, dim = self.batch * self.seq, self.cfg.dim
        if x.dtype not in (torch.float32, _TORCH[self.cfg.dtype]):
            raise TypeError(f"x must be float32 or {_TORCH[self.cfg.dtype]}, got {x.dtype}")
        _need(x, "x", (n, dim), x.dtype)
        _need(y, "y", (n, dim), torch.float32)
        L.check(L.load().llama_block_forward(ctypes.byref(self.cfg), ctypes.byref(self.wstruct), _dt(x), _p(x),
                                             _p(y), self.batch, self.seq, _p(self.ws), self.ws.numel(), _stream()),
                "llama_block_forward")
        return y


def convert_weights_f16(w: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """IEEE fp16 copy of a bf16 weight tensor (out may be w itself, viewed as
    fp16 afterwards), by the library's load-time conversion: the one its fp16
    matrix-core products otherwise apply to bf16 weights in registers."""
    _dev(w)
    if w.dtype != torch.bfloat16:
        raise TypeError("convert_weights_f16 takes a bf16 tensor")
    if out is None:
        out = torch.empty(w.shape, dtype=torch.float16, device=w.device)
    _dev(out)
    if out.numel() != w.numel() or out.element_size() != 2:
        raise ValueError("out must hold as many 16-bit values as w")
    L.check(L.load().llama_convert_weights_f16(_p(w), _p(out), w.numel(), _stream()), "llama_convert_weights_f16")
    return out


# Projections whose weights LLAMA_NUM_W_F16 supplies as fp16, by the operand bit that selects each.
_W_F16_OF = ((L.NUM_QKV_A_F16, ("wq", "wk", "wv")), (L.NUM_O_A_F16, ("wo",)),
             (L.NUM_FFN_A_F16, ("w_gate", "w_up")), (L.NUM_DOWN_A_F16, ("w_down",)))
_NUM_DEFAULT_SET = L.NUM_ATTN_F16 | L.NUM_QKV_A_F16 | L.NUM_O_A_F16 | L.NUM_FFN_A_F16


def with_f16_weights(numerics: int, weights: Dict[str, torch.Tensor]):
    """(numerics | NUM_W_F16, weights) for a bf16 block: the projections whose
    activation operand `numerics` makes fp16 are replaced by fp16 copies; the
    rest (gains, bf16-operand projections) are the same tensors."""
    num = numerics if numerics & L.NUM_EXPLICIT else _NUM_DEFAULT_SET
    out = dict(weights)
    for bit, keys in _W_F16_OF:
        if num & bit:
            for k in keys:
                out[k] = convert_weights_f16(weights[k])
    return numerics | L.NUM_W_F16, out


def axpby(z: torch.Tensor, x: torch.Tensor, y: torch.Tensor, a: float, b: float) -> torch.Tensor:
    """z = a x + b y over fp32 tensors of one size (z may be x or y)."""
    _dev(z, x, y)
    L.check(L.load().llama_axpby(_p(z), _p(x), _p(y), a, b, z.numel(), _stream()), "llama_axpby")
    return z


class TrainBlock:
    """An fp32 block for training: forward keeping the linear outputs,
    manual backward into gradient buffers, and an SGD step, all in the
    library's kernels. Weights are updated in place."""

    def __init__(self, cfg: L.LlamaConfig, weights: Dict[str, torch.Tensor], batch: int, seq: int):
        self.cfg, self.weights, self.batch, self.seq = cfg, weights, batch, seq
        dev = weights["wq"].device
        self.wstruct = block_weights_struct(weights)
        self.grads = {k: torch.zeros_like(weights[k]) for k in BLOCK_KEYS}
        self.gstruct = block_weights_struct(self.grads)
        n = ctypes.c_size_t(0)
        L.check(L.load().llama_block_train_saved_size(ctypes.byref(cfg), batch, seq, ctypes.byref(n)),
                "llama_block_train_saved_size")
        self.saved = _ws(n.value, dev)
        self.ws = _ws(workspace_bytes(cfg, L.OP_BLOCK_BACKWARD, batch, seq), dev)
        self.y = torch.empty((batch * seq, cfg.dim), dtype=torch.float32, device=dev)
        self.dx = torch.empty_like(self.y)
        self.dy = torch.empty_like(self.y)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        _dev(x)
        L.check(L.load().llama_block_train_forward(ctypes.byref(self.cfg), ctypes.byref(self.wstruct), _p(x), _p(self.y),
                                                   _p(self.saved), self.saved.numel(), self.batch, self.seq,
                                                   _p(self.ws), self.ws.numel(), _stream()),
                "llama_block_train_forward")
        return self.y

    def backward(self, x: torch.Tensor, dy: torch.Tensor) -> torch.Tensor:
        """dx for the upstream gradient dy; weight gradients land in self.grads."""
        _dev(x, dy)
        L.check(L.load().llama_block_backward(ctypes.byref(self.cfg), ctypes.byref(self.wstruct), _p(x), _p(self.saved),
                                              self.saved.numel(), _p(dy), _p(self.dx), ctypes.byref(self.gstruct),
                                              self.batch, self.seq, _p(self.ws), self.ws.numel(), _stream()),
                "llama_block_backward")
        return self.dx

    def train_step(self, x: torch.Tensor, target: torch.Tensor, lr: float) -> torch.Tensor:
        """One SGD step on the loss 0.5 * ||y - target||^2: forward, dL/dy = y -
        target, backward, w <- w - lr * dL/dw. Returns y before the update."""
        y = self.forward(x)
        axpby(self.dy, y, target, 1.0, -1.0)
        self.backward(x, self.dy)
        for k in BLOCK_KEYS:
            axpby(self.weights[k], self.weights[k], self.grads[k], 1.0, -lr)
        return y


def block_forward(cfg: L.LlamaConfig, weights: Dict[str, torch.Tensor], x: torch.Tensor, batch: int,
                  seq: int) -> torch.Tensor:
    return Block(cfg, weights, batch, seq)(x).clone()


class Model:
    """Whole-model weights (device tensors) plus the host-side layer table."""

    def __init__(self, cfg: L.LlamaConfig, layers: Sequence[Dict[str, torch.Tensor]],
                 tok_embeddings: torch.Tensor, final_norm: torch.Tensor, output: torch.Tensor):
        self.cfg = cfg
        self.layers = list(layers)
        self.tensors = (tok_embeddings, final_norm, output)
        arr = (L.BlockWeights * len(self.layers))(*[block_weights_struct(w) for w in self.layers])
        self._arr = arr
        _dev(tok_embeddings, final_norm, output)
        self.wstruct = L.ModelWeights(tok_embeddings.data_ptr(), ctypes.cast(arr, ctypes.POINTER(L.BlockWeights)),
                                      final_norm.data_ptr(), output.data_ptr(), None)
        self._ws = {}
        self.decode_pack = None

    def pack_for_decode(self) -> torch.Tensor:
        """Repack the projections into matrix-core tile order for decode (a
        load-time copy of the weights); later decode calls stream from it."""
        lib = L.load()
        n = ctypes.c_size_t(0)
        L.check(lib.llama_decode_pack_size(ctypes.byref(self.cfg), ctypes.byref(n)), "llama_decode_pack_size")
        pack = torch.empty(n.value, dtype=torch.uint8, device=self.tensors[0].device)
        L.check(lib.llama_pack_decode_weights(ctypes.byref(self.cfg), ctypes.byref(self.wstruct), _p(pack),
                                              pack.numel(), _stream()), "llama_pack_decode_weights")
        self.decode_pack = pack
        self.wstruct.decode_pack = pack.data_ptr()
        return pack

    def workspace(self, op: int, batch: int, seq: int, device) -> torch.Tensor:
        key = (op, batch, seq)
        if key not in self._ws:
            self._ws[key] = _ws(workspace_bytes(self.cfg, op, batch, seq), device)
        return self._ws[key]

    def new_cache(self, batch: int, device) -> torch.Tensor:
        return torch.zeros(self.cache_shape(batch), dtype=_TORCH[self.cfg.dtype], device=device)

    def cache_shape(self, batch: int):
        c = self.cfg
        return (c.n_layers, batch, c.n_kv_heads or c.n_heads, c.max_seq, c.dim // c.n_heads)

    def _check_caches(self, batch: int, k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
        for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
            _need(t, name, self.cache_shape(batch), _TORCH[self.cfg.dtype])

    def forward(self, tokens: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                start_pos: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Prefill tokens [B, T] (int32). start_pos (int32 [B]): the sequences
        continue cached prefixes of those lengths (None: all start at 0)."""
        _dev(tokens, k_cache, v_cache, start_pos, logits)
        if tokens.dim() != 2:
            raise ValueError("tokens must be [batch, seq]")
        B, T = tokens.shape
        _need(tokens, "tokens", (B, T), torch.int32)
        if T > self.cfg.max_seq:
            raise ValueError(f"seq {T} exceeds max_seq {self.cfg.max_seq}")
        if start_pos is not None:
            _need(start_pos, "start_pos", (B,), torch.int32)
        self._check_caches(B, k_cache, v_cache)
        if logits is None:
            logits = torch.empty((B, T, self.cfg.vocab), dtype=torch.float32, device=tokens.device)
        _need(logits, "logits", (B, T, self.cfg.vocab), torch.float32)
        ws = self.workspace(L.OP_MODEL_FORWARD, B, T, tokens.device)
        L.check(L.load().llama_model_forward(ctypes.byref(self.cfg), ctypes.byref(self.wstruct), _p(tokens),
                                             _p(start_pos), B, T, _p(k_cache), _p(v_cache), _p(logits), _p(ws),
                                             ws.numel(), _stream()),
                "llama_model_forward")
        return logits

    def generate(self, prompt: torch.Tensor, n_new: int, k_cache: torch.Tensor,
                 v_cache: torch.Tensor) -> torch.Tensor:
        """Greedy generation: prefill prompt [B, T] (int32) from an empty
        cache, then n_new tokens, each the argmax of the previous step's
        logits and fed back through one decode step. Returns [B, n_new] int32.
        Every step runs on the GPU; the host only enqueues."""
        _dev(prompt, k_cache, v_cache)
        B, T = prompt.shape
        if T + n_new - 1 > self.cfg.max_seq:
            raise ValueError("prompt plus generated tokens exceed max_seq")
        out = torch.empty((B, n_new), dtype=torch.int32, device=prompt.device)
        if n_new == 0:
            return out
        logits = self.forward(prompt, k_cache, v_cache)
        tok = argmax(logits[:, -1].contiguous())
        out[:, 0] = tok
        step_logits = torch.empty((B, self.cfg.vocab), dtype=torch.float32, device=prompt.device)
        for i in range(1, n_new):
            pos = torch.full((B,), T + i - 1, dtype=torch.int32, device=prompt.device)
            self.decode(tok, pos, k_cache, v_cache, step_logits)
            tok = argmax(step_logits)
            out[:, i] = tok
        return out

    def decode(self, tokens: torch.Tensor, pos: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
               logits: Optional[torch.Tensor] = None) -> torch.Tensor:
        _dev(tokens, pos, k_cache, v_cache, logits)
        if tokens.dim() != 1:
            raise ValueError("tokens must be [batch]")
        B = tokens.shape[0]
        _need(tokens, "tokens", (B,), torch.int32)
        _need(pos, "pos", (B,), torch.int32)
        self._check_caches(B, k_cache, v_cache)
        if logits is None:
            logits = torch.empty((B, self.cfg.vocab), dtype=torch.float32, device=tokens.device)
        _need(logits, "logits", (B, self.cfg.vocab), torch.float32)
        ws = self.workspace(L.OP_MODEL_DECODE, B, 1, tokens.device)
        L.check(L.load().llama_model_decode(ctypes.byref(self.cfg), ctypes.byref(self.wstruct), _p(tokens), _p(pos),
                                            B, _p(k_cache), _p(v_cache), _p(logits), _p(ws), ws.numel(), _stream()),
                "llama_model_decode")
        return logits
