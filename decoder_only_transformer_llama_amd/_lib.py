"""ctypes binding of libllama_mi355x.so (declared in include/llama_mi355x.h).

Argument marshalling only: every computation runs inside the library's HIP
kernels. Loading fails loudly when the library has not been built; there is no
other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# LLAMA_MI355X_LIB may point at another build of the same library (A/B timing).
LIB_PATH = os.environ.get("LLAMA_MI355X_LIB") or os.path.join(HERE, "libllama_mi355x.so")

LLAMA_F32, LLAMA_BF16 = 0, 1
LLAMA_OK = 0
LLAMA_ERR_NULL, LLAMA_ERR_SHAPE, LLAMA_ERR_DTYPE, LLAMA_ERR_WORKSPACE = -1, -2, -3, -4
LLAMA_ERR_POSITION, LLAMA_ERR_UNSUPPORTED, LLAMA_ERR_HIP = -5, -6, -7
OP_CAUSAL_ATTN, OP_SWIGLU_FFN, OP_BLOCK_FORWARD, OP_MODEL_FORWARD, OP_MODEL_DECODE = 1, 2, 3, 4, 5
OP_CAUSAL_ATTN_BACKWARD, OP_BLOCK_BACKWARD = 6, 7

NUM_DEFAULT = 0
NUM_EXPLICIT = 1 << 31
NUM_QKV_A_PAIR, NUM_QK_PAIR, NUM_V_PAIR = 1 << 0, 1 << 1, 1 << 2
NUM_O_A_PAIR, NUM_FFN_A_PAIR, NUM_DOWN_A_PAIR = 1 << 3, 1 << 4, 1 << 5
NUM_ATTN_F16 = 1 << 6
NUM_QKV_A_F16, NUM_O_A_F16, NUM_FFN_A_F16, NUM_DOWN_A_F16 = 1 << 7, 1 << 8, 1 << 9, 1 << 10
NUM_GEMM_F16 = NUM_QKV_A_F16 | NUM_O_A_F16 | NUM_FFN_A_F16 | NUM_DOWN_A_F16
NUM_W_F16 = 1 << 11
NORM_PRE, NORM_POST, NORM_NONE = 0, 1, 2

EXPORTS = (
    "llama_hidden_dim", "llama_rmsnorm", "llama_rope", "llama_linear", "llama_causal_attn",
    "llama_swiglu_ffn", "llama_block_forward", "llama_model_forward", "llama_model_decode",
    "llama_workspace_size", "llama_status_string", "llama_last_error", "llama_trace_begin", "llama_trace_end",
    "llama_trace_label", "llama_argmax", "llama_decode_pack_size", "llama_pack_decode_weights",
    "llama_causal_attn_backward", "llama_block_train_saved_size", "llama_block_train_forward",
    "llama_block_backward", "llama_axpby", "llama_convert_weights_f16", "llama_model_decode_static",
    "llama_decode_pack_max_read",
)


class LlamaConfig(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("vocab", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("numerics", ctypes.c_uint32), ("n_kv_heads", ctypes.c_int32), ("norm_placement", ctypes.c_int32)]


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")]


class ModelWeights(ctypes.Structure):
    _fields_ = [("tok_embeddings", ctypes.c_void_p), ("layers", ctypes.POINTER(BlockWeights)),
                ("final_norm", ctypes.c_void_p), ("output", ctypes.c_void_p), ("decode_pack", ctypes.c_void_p)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m decoder_only_transformer_llama_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    cfgp = ctypes.POINTER(LlamaConfig)
    sig = {
        "llama_hidden_dim": [i32, i32],
        "llama_rmsnorm": [i32, i32, vp, vp, vp, i64, i32, f32, vp],
        "llama_rope": [i32, vp, vp, vp, i64, i32, i32, f32, vp],
        "llama_linear": [i32, i32, i32, vp, vp, vp, i64, i32, i32, vp],
        "llama_causal_attn": [i32, i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, sz, vp],
        "llama_swiglu_ffn": [i32, i32, vp, vp, vp, vp, vp, i64, i32, i32, vp, sz, vp],
        "llama_block_forward": [cfgp, ctypes.POINTER(BlockWeights), i32, vp, vp, i32, i32, vp, sz, vp],
        "llama_model_forward": [cfgp, ctypes.POINTER(ModelWeights), vp, vp, i32, i32, vp, vp, vp, vp, sz, vp],
        "llama_model_decode": [cfgp, ctypes.POINTER(ModelWeights), vp, vp, i32, vp, vp, vp, vp, sz, vp],
        "llama_workspace_size": [cfgp, i32, i32, i32, ctypes.POINTER(sz)],
        "llama_status_string": [i32],
        "llama_last_error": [],
        "llama_trace_begin": [ctypes.POINTER(vp), i32],
        "llama_trace_end": [],
        "llama_trace_label": [i32],
        "llama_argmax": [vp, i64, i32, vp, vp],
        "llama_decode_pack_size": [cfgp, ctypes.POINTER(sz)],
        "llama_pack_decode_weights": [cfgp, ctypes.POINTER(ModelWeights), vp, sz, vp],
        "llama_causal_attn_backward": [i32, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, sz, vp],
        "llama_block_train_saved_size": [cfgp, i32, i32, ctypes.POINTER(sz)],
        "llama_block_train_forward": [cfgp, ctypes.POINTER(BlockWeights), vp, vp, vp, sz, i32, i32, vp, sz, vp],
        "llama_block_backward": [cfgp, ctypes.POINTER(BlockWeights), vp, vp, sz, vp, vp, ctypes.POINTER(BlockWeights),
                                 i32, i32, vp, sz, vp],
        "llama_axpby": [vp, vp, vp, f32, f32, i64, vp],
        "llama_convert_weights_f16": [vp, vp, i64, vp],
        "llama_model_decode_static": [cfgp, ctypes.POINTER(ModelWeights), vp, vp, i32, vp, vp, vp, vp],
        "llama_decode_pack_max_read": [cfgp, ctypes.POINTER(sz)],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = (ctypes.c_char_p if name in ("llama_status_string", "llama_last_error", "llama_trace_label")
                      else ctypes.c_int)
    _lib = lib
    return lib


class LlamaError(RuntimeError):
    def __init__(self, status: int, what: str):
        lib = load()
        msg = lib.llama_status_string(status).decode()
        if status == LLAMA_ERR_HIP:
            msg += ": " + lib.llama_last_error().decode()
        super().__init__(f"{what}: {msg} (status {status})")
        self.status = status


def check(status: int, what: str) -> None:
    if status != LLAMA_OK:
        raise LlamaError(status, what)
