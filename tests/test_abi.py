"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, the header compiles as C and C++, and host-side validation
returns its status codes before anything touches the device."""
import ctypes
import os
import re
import subprocess

import pytest

from decoder_only_transformer_llama_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llama_mi355x.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(llama_\w+)\s*\(", src, re.M)))


def test_header_declares_the_bound_entry_points():
    assert _declared() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = L.load()
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (llama_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


@pytest.mark.parametrize("lang,compiler", [("c", "gcc"), ("c++", "g++")])
def test_header_compiles(lang, compiler, tmp_path):
    src = tmp_path / ("t.c" if lang == "c" else "t.cpp")
    src.write_text('#include "llama_mi355x.h"\nint main(void){llama_config c; (void)c; return 0;}\n')
    r = subprocess.run([compiler, "-fsyntax-only", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_struct_layout_matches_header():
    assert ctypes.sizeof(L.LlamaConfig) == 48
    assert ctypes.sizeof(L.BlockWeights) == 9 * 8
    assert ctypes.sizeof(L.ModelWeights) == 5 * 8


def test_hidden_dim_and_status_strings():
    lib = L.load()
    for d, h in [(256, 768), (4096, 11008), (5120, 13824), (6656, 17920), (8192, 22016)]:
        assert lib.llama_hidden_dim(d, 256) == h
    assert lib.llama_hidden_dim(0, 256) == -1
    assert lib.llama_status_string(0) == b"ok"
    assert b"workspace" in lib.llama_status_string(L.LLAMA_ERR_WORKSPACE)
    assert lib.llama_last_error() == b""


def _cfg(**kw):
    base = dict(dim=4096, n_heads=32, hidden=11008, n_layers=32, vocab=32000, max_seq=2048, norm_eps=1e-6,
                rope_theta=1e4, dtype=L.LLAMA_BF16, numerics=0, n_kv_heads=0, norm_placement=0)
    base.update(kw)
    return L.LlamaConfig(*[base[k] for k, _ in L.LlamaConfig._fields_])


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def test_workspace_size_and_validation():
    lib = L.load()
    n = ctypes.c_size_t()
    c = _cfg()
    assert lib.llama_workspace_size(ctypes.byref(c), L.OP_BLOCK_FORWARD, 1, 2048, ctypes.byref(n)) == 0
    # q,k hi/lo, v^T hi/lo, attention out hi/lo (2 B each) + h f32 + u hi/lo + rope table
    assert n.value >= 2048 * 4096 * (2 * 8 + 4) + 2048 * 11008 * 4
    assert lib.llama_workspace_size(ctypes.byref(c), L.OP_MODEL_DECODE, 32, 1, ctypes.byref(n)) == 0
    n32 = n.value
    # more than 32 sequences run in chunks of 32 that reuse one chunk's workspace
    assert lib.llama_workspace_size(ctypes.byref(c), L.OP_MODEL_DECODE, 33, 1, ctypes.byref(n)) == 0
    assert n.value == n32
    # caches up to 16384 positions (more key ranges, more room for their states)
    assert lib.llama_workspace_size(ctypes.byref(_cfg(max_seq=4096)), L.OP_MODEL_DECODE, 4, 1, ctypes.byref(n)) == 0
    assert lib.llama_workspace_size(ctypes.byref(_cfg(max_seq=32768)), L.OP_MODEL_DECODE, 4, 1,
                                    ctypes.byref(n)) == L.LLAMA_ERR_UNSUPPORTED
    assert lib.llama_workspace_size(ctypes.byref(c), L.OP_MODEL_FORWARD, 1, 4096, ctypes.byref(n)) == \
        L.LLAMA_ERR_POSITION
    assert lib.llama_workspace_size(ctypes.byref(_cfg(dim=4001)), L.OP_BLOCK_FORWARD, 1, 8,
                                    ctypes.byref(n)) == L.LLAMA_ERR_SHAPE
    assert lib.llama_workspace_size(ctypes.byref(_cfg(n_heads=16)), L.OP_BLOCK_FORWARD, 1, 8,
                                    ctypes.byref(n)) == L.LLAMA_ERR_UNSUPPORTED      # head_dim 256
    assert lib.llama_workspace_size(ctypes.byref(_cfg(dtype=7)), L.OP_BLOCK_FORWARD, 1, 8,
                                    ctypes.byref(n)) == L.LLAMA_ERR_DTYPE
    assert lib.llama_workspace_size(None, L.OP_BLOCK_FORWARD, 1, 8, ctypes.byref(n)) == L.LLAMA_ERR_NULL


def test_entry_points_reject_bad_arguments_before_any_launch():
    lib = L.load()
    c = _cfg()
    w = L.BlockWeights(*([0x1000] * 9))
    assert lib.llama_rmsnorm(L.LLAMA_BF16, L.LLAMA_F32, None, None, FAKE, 4, 4096, 1e-6, None) == L.LLAMA_ERR_NULL
    assert lib.llama_rmsnorm(5, L.LLAMA_F32, FAKE, None, FAKE, 4, 4096, 1e-6, None) == L.LLAMA_ERR_DTYPE
    assert lib.llama_rmsnorm(L.LLAMA_F32, L.LLAMA_F32, FAKE, None, FAKE, -1, 4096, 1e-6, None) == L.LLAMA_ERR_SHAPE
    assert lib.llama_rope(L.LLAMA_F32, FAKE, FAKE, FAKE, 4, 2, 7, 1e4, None) == L.LLAMA_ERR_SHAPE   # odd head_dim
    assert lib.llama_linear(L.LLAMA_BF16, L.LLAMA_BF16, L.LLAMA_F32, FAKE, FAKE, FAKE, 4, 64, 100, None) == \
        L.LLAMA_ERR_SHAPE                                                                              # k % 64
    assert lib.llama_causal_attn(L.LLAMA_BF16, L.LLAMA_F32, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 96, FAKE, 1 << 30,
                                 None) == L.LLAMA_ERR_UNSUPPORTED
    assert lib.llama_causal_attn(L.LLAMA_BF16, L.LLAMA_F32, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, FAKE, 16,
                                 None) == L.LLAMA_ERR_WORKSPACE
    assert lib.llama_swiglu_ffn(L.LLAMA_BF16, L.LLAMA_F32, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 4096, 11000, FAKE,
                                1 << 40, None) == L.LLAMA_ERR_UNSUPPORTED
    assert lib.llama_block_forward(ctypes.byref(c), ctypes.byref(w), L.LLAMA_BF16, FAKE, FAKE, 1, 16, FAKE, 16,
                                   None) == L.LLAMA_ERR_WORKSPACE
    assert lib.llama_block_forward(ctypes.byref(c), None, L.LLAMA_BF16, FAKE, FAKE, 1, 16, FAKE, 1 << 40,
                                   None) == L.LLAMA_ERR_NULL
    wn = L.BlockWeights(*([0x1000] * 8 + [0]))
    assert lib.llama_block_forward(ctypes.byref(c), ctypes.byref(wn), L.LLAMA_BF16, FAKE, FAKE, 1, 16, FAKE,
                                   1 << 40, None) == L.LLAMA_ERR_NULL
    cf = _cfg(dtype=L.LLAMA_F32)
    assert lib.llama_block_forward(ctypes.byref(cf), ctypes.byref(w), L.LLAMA_BF16, FAKE, FAKE, 1, 16, FAKE,
                                   1 << 40, None) == L.LLAMA_ERR_DTYPE
    layers = (L.BlockWeights * 32)(*([w] * 32))
    mw = L.ModelWeights(0x1000, ctypes.cast(layers, ctypes.POINTER(L.BlockWeights)), 0x1000, 0x1000)
    assert lib.llama_model_forward(ctypes.byref(c), ctypes.byref(mw), FAKE, None, 1, 4096, FAKE, FAKE, FAKE, FAKE,
                                   1 << 40, None) == L.LLAMA_ERR_POSITION
    assert lib.llama_model_forward(ctypes.byref(c), ctypes.byref(mw), FAKE, FAKE, 1, 4096, FAKE, FAKE, FAKE, FAKE,
                                   1 << 40, None) == L.LLAMA_ERR_POSITION
    assert lib.llama_model_forward(ctypes.byref(cf), ctypes.byref(mw), FAKE, None, 1, 16, FAKE, FAKE, FAKE, FAKE,
                                   1 << 40, None) == L.LLAMA_ERR_UNSUPPORTED
    assert lib.llama_model_forward(ctypes.byref(c), ctypes.byref(mw), FAKE, FAKE, 1, 16, FAKE, FAKE, FAKE, FAKE,
                                   16, None) == L.LLAMA_ERR_WORKSPACE
    assert lib.llama_model_decode(ctypes.byref(_cfg(max_seq=32768)), ctypes.byref(mw), FAKE, FAKE, 4, FAKE, FAKE,
                                  FAKE, FAKE, 1 << 40, None) == L.LLAMA_ERR_UNSUPPORTED
    assert lib.llama_model_decode(ctypes.byref(c), ctypes.byref(mw), FAKE, FAKE, 33, FAKE, FAKE, FAKE, FAKE,
                                  16, None) == L.LLAMA_ERR_WORKSPACE
    assert lib.llama_model_decode(ctypes.byref(c), ctypes.byref(mw), FAKE, None, 4, FAKE, FAKE, FAKE, FAKE,
                                  1 << 40, None) == L.LLAMA_ERR_NULL
    assert lib.llama_model_decode(ctypes.byref(c), ctypes.byref(mw), FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE,
                                  16, None) == L.LLAMA_ERR_WORKSPACE
    n = ctypes.c_size_t()
    assert lib.llama_decode_pack_size(ctypes.byref(c), ctypes.byref(n)) == 0
    # 32 layers of (3d + d + 2h) x d + d x h, plus the head: exactly the weight bytes (all heights are multiples of 32)
    assert n.value == (32 * (4 * 4096 * 4096 + 3 * 4096 * 11008) + 32000 * 4096) * 2
    assert lib.llama_pack_decode_weights(ctypes.byref(c), ctypes.byref(mw), FAKE, 16, None) == L.LLAMA_ERR_WORKSPACE
    assert lib.llama_pack_decode_weights(ctypes.byref(cf), ctypes.byref(mw), FAKE, 1 << 40, None) == \
        L.LLAMA_ERR_UNSUPPORTED
    # fp16 prefill weights: the decode pack is built from bf16 weights, and a
    # decode step without a pack would read the projections as bf16
    cw = _cfg(numerics=L.NUM_W_F16)
    assert lib.llama_pack_decode_weights(ctypes.byref(cw), ctypes.byref(mw), FAKE, 1 << 40, None) == \
        L.LLAMA_ERR_UNSUPPORTED
    assert lib.llama_model_decode(ctypes.byref(cw), ctypes.byref(mw), FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE,
                                  1 << 40, None) == L.LLAMA_ERR_UNSUPPORTED
    assert lib.llama_convert_weights_f16(FAKE, FAKE, -1, None) == L.LLAMA_ERR_SHAPE
    assert lib.llama_convert_weights_f16(None, FAKE, 8, None) == L.LLAMA_ERR_NULL
    assert lib.llama_convert_weights_f16(None, None, 0, None) == 0                    # nothing to do
    assert lib.llama_convert_weights_f16(0x1000, 0x1008, 8, None) == L.LLAMA_ERR_SHAPE  # partial overlap


def test_grouped_kv_heads_validation_and_sizes():
    """n_kv_heads: 0 means n_heads; otherwise a divisor of n_heads with groups
    of 1, 2, 4 or 8 query heads per key/value head (bf16 only), and a key/value
    width that is a multiple of 128 columns."""
    lib = L.load()
    n = ctypes.c_size_t()

    def ws(**kw):
        return lib.llama_workspace_size(ctypes.byref(_cfg(**kw)), L.OP_BLOCK_FORWARD, 1, 64, ctypes.byref(n))

    assert ws(n_kv_heads=8) == 0 and ws(n_kv_heads=32) == 0 and ws(n_kv_heads=16) == 0
    assert ws(n_kv_heads=-1) == L.LLAMA_ERR_SHAPE
    assert ws(n_kv_heads=5) == L.LLAMA_ERR_SHAPE            # not a divisor of 32
    assert ws(n_kv_heads=64) == L.LLAMA_ERR_SHAPE           # more key/value heads than query heads
    assert ws(n_kv_heads=2) == L.LLAMA_ERR_UNSUPPORTED      # groups of 16
    assert ws(n_kv_heads=8, dtype=L.LLAMA_F32) == L.LLAMA_ERR_UNSUPPORTED
    assert ws(dim=512, n_heads=8, hidden=1536, n_kv_heads=1) == L.LLAMA_ERR_UNSUPPORTED   # width 64
    assert ws(dim=512, n_heads=8, hidden=1536, n_kv_heads=2) == 0                         # width 128
    # fp16 attention operands are single values: no q/k or v pairs alongside
    assert ws(numerics=L.NUM_EXPLICIT | L.NUM_ATTN_F16 | L.NUM_O_A_PAIR) == 0
    assert ws(numerics=L.NUM_EXPLICIT | L.NUM_ATTN_F16 | L.NUM_QK_PAIR) == L.LLAMA_ERR_UNSUPPORTED
    assert ws(numerics=L.NUM_EXPLICIT | L.NUM_ATTN_F16 | L.NUM_V_PAIR) == L.LLAMA_ERR_UNSUPPORTED
    # fp16 projection operands are single values as well
    assert ws(numerics=L.NUM_EXPLICIT | L.NUM_GEMM_F16) == 0
    assert ws(numerics=L.NUM_QK_PAIR) == L.LLAMA_ERR_UNSUPPORTED             # option bits need EXPLICIT
    assert ws(numerics=L.NUM_EXPLICIT | (1 << 12)) == L.LLAMA_ERR_UNSUPPORTED  # unknown bit
    # fp16 weights: alone (the default operand set) or among explicit bits
    assert ws(numerics=L.NUM_W_F16) == 0
    assert ws(numerics=L.NUM_EXPLICIT | L.NUM_GEMM_F16 | L.NUM_W_F16) == 0
    assert ws(numerics=L.NUM_W_F16 | L.NUM_ATTN_F16) == L.LLAMA_ERR_UNSUPPORTED
    for pair in (L.NUM_QKV_A_PAIR, L.NUM_O_A_PAIR, L.NUM_FFN_A_PAIR, L.NUM_DOWN_A_PAIR):
        assert ws(numerics=L.NUM_EXPLICIT | L.NUM_GEMM_F16 | pair) == L.LLAMA_ERR_UNSUPPORTED
    # fewer key/value heads shrink the packed decode weights by exactly the Wk, Wv rows
    for nkv in (32, 8):
        assert lib.llama_decode_pack_size(ctypes.byref(_cfg(n_kv_heads=nkv)), ctypes.byref(n)) == 0
        kvd = nkv * 128
        assert n.value == (32 * ((2 * 4096 + 2 * kvd) * 4096 + 3 * 4096 * 11008) + 32000 * 4096) * 2


def test_norm_placement_validation():
    """Blocks take pre-, post- or no-norm; the model entry points only pre-norm."""
    lib = L.load()
    n = ctypes.c_size_t()
    for placement, st in ((L.NORM_PRE, 0), (L.NORM_POST, 0), (L.NORM_NONE, 0), (3, L.LLAMA_ERR_UNSUPPORTED),
                          (-1, L.LLAMA_ERR_UNSUPPORTED)):
        c = _cfg(norm_placement=placement)
        assert lib.llama_workspace_size(ctypes.byref(c), L.OP_BLOCK_FORWARD, 1, 64, ctypes.byref(n)) == st
    for placement in (L.NORM_POST, L.NORM_NONE):
        c = _cfg(norm_placement=placement)
        assert lib.llama_workspace_size(ctypes.byref(c), L.OP_MODEL_FORWARD, 1, 64, ctypes.byref(n)) == \
            L.LLAMA_ERR_UNSUPPORTED
        assert lib.llama_workspace_size(ctypes.byref(c), L.OP_MODEL_DECODE, 4, 1, ctypes.byref(n)) == \
            L.LLAMA_ERR_UNSUPPORTED


def test_training_entry_points_validate_before_any_launch():
    lib = L.load()
    n = ctypes.c_size_t()
    f32 = dict(dim=256, n_heads=2, hidden=768, dtype=L.LLAMA_F32)
    c = _cfg(**f32)
    assert lib.llama_block_train_saved_size(ctypes.byref(c), 2, 37, ctypes.byref(n)) == 0
    # q, k, v, a, h [74, 256] + gate, up [74, 768] + lse [2, 2, 37], 256-byte aligned pieces (+256)
    pieces = [74 * 256 * 4] * 5 + [74 * 768 * 4] * 2 + [2 * 2 * 37 * 4]
    assert n.value == sum((p + 255) // 256 * 256 for p in pieces[:-1]) + pieces[-1] + 256
    assert lib.llama_workspace_size(ctypes.byref(c), L.OP_BLOCK_BACKWARD, 2, 37, ctypes.byref(n)) == 0
    for bad, st in ((dict(dtype=L.LLAMA_BF16), L.LLAMA_ERR_UNSUPPORTED),
                    (dict(norm_placement=L.NORM_POST), L.LLAMA_ERR_UNSUPPORTED),
                    (dict(n_kv_heads=1), L.LLAMA_ERR_UNSUPPORTED)):
        cb = _cfg(**{**f32, **bad})
        assert lib.llama_block_train_saved_size(ctypes.byref(cb), 2, 37, ctypes.byref(n)) == st
        assert lib.llama_workspace_size(ctypes.byref(cb), L.OP_BLOCK_BACKWARD, 2, 37, ctypes.byref(n)) == st
    w = L.BlockWeights(*([0x1000] * 9))
    assert lib.llama_block_train_forward(ctypes.byref(c), ctypes.byref(w), FAKE, FAKE, FAKE, 16, 2, 37, FAKE, 1 << 40,
                                         None) == L.LLAMA_ERR_WORKSPACE
    assert lib.llama_block_train_forward(ctypes.byref(c), ctypes.byref(w), None, FAKE, FAKE, 1 << 40, 2, 37, FAKE,
                                         1 << 40, None) == L.LLAMA_ERR_NULL
    gn = L.BlockWeights(*([0x1000] * 8 + [0]))
    assert lib.llama_block_backward(ctypes.byref(c), ctypes.byref(w), FAKE, FAKE, 1 << 40, FAKE, FAKE, ctypes.byref(gn),
                                    2, 37, FAKE, 1 << 40, None) == L.LLAMA_ERR_NULL
    assert lib.llama_block_backward(ctypes.byref(c), ctypes.byref(w), FAKE, FAKE, 1 << 40, FAKE, FAKE, ctypes.byref(w),
                                    2, 37, FAKE, 16, None) == L.LLAMA_ERR_WORKSPACE
    assert lib.llama_causal_attn_backward(L.LLAMA_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, FAKE,
                                          1 << 40, None) == L.LLAMA_ERR_UNSUPPORTED
    assert lib.llama_causal_attn_backward(L.LLAMA_F32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 96, FAKE,
                                          1 << 40, None) == L.LLAMA_ERR_UNSUPPORTED
    assert lib.llama_causal_attn_backward(L.LLAMA_F32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 64, FAKE,
                                          16, None) == L.LLAMA_ERR_WORKSPACE
    assert lib.llama_axpby(None, FAKE, FAKE, 1.0, 1.0, 4, None) == L.LLAMA_ERR_NULL
    assert lib.llama_axpby(FAKE, FAKE, FAKE, 1.0, 1.0, -1, None) == L.LLAMA_ERR_SHAPE


@pytest.mark.parametrize("wid", [4, 5, 101, 105, 106, 108])
def test_decode_pack_reads_stay_inside_the_pack(wid):
    """Every skinny-GEMM launch of a decode step reads the weight pack through
    its tile, split-K and block addressing; the furthest byte any launch reads
    (computed by the library from the launches' own addressing, host only)
    must be the pack's last byte: not past it (an out-of-bounds read), and
    not short of it (a part of the pack never streamed)."""
    import torch
    from decoder_only_transformer_llama_amd import inputs as I, ops
    w = I.workload(wid)
    cfg = ops.config(w.dim, w.n_heads, w.hidden, dtype=torch.bfloat16, n_layers=w.n_layers, vocab=w.vocab,
                     max_seq=w.max_seq, eps=w.eps, n_kv_heads=w.n_kv_heads)
    lib = L.load()
    size, end = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.llama_decode_pack_size(ctypes.byref(cfg), ctypes.byref(size)) == L.LLAMA_OK
    assert lib.llama_decode_pack_max_read(ctypes.byref(cfg), ctypes.byref(end)) == L.LLAMA_OK
    assert end.value == size.value, (end.value, size.value)


def test_build_rejects_kernels_that_spill_to_scratch():
    """The build parses hipcc's per-kernel resource report and names every
    kernel with scratch memory per lane (a spill); kernels without it pass."""
    from decoder_only_transformer_llama_amd import build as B
    log = "\n".join([
        "k.hip:1:1: remark: Function Name: _Z4goodv [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:9:1: remark: Function Name: _Z5spillv [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:9:1: remark:     VGPRs Spill: 1 [-Rpass-analysis=kernel-resource-usage]",
        "k.hip:9:1: remark:     ScratchSize [bytes/lane]: 8 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert B._scratch_kernels(log) == ["_Z5spillv (8 bytes/lane)"]
    assert B._scratch_kernels("\n".join(log.splitlines()[:2])) == []
    assert "-Rpass-analysis=kernel-resource-usage" in B.FLAGS
