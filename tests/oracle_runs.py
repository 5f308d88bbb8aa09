"""Oracle runs over device-resident seeded workloads: the inputs are copied to
the host (they come from the seeded generator, not from the library) and the
fp64 oracle recomputes selected outputs, streaming one layer at a time."""
import numpy as np
import torch

from decoder_only_transformer_llama_amd import inputs as I
from oracle import llama_oracle as O


def oracle_decode_rows(wl, rows):
    """Logits of the decode step for sequences `rows` of a DecodeWorkload.

    The cache slots 0..pos-1 are regenerated from the seeded generator on the
    workload's device for exactly these sequences; slot pos is written by the
    oracle itself."""
    w = wl.w
    rows = list(rows)
    toks = wl.tokens.cpu().numpy()[rows]
    pos = wl.pos.cpu().numpy()[rows]
    dev = wl.tokens.device

    def get_layer(l):
        wt = {k: O.f64(v.cpu()) for k, v in wl.layers[l].items()}
        kc, vc = I.kv_cache_layer(w, l, w.decode_pos, device=dev)
        idx = torch.tensor(rows, device=dev)
        return wt, O.f64(kc[idx].cpu()), O.f64(vc[idx].cpu())

    g = wl.globals
    return O.model_decode(toks, pos, O.f64(g["tok_embeddings"].cpu()), get_layer, w.n_layers,
                          O.f64(g["final_norm"].cpu()), O.f64(g["output"].cpu()), w.n_heads, w.eps, w.theta)
