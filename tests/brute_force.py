"""Explicit-loop, scalar-by-scalar second implementation of the block, written
independently of oracle/llama_oracle.py (no NumPy vectorisation, no shared
helpers) to pin the oracle on tiny inputs. Python floats are IEEE doubles.

Definitions followed: paperfordummies.in "LLaMA: Open and Efficient Foundation
Language Models", sections "The one formula" and "The code" (rms_norm, silu,
swiglu_ffn, rope, pre_norm_block); chenyuan1125.github.io "LLaMA: No
Architecture Revolution ...", section "An Architecture Recipe Without an
Invention Myth" (gain g on RMSNorm)."""
import math


def rmsnorm_rows(x, g, eps):
    out = []
    for row in x:
        s = 0.0
        for v in row:
            s += v * v
        r = math.sqrt(s / len(row) + eps)
        out.append([row[i] / r * (1.0 if g is None else g[i]) for i in range(len(row))])
    return out


def matvec_rows(x, w):
    """x [T][K], w [N][K] -> [T][N] with y[t][n] = sum_k x[t][k] * w[n][k]."""
    out = []
    for row in x:
        o = []
        for wn in w:
            acc = 0.0
            for k in range(len(row)):
                acc += row[k] * wn[k]
            o.append(acc)
        out.append(o)
    return out


def rope_rows(x, positions, head_dim, theta):
    out = []
    for t, row in enumerate(x):
        o = list(row)
        p = positions[t]
        for h0 in range(0, len(row), head_dim):
            for i in range(head_dim // 2):
                ang = p * theta ** (-(2.0 * i) / head_dim)
                c, s = math.cos(ang), math.sin(ang)
                a, b = row[h0 + 2 * i], row[h0 + 2 * i + 1]
                o[h0 + 2 * i] = a * c - b * s
                o[h0 + 2 * i + 1] = a * s + b * c
        out.append(o)
    return out


def silu(v):
    return v / (1.0 + math.exp(-v)) if v > -700 else 0.0 * v


def attention(q, k, v, batch, seq, n_heads, n_kv_heads=None):
    """Explicit loops; with n_kv_heads < n_heads, query head h reads key/value
    head h * n_kv_heads // n_heads (consecutive groups)."""
    d = len(q[0])
    hd = d // n_heads
    n_kv = n_kv_heads or n_heads
    out = [[0.0] * d for _ in range(batch * seq)]
    for b in range(batch):
        for h in range(n_heads):
            kvh = h * n_kv // n_heads
            for i in range(seq):
                qi = q[b * seq + i]
                scores = []
                for j in range(i + 1):            # keys 0..i, diagonal included
                    kj = k[b * seq + j]
                    acc = 0.0
                    for e in range(hd):
                        acc += qi[h * hd + e] * kj[kvh * hd + e]
                    scores.append(acc / math.sqrt(hd))
                m = max(scores)
                ex = [math.exp(s - m) for s in scores]
                tot = sum(ex)
                for e in range(hd):
                    acc = 0.0
                    for j in range(i + 1):
                        acc += ex[j] / tot * v[b * seq + j][kvh * hd + e]
                    out[b * seq + i][h * hd + e] = acc
    return out


def block(x, w, batch, seq, n_heads, eps, theta):
    d = len(x[0])
    hd = d // n_heads
    pos = [float(s) for _ in range(batch) for s in range(seq)]
    z = rmsnorm_rows(x, w["attn_norm"], eps)
    q = rope_rows(matvec_rows(z, w["wq"]), pos, hd, theta)
    k = rope_rows(matvec_rows(z, w["wk"]), pos, hd, theta)
    v = matvec_rows(z, w["wv"])
    a = attention(q, k, v, batch, seq, n_heads)
    o = matvec_rows(a, w["wo"])
    h = [[x[t][c] + o[t][c] for c in range(d)] for t in range(len(x))]
    z2 = rmsnorm_rows(h, w["ffn_norm"], eps)
    gate = matvec_rows(z2, w["w_gate"])
    up = matvec_rows(z2, w["w_up"])
    u = [[silu(gate[t][j]) * up[t][j] for j in range(len(gate[t]))] for t in range(len(gate))]
    dn = matvec_rows(u, w["w_down"])
    return [[h[t][c] + dn[t][c] for c in range(d)] for t in range(len(x))]


def add_rows(a, b):
    return [[a[t][c] + b[t][c] for c in range(len(a[t]))] for t in range(len(a))]


def attn_branch(z, w, batch, seq, n_heads, theta):
    hd = len(z[0]) // n_heads
    pos = [float(s) for _ in range(batch) for s in range(seq)]
    q = rope_rows(matvec_rows(z, w["wq"]), pos, hd, theta)
    k = rope_rows(matvec_rows(z, w["wk"]), pos, hd, theta)
    return matvec_rows(attention(q, k, matvec_rows(z, w["wv"]), batch, seq, n_heads), w["wo"])


def ffn_branch(z, w):
    gate, up = matvec_rows(z, w["w_gate"]), matvec_rows(z, w["w_up"])
    u = [[silu(gate[t][j]) * up[t][j] for j in range(len(gate[t]))] for t in range(len(gate))]
    return matvec_rows(u, w["w_down"])


def post_norm_block(x, w, batch, seq, n_heads, eps, theta):
    """Norm on the trunk after each residual add (2017 ordering)."""
    h = rmsnorm_rows(add_rows(x, attn_branch(x, w, batch, seq, n_heads, theta)), w["attn_norm"], eps)
    return rmsnorm_rows(add_rows(h, ffn_branch(h, w)), w["ffn_norm"], eps)


def no_norm_block(x, w, batch, seq, n_heads, theta):
    """Pre-norm block with both norms removed."""
    h = add_rows(x, attn_branch(x, w, batch, seq, n_heads, theta))
    return add_rows(h, ffn_branch(h, w))
