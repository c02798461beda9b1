"""Brute-force scalar versions of the layer's steps, for tiny inputs only.

Plain Python loops over floats (math module), written independently of the
oracle, used to pin it: a dropped term, a transposed operand or a wrong
index in the oracle shows up as a mismatch here.
"""

import math


def matvec_rows(x, w):
    """y[s][n] = sum_k x[s][k] * w[n][k]."""
    return [[sum(xs[kk] * w[n][kk] for kk in range(len(xs))) for n in range(len(w))] for xs in x]


def rmsnorm_row(row, g, eps):
    ms = sum(v * v for v in row) / len(row)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r * gg for v, gg in zip(row, g)]


def rope_row(row, p_t, p_h, p_w, theta, axes):
    hd = len(row)
    half = hd // 2
    out = list(row)
    for i in range(half):
        p = (p_t, p_h, p_w)[axes[i]]
        ang = p * theta ** (-2.0 * i / hd)
        a, b = row[i], row[i + half]
        out[i] = a * math.cos(ang) - b * math.sin(ang)
        out[i + half] = a * math.sin(ang) + b * math.cos(ang)
    return out


def attention(q, k, v, nh, nkv, hd):
    """q: [S][nh*hd], k/v: [S][nkv*hd] flat rows. Causal per-pair loop."""
    s_len = len(q)
    grp = nh // nkv
    out = [[0.0] * (nh * hd) for _ in range(s_len)]
    for h in range(nh):
        g = h // grp
        for s in range(s_len):
            qs = q[s][h * hd:(h + 1) * hd]
            sc = []
            for j in range(s + 1):
                kj = k[j][g * hd:(g + 1) * hd]
                sc.append(sum(a * b for a, b in zip(qs, kj)) / math.sqrt(hd))
            m = max(sc)
            e = [math.exp(z - m) for z in sc]
            den = sum(e)
            for d in range(hd):
                out[s][h * hd + d] = sum(e[j] / den * v[j][g * hd + d] for j in range(s + 1))
    return out


def layer(x, w, nh, nkv, hd, eps, theta, axes, pos, ds_rows=(), ds=()):
    """Whole layer on nested lists; pos = (t_list, h_list, w_list)."""
    s_len = len(x)
    xn = [rmsnorm_row(r, w["attn_norm"], eps) for r in x]
    q = matvec_rows(xn, w["wq"])
    k = matvec_rows(xn, w["wk"])
    v = matvec_rows(xn, w["wv"])

    def norm_rope(rows, heads, g):
        out = []
        for s, r in enumerate(rows):
            new = []
            for h in range(heads):
                seg = rmsnorm_row(r[h * hd:(h + 1) * hd], g, eps)
                new += rope_row(seg, pos[0][s], pos[1][s], pos[2][s], theta, axes)
            out.append(new)
        return out

    q = norm_rope(q, nh, w["q_norm"])
    k = norm_rope(k, nkv, w["k_norm"])
    o = attention(q, k, v, nh, nkv, hd)
    proj = matvec_rows(o, w["wo"])
    y1 = [[a + b for a, b in zip(x[s], proj[s])] for s in range(s_len)]
    yn = [rmsnorm_row(r, w["ffn_norm"], eps) for r in y1]
    gate = matvec_rows(yn, w["w_gate"])
    up = matvec_rows(yn, w["w_up"])
    act = [[(gv / (1.0 + math.exp(-gv))) * uv for gv, uv in zip(gr, ur)] for gr, ur in zip(gate, up)]
    down = matvec_rows(act, w["w_down"])
    y2 = [[a + b for a, b in zip(y1[s], down[s])] for s in range(s_len)]
    for kk, r in enumerate(ds_rows):
        y2[r] = [a + b for a, b in zip(y2[r], ds[kk])]
    return y2
