"""Float64 definitions for a vision-tower attention block's position encoding and attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by the tests, the smoke check
and the bench's CPU-baseline leg, never by the product path.

Sources:
  * inferencelayer 0.2.3, ``vision.rs``: ``rope_tables_2d`` (2-D rope tables over a block-major
    patch grid: the rotary half of the head split evenly between the row and the column axis,
    frequencies theta^(-2i/half), ``emb = cat(freqs, freqs)``) and the vision block's
    ``attention`` (``rotate_half`` application on split halves, full bidirectional softmax
    attention with scale 1/sqrt(head_dim)).
  * cortiq-engine 0.8.51, ``onevision2.rs``: module doc and ``rope_tables`` (three axes t, h, w
    splitting the half-dimension 4:6:6, each axis theta^(-i/n_axis), angles concatenated with
    themselves, patches in merge-block order), ``split_rope`` (the interleaved ``rotate_half``
    on adjacent lanes, where the two lanes of a pair take the table entries of their own index,
    hence different angles, as the module doc states) and ``attend`` (bidirectional attention).
"""

import numpy as np


def merge_block_positions(t, h, w, merge):
    """(frame, row, col) of every patch, frames in order and, within a frame, merge blocks of
    merge x merge patches in row-major block order, each block's patches row-major."""
    out = []
    for f in range(t):
        for a in range(h // merge):
            for b in range(w // merge):
                for mh in range(merge):
                    for mw in range(merge):
                        out.append((f, a * merge + mh, b * merge + mw))
    return np.array(out, dtype=np.int64).reshape(-1, 3)


def rope_tables_2d(grid, head_dim, theta, merge):
    """cos, sin [n, head_dim] of the 2-D tables (inferencelayer ``rope_tables_2d``): with half =
    head_dim/2 and nf = half/2, freqs = [r inv_0 .. r inv_{nf-1} | c inv_0 .. c inv_{nf-1}],
    inv_i = theta^(-2i/half), then emb = cat(freqs, freqs)."""
    half = head_dim // 2
    nf = half // 2
    inv = np.array([theta ** (-(2.0 * i) / half) for i in range(nf)])
    pos = merge_block_positions(*grid, merge)
    freqs = np.concatenate([pos[:, 1:2] * inv[None, :], pos[:, 2:3] * inv[None, :]], axis=1)
    emb = np.concatenate([freqs, freqs], axis=1)
    return np.cos(emb), np.sin(emb)


def rope_tables_3axis(grid, head_dim, theta, merge):
    """cos, sin [n, head_dim] of the three-axis tables (onevision2 ``rope_tables``): half =
    head_dim/2 angles split 4:6:6 between t, h, w (unit = half/16), axis frequencies
    theta^(-i/n_axis), angle j = [t it | row ih | col iw][j], entry j of the table uses angle
    j mod half."""
    half = head_dim // 2
    unit = half // 16
    nt, nh, nw = 4 * unit, 6 * unit, 6 * unit

    def inv(n):
        return np.array([theta ** (-float(i) / n) for i in range(n)])

    pos = merge_block_positions(*grid, merge)
    ang = np.concatenate([pos[:, 0:1] * inv(nt)[None, :], pos[:, 1:2] * inv(nh)[None, :],
                          pos[:, 2:3] * inv(nw)[None, :]], axis=1)
    emb = ang[:, np.arange(head_dim) % half]
    return np.cos(emb), np.sin(emb)


def rope_split_half(x, cos, sin):
    """x [n, heads, hd] -> x * cos + rotate_half(x) * sin with rotate_half(x) = [-x[half:], x[:half]]
    (inferencelayer vision ``attention``), cos/sin [n, hd] shared by every head."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    rot = np.concatenate([-x[..., half:], x[..., :half]], axis=-1)
    return x * cos[:, None, :] + rot * sin[:, None, :]


def rope_adjacent(x, cos, sin):
    """x [n, heads, hd] -> for each even lane i: y_i = x_i c_i - x_{i+1} s_i,
    y_{i+1} = x_{i+1} c_{i+1} + x_i s_{i+1} (onevision2 ``split_rope``)."""
    x = np.asarray(x, dtype=np.float64)
    c, s = cos[:, None, :], sin[:, None, :]
    y = np.empty_like(x)
    y[..., 0::2] = x[..., 0::2] * c[..., 0::2] - x[..., 1::2] * s[..., 0::2]
    y[..., 1::2] = x[..., 1::2] * c[..., 1::2] + x[..., 0::2] * s[..., 1::2]
    return y


def bidirectional_attention(q, k, v):
    """Full (non-causal) softmax attention, scale 1/sqrt(head_dim): q [S, nh, hd], k, v
    [S, nkv, hd]; query head h reads key/value head h / (nh / nkv) (inferencelayer vision
    ``attention``, onevision2 ``attend``)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s, nh, hd = q.shape
    nkv = k.shape[1]
    group = nh // nkv
    out = np.empty((s, nh, hd))
    for h in range(nh):
        g = h // group
        z = (q[:, h, :] @ k[:, g, :].T) / np.sqrt(hd)
        z = z - z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out
