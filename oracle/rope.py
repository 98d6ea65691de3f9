"""Float64 reference of rotary position embedding (RoPE) on queries and keys.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix (textbook page, attention chapter, "Как в attention
попадает позиция" and the table "Прямой проход по шагам", step 4): LLaMA,
Mistral, Mixtral and Gemma rotate q and k by a position-dependent angle so
that q_i . k_j depends only on i - j; V is not rotated; K enters the cache
already rotated (section on the layer cache), and with padding the rotation
takes explicit per-token positions instead of start_pos, start_pos + 1, ...
The head size must be even (section "Размерности", the head-size check).

What they leave open, and the reading taken here: the pages defer the
formula to RoFormer (Su et al., arXiv:2104.09864, which they cite).  From that
paper: coordinates are rotated in pairs, pair m by the angle p * theta_m with
theta_m = base^(-2m/Dh), base = 10000, counter-clockwise (the 2x2 block
[[cos, -sin], [sin, cos]] of its rotation matrix).  Two pairings are in use
and both are provided: ``style="pairs"`` rotates (x[2m], x[2m+1]) as in the
paper; ``style="half"`` rotates (x[m], x[m + Dh/2]), the layout of GPT-NeoX
and of LLaMA checkpoints in the Hugging Face format.  The base is a
parameter.
"""

import numpy as np


def rope_angles(positions, Dh, base=10000.0):
    """angle[..., m] = p * base**(-2m/Dh) for m = 0 .. Dh/2 - 1 (RoFormer,
    section 3.2: theta_i = 10000^(-2(i-1)/d) for i = 1 .. d/2)."""
    if Dh % 2:
        raise ValueError("RoPE needs an even head size")
    m = np.arange(Dh // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * m / Dh)
    return np.asarray(positions, dtype=np.float64)[..., None] * theta


def rope_table_ref(P, Dh, base=10000.0):
    """[P, Dh] table of positions 0 .. P-1: cos of the angles in columns
    0 .. Dh/2 - 1 and sin in columns Dh/2 .. Dh - 1."""
    a = rope_angles(np.arange(P), Dh, base)
    return np.concatenate([np.cos(a), np.sin(a)], axis=-1)


def rope_ref(X, positions, base=10000.0, style="pairs"):
    """Rotate X [B, H, S, Dh] (float64) by the positions [B, S] (or [S]).

    Pair (a, b) of token position p becomes (a cos - b sin, a sin + b cos)
    with angle p * theta_m.  Returns a new float64 array.
    """
    X = np.asarray(X, dtype=np.float64)
    B, H, S, Dh = X.shape
    pos = np.broadcast_to(np.asarray(positions), (B, S))
    ang = rope_angles(pos, Dh, base)[:, None, :, :]  # [B, 1, S, Dh/2]
    c, s = np.cos(ang), np.sin(ang)
    Y = np.empty_like(X)
    if style == "pairs":
        a, b = X[..., 0::2], X[..., 1::2]
        Y[..., 0::2] = a * c - b * s
        Y[..., 1::2] = a * s + b * c
    elif style == "half":
        a, b = X[..., : Dh // 2], X[..., Dh // 2:]
        Y[..., : Dh // 2] = a * c - b * s
        Y[..., Dh // 2:] = a * s + b * c
    else:
        raise ValueError("style must be 'pairs' or 'half'")
    return Y


def append_rope_ref(Kc, Vc, Knew, Vnew, pos, positions=None, rolling=False, base=10000.0,
                    style="pairs"):
    """Cache append with the keys rotated first: K goes into the cache after
    RoPE, V as it is (textbook, the layer-cache section).  Row i of sequence b
    is rotated by positions[b, i], or by its absolute position pos[b] + i when
    no positions are given, then written as ``append_ref`` writes it."""
    from .attention import append_ref

    Knew = np.asarray(Knew, dtype=np.float64)
    B, _, Snew, _ = Knew.shape
    if positions is None:
        positions = np.asarray(pos, dtype=np.int64)[:, None] + np.arange(Snew)[None, :]
    return append_ref(Kc, Vc, rope_ref(Knew, positions, base, style), Vnew, pos, rolling)
