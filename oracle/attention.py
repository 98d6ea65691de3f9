"""Float64 CPU oracle for causal scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it and shares no code with it.

What is computed, per batch entry b and query head h (sources: the attention
chapter of the LLM-architecture textbook page, "Механизм внимания",
section "Scaled dot-product attention" and its worked example
"Численный пример"; the Chinese multi-head attention post "多头注意力机制",
its mask and softmax sections):

    g      = kv_head_of(h)                      (GQA/MQA mapping)
    A      = scale * Q[b,h] @ K[b,g]^T          (scores)
    A[i,j] = -inf where (i, j) is not allowed   (causal mask, sliding window)
    m_i    = max_j A[i,j];  E = exp(A - m);  l_i = sum_j E[i,j];  P = E / l
    O[b,h] = P @ V[b,g]
    LSE[b,h,i] = m_i + ln l_i                   (natural-log log-sum-exp of
                                                 the scaled, masked scores)

The full score matrix is materialised on purpose: the oracle is the plain
definition, not the tiled algorithm, so a reader can check it against the
formula by eye.  Everything is float64; callers pass the exact stored input
values (bf16 or fp32) already widened to float64.

Readings taken where the pages leave a choice open:
  * the mask value is -inf (the Swedish page uses -1e9, the other pages -inf;
    the two agree whenever a row has a visible key, which the diagonal
    guarantees here);
  * the sliding window admits key j for query i iff 0 <= i - j < window
    (window keys including the query itself); the textbook's own repository
    admits i - j <= W, one more key;
  * a window requires the causal mask (the textbook defines the window as a
    cut of the causal past), so window > 0 with causal=False is an error;
  * prefill has as many keys as queries and the causal mask is aligned at the
    top-left corner: query i sees keys j <= i;
  * a decode step's cached length counts the current token: the query row
    sits at position lens-1 and sees keys 0..lens-1;
  * a chunk of Sq new queries appended to a cache of lens keys (chunked
    prefill) is aligned at the bottom-right corner: its query i sits at
    absolute position lens - Sq + i (the textbook's step-by-step forward pass
    takes mask rows from start_pos on), so the chunk's queries see every
    earlier cached key and causally each other;
  * a rolling-buffer cache of capacity W stores position p in slot p mod W;
    with the new token appended first, the buffer holds exactly the W
    positions a window of W admits, in rotated order, which the softmax does
    not see;
  * a key-padding mask (textbook, "Паддинг" under "Прямой проход по шагам":
    the padding's key mask is added to the causal mask and the window, one
    mask per batch row) hides key j of sequence b wherever key_mask[b, j] is
    false, on top of the causal mask and the window; a hidden key's weight
    is exactly 0, so its K and V must hold finite values (0 * NaN is NaN);
  * a query row that sees no key at all (possible only with a key-padding
    mask, e.g. a left-pad query) gets O = 0 and LSE = -inf: an empty weighted
    sum, where the textbook's masked_fill followed by softmax would give NaN;
  * the backward pass differentiates the same definition: the softmax
    Jacobian is dp_i/dz_j = p_i (delta_ij - p_j) (textbook, "Почему делить
    на корень из d_h"), the rest is the chain rule through the two products;
    a K/V head shared by G query heads collects the gradients of all of them.
"""

import numpy as np


def kv_head_of(h, n_q_heads, n_kv_heads):
    """K/V head used by query head ``h``: g(h) = floor(h / (H / G)).

    Textbook page, section "Виды по числу голов K/V: MHA, GQA, MQA": query
    heads are split into G consecutive groups of H/G heads; MHA is G = H,
    MQA is G = 1, and H not divisible by G is rejected (ValueError), as the
    page's constructor does.
    """
    if n_kv_heads <= 0 or n_q_heads <= 0:
        raise ValueError("head counts must be positive")
    if n_q_heads % n_kv_heads != 0:
        raise ValueError("number of query heads must be a multiple of K/V heads")
    group = n_q_heads // n_kv_heads
    return h // group


def allowed_mask(row_positions, n_keys, causal, window):
    """Boolean [len(row_positions), n_keys]: True where query may see key.

    Causal mask (textbook page, section "Маскирование"; Chinese post, the
    mask matrix M with -inf above the diagonal): key j is hidden from the
    query at position i when j > i.  Sliding window (textbook page, section
    "Скользящее окно", read with the window counted as in the long-context
    GQA workload: the query sees keys i-window+1 .. i): hidden when
    i - j >= window.
    """
    if window > 0 and not causal:
        raise ValueError("a sliding window needs the causal mask")
    i = np.asarray(row_positions, dtype=np.int64)[:, None]
    j = np.arange(n_keys, dtype=np.int64)[None, :]
    ok = np.ones((i.shape[0], n_keys), dtype=bool)
    if causal:
        ok &= j <= i
    if window > 0:
        ok &= (i - j) < window
    return ok


def softmax_rows(A):
    """Numerically stable row softmax: subtract the row max, exp, normalise.

    Swedish/English attention note (its ``softmax`` helper) and the German
    page's hand computation ("Von Hand"): x - max, e = exp, e / sum.
    Entries equal to -inf get weight exactly 0 (Chinese post, the
    softmax(3, 1, -inf) example).  Returns (P, m, l) with m the row max and
    l the row sum of exp(A - m).
    """
    A = np.asarray(A, dtype=np.float64)
    m = A.max(axis=-1, keepdims=True)
    E = np.exp(A - m)
    l = E.sum(axis=-1, keepdims=True)
    return E / l, m[..., 0], l[..., 0]


def head_attention(q_rows, row_positions, K, V, causal, window, scale,
                   return_probs=False, key_ok=None):
    """Attention of some query rows of one head against one K/V head.

    q_rows: [R, Dh] float64, row_positions: [R] absolute query positions,
    K, V: [T_kv, Dh], key_ok: optional [T_kv] booleans (False: padding key).
    Returns (O [R, Dh], LSE [R]) and, if asked, P [R, T_kv].  Steps follow the
    textbook's formula softmax(QK^T / sqrt(d_h) + M) V (section "Scaled
    dot-product attention") with the scale passed in.  A row with no visible
    key gets O = 0, LSE = -inf (and P = 0).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    A = scale * (q_rows @ K.T)
    ok = allowed_mask(row_positions, K.shape[0], causal, window)
    if key_ok is not None:
        ok &= np.asarray(key_ok, dtype=bool)[None, :]
    seen = ok.any(axis=1)
    A = np.where(ok, A, -np.inf)
    A[~seen] = 0.0  # placeholder, overwritten below
    P, m, l = softmax_rows(A)
    P[~seen] = 0.0
    O = P @ V
    LSE = m + np.log(l)
    LSE[~seen] = -np.inf
    if return_probs:
        return O, LSE, P
    return O, LSE


def _check_prefill_shapes(Q, K, V):
    if Q.ndim != 4 or K.ndim != 4 or V.ndim != 4:
        raise ValueError("Q, K, V must be [B, heads, S, Dh]")
    B, Nq, S, Dh = Q.shape
    if K.shape != V.shape or K.shape[0] != B or K.shape[2] != S or K.shape[3] != Dh:
        raise ValueError("K and V must be [B, Nkv, S, Dh] matching Q")
    return B, Nq, K.shape[1], S, Dh


def attention_ref(Q, K, V, causal=True, window=0, scale=None, key_mask=None):
    """Full prefill attention.  Q: [B,Nq,S,Dh], K,V: [B,Nkv,S,Dh].

    Returns O [B,Nq,S,Dh] and LSE [B,Nq,S], both float64.  ``scale`` defaults
    to 1/sqrt(Dh), the head size (textbook, "Почему делить на корень из d_h").
    ``key_mask``: optional [B, S] booleans, False for padding keys.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, Nq, Nkv, S, Dh = _check_prefill_shapes(Q, K, V)
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    O = np.empty((B, Nq, S, Dh))
    LSE = np.empty((B, Nq, S))
    rows = np.arange(S)
    for b in range(B):
        for h in range(Nq):
            g = kv_head_of(h, Nq, Nkv)
            O[b, h], LSE[b, h] = head_attention(
                Q[b, h], rows, K[b, g], V[b, g], causal, window, scale,
                key_ok=None if key_mask is None else key_mask[b])
    return O, LSE


def attention_rows_ref(Q, K, V, triples, causal=True, window=0, scale=None):
    """Selected output rows of prefill attention.

    ``triples`` is a sequence of (b, h, i).  Each row is computed on its own
    as a 1 x S score vector; returns O [n, Dh] and LSE [n].
    """
    B, Nq, Nkv, S, Dh = _check_prefill_shapes(Q, K, V)
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    n = len(triples)
    O = np.empty((n, Dh))
    LSE = np.empty(n)
    for t, (b, h, i) in enumerate(triples):
        g = kv_head_of(h, Nq, Nkv)
        q = np.asarray(Q[b, h, i], dtype=np.float64)[None, :]
        o, lse = head_attention(q, [i], np.asarray(K[b, g], dtype=np.float64),
                                np.asarray(V[b, g], dtype=np.float64),
                                causal, window, scale)
        O[t], LSE[t] = o[0], lse[0]
    return O, LSE


def decode_ref(q, Kc, Vc, lens, scale=None, rows=None, window=0, key_mask=None):
    """One decode step against a KV cache.

    q: [B,Nq,Dh], Kc, Vc: [B,Nkv,Tcap,Dh], lens: [B] with 1 <= lens[b] <= Tcap.
    Sequence b's query sees its cached keys 0..lens[b]-1 (the new token's
    key is already in the cache) -- textbook, sections "KV-кэш" and
    "Prefill и decode": a decode step is a single score row of length t.
    With ``window`` > 0 only the keys lens[b]-window .. lens[b]-1 are visible
    (section "Скользящее окно", in the i - j < window convention).
    Entries past lens[b] are never read.  ``scale`` defaults to 1/sqrt(Dh).
    ``key_mask``: optional [B, Tcap] booleans over the cache slots, False for
    padding keys.
    ``rows`` optionally restricts the work to (b, h) pairs; then O is
    [len(rows), Dh] and LSE [len(rows)].  Otherwise O [B,Nq,Dh], LSE [B,Nq].
    """
    B, Nq, Dh = q.shape
    Nkv = Kc.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    pairs = rows if rows is not None else [(b, h) for b in range(B) for h in range(Nq)]
    O = np.empty((len(pairs), Dh))
    LSE = np.empty(len(pairs))
    for t, (b, h) in enumerate(pairs):
        n = int(lens[b])
        if n < 1 or n > Kc.shape[2]:
            raise ValueError("cache length out of range")
        g = kv_head_of(h, Nq, Nkv)
        qrow = np.asarray(q[b, h], dtype=np.float64)[None, :]
        Kb = np.asarray(Kc[b, g, :n], dtype=np.float64)
        Vb = np.asarray(Vc[b, g, :n], dtype=np.float64)
        o, lse = head_attention(qrow, [n - 1], Kb, Vb, True, window, scale,
                                key_ok=None if key_mask is None else key_mask[b][:n])
        O[t], LSE[t] = o[0], lse[0]
    if rows is None:
        return O.reshape(B, Nq, Dh), LSE.reshape(B, Nq)
    return O, LSE


def chunk_ref(Q, Kc, Vc, lens, window=0, scale=None, rows=None, key_mask=None):
    """Chunked prefill: Sq new queries per sequence against a KV cache.

    Q: [B,Nq,Sq,Dh]; Kc, Vc: [B,Nkv,Tcap,Dh] already holding the chunk's own
    keys; lens: [B] cached keys per sequence including the chunk, with
    Sq <= lens[b] <= Tcap.  Query i of sequence b sits at absolute position
    lens[b] - Sq + i and sees keys j <= its position (and, with ``window``,
    position - j < window).  Textbook, "Prefill и decode": a long prompt can be
    filled chunk by chunk, with the causal mask again inside the chunk;
    "Прямой проход по шагам" and "Типичные ошибки и тонкости": the mask rows
    start at the first new position, not at 0.
    ``rows`` optionally restricts the work to (b, h, i) triples; then O is
    [len(rows), Dh] and LSE [len(rows)].  Otherwise O [B,Nq,Sq,Dh], LSE [B,Nq,Sq].
    ``key_mask``: optional [B, Tcap] booleans over the cache slots, False for
    padding keys.
    """
    B, Nq, Sq, Dh = Q.shape
    Nkv = Kc.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    for b in range(B):
        if not Sq <= int(lens[b]) <= Kc.shape[2]:
            raise ValueError("cache length must cover the chunk and fit the cache")
    if rows is not None:
        O = np.empty((len(rows), Dh))
        LSE = np.empty(len(rows))
        for t, (b, h, i) in enumerate(rows):
            n = int(lens[b])
            g = kv_head_of(h, Nq, Nkv)
            qrow = np.asarray(Q[b, h, i], dtype=np.float64)[None, :]
            o, lse = head_attention(qrow, [n - Sq + i], np.asarray(Kc[b, g, :n], dtype=np.float64),
                                    np.asarray(Vc[b, g, :n], dtype=np.float64), True, window, scale,
                                    key_ok=None if key_mask is None else key_mask[b][:n])
            O[t], LSE[t] = o[0], lse[0]
        return O, LSE
    O = np.empty((B, Nq, Sq, Dh))
    LSE = np.empty((B, Nq, Sq))
    for b in range(B):
        n = int(lens[b])
        positions = np.arange(n - Sq, n)
        for h in range(Nq):
            g = kv_head_of(h, Nq, Nkv)
            O[b, h], LSE[b, h] = head_attention(
                np.asarray(Q[b, h], dtype=np.float64), positions,
                np.asarray(Kc[b, g, :n], dtype=np.float64),
                np.asarray(Vc[b, g, :n], dtype=np.float64), True, window, scale,
                key_ok=None if key_mask is None else key_mask[b][:n])
    return O, LSE


def append_ref(Kc, Vc, Knew, Vnew, pos, rolling=False):
    """Write new K/V rows into a cache; returns the updated copies.

    Kc, Vc: [B,Nkv,Tcap,...]; Knew, Vnew: [B,Nkv,Snew,...]; pos: [B] absolute
    position of each sequence's first new row (its token count before the
    append).  Row i lands in slot pos[b] + i of a linear cache (textbook,
    "Прямой проход по шагам": the new K and V are concatenated after the
    cached ones), or in slot (pos[b] + i) mod Tcap of a rolling buffer
    ("Скользящее окно": only the last positions are kept; Mistral's rolling
    buffer cache).  Rows are written in order, so when a rolling append is
    longer than the buffer the latest rows win.  A linear append past Tcap is
    an error.
    """
    Kc = np.array(Kc, copy=True)
    Vc = np.array(Vc, copy=True)
    B, Nkv, Tcap = Kc.shape[:3]
    Snew = Knew.shape[2]
    for b in range(B):
        p0 = int(pos[b])
        if p0 < 0 or (not rolling and p0 + Snew > Tcap):
            raise ValueError("append outside the cache")
        for i in range(Snew):
            slot = (p0 + i) % Tcap if rolling else p0 + i
            Kc[b, :, slot] = Knew[b, :, i]
            Vc[b, :, slot] = Vnew[b, :, i]
    return Kc, Vc


def softmax_vjp(P, dP):
    """Vector-Jacobian product of the row softmax: given P = softmax(Z) row by
    row and dL/dP, returns dL/dZ.

    Textbook, "Почему делить на корень из d_h": dp_i/dz_j = p_i (delta_ij - p_j),
    so dL/dz_j = sum_i dL/dp_i * p_i (delta_ij - p_j) = p_j (dP_j - sum_i p_i dP_i).
    Masked entries have p = 0 and receive 0.
    """
    P = np.asarray(P, dtype=np.float64)
    dP = np.asarray(dP, dtype=np.float64)
    return P * (dP - np.sum(P * dP, axis=-1, keepdims=True))


def backward_ref(Q, K, V, dO, causal=True, window=0, scale=None, key_mask=None):
    """Gradients of the prefill attention output with respect to Q, K and V.

    Q: [B,Nq,S,Dh], K, V: [B,Nkv,S,Dh], dO = dL/dO: [B,Nq,S,Dh].  Returns
    (dQ, dK, dV) in float64 with the shapes of Q, K, V.  Per (b, h) with
    g = kv_head_of(h), by the chain rule through A = scale * Q K^T + M,
    P = softmax(A) (row-wise), O = P V:
        dV[g] += P^T dO,   dP = dO V^T,   dA = softmax_vjp(P, dP),
        dQ     = scale * dA K,   dK[g] += scale * dA^T Q.
    A K/V head shared by several query heads (GQA/MQA) sums their
    contributions (textbook, "Как K/V-головы доходят до голов Q": the shared
    head is repeated, so its gradient is the sum over the repeats).  The
    weights are recomputed from the inputs here, as the textbook's
    FlashAttention section says the backward pass does.  ``key_mask``:
    optional [B, S] booleans, False for padding keys (the forward's mask, so
    a hidden key has weight 0 and receives no gradient, and a query row that
    sees no key has O = 0 and gradient 0).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, Nq, Nkv, S, Dh = _check_prefill_shapes(Q, K, V)
    if dO.shape != Q.shape:
        raise ValueError("dO must have the shape of Q")
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    rows = np.arange(S)
    for b in range(B):
        for h in range(Nq):
            g = kv_head_of(h, Nq, Nkv)
            _, _, P = head_attention(Q[b, h], rows, K[b, g], V[b, g], causal, window, scale,
                                     return_probs=True,
                                     key_ok=None if key_mask is None else key_mask[b])
            dV[b, g] += P.T @ dO[b, h]
            dP = dO[b, h] @ V[b, g].T
            dA = softmax_vjp(P, dP)
            dQ[b, h] = scale * (dA @ K[b, g])
            dK[b, g] += scale * (dA.T @ Q[b, h])
    return dQ, dK, dV


def backward_rows_ref(Q, K, V, dO, q_rows=(), kv_rows=(), causal=True, window=0, scale=None,
                      key_mask=None):
    """Selected rows of the gradients of ``backward_ref``, for inputs too long
    for the full score matrices.

    q_rows: (b, h, i) triples -> dQ[b, h, i]; kv_rows: (b, g, j) triples ->
    dK[b, g, j] and dV[b, g, j].  Same chain rule as ``backward_ref``, taken
    one query row at a time: the row's weights P_i (``head_attention``), its
    dP_i = V dO_i and dA_i = softmax_vjp(P_i, dP_i); dQ_i = scale * dA_i K,
    and key j collects P_ij dO_i into dV_j and scale * dA_ij Q_i into dK_j
    from every query row i of the group's heads that sees it.  Arrays may be
    memory-mapped or lazily widened; only the rows used are read.  ``key_mask``
    as in ``backward_ref``: a padding key is seen by no query row.
    Returns (dQ_rows [len(q_rows), Dh], dK_rows, dV_rows [len(kv_rows), Dh]).
    """
    B, Nq, S, Dh = Q.shape
    Nkv = K.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    group = Nq // Nkv
    heads, rows = {}, {}

    def head_kv(b, g):
        if (b, g) not in heads:
            heads[(b, g)] = (np.asarray(K[b, g], dtype=np.float64),
                             np.asarray(V[b, g], dtype=np.float64))
        return heads[(b, g)]

    def row_grads(b, h, i):
        if (b, h, i) not in rows:
            Kb, Vb = head_kv(b, kv_head_of(h, Nq, Nkv))
            q = np.asarray(Q[b, h, i], dtype=np.float64)[None, :]
            _, _, P = head_attention(q, [i], Kb, Vb, causal, window, scale, return_probs=True,
                                     key_ok=None if key_mask is None else key_mask[b])
            dP = np.asarray(dO[b, h, i], dtype=np.float64)[None, :] @ Vb.T
            rows[(b, h, i)] = (P[0], softmax_vjp(P, dP)[0])
        return rows[(b, h, i)]

    dQ = np.empty((len(q_rows), Dh))
    for t, (b, h, i) in enumerate(q_rows):
        _, dA = row_grads(b, h, i)
        dQ[t] = scale * (dA @ head_kv(b, kv_head_of(h, Nq, Nkv))[0])
    dK = np.zeros((len(kv_rows), Dh))
    dV = np.zeros((len(kv_rows), Dh))
    for t, (b, g, j) in enumerate(kv_rows):
        # query rows that see key j: allowed_mask's rule along its column j
        i_all = np.arange(S)
        seen = np.ones(S, dtype=bool)
        if causal:
            seen &= j <= i_all
        if window > 0:
            seen &= (i_all - j) < window
        if key_mask is not None and not key_mask[b][j]:
            seen[:] = False
        for h in range(g * group, (g + 1) * group):
            for i in np.flatnonzero(seen):
                P, dA = row_grads(b, h, int(i))
                dV[t] += P[j] * np.asarray(dO[b, h, i], dtype=np.float64)
                dK[t] += scale * dA[j] * np.asarray(Q[b, h, i], dtype=np.float64)
    return dQ, dK, dV
