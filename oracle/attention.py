"""Float64 CPU oracle for exact attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module.  The GPU path never imports it.

Conventions (shared with the C ABI only by *meaning*, not by code):

* Tensors are ``[B, H, N, D]`` arrays (any float dtype; they are upcast to
  float64 exactly).  ``lse`` is ``[B, H, N]``.
* ``scale`` multiplies Q K^T before the mask and the softmax, and scales
  dQ and dK in the backward pass ([FA-CUDA] §1; [FA-WHY] §3.3).
* ``causal`` masks key j for query i when j > i, i.e. a square, top-left
  aligned mask with -inf ([FA-CUDA] §1).
* The log-sum-exp uses the natural logarithm: LSE_i = m_i + ln l_i
  ([FA-WHY] §3.2, last remark of the section).
* Grouped heads: K and V may have H_kv heads with H_kv dividing the H query
  heads (H_kv = 1: multi-query).  Query head h then reads K/V head
  h // (H / H_kv) ("CUDA FlashAttention ...", §7 lists GQA/MQA among the
  features a production kernel has to handle); the gradients of a shared
  K/V head sum over the query heads of its group.
* ``key_mask`` (optional, ``[B, N]``, nonzero = visible) is a key-padding
  mask: score S_ij of batch element b is -inf where key j is not visible,
  before the max, like the causal mask.  It is how padded variable-length
  batches are described ([FA-MI50] §4.3: padding masks of variable-length
  sequences; §5.1: random mask patterns as a test).  A row that sees no
  visible key has no defined softmax; the reading taken here is O_i = 0 and
  LSE_i = -inf, and such a row contributes nothing to any gradient (the -inf
  guard of [FA-CUDA] §6: with m = -inf nothing is exponentiated against it).

Source titles: [FA-CUDA] "CUDA FlashAttention: from online softmax to the
long-sequence IO limit"; [FA-ALGO] "FlashAttention algorithm details" (ch. 4);
[FA-WHY] "Why FlashAttention does not need to store the attention matrix";
[FA-MI50] "FlashAttention dataflow and engineering validation on MI50".
"""

from __future__ import annotations

import math

import numpy as np

from .dropout import dropout_keep_rows, dropout_threshold

NEG_INF = -np.inf


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _check4(*arrays):
    for a in arrays:
        if a.ndim != 4:
            raise ValueError("expected [B, H, N, D] arrays, got shape %r" % (a.shape,))


def _group(q, k):
    """Query heads per K/V head (H // H_kv); checks that H_kv divides H."""
    H, Hkv = q.shape[1], k.shape[1]
    if Hkv < 1 or H % Hkv != 0:
        raise ValueError("K/V heads (%d) must divide query heads (%d)" % (Hkv, H))
    return H // Hkv


# ---------------------------------------------------------------------------
# Plain definition: two-pass safe softmax over complete, materialised rows.
# ---------------------------------------------------------------------------
def _scores_block(qh, kh, i0, i1, causal, scale, rows=None, vis=None):
    """Score rows S = scale * Q K^T with the causal -inf mask applied.

    Rows are query indices i0..i1-1, or the explicit index array ``rows``.
    With ``causal`` the block only ever sees keys 0..max(row), so it is
    truncated there; the truncated columns would all be -inf anyway.
    ``vis`` (bool [N]) sets the columns of invisible keys to -inf.
    Definition: [FA-CUDA] §1 (S = QK^T/sqrt(D) + M, M_ij = -inf for j > i).
    """
    if rows is None:
        rows = np.arange(i0, i1)
    nk = int(rows.max()) + 1 if causal else kh.shape[0]
    s = scale * (qh[rows] @ kh[:nk].T)
    if causal:
        cols = np.arange(nk)[None, :]
        s = np.where(cols > rows[:, None], NEG_INF, s)
    if vis is not None:
        s = np.where(vis[None, :nk], s, NEG_INF)
    return s, nk


def _safe_softmax_rows(s):
    """Safe softmax of complete rows: subtract the row max, exponentiate,
    normalise ([FA-WHY] §3.1).  Returns (P, m, l) with l = sum exp(s - m).
    A row whose scores are all -inf gets P = 0, m = -inf and l = 0."""
    m = s.max(axis=1)
    seen = np.isfinite(m)
    e = np.exp(s - np.where(seen, m, 0.0)[:, None])
    l = e.sum(axis=1)
    return e / np.where(seen, l, 1.0)[:, None], m, l


def _visibility(key_mask, B, N):
    """key_mask [B, N] -> bool array, or None for no mask."""
    if key_mask is None:
        return None
    vis = np.asarray(key_mask) != 0
    if vis.shape != (B, N):
        raise ValueError("key_mask must be [B, N] = %r, got %r" % ((B, N), vis.shape))
    return vis


def _drop(dropout, B, H, N, b, h, rows, nk):
    """Keep mask times the keep scale for query rows ``rows`` of head (b, h),
    over keys 0..nk-1, or None without dropout.  ``dropout`` is (p, seed,
    offset), or (p, seed, offset, head_numbers) where head_numbers[b][h] is
    the head number the generator's counter uses (default b*H + h) -- so a
    few heads of a larger problem can be checked on their own."""
    if dropout is None:
        return None
    p, seed, offset = dropout[:3]
    bh = int(dropout[3][b][h]) if len(dropout) > 3 else b * H + h
    _, keep_scale = dropout_threshold(p)
    return dropout_keep_rows(bh, N, p, seed, offset, rows=rows)[:, :nk] * keep_scale


def attention_forward(q, k, v, causal, scale, row_block=256, rows=None, key_mask=None, dropout=None):
    """O = softmax(scale * Q K^T + M) V and LSE, by the plain definition.

    For every (b, h) and every block of ``row_block`` query rows the complete
    score rows are materialised in float64, softmax is taken with the
    two-pass safe formula and O = P V.  LSE_i = m_i + ln(sum_j exp(S_ij - m_i)).
    Sources: [FA-CUDA] §1 (definition), [FA-WHY] §3.1 (safe softmax) and
    §3.2 (LSE = m + log l).

    ``rows``: optional 1-D array of query indices; then only those rows are
    computed (for every head) and the outputs have len(rows) in place of N.
    ``key_mask``: optional [B, N] key-padding mask (see the module notes);
    rows without a visible key get O = 0 and LSE = -inf.
    ``dropout``: optional (p, seed, offset); O = (P * Z / (1 - p')) V with the
    keep mask Z of ``oracle.dropout`` (LSE stays that of the undropped P).

    Returns (O, LSE) as float64 arrays of shape [B,H,R,D] and [B,H,R].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check4(q, k, v)
    B, H, N, D = q.shape
    grp = _group(q, k)
    vis = _visibility(key_mask, B, N)
    sel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = sel.shape[0]
    o = np.empty((B, H, R, D))
    lse = np.empty((B, H, R))
    for b in range(B):
        for h in range(H):
            qh, kh, vh = q[b, h], k[b, h // grp], v[b, h // grp]
            for r0 in range(0, R, row_block):
                r1 = min(R, r0 + row_block)
                s, nk = _scores_block(qh, kh, 0, 0, causal, scale, rows=sel[r0:r1],
                                      vis=None if vis is None else vis[b])
                p, m, l = _safe_softmax_rows(s)
                z = _drop(dropout, B, H, N, b, h, sel[r0:r1], nk)
                o[b, h, r0:r1] = (p if z is None else p * z) @ vh[:nk]
                lse[b, h, r0:r1] = np.where(np.isfinite(m), m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return o, lse


def attention_probs(q, k, causal, scale):
    """The full probability matrix P for one head (q, k: [N, D]).

    For small inputs only (it is N x N).  Same definition as above.
    """
    q, k = _f64(q), _f64(k)
    n = q.shape[0]
    s, _ = _scores_block(q, k, 0, n, False, scale)
    if causal:
        s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], NEG_INF, s)
    p, _, _ = _safe_softmax_rows(s)
    return p


def attention_backward(q, k, v, do, causal, scale, row_block=256, key_mask=None, dropout=None):
    """dQ, dK, dV of L with dL/dO = ``do``, by the plain definition.

    With P the forward probabilities and G = dO:
        dP = G V^T,  Delta_i = sum_j P_ij dP_ij,  dS = P * (dP - Delta),
        dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T G.
    [FA-WHY] §3.3 states these formulas including the scale factor;
    [FA-ALGO] §4.3.1 gives the same ones with the scale omitted.  P is
    materialised in float64 a block of query rows at a time; sums over
    query rows are split over those blocks.  With ``key_mask``, P is the
    masked softmax (zero for invisible keys and for rows with no visible key).
    With ``dropout`` (p, seed, offset) and D = Z / (1 - p') the scaled keep
    mask, the output is O = (P*D) V, so dV = (P*D)^T G, dP = (G V^T) * D,
    Delta_i = sum_j P_ij dP_ij (= rowsum(G * O)) and dS = P * (dP - Delta).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _check4(q, k, v, do)
    B, H, N, D = q.shape
    grp = _group(q, k)
    vis = _visibility(key_mask, B, N)
    dq = np.zeros((B, H, N, D))
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            hk = h // grp  # the K/V head this query head reads; its gradients sum over the group
            qh, kh, vh, gh = q[b, h], k[b, hk], v[b, hk], do[b, h]
            for i0 in range(0, N, row_block):
                i1 = min(N, i0 + row_block)
                s, nk = _scores_block(qh, kh, i0, i1, causal, scale, vis=None if vis is None else vis[b])
                p, _, _ = _safe_softmax_rows(s)
                g = gh[i0:i1]
                z = _drop(dropout, B, H, N, b, h, np.arange(i0, i1), nk)
                dv[b, hk, :nk] += (p if z is None else p * z).T @ g
                dp = g @ vh[:nk].T
                if z is not None:
                    dp = dp * z
                delta = (p * dp).sum(axis=1)
                ds = p * (dp - delta[:, None])
                dq[b, h, i0:i1] = scale * (ds @ kh[:nk])
                dk[b, hk, :nk] += scale * (ds.T @ qh[i0:i1])
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Online (streaming) recurrence, written separately from the definition above.
# ---------------------------------------------------------------------------
def merge_states(m_a, l_a, o_a, m_b, l_b, o_b):
    """Merge two partial softmax states of the same query rows.

    A state (m, l, o) holds the running max m, l = sum exp(s - m) and the
    unnormalised o = sum exp(s - m) v over the keys it has seen.  The merged
    state takes m = max(m_a, m_b) and rescales each side by exp(m_side - m)
    ([FA-CUDA] §4, alpha and beta).  A side with m = -inf has seen no
    visible key and contributes zero (the guard of [FA-CUDA] §6 and
    [FA-WHY] §3.2: its rescale factor is taken as 0, never exp(-inf+inf)).

    Arrays: m_*, l_* shape [R]; o_* shape [R, D] (or None to skip o).
    """
    m_a, l_a, m_b, l_b = _f64(m_a), _f64(l_a), _f64(m_b), _f64(l_b)
    m = np.maximum(m_a, m_b)
    fin = np.isfinite(m)
    m_safe = np.where(fin, m, 0.0)
    alpha = np.where(np.isneginf(m_a), 0.0, np.exp(np.where(np.isneginf(m_a), 0.0, m_a) - m_safe))
    beta = np.where(np.isneginf(m_b), 0.0, np.exp(np.where(np.isneginf(m_b), 0.0, m_b) - m_safe))
    l = alpha * l_a + beta * l_b
    if o_a is None:
        return m, l, None
    o = alpha[:, None] * _f64(o_a) + beta[:, None] * _f64(o_b)
    return m, l, o


def online_forward(q, k, v, causal, scale, block_q=64, block_k=64,
                   ablate_rescale=False, trace_row=None):
    """Tiled attention with the online softmax recurrence, one head.

    q, k, v: [N, D].  The outer loop walks query tiles of ``block_q`` rows,
    the inner loop key/value tiles of ``block_k`` keys ([FA-ALGO] §4.2.1;
    [FA-CUDA] §5.1).  Per tile ([FA-WHY] §3.2; [FA-ALGO] §4.2.1 steps 1-5):

        S    = scale * Q_i K_j^T, causal entries j > i set to -inf first
        m'   = max(m, rowmax S)
        corr = exp(m - m')           (0 when m is still -inf)
        l    = corr * l + rowsum exp(S - m')
        O    = corr * O + exp(S - m') V_j
        m    = m'

    and finally O / l and LSE = m + ln l.  Key tiles that lie wholly above
    the diagonal are skipped ([FA-WHY] §4.5).

    ``ablate_rescale=True`` replaces corr by 1, reproducing the broken
    variant of [FA-WHY] §09; it exists only so a test can show the pin
    catches that mistake.  ``trace_row`` (an int) records, for that query
    row, (key tile start, m, l, corr) after every key tile it visits.

    Returns (O [N,D], LSE [N], info) where info holds ``tiles`` (number of
    (query tile, key tile) pairs computed) and ``trace`` (list or None).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    o_out = np.empty((n, d))
    lse_out = np.empty(n)
    tiles = 0
    trace = [] if trace_row is not None else None
    for i0 in range(0, n, block_q):
        i1 = min(n, i0 + block_q)
        m = np.full(i1 - i0, NEG_INF)
        l = np.zeros(i1 - i0)
        acc = np.zeros((i1 - i0, d))
        for j0 in range(0, n, block_k):
            j1 = min(n, j0 + block_k)
            if causal and j0 > i1 - 1:
                break  # every later key tile is above the diagonal too
            tiles += 1
            s = scale * (q[i0:i1] @ k[j0:j1].T)
            if causal:
                rows = np.arange(i0, i1)[:, None]
                cols = np.arange(j0, j1)[None, :]
                s = np.where(cols > rows, NEG_INF, s)
            m_new = np.maximum(m, s.max(axis=1))
            m_ref = np.where(np.isneginf(m_new), 0.0, m_new)
            if ablate_rescale:
                corr = np.ones_like(m)
            else:
                corr = np.where(np.isneginf(m), 0.0, np.exp(np.where(np.isneginf(m), 0.0, m) - m_ref))
            p = np.exp(s - m_ref[:, None])
            l = corr * l + p.sum(axis=1)
            acc = corr[:, None] * acc + p @ v[j0:j1]
            m = m_new
            if trace is not None and i0 <= trace_row < i1:
                r = trace_row - i0
                trace.append((j0, float(m[r]), float(l[r]), float(corr[r])))
        o_out[i0:i1] = acc / l[:, None]
        lse_out[i0:i1] = m + np.log(l)
    return o_out, lse_out, {"tiles": tiles, "trace": trace}


def attention_partial(q, k, v, causal, scale, key_lo, key_hi):
    """Attention of every query over the keys key_lo .. key_hi-1 only.

    Returns (O_s, LSE_s): O_s [B,H,N,D] is the output normalised over that key
    range, LSE_s [B,H,N] the natural-log log-sum-exp of the masked scores in
    the range; a row that sees no key of the range (causal, i < key_lo) gets
    O_s = 0 and LSE_s = -inf.  This is the local state a key split produces
    before merging ("CUDA FlashAttention ...", §7).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check4(q, k, v)
    B, H, N, D = q.shape
    o = np.zeros((B, H, N, D))
    lse = np.full((B, H, N), NEG_INF)
    cols = np.arange(key_lo, key_hi)
    if key_hi <= key_lo:
        return o, lse
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h, key_lo:key_hi].T)
            if causal:
                s = np.where(cols[None, :] > np.arange(N)[:, None], NEG_INF, s)
            m = s.max(axis=1)
            seen = np.isfinite(m)
            mm = np.where(seen, m, 0.0)
            e = np.exp(s - mm[:, None])
            l = e.sum(axis=1)
            o[b, h, seen] = (e[seen] / l[seen, None]) @ v[b, h, key_lo:key_hi]
            lse[b, h, seen] = m[seen] + np.log(l[seen])
    return o, lse


def merge_lse(lses, outs):
    """Combine per-split (LSE_s, O_s) pairs (O_s normalised within split s):
    LSE = m + ln sum_s exp(LSE_s - m), O = sum_s exp(LSE_s - LSE) O_s, with
    m = max_s LSE_s; splits with LSE_s = -inf weigh zero.  This is the merge
    of [FA-CUDA] §4 written for normalised partial outputs."""
    lses = [_f64(x) for x in lses]
    m = np.max(np.stack(lses), axis=0)
    mm = np.where(np.isfinite(m), m, 0.0)
    ws = [np.where(np.isneginf(x), 0.0, np.exp(np.where(np.isneginf(x), 0.0, x) - mm)) for x in lses]
    tot = sum(ws)
    lse = np.where(tot > 0, mm + np.log(np.where(tot > 0, tot, 1.0)), NEG_INF)
    o = sum(w[..., None] * _f64(x) for w, x in zip(ws, outs)) / np.where(tot > 0, tot, 1.0)[..., None]
    return o, lse


def causal_tile_count(n, block):
    """Number of (query tile, key tile) pairs a causal tiled pass computes
    when tiles wholly above the diagonal are skipped ([FA-WHY] §4.5),
    counted by enumeration."""
    t = -(-n // block)
    count = 0
    for i in range(t):
        for j in range(t):
            if j * block <= i * block + block - 1:
                count += 1
    return count


def key_tile_words(key_mask, block=64):
    """Block-level flags of a key-padding mask: [FA-MI50] §4.3 asks that a
    padding mask be compressed beforehand into per-block marks, so that the
    block loop branches once per block instead of per element.

    For batch element b and key tile t (keys block*t .. block*t + block-1),
    bit j of words[b][t] is set iff key block*t + j exists (< N) and is
    visible.  A zero word is a tile to skip, an all-ones word one that needs
    no element test.  Returns (words: list of lists of Python ints,
    tiles: for each b, the ascending indices of tiles with a nonzero word).
    Plain loops over the mask, one key at a time.
    """
    m = np.asarray(key_mask)
    B, N = m.shape
    T = -(-N // block)
    words, tiles = [], []
    for b in range(B):
        row_words, row_tiles = [], []
        for t in range(T):
            w = 0
            for j in range(block):
                key = block * t + j
                if key < N and m[b, key] != 0:
                    w |= 1 << j
            row_words.append(w)
            if w != 0:
                row_tiles.append(t)
        words.append(row_words)
        tiles.append(row_tiles)
    return words, tiles


# ---------------------------------------------------------------------------
# Pure-Python brute force for tiny inputs.
# ---------------------------------------------------------------------------
def brute_force_forward(q, k, v, causal, scale, visible=None, keep=None, keep_scale=1.0):
    """Attention of one head with Python floats, math.exp and math.fsum.

    q, k, v: nested sequences [N][D] (N <= 8 expected).  Direct transcription
    of the definition ([FA-CUDA] §1, safe softmax per [FA-WHY] §3.1), no
    numpy.  ``visible``: optional sequence of N truth values; only those keys
    take part.  A row with no key gets O = 0 and LSE = -inf.  ``keep``:
    optional [N][N] truth values of a dropout mask; the probability of a
    dropped pair is zeroed and a kept one multiplied by ``keep_scale`` before
    it weights V (the LSE is unchanged).
    Returns (O as list of lists, LSE as list).
    """
    n = len(q)
    d = len(q[0])
    out, lse = [], []
    for i in range(n):
        keys = [j for j in (range(i + 1) if causal else range(n)) if visible is None or visible[j]]
        if not keys:
            out.append([0.0] * d)
            lse.append(-math.inf)
            continue
        s = [scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = math.fsum(e)
        row = []
        w = [e[idx] * ((keep_scale if keep[i][j] else 0.0) if keep is not None else 1.0)
             for idx, j in enumerate(keys)]
        for t in range(d):
            row.append(math.fsum(w[idx] * v[j][t] for idx, j in enumerate(keys)) / tot)
        out.append(row)
        lse.append(m + math.log(tot))
    return out, lse
