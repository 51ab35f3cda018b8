"""CPU oracle for exact scaled-dot-product attention (float64, numpy).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library; its inputs
are plain float64 arrays decoded from the seeded generator.

What it computes, and where that is defined:

* ``attention`` is the plain definition written out: scores S = scale * Q K^T,
  the causal mask, a max-subtracted row softmax P, then O = P V, one (b, h)
  head at a time, with S and P fully materialised. This is the three-step
  naive attention of "Describe Flash Attention at a high level"
  (mantramindai.in), section "What naive attention does", and of "How
  FlashAttention Speeds Up the Attention Layer" (hassanahmed.net), the
  section on the obvious three-step formulation. The max subtraction is the
  numerical-stability step the hassanahmed.net page describes in its online
  softmax section. It also returns the per-row log-sum-exp
  LSE_i = ln sum_j exp(S_ij), which the pages do not define (reading: natural
  log over the visible keys, in float).
* ``online_attention`` is the streaming recurrence of the mantramindai.in
  page, section "The two ideas", idea 2: every query row keeps a running max,
  running sum and running output; each key block's own (max, sum, output) is
  merged into them, the old sum and output shrinking by exp(m_old - m_new)
  when the max rises, and the output is divided by the sum once at the end.
  Written here as a fold of per-block partials with the same merge rule that
  ``split_decode`` applies to its chunks, vectorised over rows. It is an
  oracle of the algorithm the fused kernel runs, pinned against
  ``attention``.
* ``split_decode`` follows the same page's follow-up on decode (Flash-Decoding):
  one query row, the keys cut into chunks that are processed independently,
  each chunk yielding (max, sum, unnormalised output), and the chunks merged
  with the same max-and-sum rule.
* ``decode`` is the plain definition for one query row per head.
* ``paged_decode`` is ``decode`` over a paged cache: each sequence's keys
  live in fixed-size pages of a shared pool, located through a block table.
  The pages name paged decode kernels as what serving engines use for decode
  ("Describe Flash Attention at a high level", the paragraph on how the
  kernel is reached through frameworks; "flashattention-memory-bound"
  (appliedaiprep.com), the follow-up on long-context serving) but give no
  layout. Reading: pool [num_pages, H, page_size, d]; key j of sequence b is
  row j % page_size of pool page block_table[b, j // page_size], for
  j < seq_lens[b]. The oracle gathers those rows into a contiguous cache and
  applies the plain definition; a sequence of length 0 gives a zero output
  (reading: an idle batch slot).
* ``attention_grad`` is the gradient of the plain definition with respect to
  Q, K and V for an upstream gradient dO, written out from the chain rule
  (dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dP * P)), dQ = scale dS K,
  dK = scale dS^T Q), with P materialised. The pages do not print it: they
  say the backward pass recomputes the score tiles from Q, K and V instead of
  storing P ("Describe Flash Attention at a high level", section "The two
  ideas", item 3; "How FlashAttention Speeds Up the Attention Layer", the
  paragraph on training), and that gradients match standard attention (the
  first page, "Follow-up questions to expect"). It is pinned by central
  finite differences of ``attention`` and by closed forms.

Readings where the pages are silent (also listed in the design notes):
  - scale is a caller argument; the pages write 1/sqrt(d); the oracle rounds
    it to float32 first, as the kernels receive a float32;
  - causal: key j is visible to query i iff j <= i (same N for Q and K);
  - masked logits are -inf before the row max; every row sees key 0.

Pins: every function here is pinned against brute force, closed forms and
invariants: the forward and decode functions by tests/test_oracle.py, the
gradients by tests/test_oracle_grad.py and the paged decode by
tests/test_oracle_paged.py; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np


def _f32(scale: float) -> float:
    """The float32 value the kernels receive for ``scale``, as float64."""
    return float(np.float32(scale))


def _head_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, s: float, rows=None):
    """Naive attention for one head. q: [N,d], k/v: [Nk,d]; rows: optional query-row subset."""
    qi = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    S = s * (q[qi] @ k.T)                                  # scores, [len(qi), Nk]
    if causal:
        S = np.where(np.arange(k.shape[0])[None, :] > qi[:, None], -np.inf, S)
    m = S.max(axis=1, keepdims=True)                       # row max (finite: key 0 is visible)
    P = np.exp(S - m)                                      # exp(-inf) = 0 for masked keys
    l = P.sum(axis=1, keepdims=True)
    P = P / l                                              # softmax
    O = P @ v
    lse = m[:, 0] + np.log(l[:, 0])
    return O, lse, P


def attention(q, k, v, causal: bool, scale: float, rows=None, heads=None):
    """Exact attention by the plain definition.

    q, k, v: float64 arrays [B, H, N, d] (k, v may have Nk rows). Returns
    (O [B,H,len(rows),d], LSE [B,H,len(rows)]), computed one head at a time.
    ``rows`` restricts the query rows (for sampled checks at large N);
    ``heads`` restricts the (b, h) pairs (others are left as NaN).
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, H, N, d = q.shape
    nr = N if rows is None else len(rows)
    O = np.full((B, H, nr, v.shape[-1]), np.nan)
    L = np.full((B, H, nr), np.nan)
    s = _f32(scale)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        O[b, h], L[b, h], _ = _head_attention(q[b, h], k[b, h], v[b, h], causal, s, rows)
    return O, L


def _block_partial(S: np.ndarray, v: np.ndarray):
    """(max, sum, unnormalised output) of one key block for every row.

    S: [rows, keys] scaled scores of the block (-inf where masked); v: [keys, dv].
    m = row max of S; l = sum exp(S - m); o = exp(S - m) V. A row with no
    visible key in the block gives (-inf, 0, 0).
    """
    m = S.max(axis=1)
    finite = np.isfinite(m)
    P = np.exp(S - np.where(finite, m, 0.0)[:, None])      # exp(-inf) = 0 for masked keys
    return m, P.sum(axis=1), P @ v


def _merge(a, b):
    """Merge two (max, sum, unnormalised output) triples over disjoint key sets.

    Both are brought to the larger maximum M: sums and outputs are multiplied
    by exp(m - M) before they are added. A side with m = -inf (no keys)
    contributes nothing.
    """
    (m1, l1, o1), (m2, l2, o2) = a, b
    M = np.maximum(m1, m2)
    w1 = np.where(np.isfinite(m1), np.exp(m1 - np.where(np.isfinite(M), M, 0.0)), 0.0)
    w2 = np.where(np.isfinite(m2), np.exp(m2 - np.where(np.isfinite(M), M, 0.0)), 0.0)
    return M, w1 * l1 + w2 * l2, w1[:, None] * o1 + w2[:, None] * o2


def online_attention(q, k, v, causal: bool, scale: float, block: int):
    """The streaming (online-softmax) recurrence over key blocks, float64, one head.

    q: [N,d], k/v: [Nk,d]. Returns (O, LSE). Every query row carries a
    running state (max m, sum l, unnormalised output acc), starting empty
    (-inf, 0, 0). The keys are visited in blocks of ``block``; each block's own
    (max, sum, output) is merged into the state, which rescales the old sum and
    output by exp(m_old - m_new) when the maximum rises. At the end O = acc / l
    and LSE = m + ln l.
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    s = _f32(scale)
    N, Nk = q.shape[0], k.shape[0]
    rows = np.arange(N)
    state = (np.full(N, -np.inf), np.zeros(N), np.zeros((N, v.shape[1])))
    for start in range(0, Nk, block):
        keys = np.arange(start, min(Nk, start + block))
        S = s * (q @ k[keys].T)
        if causal:
            S = np.where(keys[None, :] > rows[:, None], -np.inf, S)   # keys beyond the row are masked
        state = _merge(state, _block_partial(S, v[keys]))
    m, l, acc = state
    return acc / l[:, None], m + np.log(l)


def decode(q, kc, vc, scale: float | None = None):
    """One query row per head over a whole cache, by the plain definition.

    q: [B,H,d] (or [B,H,1,d]); kc, vc: [B,H,Lkv,d]. Non-causal over the
    cache. scale defaults to 1/sqrt(d) (rounded to float32). Returns
    (o [B,H,d], lse [B,H]).
    """
    q = np.asarray(q, np.float64)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    kc, vc = np.asarray(kc, np.float64), np.asarray(vc, np.float64)
    d = q.shape[-1]
    s = _f32(1.0 / np.sqrt(d) if scale is None else scale)
    B, H = q.shape[:2]
    o = np.empty((B, H, vc.shape[-1]))
    lse = np.empty((B, H))
    for b in range(B):
        for h in range(H):
            O, L, _ = _head_attention(q[b, h][None, :], kc[b, h], vc[b, h], False, s)
            o[b, h], lse[b, h] = O[0], L[0]
    return o, lse


def split_decode(q, kc, vc, nsplit: int, scale: float | None = None):
    """Flash-Decoding for one head: split the keys, reduce each chunk, merge.

    q: [d]; kc, vc: [Lkv, d]. The keys are cut into chunks of
    ceil(Lkv / nsplit) rows (the last chunk shorter; nsplit is first clamped
    to Lkv). Each chunk yields its max m_s, its sum l_s = sum exp(score - m_s)
    and its unnormalised output o_s = sum exp(score - m_s) v. The merge takes
    M = max m_s, weights w_s = exp(m_s - M), L = sum w_s l_s and
    o = sum w_s o_s / L. Returns (o, lse).
    """
    q, kc, vc = (np.asarray(t, np.float64) for t in (q, kc, vc))
    Lkv, d = kc.shape
    s = _f32(1.0 / np.sqrt(d) if scale is None else scale)
    nsplit = max(1, min(nsplit, Lkv))
    chunk = -(-Lkv // nsplit)
    parts = []
    for start in range(0, Lkv, chunk):
        sc = s * (kc[start:start + chunk] @ q)
        m_s = sc.max()
        p = np.exp(sc - m_s)
        parts.append((m_s, p.sum(), p @ vc[start:start + chunk]))
    M = max(p[0] for p in parts)
    w = [np.exp(m_s - M) for m_s, _, _ in parts]
    L = sum(wi * l_s for wi, (_, l_s, _) in zip(w, parts))
    o = sum(wi * o_s for wi, (_, _, o_s) in zip(w, parts)) / L
    return o, M + np.log(L)


def gather_pages(pool, table_row, length: int) -> np.ndarray:
    """Rows 0 .. length-1 of one sequence from a page pool, all heads.

    pool: [num_pages, H, page_size, d]; table_row: the sequence's block-table
    row. Returns [H, length, d]. A page id outside the pool, or a length that
    needs more pages than the row holds, raises ValueError.
    """
    num_pages, H, ps, d = pool.shape
    n_used = -(-length // ps)
    if n_used > len(table_row):
        raise ValueError(f"length {length} needs {n_used} pages, the block table holds {len(table_row)}")
    out = np.empty((H, length, d), dtype=pool.dtype)
    for i in range(n_used):
        page = int(table_row[i])
        if not 0 <= page < num_pages:
            raise ValueError(f"page id {page} outside the pool of {num_pages} pages")
        rows = min(ps, length - i * ps)                    # the last page may be partly filled
        out[:, i * ps:i * ps + rows] = pool[page, :, :rows]
    return out


def paged_decode(q, k_pages, v_pages, block_table, seq_lens, scale: float | None = None):
    """One query row per head over a paged cache: gather, then ``decode``.

    q: [B,H,d]; k_pages, v_pages: [num_pages, H, page_size, d];
    block_table: [B, max_pages] integers; seq_lens: [B]. Returns
    (o [B,H,d], lse [B,H]); a sequence of length 0 gives o = 0 and
    lse = -inf.
    """
    q = np.asarray(q, np.float64)
    B, H, d = q.shape
    o = np.zeros((B, H, np.shape(v_pages)[-1]))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        length = int(seq_lens[b])
        if length < 0:
            raise ValueError(f"negative sequence length {length}")
        if length == 0:
            continue
        kc = gather_pages(k_pages, block_table[b], length)
        vc = gather_pages(v_pages, block_table[b], length)
        o[b:b + 1], lse[b:b + 1] = decode(q[b:b + 1], np.asarray(kc, np.float64)[None],
                                          np.asarray(vc, np.float64)[None], scale)
    return o, lse


def _head_attention_grad(q, k, v, do, causal: bool, s: float):
    """Gradients of O = softmax(s Q K^T [+ mask]) V for one head, given dO = dL/dO.

    q: [N,d]; k, v: [Nk,d]; do: [N,dv]. Returns (dQ, dK, dV).
    """
    _, _, P = _head_attention(q, k, v, causal, s)
    dV = P.T @ do                                          # O = P V
    dP = do @ v.T
    D = np.sum(dP * P, axis=1, keepdims=True)               # rowsum(dP * P) = rowsum(dO * O)
    dS = P * (dP - D)                                       # softmax Jacobian applied row by row
    dQ = s * (dS @ k)                                       # S = s Q K^T
    dK = s * (dS.T @ q)
    return dQ, dK, dV


def attention_grad(q, k, v, do, causal: bool, scale: float, heads=None):
    """Exact gradients of attention w.r.t. Q, K, V (float64), one head at a time.

    q, k, v, do: [B, H, N, d]. Returns (dQ, dK, dV) with the shapes of q, k,
    v; heads outside ``heads`` are left as NaN.
    """
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    B, H = q.shape[:2]
    dQ, dK, dV = np.full(q.shape, np.nan), np.full(k.shape, np.nan), np.full(v.shape, np.nan)
    s = _f32(scale)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        dQ[b, h], dK[b, h], dV[b, h] = _head_attention_grad(q[b, h], k[b, h], v[b, h], do[b, h], causal, s)
    return dQ, dK, dV


def naive_workspace_bytes(B: int, H: int, N: int, elem_bytes: int) -> int:
    """Bytes of one materialised N x N score (or probability) matrix for all heads."""
    return B * H * N * N * elem_bytes


def attention_flops(B: int, H: int, N: int, d: int, causal: bool) -> int:
    """Algorithmic forward FLOPs: 4*d per visible (query, key) pair (QK^T and PV)."""
    pairs = N * (N + 1) // 2 if causal else N * N
    return 4 * d * B * H * pairs
