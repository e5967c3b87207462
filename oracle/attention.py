"""Plain fp64 CPU oracle of exact scaled dot-product attention.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the bench's
CPU-baseline leg, never by the library or its Python binding.

What it computes (the "standard attention" data flow of [P1] section 1 and
the three steps of [P3] "Core idea"):

    S = scale * Q K^T                     one N x N matrix per (batch, head)
    S[i, j] = -inf for j > i              only when causal (reading below)
    P = softmax(S) row by row             three passes: max, sum of exps, divide
    O = P V
    LSE[i] = m[i] + ln(l[i])              natural-log logsumexp of row i of S

and, for training, the exact gradient of that definition (the pages give no
backward formula, only that it recomputes from saved statistics: [P2] "Core
mechanism", [P3] "A surprise"):

    dV = P^T dO
    dP = dO V^T
    delta[i] = sum_j P[i, j] dP[i, j]     taken from the materialised P
    dS = P * (dP - delta)                 softmax Jacobian applied row by row
    dQ = scale * dS K
    dK = scale * dS^T Q

Readings where the pages leave a step open:
  * Causal means a query sees keys at its own position and before it
    (diagonal included); with equal query and key lengths no row is empty.
    [P3] "Pitfalls", second pitfall.
  * LSE is stored in natural log; the GPU may use log2 internally.
  * Inputs arrive as fp64 arrays that already hold the values the GPU sees
    (rounded to the run's dtype); every step here is fp64.

Everything materialises S and P (in query-row chunks, whole rows at a time)
so that a reader can check each line against the definition by eye. No
blocking over keys, fusion or reordering happens here except in
`attention_forward_online`, which exists to restate [P1] section 2's
blockwise algorithm for the "online equals three-pass" invariant.
"""

import numpy as np

from oracle import rng as _rng

# Query rows handled per chunk: bounds the materialised S/P to
# ROW_CHUNK x N fp64 values per (batch, head) without changing any result
# (each query row is computed on its own).
ROW_CHUNK = 1024


def _check(q, k, v):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, D] shape")
    return q, k, v


def _scores(q_rows, k_all, scale, row0, causal):
    """S = scale * Q K^T for query rows row0.. of one head, masked if causal.

    [P3] "Core idea", step 1; causal exclusion as read above.
    """
    s = scale * (q_rows @ k_all.T)
    if causal:
        n_rows, n_keys = s.shape
        qi = row0 + np.arange(n_rows)[:, None]
        kj = np.arange(n_keys)[None, :]
        s = np.where(kj > qi, -np.inf, s)
    return s


def attention_probabilities(q, k, scale, causal):
    """P = softmax(scale * Q K^T [+ causal mask]) for one head, three-pass.

    The three passes of [P1] section 2's first paragraph: row max for
    stability, sum of exponentials, then the division. q, k: [N, D].
    Returns (P, m, l) with m the row max of S and l the row sum of exp(S - m).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = _scores(q, k, scale, 0, causal)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, m[:, 0], l[:, 0]


def attention_forward(q, k, v, scale, causal):
    """O and LSE of exact attention, materialising S and P (fp64).

    q, k, v: [B, H, N, D]. Returns (O [B, H, N, D], LSE [B, H, N]).
    [P1] section 1 (standard data flow), [P3] "Core idea" steps 1-3.
    """
    q, k, v = _check(q, k, v)
    B, H, N, D = q.shape
    o = np.empty((B, H, N, D), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, ROW_CHUNK):
                r1 = min(N, r0 + ROW_CHUNK)
                s = _scores(q[b, h, r0:r1], k[b, h], scale, r0, causal)
                m = s.max(axis=1, keepdims=True)          # pass 1: row max
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)           # pass 2: sum of exps
                p = e / l                                  # pass 3: divide
                o[b, h, r0:r1] = p @ v[b, h]
                lse[b, h, r0:r1] = m[:, 0] + np.log(l[:, 0])
    return o, lse


def attention_forward_online(q, k, v, scale, causal, block):
    """Blockwise online-softmax attention over key blocks (fp64).

    Restates the algorithm of [P1] section 2: keep, per query row, a running
    maximum (starting at -inf), a running sum (starting at 0) and an
    unnormalised output (starting at 0). For each block of `block` keys:
    scores of all queries against the block; new maximum = larger of the old
    one and the block's row maximum; correction = exp(old max - new max);
    block weights = exp(scores - new max); running sum = correction * sum +
    row sum of the weights; output = correction * output + weights @ V_block.
    After the last block the output is divided by the running sum. The
    pages' sketch returns no LSE; here LSE = final max + ln(final sum).

    A row whose maximum is still -inf (every key so far masked) has nothing
    to correct: its correction is taken as 0 instead of exp(-inf + inf).
    """
    q, k, v = _check(q, k, v)
    B, H, N, D = q.shape
    if block < 1:
        raise ValueError("block must be >= 1")
    o_out = np.empty((B, H, N, D), dtype=np.float64)
    lse_out = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            run_max = np.full((N, 1), -np.inf)
            run_sum = np.zeros((N, 1))
            acc = np.zeros((N, D))
            for j0 in range(0, N, block):
                j1 = min(N, j0 + block)
                s = scale * (q[b, h] @ k[b, h, j0:j1].T)
                if causal:
                    qi = np.arange(N)[:, None]
                    kj = j0 + np.arange(j1 - j0)[None, :]
                    s = np.where(kj > qi, -np.inf, s)
                m_prev = run_max
                m_curr = s.max(axis=1, keepdims=True)
                run_max = np.maximum(m_prev, m_curr)
                with np.errstate(invalid="ignore"):
                    corr = np.where(np.isneginf(run_max), 0.0,
                                    np.exp(m_prev - run_max))
                    p = np.where(np.isneginf(run_max), 0.0,
                                 np.exp(s - run_max))
                run_sum = corr * run_sum + p.sum(axis=1, keepdims=True)
                acc = corr * acc + p @ v[b, h, j0:j1]
            o_out[b, h] = acc / run_sum
            lse_out[b, h] = run_max[:, 0] + np.log(run_sum[:, 0])
    return o_out, lse_out


def attention_backward(q, k, v, do, scale, causal):
    """dQ, dK, dV of exact attention for upstream gradient dO (fp64).

    The exact gradient of attention_forward: P is materialised from its
    definition (not from a saved LSE), then
        dV = P^T dO, dP = dO V^T, delta = rowsum(P * dP),
        dS = P * (dP - delta), dQ = scale * dS K, dK = scale * dS^T Q.
    The pages only say the backward recomputes local blocks from saved
    statistics ([P2] "Core mechanism"; [P3] "A surprise"); these formulas
    are the chain rule through softmax, not taken from the pages.
    """
    q, k, v = _check(q, k, v)
    do = np.asarray(do, dtype=np.float64)
    if do.shape != q.shape:
        raise ValueError("do must have q's shape")
    B, H, N, D = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(q)
    dv = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, ROW_CHUNK):
                r1 = min(N, r0 + ROW_CHUNK)
                s = _scores(q[b, h, r0:r1], k[b, h], scale, r0, causal)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                p = e / e.sum(axis=1, keepdims=True)
                g = do[b, h, r0:r1]
                dv[b, h] += p.T @ g
                dp = g @ v[b, h].T
                delta = (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - delta)
                dq[b, h, r0:r1] = scale * (ds @ k[b, h])
                dk[b, h] += scale * (ds.T @ q[b, h, r0:r1])
    return dq, dk, dv


def attention_forward_varlen(q, k, v, cu_seqlens, scale, causal):
    """Packed variable-length batch with grouped K/V heads (fp64).

    The deployment variants named by the "Flash Attention algorithm design
    and I/O optimisation" page (variable-length batches, shared K/V heads):
    sequence b is tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of the packed
    tensors and attends only within itself; query head h reads K/V head
    h // (H // H_kv). Each (sequence, head) is exact attention, computed by
    attention_forward on that sequence's rows.

    q: [total, H, D]; k, v: [total, H_kv, D]. Returns O [total, H, D] and
    LSE [H, total]; tokens outside every sequence stay NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu = [int(x) for x in cu_seqlens]
    total, H, D = q.shape
    H_kv = k.shape[1]
    if k.shape != (total, H_kv, D) or v.shape != k.shape or H % H_kv != 0:
        raise ValueError("need q [total, H, D] and k, v [total, H_kv, D] with H_kv | H")
    group = H // H_kv
    o = np.full((total, H, D), np.nan)
    lse = np.full((H, total), np.nan)
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        if s1 <= s0:
            continue
        for h in range(H):
            hk = h // group
            ob, lb = attention_forward(q[None, None, s0:s1, h], k[None, None, s0:s1, hk],
                                       v[None, None, s0:s1, hk], scale, causal)
            o[s0:s1, h] = ob[0, 0]
            lse[h, s0:s1] = lb[0, 0]
    return o, lse


def attention_decode(q, k_cache, v_cache, cache_seqlens, scale):
    """Attention of new tokens against a key/value cache (fp64).

    The decode case of the "Flash Attention algorithm design and I/O
    optimisation" page ("Training and inference value": each step brings
    only new tokens but reads the whole, growing cache). Sequence b's cache
    holds L_b = cache_seqlens[b] tokens, of which its s_q new tokens are the
    last s_q; new token t (0-based) sits at position L_b - s_q + t and, by
    the causal rule, sees cache keys 0 .. L_b - s_q + t. Query head h reads
    K/V head h // (H // H_kv). A row that sees no key (L_b < s_q - t) gets
    O = 0 and LSE = -inf. Each visible row is exact attention over its keys:
    scores, max, exponentials, their sum, division, then P V.

    q: [B, s_q, H, D]; k_cache, v_cache: [B, cap, H_kv, D]; cache_seqlens:
    B integers in [0, cap]. Returns O [B, s_q, H, D] and LSE [B, H, s_q].
    """
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    B, s_q, H, D = q.shape
    cap, H_kv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, cap, H_kv, D) or v_cache.shape != k_cache.shape or H % H_kv:
        raise ValueError("need q [B, s_q, H, D] and caches [B, cap, H_kv, D] with H_kv | H")
    group = H // H_kv
    o = np.zeros((B, s_q, H, D))
    lse = np.full((B, H, s_q), -np.inf)
    for b in range(B):
        L = int(cache_seqlens[b])
        if not 0 <= L <= cap:
            raise ValueError("cache_seqlens outside [0, cap]")
        for t in range(s_q):
            n = min(L, L - s_q + t + 1)  # keys 0 .. L - s_q + t
            if n <= 0:
                continue
            for h in range(H):
                hk = h // group
                s = scale * (k_cache[b, :n, hk] @ q[b, t, h])
                m = s.max()
                e = np.exp(s - m)
                l = e.sum()
                o[b, t, h] = (e / l) @ v_cache[b, :n, hk]
                lse[b, h, t] = m + np.log(l)
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Exact attention over a union of disjoint key sets from the results
    over each set: the rescale-and-add of the online softmax ("From
    Self-Attention to FlashAttention", section 2) applied once per part.

    With LSE_s = ln sum_{j in set s} exp(score_j) and O_s the attention over
    set s, the whole has LSE = ln sum_s exp(LSE_s) and
    O = sum_s exp(LSE_s - LSE) O_s. Parts with LSE_s = -inf (empty sets)
    carry no weight; if every part is empty the result is O = 0, LSE = -inf.

    o_parts: [S, ..., D]; lse_parts: [S, ...]. Returns (O [..., D], LSE [...]).
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_parts - safe_m)                   # exp(-inf) = 0 for empty parts
    total = w.sum(axis=0)
    lse = np.where(total > 0, safe_m + np.log(np.where(total > 0, total, 1.0)), -np.inf)
    o = np.where((total > 0)[..., None],
                 (w[..., None] * o_parts).sum(axis=0) / np.where(total > 0, total, 1.0)[..., None],
                 0.0)
    return o, lse


def attention_forward_dropout(q, k, v, scale, causal, p, seed, offset, bh0=0):
    """Exact attention with dropout on the probabilities (fp64).

    The dropout branch that the verification answer of "Flash Attention
    algorithm design and I/O optimisation" asks to cover, read as the usual
    attention dropout: P is the softmax of the scores as in
    attention_forward (so LSE is unchanged), each probability is kept or
    dropped by the counter-based bits of oracle.rng.keep_mask, and
        O = (P * keep) V / (1 - p_eff),   p_eff = dropout_threshold(p) / 256.

    q, k, v: [B, H, N, D]; bh0 is the flattened (batch, head) index of the
    first head given (its random bits are those of head bh0 + b * H + h), so
    that one head of a larger batch can be checked on its own. Returns
    (O, LSE).
    """
    q, k, v = _check(q, k, v)
    B, H, N, D = q.shape
    inv_keep = 1.0 / (1.0 - _rng.dropout_threshold(p) / 256.0)
    o = np.empty((B, H, N, D))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, ROW_CHUNK):
                r1 = min(N, r0 + ROW_CHUNK)
                s = _scores(q[b, h, r0:r1], k[b, h], scale, r0, causal)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                prob = e / l
                keep = _rng.keep_mask(bh0 + b * H + h, np.arange(r0, r1), np.arange(N), p, seed, offset)
                o[b, h, r0:r1] = (np.where(keep, prob, 0.0) @ v[b, h]) * inv_keep
                lse[b, h, r0:r1] = m[:, 0] + np.log(l[:, 0])
    return o, lse


def attention_backward_dropout(q, k, v, do, scale, causal, p, seed, offset, bh0=0):
    """dQ, dK, dV of attention_forward_dropout for upstream gradient dO (fp64).

    With the keep decisions fixed, the forward is a smooth function of
    Q, K, V; its exact gradient is the chain rule through the scaled mask
    and the softmax:
        Pd = P * keep / (1 - p_eff),  dV = Pd^T dO,
        dP = (dO V^T) * keep / (1 - p_eff),  delta = rowsum(P * dP),
        dS = P * (dP - delta),  dQ = scale * dS K,  dK = scale * dS^T Q.
    bh0 as for attention_forward_dropout.
    """
    q, k, v = _check(q, k, v)
    do = np.asarray(do, dtype=np.float64)
    if do.shape != q.shape:
        raise ValueError("do must have q's shape")
    B, H, N, D = q.shape
    inv_keep = 1.0 / (1.0 - _rng.dropout_threshold(p) / 256.0)
    dq = np.zeros_like(q)
    dk = np.zeros_like(q)
    dv = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, ROW_CHUNK):
                r1 = min(N, r0 + ROW_CHUNK)
                s = _scores(q[b, h, r0:r1], k[b, h], scale, r0, causal)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                prob = e / e.sum(axis=1, keepdims=True)
                keep = _rng.keep_mask(bh0 + b * H + h, np.arange(r0, r1), np.arange(N), p, seed, offset)
                scale_keep = np.where(keep, inv_keep, 0.0)
                g = do[b, h, r0:r1]
                dv[b, h] += (prob * scale_keep).T @ g
                dp = (g @ v[b, h].T) * scale_keep
                delta = (prob * dp).sum(axis=1, keepdims=True)
                ds = prob * (dp - delta)
                dq[b, h, r0:r1] = scale * (ds @ k[b, h])
                dk[b, h] += scale * (ds.T @ q[b, h, r0:r1])
    return dq, dk, dv


def attention_backward_varlen(q, k, v, do, cu_seqlens, scale, causal):
    """dQ, dK, dV of attention_forward_varlen for upstream gradient dO (fp64).

    Each (sequence, query head) is its own attention problem, so its
    gradients are those of attention_backward on that sequence's rows; a K/V
    head serves the query heads h with h // (H // H_kv) equal to it, so its
    dK and dV are the sums of their contributions (the chain rule through the
    shared operand).

    q, do: [total, H, D]; k, v: [total, H_kv, D]. Returns dq [total, H, D],
    dk and dv [total, H_kv, D]; tokens outside every sequence get zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    cu = [int(x) for x in cu_seqlens]
    total, H, D = q.shape
    H_kv = k.shape[1]
    if k.shape != (total, H_kv, D) or v.shape != k.shape or do.shape != q.shape or H % H_kv:
        raise ValueError("need q, do [total, H, D] and k, v [total, H_kv, D] with H_kv | H")
    group = H // H_kv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        if s1 <= s0:
            continue
        for h in range(H):
            hk = h // group
            gq, gk, gv = attention_backward(q[None, None, s0:s1, h], k[None, None, s0:s1, hk],
                                            v[None, None, s0:s1, hk], do[None, None, s0:s1, h],
                                            scale, causal)
            dq[s0:s1, h] = gq[0, 0]
            dk[s0:s1, hk] += gk[0, 0]
            dv[s0:s1, hk] += gv[0, 0]
    return dq, dk, dv
