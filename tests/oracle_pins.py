"""Pins that tie the CPU oracle to facts fixed outside the oracle itself.

Each pin takes an oracle module (normally `oracle.attention`; the mutation
test hands in deliberately broken copies) and raises AssertionError when the
oracle disagrees with:
  * hand-derived exact examples (tests/golden/hand_examples.txt);
  * closed forms (scale = 0, N = 1, constant V, causal row 0);
  * invariants of the definition (rows of P sum to 1, permutations,
    sum of dV equals sum of dO, columns of dK sum to zero);
  * an independent scalar brute force over tiny inputs;
  * torch's fp64 CPU scaled_dot_product_attention and autograd (library
    routines for the same definition);
  * central finite differences of the forward (for the backward).
"""

import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "hand_examples.txt")


# ---------------------------------------------------------------- fixtures

def _eval(expr):
    return float(eval(expr, {"__builtins__": {}}, {"ln": math.log}))  # noqa: S307


def load_golden():
    """Parse the hand-derived examples into {name: {key: ndarray}}."""
    out, cur = {}, None
    with open(GOLDEN) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = line[1:-1]
                out[cur] = {}
                continue
            key, expr = (s.strip() for s in line.split("=", 1))
            rows = [[_eval(x) for x in r.split(",")] for r in expr.split(";")]
            out[cur][key] = np.array(rows, dtype=np.float64)
    return out


def _as_bhnd(x):
    """[N, D] -> [1, 1, N, D]."""
    return np.asarray(x, dtype=np.float64)[None, None]


def _rand(shape, seed, mult=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mult


# ---------------------------------------------------------------- brute force

def brute_force(q, k, v, scale, causal):
    """Scalar loops over one head; keys a query may see are enumerated
    instead of masked. q, k, v: nested lists [N][D]."""
    n, d = len(q), len(q[0])
    o, lse = [], []
    for i in range(n):
        keys = list(range(i + 1)) if causal else list(range(n))
        s = [scale * sum(q[i][t] * k[j][t] for t in range(d)) for j in keys]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        tot = sum(w)
        o.append([sum(w[a] * v[j][t] for a, j in enumerate(keys)) / tot
                  for t in range(d)])
        lse.append(m + math.log(tot))
    return o, lse


# ---------------------------------------------------------------- forward pins

def pin_golden_forward(orc):
    for name, ex in load_golden().items():
        q, k, v = (_as_bhnd(ex[x]) for x in ("q", "k", "v"))
        scale = float(ex["scale"][0, 0])
        for causal, tag in ((False, "full"), (True, "causal")):
            o, lse = orc.attention_forward(q, k, v, scale, causal)
            np.testing.assert_allclose(o[0, 0], ex["o_" + tag], atol=1e-14,
                                       err_msg=f"golden {name} o_{tag}")
            np.testing.assert_allclose(lse[0, 0], ex["lse_" + tag][:, 0], atol=1e-14,
                                       err_msg=f"golden {name} lse_{tag}")


def pin_brute_force(orc):
    for seed, (n, d) in enumerate([(1, 1), (2, 3), (5, 4), (8, 2), (7, 3)]):
        q, k, v = (_rand((1, 2, n, d), 100 + 3 * seed + t) for t in range(3))
        scale = 0.7
        for causal in (False, True):
            o, lse = orc.attention_forward(q, k, v, scale, causal)
            for h in range(2):
                bo, bl = brute_force(q[0, h].tolist(), k[0, h].tolist(),
                                     v[0, h].tolist(), scale, causal)
                np.testing.assert_allclose(o[0, h], np.array(bo), atol=1e-13, rtol=0)
                np.testing.assert_allclose(lse[0, h], np.array(bl), atol=1e-13, rtol=0)


def pin_online_equals_three_pass(orc):
    """[P1] section 2: the blockwise online result equals three-pass softmax."""
    q, k, v = (_rand((1, 2, 150, 16), 7 + t) for t in range(3))
    for causal in (False, True):
        o3, l3 = orc.attention_forward(q, k, v, 0.25, causal)
        for block in (1, 7, 128, 150, 1000):
            oo, lo = orc.attention_forward_online(q, k, v, 0.25, causal, block)
            np.testing.assert_allclose(oo, o3, atol=1e-12, rtol=0)
            np.testing.assert_allclose(lo, l3, atol=1e-12, rtol=0)


def pin_rows_sum_to_one(orc):
    q, k = (_rand((33, 8), 11 + t) for t in range(2))
    for causal in (False, True):
        p, m, l = orc.attention_probabilities(q, k, 0.5, causal)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14, rtol=0)
        if causal:
            assert np.all(np.triu(p, 1) == 0.0)
        s = 0.5 * q @ k.T
        if causal:
            s = np.where(np.triu(np.ones_like(s), 1) > 0, -np.inf, s)
        np.testing.assert_allclose(m, s.max(axis=1), atol=0, rtol=0)


def pin_constant_v(orc):
    q, k = (_rand((2, 3, 40, 8), 21 + t) for t in range(2))
    c = _rand((8,), 23)
    v = np.broadcast_to(c, (2, 3, 40, 8)).copy()
    for causal in (False, True):
        o, _ = orc.attention_forward(q, k, v, 0.3, causal)
        np.testing.assert_allclose(o, v, atol=1e-14, rtol=1e-14)


def pin_causal_row0(orc):
    q, k, v = (_rand((1, 2, 17, 5), 31 + t) for t in range(3))
    o, lse = orc.attention_forward(q, k, v, 0.9, True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.9 * (q[:, :, 0] * k[:, :, 0]).sum(-1),
                               atol=1e-14, rtol=0)


def pin_scale_zero(orc):
    """scale = 0: uniform weights over the visible keys."""
    n = 23
    q, k, v = (_rand((1, 2, n, 6), 41 + t) for t in range(3))
    o, lse = orc.attention_forward(q, k, v, 0.0, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape),
                               atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse, np.log(n), atol=1e-14, rtol=0)
    o, lse = orc.attention_forward(q, k, v, 0.0, True)
    cum = np.cumsum(v, axis=2) / np.arange(1, n + 1)[None, None, :, None]
    np.testing.assert_allclose(o, cum, atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, n + 1)), lse.shape),
                               atol=1e-14, rtol=0)


def pin_single_key(orc):
    """N = 1: the only weight is 1 and LSE is the single score."""
    q, k, v = (_rand((2, 3, 1, 7), 51 + t) for t in range(3))
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, 1.3, causal)
        np.testing.assert_array_equal(o, v)
        np.testing.assert_allclose(lse, 1.3 * (q * k).sum(-1)[..., 0][..., None],
                                   atol=1e-14, rtol=0)


def pin_permutations(orc):
    """Non-causal: permuting keys with their values changes nothing;
    permuting queries permutes the rows of O and LSE."""
    q, k, v = (_rand((1, 1, 29, 8), 61 + t) for t in range(3))
    o, lse = orc.attention_forward(q, k, v, 0.4, False)
    perm = np.random.default_rng(5).permutation(29)
    o2, lse2 = orc.attention_forward(q, k[:, :, perm], v[:, :, perm], 0.4, False)
    np.testing.assert_allclose(o2, o, atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-14, rtol=0)
    o3, lse3 = orc.attention_forward(q[:, :, perm], k, v, 0.4, False)
    np.testing.assert_allclose(o3, o[:, :, perm], atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse3, lse[:, :, perm], atol=1e-14, rtol=0)


def pin_torch_sdpa(orc):
    """torch's fp64 CPU scaled_dot_product_attention and logsumexp."""
    q, k, v = (_rand((2, 3, 70, 16), 71 + t) for t in range(3))
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, 0.21, causal)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=0.21).numpy()
        np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)
        s = 0.21 * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.ones(70, 70, dtype=torch.bool).triu(1), -math.inf)
        np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12, rtol=0)


def pin_row_chunking(orc):
    """Results do not depend on the row-chunk size used to bound memory."""
    q, k, v = (_rand((1, 1, 37, 4), 81 + t) for t in range(3))
    old = orc.ROW_CHUNK
    try:
        orc.ROW_CHUNK = 1024
        o_a, l_a = orc.attention_forward(q, k, v, 0.5, True)
        g_a = orc.attention_backward(q, k, v, v[:, :, ::-1].copy(), 0.5, True)
        orc.ROW_CHUNK = 5
        o_b, l_b = orc.attention_forward(q, k, v, 0.5, True)
        g_b = orc.attention_backward(q, k, v, v[:, :, ::-1].copy(), 0.5, True)
    finally:
        orc.ROW_CHUNK = old
    np.testing.assert_allclose(o_b, o_a, atol=1e-15, rtol=0)
    np.testing.assert_allclose(l_b, l_a, atol=1e-15, rtol=0)
    for a, b in zip(g_a, g_b):
        np.testing.assert_allclose(b, a, atol=1e-14, rtol=0)


# ---------------------------------------------------------------- backward pins

def pin_golden_backward(orc):
    ex = load_golden()
    a = ex["A"]
    dq, dk, dv = orc.attention_backward(*(_as_bhnd(a[x]) for x in ("q", "k", "v", "do")),
                                        float(a["scale"][0, 0]), True)
    np.testing.assert_allclose(dq[0, 0], a["dq_causal"], atol=1e-14)
    np.testing.assert_allclose(dk[0, 0], a["dk_causal"], atol=1e-14)
    np.testing.assert_allclose(dv[0, 0], a["dv_causal"], atol=1e-14)
    b = ex["B"]
    dq, dk, dv = orc.attention_backward(*(_as_bhnd(b[x]) for x in ("q", "k", "v", "do")),
                                        float(b["scale"][0, 0]), False)
    np.testing.assert_allclose(dq[0, 0], b["dq_full"], atol=1e-14)
    np.testing.assert_allclose(dk[0, 0], b["dk_full"], atol=1e-14)
    np.testing.assert_allclose(dv[0, 0], b["dv_full"], atol=1e-14)


def pin_finite_differences(orc):
    """Central differences of L = sum(O * dO) match dQ, dK, dV."""
    h = 1e-6
    for causal in (False, True):
        q, k, v, do = (_rand((1, 2, 5, 3), 91 + t) for t in range(4))
        grads = orc.attention_backward(q, k, v, do, 0.8, causal)
        for which in range(3):
            base = [q, k, v]
            num = np.zeros_like(q)
            it = np.nditer(q, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                plus = [x.copy() for x in base]
                minus = [x.copy() for x in base]
                plus[which][idx] += h
                minus[which][idx] -= h
                lp = (orc.attention_forward(*plus, 0.8, causal)[0] * do).sum()
                lm = (orc.attention_forward(*minus, 0.8, causal)[0] * do).sum()
                num[idx] = (lp - lm) / (2 * h)
            err = np.abs(grads[which] - num).max() / max(1.0, np.abs(num).max())
            assert err < 1e-7, (causal, which, err)


def pin_grad_sums(orc):
    """sum_j dV_j = sum_i dO_i (rows of P sum to 1); sum_j dK_j = 0 (rows
    of dS sum to 0)."""
    q, k, v, do = (_rand((2, 2, 31, 6), 101 + t) for t in range(4))
    for causal in (False, True):
        dq, dk, dv = orc.attention_backward(q, k, v, do, 0.6, causal)
        np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12, rtol=0)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12, rtol=0)


def pin_constant_v_grads(orc):
    q, k, do = (_rand((1, 2, 19, 4), 111 + t) for t in range(3))
    v = np.broadcast_to(_rand((4,), 114), q.shape).copy()
    for causal in (False, True):
        dq, dk, dv = orc.attention_backward(q, k, v, do, 0.6, causal)
        np.testing.assert_allclose(dq, 0.0, atol=1e-13)
        np.testing.assert_allclose(dk, 0.0, atol=1e-13)


def pin_scale_zero_grads(orc):
    """scale = 0, causal: dQ = dK = 0 and dV_j = sum_{i >= j} dO_i / (i + 1)."""
    n = 13
    q, k, v, do = (_rand((1, 2, n, 3), 121 + t) for t in range(4))
    dq, dk, dv = orc.attention_backward(q, k, v, do, 0.0, True)
    np.testing.assert_array_equal(dq, 0.0)
    np.testing.assert_array_equal(dk, 0.0)
    w = do / np.arange(1, n + 1)[None, None, :, None]
    expect = np.flip(np.cumsum(np.flip(w, axis=2), axis=2), axis=2)
    np.testing.assert_allclose(dv, expect, atol=1e-14, rtol=0)


def pin_delta_two_ways(orc):
    """rowsum(P * dP) equals rowsum(dO * O), the form a fused backward uses."""
    q, k, v, do = (_rand((45, 8), 131 + t) for t in range(4))
    for causal in (False, True):
        p, _, _ = orc.attention_probabilities(q, k, 0.35, causal)
        o, _ = orc.attention_forward(_as_bhnd(q), _as_bhnd(k), _as_bhnd(v), 0.35, causal)
        a = (p * (do @ v.T)).sum(axis=1)
        b = (do * o[0, 0]).sum(axis=1)
        np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)


def pin_torch_autograd(orc):
    q, k, v, do = (_rand((1, 2, 40, 8), 141 + t) for t in range(4))
    for causal in (False, True):
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=0.45)
        out.backward(torch.from_numpy(do))
        got = orc.attention_backward(q, k, v, do, 0.45, causal)
        for g, t in zip(got, (tq, tk, tv)):
            np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-12, rtol=0)


# ---------------------------------------------------------------- packed / grouped

def brute_force_varlen(q, k, v, cu, scale, causal):
    """Scalar loops over a packed batch: sequence b is tokens cu[b]..cu[b+1]-1,
    query head h uses K/V head h // (H // H_kv). q: [total][H][D] nested lists."""
    total, H, D = len(q), len(q[0]), len(q[0][0])
    group = H // len(k[0])
    o = [[[math.nan] * D for _ in range(H)] for _ in range(total)]
    lse = [[math.nan] * total for _ in range(H)]
    for b in range(len(cu) - 1):
        for h in range(H):
            hk = h // group
            for i in range(cu[b], cu[b + 1]):
                keys = range(cu[b], i + 1) if causal else range(cu[b], cu[b + 1])
                s = [scale * sum(q[i][h][t] * k[j][hk][t] for t in range(D)) for j in keys]
                m = max(s)
                wts = [math.exp(x - m) for x in s]
                tot = sum(wts)
                for t in range(D):
                    o[i][h][t] = sum(wt * v[j][hk][t] for wt, j in zip(wts, keys)) / tot
                lse[h][i] = m + math.log(tot)
    return o, lse


def pin_varlen_brute_force(orc):
    """Packed sequences with shared K/V heads against independent scalar loops
    (lengths 3, 1, 0, 5; H = 4 over H_kv = 2, and MQA H_kv = 1)."""
    cu = [0, 3, 4, 4, 9]
    for H_kv in (2, 1):
        q = _rand((9, 4, 3), 31)
        k = _rand((9, H_kv, 3), 32)
        v = _rand((9, H_kv, 3), 33)
        for causal in (False, True):
            o, lse = orc.attention_forward_varlen(q, k, v, cu, 0.7, causal)
            bo, bl = brute_force_varlen(q.tolist(), k.tolist(), v.tolist(), cu, 0.7, causal)
            np.testing.assert_allclose(o, np.array(bo), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-12)


def pin_varlen_sequences_independent(orc):
    """Changing the tokens of one sequence leaves every other sequence's
    outputs unchanged, and reordering the sequences in the pack moves their
    outputs with them."""
    cu = [0, 5, 7, 13]
    q, k, v = (_rand((13, 2, 4), s) for s in (41, 42, 43))
    o, lse = orc.attention_forward_varlen(q, k, v, cu, 0.5, True)
    k2 = k.copy()
    k2[5:7] += _rand((2, 2, 4), 44)
    o2, _ = orc.attention_forward_varlen(q, k2, v, cu, 0.5, True)
    np.testing.assert_array_equal(o2[:5], o[:5])
    np.testing.assert_array_equal(o2[7:], o[7:])
    assert np.abs(o2[5:7] - o[5:7]).max() > 1e-3
    perm = list(range(7, 13)) + list(range(0, 5)) + list(range(5, 7))
    o3, lse3 = orc.attention_forward_varlen(q[perm], k[perm], v[perm], [0, 6, 11, 13], 0.5, True)
    np.testing.assert_allclose(o3, o[perm], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse3, lse[:, perm], rtol=0, atol=1e-12)


VARLEN_PINS = [pin_varlen_brute_force, pin_varlen_sequences_independent]

def pin_varlen_backward_finite_differences(orc):
    """The packed, grouped-head backward against central differences of the
    packed forward (lengths 3, 0, 4; H = 4 over H_kv = 2 and MQA H_kv = 1)."""
    cu = [0, 3, 3, 7]
    for H_kv in (2, 1):
        q = _rand((7, 4, 2), 101)
        k = _rand((7, H_kv, 2), 102 + H_kv)
        v = _rand((7, H_kv, 2), 104 + H_kv)
        g = _rand((7, 4, 2), 106)
        for causal in (False, True):
            grads = orc.attention_backward_varlen(q, k, v, g, cu, 0.9, causal)
            for idx, x in enumerate((q, k, v)):
                num = np.zeros_like(x)
                for pos in np.ndindex(x.shape):
                    xp, xm = x.copy(), x.copy()
                    xp[pos] += 1e-6
                    xm[pos] -= 1e-6
                    ap, am = [q, k, v], [q, k, v]
                    ap[idx], am[idx] = xp, xm
                    fp = (orc.attention_forward_varlen(*ap, cu, 0.9, causal)[0] * g).sum()
                    fm = (orc.attention_forward_varlen(*am, cu, 0.9, causal)[0] * g).sum()
                    num[pos] = (fp - fm) / 2e-6
                err = np.abs(num - grads[idx]).max() / max(1.0, np.abs(num).max())
                assert err < 1e-7, (H_kv, causal, idx, err)


VARLEN_BWD_PINS = [pin_varlen_backward_finite_differences]


def brute_force_decode(q, kc, vc, lens, scale):
    """Scalar loops for decode: new token t of sequence b sits at position
    L_b - s_q + t and sees cache keys 0 .. L_b - s_q + t; query head h uses
    K/V head h // (H // H_kv); a row with no visible key is O = 0,
    LSE = -inf. q: [B][s_q][H][D]; caches [B][cap][H_kv][D] nested lists."""
    B, s_q, H, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    group = H // len(kc[0][0])
    o = [[[[0.0] * D for _ in range(H)] for _ in range(s_q)] for _ in range(B)]
    lse = [[[-math.inf] * s_q for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for t in range(s_q):
            last = lens[b] - s_q + t  # last visible key position
            keys = [j for j in range(lens[b]) if j <= last]
            if not keys:
                continue
            for h in range(H):
                hk = h // group
                sc = [scale * sum(q[b][t][h][d] * kc[b][j][hk][d] for d in range(D)) for j in keys]
                m = max(sc)
                wts = [math.exp(x - m) for x in sc]
                tot = sum(wts)
                for d in range(D):
                    o[b][t][h][d] = sum(wt * vc[b][j][hk][d] for wt, j in zip(wts, keys)) / tot
                lse[b][h][t] = m + math.log(tot)
    return o, lse


def pin_decode_brute_force(orc):
    """Decode against scalar loops: two sequences (cache lengths 5 and 1 of
    capacity 6, two new tokens each, so one row of the second sees no key),
    4 query heads over 2 K/V heads."""
    q = _rand((2, 2, 4, 3), 51)
    kc = _rand((2, 6, 2, 3), 52)
    vc = _rand((2, 6, 2, 3), 53)
    lens = [5, 1]
    o, lse = orc.attention_decode(q, kc, vc, lens, 0.8)
    bo, bl = brute_force_decode(q.tolist(), kc.tolist(), vc.tolist(), lens, 0.8)
    np.testing.assert_allclose(o, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(np.array(bl)))
    fin = np.isfinite(np.array(bl))
    np.testing.assert_allclose(lse[fin], np.array(bl)[fin], rtol=0, atol=1e-12)
    assert np.isneginf(lse[1, :, 0]).all() and (o[1, 0] == 0).all()


def pin_decode_is_causal_suffix(orc):
    """Decoding the last s_q tokens of a sequence against its cache gives the
    last s_q rows of the causal forward over the whole sequence (the forward
    oracle is pinned on its own); cache slots past the length are ignored."""
    L, cap, s_q, H, H_kv, D = 7, 10, 3, 4, 2, 5
    qf = _rand((H, L, D), 61)
    kf = _rand((H_kv, L, D), 62)
    vf = _rand((H_kv, L, D), 63)
    group = H // H_kv
    ref_o, ref_l = orc.attention_forward(qf[None], np.repeat(kf, group, axis=0)[None],
                                         np.repeat(vf, group, axis=0)[None], 0.6, True)
    kc = np.full((1, cap, H_kv, D), 1e6)
    vc = np.full((1, cap, H_kv, D), -1e6)
    kc[0, :L] = kf.transpose(1, 0, 2)
    vc[0, :L] = vf.transpose(1, 0, 2)
    q = qf[:, L - s_q:].transpose(1, 0, 2)[None]
    o, lse = orc.attention_decode(q, kc, vc, [L], 0.6)
    np.testing.assert_allclose(o[0], ref_o[0, :, L - s_q:].transpose(1, 0, 2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], ref_l[0, :, L - s_q:], rtol=0, atol=1e-12)


def pin_merge_partials(orc):
    """Attention over all keys equals the merge of attention over disjoint
    key subsets (one of them empty), in any order; all-empty gives O = 0,
    LSE = -inf."""
    q = _rand((1, 1, 3, 4), 71)
    k = _rand((1, 1, 11, 4), 72)
    v = _rand((1, 1, 11, 4), 73)
    whole_o, whole_l = orc.attention_forward(
        np.concatenate([q, np.zeros((1, 1, 8, 4))], axis=2), k, v, 0.9, False)
    parts = [[0, 4, 9], [1, 2, 3, 10], [5, 6, 7, 8]]
    os_, ls_ = [], []
    for idx in parts:
        po, pl = orc.attention_forward(
            np.concatenate([q, np.zeros((1, 1, len(idx) - 3, 4))], axis=2) if len(idx) > 3 else q,
            k[:, :, idx], v[:, :, idx], 0.9, False)
        os_.append(po[0, 0, :3])
        ls_.append(pl[0, 0, :3])
    os_.append(np.zeros((3, 4)))
    ls_.append(np.full(3, -np.inf))
    for order in ([0, 1, 2, 3], [3, 2, 0, 1]):
        o, l = orc.merge_partials(np.stack([os_[i] for i in order]), np.stack([ls_[i] for i in order]))
        np.testing.assert_allclose(o, whole_o[0, 0, :3], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, whole_l[0, 0, :3], rtol=0, atol=1e-12)
    o, l = orc.merge_partials(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert (o == 0).all() and np.isneginf(l).all()


DECODE_PINS = [pin_decode_brute_force, pin_decode_is_causal_suffix, pin_merge_partials]

# --- dropout ------------------------------------------------------------------

# Known-answer vectors of Philox4x32-10 (counter, key) -> output, as published
# with the generator's reference implementation (Random123).
PHILOX_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


def _philox_scalar(ctr, key):
    """Philox4x32-10 on Python integers, one counter at a time."""
    c0, c1, c2, c3 = ctr
    k0, k1 = key
    for _ in range(10):
        p0 = 0xD2511F53 * c0
        p1 = 0xCD9E8D57 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0, p1 & 0xFFFFFFFF, (p0 >> 32) ^ c3 ^ k1,
                          p0 & 0xFFFFFFFF)
        k0 = (k0 + 0x9E3779B9) & 0xFFFFFFFF
        k1 = (k1 + 0xBB67AE85) & 0xFFFFFFFF
    return c0, c1, c2, c3


def pin_philox_known_answers(orc):
    """The oracle's vectorised generator reproduces the published vectors."""
    for ctr, key, out in PHILOX_KAT:
        assert _philox_scalar(ctr, key) == out
        got = orc._rng.philox4x32_10(*ctr, *key)
        assert tuple(int(x) for x in got) == out


def brute_force_dropout(q, k, v, scale, causal, p, seed, offset):
    """Scalar loops: keep bit of (b, h, i, j) from one Philox call per 4x4
    block (word i % 4, byte j % 4 of counter (j//4, i//4, b*H + h, offset)),
    dropped when the byte is below floor(256 p + 0.5)."""
    B, H, N, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    thr = math.floor(float(np.float32(p)) * 256.0 + 0.5)
    inv_keep = 1.0 / (1.0 - thr / 256.0)
    key = (seed & 0xFFFFFFFF, seed >> 32)
    o = [[[[0.0] * D for _ in range(N)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                sc = [scale * sum(q[b][h][i][t] * k[b][h][j][t] for t in range(D)) for j in keys]
                m = max(sc)
                wts = [math.exp(x - m) for x in sc]
                tot = sum(wts)
                lse[b][h][i] = m + math.log(tot)
                for j, wt in zip(keys, wts):
                    word = _philox_scalar((j // 4, i // 4, b * H + h, offset), key)[i % 4]
                    if (word >> (8 * (j % 4))) & 0xFF < thr:
                        continue
                    for t in range(D):
                        o[b][h][i][t] += wt / tot * inv_keep * v[b][h][j][t]
    return o, lse


def pin_dropout_brute_force(orc):
    """Dropout forward against scalar loops with their own generator (two
    heads, N = 9 crossing 4x4 block edges, a 64-bit seed and an offset)."""
    q, k, v = (_rand((1, 2, 9, 3), s) for s in (81, 82, 83))
    seed = 0x1234_5678_9ABC_DEF0
    for causal in (False, True):
        for pr in (0.3, 0.5):
            o, lse = orc.attention_forward_dropout(q, k, v, 0.7, causal, pr, seed, 5)
            bo, bl = brute_force_dropout(q.tolist(), k.tolist(), v.tolist(), 0.7, causal, pr,
                                         seed, 5)
            np.testing.assert_allclose(o, np.array(bo), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, np.array(bl), rtol=0, atol=1e-12)


def pin_dropout_p_zero(orc):
    """p = 0 keeps everything: forward and backward equal the plain ones."""
    q, k, v, g = (_rand((2, 2, 11, 4), s) for s in (84, 85, 86, 87))
    for causal in (False, True):
        o, lse = orc.attention_forward_dropout(q, k, v, 0.6, causal, 0.0, 99, 0)
        ro, rl = orc.attention_forward(q, k, v, 0.6, causal)
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-14)
        np.testing.assert_array_equal(lse, rl)
        grads = orc.attention_backward_dropout(q, k, v, g, 0.6, causal, 0.0, 99, 0)
        refs = orc.attention_backward(q, k, v, g, 0.6, causal)
        for a, r in zip(grads, refs):
            np.testing.assert_allclose(a, r, rtol=0, atol=1e-13)


def pin_dropout_keep_rate(orc):
    """The fraction kept over 2 heads x 512 x 512 elements is within five
    standard deviations of 1 - floor(256 p + 0.5) / 256, and masks of
    different heads, offsets or seeds differ as independent ones would."""
    n = 512
    for pr in (0.1, 0.5):
        thr = math.floor(pr * 256 + 0.5)
        keep_p = 1 - thr / 256
        masks = [orc._rng.keep_mask(bh, np.arange(n), np.arange(n), pr, seed, off)
                 for bh, seed, off in ((0, 7, 0), (1, 7, 0), (0, 7, 1), (0, 8, 0))]
        total = np.concatenate([m.ravel() for m in masks[:2]])
        sd = math.sqrt(keep_p * (1 - keep_p) / total.size)
        assert abs(total.mean() - keep_p) < 5 * sd, (total.mean(), keep_p)
        differ = 2 * keep_p * (1 - keep_p)
        for other in masks[1:]:
            frac = (other != masks[0]).mean()
            assert abs(frac - differ) < 5 * math.sqrt(differ * (1 - differ) / other.size)


def pin_dropout_finite_differences(orc):
    """With the keep bits fixed the dropout forward is smooth in Q, K, V; its
    central differences match the dropout backward."""
    q, k, v, g = (_rand((1, 1, 6, 3), s) for s in (91, 92, 93, 94))
    for causal in (False, True):
        grads = orc.attention_backward_dropout(q, k, v, g, 0.8, causal, 0.4, 2024, 3)
        for idx, x in enumerate((q, k, v)):
            num = np.zeros_like(x)
            for pos in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[pos] += 1e-6
                xm[pos] -= 1e-6
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[idx], args_m[idx] = xp, xm
                fp = (orc.attention_forward_dropout(*args_p, 0.8, causal, 0.4, 2024, 3)[0] * g).sum()
                fm = (orc.attention_forward_dropout(*args_m, 0.8, causal, 0.4, 2024, 3)[0] * g).sum()
                num[pos] = (fp - fm) / 2e-6
            err = np.abs(num - grads[idx]).max() / max(1.0, np.abs(num).max())
            assert err < 1e-7, (idx, causal, err)


DROPOUT_PINS = [pin_philox_known_answers, pin_dropout_brute_force, pin_dropout_p_zero,
                pin_dropout_keep_rate, pin_dropout_finite_differences]



FORWARD_PINS = [pin_golden_forward, pin_brute_force, pin_online_equals_three_pass,
                pin_rows_sum_to_one, pin_constant_v, pin_causal_row0, pin_scale_zero,
                pin_single_key, pin_permutations, pin_torch_sdpa, pin_row_chunking]
BACKWARD_PINS = [pin_golden_backward, pin_finite_differences, pin_grad_sums,
                 pin_constant_v_grads, pin_scale_zero_grads, pin_delta_two_ways,
                 pin_torch_autograd]
ALL_PINS = (FORWARD_PINS + BACKWARD_PINS + VARLEN_PINS + VARLEN_BWD_PINS + DECODE_PINS +
            DROPOUT_PINS)
