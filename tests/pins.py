"""Checks that tie the oracle to facts outside itself.

Each ``pin_*`` takes an implementation namespace ``impl`` exposing
``forward(q,k,v,scale,causal)``, ``forward_rows(q,k,v,scale,causal,rows)``,
``softmax_rows(s)``, ``scores_rows(...)``, ``backward(q,k,v,do,scale,causal)`` and
``forward_kvcache(q,k,v,kv_len,scale,causal)`` and
``forward_masked(q,k,v,seqlens,window,scale,causal)``
(the oracle, or a deliberately broken copy of it in the mutation test) and
raises AssertionError when the implementation disagrees with:

* closed forms the definition fixes (identical keys, a dominant key, row 0
  under the causal mask, a hand-worked two-token example);
* invariants (row sums of P, permutation of K/V rows, shifts of K and V);
* an independent scalar brute force written here with ``math.exp``/``math.fsum``;
* central finite differences of L = sum(O * dO) for the gradients;
* gradient identities (sum_j dK_j = 0, sum_j dV_j = sum_i dO_i);
* for the KV-cache forward: a scalar brute force over ragged cache lengths,
  the square case (ordinary attention), cache rows past the length being
  ignored, identical keys, and the newest query seeing the whole cache;
* for the padded / sliding-window forward: a scalar brute force, reductions
  to plain attention (no mask, a window covering everything, a padded
  sequence against its unpadded self) and window closed forms.
"""
from __future__ import annotations

import itertools
import math

import numpy as np


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- forward ---

def pin_rows_sum_to_one(impl):
    rng = _rng(11)
    for causal in (False, True):
        q, k = rng.standard_normal((9, 5)), rng.standard_normal((9, 5))
        s = impl.scores_rows(q, k, 0.7, causal, np.arange(9))
        p, _ = impl.softmax_rows(s)
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-14
        if causal:
            assert np.all(p[np.triu_indices(9, 1)] == 0.0)


def pin_identical_keys(impl):
    """All keys equal: P is uniform over visible keys, O is the (prefix) mean of V."""
    rng = _rng(12)
    N, d = 13, 6
    q = rng.standard_normal((1, 1, N, d))
    k = np.repeat(rng.standard_normal((1, 1, 1, d)), N, axis=2)
    v = rng.standard_normal((1, 1, N, d))
    scale = 0.37
    for causal in (False, True):
        o, lse = impl.forward(q, k, v, scale, causal)
        qk = scale * (q[0, 0] @ k[0, 0, 0])
        for i in range(N):
            n_vis = i + 1 if causal else N
            want = v[0, 0, :n_vis].mean(axis=0)
            assert np.max(np.abs(o[0, 0, i] - want)) < 1e-13
            assert abs(lse[0, 0, i] - (qk[i] + math.log(n_vis))) < 1e-12


def pin_dominant_key(impl):
    """K_j = c e_j, Q_i = e_pi(i), scale 1: row i puts weight ~1 on key pi(i)."""
    N = d = 8
    c = 50.0
    k = c * np.eye(N)[None, None]
    v = _rng(13).standard_normal((1, 1, N, d))
    for causal in (False, True):
        pi = [i // 2 for i in range(N)] if causal else [(3 * i + 1) % N for i in range(N)]
        q = np.eye(N)[pi][None, None]
        o, lse = impl.forward(q, k, v, 1.0, causal)
        for i in range(N):
            assert np.max(np.abs(o[0, 0, i] - v[0, 0, pi[i]])) < 1e-15
            n_vis = i + 1 if causal else N
            want_lse = c + math.log1p((n_vis - 1) * math.exp(-c))
            assert abs(lse[0, 0, i] - want_lse) < 1e-12


def pin_causal_row0(impl):
    rng = _rng(14)
    q, k, v = (rng.standard_normal((2, 3, 7, 4)) for _ in range(3))
    o, lse = impl.forward(q, k, v, 0.5, True)
    assert np.max(np.abs(o[:, :, 0] - v[:, :, 0])) < 1e-15
    want = 0.5 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    assert np.max(np.abs(lse[:, :, 0] - want)) < 1e-14


def pin_permutation_invariance(impl):
    rng = _rng(15)
    q, k, v = (rng.standard_normal((1, 2, 11, 5)) for _ in range(3))
    perm = rng.permutation(11)
    o1, l1 = impl.forward(q, k, v, 0.8, False)
    o2, l2 = impl.forward(q, k[:, :, perm], v[:, :, perm], 0.8, False)
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13


def pin_shifts(impl):
    rng = _rng(16)
    q, k, v = (rng.standard_normal((1, 1, 10, 4)) for _ in range(3))
    c = rng.standard_normal(4)
    for causal in (False, True):
        o, lse = impl.forward(q, k, v, 0.6, causal)
        o_k, lse_k = impl.forward(q, k + c, v, 0.6, causal)      # K -> K + 1 c^T
        assert np.max(np.abs(o_k - o)) < 1e-12
        assert np.max(np.abs(lse_k - (lse + 0.6 * (q[..., :] @ c)))) < 1e-12
        o_v, lse_v = impl.forward(q, k, v + c, 0.6, causal)      # V -> V + 1 c^T
        assert np.max(np.abs(o_v - (o + c))) < 1e-12 and np.max(np.abs(lse_v - lse)) < 1e-15
        o_a, lse_a = impl.forward(2.5 * q, k, v, 0.6 / 2.5, causal)  # (aQ, s/a) == (Q, s)
        assert np.max(np.abs(o_a - o)) < 1e-12 and np.max(np.abs(lse_a - lse)) < 1e-12


def brute_force_forward(q, k, v, scale, causal, H_kv):
    """Scalar loops with math.exp and math.fsum; no numpy arithmetic."""
    B, H, N, d = q.shape
    g = H // H_kv
    o = [[[[0.0] * v.shape[3] for _ in range(N)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b, h, i in itertools.product(range(B), range(H), range(N)):
        kv = h // g
        js = range(i + 1) if causal else range(N)
        s = {j: scale * math.fsum(float(q[b, h, i, t]) * float(k[b, kv, j, t]) for t in range(d))
             for j in js}
        mx = max(s.values())
        w = {j: math.exp(s[j] - mx) for j in js}
        tot = math.fsum(w.values())
        lse[b][h][i] = mx + math.log(tot)
        for t in range(v.shape[3]):
            o[b][h][i][t] = math.fsum(w[j] * float(v[b, kv, j, t]) for j in js) / tot
    return np.array(o), np.array(lse)


def pin_brute_force(impl):
    rng = _rng(17)
    cases = [(1, 1, 1, 1, 1), (1, 2, 2, 5, 3), (2, 4, 2, 9, 4), (1, 4, 1, 16, 8), (1, 3, 3, 16, 2)]
    for (B, H, H_kv, N, d), causal in itertools.product(cases, (False, True)):
        q = rng.standard_normal((B, H, N, d)) * 1.5
        k = rng.standard_normal((B, H_kv, N, d)) * 1.5
        v = rng.standard_normal((B, H_kv, N, d))
        scale = 1.0 / math.sqrt(d)
        o, lse = impl.forward(q, k, v, scale, causal)
        o_b, lse_b = brute_force_forward(q, k, v, scale, causal, H_kv)
        assert np.max(np.abs(o - o_b)) < 1e-13, (B, H, H_kv, N, d, causal)
        assert np.max(np.abs(lse - lse_b)) < 1e-13


def pin_worked_example(impl):
    """Two tokens, d = 1, scale 1: q = (1, 2), k = (0, 1), v = (1, 3).

    Row 0 scores (0, 1), row 1 scores (0, 2), so with e = exp(1):
      non-causal O = ((1+3e)/(1+e), (1+3e^2)/(1+e^2)), LSE = (ln(1+e), ln(1+e^2));
      causal     O = (1, (1+3e^2)/(1+e^2)),          LSE = (0, ln(1+e^2)).
    """
    e = math.e
    q = np.array([1.0, 2.0]).reshape(1, 1, 2, 1)
    k = np.array([0.0, 1.0]).reshape(1, 1, 2, 1)
    v = np.array([1.0, 3.0]).reshape(1, 1, 2, 1)
    want = {
        False: ([(1 + 3 * e) / (1 + e), (1 + 3 * e * e) / (1 + e * e)],
                [math.log(1 + e), math.log(1 + e * e)]),
        True: ([1.0, (1 + 3 * e * e) / (1 + e * e)], [0.0, math.log(1 + e * e)]),
    }
    for causal, (wo, wl) in want.items():
        o, lse = impl.forward(q, k, v, 1.0, causal)
        assert np.max(np.abs(o.reshape(2) - wo)) < 1e-15
        assert np.max(np.abs(lse.reshape(2) - wl)) < 1e-15


def pin_forward_rows(impl):
    """Row subsets give the same rows as the full computation."""
    rng = _rng(18)
    q, k, v = (rng.standard_normal((40, 6)) for _ in range(3))
    rows = [0, 3, 17, 39]
    for causal in (False, True):
        of, lf = impl.forward(q[None, None], k[None, None], v[None, None], 0.4, causal)
        orow, lrow = impl.forward_rows(q, k, v, 0.4, causal, rows)
        assert np.max(np.abs(orow - of[0, 0, rows])) < 1e-14
        assert np.max(np.abs(lrow - lf[0, 0, rows])) < 1e-14


# ---------------------------------------------------------- KV-cache decode ---

def brute_force_kvcache(q, k, v, kv_len, scale, causal):
    """Scalar loops: query i of batch b stands at position kv_len[b] - N_q + i."""
    B, H, n_q, d = q.shape
    H_kv = k.shape[1]
    g = H // H_kv
    o = np.zeros((B, H, n_q, v.shape[3]))
    lse = np.full((B, H, n_q), -math.inf)
    for b, h, i in itertools.product(range(B), range(H), range(n_q)):
        n = int(kv_len[b])
        last = min(n - 1, n - n_q + i) if causal else n - 1
        js = list(range(last + 1))
        if not js:
            continue
        kv = h // g
        s = [scale * math.fsum(float(q[b, h, i, t]) * float(k[b, kv, j, t]) for t in range(d)) for j in js]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = math.fsum(w)
        lse[b, h, i] = mx + math.log(tot)
        for t in range(v.shape[3]):
            o[b, h, i, t] = math.fsum(wj * float(v[b, kv, j, t]) for wj, j in zip(w, js)) / tot
    return o, lse


def pin_kvcache_brute_force(impl):
    """Ragged cache lengths (including 0 and lengths below N_q), GQA, both masks."""
    rng = _rng(21)
    cases = [(1, 1, 1, 1, 9, 4, [9]), (2, 4, 2, 3, 11, 5, [11, 2]), (3, 6, 3, 2, 7, 3, [0, 1, 7]),
             (1, 2, 1, 5, 16, 8, [13])]
    for (B, H, H_kv, n_q, n_kv, d, lens), causal in itertools.product(cases, (False, True)):
        q = rng.standard_normal((B, H, n_q, d)) * 1.5
        k = rng.standard_normal((B, H_kv, n_kv, d)) * 1.5
        v = rng.standard_normal((B, H_kv, n_kv, d))
        scale = 1.0 / math.sqrt(d)
        o, lse = impl.forward_kvcache(q, k, v, lens, scale, causal)
        o_b, lse_b = brute_force_kvcache(q, k, v, lens, scale, causal)
        assert np.max(np.abs(o - o_b)) < 1e-13, (B, H, n_q, lens, causal)
        fin = np.isfinite(lse_b)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.max(np.abs(lse[fin] - lse_b[fin]), initial=0.0) < 1e-13


def pin_kvcache_square_case(impl):
    """N_q = N_kv with the full cache is ordinary attention (top-left = bottom-right)."""
    rng = _rng(22)
    q = rng.standard_normal((2, 4, 9, 5))
    k, v = rng.standard_normal((2, 2, 9, 5)), rng.standard_normal((2, 2, 9, 5))
    for causal in (False, True):
        o1, l1 = impl.forward_kvcache(q, k, v, None, 0.6, causal)
        o2, l2 = impl.forward(q, k, v, 0.6, causal)
        assert np.max(np.abs(o1 - o2)) < 1e-14 and np.max(np.abs(l1 - l2)) < 1e-14


def pin_kvcache_tail_ignored(impl):
    """Cache rows at or past kv_len never matter; kv_len = n equals a cache of n rows."""
    rng = _rng(23)
    q = rng.standard_normal((2, 2, 3, 4))
    k, v = rng.standard_normal((2, 1, 12, 4)), rng.standard_normal((2, 1, 12, 4))
    lens = [7, 12]
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 7:] = 1e3
    v2[0, :, 7:] = -1e3
    for causal in (False, True):
        o1, l1 = impl.forward_kvcache(q, k, v, lens, 0.5, causal)
        o2, l2 = impl.forward_kvcache(q, k2, v2, lens, 0.5, causal)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        o3, l3 = impl.forward_kvcache(q[:1], k[:1, :, :7], v[:1, :, :7], None, 0.5, causal)
        assert np.max(np.abs(o3 - o1[:1])) < 1e-15 and np.max(np.abs(l3 - l1[:1])) < 1e-15


def pin_kvcache_identical_keys(impl):
    """Identical keys: row i averages the V rows it sees, LSE = q.k*scale + ln(count)."""
    rng = _rng(24)
    n_q, n_kv, d = 4, 10, 3
    q = rng.standard_normal((1, 1, n_q, d))
    k = np.repeat(rng.standard_normal((1, 1, 1, d)), n_kv, axis=2)
    v = rng.standard_normal((1, 1, n_kv, d))
    for n, causal in itertools.product((10, 6, 2), (False, True)):
        o, lse = impl.forward_kvcache(q, k, v, [n], 0.8, causal)
        for i in range(n_q):
            seen = min(n, n - n_q + i + 1) if causal else n
            if seen <= 0:
                assert np.all(o[0, 0, i] == 0) and lse[0, 0, i] == -math.inf
                continue
            assert np.max(np.abs(o[0, 0, i] - v[0, 0, :seen].mean(axis=0))) < 1e-13
            want = 0.8 * float(q[0, 0, i] @ k[0, 0, 0]) + math.log(seen)
            assert abs(lse[0, 0, i] - want) < 1e-12


def pin_kvcache_last_query_sees_all(impl):
    """The newest query sees the whole cache, so the mask cannot change its row."""
    rng = _rng(25)
    q = rng.standard_normal((2, 4, 3, 6))
    k, v = rng.standard_normal((2, 2, 8, 6)), rng.standard_normal((2, 2, 8, 6))
    oc, lc = impl.forward_kvcache(q, k, v, [8, 5], 0.4, True)
    on, ln = impl.forward_kvcache(q, k, v, [8, 5], 0.4, False)
    assert np.max(np.abs(oc[:, :, -1] - on[:, :, -1])) < 1e-15
    assert np.max(np.abs(lc[:, :, -1] - ln[:, :, -1])) < 1e-15
    assert np.max(np.abs(oc[:, :, 0] - on[:, :, 0])) > 1e-3   # earlier rows do differ


# --------------------------------------------------- padding and window ---

def brute_force_masked(q, k, v, lens, window, scale, causal):
    """Scalar loops over each row's visible keys, written out independently."""
    B, H, N, d = q.shape
    g = H // k.shape[1]
    o = np.zeros((B, H, N, v.shape[3]))
    lse = np.full((B, H, N), -math.inf)
    for b, h, i in itertools.product(range(B), range(H), range(N)):
        n = int(lens[b])
        if i >= n:
            continue
        js = [j for j in range(n) if (not causal or j <= i) and (window is None or window < 0 or j >= i - window)]
        kv = h // g
        s = [scale * math.fsum(float(q[b, h, i, t]) * float(k[b, kv, j, t]) for t in range(d)) for j in js]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = math.fsum(w)
        lse[b, h, i] = mx + math.log(tot)
        for t in range(v.shape[3]):
            o[b, h, i, t] = math.fsum(wj * float(v[b, kv, j, t]) for wj, j in zip(w, js)) / tot
    return o, lse


def pin_masked_brute_force(impl):
    rng = _rng(26)
    cases = [(2, 4, 2, 9, 3, [9, 4], None, True), (2, 2, 1, 11, 4, [11, 0], 3, True),
             (3, 2, 2, 8, 2, [1, 8, 5], 0, True), (2, 4, 4, 10, 3, [10, 6], None, False),
             (1, 2, 1, 16, 5, [13], 7, True)]
    for B, H, H_kv, N, d, lens, window, causal in cases:
        q = rng.standard_normal((B, H, N, d)) * 1.5
        k = rng.standard_normal((B, H_kv, N, d)) * 1.5
        v = rng.standard_normal((B, H_kv, N, d))
        o, lse = impl.forward_masked(q, k, v, lens, window, 0.6, causal)
        o_b, lse_b = brute_force_masked(q, k, v, lens, window, 0.6, causal)
        assert np.max(np.abs(o - o_b)) < 1e-13, (lens, window, causal)
        fin = np.isfinite(lse_b)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.max(np.abs(lse[fin] - lse_b[fin]), initial=0.0) < 1e-13


def pin_masked_reductions(impl):
    """No padding and no window is plain attention; a window covering the whole
    sequence changes nothing; a padded sequence equals the unpadded one."""
    rng = _rng(27)
    q = rng.standard_normal((2, 4, 12, 5))
    k, v = rng.standard_normal((2, 2, 12, 5)), rng.standard_normal((2, 2, 12, 5))
    for causal in (False, True):
        o0, l0 = impl.forward(q, k, v, 0.5, causal)
        o1, l1 = impl.forward_masked(q, k, v, None, None, 0.5, causal)
        assert np.max(np.abs(o1 - o0)) < 1e-15 and np.max(np.abs(l1 - l0)) < 1e-15
        om, lm = impl.forward_masked(q, k, v, [12, 7], None, 0.5, causal)
        ot, lt = impl.forward(q[1:, :, :7], k[1:, :, :7], v[1:, :, :7], 0.5, causal)
        assert np.max(np.abs(om[1, :, :7] - ot[0])) < 1e-14 and np.max(np.abs(lm[1, :, :7] - lt[0])) < 1e-14
        assert np.all(om[1, :, 7:] == 0) and np.all(lm[1, :, 7:] == -math.inf)
    o0, l0 = impl.forward(q, k, v, 0.5, True)
    ow, lw = impl.forward_masked(q, k, v, None, 11, 0.5, True)
    assert np.max(np.abs(ow - o0)) < 1e-15 and np.max(np.abs(lw - l0)) < 1e-15
    ow, lw = impl.forward_masked(q, k, v, None, 10, 0.5, True)   # the last row loses key 0
    assert np.max(np.abs(ow[:, :, :11] - o0[:, :, :11])) < 1e-15
    assert np.max(np.abs(ow[:, :, 11] - o0[:, :, 11])) > 1e-6


def pin_masked_window_closed_forms(impl):
    """window 0: every row sees only itself (O_i = V_i, LSE_i = scale q_i.k_i);
    window 1 with identical keys: the mean of V_{i-1} and V_i."""
    rng = _rng(28)
    q = rng.standard_normal((1, 2, 9, 4))
    k, v = rng.standard_normal((1, 1, 9, 4)), rng.standard_normal((1, 1, 9, 4))
    o, lse = impl.forward_masked(q, k, v, None, 0, 0.7, True)
    assert np.max(np.abs(o[0] - v[0, 0][None])) < 1e-15
    assert np.max(np.abs(lse[0] - 0.7 * np.einsum("hid,id->hi", q[0], k[0, 0]))) < 1e-14
    k1 = np.repeat(k[:, :, :1], 9, axis=2)
    o, lse = impl.forward_masked(q, k1, v, None, 1, 0.7, True)
    want = np.concatenate([v[0, 0, :1], 0.5 * (v[0, 0, :-1] + v[0, 0, 1:])])
    assert np.max(np.abs(o[0] - want[None])) < 1e-14


# --------------------------------------------------------------- backward ---

def _loss(impl, q, k, v, do, scale, causal):
    o, _ = impl.forward(q, k, v, scale, causal)
    return math.fsum((o * do).ravel().tolist())


def pin_finite_differences(impl):
    rng = _rng(19)
    h = 1e-6
    for (B, H, H_kv, N, d), causal in itertools.product([(1, 1, 1, 6, 3), (1, 4, 2, 5, 2)], (False, True)):
        q = rng.standard_normal((B, H, N, d))
        k = rng.standard_normal((B, H_kv, N, d))
        v = rng.standard_normal((B, H_kv, N, d))
        do = rng.standard_normal((B, H, N, d))
        scale = 0.9
        dq, dk, dv = impl.backward(q, k, v, do, scale, causal)
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                args = {"q": q, "k": k, "v": v}
                lp = _loss(impl, *(xp if n == name else args[n] for n in "qkv"), do, scale, causal)
                lm = _loss(impl, *(xm if n == name else args[n] for n in "qkv"), do, scale, causal)
                num[idx] = (lp - lm) / (2 * h)
            assert np.max(np.abs(num - g)) < 1e-7, (name, causal, np.max(np.abs(num - g)))


def pin_gradient_identities(impl):
    rng = _rng(20)
    B, H, H_kv, N, d = 2, 4, 2, 12, 5
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H_kv, N, d))
    v = rng.standard_normal((B, H_kv, N, d))
    do = rng.standard_normal((B, H, N, d))
    for causal in (False, True):
        dq, dk, dv = impl.backward(q, k, v, do, 0.45, causal)
        assert np.max(np.abs(dk.sum(axis=2))) < 1e-12                       # sum_j dS_ij = 0
        do_group = do.reshape(B, H_kv, H // H_kv, N, d).sum(axis=2)
        assert np.max(np.abs(dv.sum(axis=2) - do_group.sum(axis=2))) < 1e-12  # P rows sum to 1
        if causal:
            # the last key is seen only by the last query: dV_{N-1} = sum over group of dO_{N-1} * P[N-1,N-1]
            _, lse = impl.forward(q, k, v, 0.45, True)
            g = H // H_kv
            for b, kv in itertools.product(range(B), range(H_kv)):
                want = np.zeros(d)
                for h in range(kv * g, (kv + 1) * g):
                    p_last = math.exp(0.45 * float(q[b, h, N - 1] @ k[b, kv, N - 1]) - lse[b, h, N - 1])
                    want += p_last * do[b, h, N - 1]
                assert np.max(np.abs(dv[b, kv, N - 1] - want)) < 1e-12


FORWARD_PINS = [pin_rows_sum_to_one, pin_identical_keys, pin_dominant_key, pin_causal_row0,
                pin_permutation_invariance, pin_shifts, pin_brute_force, pin_worked_example,
                pin_forward_rows]
def pin_masked_rows(impl):
    """Row subsets of one head agree with the whole-sequence computation."""
    rng = _rng(29)
    q = rng.standard_normal((1, 1, 30, 4))
    k, v = rng.standard_normal((1, 1, 30, 4)), rng.standard_normal((1, 1, 30, 4))
    rows = [0, 5, 17, 21, 29]
    for n, window, causal in ((30, None, True), (22, 6, True), (25, None, False), (30, 0, True)):
        of, lf = impl.forward_masked(q, k, v, [n], window, 0.9, causal)
        orow, lrow = impl.forward_masked_rows(q[0, 0], k[0, 0], v[0, 0], n, window, 0.9, causal, rows)
        assert np.max(np.abs(orow - of[0, 0, rows])) < 1e-14
        fin = np.isfinite(lf[0, 0, rows])
        assert np.array_equal(np.isfinite(lrow), fin)
        assert np.max(np.abs(lrow[fin] - lf[0, 0, rows][fin]), initial=0.0) < 1e-14


def pin_masked_backward(impl):
    """Central finite differences of sum(O * dO) through forward_masked; no
    mask reduces to backward; padding rows and keys get zero gradients."""
    rng = _rng(30)
    h = 1e-6
    for lens, window in (([6, 3], None), ([7, 7], 2), ([5, 0], 1)):
        B, H, H_kv, N, d = 2, 2, 1, 7, 2
        q = rng.standard_normal((B, H, N, d))
        k = rng.standard_normal((B, H_kv, N, d))
        v = rng.standard_normal((B, H_kv, N, d))
        do = rng.standard_normal((B, H, N, d))
        dq, dk, dv = impl.backward_masked(q, k, v, do, lens, window, 0.8, True)

        def loss(qq, kk, vv):
            o, _ = impl.forward_masked(qq, kk, vv, lens, window, 0.8, True)
            return math.fsum((o * do).ravel().tolist())
        for name, x, gr in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                args = {"q": q, "k": k, "v": v}
                lp = loss(*(xp if n == name else args[n] for n in "qkv"))
                lm = loss(*(xm if n == name else args[n] for n in "qkv"))
                num[idx] = (lp - lm) / (2 * h)
            assert np.max(np.abs(num - gr)) < 1e-7, (name, lens, window)
        for b, n in enumerate(lens):
            assert np.all(dq[b, :, n:] == 0) and np.all(dk[b, :, n:] == 0) and np.all(dv[b, :, n:] == 0)
    q, k, v, do = (rng.standard_normal((2, 4, 9, 3)) if i != 1 and i != 2 else rng.standard_normal((2, 2, 9, 3))
                   for i in range(4))
    for causal in (False, True):
        a = impl.backward(q, k, v, do, 0.5, causal)
        m = impl.backward_masked(q, k, v, do, None, None, 0.5, causal)
        for x, y in zip(a, m):
            assert np.max(np.abs(x - y)) < 1e-13


def pin_blocksparse(impl):
    """All blocks on is plain attention; block-diagonal blocks are independent
    attentions over each block; a scalar brute force; rows whose blocks are
    all off (or all in the future) come back O = 0, LSE = -inf; gradients
    match central finite differences."""
    rng = _rng(31)
    B, H, H_kv, N, d, blk = 2, 2, 1, 12, 3, 4
    q = rng.standard_normal((B, H, N, d))
    k, v = rng.standard_normal((B, H_kv, N, d)), rng.standard_normal((B, H_kv, N, d))
    nb = N // blk
    for causal in (False, True):
        o0, l0 = impl.forward(q, k, v, 0.7, causal)
        o1, l1 = impl.forward_blocksparse(q, k, v, np.ones((H, nb, nb)), blk, 0.7, causal)
        assert np.max(np.abs(o1 - o0)) < 1e-14 and np.max(np.abs(l1 - l0)) < 1e-14
        od, ld = impl.forward_blocksparse(q, k, v, np.stack([np.eye(nb)] * H), blk, 0.7, causal)
        for bi in range(nb):
            sl = slice(bi * blk, (bi + 1) * blk)
            ob, lb = impl.forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.7, causal)
            assert np.max(np.abs(od[:, :, sl] - ob)) < 1e-14 and np.max(np.abs(ld[:, :, sl] - lb)) < 1e-14
    bm = rng.integers(0, 2, (H, nb, nb))
    bm[0, 1, :] = 0                      # query block 1 of head 0 sees nothing
    bm[1, 0, :] = 0
    bm[1, 0, 2] = 1                      # only a future block: nothing under the causal mask
    for causal in (False, True):
        o, lse = impl.forward_blocksparse(q, k, v, bm, blk, 0.7, causal)
        for b, h, i in itertools.product(range(B), range(H), range(N)):
            js = [j for j in range(N) if bm[h, i // blk, j // blk] and (not causal or j <= i)]
            if not js:
                assert np.all(o[b, h, i] == 0) and lse[b, h, i] == -math.inf
                continue
            s_ = [0.7 * math.fsum(float(q[b, h, i, t]) * float(k[b, 0, j, t]) for t in range(d)) for j in js]
            mx = max(s_)
            w = [math.exp(x - mx) for x in s_]
            tot = math.fsum(w)
            assert abs(lse[b, h, i] - (mx + math.log(tot))) < 1e-13
            for t in range(d):
                assert abs(o[b, h, i, t] - math.fsum(wj * float(v[b, 0, j, t]) for wj, j in zip(w, js)) / tot) < 1e-13
    do = rng.standard_normal(q.shape)
    dq, dk, dv = impl.backward_blocksparse(q, k, v, do, bm, blk, 0.7, True)

    def loss(qq, kk, vv):
        o, _ = impl.forward_blocksparse(qq, kk, vv, bm, blk, 0.7, True)
        return math.fsum((o * do).ravel().tolist())
    hh = 1e-6
    for name, x, gr in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in list(np.ndindex(*x.shape))[::7]:
            xp = x.copy(); xp[idx] += hh
            xm = x.copy(); xm[idx] -= hh
            args = {"q": q, "k": k, "v": v}
            num = (loss(*(xp if n == name else args[n] for n in "qkv")) -
                   loss(*(xm if n == name else args[n] for n in "qkv"))) / (2 * hh)
            assert abs(num - gr[idx]) < 1e-7, (name, idx)


def pin_blocksparse_rows(impl):
    """Row subsets of one head agree with the whole computation."""
    rng = _rng(32)
    q = rng.standard_normal((1, 2, 24, 3))
    k, v = rng.standard_normal((1, 1, 24, 3)), rng.standard_normal((1, 1, 24, 3))
    bm = rng.integers(0, 2, (2, 4, 4))
    bm[1, 2, :] = 0
    rows = [0, 5, 13, 14, 23]
    for causal in (False, True):
        of, lf = impl.forward_blocksparse(q, k, v, bm, 6, 0.9, causal)
        for h in range(2):
            orow, lrow = impl.forward_blocksparse_rows(q[0, h], k[0, 0], v[0, 0], bm[h], 6, 0.9, causal, rows)
            assert np.max(np.abs(orow - of[0, h, rows])) < 1e-14
            fin = np.isfinite(lf[0, h, rows])
            assert np.array_equal(np.isfinite(lrow), fin)
            assert np.max(np.abs(lrow[fin] - lf[0, h, rows][fin]), initial=0.0) < 1e-14


MASKED_PINS = [pin_blocksparse, pin_blocksparse_rows, pin_masked_brute_force, pin_masked_reductions, pin_masked_window_closed_forms, pin_masked_rows,
               pin_masked_backward]
KVCACHE_PINS = [pin_kvcache_brute_force, pin_kvcache_square_case, pin_kvcache_tail_ignored,
                pin_kvcache_identical_keys, pin_kvcache_last_query_sees_all]
BACKWARD_PINS = [pin_finite_differences, pin_gradient_identities]
ALL_PINS = FORWARD_PINS + KVCACHE_PINS + MASKED_PINS + BACKWARD_PINS
