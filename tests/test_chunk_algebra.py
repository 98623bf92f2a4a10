"""The chunked (WY / UT) form used by the GPU kernels, in plain fp64, equals the
token recurrence of the oracle.

This checks the algebra only (no kernel, no rounding): a chunk of L <= 64
tokens, split into 16-token sub-chunks with per-sub-chunk reference points so
that every factorised exponential stays inside fp32 range when
lower_bound >= -5 (|sum of 16 gates| <= 80 < ln(FLT_MAX)).

Within a chunk with start state S0 (V x K), cumulative gates G_r (per channel)
and Gamma_r = exp(G_r):
    A   = StrictLower(diag(beta) (K^.Gamma)(K^/Gamma)^T)
    Tm  = (I + A)^-1
    W   = Tm diag(beta) (K^.Gamma),   U~ = Tm diag(beta) V
    U   = U~ - W S0^T
    O   = scale [(Q^.Gamma) S0^T + Lower((Q^.Gamma)(K^/Gamma)^T) U]
    S1  = S0 Diag(Gamma_L) + U^T (K^.Gamma_L/Gamma)
"""
import math

import numpy as np
import pytest

from oracle import kda_oracle
import kda_inputs


def chunk_forward(q, k, v, g, b, A_log, dt, lb, scale, S0, C=64, SUB=16):
    """fp64 chunked form for one (sequence, head). q,k,g [T,K]; v [T,V]; b [T]."""
    T, K = q.shape
    S = S0.copy()
    out = np.zeros((T, v.shape[1]))
    rate = math.exp(A_log)
    for c0 in range(0, T, C):
        L = min(C, T - c0)
        qq = q[c0:c0 + L] / np.sqrt((q[c0:c0 + L] ** 2).sum(1, keepdims=True) + 1e-6)
        kk = k[c0:c0 + L] / np.sqrt((k[c0:c0 + L] ** 2).sum(1, keepdims=True) + 1e-6)
        vv = v[c0:c0 + L]
        beta = 1 / (1 + np.exp(-b[c0:c0 + L]))
        gate = lb / (1 + np.exp(-rate * (g[c0:c0 + L] + dt)))
        nsub = (L + SUB - 1) // SUB
        # sub-chunk local cumulative gates and reference points
        Gs = np.zeros((L, K))
        ref = np.zeros((nsub + 1, K))
        for w in range(nsub):
            a, e = w * SUB, min(L, (w + 1) * SUB)
            Gs[a:e] = np.cumsum(gate[a:e], axis=0)
            ref[w + 1] = ref[w] + Gs[e - 1]
        sub = np.arange(L) // SUB
        G = Gs + ref[sub]                           # chunk-relative cumulative gate
        A = np.zeros((L, L))
        Aqk = np.zeros((L, L))
        for wa in range(nsub):
            ra = slice(wa * SUB, min(L, (wa + 1) * SUB))
            erow = np.exp(Gs[ra])                   # <= 1
            for wb in range(wa + 1):
                rb = slice(wb * SUB, min(L, (wb + 1) * SUB))
                if wb == wa:
                    col = kk[rb] * np.exp(-Gs[rb])  # <= e^80 when lb >= -5
                    A[ra, rb] = np.tril((kk[ra] * erow) @ col.T, -1)
                    Aqk[ra, rb] = np.tril((qq[ra] * erow) @ col.T, 0)
                else:
                    end_b = ref[wb + 1]
                    col = kk[rb] * np.exp(end_b - G[rb])          # <= 1
                    d = np.exp(ref[wa] - end_b)                   # <= 1
                    A[ra, rb] = (kk[ra] * erow * d) @ col.T
                    Aqk[ra, rb] = (qq[ra] * erow * d) @ col.T
        A = beta[:, None] * A
        Tm = np.linalg.inv(np.eye(L) + A)
        Gam = np.exp(G)
        W = Tm @ (beta[:, None] * kk * Gam)
        Ut = Tm @ (beta[:, None] * vv)
        U = Ut - W @ S.T
        out[c0:c0 + L] = scale * ((qq * Gam) @ S.T + Aqk @ U)
        GL = ref[nsub]
        S = S * np.exp(GL)[None, :] + U.T @ (kk * np.exp(GL[None, :] - G))
    return out, S


@pytest.mark.parametrize("T,lb", [(150, -5.0), (64, -2.0), (200, 0.0), (17, -5.0), (129, -0.3)])
def test_chunk_form_equals_recurrence(T, lb):
    d = kda_inputs.make_inputs(kda_inputs.custom(T=T, H=2, seed=31, state='fp32', lower_bound=lb))
    S0 = d['initial_state'].double().numpy()
    out, fin = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'],
                          d['dt_bias'], d['lower_bound'], initial_state=d['initial_state'])
    f = lambda t: t.float().double().numpy()
    for h in range(2):
        o, S = chunk_forward(f(d['q'])[0, :, h], f(d['k'])[0, :, h], f(d['v'])[0, :, h],
                             f(d['g'])[0, :, h], f(d['beta'])[0, :, h], float(d['A_log'][h]),
                             f(d['dt_bias'])[h], float(np.float32(lb)), float(np.float32(d['scale'])),
                             S0[0, h])
        np.testing.assert_allclose(o, out[:, h], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(S, fin[0, h], rtol=1e-9, atol=1e-12)


def test_factorised_exponentials_stay_in_fp32_range():
    """With lb >= -5 every factor the kernels form is within fp32 range."""
    lb, SUB = -5.0, 16
    worst = -lb * SUB                               # |sum of 16 gates| < 80
    assert worst < math.log(np.finfo(np.float32).max)


def test_split_diagonal_block_with_excluded_channels():
    """Unbounded gate, a sub-chunk in which some channels' 8-token halves span more than 200
    (log2 units): the split form takes the other channels (the excluded ones' factors, which
    may overflow, are zeroed by selects after they are formed) and the excluded channels'
    entries are summed token pair by token pair from running products of the per-token
    decays (each at most 1). In fp32, the two parts added give every kept entry (key i <= row
    r) finite and equal to the direct sum sum_c k_r k_i 2^(Gs_r - Gs_i)."""
    rng = np.random.default_rng(9)
    SUB, K = 16, 128
    for frac, span in ((0.07, 400.0), (0.3, 900.0), (1.0, 250.0)):
        raw = rng.exponential(1.0, size=(SUB, K))
        gates = -raw / raw[:8].sum(0, keepdims=True).max() * 150.0        # halves within 200 ...
        bad_ch = rng.random(K) < frac
        gates[:, bad_ch] *= span / 150.0                                   # ... except these channels
        Gs = np.cumsum(gates, axis=0)
        g7, g15 = Gs[7], Gs[15]
        excluded = np.maximum(-g7, g7 - g15) > 200
        assert excluded.any() and not excluded[~bad_ch].any()
        hi = (np.arange(SUB) >= 8)[:, None]
        k = rng.standard_normal((SUB, K))
        k /= np.sqrt((k ** 2).sum(1, keepdims=True))
        with np.errstate(over='ignore', invalid='ignore'):
            m = np.where(hi, 0.5 * (g7 + g15), 0.5 * g7)
            up, dn = np.exp2(Gs - m), np.exp2(m - Gs)
            ex = np.exp2(np.where(hi, Gs - g7, g7 - Gs))
            zero = lambda x: np.where(excluded[None, :], 0.0, x).astype(np.float32)
            d1 = zero(k * up) @ zero(k * dn).T
            d2 = zero(np.where(hi, k * ex, 0.0)) @ zero(np.where(hi, 0.0, k * ex)).T
        merged = np.where(hi == hi.T, d1, d2)
        # the excluded channels, entry by entry: E(r, i) = prod of decays of tokens i+1..r
        al = np.exp2(np.diff(np.vstack([np.zeros((1, K)), Gs]), axis=0)).astype(np.float32)
        ks = np.where(excluded[None, :], k, 0.0).astype(np.float32)
        pair = np.zeros((SUB, SUB), np.float32)
        for r in range(SUB):
            E = np.ones(K, np.float32)
            for i in range(r, -1, -1):
                if i < r:
                    E = E * al[i + 1]
                pair[r, i] = np.float32((ks[r] * ks[i] * E).sum(dtype=np.float32))
        total = merged + pair
        direct = np.einsum('rc,ic,ric->ri', k, k, np.exp2(np.minimum(Gs[:, None, :] - Gs[None, :, :], 0.0)))
        keep = np.tril(np.ones((SUB, SUB), bool))
        assert np.isfinite(total[keep]).all()
        np.testing.assert_allclose(total[keep], direct[keep], rtol=1e-4, atol=1e-6)


def test_midpoint_diagonal_block():
    """Unbounded gate, sub-chunk gate sums in [-200, -118) (log2 units): the diagonal 16x16
    block from factors 2^(Gs - m) (rows) and 2^(m - Gs) (columns) about one midpoint per
    channel, m = g15 / 2 (g15: the channel's sum at token 15, its smallest), keeps every
    factor within 2^(+-100) and, computed in fp32, gives every kept entry (key i <= row r)
    finite and equal to the direct sum sum_c k_r k_i 2^(Gs_r - Gs_i); entries above the
    diagonal may overflow and are masked by the kernels."""
    rng = np.random.default_rng(7)
    SUB, K = 16, 128
    for total in (-119.0, -150.0, -199.9):
        raw = rng.exponential(1.0, size=(SUB, K))
        gates = -raw / raw.sum(0, keepdims=True).max() * (-total)
        Gs = np.cumsum(gates, axis=0)
        g15 = Gs[15]
        assert -Gs.min() > 118 and -g15.min() <= 200 and np.isclose(Gs.min(), g15.min())
        m = 0.5 * g15
        up, dn = np.exp2(Gs - m), np.exp2(m - Gs)
        assert np.abs(np.log2(up)).max() <= 100 and np.abs(np.log2(dn)).max() <= 100
        k = rng.standard_normal((SUB, K))
        k /= np.sqrt((k ** 2).sum(1, keepdims=True))
        direct = np.einsum('rc,ic,ric->ri', k, k, np.exp2(np.minimum(Gs[:, None, :] - Gs[None, :, :], 0.0)))
        with np.errstate(over='ignore', invalid='ignore'):
            d = (k * up).astype(np.float32) @ (k * dn).astype(np.float32).T
        keep = np.tril(np.ones((SUB, SUB), bool))
        assert np.isfinite(d[keep]).all()
        np.testing.assert_allclose(d[keep], direct[keep], rtol=1e-4, atol=1e-6)


def test_split_diagonal_block():
    """Unbounded gate, sub-chunk gate sums below -118 (log2 units) whose 8-token halves each
    span at most 200: the diagonal 16x16 block in its split form -- entries within a half
    from factors about that half's per-channel midpoint (g7 / 2, (g7 + g15) / 2), entries of
    a second-half row against a first-half column from 2^(Gs - g7) and 2^(g7 - Gs) -- keeps
    every factor within 2^(+-100) and, computed in fp32 and merged by half, gives every kept
    entry (key i <= row r) finite and equal to the direct sum sum_c k_r k_i 2^(Gs_r - Gs_i);
    entries above the diagonal or across the halves of the first product may overflow,
    which is why the kernels merge and mask with selects."""
    rng = np.random.default_rng(5)
    SUB, K = 16, 128
    for h1, h2 in ((-119.0, -5.0), (-150.0, -199.0), (-199.0, -199.0), (-60.0, -190.0)):
        # per-token log2 decays whose most negative channel sums to h1 over tokens 0-7 and
        # h2 over tokens 8-15
        raw = rng.exponential(1.0, size=(SUB, K))
        gates = np.empty_like(raw)
        gates[:8] = -raw[:8] / raw[:8].sum(0, keepdims=True).max() * (-h1)
        gates[8:] = -raw[8:] / raw[8:].sum(0, keepdims=True).max() * (-h2)
        Gs = np.cumsum(gates, axis=0)                    # [token, channel], <= 0, decreasing
        g7, g15 = Gs[7], Gs[15]
        assert max((-g7).max(), (g7 - g15).max()) <= 200 + 1e-9
        hi = (np.arange(SUB) >= 8)[:, None]
        m = np.where(hi, 0.5 * (g7 + g15), 0.5 * g7)    # per-token, per-channel reference
        up, dn = np.exp2(Gs - m), np.exp2(m - Gs)
        assert np.abs(np.log2(up)).max() <= 100 and np.abs(np.log2(dn)).max() <= 100
        ex = np.exp2(np.where(hi, Gs - g7, g7 - Gs))
        assert ex.max() <= 1.0
        k = rng.standard_normal((SUB, K))
        k /= np.sqrt((k ** 2).sum(1, keepdims=True))
        direct = np.einsum('rc,ic,ric->ri', k, k, np.exp2(Gs[:, None, :] - Gs[None, :, :]))
        with np.errstate(over='ignore', invalid='ignore'):
            d1 = (k * up).astype(np.float32) @ (k * dn).astype(np.float32).T
        rows2 = np.where(hi, k * ex, 0.0).astype(np.float32)
        cols2 = np.where(hi, 0.0, k * ex).astype(np.float32)
        d2 = rows2 @ cols2.T
        same = hi == hi.T                                # row and column in the same half
        merged = np.where(same, d1, d2)
        keep = np.tril(np.ones((SUB, SUB), bool))
        assert np.isfinite(merged[keep]).all()
        np.testing.assert_allclose(merged[keep], direct[keep], rtol=1e-4, atol=1e-6)
        # one reference point for the whole sub-chunk would need 2^-Gs beyond 2^118
        assert -Gs.min() > 118
