"""Pins for the CPU oracle (no GPU).

Every check here compares the oracle with something other than itself:
closed forms of special cases, a brute-force unrolled-product expansion of the
recurrence, exact identities (chaining, varlen, structure) and the independent
numpy transcription. A plausible slip in the oracle -- a dropped term, a wrong
sign, decay applied after the update, the read-out taken from the old state, a
transposed state index, a wrong gate constant -- fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import kda_oracle, kda_oracle_numpy
import kda_inputs


def bf(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def f64(t):
    return t.float().double().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def rand_inputs(B=1, T=6, H=2, K=8, V=8, seed=0, lb=-1.3):
    w = kda_inputs.custom(B=B, T=T, H=H, K=K, V=V, seed=seed, lower_bound=lb)
    d = kda_inputs.make_inputs(w)
    return d


# --------------------------------------------------------------------------
# brute force: S_T = S0 M_1..M_T + sum_t beta_t v_t k^_t^T M_{t+1}..M_T,
# M_t = Diag(alpha_t)(I - beta_t k^_t k^_t^T), o_t = scale S_t q^_t
# --------------------------------------------------------------------------
@pytest.mark.parametrize("K,V,T", [(8, 8, 6), (8, 5, 8), (128, 128, 4)])
def test_unrolled_product_expansion(K, V, T):
    H = 2
    d = rand_inputs(T=T, H=H, K=K, V=V, seed=3, lb=-1.3)
    rng = np.random.default_rng(1)
    S0 = rng.standard_normal((1, H, V, K))
    out, fin = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'],
                          d['dt_bias'], d['lower_bound'], initial_state=S0)
    q, k, v, g, b = (f64(d[n])[0] for n in ('q', 'k', 'v', 'g', 'beta'))
    A_log, dt = f64(d['A_log']), f64(d['dt_bias'])
    lb, scale = float(np.float32(d['lower_bound'])), float(np.float32(d['scale']))
    for h in range(H):
        Ms, adds, qs = [], [], []
        for t in range(T):
            kh = k[t, h] / math.sqrt(k[t, h] @ k[t, h] + 1e-6)
            qh = q[t, h] / math.sqrt(q[t, h] @ q[t, h] + 1e-6)
            beta = 1 / (1 + math.exp(-b[t, h]))
            alpha = np.exp(lb / (1 + np.exp(-math.exp(A_log[h]) * (g[t, h] + dt[h]))))
            Ms.append(np.diag(alpha) @ (np.eye(K) - beta * np.outer(kh, kh)))
            adds.append(beta * np.outer(v[t, h], kh))
            qs.append(qh)
        for t in range(T):
            P = np.eye(K)
            for s in range(t + 1):
                P = P @ Ms[s]
            St = S0[0, h] @ P
            for s in range(t + 1):
                Q = np.eye(K)
                for r in range(s + 1, t + 1):
                    Q = Q @ Ms[r]
                St = St + adds[s] @ Q
            np.testing.assert_allclose(out[t, h], scale * St @ qs[t], rtol=1e-11, atol=1e-12)
            if t == T - 1:
                np.testing.assert_allclose(fin[0, h], St, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# beta = 0 (logit -inf): no update, S_t = S0 Diag(exp(sum gates))
# --------------------------------------------------------------------------
def _beta0_case(T, K, gate_x, A_log_val, lb, S0=None, q=None):
    """Inputs with beta logits -inf and g + dt_bias = gate_x (per channel)."""
    H, V = 1, 4
    g = torch.zeros(1, T, H, K, dtype=torch.bfloat16)
    dt = torch.tensor(np.asarray(gate_x, np.float32).reshape(1, K))
    beta = torch.full((1, T, H), float('-inf'), dtype=torch.bfloat16)
    rng = np.random.default_rng(7)
    qq = bf(rng.standard_normal((1, T, H, K))) if q is None else q
    kk = bf(rng.standard_normal((1, T, H, K)))
    vv = bf(rng.standard_normal((1, T, H, V)))
    if S0 is None:
        S0 = rng.standard_normal((1, H, V, K))
    out, fin = kda_oracle(qq, kk, vv, g, beta, 0.5, torch.tensor([A_log_val], dtype=torch.float32),
                          dt, lb, initial_state=S0)
    return out, fin, S0, qq


def test_beta_zero_gives_pure_decay():
    K, T, lb = 8, 5, -2.0
    out, fin, S0, qq = _beta0_case(T, K, np.zeros(K), 0.0, lb)
    # g + dt = 0 -> sigmoid(0) = 1/2 -> gate = lb/2 per token, exactly
    np.testing.assert_allclose(fin[0, 0], S0[0, 0] * math.exp(T * lb / 2), rtol=1e-14)
    q = f64(qq)[0, :, 0]
    for t in range(T):
        qh = q[t] / math.sqrt(q[t] @ q[t] + 1e-6)
        np.testing.assert_allclose(out[t, 0], 0.5 * (S0[0, 0] * math.exp((t + 1) * lb / 2)) @ qh,
                                   rtol=1e-13, atol=1e-15)


def test_zero_state_beta_zero_is_exactly_zero():
    out, fin, _, _ = _beta0_case(6, 8, np.zeros(8), 0.3, -5.0, S0=np.zeros((1, 1, 4, 8)))
    assert np.all(out == 0) and np.all(fin == 0)


def test_gate_constants():
    """gate = lb * sigmoid(exp(A_log) * (g + dt_bias)), pinned at points where sigmoid is known."""
    K, T, lb = 6, 3, -1.5
    ln3 = float(np.float32(math.log(3.0)))
    # channel: x  (A_log = 0 -> rate 1):  sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4,
    # sigma(0) = 1/2, sigma(+60) ~ 1, sigma(-60) ~ 0, and x = 1 (generic)
    xs = np.array([ln3, -ln3, 0.0, 60.0, -60.0, 1.0], np.float32)
    out, fin, S0, _ = _beta0_case(T, K, xs, 0.0, lb)
    expect_gate = lb * np.array([0.75, 0.25, 0.5, 1.0, 0.0, 1 / (1 + math.exp(-1.0))])
    ratio = fin[0, 0] / S0[0, 0]                        # column c scaled by exp(T gate_c)
    np.testing.assert_allclose(np.log(ratio), np.broadcast_to(T * expect_gate, ratio.shape),
                               rtol=2e-7, atol=1e-12)
    # the rate exp(A_log): A_log = ln 2 doubles x; x = ln3/2 -> sigma(ln 3) = 3/4
    ln2 = float(np.float32(math.log(2.0)))
    out, fin, S0, _ = _beta0_case(T, K, np.full(K, ln3 / 2, np.float32), ln2, lb)
    np.testing.assert_allclose(np.log(fin[0, 0] / S0[0, 0]), T * lb * 0.75, rtol=2e-7)
    # lower_bound = 0 -> no decay at all
    out, fin, S0, _ = _beta0_case(T, K, xs, 0.7, 0.0)
    np.testing.assert_array_equal(fin[0, 0], S0[0, 0])


def test_gate_symmetry():
    """sigma(y) + sigma(-y) = 1  =>  gate(x) + gate(-x) = lb (per channel)."""
    K, T, lb = 16, 2, -3.0
    rng = np.random.default_rng(5)
    xs = rng.standard_normal(K).astype(np.float32)
    _, f1, S0, _ = _beta0_case(T, K, xs, 0.4, lb)
    _, f2, _, _ = _beta0_case(T, K, -xs, 0.4, lb)
    s = np.log(f1[0, 0] / S0[0, 0]) + np.log(f2[0, 0] / S0[0, 0])
    np.testing.assert_allclose(s, T * lb, rtol=1e-12)


# --------------------------------------------------------------------------
# decay-free, beta = 1, signed basis keys: exact column erase/write
# --------------------------------------------------------------------------
def test_basis_keys_closed_form():
    K = V = 128
    T, H = 40, 1
    rng = np.random.default_rng(11)
    cols = rng.integers(0, K, T)
    sign = rng.choice([-1.0, 1.0], T)
    k = np.zeros((1, T, H, K), np.float32)
    k[0, np.arange(T), 0, cols] = sign
    v = rng.standard_normal((1, T, H, V)).astype(np.float32)
    q = rng.standard_normal((1, T, H, K)).astype(np.float32)
    q[0, 3, 0] = 0.0                          # a zero query reads exactly 0
    q[0, 5, 0] = 0.0
    q[0, 5, 0, :2] = [3.0, 4.0]              # q^ = (3,4)/sqrt(25 + 1e-6)
    kb, vb, qb = bf(k), bf(v), bf(q)
    g = bf(rng.standard_normal((1, T, H, K)))
    beta = torch.full((1, T, H), float('inf'), dtype=torch.bfloat16)
    S0 = rng.standard_normal((1, H, V, K))
    scale = 0.25
    out, fin = kda_oracle(qb, kb, vb, g, beta, scale, torch.zeros(1), torch.zeros(1, K), 0.0,
                          initial_state=S0)
    rho = 1.0 / (1.0 + 1e-6)
    S = S0[0, 0].copy()
    vv, qq = f64(vb)[0, :, 0], f64(qb)[0, :, 0]
    for t in range(T):
        c = cols[t]
        S[:, c] = (1 - rho) * S[:, c] + sign[t] * math.sqrt(rho) * vv[t]
        qh = qq[t] / math.sqrt(qq[t] @ qq[t] + 1e-6)
        np.testing.assert_allclose(out[t, 0], scale * S @ qh, rtol=1e-12, atol=1e-14)
    assert np.all(out[3, 0] == 0.0)
    np.testing.assert_allclose(out[5, 0], scale * (3 * S5(S0, cols, sign, vv, rho, 5)[:, 0] +
                                                   4 * S5(S0, cols, sign, vv, rho, 5)[:, 1])
                               / math.sqrt(25 + 1e-6), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin[0, 0], S, rtol=1e-12, atol=1e-14)


def S5(S0, cols, sign, vv, rho, upto):
    S = S0[0, 0].copy()
    for t in range(upto + 1):
        c = cols[t]
        S[:, c] = (1 - rho) * S[:, c] + sign[t] * math.sqrt(rho) * vv[t]
    return S


def test_orthonormal_keys_store_values():
    """Distinct basis keys with beta = 1 and no decay store v (up to rho) and read it back."""
    K = V = 128
    T = 16
    rng = np.random.default_rng(2)
    k = np.zeros((1, T, 1, K), np.float32)
    k[0, np.arange(T), 0, np.arange(T) * 3] = 1.0
    v = rng.standard_normal((1, T, 1, V)).astype(np.float32)
    q = k.copy()                                  # query the key just written
    out, fin = kda_oracle(bf(q), bf(k), bf(v), bf(np.zeros_like(k)),
                          torch.full((1, T, 1), float('inf'), dtype=torch.bfloat16), 1.0,
                          torch.zeros(1), torch.zeros(1, K), 0.0)
    rho = 1 / (1 + 1e-6)
    np.testing.assert_allclose(out[:, 0], rho * f64(bf(v))[0, :, 0], rtol=1e-12)


def test_zero_key_leaves_state_unchanged():
    K, V, T = 8, 8, 4
    d = rand_inputs(T=T, H=1, K=K, V=V, seed=9, lb=0.0)
    d['k'] = torch.zeros_like(d['k'])
    S0 = np.random.default_rng(3).standard_normal((1, 1, V, K))
    _, fin = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'],
                        d['dt_bias'], 0.0, initial_state=S0)
    np.testing.assert_array_equal(fin, S0)


# --------------------------------------------------------------------------
# exact identities
# --------------------------------------------------------------------------
def test_chaining_equals_one_call():
    d = kda_inputs.make_inputs(kda_inputs.custom(T=37, H=2, seed=4, lower_bound=-1.0))
    S0 = np.random.default_rng(0).standard_normal((1, 2, 128, 128)) * 0.02
    full_o, full_f = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'],
                                d['dt_bias'], d['lower_bound'], initial_state=S0)
    for split in (1, 11, 36):
        sl = lambda x, a, b: x[:, a:b].contiguous()
        o1, f1 = kda_oracle(*(sl(d[n], 0, split) for n in ('q', 'k', 'v', 'g', 'beta')), d['scale'],
                            d['A_log'], d['dt_bias'], d['lower_bound'], initial_state=S0)
        o2, f2 = kda_oracle(*(sl(d[n], split, 37) for n in ('q', 'k', 'v', 'g', 'beta')), d['scale'],
                            d['A_log'], d['dt_bias'], d['lower_bound'], initial_state=f1)
        np.testing.assert_array_equal(np.concatenate([o1, o2]), full_o)
        np.testing.assert_array_equal(f2, full_f)


def test_varlen_equals_separate_calls():
    lens = [5, 0, 12, 13, 1]
    d = kda_inputs.make_inputs(kda_inputs.custom(lengths=lens, H=2, seed=6, state='fp32', lower_bound=-2.0))
    cu = d['cu_seqlens']
    o, f = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                      d['lower_bound'], initial_state=d['initial_state'], cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = lambda x: x[:, a:b].contiguous()
        on, fn = kda_oracle(*(sl(d[k]) for k in ('q', 'k', 'v', 'g', 'beta')), d['scale'], d['A_log'],
                            d['dt_bias'], d['lower_bound'], initial_state=d['initial_state'][n:n + 1])
        np.testing.assert_array_equal(o[a:b], on)
        np.testing.assert_array_equal(f[n], fn[0])
    # zero-length sequence: final == initial
    np.testing.assert_array_equal(f[1], d['initial_state'][1].double().numpy())


def test_batch_rows_are_independent_sequences():
    d = kda_inputs.make_inputs(kda_inputs.custom(B=3, T=9, H=2, seed=8, state='bf16'))
    o, f = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                      d['lower_bound'], initial_state=d['initial_state'])
    for b in range(3):
        sl = lambda x: x[b:b + 1].contiguous()
        ob, fb = kda_oracle(*(sl(d[k]) for k in ('q', 'k', 'v', 'g', 'beta')), d['scale'], d['A_log'],
                            d['dt_bias'], d['lower_bound'], initial_state=d['initial_state'][b:b + 1])
        np.testing.assert_array_equal(o[b * 9:(b + 1) * 9], ob)
        np.testing.assert_array_equal(f[b], fb[0])


def test_value_channel_permutation_and_linearity():
    d = kda_inputs.make_inputs(kda_inputs.custom(T=20, H=2, seed=10, lower_bound=-0.7))
    rng = np.random.default_rng(4)
    S0 = rng.standard_normal((1, 2, 128, 128)) * 0.1
    o, f = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                      d['lower_bound'], initial_state=S0)
    perm = rng.permutation(128)
    op, fp = kda_oracle(d['q'], d['k'], d['v'][..., perm].contiguous(), d['g'], d['beta'], d['scale'],
                        d['A_log'], d['dt_bias'], d['lower_bound'], initial_state=S0[:, :, perm])
    np.testing.assert_array_equal(op, o[:, :, perm])
    np.testing.assert_array_equal(fp, f[:, :, perm])
    o2, f2 = kda_oracle(d['q'], d['k'], (d['v'].float() * 2).to(torch.bfloat16), d['g'], d['beta'],
                        d['scale'], d['A_log'], d['dt_bias'], d['lower_bound'], initial_state=2 * S0)
    np.testing.assert_array_equal(o2, 2 * o)
    np.testing.assert_array_equal(f2, 2 * f)


def test_head_subset_and_threads():
    d = kda_inputs.make_inputs(kda_inputs.custom(T=33, H=4, seed=12))
    o, f = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                      d['lower_bound'], nthreads=1)
    o4, f4 = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                        d['lower_bound'], nthreads=4)
    np.testing.assert_array_equal(o, o4)
    np.testing.assert_array_equal(f, f4)
    os_, fs = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                         d['lower_bound'], heads=[3, 1])
    np.testing.assert_array_equal(os_, o[:, [3, 1]])
    np.testing.assert_array_equal(fs, f[:, [3, 1]])


def test_numpy_transcription_matches_c():
    lens = [7, 0, 19]
    d = kda_inputs.make_inputs(kda_inputs.custom(lengths=lens, H=2, seed=13, state='fp32', lower_bound=-4.0))
    o, f = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                      d['lower_bound'], initial_state=d['initial_state'], cu_seqlens=d['cu_seqlens'])
    on, fn = kda_oracle_numpy(*(f64(d[k]) for k in ('q', 'k', 'v', 'g', 'beta')),
                              float(np.float32(d['scale'])), f64(d['A_log']), f64(d['dt_bias']),
                              float(np.float32(d['lower_bound'])),
                              initial_state=f64(d['initial_state']), cu_seqlens=d['cu_seqlens'].numpy())
    np.testing.assert_allclose(o, on, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(f, fn, rtol=1e-12, atol=1e-14)


def test_bad_arguments_raise():
    d = kda_inputs.make_inputs(kda_inputs.custom(T=4, H=1))
    with pytest.raises(ValueError):
        kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], 1.0, d['A_log'], d['dt_bias'], -1.0,
                   heads=[5])
    with pytest.raises(ValueError):
        kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], 1.0, d['A_log'], d['dt_bias'], -1.0,
                   cu_seqlens=torch.tensor([0, 3, 9]))


def test_gate_parameters_indexed_per_head_and_channel():
    """A_log is per head and dt_bias per (head, channel): pinned with beta = 0 closed forms."""
    H, K, V, T, lb = 3, 5, 2, 2, -2.0
    ln2 = float(np.float32(math.log(2.0)))
    ln3 = float(np.float32(math.log(3.0)))
    A_log = torch.tensor([0.0, ln2, 0.0], dtype=torch.float32)
    # x = g + dt with g = 0; per head a different channel pattern
    dt = np.array([[ln3, 0.0, -ln3, 60.0, -60.0],
                   [ln3 / 2, -ln3 / 2, 0.0, 0.0, ln3 / 2],
                   [0.0, 60.0, ln3, -ln3, 0.0]], np.float32)
    expect = np.array([[0.75, 0.5, 0.25, 1.0, 0.0],
                       [0.75, 0.25, 0.5, 0.5, 0.75],      # rate exp(ln 2) = 2 doubles x
                       [0.5, 1.0, 0.75, 0.25, 0.5]]) * lb
    rng = np.random.default_rng(21)
    S0 = rng.standard_normal((1, H, V, K))
    q = bf(rng.standard_normal((1, T, H, K)))
    k = bf(rng.standard_normal((1, T, H, K)))
    v = bf(rng.standard_normal((1, T, H, V)))
    g = torch.zeros(1, T, H, K, dtype=torch.bfloat16)
    beta = torch.full((1, T, H), float('-inf'), dtype=torch.bfloat16)
    _, fin = kda_oracle(q, k, v, g, beta, 1.0, A_log, torch.tensor(dt), lb, initial_state=S0)
    got = np.log(fin[0] / S0[0]) / T                      # [H, V, K] per-channel gate
    np.testing.assert_allclose(got, np.broadcast_to(expect[:, None, :], got.shape), rtol=2e-7, atol=1e-12)


# --------------------------------------------------------------------------
# fusion switches (use_gate_in_kernel / use_qk_l2norm_in_kernel /
# use_beta_sigmoid_in_kernel off): closed forms
# --------------------------------------------------------------------------
def test_gate_off_pure_decay_with_clamp():
    """Gate activation off and beta = 0: S_T = S0 exp(sum_t clamp(g_t, lb, 0)) per channel."""
    K, V, T, H, lb = 8, 4, 5, 1, -2.0
    rng = np.random.default_rng(21)
    gt = np.array([-0.75, -7.0, 0.5, 0.0, -2.0, -1.5, -0.25, -3.0], np.float32)   # bf16-exact
    g = bf(np.broadcast_to(gt, (1, T, H, K)).copy())
    q = bf(rng.standard_normal((1, T, H, K)))
    k = bf(rng.standard_normal((1, T, H, K)))
    v = bf(rng.standard_normal((1, T, H, V)))
    beta = bf(np.zeros((1, T, H)))                      # beta given directly: 0
    S0 = rng.standard_normal((1, H, V, K))
    out, fin = kda_oracle(q, k, v, g, beta, 0.5, None, None, lb, initial_state=S0,
                          use_gate_in_kernel=False, use_beta_sigmoid_in_kernel=False)
    gc = np.clip(gt.astype(np.float64), lb, 0.0)
    np.testing.assert_allclose(fin[0, 0], S0[0, 0] * np.exp(T * gc)[None, :], rtol=1e-14)
    qq = f64(q)[0, :, 0]
    for t in range(T):
        qh = qq[t] / math.sqrt(qq[t] @ qq[t] + 1e-6)
        np.testing.assert_allclose(out[t, 0], 0.5 * (S0[0, 0] * np.exp((t + 1) * gc)[None, :]) @ qh,
                                   rtol=1e-13, atol=1e-15)


def _basis_case(T, seed, beta_val, norm_on, beta_logit):
    K = V = 128
    rng = np.random.default_rng(seed)
    cols = rng.integers(0, K, T)
    sign = rng.choice([-1.0, 1.0], T)
    k = np.zeros((1, T, 1, K), np.float32)
    k[0, np.arange(T), 0, cols] = sign
    v = bf(rng.standard_normal((1, T, 1, V)))
    q = bf(rng.standard_normal((1, T, 1, K)))
    S0 = rng.standard_normal((1, 1, V, K))
    beta = (torch.full((1, T, 1), beta_logit, dtype=torch.bfloat16) if beta_logit is not None
            else bf(np.full((1, T, 1), beta_val)))
    out, fin = kda_oracle(q, bf(k), v, bf(np.zeros((1, T, 1, K))), beta, 0.25, torch.zeros(1),
                          torch.zeros(1, K), 0.0, initial_state=S0, use_qk_l2norm_in_kernel=norm_on,
                          use_beta_sigmoid_in_kernel=beta_logit is not None)
    return out, fin, S0, cols, sign, f64(v)[0, :, 0], f64(q)[0, :, 0]


def test_norm_off_basis_keys_replace_columns_exactly():
    """Norm off, beta = 1, no decay: k = +-e_c writes v into column c exactly (no 1e-6 shrink)
    and q is read as given (not normalised)."""
    T = 30
    out, fin, S0, cols, sign, vv, qq = _basis_case(T, 5, None, False, float('inf'))
    S = S0[0, 0].copy()
    for t in range(T):
        S[:, cols[t]] = sign[t] * vv[t]
        np.testing.assert_allclose(out[t, 0], 0.25 * S @ qq[t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin[0, 0], S, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("bval", [0.5, 0.25, 1.0])
def test_beta_off_basis_keys_closed_form(bval):
    """Beta given directly (b), norm on: column c <- (1 - b rho) S_c + b sign sqrt(rho) v."""
    T = 24
    out, fin, S0, cols, sign, vv, qq = _basis_case(T, 8, bval, True, None)
    rho = 1.0 / (1.0 + 1e-6)
    S = S0[0, 0].copy()
    for t in range(T):
        c = cols[t]
        S[:, c] = (1 - bval * rho) * S[:, c] + bval * sign[t] * math.sqrt(rho) * vv[t]
        qh = qq[t] / math.sqrt(qq[t] @ qq[t] + 1e-6)
        np.testing.assert_allclose(out[t, 0], 0.25 * S @ qh, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fin[0, 0], S, rtol=1e-12, atol=1e-14)


def test_numpy_transcription_matches_c_with_switches_off():
    lens = [9, 0, 14]
    d = kda_inputs.make_inputs(kda_inputs.custom(lengths=lens, H=2, seed=17, state='fp32', lower_bound=-1.5))
    sw = dict(use_gate_in_kernel=False, use_qk_l2norm_in_kernel=False, use_beta_sigmoid_in_kernel=False)
    beta01 = torch.sigmoid(d['beta'].float()).to(torch.bfloat16)   # a probability-valued beta input
    o, f = kda_oracle(d['q'], d['k'], d['v'], d['g'], beta01, d['scale'], None, None, d['lower_bound'],
                      initial_state=d['initial_state'], cu_seqlens=d['cu_seqlens'], **sw)
    on, fn = kda_oracle_numpy(*(f64(t) for t in (d['q'], d['k'], d['v'], d['g'], beta01)),
                              float(np.float32(d['scale'])), None, None, float(np.float32(d['lower_bound'])),
                              initial_state=f64(d['initial_state']), cu_seqlens=d['cu_seqlens'].numpy(), **sw)
    # unnormalised keys (|k|^2 ~ 128) grow the state: allow for the different summation
    # orders of numpy's dot and the C loops
    np.testing.assert_allclose(o, on, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(f, fn, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# gate without the safe bound (safe_gate off): gate = -exp(A_log) softplus(g + dt_bias),
# or min(g, 0) when the activation is not fused; lower_bound is not used
# --------------------------------------------------------------------------
def _beta0_unbounded(T, K, gate_x, A_log_val, lb, S0=None):
    H, V = 1, 4
    g = torch.zeros(1, T, H, K, dtype=torch.bfloat16)
    dt = torch.tensor(np.asarray(gate_x, np.float32).reshape(1, K))
    beta = torch.full((1, T, H), float('-inf'), dtype=torch.bfloat16)
    rng = np.random.default_rng(9)
    q = bf(rng.standard_normal((1, T, H, K)))
    k = bf(rng.standard_normal((1, T, H, K)))
    v = bf(rng.standard_normal((1, T, H, V)))
    if S0 is None:
        S0 = rng.standard_normal((1, H, V, K))
    out, fin = kda_oracle(q, k, v, g, beta, 0.5, torch.tensor([A_log_val], dtype=torch.float32), dt, lb,
                          initial_state=S0, safe_gate=False)
    return out, fin, S0


def test_unbounded_gate_constants():
    """softplus pinned where it has closed forms: softplus(0) = ln 2, softplus(ln 3) = ln 4,
    softplus(-ln 3) = ln(4/3), softplus(ln(e - 1)) = 1, softplus(40) = 40 (+4e-18),
    softplus(-40) = 4e-18; lower_bound (-0.1 here) must not cap the gate."""
    K, T = 6, 3
    ln3 = float(np.float32(math.log(3.0)))
    lem1 = float(np.float32(math.log(math.e - 1.0)))
    xs = np.array([0.0, ln3, -ln3, lem1, 40.0, -40.0], np.float32)
    _, fin, S0 = _beta0_unbounded(T, K, xs, 0.0, -0.1)
    sp = np.array([math.log(2.0), math.log(4.0), math.log(4.0 / 3.0), 1.0, 40.0, 0.0])
    ratio = fin[0, 0] / S0[0, 0]
    np.testing.assert_allclose(np.log(ratio), np.broadcast_to(-T * sp, ratio.shape), rtol=1e-7, atol=1e-15)
    # the rate exp(A_log): A_log = ln 2 doubles the gate
    ln2 = float(np.float32(math.log(2.0)))
    _, fin, S0 = _beta0_unbounded(T, K, np.zeros(K, np.float32), ln2, -0.1)
    np.testing.assert_allclose(np.log(fin[0, 0] / S0[0, 0]), -T * 2.0 * math.log(2.0), rtol=1e-7)


def test_unbounded_gate_huge_decay_is_a_reset():
    """gate = -1e4: exp(gate) = 0, so every token sees an empty state:
    S_t = beta_t v_t k^_t^T and o_t = scale beta_t (k^_t . q^_t) v_t."""
    K = V = 16
    T, H = 7, 1
    rng = np.random.default_rng(31)
    q = bf(rng.standard_normal((1, T, H, K)))
    k = bf(rng.standard_normal((1, T, H, K)))
    v = bf(rng.standard_normal((1, T, H, V)))
    b = bf(rng.standard_normal((1, T, H)))
    g = torch.zeros(1, T, H, K, dtype=torch.bfloat16)
    dt = torch.full((H, K), 1.0e4)
    S0 = rng.standard_normal((1, H, V, K))
    out, fin = kda_oracle(q, k, v, g, b, 0.75, torch.zeros(H), dt, -5.0, initial_state=S0, safe_gate=False)
    qq, kk, vv, bb = f64(q)[0, :, 0], f64(k)[0, :, 0], f64(v)[0, :, 0], f64(b)[0, :, 0]
    for t in range(T):
        qh = qq[t] / math.sqrt(qq[t] @ qq[t] + 1e-6)
        kh = kk[t] / math.sqrt(kk[t] @ kk[t] + 1e-6)
        beta = 1.0 / (1.0 + math.exp(-bb[t]))
        np.testing.assert_allclose(out[t, 0], 0.75 * beta * (kh @ qh) * vv[t], rtol=1e-12, atol=1e-15)
        if t == T - 1:
            np.testing.assert_allclose(fin[0, 0], beta * np.outer(vv[t], kh), rtol=1e-12, atol=1e-15)


def test_unbounded_gate_off_is_min_zero():
    """Activation off, no safe bound, beta = 0: S_T = S0 exp(T min(g, 0)) per channel --
    -7 and -30 pass unclamped (the bounded reading would cap them at lower_bound)."""
    K, V, T, H = 8, 4, 3, 1
    rng = np.random.default_rng(23)
    gt = np.array([-0.75, -7.0, 0.5, 0.0, -30.0, -1.5, 3.0, -0.125], np.float32)   # bf16-exact
    g = bf(np.broadcast_to(gt, (1, T, H, K)).copy())
    q = bf(rng.standard_normal((1, T, H, K)))
    k = bf(rng.standard_normal((1, T, H, K)))
    v = bf(rng.standard_normal((1, T, H, V)))
    S0 = rng.standard_normal((1, H, V, K))
    _, fin = kda_oracle(q, k, v, g, bf(np.zeros((1, T, H))), 0.5, None, None, -2.0, initial_state=S0,
                        use_gate_in_kernel=False, use_beta_sigmoid_in_kernel=False, safe_gate=False)
    np.testing.assert_allclose(fin[0, 0], S0[0, 0] * np.exp(T * np.minimum(gt.astype(np.float64), 0.0))[None, :],
                               rtol=1e-14)


@pytest.mark.parametrize("fused", [True, False])
def test_numpy_transcription_matches_c_unbounded_gate(fused):
    lens = [11, 0, 6]
    d = kda_inputs.make_inputs(kda_inputs.custom(lengths=lens, H=2, seed=29, state='fp32', lower_bound=-1.0))
    g = d['g'] if fused else (-torch.abs(d['g'].float()) * 3).to(torch.bfloat16)
    sw = dict(use_gate_in_kernel=fused, safe_gate=False)
    al, dt = (d['A_log'], d['dt_bias']) if fused else (None, None)
    o, f = kda_oracle(d['q'], d['k'], d['v'], g, d['beta'], d['scale'], al, dt, d['lower_bound'],
                      initial_state=d['initial_state'], cu_seqlens=d['cu_seqlens'], **sw)
    on, fn = kda_oracle_numpy(*(f64(t) for t in (d['q'], d['k'], d['v'], g, d['beta'])),
                              float(np.float32(d['scale'])), None if al is None else f64(al),
                              None if dt is None else f64(dt), float(np.float32(d['lower_bound'])),
                              initial_state=f64(d['initial_state']), cu_seqlens=d['cu_seqlens'].numpy(), **sw)
    np.testing.assert_allclose(o, on, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(f, fn, rtol=1e-12, atol=1e-14)
