"""The seeded input recipe is deterministic and has the stated shapes/distributions."""
import math

import torch

import kda_inputs


def test_deterministic_and_shapes():
    w = kda_inputs.custom(B=2, T=1500, H=3, state='fp32')
    a = kda_inputs.make_inputs(w)
    b = kda_inputs.make_inputs(w)
    for n in ('q', 'k', 'v', 'g', 'beta', 'A_log', 'dt_bias', 'initial_state'):
        assert torch.equal(a[n], b[n]), n
    assert a['q'].shape == (2, 1500, 3, 128) and a['q'].dtype == torch.bfloat16
    assert a['beta'].shape == (2, 1500, 3) and a['beta'].dtype == torch.bfloat16
    assert a['A_log'].shape == (3,) and a['A_log'].dtype == torch.float32
    assert a['dt_bias'].shape == (3, 128)
    assert a['initial_state'].shape == (2, 3, 128, 128) and a['initial_state'].dtype == torch.float32
    assert float(a['A_log'].min()) >= 0 and float(a['A_log'].max()) <= math.log(16)


def test_named_workloads():
    w0 = kda_inputs.workload(0)
    assert (w0.B, w0.T, w0.H, w0.lower_bound, w0.state, w0.final) == (1, 256, 2, -5.0, None, 'fp32')
    w1 = kda_inputs.workload(1)
    assert (w1.B, w1.T, w1.H) == (1, 8192, 64)
    w2 = kda_inputs.workload(2)
    assert w2.lengths == [1024] * 8 and w2.state == 'fp32'
    w3 = kda_inputs.workload(3)
    assert len(w3.lengths) == 32 and all(64 <= L <= 4096 for L in w3.lengths)
    assert w3.T == sum(w3.lengths) and w3.state == 'bf16' and w3.lower_bound == -2.0
    w4 = kda_inputs.workload(4)
    assert (w4.B, w4.T, w4.H, w4.state) == (4, 32768, 64, 'fp32')
    w5 = kda_inputs.workload(5)
    assert w5.lengths == [1] * 256 and (w5.T, w5.H, w5.state, w5.final) == (256, 64, 'fp32', 'fp32')


def test_distribution_moments():
    d = kda_inputs.make_inputs(kda_inputs.custom(T=4096, H=4, state='fp32'))
    for n in ('q', 'k', 'v', 'g'):
        x = d[n].float()
        assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1) < 0.01, n
    s = d['initial_state']
    assert abs(float(s.std()) - 0.02) < 0.001
