"""The per-kernel timing hook of kda_fwd on the GPU.

While timing is on, each call records HIP events around its kernels. The
results must not change, every kernel a call launches must be counted once
per call (the varlen scheduler only when cu_seqlens is given), and the timed
intervals must be positive and fit inside the wall time of the calls.
"""
import time

import pytest
import torch

import kda_inputs
import gated_delta_rule_87_amd as kda

pytestmark = pytest.mark.gpu


def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def say(*a):
    print("[gpu-test]", *a, flush=True)


@pytest.mark.parametrize("varlen", [False, True], ids=["fixed", "varlen"])
def test_profile_hook_counts_and_results(varlen):
    device = dev()
    if varlen:
        w = kda_inputs.custom(lengths=[70, 0, 130, 5, 64], H=3, state='fp32')
    else:
        w = kda_inputs.custom(B=2, T=200, H=3, state='bf16', final='bf16')
    say(f"timing hook, {w.name}")
    x = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in kda_inputs.make_inputs(w).items()}
    B, T, H = x['q'].shape[:3]
    sdt = torch.float32 if w.final == 'fp32' else torch.bfloat16

    def call():
        out = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device=device)
        fin = torch.empty(w.n_seqs, H, 128, 128, dtype=sdt, device=device)
        kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'],
                x['lower_bound'], initial_state=x['initial_state'], final_state=fin, cu_seqlens=x['cu_seqlens'])
        return out, fin

    ref_out, ref_fin = call()
    torch.cuda.synchronize()
    calls = 3
    kda.profile_start(calls + 2)   # more slots than calls: the unused ones must not count
    t0 = time.perf_counter()
    res = [call() for _ in range(calls)]
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    per = kda.profile_stop()
    for out, fin in res:
        assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin), "timing changed the results"
    want = {"kda_sched_kernel": calls if varlen else 0, "kda_intra_kernel": calls, "kda_chain_kernel": calls}
    assert {k: n for k, (_, n) in per.items()} == want
    for name, (ms, n) in per.items():
        if n:
            assert 0.0 < ms <= wall_ms, (name, ms, wall_ms)
    assert sum(ms for ms, _ in per.values()) <= wall_ms
    with pytest.raises(kda.KDAError):
        kda.profile_stop()   # timing is off again
