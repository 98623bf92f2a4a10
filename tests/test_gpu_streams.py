"""Reentrancy of the C ABI on the GPU.

kda_fwd and kda_fwd_recurrent keep no state between calls and write only the
caller's buffers and workspace, so calls on different streams may run at the
same time, and different host threads may call at once. Each test runs calls
that overlap in both ways and requires every result to equal the same call run
alone, bit for bit (the kernels are deterministic). All streams keep the
default priority.
"""
import threading

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


class Job:
    """One forward call with its own inputs, outputs and workspace."""

    def __init__(self, w, seed, device, path="chunked"):
        w.seed = seed
        self.x = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in kda_inputs.make_inputs(w).items()}
        B, T, H = self.x['q'].shape[:3]
        self.path = path
        self.out = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device=device)
        self.fin = torch.empty(w.n_seqs, H, 128, 128, dtype=torch.float32, device=device)
        N = w.n_seqs if self.x['cu_seqlens'] is not None else 0
        self.ws = torch.empty(max(1, kda.workspace_size(B, T, H, N)), dtype=torch.uint8, device=device)

    def __call__(self):
        x = self.x
        if self.path == "chunked":
            kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], self.out, x['A_log'], x['dt_bias'],
                    x['lower_bound'], initial_state=x['initial_state'], final_state=self.fin,
                    cu_seqlens=x['cu_seqlens'], workspace=self.ws, force_chunked=True)
        else:
            kda.fwd_recurrent(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], self.out, x['A_log'],
                              x['dt_bias'], x['lower_bound'], initial_state=x['initial_state'],
                              final_state=self.fin, cu_seqlens=x['cu_seqlens'])

    def result(self):
        return self.out.clone(), self.fin.clone()


def jobs(device):
    return [Job(kda_inputs.custom(lengths=[300, 0, 70, 129], H=4, state='fp32'), 1, device),
            Job(kda_inputs.custom(B=2, T=1000, H=3, state='fp32', lower_bound=-1.0), 2, device),
            Job(kda_inputs.custom(lengths=[1] * 64, H=8, state='fp32'), 3, device, path="recurrent")]


def references(js):
    refs = []
    for j in js:   # each call alone on the current stream
        j()
        torch.cuda.synchronize()
        refs.append(j.result())
    return refs


def test_calls_on_concurrent_streams():
    device = dev()
    js = jobs(device)
    refs = references(js)
    say("three calls on three streams, enqueued together, three rounds")
    streams = [torch.cuda.Stream(device) for _ in js]
    for rnd in range(3):
        for j in js:   # results of the round before must not leak into this one
            j.out.zero_()
            j.fin.zero_()
        torch.cuda.synchronize()
        for j, st in zip(js, streams):
            st.wait_stream(torch.cuda.current_stream(device))
            with torch.cuda.stream(st):
                j()
        torch.cuda.synchronize()
        for i, (j, (ro, rf)) in enumerate(zip(js, refs)):
            o, f = j.result()
            assert torch.equal(o, ro) and torch.equal(f, rf), f"round {rnd}: call {i} differs from its lone run"


def test_calls_from_two_host_threads():
    device = dev()
    js = jobs(device)[:2]
    refs = references(js)
    say("two host threads, each calling on its own stream, five calls each")
    errors = []

    def worker(j, ref, rounds):
        try:
            st = torch.cuda.Stream(device)
            for _ in range(rounds):
                with torch.cuda.stream(st):
                    j()
                st.synchronize()
                o, f = j.result()
                if not (torch.equal(o, ref[0]) and torch.equal(f, ref[1])):
                    errors.append("a threaded call differs from its lone run")
        except Exception as e:   # reported in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(j, r, 5)) for j, r in zip(js, refs)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
