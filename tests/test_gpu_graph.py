"""HIP graph capture of both entry points (GPU).

A serving loop captures its per-step work once and replays it. kda_fwd and
kda_fwd_recurrent allocate nothing when the workspace is passed in, launch only
kernels on the caller's stream and never synchronise, so they can be captured.
Each test captures one call, then replays it several times with new input
contents copied into the captured buffers, with eager work and synchronisations
between the replays, and requires every replay to equal an eager call on the
same inputs bit for bit (same kernels, deterministic).
"""
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


def _inputs(w, seed, device):
    w.seed = seed
    d = kda_inputs.make_inputs(w)
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def test_graph_replay_chunked():
    device = dev()
    w = kda_inputs.custom(lengths=[70, 0, 130, 5, 64], H=3, state='fp32')
    say("graph capture of kda_fwd (varlen, fp32 state), 3 replays")
    x = _inputs(w, 0, device)
    B, T, H = x['q'].shape[:3]
    out = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device=device)
    fin = torch.empty(w.n_seqs, H, 128, 128, dtype=torch.float32, device=device)
    ws = torch.empty(kda.workspace_size(B, T, H, w.n_seqs), dtype=torch.uint8, device=device)

    def call(o, f):
        kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], o, x['A_log'], x['dt_bias'],
                x['lower_bound'], initial_state=x['initial_state'], final_state=f, cu_seqlens=x['cu_seqlens'],
                workspace=ws)

    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream(device))
    with torch.cuda.stream(side):   # warm-up outside the capture
        call(out, fin)
    torch.cuda.current_stream(device).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, fin)
    for rep, seed in enumerate([1, 2, 3]):
        nx = _inputs(w, seed, device)
        for n in ('q', 'k', 'v', 'g', 'beta', 'A_log', 'dt_bias', 'initial_state'):
            x[n].copy_(nx[n])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_ref = torch.empty_like(out)
        f_ref = torch.empty_like(fin)
        call(o_ref, f_ref)   # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), f"replay {rep}: out differs from the eager call"
        assert torch.equal(fin, f_ref), f"replay {rep}: final state differs from the eager call"


def test_graph_replay_decode_loop():
    """A decode loop: one token per sequence per step, the state updated in place
    (initial_state is final_state); 4 replays of the captured step against 4 eager steps."""
    device = dev()
    N, H = 64, 8
    w = kda_inputs.custom(lengths=[1] * N, H=H, state='fp32')
    say(f"graph capture of kda_fwd_recurrent, decode step of {N} sequences x {H} heads, 4 replays")
    x = _inputs(w, 10, device)
    st0 = x['initial_state'].clone()
    out = torch.empty(1, N, H, 128, dtype=torch.bfloat16, device=device)
    state = st0.clone()

    def step(o, s):
        kda.fwd_recurrent(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], o, x['A_log'], x['dt_bias'],
                          x['lower_bound'], initial_state=s, final_state=s, cu_seqlens=x['cu_seqlens'])

    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream(device))
    with torch.cuda.stream(side):
        step(out, state)
    torch.cuda.current_stream(device).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out, state)
    state.copy_(st0)
    ref_state = st0.clone()
    for t in range(4):
        nx = _inputs(w, 20 + t, device)
        for n in ('q', 'k', 'v', 'g', 'beta'):
            x[n].copy_(nx[n])
        torch.cuda.synchronize()
        g.replay()
        o_ref = torch.empty_like(out)
        step(o_ref, ref_state)   # eager twin of the same step
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), f"step {t}: out differs from the eager step"
        assert torch.equal(state, ref_state), f"step {t}: state differs from the eager step"


def test_graph_replay_segmented_chain():
    """The segment-parallel chain (maps pass, scan, outputs pass) captured and replayed."""
    device = dev()
    w = kda_inputs.custom(B=1, T=4096, H=2, state='fp32', lower_bound=-0.05)
    say("graph capture of kda_fwd with the segmented chain (T=4096, H=2), 3 replays")
    x = _inputs(w, 0, device)
    B, T, H = x['q'].shape[:3]
    out = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device=device)
    fin = torch.empty(B, H, 128, 128, dtype=torch.float32, device=device)
    ws = torch.empty(kda.workspace_size(B, T, H), dtype=torch.uint8, device=device)

    def call(o, f):
        kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], o, x['A_log'], x['dt_bias'],
                x['lower_bound'], initial_state=x['initial_state'], final_state=f, workspace=ws)

    side = torch.cuda.Stream(device)
    side.wait_stream(torch.cuda.current_stream(device))
    with torch.cuda.stream(side):
        call(out, fin)
    torch.cuda.current_stream(device).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, fin)
    for rep, seed in enumerate([1, 2, 3]):
        nx = _inputs(w, seed, device)
        for n in ('q', 'k', 'v', 'g', 'beta', 'A_log', 'dt_bias', 'initial_state'):
            x[n].copy_(nx[n])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_ref, f_ref = torch.empty_like(out), torch.empty_like(fin)
        call(o_ref, f_ref)
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref) and torch.equal(fin, f_ref), f"replay {rep} differs from the eager call"
