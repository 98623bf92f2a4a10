"""GPU: fixed-length calls given less workspace than kda_fwd_workspace_size run in windows
of chunk columns (kda_fwd_workspace_min in include/kda.h). Each window runs the same
per-chunk arithmetic as one full launch and the state crosses windows in fp32, so a
windowed call must return the same bits as the unwindowed one: out and final_state are
compared bit for bit against the full-workspace call (itself checked against the oracle
in test_gpu_parity), and one windowed case is also compared with the oracle directly.
"""
import ctypes

import numpy as np
import pytest
import torch

import kda_inputs
from oracle import kda_oracle
import gated_delta_rule_87_amd as kda

pytestmark = pytest.mark.gpu

CH = 64


def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def say(*a):
    print("[gpu-test]", *a, flush=True)


def inputs(B, T, H, seed, state):
    w = kda_inputs.Workload(f"win_B{B}_T{T}_H{H}", B=B, T=T, H=H, state=state, seed=seed)
    d = kda_inputs.make_inputs(w)
    return {k: (v.to(dev()) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def ws_for_width(B, T, H, width, own_carry):
    """Workspace bytes that give windows of `width` chunk columns (the plan takes the
    fewest windows that fit, then balances their widths)."""
    col = B * H * kda.record_bytes()
    carry = -(-(B * H * 128 * 128 * 4) // 256) * 256 if own_carry else 0
    return carry + width * col


def run(x, B, T, H, ws_bytes, fin_dtype, init=None, alias=False, safe_gate=True):
    out = torch.full((B, T, H, 128), float('nan'), dtype=torch.bfloat16, device=dev())
    fin = None
    if alias:
        fin = init
    elif fin_dtype is not None:
        fin = torch.full((B, H, 128, 128), float('nan'), dtype=fin_dtype, device=dev())
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev())
    kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'],
            x['lower_bound'], initial_state=init, final_state=fin, workspace=ws, safe_gate=safe_gate)
    torch.cuda.synchronize()
    return out, fin


# (B, T, H): ragged last chunk, several rows, a row of one chunk
SHAPES = [(2, 1000, 4), (3, 448, 2), (1, 64, 3)]
STATES = [  # (initial dtype, final dtype, final aliases initial)
    (None, None, False), (None, torch.float32, False), (torch.float32, torch.float32, False),
    (torch.bfloat16, torch.bfloat16, False), (torch.float32, None, False), (torch.float32, torch.float32, True),
    (torch.bfloat16, torch.bfloat16, True)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("states", STATES)
def test_windowed_bit_identical(shape, states):
    B, T, H = shape
    idt, fdt, alias = states
    nc_row = -(-T // CH)
    x = inputs(B, T, H, seed=B * 100 + T, state={None: None, torch.float32: 'fp32', torch.bfloat16: 'bf16'}[idt])
    init = x['initial_state']
    full = kda.workspace_size(B, T, H)
    ref_init = init.clone() if (alias and init is not None) else init
    o_ref, f_ref = run(x, B, T, H, full, fdt, init=ref_init.clone() if alias else ref_init, alias=alias)
    own_carry = fdt is not torch.float32
    widths = sorted({1, 2, max(1, nc_row // 3), nc_row - 1} - {0})
    for width in widths:
        if width >= nc_row:
            continue
        wsb = ws_for_width(B, T, H, width, own_carry)
        assert wsb < full and (not own_carry or kda.workspace_min(B, T, H) <= wsb)
        o, f = run(x, B, T, H, wsb, fdt, init=ref_init.clone() if alias else init, alias=alias)
        say(f"B={B} T={T} H={H} states={states} width={width}: windows={-(-nc_row // width)}")
        assert torch.isfinite(o.float()).all()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"out differs at width {width}"
        if f_ref is not None:
            assert torch.equal(f.view(torch.int16) if f.dtype == torch.bfloat16 else f.view(torch.int32),
                               f_ref.view(torch.int16) if f_ref.dtype == torch.bfloat16 else f_ref.view(torch.int32)), \
                f"final_state differs at width {width}"


def test_windowed_unbounded_gate_bit_identical():
    B, T, H = 2, 700, 3
    x = inputs(B, T, H, seed=7, state='fp32')
    o_ref, f_ref = run(x, B, T, H, kda.workspace_size(B, T, H), torch.float32, init=x['initial_state'],
                       safe_gate=False)
    o, f = run(x, B, T, H, ws_for_width(B, T, H, 3, False), torch.float32, init=x['initial_state'],
               safe_gate=False)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(f.view(torch.int32), f_ref.view(torch.int32))


def test_windowed_against_oracle():
    """One windowed call (windows of 2 chunk columns, own carry) against the fp64 oracle."""
    B, T, H = 2, 600, 2
    x = inputs(B, T, H, seed=11, state='bf16')
    o, f = run(x, B, T, H, ws_for_width(B, T, H, 2, True), torch.bfloat16, init=x['initial_state'])
    c = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    ro, rf = kda_oracle(c['q'], c['k'], c['v'], c['g'], c['beta'], c['scale'], c['A_log'], c['dt_bias'],
                        c['lower_bound'], initial_state=c['initial_state'], cu_seqlens=None)
    on = o.float().cpu().numpy().astype(np.float64)
    ro = np.asarray(ro, np.float64).reshape(on.shape)
    rel = np.linalg.norm(on - ro) / np.linalg.norm(ro)
    frel = np.linalg.norm(f.float().cpu().numpy() - np.asarray(rf).reshape(f.shape)) / np.linalg.norm(rf)
    say(f"windowed vs oracle: out max-abs {np.abs(on - ro).max():.3e} rel-L2 {rel:.3e}, final rel-L2 {frel:.3e}")
    assert np.abs(on - ro).max() <= 2e-2 and rel <= 5e-3 and frel <= 5e-3


def test_workspace_below_minimum_rejected():
    B, T, H = 1, 256, 2
    x = inputs(B, T, H, seed=3, state=None)
    out = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device=dev())
    ws = torch.empty(kda.workspace_min(B, T, H) - 256, dtype=torch.uint8, device=dev())
    with pytest.raises(kda.KDAError):
        kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'],
                x['lower_bound'], workspace=ws)


def test_windowed_instead_of_segmented_chain():
    """Few (row, head) chains on a long row: the full workspace runs the segment-parallel
    chain, a windowed call the plain chain window by window. The two differ in rounding
    order, so both are compared with the oracle (lower_bound near 0, so that the state
    carries across segments and windows)."""
    B, T, H = 1, 4096, 2
    w = kda_inputs.custom(B=B, T=T, H=H, state='fp32', lower_bound=-0.05, seed=21)
    d = kda_inputs.make_inputs(w)
    x = {k: (v.to(dev()) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    full = kda.workspace_size(B, T, H)
    assert full > (T // CH) * H * kda.record_bytes()   # the segment maps and states come on top
    ro, rf = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                        d['lower_bound'], initial_state=d['initial_state'], cu_seqlens=None)
    for wsb, tag in ((full, "segmented"), (ws_for_width(B, T, H, 16, False), "windowed x16")):
        o, f = run(x, B, T, H, wsb, torch.float32, init=x['initial_state'])
        on = o.float().cpu().numpy().astype(np.float64).reshape(np.asarray(ro).shape)
        rel = np.linalg.norm(on - ro) / np.linalg.norm(ro)
        frel = np.linalg.norm(f.cpu().numpy() - rf) / np.linalg.norm(rf)
        say(f"{tag}: out max-abs {np.abs(on - ro).max():.3e} rel-L2 {rel:.3e}, final rel-L2 {frel:.3e}")
        assert np.abs(on - ro).max() <= 2e-2 and rel <= 5e-3 and frel <= 2e-3


# ---- varlen calls in windows of chunk slots --------------------------------------------

def al(x):
    return -(-x // 256) * 256


def vws_for_width(T, H, N, width):
    """Workspace bytes that give varlen windows of `width` chunk slots (tables, two carry
    slots of fp32 state and `width` slots of records; see plan_vwindows)."""
    mc = T // CH + N
    fixed = 2 * al(N * 8) + al(mc * 8) + 2 * al(N * 4) + al((mc + 1) * 4) + al(2 * H * 128 * 128 * 4)
    return fixed + width * H * kda.record_bytes()


def vinputs(lengths, H, seed, state, lower_bound=-5.0):
    w = kda_inputs.custom(lengths=lengths, H=H, state=state, final=state or 'fp32', seed=seed,
                          lower_bound=lower_bound)
    d = kda_inputs.make_inputs(w)
    return w, {k: (v.to(dev()) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def vrun(w, x, ws_bytes, fin_dtype, init=None, alias=False, safe_gate=True):
    T, H, N = w.T, w.H, w.n_seqs
    out = torch.full((1, T, H, 128), float('nan'), dtype=torch.bfloat16, device=dev())
    fin = init if alias else (None if fin_dtype is None else
                              torch.full((N, H, 128, 128), float('nan'), dtype=fin_dtype, device=dev()))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev())
    kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'],
            x['lower_bound'], initial_state=init, final_state=fin, cu_seqlens=x['cu_seqlens'], workspace=ws,
            safe_gate=safe_gate)
    torch.cuda.synchronize()
    return out, fin


def same_bits(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


# lengths: empty sequences, one token, exact chunk multiples, long ones crossing many windows
VLENGTHS = [
    [700, 0, 3, 1500, 64, 0, 129, 1],
    [0, 0, 2000],
    [64] * 12 + [1000],
    [5, 0, 0, 7, 300, 0],
]


@pytest.mark.parametrize("lengths", VLENGTHS)
@pytest.mark.parametrize("states", [(None, torch.float32, False), (torch.float32, torch.float32, False),
                                    (torch.bfloat16, torch.bfloat16, False), (torch.float32, torch.float32, True),
                                    (torch.bfloat16, None, False)])
def test_varlen_windowed_bit_identical(lengths, states):
    idt, fdt, alias = states
    H = 3
    sname = {None: None, torch.float32: 'fp32', torch.bfloat16: 'bf16'}[idt]
    w, x = vinputs(lengths, H, seed=len(lengths) * 7 + sum(lengths) % 97, state=sname)
    T, N = w.T, w.n_seqs
    init = x['initial_state']
    full = kda.workspace_size(1, T, H, N)
    o_ref, f_ref = vrun(w, x, full, fdt, init=init.clone() if alias else init, alias=alias)
    mc = T // CH + N
    for width in sorted({1, 2, 5, max(1, mc // 2)}):
        if width >= mc:
            continue
        wsb = vws_for_width(T, H, N, width)
        assert kda.workspace_min(1, T, H, N) <= wsb < full
        o, f = vrun(w, x, wsb, fdt, init=init.clone() if alias else init, alias=alias)
        say(f"lengths={lengths} states={states} width={width}: windows={-(-mc // width)}")
        assert same_bits(o, o_ref), f"out differs at width {width}"
        if f_ref is not None:
            assert same_bits(f, f_ref), f"final_state differs at width {width}"


def test_varlen_windowed_unbounded_gate_and_oracle():
    lengths = [300, 0, 900, 17]
    w, x = vinputs(lengths, 2, seed=5, state='fp32')
    T, H, N = w.T, w.H, w.n_seqs
    for safe in (True, False):
        o_ref, f_ref = vrun(w, x, kda.workspace_size(1, T, H, N), torch.float32, init=x['initial_state'],
                            safe_gate=safe)
        o, f = vrun(w, x, vws_for_width(T, H, N, 3), torch.float32, init=x['initial_state'], safe_gate=safe)
        assert same_bits(o, o_ref) and same_bits(f, f_ref), f"safe_gate={safe}"
    c = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    ro, rf = kda_oracle(c['q'], c['k'], c['v'], c['g'], c['beta'], c['scale'], c['A_log'], c['dt_bias'],
                        c['lower_bound'], initial_state=c['initial_state'], cu_seqlens=c['cu_seqlens'],
                        safe_gate=False)
    on = o.float().cpu().numpy().astype(np.float64).reshape(np.asarray(ro).shape)
    rel = np.linalg.norm(on - ro) / np.linalg.norm(ro)
    frel = np.linalg.norm(f.cpu().numpy() - rf) / np.linalg.norm(rf)
    say(f"varlen windowed (unbounded) vs oracle: out max-abs {np.abs(on - ro).max():.3e} rel-L2 {rel:.3e}, "
        f"final rel-L2 {frel:.3e}")
    assert np.abs(on - ro).max() <= 2e-2 and rel <= 5e-3 and frel <= 2e-3
