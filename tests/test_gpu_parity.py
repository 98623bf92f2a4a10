"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (whole tensor): out max-abs <= 2e-2 and rel-L2 <= 5e-3;
final_state rel-L2 <= 2e-3 for fp32 state and <= 5e-3 for bf16 state (bf16
rounding of the state alone costs ~1.6e-3). rel-L2 = ||x - ref|| / ||ref||.

Full-size workloads are compared on every head, element by element, at the real
shape and in the same launch configuration the bench times: finiteness over the
whole out and final_state first, then the oracle in batches of heads (every
(sequence, head) chain is independent), with the errors summed over the whole
tensor. Each comparison records its margins (tests/parity_margins.py), which the
session prints at its end.
"""
import functools
import math

import numpy as np
import pytest
import torch

import kda_inputs
import parity_margins
from oracle import kda_oracle
import gated_delta_rule_87_amd as kda

pytestmark = pytest.mark.gpu

OUT_MAXABS, OUT_REL = 2e-2, 5e-3
FIN_REL = {'fp32': 2e-3, 'bf16': 5e-3}


def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def say(*a):
    print("[gpu-test]", *a, flush=True)


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return np.linalg.norm(x - ref) / (den if den > 0 else 1.0)


def to_dev(d, device):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def run_dev(d, w, path="chunked", final=None, out_fill=0.0, **kw):
    """Run the HIP path on inputs d (CPU tensors). Returns the device tensors (out, final or None)."""
    device = dev()
    x = to_dev(d, device)
    B, T, H = x['q'].shape[:3]
    out = torch.full((B, T, H, 128), out_fill, dtype=torch.bfloat16, device=device)
    fdt = w.final if final is None else final
    fin = None
    if fdt is not None:
        fin = torch.full((w.n_seqs, H, 128, 128), float('nan'),
                         dtype=torch.float32 if fdt == 'fp32' else torch.bfloat16, device=device)
    if path == "chunked":   # the chunked kernels, also for decode-sized calls
        fn = functools.partial(kda.fwd, force_chunked=True)
    elif path == "auto":    # kda_fwd's own choice
        fn = kda.fwd
    else:
        fn = kda.fwd_recurrent
    fn(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'], x['lower_bound'],
       initial_state=x['initial_state'], final_state=fin, cu_seqlens=x['cu_seqlens'], **kw)
    torch.cuda.synchronize()
    return out, fin


def run(d, w, path="chunked", final=None, out_fill=0.0):
    """Run the HIP path on inputs d (CPU tensors). Returns (out [B*T,H,V] fp64, final fp64 or None)."""
    out, fin = run_dev(d, w, path, final, out_fill)
    B, T, H = out.shape[:3]
    o = out.float().double().cpu().numpy().reshape(B * T, H, 128)
    f = fin.float().double().cpu().numpy() if fin is not None else None
    return o, f


def check(o, f, ro, rf, fdt, tag, heads=None):
    if o.size:
        assert np.isfinite(o).all(), f"{tag}: non-finite output"
    if f is not None:
        assert np.isfinite(f).all(), f"{tag}: non-finite final state"
    if heads is not None:
        o = o[:, heads]
        f = f[:, heads] if f is not None else None
    mae = float(np.abs(o - ro).max()) if o.size else 0.0
    r = rel_l2(o, ro) if o.size else 0.0
    msg = f"{tag}: out max-abs {mae:.3e} rel-L2 {r:.3e}"
    fr = None
    if f is not None:
        fr = rel_l2(f, rf)
        msg += f" | final rel-L2 {fr:.3e}"
    say(msg)
    parity_margins.record(tag, False, mae, r, fr, FIN_REL[fdt] if f is not None else None)
    assert mae <= OUT_MAXABS and r <= OUT_REL, msg
    if f is not None:
        assert fr <= FIN_REL[fdt], msg


class HeadErrors:
    """Errors summed over a whole (tokens, heads, V) output and (seqs, heads, V, K) state,
    fed one batch of heads at a time."""

    def __init__(self, H):
        self.o_num = np.zeros(H)
        self.o_den = np.zeros(H)
        self.f_num = np.zeros(H)
        self.f_den = np.zeros(H)
        self.mae = 0.0

    def add(self, h0, o, ro, f=None, rf=None):
        hs = slice(h0, h0 + ro.shape[1])
        if o.size:
            diff = o.astype(np.float64) - ro
            self.mae = max(self.mae, float(np.abs(diff).max()))
            self.o_num[hs] = np.einsum('thv,thv->h', diff, diff)
            self.o_den[hs] = np.einsum('thv,thv->h', ro, ro)
            del diff
        if f is not None:
            df = f.astype(np.float64) - rf
            self.f_num[hs] = np.einsum('nhvk,nhvk->h', df, df)
            self.f_den[hs] = np.einsum('nhvk,nhvk->h', rf, rf)

    @staticmethod
    def _rel(num, den):
        d = float(den.sum())
        return math.sqrt(float(num.sum()) / (d if d > 0 else 1.0))

    def check(self, tag, fdt, with_final=True):
        r = self._rel(self.o_num, self.o_den)
        per_head = np.sqrt(self.o_num / np.where(self.o_den > 0, self.o_den, 1.0))
        wh = int(np.argmax(per_head))
        msg = (f"{tag} (all {len(per_head)} heads): out max-abs {self.mae:.3e} rel-L2 {r:.3e} "
               f"(worst head {wh}: {per_head[wh]:.3e})")
        fr = None
        if with_final:
            fr = self._rel(self.f_num, self.f_den)
            msg += f" | final rel-L2 {fr:.3e}"
        say(msg)
        parity_margins.record(tag, True, self.mae, r, fr, FIN_REL[fdt] if with_final else None,
                              f"h{wh} {per_head[wh]:.2e}")
        assert self.mae <= OUT_MAXABS and r <= OUT_REL, msg
        if with_final:
            assert fr <= FIN_REL[fdt], msg


def compare_all_heads(out, fin, d, fdt, tag, batch=16, **oracle_kw):
    """Device results (out [B,T,H,V] bf16, fin [nseq,H,V,K] or None) against the oracle on
    every head. Finiteness is asserted over the whole tensors before any comparison."""
    assert bool(torch.isfinite(out).all()), f"{tag}: non-finite output"
    if fin is not None:
        assert bool(torch.isfinite(fin.float()).all()), f"{tag}: non-finite final state"
    H = out.shape[2]
    o_all = out.float().cpu().numpy().reshape(-1, H, 128)
    f_all = fin.float().cpu().numpy() if fin is not None else None
    errs = HeadErrors(H)
    for h0 in range(0, H, batch):
        h1 = min(H, h0 + batch)
        ro, rf = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                            d['lower_bound'], initial_state=d['initial_state'], cu_seqlens=d['cu_seqlens'],
                            heads=list(range(h0, h1)), want_final=fin is not None, **oracle_kw)
        errs.add(h0, o_all[:, h0:h1], ro, None if f_all is None else f_all[:, h0:h1], rf)
        del ro, rf
    errs.check(tag, fdt, with_final=fin is not None)
    return errs


def oracle_for(d, heads=None):
    return kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                      d['lower_bound'], initial_state=d['initial_state'], cu_seqlens=d['cu_seqlens'],
                      heads=heads)


# ---------------------------------------------------------------------------
SMALL = [
    dict(B=1, T=256, H=2),                                          # the tiny workload's shape
    dict(B=1, T=200, H=3, state='fp32', lower_bound=-5.0),          # 3 chunks + ragged tail
    dict(B=2, T=130, H=2, state='bf16', final='bf16', lower_bound=-2.0),
    dict(B=1, T=64, H=1, lower_bound=0.0),                          # decay-free
    dict(B=1, T=1, H=2, state='fp32', lower_bound=-0.1),
    dict(B=3, T=17, H=4, state='fp32', lower_bound=-1.0, seed=5),
    dict(lengths=[0, 1, 15, 16, 17, 63, 64, 65, 127, 129], H=2, state='fp32'),
    dict(lengths=[1] * 40 + [3] * 10 + [0, 0], H=3, state='bf16', final='bf16', lower_bound=-3.0),
    dict(lengths=[300, 0, 5], H=2, final=None),
    dict(B=1, T=333, H=2, state='fp32', lower_bound=-0.01, seed=7),  # near decay-free, long
]


@pytest.mark.parametrize("path", ["chunked", "recurrent"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_parity(case, path):
    w = kda_inputs.custom(**SMALL[case])
    say(f"small case {case} {SMALL[case]} path={path}")
    d = kda_inputs.make_inputs(w)
    ro, rf = oracle_for(d)
    o, f = run(d, w, path)
    check(o, f, ro, rf if w.final else None, w.final, f"case{case}/{path}")


def test_tiny_workload_full():
    w = kda_inputs.workload(0)
    say("workload 0 (tiny)")
    d = kda_inputs.make_inputs(w)
    ro, rf = oracle_for(d)
    o, f = run(d, w)
    check(o, f, ro, rf, 'fp32', "tiny")


def test_out_fully_written_deterministic_and_aliasing():
    w = kda_inputs.custom(lengths=[70, 1, 0, 200], H=2, state='fp32')
    say("NaN-prefilled out, determinism, initial==final aliasing")
    d = kda_inputs.make_inputs(w)
    o1, f1 = run(d, w, out_fill=float('nan'))
    assert np.isfinite(o1).all(), "some out element was not written"
    o2, f2 = run(d, w, out_fill=float('nan'))
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2), "run-to-run results differ"
    device = dev()
    x = to_dev(d, device)
    st = x['initial_state'].clone()
    out = torch.empty(1, w.T, 2, 128, dtype=torch.bfloat16, device=device)
    kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'],
            x['lower_bound'], initial_state=st, final_state=st, cu_seqlens=x['cu_seqlens'])
    torch.cuda.synchronize()
    assert np.array_equal(st.double().cpu().numpy(), f1)
    assert np.array_equal(out.float().double().cpu().numpy().reshape(-1, 2, 128), o1)


@pytest.mark.parametrize("path", ["chunked", "recurrent"])
@pytest.mark.parametrize("shape", [dict(B=2, T=0, H=3, state='fp32'),
                                   dict(B=1, T=0, H=2, state='bf16', final='bf16'),
                                   dict(B=2, T=0, H=2),
                                   dict(lengths=[0, 0, 0], H=2, state='fp32')],
                         ids=["fixed_fp32", "fixed_bf16", "fixed_stateless", "varlen_fp32"])
def test_empty_input(shape, path):
    """No tokens at all (T = 0: the token tensors are empty and their data pointers NULL):
    final_state is written for every (sequence, head) and equals the initial state bit for
    bit, or zeros without one; the oracle agrees."""
    w = kda_inputs.custom(**shape)
    say(f"empty input {shape} path={path}")
    d = kda_inputs.make_inputs(w)
    assert d['q'].numel() == 0
    o, f = run(d, w, path)
    ro, rf = oracle_for(d)
    assert o.size == 0 and ro.size == 0
    ref = d['initial_state'].double().numpy() if d['initial_state'] is not None else np.zeros_like(f)
    assert np.array_equal(f, ref), "final_state differs from the initial state"
    assert np.array_equal(rf, ref)


def test_beta_zero_zero_state_exact():
    """beta logits -inf and no initial state: out and final_state are exactly 0."""
    w = kda_inputs.custom(T=150, H=2)
    d = kda_inputs.make_inputs(w)
    d['beta'] = torch.full_like(d['beta'], float('-inf'))
    o, f = run(d, w)
    assert np.all(o == 0) and np.all(f == 0)


@pytest.mark.parametrize("path", ["chunked", "recurrent"])
def test_edge_values(path):
    """All-zero query and key rows (they normalise to zero, not NaN), beta logits of +inf
    (beta = 1) and -inf (beta = 0), and rows scaled by 2^10 (the L2 norm removes the
    scale), in and across chunks, against the oracle."""
    w = kda_inputs.custom(B=1, T=200, H=2, state='fp32', lower_bound=-2.0, seed=3)
    d = kda_inputs.make_inputs(w)
    for t in (3, 64, 130):
        d['q'][0, t] = 0
    for t in (5, 65, 131, 199):
        d['k'][0, t] = 0
    for t in (7, 100):
        d['beta'][0, t] = float('inf')
    for t in (8, 101, 102):
        d['beta'][0, t] = float('-inf')
    for t in (20, 90):
        d['q'][0, t] *= 1024
        d['k'][0, t + 1] *= 1024
    say(f"edge values (zero rows, beta logits +-inf, 2^10-scaled rows) path={path}")
    ro, rf = oracle_for(d)
    o, f = run(d, w, path)
    check(o, f, ro, rf, 'fp32', f"edge values/{path}")


# ---------------------------------------------------------------------------
# kda_fwd's own choice of path: decode-sized calls go to the token-recurrent kernel
@pytest.mark.parametrize("shape,expect", [
    (dict(B=2, T=8, H=3, state='fp32'), "recurrent"),
    (dict(B=1, T=9, H=2, state='fp32', lower_bound=-1.0), "chunked"),
    (dict(lengths=[1] * 20 + [3, 0], H=2, state='fp32'), "recurrent"),      # 23 tokens, 22 sequences
    (dict(lengths=[40, 1, 1, 2], H=2, state='bf16', final='bf16'), "chunked"),  # 44 tokens, 4 sequences
], ids=["fixed_T8", "fixed_T9", "varlen_decode", "varlen_44_over_4"])
def test_auto_path(shape, expect, capfd, monkeypatch):
    w = kda_inputs.custom(**shape)
    say(f"path chosen by kda_fwd for {shape}: expect {expect}")
    d = kda_inputs.make_inputs(w)
    ro, rf = oracle_for(d)
    monkeypatch.setenv("KDA_LOG", "1")
    o, f = run(d, w, "auto")
    err = capfd.readouterr().err
    assert ("path=recurrent" in err) == (expect == "recurrent"), err
    check(o, f, ro, rf, w.final, f"auto path {expect}")


@pytest.mark.parametrize("entry", ["kda_fwd", "kda_fwd_recurrent"])
def test_plain_exports(entry):
    """The plain C entry points (all input processing fused, safe gate), called through
    ctypes with device pointers, against the oracle."""
    import ctypes
    w = kda_inputs.custom(lengths=[150, 3, 0, 77], H=2, state='fp32', lower_bound=-3.0)
    say(f"plain export {entry}, {w.lengths}")
    d = kda_inputs.make_inputs(w)
    device = dev()
    x = to_dev(d, device)
    B, T, H = x['q'].shape[:3]
    N = w.n_seqs
    out = torch.full((B, T, H, 128), float('nan'), dtype=torch.bfloat16, device=device)
    fin = torch.full((N, H, 128, 128), float('nan'), dtype=torch.float32, device=device)
    L = kda.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    args = (P(x['q']), P(x['k']), P(x['v']), P(x['g']), P(x['beta']), x['scale'], P(out), P(x['A_log']),
            P(x['dt_bias']), x['lower_bound'], P(x['initial_state']), kda.STATE_FP32, P(fin), kda.STATE_FP32,
            P(x['cu_seqlens']), N, B, T, H, 128, 128)
    if entry == "kda_fwd":
        ws = torch.empty(kda.workspace_size(B, T, H, N), dtype=torch.uint8, device=device)
        rc = L.kda_fwd(*args, P(ws), ws.numel(), stream)
    else:
        rc = L.kda_fwd_recurrent(*args, stream)
    assert rc == 0, kda.status_string(rc)
    torch.cuda.synchronize()
    ro, rf = oracle_for(d)
    check(out.float().double().cpu().numpy().reshape(B * T, H, 128), fin.double().cpu().numpy(), ro, rf, 'fp32',
          f"plain {entry}")


# ---------------------------------------------------------------------------
# full-size workloads, every head
@pytest.mark.parametrize("idx", [1, 2, 3])
def test_full_size_all_heads(idx):
    w = kda_inputs.workload(idx)
    say(f"workload {idx} {w.name}: all heads")
    d = kda_inputs.make_inputs(w)
    out, fin = run_dev(d, w)
    compare_all_heads(out, fin, d, w.final, w.name)


# mid-size shapes between the small cases and the full workloads: head counts that are
# not multiples of 8, chains on two and four value tiles per workgroup, ragged rows and
# sequences, the segmented chain at 16 heads, every state dtype
MEDIUM = [
    dict(B=3, T=777, H=5, state='fp32', lower_bound=-3.0, seed=11),
    dict(B=1, T=4099, H=12, state='bf16', final='bf16', seed=12),
    dict(B=2, T=2048, H=24, lower_bound=-0.5, seed=13),
    dict(lengths=[1000, 17, 2500, 64, 0, 333], H=20, state='fp32', seed=14),   # 4 value tiles per workgroup
    dict(B=1, T=8192, H=16, seed=15),                                          # segmented chain (4 segments)
    dict(B=1, T=1100, H=96, seed=16),                                          # more heads than the workloads
    dict(lengths=[700, 300, 1], H=128, state='bf16', final='bf16', seed=17),
]


@pytest.mark.parametrize("case", range(len(MEDIUM)))
def test_medium_shapes_all_heads(case):
    w = kda_inputs.custom(**MEDIUM[case])
    say(f"medium case {case} {MEDIUM[case]}: all heads")
    d = kda_inputs.make_inputs(w)
    out, fin = run_dev(d, w)
    compare_all_heads(out, fin, d, w.final, f"medium {case} {w.name}")


@pytest.mark.parametrize("path", ["recurrent", "chunked"])
def test_decode_step_all_heads(path):
    """One generation step (one token per sequence, fp32 state in and out), every head."""
    w = kda_inputs.workload(5)
    say(f"workload 5 {w.name} path={path}: all heads")
    d = kda_inputs.make_inputs(w)
    out, fin = run_dev(d, w, path)
    compare_all_heads(out, fin, d, w.final, f"{w.name}/{path}")


def test_batched_long_one_call_vs_chained():
    """B=4, T=32768: one call, and four chained 8192-token calls (final -> initial), each
    against the other and both against the oracle on every head."""
    w = kda_inputs.workload(4)
    say("workload 4: drawing inputs")
    d = kda_inputs.make_inputs(w)
    device = dev()
    x = to_dev(d, device)
    B, T, H = 4, 32768, 64
    say("workload 4: one call")
    out1 = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device=device)
    fin1 = torch.empty(B, H, 128, 128, dtype=torch.float32, device=device)
    kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out1, x['A_log'], x['dt_bias'],
            x['lower_bound'], initial_state=x['initial_state'], final_state=fin1)
    say("workload 4: four chained 8192-token calls")
    out2 = torch.empty_like(out1)
    st = x['initial_state'].clone()
    for c in range(4):
        sl = lambda t: t[:, c * 8192:(c + 1) * 8192].contiguous()
        oc = torch.empty(B, 8192, H, 128, dtype=torch.bfloat16, device=device)
        nxt = torch.empty_like(st)
        kda.fwd(sl(x['q']), sl(x['k']), sl(x['v']), sl(x['g']), sl(x['beta']), x['scale'], oc, x['A_log'],
                x['dt_bias'], x['lower_bound'], initial_state=st, final_state=nxt)
        out2[:, c * 8192:(c + 1) * 8192] = oc
        st = nxt
    torch.cuda.synchronize()
    del x
    for t, tg in ((out1, "one call"), (out2, "chained")):
        assert bool(torch.isfinite(t).all()), f"batched {tg}: non-finite output"
    assert bool(torch.isfinite(fin1).all()) and bool(torch.isfinite(st).all())
    # one call against the chained calls, over the whole tensors (on the device)
    num = den = 0.0
    mx = 0.0
    for b in range(B):
        a, c = out1[b].float(), out2[b].float()
        num += float(((a - c) ** 2).sum())
        den += float((a ** 2).sum())
        mx = max(mx, float((a - c).abs().max()))
    r_o = math.sqrt(num / den)
    r_f = float(torch.linalg.vector_norm(st - fin1) / torch.linalg.vector_norm(fin1))
    say(f"one vs chained: out rel-L2 {r_o:.3e} max-abs {mx:.3e} final rel-L2 {r_f:.3e}")
    parity_margins.record("batched one vs chained", True, mx, r_o, r_f, FIN_REL['fp32'])
    assert r_o <= OUT_REL and mx <= OUT_MAXABS and r_f <= FIN_REL['fp32']
    say("workload 4: oracle on every head, in batches of 8")
    o1 = out1.float().cpu().numpy().reshape(B * T, H, 128)
    o2 = out2.float().cpu().numpy().reshape(B * T, H, 128)
    f1, f2 = fin1.cpu().numpy(), st.cpu().numpy()
    del out1, out2
    e1, e2 = HeadErrors(H), HeadErrors(H)
    for h0 in range(0, H, 8):
        hs = list(range(h0, h0 + 8))
        ro, rf = oracle_for(d, heads=hs)
        e1.add(h0, o1[:, h0:h0 + 8], ro, f1[:, h0:h0 + 8], rf)
        e2.add(h0, o2[:, h0:h0 + 8], ro, f2[:, h0:h0 + 8], rf)
        del ro, rf
    e1.check("batched_B4_T32768 one call", 'fp32')
    e2.check("batched_B4_T32768 chained", 'fp32')


# ---------------------------------------------------------------------------
# fusion switches off: pre-activated gate, pre-normalised q/k, beta given directly
def _unfused_inputs(d, gate, norm, beta):
    """Inputs as the caller would pass them with a switch off (still bf16)."""
    d = dict(d)
    if not gate:   # log-decays, partly outside [lower_bound, 0] so the clamp is exercised
        d['g'] = (d['g'].float() * 1.5 - 1.0).to(torch.bfloat16)
        d['A_log'] = d['dt_bias'] = None
    if not norm:   # unit rows (the delta rule needs |k| ~ 1 to stay a contraction)
        for n in ('q', 'k'):
            x = d[n].float()
            d[n] = (x / x.norm(dim=-1, keepdim=True).clamp_min(1e-3)).to(torch.bfloat16)
    if not beta:
        d['beta'] = torch.sigmoid(d['beta'].float()).to(torch.bfloat16)
    return d


SWITCHES = [(False, True, True), (True, False, True), (True, True, False), (False, False, False)]


@pytest.mark.parametrize("path", ["chunked", "recurrent"])
@pytest.mark.parametrize("sw", SWITCHES, ids=["gate_off", "norm_off", "beta_off", "all_off"])
@pytest.mark.parametrize("shape", [dict(B=1, T=200, H=3, state='fp32', lower_bound=-3.0),
                                   dict(lengths=[70, 0, 130, 5], H=2, state='bf16', final='bf16')],
                         ids=["fixed", "varlen"])
def test_fusion_switches_off(shape, sw, path):
    gate, norm, beta = sw
    w = kda_inputs.custom(**shape)
    say(f"switches gate={gate} norm={norm} beta={beta} {shape} path={path}")
    d = _unfused_inputs(kda_inputs.make_inputs(w), gate, norm, beta)
    kw = dict(use_gate_in_kernel=gate, use_qk_l2norm_in_kernel=norm, use_beta_sigmoid_in_kernel=beta)
    ro, rf = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                        d['lower_bound'], initial_state=d['initial_state'], cu_seqlens=d['cu_seqlens'], **kw)
    device = dev()
    x = to_dev(d, device)
    B, T, H = x['q'].shape[:3]
    out = torch.full((B, T, H, 128), float('nan'), dtype=torch.bfloat16, device=device)
    fin = torch.full((w.n_seqs, H, 128, 128), float('nan'),
                     dtype=torch.float32 if w.final == 'fp32' else torch.bfloat16, device=device)
    fn = functools.partial(kda.fwd, force_chunked=True) if path == "chunked" else kda.fwd_recurrent
    fn(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'], x['lower_bound'],
       initial_state=x['initial_state'], final_state=fin, cu_seqlens=x['cu_seqlens'], **kw)
    torch.cuda.synchronize()
    o = out.float().double().cpu().numpy().reshape(B * T, H, 128)
    f = fin.float().double().cpu().numpy()
    check(o, f, ro, rf, w.final, f"switches {sw}/{path}")


# ---------------------------------------------------------------------------
# gate without the safe bound (safe_gate off): -exp(A_log) softplus(g + dt_bias), or
# min(g, 0) unfused. The regimes steer the 16-token gate sums: "mild" keeps every
# sub-chunk on the factorised MFMA path, "strong" and "unfused" push most sub-chunks
# past it (split-form or entry-by-entry diagonal blocks), "mixed" puts huge and tiny per-channel
# gates in the same sub-chunks and mixes both kinds of heads, "tiers" gives the heads
# gate rates 3, 9 and 40 (the last H of them), whose 16-token sums put every sub-chunk
# of a head on one diagonal-block form: factorised from the sub-chunk start, the split
# form (each 8-token half about its own midpoints), entry by entry.
def _unbounded_inputs(d, regime):
    d = dict(d)
    H, K = d['dt_bias'].shape
    if regime == "mild":
        d['A_log'] = torch.full((H,), -3.5)
    elif regime == "tiers":
        d['A_log'] = torch.log(torch.tensor([3.0, 9.0, 40.0][-H:]))
    elif regime == "mixed":
        al = torch.full((H,), math.log(16.0))
        al[0::2] = -3.0
        d['A_log'] = al
        dt = d['dt_bias'].clone()
        dt[:, 0::2] += 6.0     # softplus ~ 6: about -96 per token at rate 16
        dt[:, 1::2] -= 6.0     # softplus ~ 0.0025
        d['dt_bias'] = dt
    elif regime == "unfused":
        d['g'] = (-d['g'].float().abs() * 12.0).to(torch.bfloat16)
        d['A_log'] = d['dt_bias'] = None
    return d


@pytest.mark.parametrize("path", ["chunked", "recurrent"])
@pytest.mark.parametrize("regime", ["mild", "strong", "mixed", "unfused", "tiers"])
@pytest.mark.parametrize("shape", [dict(B=1, T=200, H=3, state='fp32', lower_bound=-3.0),
                                   dict(lengths=[70, 0, 130, 5, 64], H=2, state='bf16', final='bf16')],
                         ids=["fixed", "varlen"])
def test_unbounded_gate(shape, regime, path):
    w = kda_inputs.custom(**shape)
    say(f"unbounded gate regime={regime} {shape} path={path}")
    d = _unbounded_inputs(kda_inputs.make_inputs(w), regime)
    kw = dict(use_gate_in_kernel=regime != "unfused", safe_gate=False)
    ro, rf = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                        d['lower_bound'], initial_state=d['initial_state'], cu_seqlens=d['cu_seqlens'], **kw)
    device = dev()
    x = to_dev(d, device)
    B, T, H = x['q'].shape[:3]
    out = torch.full((B, T, H, 128), float('nan'), dtype=torch.bfloat16, device=device)
    fin = torch.full((w.n_seqs, H, 128, 128), float('nan'),
                     dtype=torch.float32 if w.final == 'fp32' else torch.bfloat16, device=device)
    fn = functools.partial(kda.fwd, force_chunked=True) if path == "chunked" else kda.fwd_recurrent
    # lower_bound is ignored by this gate: pass a value the safe gate would reject
    fn(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'], -9.0,
       initial_state=x['initial_state'], final_state=fin, cu_seqlens=x['cu_seqlens'], **kw)
    torch.cuda.synchronize()
    o = out.float().double().cpu().numpy().reshape(B * T, H, 128)
    f = fin.float().double().cpu().numpy()
    check(o, f, ro, rf, w.final, f"unbounded {regime}/{path}")


@pytest.mark.parametrize("regime", ["strong", "mixed"])
def test_unbounded_gate_full_size_all_heads(regime):
    """T=8192, H=64 (the prefill workload's shape and launch) with the unbounded gate,
    every head."""
    w = kda_inputs.workload(1)
    say(f"workload 1 with the unbounded gate ({regime}): all heads")
    d = _unbounded_inputs(kda_inputs.make_inputs(w), regime)
    out, fin = run_dev(d, w, safe_gate=False)
    compare_all_heads(out, fin, d, 'fp32', f"prefill unbounded {regime}", safe_gate=False)


# ---------------------------------------------------------------------------
# more than 2^31 elements per input tensor: every token, record and output offset
# must be computed in 64 bits. T * H * 128 = (2^18 + 64) * 64 * 128 > 2^31. Every head
# is checked for finiteness; eight heads (one per h mod 8, the last one among them, so
# the highest offsets are compared) against the oracle, which would need 17 GB of host
# inputs for all 64.
@pytest.mark.parametrize("path", ["chunked", "recurrent"])
def test_offsets_beyond_2g_elements(path):
    device = dev()
    w = kda_inputs.Workload("offsets_T262208_H64", B=1, T=2 ** 18 + 64, H=64, state='fp32')
    assert w.T * w.H * 128 > 2 ** 31
    say(f"{w.name}: {w.T} tokens x {w.H} heads, path={path} (inputs drawn on the device)")
    x = kda_inputs.make_inputs_device(w, device)
    out = torch.empty(1, w.T, w.H, 128, dtype=torch.bfloat16, device=device)
    fin = torch.empty(1, w.H, 128, 128, dtype=torch.float32, device=device)
    fn = functools.partial(kda.fwd, force_chunked=True) if path == "chunked" else kda.fwd_recurrent
    fn(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'], x['lower_bound'],
       initial_state=x['initial_state'], final_state=fin)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(fin).all()), "non-finite results"
    # one head for every value of h mod 8 (the chain kernel places a head's workgroups on
    # XCD h mod 8), the last head among them, so the highest offsets are compared
    heads = [0, 9, 18, 27, 36, 45, 54, 63]
    cpu = {n: x[n][:, :, heads].contiguous().cpu() for n in ('q', 'k', 'v', 'g', 'beta')}
    ro, rf = kda_oracle(cpu['q'], cpu['k'], cpu['v'], cpu['g'], cpu['beta'], x['scale'],
                        x['A_log'][heads].cpu(), x['dt_bias'][heads].cpu(), x['lower_bound'],
                        initial_state=x['initial_state'][:, heads].contiguous().cpu())
    o = out[:, :, heads].float().double().cpu().numpy().reshape(w.T, len(heads), 128)
    f = fin[:, heads].double().cpu().numpy()
    del x, out
    check(o, f, ro, rf, 'fp32', f"{w.name}/{path}")


# ---------------------------------------------------------------------------
# power-of-two scaling of v and the initial state: the forward is linear in (v, S0),
# and every internal rescaling in the kernels (the U~ column scales, the state-row and
# U-column scales of the chain) is a power of two, so out and final_state must scale
# by exactly the same power of two, bit for bit
@pytest.mark.parametrize("path", ["chunked", "recurrent"])
@pytest.mark.parametrize("state", ["fp32", "bf16"])
def test_power_of_two_scaling_is_exact(state, path):
    device = dev()
    w = kda_inputs.custom(lengths=[150, 64, 1, 77], H=2, state=state, final=state)
    d = kda_inputs.make_inputs(w)
    ref_o, ref_f = run(d, w, path)
    for k in (-10, 16):
        say(f"scale v and initial state by 2^{k}, state={state}, path={path}")
        ds = dict(d)
        ds['v'] = (d['v'].float() * 2.0 ** k).to(torch.bfloat16)
        ds['initial_state'] = (d['initial_state'].float() * 2.0 ** k).to(d['initial_state'].dtype)
        assert torch.equal(ds['v'].float(), d['v'].float() * 2.0 ** k)   # the scaling itself is exact
        o, f = run(ds, w, path)
        assert np.array_equal(o, ref_o * 2.0 ** k), f"out does not scale exactly by 2^{k}"
        assert np.array_equal(f, ref_f * 2.0 ** k), f"final state does not scale exactly by 2^{k}"


@pytest.mark.parametrize("path", ["chunked", "recurrent"])
def test_scale_zero_and_sign(path):
    """scale only multiplies the read-out: scale = 0 gives out == 0 exactly, -scale gives
    -out bit for bit, and the final state does not depend on it."""
    w = kda_inputs.custom(lengths=[100, 3, 64], H=2, state='fp32')
    d = kda_inputs.make_inputs(w)
    say(f"scale 0 / sign, path={path}")
    o, f = run(d, w, path)
    o0, f0 = run(dict(d, scale=0.0), w, path)
    on, fn = run(dict(d, scale=-d['scale']), w, path)
    assert np.all(o0 == 0.0), "scale = 0 must give a zero output"
    assert np.array_equal(on, -o), "negating scale must negate out exactly"
    assert np.array_equal(f0, f) and np.array_equal(fn, f), "final state must not depend on scale"


# ---------------------------------------------------------------------------
# segment-parallel state chain: with few (row, head) chains on long fixed-length rows
# the chain is cut into segments (affine maps, a scan, then the outputs). Checked
# against the oracle and against the plain chain (KDA_CHAIN_SEGMENTS=1) on the same
# inputs; KDA_LOG shows which segment count ran.
# Gates with long memory (lower_bound near 0): a segment's initial state then still
# matters at its end, so the P maps and the scan are exercised (with lower_bound = -5 a
# 512-token segment forgets its initial state entirely and P underflows to 0).
SEG_SHAPES = [
    (dict(B=1, T=4096, H=2, state='fp32', lower_bound=-0.01), 8),                     # 8 segments of 8 chunks
    (dict(B=2, T=4000, H=2, state='bf16', final='bf16', lower_bound=-0.05), 4),       # ragged last chunk
    (dict(B=1, T=4096, H=1, final=None, lower_bound=-0.3), 8),                        # stateless, no final state
    (dict(B=1, T=4096, H=2, state='fp32', lower_bound=-5.0), 8),                      # short memory
    (dict(lengths=[4096], H=2, state='fp32', lower_bound=-0.01), 8),                  # varlen, one sequence
    # varlen, uneven: 94, 40, 2 and 0 chunks in 4 segments each (empty segments included)
    (dict(lengths=[6000, 2500, 70, 0], H=1, state='bf16', final='bf16', lower_bound=-0.05), 4),
]


@pytest.mark.parametrize("shape,nseg", SEG_SHAPES,
                         ids=["T4096_H2_fp32_lb0.01", "B2_T4000_H2_bf16_lb0.05", "T4096_H1_nofinal_lb0.3",
                              "T4096_H2_fp32_lb5", "varlen_4096_H2", "varlen_uneven_H1_bf16"])
def test_segmented_chain(shape, nseg, capfd, monkeypatch):
    w = kda_inputs.custom(**shape)
    say(f"segmented chain {shape}")
    d = kda_inputs.make_inputs(w)
    ro, rf = oracle_for(d)
    monkeypatch.setenv("KDA_LOG", "1")
    o, f = run(d, w)
    assert f"segments={nseg}" in capfd.readouterr().err, "the segmented chain did not run"
    check(o, f, ro, rf if w.final else None, w.final, f"segmented x{nseg}")
    monkeypatch.setenv("KDA_CHAIN_SEGMENTS", "1")
    o1, f1 = run(d, w)
    assert "segments=1" in capfd.readouterr().err
    check(o1, f1, ro, rf if w.final else None, w.final, "plain chain")
    say(f"segmented vs plain: out max-abs {np.abs(o - o1).max():.3e}")


def test_segmented_chain_unbounded_mild_gate(capfd, monkeypatch):
    """The gate without the safe bound at a small rate (long memory), segmented chain."""
    w = kda_inputs.custom(B=1, T=4096, H=2, state='fp32')
    d = _unbounded_inputs(kda_inputs.make_inputs(w), "mild")
    say("segmented chain, unbounded mild gate")
    ro, rf = kda_oracle(d['q'], d['k'], d['v'], d['g'], d['beta'], d['scale'], d['A_log'], d['dt_bias'],
                        d['lower_bound'], initial_state=d['initial_state'], safe_gate=False)
    monkeypatch.setenv("KDA_LOG", "1")
    device = dev()
    x = to_dev(d, device)
    out = torch.empty(1, w.T, 2, 128, dtype=torch.bfloat16, device=device)
    fin = torch.empty(1, 2, 128, 128, dtype=torch.float32, device=device)
    kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'], x['lower_bound'],
            initial_state=x['initial_state'], final_state=fin, safe_gate=False)
    torch.cuda.synchronize()
    assert "segments=8" in capfd.readouterr().err
    check(out.float().double().cpu().numpy().reshape(w.T, 2, 128), fin.double().cpu().numpy(), ro, rf, 'fp32',
          "segmented, unbounded mild gate")


def test_segmented_chain_tp8_share_all_heads():
    """One GPU's share under 8-way head parallelism (T=8192, H=8), segmented chain, every head."""
    w = kda_inputs.workload(6)
    say(f"workload 6 {w.name}: all heads")
    d = kda_inputs.make_inputs(w)
    out, fin = run_dev(d, w)
    compare_all_heads(out, fin, d, w.final, w.name, batch=8)


def test_segmented_chain_long_single_sequence(capfd, monkeypatch):
    """131072 tokens on one head: 32 segments of 64 chunks and a 32-step scan, with a
    long-memory gate so every segment's map carries the state."""
    w = kda_inputs.custom(B=1, T=131072, H=1, state='fp32', lower_bound=-0.01)
    say(f"long single sequence {w.T} tokens, segmented chain")
    d = kda_inputs.make_inputs(w)
    monkeypatch.setenv("KDA_LOG", "1")
    o, f = run(d, w)
    assert "segments=32" in capfd.readouterr().err
    ro, rf = oracle_for(d)
    check(o, f, ro, rf, 'fp32', "131072 tokens, 32 segments")
