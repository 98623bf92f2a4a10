"""C-ABI checks that need no GPU: libkda.so loads, exports every function that
include/kda.h declares, sizes its workspace as documented, and rejects bad
arguments on the host before anything is launched (status codes per the
header, following the FlashKDA "Kernel API" table constraints).

Only argument combinations that fail validation are passed here, so no HIP
call is ever made; the fake device pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import gated_delta_rule_87_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, ENULL, ESHAPE, EDTYPE, EVALUE, EALIGN, EWS, EHIP, ECAP = range(9)
FAKE = 0x10000000          # 256-byte aligned fake device address (never dereferenced)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(kda_\w+)\s*\(", src, flags=re.M)))


def test_header_symbols_exported():
    names = declared_functions()
    assert {"kda_fwd", "kda_fwd_recurrent", "kda_fwd_workspace_size", "kda_status_string",
            "kda_version", "kda_profile_start", "kda_profile_stop", "kda_profile_kernel_count",
            "kda_profile_kernel_name", "kda_fwd_ex", "kda_fwd_recurrent_ex", "kda_fwd_noalloc",
            "kda_noalloc_capacity", "kda_fwd_workspace_min"} <= set(names)
    L = ctypes.CDLL(kda.LIB_PATH)
    for n in names:
        assert hasattr(L, n), f"libkda.so does not export {n}"


def test_version_and_status_strings():
    L = kda.lib()
    assert b"gfx950" in L.kda_version()
    for code in range(9):
        s = kda.status_string(code)
        assert s.startswith("KDA_"), s
    assert "unknown" in kda.status_string(99)


def test_workspace_size():
    rec = 76288                         # bytes per (64-token chunk, head)
    al = lambda x: (x + 255) // 256 * 256
    assert kda.workspace_size(1, 8192, 64) == al(128 * 64 * rec)
    # beyond 4 GiB on the plain chain: windows of chunk columns within 4 GiB (fp32 carry of
    # 64 KiB per (row, head), then the fewest windows that fit, with balanced widths)
    carry, col = al(4 * 64 * 128 * 128 * 4), 4 * 64 * rec
    fit = ((4 << 30) - carry) // col
    count = -(-512 // fit)
    assert kda.workspace_size(4, 32768, 64) == carry + -(-512 // count) * col <= 4 << 30
    assert kda.workspace_size(1, 100, 2) == al(2 * 2 * rec)             # ceil(100/64) = 2
    # varlen: floor(T/64) + N chunk slots, plus the tables
    ws = kda.workspace_size(1, 8192, 64, 8)
    assert ws == al((128 + 8) * 64 * rec) + al(8 * 8) + al((128 + 8) * 8) + al(8 * 8) + al(8 * 4)
    assert kda.workspace_size(1, 0, 4) == 0
    assert kda.workspace_size(0, 10, 4) == 0 and kda.workspace_size(1, -1, 4) == 0
    assert kda.workspace_size(1, 10, 0) == 0


def call(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=0.088, out=FAKE, A_log=FAKE, dt_bias=FAKE,
             lb=-5.0, init=None, idt=0, fin=None, fdt=0, cu=None, N=0, B=1, T=64, H=2, K=128, V=128,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    L = kda.lib()
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.kda_fwd(P(a['q']), P(a['k']), P(a['v']), P(a['g']), P(a['beta']), a['scale'], P(a['out']),
                     P(a['A_log']), P(a['dt_bias']), a['lb'], P(a['init']), a['idt'], P(a['fin']), a['fdt'],
                     P(a['cu']), a['N'], a['B'], a['T'], a['H'], a['K'], a['V'], P(a['ws']), a['wsb'],
                     P(a['stream']))


def call_rec(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=0.088, out=FAKE, A_log=FAKE, dt_bias=FAKE,
             lb=-5.0, init=None, idt=0, fin=None, fdt=0, cu=None, N=0, B=1, T=64, H=2, K=128, V=128)
    a.update(kw)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return kda.lib().kda_fwd_recurrent(P(a['q']), P(a['k']), P(a['v']), P(a['g']), P(a['beta']), a['scale'],
                                       P(a['out']), P(a['A_log']), P(a['dt_bias']), a['lb'], P(a['init']),
                                       a['idt'], P(a['fin']), a['fdt'], P(a['cu']), a['N'], a['B'], a['T'],
                                       a['H'], a['K'], a['V'], None)


@pytest.mark.parametrize("fn", [call, call_rec])
def test_validation_errors(fn):
    # K = V = 128 only
    assert fn(K=64) == ESHAPE and fn(V=256) == ESHAPE
    assert fn(B=0) == ESHAPE and fn(T=-1) == ESHAPE and fn(H=0) == ESHAPE
    # cu_seqlens requires B == 1 and N >= 1
    assert fn(cu=FAKE, N=2, B=2) == ESHAPE
    assert fn(cu=FAKE, N=0) == ESHAPE
    # required pointers
    for name in ("q", "k", "v", "g", "beta", "out", "A_log", "dt_bias"):
        assert fn(**{name: None}) == ENULL, name
    # T = 0: the token buffers hold no element and may be NULL (an empty tensor's data
    # pointer); the checks after the pointer checks still apply (here: lower_bound)
    empty = dict(q=None, k=None, v=None, g=None, beta=None, out=None)
    assert fn(T=0, lb=-5.5, **empty) == EVALUE
    assert fn(T=0, cu=FAKE, N=3, lb=-5.5, **empty) == EVALUE
    assert fn(T=0, A_log=None, **empty) == ENULL                  # per-head parameters still required
    # state dtypes
    assert fn(init=FAKE, idt=7) == EDTYPE
    assert fn(init=FAKE, idt=1, fin=FAKE, fdt=2) == EDTYPE        # must match
    assert fn(init=FAKE, idt=0) == EDTYPE                          # pointer without dtype
    assert fn(init=None, idt=2) == ENULL                           # dtype without pointer
    assert fn(fin=None, fdt=1) == ENULL
    # lower_bound in [-5, 0], finite scale
    assert fn(lb=-5.5) == EVALUE and fn(lb=0.5) == EVALUE and fn(lb=float('nan')) == EVALUE
    assert fn(scale=float('inf')) == EVALUE
    # alignment
    assert fn(q=FAKE + 8) == EALIGN
    assert fn(out=FAKE + 2) == EALIGN
    assert fn(init=FAKE + 4, idt=2) == EALIGN
    assert fn(cu=FAKE + 4, N=1) == EALIGN


def test_workspace_errors():
    need = kda.workspace_size(1, 64, 2)
    assert call(ws=None, wsb=0) == EWS
    assert call(ws=FAKE, wsb=need - 1) == EWS      # one chunk per row: no smaller windowed form
    assert call(ws=FAKE + 16, wsb=need) == EALIGN
    # fixed length: below the windowed minimum is rejected before anything is launched
    mn = kda.workspace_min(2, 1000, 4)
    assert call(B=2, T=1000, H=4, ws=FAKE, wsb=mn - 1) == EWS
    # varlen: below the windowed minimum (tables, two carry slots, one slot of records)
    vmn = kda.workspace_min(1, 1000, 4, 3)
    assert vmn < kda.workspace_size(1, 1000, 4, 3)
    assert call(T=1000, H=4, cu=FAKE, N=3, ws=FAKE, wsb=vmn - 1) == EWS


def test_workspace_min():
    """One chunk column (B * H records) and an fp32 carry of 64 KiB per (row, head), or the
    full size when that is smaller; varlen calls: the full size."""
    rec = kda.record_bytes()
    al = lambda x: (x + 255) // 256 * 256
    for B, T, H in [(1, 8192, 64), (4, 32768, 64), (2, 1000, 4), (3, 200, 1)]:
        full = kda.workspace_size(B, T, H)
        assert kda.workspace_min(B, T, H) == min(full, al(B * H * 128 * 128 * 4) + B * H * rec)
    assert kda.workspace_min(1, 64, 2) == kda.workspace_size(1, 64, 2)    # one chunk per row
    # varlen: the tables (seq_tab, seq_span: 8 B per sequence; chunk_tab 8 B per chunk slot;
    # seq_order, nz_seq 4 B per sequence; win_first 4 B per slot + 1), two fp32 carry slots
    # of H states and one slot of H records
    for T, H, N in [(8192, 64, 8), (1000, 4, 3), (131072, 64, 32)]:
        mc = T // 64 + N
        fixed = 2 * al(N * 8) + al(mc * 8) + 2 * al(N * 4) + al((mc + 1) * 4) + al(2 * H * 128 * 128 * 4)
        assert kda.workspace_min(1, T, H, N) == min(kda.workspace_size(1, T, H, N), fixed + H * rec)
    # beyond 4 GiB on the plain chain, varlen calls also get a windowed size within 4 GiB
    assert kda.workspace_size(1, 131072, 64, 32) <= 4 << 30
    assert kda.workspace_size(1, 26810, 64, 32) > 1 << 30     # 2.2 GB: one launch pair
    assert kda.workspace_min(1, 0, 4) == 0 and kda.workspace_min(0, 10, 4) == 0


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kda.fwd(q, q, q, q, torch.zeros(1, 4, 1, dtype=torch.bfloat16), 1.0, q.clone(),
                torch.zeros(1), torch.zeros(1, 128), -1.0)


def test_api_table_fixture_matches_binding():
    """tests/golden/api_table.txt restates the pages' parameter table; the binding enforces it."""
    rows = [ln.split("|") for ln in open(os.path.join(ROOT, "tests", "golden", "api_table.txt"))
            if ln.strip() and not ln.startswith("#")]
    table = {r[0].strip(): (r[1].strip(), r[2].strip()) for r in rows}
    assert table["q"] == ("bf16", "[B, T, H, K]") and table["v"] == ("bf16", "[B, T, H, V]")
    assert table["beta"] == ("bf16", "[B, T, H]") and table["out"] == ("bf16", "[B, T, H, V]")
    assert table["A_log"] == ("fp32", "[H]") and table["dt_bias"] == ("fp32", "[H, K]")
    assert table["cu_seqlens"] == ("int64", "[N+1]")
    assert table["initial_state"][0] == "bf16/fp32/None"


def test_profile_hook_host_paths():
    """Timing-hook argument checks that make no HIP call (no start with a valid count)."""
    L = kda.lib()
    n = L.kda_profile_kernel_count()
    assert n == 3
    assert [L.kda_profile_kernel_name(i) for i in range(n)] == [b"kda_sched_kernel", b"kda_intra_kernel",
                                                                   b"kda_chain_kernel"]
    assert L.kda_profile_kernel_name(-1) == b"" and L.kda_profile_kernel_name(n) == b""
    assert L.kda_profile_start(0) == EVALUE
    assert L.kda_profile_start(65537) == EVALUE
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    assert L.kda_profile_stop(None, cnt, n) == ENULL
    assert L.kda_profile_stop(ms, cnt, n - 1) == ESHAPE
    assert L.kda_profile_stop(ms, cnt, n) == EVALUE      # timing was never started


def call_ex(flags, recurrent=False, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=0.088, out=FAKE, A_log=FAKE, dt_bias=FAKE,
             lb=-5.0, init=None, idt=0, fin=None, fdt=0, cu=None, N=0, B=1, T=64, H=2, K=128, V=128,
             ws=None, wsb=0)
    a.update(kw)
    L = kda.lib()
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    head = (P(a['q']), P(a['k']), P(a['v']), P(a['g']), P(a['beta']), a['scale'], P(a['out']), P(a['A_log']),
            P(a['dt_bias']), a['lb'], P(a['init']), a['idt'], P(a['fin']), a['fdt'], P(a['cu']), a['N'], a['B'],
            a['T'], a['H'], a['K'], a['V'], flags)
    if recurrent:
        return L.kda_fwd_recurrent_ex(*head, None)
    return L.kda_fwd_ex(*head, P(a['ws']), a['wsb'], None)


@pytest.mark.parametrize("recurrent", [False, True])
def test_fusion_flag_validation(recurrent):
    """Unknown flag bits are rejected; A_log/dt_bias are required only with the fused gate
    (a later shape error shows the NULL pointers passed the pointer checks)."""
    for bad in (0x20, 0x40, 0xffffffff):
        assert call_ex(bad, recurrent) == EVALUE
    # KDA_PATH_CHUNKED (0x10) is a kda_fwd_ex switch only; there it passes the flag check
    # (the later shape error shows it)
    if recurrent:
        assert call_ex(0x10 | 7, recurrent) == EVALUE
    else:
        assert call_ex(0x10 | 7, recurrent, K=64) == ESHAPE
    assert call_ex(7, recurrent, A_log=None) == ENULL
    assert call_ex(7, recurrent, dt_bias=None) == ENULL
    assert call_ex(1, recurrent, dt_bias=None) == ENULL
    for flags in (0, 2, 4, 6):
        assert call_ex(flags, recurrent, A_log=None, dt_bias=None, K=64) == ESHAPE
        assert call_ex(flags, recurrent, A_log=None, dt_bias=None, g=None) == ENULL


@pytest.mark.parametrize("recurrent", [False, True])
def test_unbounded_gate_skips_lower_bound_check(recurrent):
    """lower_bound is checked only for the safe gate: with KDA_GATE_UNBOUNDED an
    out-of-range or NaN value passes (the later shape error shows the value check passed)."""
    for lb in (-7.0, 1.0, float("nan")):
        assert call_ex(7, recurrent, lb=lb) == EVALUE
        assert call_ex(7 | 8, recurrent, lb=lb, K=64) == ESHAPE
        assert call_ex(8, recurrent, lb=lb, A_log=None, dt_bias=None, K=64) == ESHAPE


def test_workspace_size_with_segmented_chain():
    """Few (row, head) chains on long rows: the workspace adds the segment maps (256 x 128
    fp32 per segment and head) and the segment initial states (128 x 128 fp32)."""
    rec = 76288
    al = lambda x: (x + 255) // 256 * 256
    nseg = 8   # 8 heads x 8192 tokens: the chain is cut into 8 segments of 16 chunks
    m = 256 * 128 * 4
    i = 128 * 128 * 4
    assert kda.workspace_size(1, 8192, 8) == al(128 * 8 * rec) + al(nseg * 8 * m) + al(nseg * 8 * i)
    # enough chains for the whole GPU: no segment buffers
    assert kda.workspace_size(1, 8192, 64) == al(128 * 64 * rec)
    assert kda.workspace_size(1, 8192, 64, 8) == (al((128 + 8) * 64 * rec) + al(8 * 8) + al((128 + 8) * 8)
                                               + al(8 * 8) + al(8 * 4))
    # varlen: one sequence of 8192 tokens on 8 heads (average 128 chunks): 8 segments
    assert kda.workspace_size(1, 8192, 8, 1) == (al((128 + 1) * 8 * rec) + al(8) + al(129 * 8) + al(8) + al(4)
                                              + al(nseg * 8 * m) + al(nseg * 8 * i))
    # two sequences on 8 heads averaging 64 chunks: too short to gain 15%, no segments;
    # averaging 256 chunks: 4 segments per sequence
    assert kda.workspace_size(1, 8192, 8, 2) == (al((128 + 2) * 8 * rec) + al(16) + al(130 * 8) + al(16) + al(8))
    assert kda.workspace_size(1, 32768, 8, 2) == (al((512 + 2) * 8 * rec) + al(16) + al(514 * 8) + al(16) + al(8)
                                               + al(2 * 4 * 8 * m) + al(2 * 4 * 8 * i))


def test_noalloc_capacity_check_on_host():
    """kda_fwd_noalloc rejects, before any HIP call (KDA_ERR_CAPACITY), a call whose
    smallest workspace (kda_fwd_workspace_min) exceeds its fixed array: calls whose
    single window (one chunk column or slot of records, and the carry) does not fit.
    The capacity is the header's 256 MiB."""
    L = kda.lib()
    cap = L.kda_noalloc_capacity()
    assert cap == 256 << 20
    assert kda.workspace_min(1, 64, 2048, 1) > cap >= kda.workspace_min(1, 8192, 64, 4)
    assert kda.workspace_min(16, 8192, 128) > cap >= kda.workspace_min(1, 8192, 64)
    P = ctypes.c_void_p
    args = [P(FAKE)] * 5 + [0.088, P(FAKE), P(FAKE), P(FAKE), -5.0, None, 0, None, 0]
    assert L.kda_fwd_noalloc(*args, P(FAKE), 1, 1, 64, 2048, 128, 128, 7, None) == ECAP    # varlen, H too large
    assert L.kda_fwd_noalloc(*args, None, 0, 16, 8192, 128, 128, 128, 7, None) == ECAP    # B * H too large
