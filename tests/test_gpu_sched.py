"""GPU test of the varlen scheduler's tables (kda_sched_kernel), read back from the
workspace after a kda_fwd call and compared, exactly, with the same tables built in
Python from cu_seqlens:

  seq_tab[n]   = {first chunk, chunks} (chunks = ceil(len / 64), prefix-summed)
  seq_span[n]  = {first token, length}
  chunk_tab[i] = {first token, tokens <= 64} of chunk slot i; {0, 0} when unused
  seq_order[k] = sequences by chunk count, most first, ties by index; input order
                 when there are more than 4096 sequences

The workspace layout (256-byte aligned regions: records | seq_tab | chunk_tab |
seq_span | seq_order) is the one kda_fwd_workspace_size describes.
"""
import numpy as np
import pytest
import torch

import kda_inputs
import gated_delta_rule_87_amd as kda

pytestmark = pytest.mark.gpu

REC = 76288
SORT_MAX = 4096


def al(x):
    return (x + 255) // 256 * 256


def expected_tables(lengths, T):
    N = len(lengths)
    max_chunks = T // 64 + N
    nc = [(n + 63) // 64 for n in lengths]
    first = np.concatenate([[0], np.cumsum(nc)[:-1]]).astype(np.int64)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    seq_tab = np.stack([first, nc], 1)
    seq_span = np.stack([starts, lengths], 1)
    chunk_tab = np.zeros((max_chunks, 2), np.int64)
    for n in range(N):
        for j in range(nc[n]):
            chunk_tab[first[n] + j] = (starts[n] + 64 * j, min(64, lengths[n] - 64 * j))
    if N <= SORT_MAX:
        order = sorted(range(N), key=lambda n: (-nc[n], n))
    else:
        order = list(range(N))
    return max_chunks, seq_tab, seq_span, chunk_tab, np.array(order, np.int64)


def run_and_read(lengths, H=1):
    device = torch.device("cuda:0")
    w = kda_inputs.custom(lengths=list(lengths), H=H, final=None)
    d = kda_inputs.make_inputs(w)
    x = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    T, N = w.T, len(lengths)
    ws_bytes = kda.workspace_size(1, T, H, N)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=device)
    out = torch.empty(1, T, H, 128, dtype=torch.bfloat16, device=device)
    kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'],
            x['lower_bound'], cu_seqlens=x['cu_seqlens'], workspace=ws, force_chunked=True)
    torch.cuda.synchronize()
    b = ws.cpu().numpy()
    max_chunks = T // 64 + N
    off = al(max_chunks * H * REC)
    seq_tab = b[off:off + 8 * N].view(np.int32).reshape(N, 2)
    off = al(off + 8 * N)
    chunk_tab = b[off:off + 8 * max_chunks].view(np.int32).reshape(max_chunks, 2)
    off = al(off + 8 * max_chunks)
    seq_span = b[off:off + 8 * N].view(np.int32).reshape(N, 2)
    off = al(off + 8 * N)
    seq_order = b[off:off + 4 * N].view(np.int32)
    assert al(off + 4 * N) == ws_bytes
    return T, seq_tab, seq_span, chunk_tab, seq_order


@pytest.mark.parametrize("lengths", [
    [0, 1, 15, 16, 17, 63, 64, 65, 127, 129],
    [300, 0, 5, 300, 64, 0],
    [1] * 40 + [3] * 10 + [0, 0],
    list(np.random.default_rng(3).integers(0, 700, 37)),
])
def test_schedule_tables(lengths):
    lengths = [int(n) for n in lengths]
    print("[gpu-test] schedule tables for", len(lengths), "sequences", flush=True)
    T, seq_tab, seq_span, chunk_tab, seq_order = run_and_read(lengths)
    max_chunks, e_tab, e_span, e_chunk, e_order = expected_tables(lengths, T)
    assert np.array_equal(seq_tab, e_tab)
    assert np.array_equal(seq_span, e_span)
    assert np.array_equal(chunk_tab, e_chunk)
    assert np.array_equal(seq_order, e_order)


def test_schedule_order_beyond_sort_limit():
    """More sequences than the LDS sort holds: input order, tables still exact."""
    rng = np.random.default_rng(11)
    lengths = [int(n) for n in rng.integers(0, 3, SORT_MAX + 5)]
    print("[gpu-test] schedule tables for", len(lengths), "sequences", flush=True)
    T, seq_tab, seq_span, chunk_tab, seq_order = run_and_read(lengths)
    max_chunks, e_tab, e_span, e_chunk, e_order = expected_tables(lengths, T)
    assert np.array_equal(seq_tab, e_tab) and np.array_equal(seq_span, e_span)
    assert np.array_equal(chunk_tab, e_chunk)
    assert np.array_equal(seq_order, np.arange(len(lengths)))


@pytest.mark.parametrize("lengths,width", [
    ([0, 1, 15, 16, 17, 63, 64, 65, 127, 129], 1),
    ([300, 0, 5, 300, 64, 0], 2),
    ([0, 0, 2000, 0, 7], 4),
    (list(np.random.default_rng(4).integers(0, 500, 41)), 3),
])
def test_window_tables(lengths, width):
    """A varlen call in windows of `width` chunk slots: the scheduler's window tables, read
    back from the windowed workspace (records | seq_tab | chunk_tab | seq_span | seq_order |
    nz_seq | win_first | carry), against the same lists built in Python:
      nz_seq[k]    = the k-th sequence with at least one chunk, in index order
      win_first[w] = the first k whose sequence ends after slot w * width (w = 0 .. windows),
                     and the number of such sequences for w = windows."""
    device = torch.device("cuda:0")
    H = 1
    w = kda_inputs.custom(lengths=list(lengths), H=H, final=None)
    d = kda_inputs.make_inputs(w)
    x = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    T, N = w.T, len(lengths)
    mc = T // 64 + N
    fixed = 2 * al(N * 8) + al(mc * 8) + 2 * al(N * 4) + al((mc + 1) * 4) + al(2 * H * 128 * 128 * 4)
    ws_bytes = fixed + width * H * REC
    assert ws_bytes < kda.workspace_size(1, T, H, N)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=device)
    out = torch.empty(1, T, H, 128, dtype=torch.bfloat16, device=device)
    kda.fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], x['scale'], out, x['A_log'], x['dt_bias'],
            x['lower_bound'], cu_seqlens=x['cu_seqlens'], workspace=ws, force_chunked=True)
    torch.cuda.synchronize()
    b = ws.cpu().numpy()
    count = -(-mc // width)                  # fewest windows that fit, then balanced widths
    wd = -(-mc // count)
    assert wd == width
    off = wd * H * REC
    seq_tab = b[off:off + 8 * N].view(np.int32).reshape(N, 2)
    off = al(off + 8 * N) + al(8 * mc) + al(8 * N) + al(4 * N)
    nz_seq = b[off:off + 4 * N].view(np.int32)
    off = al(off + 4 * N)
    win_first = b[off:off + 4 * (count + 1)].view(np.int32)
    _, ref_tab, _, _, _ = expected_tables(lengths, T)
    assert np.array_equal(seq_tab, ref_tab)
    nz = [n for n in range(N) if ref_tab[n, 1] > 0]
    assert np.array_equal(nz_seq[:len(nz)], nz)
    ends = [ref_tab[n, 0] + ref_tab[n, 1] for n in nz]
    ref_first = [next((k for k, e in enumerate(ends) if e > wi * wd), len(nz)) for wi in range(count)] + [len(nz)]
    assert np.array_equal(win_first, ref_first)
