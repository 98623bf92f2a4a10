"""Seeded synthetic inputs for the KDA forward workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the product path (tests, bench) and the CPU oracle's
tests take their inputs from here, so the two sides see identical data.

Recipe (shared by every workload):
  * one CPU ``torch.Generator`` seeded with ``seed`` (0 by default);
  * draw order: sequence lengths (ragged workload only), q, k, v, g, beta,
    A_log, dt_bias, initial_state;
  * q, k, v, g, beta ~ N(0, 1) drawn in fp32 and rounded to bf16 (RNE);
  * A_log ~ U(0, ln 16) fp32;  dt_bias ~ N(0, 0.1^2) fp32 (0.1 is the std);
  * initial_state ~ N(0, 0.02^2), fp32, rounded to bf16 when the state dtype
    is bf16;
  * large tensors are drawn slab by slab (``SLAB`` tokens of all heads at a
    time) so peak host memory stays bounded; the slab size is part of the
    recipe, so the values never depend on the machine.

The kernel API these inputs feed follows the FlashKDA "Kernel API" table:
q, k, g [B, T, H, K] bf16, v [B, T, H, V] bf16, beta [B, T, H] bf16,
A_log [H] fp32, dt_bias [H, K] fp32, state [B|N, H, V, K].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

SLAB = 1024          # tokens per draw slab
K_DIM = 128
V_DIM = 128


@dataclass
class Workload:
    name: str
    B: int
    T: int                       # per-row length (B>1) or total packed length (varlen)
    H: int
    lower_bound: float = -5.0
    scale: float = 1.0 / math.sqrt(128.0)
    lengths: Optional[list] = None   # varlen sequence lengths (B must be 1)
    state: Optional[str] = None      # None | 'fp32' | 'bf16' : initial_state given?
    final: Optional[str] = 'fp32'    # final_state dtype requested (None = not requested)
    seed: int = 0
    K: int = K_DIM
    V: int = V_DIM
    extra: dict = field(default_factory=dict)

    @property
    def n_seqs(self) -> int:
        return len(self.lengths) if self.lengths is not None else self.B

    @property
    def tokens(self) -> int:
        return self.B * self.T


def ragged_lengths(gen: torch.Generator, n: int, lo: int = 64, hi: int = 4096) -> list:
    """Lengths drawn log-uniform in [lo, hi]: round(exp(U(ln lo, ln hi)))."""
    u = torch.rand(n, generator=gen, dtype=torch.float64)
    x = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    return [int(round(float(t))) for t in x]


def workload(idx: int) -> Workload:
    """The named workloads (by index): 0-4 prefill shapes, 5 a decode step, 6 the
    prefill's per-GPU share under 8-way head (tensor) parallelism."""
    if idx == 0:
        return Workload("tiny_T256_H2", B=1, T=256, H=2)
    if idx == 1:
        return Workload("prefill_T8192_H64", B=1, T=8192, H=64)
    if idx == 2:
        return Workload("varlen_8x1024_H64", B=1, T=8192, H=64, lengths=[1024] * 8, state='fp32')
    if idx == 3:
        gen = torch.Generator().manual_seed(0)
        lens = ragged_lengths(gen, 32)
        return Workload("ragged_N32_H64", B=1, T=sum(lens), H=64, lengths=lens, state='bf16',
                        final='bf16', lower_bound=-2.0, extra={'draw_lengths': True})
    if idx == 4:
        return Workload("batched_B4_T32768_H64", B=4, T=32768, H=64, state='fp32')
    if idx == 5:   # one generation step: one token per sequence, state passed in and out
        return Workload("decode_N256_H64", B=1, T=256, H=64, lengths=[1] * 256, state='fp32')
    if idx == 6:   # one GPU's share of the prefill when the 64 heads are split over 8 GPUs
        return Workload("tp8_share_T8192_H8", B=1, T=8192, H=8)
    raise ValueError(idx)


def _normal_bf16(gen, shape, std=1.0):
    """N(0, std^2) drawn in fp32 slab by slab along dim 1 (tokens), rounded to bf16."""
    out = torch.empty(shape, dtype=torch.bfloat16)
    if len(shape) >= 2 and shape[1] > SLAB:
        for b in range(shape[0]):
            for t0 in range(0, shape[1], SLAB):
                t1 = min(shape[1], t0 + SLAB)
                sub = (t1 - t0,) + tuple(shape[2:])
                out[b, t0:t1] = (torch.randn(sub, generator=gen, dtype=torch.float32) * std).to(torch.bfloat16)
    else:
        out.copy_((torch.randn(shape, generator=gen, dtype=torch.float32) * std).to(torch.bfloat16))
    return out


def make_inputs(w: Workload) -> dict:
    """Draw every input of workload ``w`` on the CPU. Returns a dict of tensors."""
    gen = torch.Generator().manual_seed(w.seed)
    if w.lengths is not None and w.extra.get('draw_lengths', False):
        ragged_lengths(gen, len(w.lengths))     # keep the draw order of the recipe
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    d = {}
    d['q'] = _normal_bf16(gen, (B, T, H, K))
    d['k'] = _normal_bf16(gen, (B, T, H, K))
    d['v'] = _normal_bf16(gen, (B, T, H, V))
    d['g'] = _normal_bf16(gen, (B, T, H, K))
    d['beta'] = _normal_bf16(gen, (B, T, H))
    d['A_log'] = torch.rand(H, generator=gen, dtype=torch.float32) * math.log(16.0)
    d['dt_bias'] = torch.randn(H, K, generator=gen, dtype=torch.float32) * 0.1
    ns = w.n_seqs
    if w.state is not None:
        s = torch.randn(ns, H, V, K, generator=gen, dtype=torch.float32) * 0.02
        d['initial_state'] = s.to(torch.bfloat16) if w.state == 'bf16' else s
    else:
        d['initial_state'] = None
    if w.lengths is not None:
        cu = [0]
        for L in w.lengths:
            cu.append(cu[-1] + L)
        d['cu_seqlens'] = torch.tensor(cu, dtype=torch.int64)
    else:
        d['cu_seqlens'] = None
    d['scale'] = float(w.scale)
    d['lower_bound'] = float(w.lower_bound)
    return d


def make_inputs_device(w: Workload, device) -> dict:
    """The same distributions drawn directly on ``device`` with a seeded device
    generator, slab by slab, for sizes the host should not hold. Draw order as in
    make_inputs; the values differ from make_inputs' (another generator)."""
    gen = torch.Generator(device=device).manual_seed(w.seed)
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V

    def normal_bf16(shape):
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
        for t0 in range(0, shape[1], SLAB):
            t1 = min(shape[1], t0 + SLAB)
            sl = (shape[0], t1 - t0) + tuple(shape[2:])
            out[:, t0:t1] = torch.randn(sl, generator=gen, dtype=torch.float32, device=device).to(torch.bfloat16)
        return out

    d = {'q': normal_bf16((B, T, H, K)), 'k': normal_bf16((B, T, H, K)), 'v': normal_bf16((B, T, H, V)),
         'g': normal_bf16((B, T, H, K)), 'beta': normal_bf16((B, T, H))}
    d['A_log'] = torch.rand(H, generator=gen, dtype=torch.float32, device=device) * math.log(16.0)
    d['dt_bias'] = torch.randn(H, K, generator=gen, dtype=torch.float32, device=device) * 0.1
    if w.state is not None:
        s = torch.randn(w.n_seqs, H, V, K, generator=gen, dtype=torch.float32, device=device) * 0.02
        d['initial_state'] = s.to(torch.bfloat16) if w.state == 'bf16' else s
    else:
        d['initial_state'] = None
    d['cu_seqlens'] = None
    if w.lengths is not None:
        cu = [0]
        for L in w.lengths:
            cu.append(cu[-1] + L)
        d['cu_seqlens'] = torch.tensor(cu, dtype=torch.int64, device=device)
    d['scale'] = float(w.scale)
    d['lower_bound'] = float(w.lower_bound)
    return d


def custom(B=1, T=64, H=1, lengths=None, state=None, final='fp32', lower_bound=-5.0, seed=0,
           scale=None, K=K_DIM, V=V_DIM) -> Workload:
    """A small workload of the same distributions (for parity and edge cases)."""
    if lengths is not None:
        B, T = 1, int(sum(lengths))
    return Workload(f"custom_B{B}_T{T}_H{H}", B=B, T=T, H=H, lower_bound=lower_bound,
                    scale=(1.0 / math.sqrt(K)) if scale is None else scale,
                    lengths=list(lengths) if lengths is not None else None,
                    state=state, final=final, seed=seed, K=K, V=V)
