"""CPU oracle for the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
bench.py may import this package. The GPU product path
(``gated_delta_rule_87_amd``) never imports it and shares no code with it.

Two independent implementations of the same plain recurrence live here:

* ``kda_oracle``        -- ctypes front end of ``kda_oracle.c`` (fp64, OpenMP
                           over independent (sequence, head) chains);
* ``kda_oracle_numpy``  -- a numpy transcription for tiny cases, used to
                           cross-check the C code.

The recurrence (per sequence and head; state S is V x K):
    q^ = q / sqrt(sum q^2 + 1e-6), k^ likewise;  beta = sigmoid(b)
    g~ = lower_bound * sigmoid(exp(A_log[h]) * (g + dt_bias[h]))
    S <- S Diag(exp(g~));  S <- S - beta (S k^ - v) k^^T;  o = scale S q^
KDA is Gated DeltaNet with a per-channel gate ("FlashKDA ... CUDA 加速實作",
section 背景); argument roles follow the "Kernel API" table of the FlashKDA
README digest. The pages print no equation: the gate form, natural exp, the
1e-6 epsilon and the operation order are this package's stated readings.

Every function here has a pin in tests/test_oracle.py (closed forms,
brute-force unrolled products, chaining/varlen/structure identities); none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

STATE_NONE, STATE_BF16, STATE_FP32, STATE_FP64 = 0, 1, 2, 3


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_fwd.argtypes = [P, P, P, P, P, ctypes.c_double, P, P, ctypes.c_double, P,
                                       ctypes.c_int, P, P, P, I64, I64, I64, I64, I64, I64, P, I64,
                                       ctypes.c_int, ctypes.c_int]
        _lib = lib
    return _lib


def _bf16_bits(x) -> np.ndarray:
    """bf16 tensor/array -> contiguous uint16 bit array (no rounding: must be bf16 already)."""
    import torch
    if isinstance(x, torch.Tensor):
        assert x.dtype == torch.bfloat16, x.dtype
        return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16
    return x


def _f32(x) -> np.ndarray:
    import torch
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().float().numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def _state(x):
    """-> (array, dtype code)."""
    import torch
    if x is None:
        return None, STATE_NONE
    if isinstance(x, torch.Tensor):
        if x.dtype == torch.bfloat16:
            return _bf16_bits(x), STATE_BF16
        if x.dtype == torch.float32:
            return _f32(x), STATE_FP32
        if x.dtype == torch.float64:
            return np.ascontiguousarray(x.detach().cpu().numpy()), STATE_FP64
        raise TypeError(x.dtype)
    x = np.ascontiguousarray(x)
    if x.dtype == np.float64:
        return x, STATE_FP64
    if x.dtype == np.float32:
        return x, STATE_FP32
    if x.dtype == np.uint16:
        return x, STATE_BF16
    raise TypeError(x.dtype)


FUSE_GATE, FUSE_QK_L2NORM, FUSE_BETA_SIGMOID = 1, 2, 4
FUSE_ALL = 7
GATE_UNBOUNDED = 8


def kda_oracle(q, k, v, g, beta, scale: float, A_log, dt_bias, lower_bound: float,
               initial_state=None, cu_seqlens=None, heads: Optional[Sequence[int]] = None,
               want_final: bool = True, nthreads: int = 0, use_gate_in_kernel: bool = True,
               use_qk_l2norm_in_kernel: bool = True, use_beta_sigmoid_in_kernel: bool = True,
               safe_gate: bool = True):
    """fp64 reference. Tensors in the kernel's storage formats (torch or numpy).

    q, k, g, v: bf16 [B, T, H, 128]; beta bf16 [B, T, H]; A_log fp32 [H];
    dt_bias fp32 [H, K]; initial_state None or [nseq, H, V, K] (bf16/fp32/fp64);
    cu_seqlens None or int64 [N+1] (B must be 1); heads: subset of head ids.
    The three switches select the fused input processing (True) or take the
    input as already processed (False): g as the log-decay clamped into
    [lower_bound, 0] (A_log, dt_bias may then be None), q and k as given, beta
    as given. ``safe_gate=False`` drops the lower bound: the fused gate is
    -exp(A_log) * softplus(g + dt_bias), the unfused one min(g, 0), and
    lower_bound is not used.

    Returns (out fp64 [B*T, nh, V], final fp64 [nseq, nh, V, K] or None).
    ``scale`` and ``lower_bound`` are taken as the fp32 values a kernel call
    would receive.
    """
    lib = _load()
    qb, kb, vb, gb, bb = (_bf16_bits(t) for t in (q, k, v, g, beta))
    B, T, H, K = qb.shape
    V = vb.shape[-1]
    assert kb.shape == (B, T, H, K) and gb.shape == (B, T, H, K) and vb.shape == (B, T, H, V)
    assert bb.shape == (B, T, H)
    flags = ((FUSE_GATE if use_gate_in_kernel else 0) | (FUSE_QK_L2NORM if use_qk_l2norm_in_kernel else 0)
             | (FUSE_BETA_SIGMOID if use_beta_sigmoid_in_kernel else 0) | (0 if safe_gate else GATE_UNBOUNDED))
    al = _f32(A_log) if A_log is not None else None
    dt = _f32(dt_bias) if dt_bias is not None else None
    if use_gate_in_kernel:
        assert al.shape == (H,) and dt.shape == (H, K)
    cu = None
    N = 0
    if cu_seqlens is not None:
        import torch
        cu = np.ascontiguousarray(cu_seqlens.cpu().numpy() if isinstance(cu_seqlens, torch.Tensor)
                                  else cu_seqlens, dtype=np.int64)
        N = cu.shape[0] - 1
    nseq = N if cu is not None else B
    if heads is None:
        hs = None
        nh = H
    else:
        hs = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
        nh = hs.shape[0]
    st, code = _state(initial_state)
    if st is not None:
        assert st.shape == (nseq, H, V, K), st.shape
    out = np.empty((B * T, nh, V), dtype=np.float64)
    fin = np.empty((nseq, nh, V, K), dtype=np.float64) if want_final else None
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    sc = float(np.float32(scale))
    lb = float(np.float32(lower_bound))
    rc = lib.kda_oracle_fwd(ptr(qb), ptr(kb), ptr(vb), ptr(gb), ptr(bb), sc, ptr(al), ptr(dt), lb,
                            ptr(st), code, ptr(fin), ptr(out), ptr(cu), N, B, T, H, K, V, ptr(hs),
                            nh, int(nthreads), flags)
    if rc != 0:
        raise ValueError(f"kda_oracle_fwd failed with code {rc}")
    return out, fin


def kda_oracle_numpy(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, initial_state=None,
                     cu_seqlens=None, use_gate_in_kernel=True, use_qk_l2norm_in_kernel=True,
                     use_beta_sigmoid_in_kernel=True, safe_gate=True):
    """numpy transcription of the same recurrence (tiny inputs only).

    Inputs as float64 numpy arrays holding the exact values: q, k, g [B,T,H,K],
    v [B,T,H,V], beta logits [B,T,H], A_log [H], dt_bias [H,K],
    initial_state [nseq,H,V,K] or None. Returns (out [B*T,H,V], final [nseq,H,V,K]).
    The switches have the meaning documented in kda_oracle.
    """
    q, k, v, g, beta = (np.asarray(t, dtype=np.float64) for t in (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    qf, kf, vf, gf = (t.reshape(B * T, H, -1) for t in (q, k, v, g))
    bf = beta.reshape(B * T, H)
    if cu_seqlens is None:
        bounds = [(b * T, (b + 1) * T) for b in range(B)]
    else:
        cu = [int(x) for x in np.asarray(cu_seqlens)]
        bounds = list(zip(cu[:-1], cu[1:]))
    out = np.zeros((B * T, H, V))
    fin = np.zeros((len(bounds), H, V, K))
    for n, (t0, t1) in enumerate(bounds):
        for h in range(H):
            S = np.zeros((V, K)) if initial_state is None else np.array(initial_state[n, h], dtype=np.float64)
            rate = np.exp(np.float64(A_log[h])) if use_gate_in_kernel else 0.0
            for t in range(t0, t1):
                if use_qk_l2norm_in_kernel:
                    qh = qf[t, h] / np.sqrt(np.dot(qf[t, h], qf[t, h]) + 1e-6)
                    kh = kf[t, h] / np.sqrt(np.dot(kf[t, h], kf[t, h]) + 1e-6)
                else:
                    qh, kh = qf[t, h], kf[t, h]
                b = 1.0 / (1.0 + np.exp(-bf[t, h])) if use_beta_sigmoid_in_kernel else bf[t, h]
                if use_gate_in_kernel and safe_gate:
                    gate = lower_bound / (1.0 + np.exp(-rate * (gf[t, h] + dt_bias[h])))
                elif use_gate_in_kernel:
                    gate = -rate * np.logaddexp(0.0, gf[t, h] + dt_bias[h])   # -rate * softplus
                elif safe_gate:
                    gate = np.clip(gf[t, h], lower_bound, 0.0)
                else:
                    gate = np.minimum(gf[t, h], 0.0)
                S = S * np.exp(gate)[None, :]
                S = S - b * np.outer(S @ kh - vf[t, h], kh)
                out[t, h] = scale * (S @ qh)
            fin[n, h] = S
    return out, fin
