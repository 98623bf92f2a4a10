"""MI355X (gfx950) Kimi Delta Attention forward -- Python binding of libkda.so.

Argument marshalling only: every step of the forward runs in the HIP kernels
behind the C ABI declared in include/kda.h. PyTorch provides device memory
(including the workspace, from its caching allocator) and the current stream.

    import gated_delta_rule_87_amd as kda
    kda.fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
            initial_state=None, final_state=None, cu_seqlens=None)

mirrors ``flash_kda.fwd`` and its parameter table ("Kernel API" of the
FlashKDA README digest): q, k, g bf16 [B, T, H, 128]; v bf16 [B, T, H, 128];
beta bf16 [B, T, H] (logits); out bf16 [B, T, H, 128] written in place;
A_log fp32 [H]; dt_bias fp32 [H, 128]; lower_bound in [-5, 0]; states bf16 or
fp32 [B|N, H, 128, 128] with equal dtypes; cu_seqlens int64 [N+1] with B = 1.
Returns None. There is no CPU fallback: if libkda.so is missing or fails to
load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["fwd", "fwd_recurrent", "workspace_size", "workspace_min", "record_bytes", "lib", "KDAError", "status_string", "LIB_PATH",
           "profile_start", "profile_stop"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

STATE_NONE, STATE_BF16, STATE_FP32 = 0, 1, 2
FUSE_GATE, FUSE_QK_L2NORM, FUSE_BETA_SIGMOID = 1, 2, 4
GATE_UNBOUNDED = 8
PATH_CHUNKED = 16
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE", 4: "KDA_ERR_VALUE",
           5: "KDA_ERR_ALIGN", 6: "KDA_ERR_WORKSPACE", 7: "KDA_ERR_HIP", 8: "KDA_ERR_CAPACITY"}

_lib = None


class KDAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


def _setup(L):
    """Declare the C signatures of include/kda.h on a loaded libkda.so."""
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    F = ctypes.c_float
    L.kda_fwd_workspace_size.restype = ctypes.c_size_t
    L.kda_fwd_workspace_size.argtypes = [I64, I64, I64, I64]
    L.kda_fwd_workspace_min.restype = ctypes.c_size_t
    L.kda_fwd_workspace_min.argtypes = [I64, I64, I64, I64]
    L.kda_fwd.restype = I
    L.kda_fwd.argtypes = [P, P, P, P, P, F, P, P, P, F, P, I, P, I, P, I64, I64, I64, I64, I64, I64, P,
                          ctypes.c_size_t, P]
    L.kda_fwd_recurrent.restype = I
    L.kda_fwd_recurrent.argtypes = [P, P, P, P, P, F, P, P, P, F, P, I, P, I, P, I64, I64, I64, I64, I64,
                                    I64, P]
    U32 = ctypes.c_uint32
    L.kda_fwd_ex.restype = I
    L.kda_fwd_ex.argtypes = [P, P, P, P, P, F, P, P, P, F, P, I, P, I, P, I64, I64, I64, I64, I64, I64, U32, P,
                             ctypes.c_size_t, P]
    L.kda_fwd_recurrent_ex.restype = I
    L.kda_fwd_recurrent_ex.argtypes = [P, P, P, P, P, F, P, P, P, F, P, I, P, I, P, I64, I64, I64, I64, I64,
                                       I64, U32, P]
    L.kda_fwd_noalloc.restype = I
    L.kda_fwd_noalloc.argtypes = [P, P, P, P, P, F, P, P, P, F, P, I, P, I, P, I64, I64, I64, I64, I64, I64, U32,
                                  P]
    L.kda_noalloc_capacity.restype = ctypes.c_size_t
    L.kda_noalloc_capacity.argtypes = []
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_status_string.argtypes = [I]
    L.kda_version.restype = ctypes.c_char_p
    L.kda_version.argtypes = []
    L.kda_profile_start.restype = I
    L.kda_profile_start.argtypes = [I]
    L.kda_profile_stop.restype = I
    L.kda_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I), I]
    L.kda_profile_kernel_count.restype = I
    L.kda_profile_kernel_count.argtypes = []
    L.kda_profile_kernel_name.restype = ctypes.c_char_p
    L.kda_profile_kernel_name.argtypes = [I]
    return L


def lib():
    """Load libkda.so (built in-tree by gated_delta_rule_87_amd.build). Raises if missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkda.so not built ({LIB_PATH}); run python -m gated_delta_rule_87_amd.build")
        _lib = _setup(ctypes.CDLL(LIB_PATH))
    return _lib


def status_string(code: int) -> str:
    return lib().kda_status_string(int(code)).decode()


def workspace_size(B: int, T: int, H: int, N: int = 0) -> int:
    """Bytes of workspace kda_fwd needs (N = number of sequences with cu_seqlens, else 0)."""
    return int(lib().kda_fwd_workspace_size(int(B), int(T), int(H), int(N)))


def workspace_min(B: int, T: int, H: int, N: int = 0) -> int:
    """Smallest workspace kda_fwd accepts; fixed-length calls given less than
    workspace_size run in windows of chunk columns (kda_fwd_workspace_min)."""
    return int(lib().kda_fwd_workspace_min(int(B), int(T), int(H), int(N)))


def record_bytes() -> int:
    """Workspace bytes per 64-token chunk and head (the intra kernel's record)."""
    return workspace_size(1, 64, 1, 0)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(name, t, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _state_code(t: Optional[torch.Tensor]) -> int:
    if t is None:
        return STATE_NONE
    if t.dtype == torch.bfloat16:
        return STATE_BF16
    if t.dtype == torch.float32:
        return STATE_FP32
    raise ValueError(f"state must be bf16 or fp32, got {t.dtype}")


def _flags(use_gate_in_kernel, use_qk_l2norm_in_kernel, use_beta_sigmoid_in_kernel, safe_gate=True) -> int:
    return ((FUSE_GATE if use_gate_in_kernel else 0) | (FUSE_QK_L2NORM if use_qk_l2norm_in_kernel else 0)
            | (FUSE_BETA_SIGMOID if use_beta_sigmoid_in_kernel else 0) | (0 if safe_gate else GATE_UNBOUNDED))


def _prepare(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state, cu_seqlens, gate_fused=True):
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B, T, H, K]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    B, T, H, K = q.shape
    V = v.shape[-1] if isinstance(v, torch.Tensor) and v.dim() == 4 else -1
    if K != 128 or V != 128:
        raise ValueError(f"K = V = 128 is required (got K={K}, V={V})")
    for name, t in (("q", q), ("k", k), ("g", g)):
        _check(name, t, torch.bfloat16, (B, T, H, K), dev)
    _check("v", v, torch.bfloat16, (B, T, H, V), dev)
    _check("beta", beta, torch.bfloat16, (B, T, H), dev)
    _check("out", out, torch.bfloat16, (B, T, H, V), dev)
    if gate_fused or A_log is not None:
        _check("A_log", A_log, torch.float32, (H,), dev)
    if gate_fused or dt_bias is not None:
        _check("dt_bias", dt_bias, torch.float32, (H, K), dev)
    N = 0
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be int64 [N+1] with N >= 1")
        _check("cu_seqlens", cu_seqlens, torch.int64, tuple(cu_seqlens.shape), dev)
        N = cu_seqlens.numel() - 1
    nseq = N if cu_seqlens is not None else B
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None:
            _check(name, t, t.dtype, (nseq, H, V, K), dev)
            _state_code(t)
    if initial_state is not None and final_state is not None and initial_state.dtype != final_state.dtype:
        raise ValueError("initial_state and final_state must have the same dtype")
    return B, T, H, K, V, N


def _stream_ptr(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def fwd(q, k, v, g, beta, scale: float, out, A_log, dt_bias, lower_bound: float,
        initial_state=None, final_state=None, cu_seqlens=None, workspace: Optional[torch.Tensor] = None,
        use_gate_in_kernel: bool = True, use_qk_l2norm_in_kernel: bool = True,
        use_beta_sigmoid_in_kernel: bool = True, safe_gate: bool = True, force_chunked: bool = False):
    """Chunked KDA forward; writes ``out`` (and ``final_state``) in place, returns None.

    Decode-sized calls (fixed length T <= 8, or varlen with at most two tokens per
    sequence on average) run on the token-recurrent kernel instead, unless
    ``force_chunked`` is set (KDA_PATH_CHUNKED of kda_fwd_ex).

    ``workspace``: a uint8 device tensor (allocated here when None). Fixed-length
    calls given less than workspace_size (at least workspace_min) run in windows of
    chunk columns; a workspace below the minimum is rejected by the library
    (KDAError with KDA_ERR_WORKSPACE).

    The three switches select the in-kernel input processing (default) or take
    that input as already processed: g as the log-decay (clamped into
    [lower_bound, 0]; A_log and dt_bias may be None), q and k as given, beta as
    given. ``safe_gate=False`` drops the lower bound: the gate is
    -exp(A_log) * softplus(g + dt_bias) (or min(g, 0) unfused) and lower_bound is
    ignored (kda_fwd_ex in include/kda.h).
    """
    flags = _flags(use_gate_in_kernel, use_qk_l2norm_in_kernel, use_beta_sigmoid_in_kernel, safe_gate)
    if force_chunked:
        flags |= PATH_CHUNKED
    B, T, H, K, V, N = _prepare(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state, cu_seqlens,
                                gate_fused=use_gate_in_kernel)
    L = lib()
    if workspace is None:
        workspace = torch.empty(max(workspace_size(B, T, H, N), 1), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device:
        raise ValueError(f"workspace must be on {q.device}")
    rc = L.kda_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(out), _ptr(A_log),
                      _ptr(dt_bias), float(lower_bound), _ptr(initial_state), _state_code(initial_state),
                      _ptr(final_state), _state_code(final_state), _ptr(cu_seqlens), N, B, T, H, K, V, flags,
                      _ptr(workspace), workspace.numel() * workspace.element_size(), _stream_ptr(q.device))
    if rc != 0:
        raise KDAError(rc, status_string(rc))
    return None


def fwd_recurrent(q, k, v, g, beta, scale: float, out, A_log, dt_bias, lower_bound: float,
                  initial_state=None, final_state=None, cu_seqlens=None, use_gate_in_kernel: bool = True,
                  use_qk_l2norm_in_kernel: bool = True, use_beta_sigmoid_in_kernel: bool = True,
                  safe_gate: bool = True):
    """Token-by-token KDA forward (online generation / reference); same contract as fwd."""
    flags = _flags(use_gate_in_kernel, use_qk_l2norm_in_kernel, use_beta_sigmoid_in_kernel, safe_gate)
    B, T, H, K, V, N = _prepare(q, k, v, g, beta, out, A_log, dt_bias, initial_state, final_state, cu_seqlens,
                                gate_fused=use_gate_in_kernel)
    rc = lib().kda_fwd_recurrent_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(out),
                                    _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
                                    _state_code(initial_state), _ptr(final_state), _state_code(final_state),
                                    _ptr(cu_seqlens), N, B, T, H, K, V, flags, _stream_ptr(q.device))
    if rc != 0:
        raise KDAError(rc, status_string(rc))
    return None


def profile_start(max_calls: int) -> None:
    """Time each kernel of the next ``max_calls`` fwd calls with HIP events on their stream."""
    rc = lib().kda_profile_start(int(max_calls))
    if rc != 0:
        raise KDAError(rc, status_string(rc))


def profile_stop() -> dict:
    """Wait for the timed calls; return {kernel name: (summed ms, launches)} and stop timing."""
    L = lib()
    n = L.kda_profile_kernel_count()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    rc = L.kda_profile_stop(ms, cnt, n)
    if rc != 0:
        raise KDAError(rc, status_string(rc))
    return {L.kda_profile_kernel_name(i).decode(): (ms[i], cnt[i]) for i in range(n)}
