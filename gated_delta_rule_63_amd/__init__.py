"""MI355X (gfx950) chunked prefill of Kimi Delta Attention (KDA).

    o_t = S_t^T q_t,  S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T

per (sequence, head), K = V = 128, bf16 or fp32 q/k/v, fp32 g/beta/state, batched
or variable-length (cu_seqlens), optional initial and final states. The work
runs in the HIP library libkda.so (include/kda.h); this module only marshals
torch tensors (device memory and the current stream) into its C ABI.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from ._lib import KDA_BF16, KDA_F32, KERNELS, Desc, KDAError, Layout, lib, status_string  # noqa: F401

__all__ = ["fwd", "gdn_fwd", "fwd_noalloc", "noalloc_max_workspace", "fwd_workspace_size", "kernel_workspace_size", "decode_step", "fwd_staged", "Staged", "KDAError", "status_string", "version"]

D = 128


def version() -> int:
    return int(lib().kda_version())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _desc(q: torch.Tensor, cu_seqlens: Optional[torch.Tensor]) -> Desc:
    B, T, H, K = q.shape
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    dt = {torch.bfloat16: KDA_BF16, torch.float32: KDA_F32}.get(q.dtype, -1)
    return Desc(B, T, H, K, K, N, dt, KDA_F32, None, 0)


def _check_inputs(q, k, v, g, beta, cu_seqlens, scalar_gate=False, _device=True):
    """Raises ValueError unless the inputs are what the C ABI reads: contiguous
    tensors on one GPU with the shapes and dtypes of include/kda.h. (_device=False
    skips the GPU requirement only, so the checks can be exercised on the CPU.)"""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        if (_device and not t.is_cuda) or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be a contiguous device tensor on q's device")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    if g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise ValueError("g and beta must be float32")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, T, H, 128]")
    if g.shape != (q.shape[:3] if scalar_gate else q.shape):
        raise ValueError("g must be [B, T, H]" if scalar_gate else "g must be [B, T, H, 128]")
    if beta.shape != q.shape[:3]:
        raise ValueError("beta must be [B, T, H]")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
                                   or cu_seqlens.numel() < 1 or not cu_seqlens.is_contiguous()
                                   or cu_seqlens.device != dev):
        raise ValueError("cu_seqlens must be a contiguous int32 [N + 1] tensor on q's device")
    if cu_seqlens is not None and q.shape[0] != 1:
        raise ValueError("with cu_seqlens the batch dimension must be 1 (sequences packed into one row)")


def _check_state(name, t, shape, device):
    """A state tensor the kernels read or write: contiguous fp32 of `shape` on `device`."""
    if t is None:
        return
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape) or t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor on q's device")


def _check_out(name, t, shape, device):
    """An output the kernels write: contiguous fp32 of `shape` on `device`."""
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape) or t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 {list(shape)} tensor on q's device")


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
        cu_seqlens: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
        output_final_state: bool = True, out: Optional[torch.Tensor] = None,
        final_state: Optional[torch.Tensor] = None,
        stream: Optional[torch.cuda.Stream] = None,
        kernel: str = "auto", workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """KDA chunked forward. Shapes: q, k, v, g [B, T, H, 128]; beta [B, T, H];
    cu_seqlens int32 [N + 1] (B == 1); initial_state / final state [N, H, 128, 128] fp32.

    Returns (o fp32 [B, T, H, 128], hT or None). Tensors must be contiguous and on
    one GPU; q, k, v share a dtype (bf16 or fp32); g and beta are fp32.
    kernel: "auto" (kda_fwd), or "pipe", "serial", "chunk16", "two_pass" to run
    that one forward kernel (kda_fwd_kernel). workspace: an optional device
    tensor handed over as desc->workspace (see kernel_workspace_size).
    """
    if kernel == "auto":
        return _forward("kda_fwd", q, k, v, g, beta, cu_seqlens, initial_state, output_final_state,
                        out, final_state, stream, workspace=workspace)
    if kernel not in KERNELS:
        raise ValueError(f"kernel must be one of {sorted(KERNELS)}")
    return _forward("kda_fwd_kernel", q, k, v, g, beta, cu_seqlens, initial_state, output_final_state,
                    out, final_state, stream, ctypes.c_int32(KERNELS[kernel]), workspace=workspace)


def fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                cu_seqlens: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
                output_final_state: bool = True, out: Optional[torch.Tensor] = None,
                final_state: Optional[torch.Tensor] = None,
                stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_fwd_noalloc: fwd() whose workspace is the library's static device array
    (no device allocation inside the call; pass `out` and `final_state` to keep
    this wrapper from allocating them). Calls that overlap on one GPU race."""
    return _forward("kda_fwd_noalloc", q, k, v, g, beta, cu_seqlens, initial_state, output_final_state,
                    out, final_state, stream)


def noalloc_max_workspace() -> int:
    """Bytes of kda_fwd_noalloc's static workspace."""
    return int(lib().kda_fwd_noalloc_max_workspace())


def fwd_workspace_size(q: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None) -> int:
    """Bytes of device workspace fwd() / gdn_fwd() use for inputs shaped like q
    (kda_fwd_workspace_size; 0 for most shapes). For few long chains, a workspace
    of at least this size selects the faster one-pass slice route and keeps fwd()
    from allocating; without one, fwd() allocates the three-slice route's."""
    return int(lib().kda_fwd_workspace_size(ctypes.byref(_desc(q, cu_seqlens))))


def kernel_workspace_size(q: torch.Tensor, kernel: str, cu_seqlens: Optional[torch.Tensor] = None) -> int:
    """Bytes of device workspace fwd(..., kernel=kernel) uses (0: none)."""
    return int(lib().kda_fwd_kernel_workspace_size(ctypes.byref(_desc(q, cu_seqlens)), KERNELS[kernel]))


def gdn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
            cu_seqlens: Optional[torch.Tensor] = None, initial_state: Optional[torch.Tensor] = None,
            output_final_state: bool = True, out: Optional[torch.Tensor] = None,
            final_state: Optional[torch.Tensor] = None,
            stream: Optional[torch.cuda.Stream] = None,
            workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gated DeltaNet forward (kda_gdn_fwd): as fwd, but g is one fp32 log-decay per
    (token, head), [B, T, H]. workspace: as for fwd (fwd_workspace_size)."""
    return _forward("kda_gdn_fwd", q, k, v, g, beta, cu_seqlens, initial_state, output_final_state,
                    out, final_state, stream, workspace=workspace)


def _forward(entry, q, k, v, g, beta, cu_seqlens, initial_state, output_final_state, out, final_state,
             stream, *extra, workspace=None):
    _check_inputs(q, k, v, g, beta, cu_seqlens, scalar_gate=(entry == "kda_gdn_fwd"))
    d = _desc(q, cu_seqlens)
    if workspace is not None:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        d.workspace = workspace.data_ptr()
        d.workspace_bytes = workspace.numel() * workspace.element_size()
    B, T, H, _ = q.shape
    sshape = (d.num_seqs, H, D, D)
    _check_state("initial_state", initial_state, sshape, q.device)
    if out is not None:
        _check_out("out", out, (B, T, H, D), q.device)
    if final_state is not None:
        _check_out("final_state", final_state, sshape, q.device)
    o = out if out is not None else torch.empty((B, T, H, D), dtype=torch.float32, device=q.device)
    hT = None
    if output_final_state:
        hT = final_state if final_state is not None else torch.empty(sshape, dtype=torch.float32, device=q.device)
    s = (stream or torch.cuda.current_stream(q.device)).cuda_stream
    rc = getattr(lib(), entry)(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                               _ptr(initial_state), _ptr(o), _ptr(hT), ctypes.byref(d), *extra,
                               ctypes.c_void_p(s))
    if rc != 0:
        raise KDAError(rc, entry)
    return o, hT


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                new_state: Optional[torch.Tensor] = None, in_place: bool = False,
                stream: Optional[torch.cuda.Stream] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One decode step for N sequences: q, k, v, g [N, 1, H, 128]; beta [N, 1, H];
    state [N, H, 128, 128] fp32 (None: zero). Returns (o fp32 [N, 1, H, 128], new state).
    With in_place=True the new state overwrites `state`."""
    _check_inputs(q, k, v, g, beta, None)
    N, T, H, _ = q.shape
    if T != 1:
        raise ValueError("decode_step takes one token per sequence ([N, 1, H, 128])")
    _check_state("state", state, (N, H, D, D), q.device)
    if out is not None:
        _check_out("out", out, (N, 1, H, D), q.device)
    if new_state is not None:
        _check_out("new_state", new_state, (N, H, D, D), q.device)
    if in_place:
        if state is None:
            raise ValueError("in_place needs a state")
        new_state = state
    elif new_state is None:
        new_state = torch.empty((N, H, D, D), dtype=torch.float32, device=q.device)
    o = out if out is not None else torch.empty((N, 1, H, D), dtype=torch.float32, device=q.device)
    d = _desc(q, None)
    s = (stream or torch.cuda.current_stream(q.device)).cuda_stream
    rc = lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                               _ptr(new_state), ctypes.byref(d), ctypes.c_void_p(s))
    if rc != 0:
        raise KDAError(rc, "kda_decode_step")
    return o, new_state


class Staged:
    """The staged path (a0 chunk map, a1 gate scan, a2 intra-chunk, a3 recurrence,
    a4 output) over one workspace. Each stage is one kernel on the current stream;
    the intermediates are tensor views into the workspace (fp32, 32-token chunks)."""

    def __init__(self, q, k, v, g, beta, cu_seqlens=None, initial_state=None, workspace=None):
        _check_inputs(q, k, v, g, beta, cu_seqlens)
        self.q, self.k, self.v, self.g, self.beta, self.cu = q, k, v, g, beta, cu_seqlens
        self.h0 = initial_state
        self.desc = _desc(q, cu_seqlens)
        L = Layout()
        rc = lib().kda_staged_layout(ctypes.byref(self.desc), ctypes.byref(L))
        if rc != 0:
            raise KDAError(rc, "kda_staged_layout")
        self.layout = L
        if workspace is None:
            workspace = torch.empty(L.total, dtype=torch.uint8, device=q.device)
        if workspace.numel() < L.total:
            raise ValueError("workspace too small")
        self.ws = workspace
        self.desc.workspace = ctypes.c_void_p(workspace.data_ptr())
        self.desc.workspace_bytes = workspace.numel()
        B, T, H, _ = q.shape
        N, S, C = self.desc.num_seqs, L.nslots, L.chunk

        def view(off, shape, dtype):
            n = 1
            for x in shape:
                n *= x
            item = torch.empty((), dtype=dtype).element_size()
            return workspace[off:off + n * item].view(dtype).view(*shape)

        self.map = view(L.map, (S, 4), torch.int32)
        self.seqinfo = view(L.seqinfo, (max(N, 1), 2), torch.int32)
        self.Gamma = view(L.Gamma, (B, T, H, D), torch.float32)
        self.gl = view(L.gl, (S, H, D), torch.float32)
        self.W = view(L.W, (B, T, H, D), torch.float32)
        self.U = view(L.U, (B, T, H, D), torch.float32)
        self.Kt = view(L.Kt, (B, T, H, D), torch.float32)
        self.Qg = view(L.Qg, (B, T, H, D), torch.float32)
        self.M = view(L.M, (S, H, C, C), torch.float32)
        self.hc = view(L.hc, (S, H, D, D), torch.float32)
        self.Delta = view(L.Delta, (B, T, H, D), torch.float32)

    def _s(self):
        return ctypes.c_void_p(torch.cuda.current_stream(self.q.device).cuda_stream)

    def _rc(self, rc, name):
        if rc != 0:
            raise KDAError(rc, name)

    def chunk_map(self):
        self._rc(lib().kda_stage_chunk_map(_ptr(self.cu), ctypes.byref(self.desc), self._s()), "kda_stage_chunk_map")

    def gate_scan(self):
        self._rc(lib().kda_stage_gate_scan(_ptr(self.g), ctypes.byref(self.desc), self._s()), "kda_stage_gate_scan")

    def intra(self):
        self._rc(lib().kda_stage_intra(_ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(self.beta),
                                       ctypes.byref(self.desc), self._s()), "kda_stage_intra")

    def recurrence(self, final_state=None):
        self._rc(lib().kda_stage_recurrence(_ptr(self.h0), _ptr(final_state), ctypes.byref(self.desc), self._s()),
                 "kda_stage_recurrence")

    def output(self, o):
        self._rc(lib().kda_stage_output(_ptr(o), ctypes.byref(self.desc), self._s()), "kda_stage_output")


def fwd_staged(q, k, v, g, beta, cu_seqlens=None, initial_state=None, output_final_state=True,
               workspace=None):
    """kda_fwd_staged: the five stage kernels in order. Returns (o, hT or None, Staged)."""
    st = Staged(q, k, v, g, beta, cu_seqlens, initial_state, workspace)
    B, T, H, _ = q.shape
    o = torch.empty((B, T, H, D), dtype=torch.float32, device=q.device)
    hT = torch.empty((st.desc.num_seqs, H, D, D), dtype=torch.float32, device=q.device) \
        if output_final_state else None
    rc = lib().kda_fwd_staged(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                              _ptr(initial_state), _ptr(o), _ptr(hT), ctypes.byref(st.desc), st._s())
    if rc != 0:
        raise KDAError(rc, "kda_fwd_staged")
    return o, hT, st
