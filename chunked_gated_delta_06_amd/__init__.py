"""Chunked gated delta rule on AMD MI355X (gfx950): Python binding.

A thin ctypes layer over ``libgdr.so`` (the C ABI in ``include/gdr.h``).  It
only marshals arguments: PyTorch provides device memory and the current HIP
stream, every step of the operator runs in the library's HIP kernels.  There
is no fallback: if the library is missing or the tensors are not on the GPU
the calls raise.

    o, ht = chunk_fwd(q, k, v, g, beta, scale=1.0, chunk_size=64,
                      cu_seqlens=None, initial_state=None,
                      output_final_state=True, use_qk_l2norm_in_kernel=False)
    dq, dk, dv, dg, dbeta, dh0 = chunk_bwd(q, k, v, g, beta, do, dht, ...)

Shapes follow the library: q, k [B,T,H,K]; v [B,T,HV,V]; g [B,T,HV] (or
[B,T,HV,K] for a per-channel gate) and beta [B,T,HV] in float32 (``beta_logits=True``:
beta holds logits and the kernels apply the sigmoid); initial_state
[N,HV,K,V] float32; cu_seqlens int32 [N+1] (then B == 1).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "gdr.h")

GDR_BF16, GDR_FP32 = 0, 1
STATUS = {
    0: "GDR_OK", 1: "GDR_ERR_NULL_ARG", 2: "GDR_ERR_CHUNK_SIZE", 3: "GDR_ERR_SHAPE",
    4: "GDR_ERR_VARLEN", 5: "GDR_ERR_DTYPE", 6: "GDR_ERR_ALIGNMENT", 7: "GDR_ERR_WORKSPACE",
    8: "GDR_ERR_HIP", 9: "GDR_ERR_CU_SEQLENS", 10: "GDR_ERR_UNSUPPORTED", 11: "GDR_ERR_SCRATCH_LIMIT",
}


class GdrProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("HV", ctypes.c_int64), ("K", ctypes.c_int64), ("V", ctypes.c_int64),
                ("N", ctypes.c_int64), ("chunk_size", ctypes.c_int32),
                ("gate_per_channel", ctypes.c_int32), ("use_qk_l2norm", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("keep_states", ctypes.c_int32),
                ("beta_logits", ctypes.c_int32)]


class GdrFwdLayout(ctypes.Structure):
    _fields_ = [("nt_max", ctypes.c_int64), ("chunk_idx", ctypes.c_size_t),
                ("chunk_off", ctypes.c_size_t), ("seq_order", ctypes.c_size_t), ("Tm", ctypes.c_size_t),
                ("w", ctypes.c_size_t),
                ("u", ctypes.c_size_t), ("h", ctypes.c_size_t), ("v_new", ctypes.c_size_t),
                ("kscale", ctypes.c_size_t), ("kt", ctypes.c_size_t), ("dl", ctypes.c_size_t),
                ("aqk", ctypes.c_size_t), ("qgs", ctypes.c_size_t), ("total", ctypes.c_size_t)]


class GdrBwdLayout(ctypes.Structure):
    _fields_ = [("fwd", GdrFwdLayout), ("chunk_size", ctypes.c_int64), ("de_local", ctypes.c_size_t),
                ("qscale", ctypes.c_size_t),
                ("dh", ctypes.c_size_t), ("kt", ctypes.c_size_t), ("qg", ctypes.c_size_t),
                ("dl", ctypes.c_size_t), ("total", ctypes.c_size_t)]


class GdrSegLayout(ctypes.Structure):
    _fields_ = [("fwd", GdrFwdLayout), ("u_zero", ctypes.c_size_t), ("h_tr", ctypes.c_size_t),
                ("v_tr", ctypes.c_size_t), ("eye", ctypes.c_size_t), ("s_ext", ctypes.c_size_t),
                ("trans", ctypes.c_size_t), ("s_in", ctypes.c_size_t), ("total", ctypes.c_size_t)]


class GdrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """Load libgdr.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with chunked_gated_delta_06_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        PP = ctypes.POINTER(GdrProblem)
        L.gdr_abi_version.restype = ctypes.c_int
        L.gdr_status_string.restype = ctypes.c_char_p
        L.gdr_status_string.argtypes = [ctypes.c_int]
        L.gdr_check_problem.argtypes = [PP]
        L.gdr_validate_cu_seqlens.argtypes = [_P, ctypes.c_int64, ctypes.c_int64]
        L.gdr_fwd_workspace_bytes.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
        L.gdr_fwd_workspace_layout.argtypes = [PP, ctypes.POINTER(GdrFwdLayout)]
        L.gdr_chunk_fwd.argtypes = [PP] + [_P] * 9 + [_P, ctypes.c_size_t, _P]
        L.gdr_chunk_fwd_noalloc.argtypes = [PP] + [_P] * 9 + [_P]
        L.gdr_stage_timing.argtypes = [ctypes.c_int]
        L.gdr_stage_timing.restype = ctypes.c_int
        L.gdr_stage_times.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float), ctypes.c_int]
        L.gdr_stage_times.restype = ctypes.c_int
        L.gdr_chunk_table.argtypes = [PP, _P, _P, _P, _P]
        L.gdr_fwd_kkt_solve.argtypes = [PP] + [_P] * 7 + [_P]
        L.gdr_fwd_wy.argtypes = [PP] + [_P] * 9 + [_P]
        L.gdr_fwd_kkt_wy.argtypes = [PP] + [_P] * 9 + [_P]
        L.gdr_fwd_h.argtypes = [PP] + [_P] * 11 + [_P]
        L.gdr_fwd_o.argtypes = [PP] + [_P] * 8 + [_P]
        L.gdr_fwd_h_o_supported.argtypes = [PP]
        L.gdr_fwd_h_o_supported.restype = ctypes.c_int
        L.gdr_chunk_fwd_fused.argtypes = [PP]
        L.gdr_chunk_fwd_fused.restype = ctypes.c_int
        L.gdr_fwd_h_o.argtypes = [PP] + [_P] * 11 + [_P]
        L.gdr_fused_recurrent_fwd.argtypes = [PP] + [_P] * 9 + [_P]
        L.gdr_simple_gla_fwd.argtypes = [PP] + [_P] * 8 + [_P, ctypes.c_size_t, _P]
        L.gdr_segmented_workspace_bytes.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
        L.gdr_segmented_workspace_layout.argtypes = [PP, ctypes.POINTER(GdrSegLayout)]
        L.gdr_chunk_fwd_segmented.argtypes = [PP] + [_P] * 11 + [_P, ctypes.c_size_t, _P]
        L.gdr_bwd_workspace_bytes.argtypes = [PP, ctypes.POINTER(ctypes.c_size_t)]
        L.gdr_bwd_workspace_layout.argtypes = [PP, ctypes.POINTER(GdrBwdLayout)]
        L.gdr_chunk_bwd.argtypes = [PP] + [_P] * 15 + [_P, ctypes.c_size_t, _P]
        L.gdr_bwd_intra.argtypes = [PP] + [_P] * 8 + [_P]
        L.gdr_bwd_dh.argtypes = [PP] + [_P] * 12 + [_P]
        L.gdr_bwd_dqkvg.argtypes = [PP] + [_P] * 17 + [_P]
        for name in ("gdr_check_problem", "gdr_validate_cu_seqlens", "gdr_fwd_workspace_bytes",
                     "gdr_fwd_workspace_layout", "gdr_chunk_fwd", "gdr_chunk_fwd_noalloc", "gdr_chunk_table",
                     "gdr_fwd_kkt_solve", "gdr_fwd_wy", "gdr_fwd_h", "gdr_fwd_o", "gdr_fwd_h_o",
                     "gdr_fused_recurrent_fwd", "gdr_fwd_kkt_wy", "gdr_segmented_workspace_bytes",
                     "gdr_segmented_workspace_layout", "gdr_chunk_fwd_segmented", "gdr_simple_gla_fwd",
                     "gdr_bwd_workspace_bytes", "gdr_bwd_workspace_layout", "gdr_chunk_bwd",
                     "gdr_bwd_intra", "gdr_bwd_dh", "gdr_bwd_dqkvg"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _raise(st: int):
    if st == 0:
        return
    msg = lib().gdr_status_string(st).decode()
    if st == 8:
        raise GdrError(st, f"{STATUS.get(st, st)}: {msg}")
    raise ValueError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return GDR_BF16
    if dt == torch.float32:
        return GDR_FP32
    return 99      # rejected by the library with GDR_ERR_DTYPE


def make_problem(q, v, g, *, chunk_size=64, cu_seqlens=None, use_qk_l2norm=False, scale=1.0,
                 N: Optional[int] = None, keep_states: bool = False, beta_logits: bool = False) -> GdrProblem:
    """Problem description from tensor shapes (no checks beyond the shapes).
    ``keep_states`` makes gdr_chunk_fwd leave h and v_new in its workspace
    (separate scan and output stages instead of the fused one)."""
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    if N is None:
        N = (len(cu_seqlens) - 1) if cu_seqlens is not None else B
    return GdrProblem(B=B, T=T, H=H, HV=HV, K=K, V=V, N=N, chunk_size=int(chunk_size),
                      gate_per_channel=int(g.dim() == 4), use_qk_l2norm=int(bool(use_qk_l2norm)),
                      dtype=_dtype_code(q.dtype), scale=float(scale), keep_states=int(bool(keep_states)),
                      beta_logits=int(bool(beta_logits)))


def check_problem(p: GdrProblem) -> None:
    _raise(lib().gdr_check_problem(ctypes.byref(p)))


def fwd_layout(p: GdrProblem) -> GdrFwdLayout:
    lay = GdrFwdLayout()
    _raise(lib().gdr_fwd_workspace_layout(ctypes.byref(p), ctypes.byref(lay)))
    return lay


def bwd_layout(p: GdrProblem) -> GdrBwdLayout:
    lay = GdrBwdLayout()
    _raise(lib().gdr_bwd_workspace_layout(ctypes.byref(p), ctypes.byref(lay)))
    return lay


def _need_gpu(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("gdr tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("gdr tensors must be contiguous")


def _expect(name, t, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def check_tensors(p: GdrProblem, q, k, v, g, beta, cu_seqlens=None, h0=None, validate_cu=True):
    """Host-side marshalling checks: every tensor has the shape the problem
    implies, and (optionally) cu_seqlens holds a valid table."""
    B, T, H, HV, K, V, N = p.B, p.T, p.H, p.HV, p.K, p.V, p.N
    _expect("q", q, (B, T, H, K))
    _expect("k", k, (B, T, H, K))
    _expect("v", v, (B, T, HV, V))
    _expect("g", g, (B, T, HV, K) if p.gate_per_channel else (B, T, HV))
    _expect("beta", beta, (B, T, HV))
    _expect("initial_state", h0, (N, HV, K, V))
    if cu_seqlens is not None:
        _expect("cu_seqlens", cu_seqlens, (N + 1,))
        if validate_cu:
            host = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
            st = lib().gdr_validate_cu_seqlens(ctypes.c_void_p(host.data_ptr()), N, T)
            if st != 0:
                raise ValueError(lib().gdr_status_string(st).decode())


def chunk_fwd(q, k, v, g, beta, *, scale: float = 1.0, chunk_size: int = 64, cu_seqlens=None,
              initial_state=None, output_final_state: bool = True,
              use_qk_l2norm_in_kernel: bool = False, workspace: Optional[torch.Tensor] = None,
              return_workspace: bool = False, out=None, validate_cu: bool = True,
              keep_states: Optional[bool] = None, beta_logits: bool = False):
    """Forward of the chunked gated delta rule.  Returns (o, ht) (ht None when
    not requested), plus the workspace tensor when ``return_workspace``.
    ``out=(o, ht)`` supplies the output tensors; ``validate_cu`` checks a host
    copy of cu_seqlens first (one small device-to-host copy).  ``keep_states``
    (default: ``return_workspace``) keeps h and v_new in the workspace;
    otherwise the fused scan + output stage runs where the shape allows it."""
    _need_gpu(q, k, v, g, beta, cu_seqlens, initial_state)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    for name, t in (("g", g), ("beta", beta), ("initial_state", initial_state)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if keep_states is None:
        keep_states = return_workspace
    p = make_problem(q, v, g, chunk_size=chunk_size, cu_seqlens=cu_seqlens,
                     use_qk_l2norm=use_qk_l2norm_in_kernel, scale=scale, keep_states=keep_states,
                     beta_logits=beta_logits)
    lay = fwd_layout(p)
    check_tensors(p, q, k, v, g, beta, cu_seqlens, initial_state, validate_cu)
    if out is not None:
        o, ht = out
        _need_gpu(o, ht)
        _expect("o", o, v.shape)
        _expect("ht", ht, (p.N, p.HV, p.K, p.V))
        if o.dtype != q.dtype or (ht is not None and ht.dtype != torch.float32):
            raise ValueError("o must match q's dtype and ht must be float32")
    else:
        o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
        ht = (torch.empty(p.N, p.HV, p.K, p.V, dtype=torch.float32, device=q.device)
              if output_final_state else None)
    if workspace is None or workspace.numel() < lay.total:
        workspace = torch.empty(max(lay.total, 256), dtype=torch.uint8, device=q.device)
    st = lib().gdr_chunk_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(cu_seqlens), _ptr(initial_state), _ptr(o), _ptr(ht),
                             _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(q.device))
    _raise(st)
    if return_workspace:
        return o, ht, workspace
    return o, ht


def chunk_fwd_noalloc(q, k, v, g, beta, *, out, scale: float = 1.0, chunk_size: int = 64, cu_seqlens=None,
                      initial_state=None, use_qk_l2norm_in_kernel: bool = False, beta_logits: bool = False):
    """The full forward through gdr_chunk_fwd_noalloc: no workspace, the
    library's fixed per-device scratch instead; ``out=(o, ht)`` are the
    caller's output tensors (ht may be None), so this call allocates nothing.
    Calls that overlap on one device race on the scratch."""
    _need_gpu(q, k, v, g, beta, cu_seqlens, initial_state)
    o, ht = out
    _need_gpu(o, ht)
    if k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise ValueError("q, k, v and o must share one dtype")
    for name, t in (("g", g), ("beta", beta), ("initial_state", initial_state), ("ht", ht)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    p = make_problem(q, v, g, chunk_size=chunk_size, cu_seqlens=cu_seqlens,
                     use_qk_l2norm=use_qk_l2norm_in_kernel, scale=scale, beta_logits=beta_logits)
    check_tensors(p, q, k, v, g, beta, cu_seqlens, initial_state, validate_cu=False)
    _expect("o", o, v.shape)
    _expect("ht", ht, (p.N, p.HV, p.K, p.V))
    _raise(lib().gdr_chunk_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(cu_seqlens), _ptr(initial_state), _ptr(o), _ptr(ht),
                                       _stream(q.device)))
    return o, ht


def stage_timing(enable: bool) -> None:
    """Turn the library's per-stage HIP-event timing on (clearing what was
    recorded) or off, for this thread."""
    _raise(lib().gdr_stage_timing(int(bool(enable))))


def stage_times(max_stages: int = 8192) -> list:
    """[(stage name, milliseconds)] of every full forward / backward call timed
    on this thread since stage_timing(True), in launch order (waits for the
    last recorded event)."""
    names = (ctypes.c_char_p * max_stages)()
    ms = (ctypes.c_float * max_stages)()
    n = lib().gdr_stage_times(names, ms, max_stages)
    if n < 0:
        raise GdrError(8, "stage timing: HIP error")
    return [(names[i].decode(), float(ms[i])) for i in range(n)]


def workspace_views(p: GdrProblem, ws: torch.Tensor, lay: Optional[GdrFwdLayout] = None) -> dict:
    """Typed views of the forward intermediates inside a workspace tensor (of
    the layout ``lay``, by default the one gdr_chunk_fwd uses for ``p``).  A
    region the layout gives no bytes has a None view: the compact layout of the
    scalar-gate fused stages has no Tm, h or v_new and keeps u in the input
    dtype; the per-channel fused forward has no Tm, h or v_new but aqk and qgs."""
    if lay is None:
        lay = fwd_layout(p)
    nt, C, HV, K, V = lay.nt_max, p.chunk_size, p.HV, p.K, p.V
    no_tm = nt > 0 and lay.Tm == lay.w
    no_states = nt > 0 and lay.h == lay.v_new
    pc_fused = nt > 0 and lay.qgs > lay.aqk
    compact = no_tm                        # the fused stages: u in the input dtype
    qg_tiles = max(1, (lay.total - lay.qgs) // max(1, nt * HV * C * K * (2 if p.dtype == GDR_BF16 else 4))) \
        if pc_fused else 0
    dt = torch.bfloat16 if p.dtype == GDR_BF16 else torch.float32
    es = 2 if p.dtype == GDR_BF16 else 4

    def view(off, shape, dtype, esize):
        n = 1
        for s in shape:
            n *= s
        return ws[off:off + n * esize].view(dtype).view(*shape)

    return dict(
        chunk_idx=view(lay.chunk_idx, (nt, 4), torch.int32, 4),
        chunk_off=view(lay.chunk_off, (p.N + 1,), torch.int32, 4),
        seq_order=view(lay.seq_order, (p.N,), torch.int32, 4),
        Tm=None if no_tm else view(lay.Tm, (nt, HV, C, C), dt, es),
        w=view(lay.w, (nt, HV, C, K), dt, es),
        # u as the separate WY stage writes it (fp32), and the same region as the
        # fused K1 + K2 stage writes it (input dtype)
        u=None if compact else view(lay.u, (nt, HV, V, C), torch.float32, 4),
        u_fused=view(lay.u, (nt, HV, V, C), dt, es),
        h=None if no_states else view(lay.h, (nt, HV, V, K), dt, es),
        v_new=None if no_states else view(lay.v_new, (nt, HV, V, C), dt, es),
        kscale=None if p.gate_per_channel else view(lay.kscale, (nt, HV, 3 * C + 4), torch.float32, 4),
        kt=view(lay.kt, (nt, HV, C, K), dt, es) if lay.dl > lay.kt else None,
        dl=view(lay.dl, (nt, HV, K), torch.float32, 4) if lay.aqk > lay.dl else None,
        aqk=view(lay.aqk, (nt, HV, C, C), torch.float32, 4) if pc_fused else None,
        # the gated queries: one tile in the input dtype, or a hi + lo pair
        qgs=view(lay.qgs, (nt, HV, qg_tiles, C, K), dt, es) if pc_fused else None,
    )


# ---- the forward's stages one by one (tensors allocated by the caller)

def chunk_table(p: GdrProblem, cu_seqlens, chunk_idx, chunk_off):
    _raise(lib().gdr_chunk_table(ctypes.byref(p), _ptr(cu_seqlens), _ptr(chunk_idx), _ptr(chunk_off),
                                 _stream(chunk_off.device)))


def fwd_kkt_solve(p, k, g, beta, chunk_idx, chunk_off, Tm, kscale=None):
    _raise(lib().gdr_fwd_kkt_solve(ctypes.byref(p), _ptr(k), _ptr(g), _ptr(beta), _ptr(chunk_idx),
                                   _ptr(chunk_off), _ptr(Tm), _ptr(kscale), _stream(k.device)))


def fwd_wy(p, k, v, g, beta, chunk_idx, chunk_off, Tm, w, u):
    _raise(lib().gdr_fwd_wy(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(chunk_idx),
                            _ptr(chunk_off), _ptr(Tm), _ptr(w), _ptr(u), _stream(k.device)))


def fwd_kkt_wy(p, k, v, g, beta, chunk_idx, chunk_off, w, u, kscale):
    """K1 + K2 fused (scalar gate): w, u and kscale without writing Tm."""
    _raise(lib().gdr_fwd_kkt_wy(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(chunk_idx),
                                _ptr(chunk_off), _ptr(w), _ptr(u), _ptr(kscale), _stream(k.device)))


def fwd_h(p, k, w, u, g, chunk_idx, chunk_off, h0, h, v_new, ht, kscale=None):
    _raise(lib().gdr_fwd_h(ctypes.byref(p), _ptr(k), _ptr(w), _ptr(u), _ptr(g), _ptr(kscale),
                           _ptr(chunk_idx), _ptr(chunk_off), _ptr(h0), _ptr(h), _ptr(v_new), _ptr(ht),
                           _stream(k.device)))


def fwd_o(p, q, k, v_new, h, g, chunk_idx, chunk_off, o):
    _raise(lib().gdr_fwd_o(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v_new), _ptr(h), _ptr(g),
                           _ptr(chunk_idx), _ptr(chunk_off), _ptr(o), _stream(q.device)))


def fwd_h_o_supported(p) -> bool:
    return bool(lib().gdr_fwd_h_o_supported(ctypes.byref(p)))


def chunk_fwd_fused(p) -> int:
    """Which fused scan + output stage gdr_chunk_fwd runs for ``p``: 1 with the
    fused K1 + K2 stage (scalar gate), 2 the per-channel one after separate K1
    and K2, 0 none (separate stages)."""
    return int(lib().gdr_chunk_fwd_fused(ctypes.byref(p)))


def fwd_h_o(p, q, k, w, u, g, kscale, chunk_idx, chunk_off, h0, o, ht):
    _raise(lib().gdr_fwd_h_o(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(w), _ptr(u), _ptr(g), _ptr(kscale),
                             _ptr(chunk_idx), _ptr(chunk_off), _ptr(h0), _ptr(o), _ptr(ht),
                             _stream(q.device)))


def fused_recurrent_fwd(q, k, v, g, beta, *, scale: float = 1.0, cu_seqlens=None, initial_state=None,
                        output_final_state: bool = True, use_qk_l2norm_in_kernel: bool = False,
                        out=None, validate_cu: bool = True, beta_logits: bool = False):
    """Token-by-token forward of the same operator (gdr_fused_recurrent_fwd):
    no chunk table and no workspace, for decoding and short sequences.
    Returns (o, ht) (ht None when not requested); ``out=(o, ht)`` supplies the
    output tensors."""
    _need_gpu(q, k, v, g, beta, cu_seqlens, initial_state)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    for name, t in (("g", g), ("beta", beta), ("initial_state", initial_state)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    p = make_problem(q, v, g, chunk_size=64, cu_seqlens=cu_seqlens,
                     use_qk_l2norm=use_qk_l2norm_in_kernel, scale=scale, beta_logits=beta_logits)
    check_tensors(p, q, k, v, g, beta, cu_seqlens, initial_state, validate_cu)
    if out is not None:
        o, ht = out
        _need_gpu(o, ht)
        _expect("o", o, v.shape)
        _expect("ht", ht, (p.N, p.HV, p.K, p.V))
        if o.dtype != q.dtype or (ht is not None and ht.dtype != torch.float32):
            raise ValueError("o must match q's dtype and ht must be float32")
    else:
        o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
        ht = (torch.empty(p.N, p.HV, p.K, p.V, dtype=torch.float32, device=q.device)
              if output_final_state else None)
    st = lib().gdr_fused_recurrent_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(cu_seqlens), _ptr(initial_state), _ptr(o), _ptr(ht),
                                       _stream(q.device))
    _raise(st)
    return o, ht


def simple_gla_fwd(q, k, v, g, *, scale: float = 1.0, chunk_size: int = 64, cu_seqlens=None,
                   initial_state=None, output_final_state: bool = True, use_qk_l2norm_in_kernel: bool = False,
                   workspace: Optional[torch.Tensor] = None, validate_cu: bool = True):
    """Simple GLA forward (gdr_simple_gla_fwd): S_t = exp(g_t) S_{t-1} + k_t v_t^T,
    o_t = scale S_t^T q_t, through the same chunked stages.  Returns (o, ht)."""
    _need_gpu(q, k, v, g, cu_seqlens, initial_state)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    for name, t in (("g", g), ("initial_state", initial_state)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    p = make_problem(q, v, g, chunk_size=chunk_size, cu_seqlens=cu_seqlens,
                     use_qk_l2norm=use_qk_l2norm_in_kernel, scale=scale)
    lay = fwd_layout(p)
    check_tensors(p, q, k, v, g, g if g.dim() == 3 else g[..., 0], cu_seqlens, initial_state, validate_cu)
    o = torch.empty(v.shape, dtype=q.dtype, device=q.device)
    ht = (torch.empty(p.N, p.HV, p.K, p.V, dtype=torch.float32, device=q.device)
          if output_final_state else None)
    if workspace is None or workspace.numel() < lay.total:
        workspace = torch.empty(max(lay.total, 256), dtype=torch.uint8, device=q.device)
    st = lib().gdr_simple_gla_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(cu_seqlens),
                                  _ptr(initial_state), _ptr(o), _ptr(ht), _ptr(workspace),
                                  ctypes.c_size_t(workspace.numel()), _stream(q.device))
    _raise(st)
    return o, ht


def seg_layout(p: GdrProblem) -> GdrSegLayout:
    lay = GdrSegLayout()
    _raise(lib().gdr_segmented_workspace_layout(ctypes.byref(p), ctypes.byref(lay)))
    return lay


def chunk_fwd_segmented(q, k, v, g, beta, cu_seqlens, *, scale: float = 1.0, chunk_size: int = 64,
                        initial_state=None, use_qk_l2norm_in_kernel: bool = False,
                        want_transitions: bool = False, validate_cu: bool = True, beta_logits: bool = False):
    """Forward of ONE sequence (q, k [1,T,H,K] ...) split into the segments
    ``cu_seqlens`` bounds, run as the context-parallel scheme on one device
    (gdr_chunk_fwd_segmented): every segment's local end state and transition,
    the merge of the entering states, a re-run of every segment.  Returns
    (o, ht, seg_states [N+1,HV,K,V], transitions [N,HV,K,K] or None);
    ``initial_state`` is the sequence's [1,HV,K,V] initial state."""
    _need_gpu(q, k, v, g, beta, cu_seqlens, initial_state)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    for name, t in (("g", g), ("beta", beta), ("initial_state", initial_state)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    if cu_seqlens is None or cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens (int32 segment bounds) is required")
    p = make_problem(q, v, g, chunk_size=chunk_size, cu_seqlens=cu_seqlens,
                     use_qk_l2norm=use_qk_l2norm_in_kernel, scale=scale, beta_logits=beta_logits)
    lay = seg_layout(p)
    check_tensors(p, q, k, v, g, beta, cu_seqlens, None, validate_cu)
    _expect("initial_state", initial_state, (1, p.HV, p.K, p.V))
    dev = q.device
    o = torch.empty(v.shape, dtype=q.dtype, device=dev)
    ht = torch.empty(1, p.HV, p.K, p.V, dtype=torch.float32, device=dev)
    states = torch.empty(p.N + 1, p.HV, p.K, p.V, dtype=torch.float32, device=dev)
    trans = (torch.empty(p.N, p.HV, p.K, p.K, dtype=torch.float32, device=dev)
             if want_transitions else None)
    ws = torch.empty(max(lay.total, 256), dtype=torch.uint8, device=dev)
    st = lib().gdr_chunk_fwd_segmented(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(cu_seqlens), _ptr(initial_state), _ptr(o), _ptr(ht),
                                       _ptr(states), _ptr(trans), _ptr(ws), ctypes.c_size_t(ws.numel()),
                                       _stream(dev))
    _raise(st)
    return o, ht, states, trans


# ---- backward

def chunk_bwd(q, k, v, g, beta, do, dht=None, *, scale: float = 1.0, chunk_size: int = 64,
              cu_seqlens=None, initial_state=None, use_qk_l2norm_in_kernel: bool = False,
              workspace: Optional[torch.Tensor] = None, return_workspace: bool = False,
              out=None, want_dh0: bool = True, validate_cu: bool = True, reuse_forward: bool = False,
              beta_logits: bool = False):
    """Backward of the chunked gated delta rule: gradients of
    sum(o * do) + sum(ht * dht).  Returns (dq, dk, dv, dg, dbeta, dh0) (dh0 None
    when not wanted), plus the workspace when ``return_workspace``.  ``out``
    supplies the six output tensors.  ``reuse_forward`` skips the recompute of
    the forward intermediates: ``workspace`` must be the backward-sized
    workspace a ``chunk_fwd(..., keep_states=True, workspace=workspace)`` call
    on the same inputs has just filled."""
    _need_gpu(q, k, v, g, beta, do, dht, cu_seqlens, initial_state)
    if k.dtype != q.dtype or v.dtype != q.dtype or do.dtype != q.dtype:
        raise ValueError("q, k, v and do must share one dtype")
    for name, t in (("g", g), ("beta", beta), ("initial_state", initial_state), ("dht", dht)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    p = make_problem(q, v, g, chunk_size=chunk_size, cu_seqlens=cu_seqlens,
                     use_qk_l2norm=use_qk_l2norm_in_kernel, scale=scale, keep_states=reuse_forward,
                     beta_logits=beta_logits)
    lay = bwd_layout(p)
    if reuse_forward and (workspace is None or workspace.numel() < lay.total):
        raise ValueError("reuse_forward needs the backward-sized workspace the forward filled")
    check_tensors(p, q, k, v, g, beta, cu_seqlens, initial_state, validate_cu)
    _expect("do", do, v.shape)
    _expect("dht", dht, (p.N, p.HV, p.K, p.V))
    if out is not None:
        dq, dk, dv, dg, dbeta, dh0 = out
        _need_gpu(dq, dk, dv, dg, dbeta, dh0)
        for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v), ("dg", dg, g), ("dbeta", dbeta, beta)):
            _expect(name, t, ref.shape)
            if t.dtype != ref.dtype:
                raise ValueError(f"{name} must have dtype {ref.dtype}")
        _expect("dh0", dh0, (p.N, p.HV, p.K, p.V))
    else:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dg, dbeta = torch.empty_like(g), torch.empty_like(beta)
        dh0 = (torch.empty(p.N, p.HV, p.K, p.V, dtype=torch.float32, device=q.device)
               if want_dh0 else None)
    if workspace is None or workspace.numel() < lay.total:
        workspace = torch.empty(max(lay.total, 256), dtype=torch.uint8, device=q.device)
    st = lib().gdr_chunk_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(cu_seqlens), _ptr(initial_state), _ptr(do), _ptr(dht), _ptr(dq),
                             _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(workspace),
                             ctypes.c_size_t(workspace.numel()), _stream(q.device))
    _raise(st)
    res = (dq, dk, dv, dg, dbeta, dh0)
    if return_workspace:
        return res + (workspace,)
    return res


def bwd_workspace_views(p: GdrProblem, ws: torch.Tensor) -> dict:
    """Typed views of the backward's intermediates (forward ones included)."""
    lay = bwd_layout(p)
    # the chunk size the backward runs at (a per-channel gate, and fp32 with
    # K = 128, run chunk 64 problems at 32)
    pe = GdrProblem.from_buffer_copy(p)
    pe.chunk_size = int(lay.chunk_size)
    views = workspace_views(pe, ws, lay.fwd)
    nt, C, HV, K, V = lay.fwd.nt_max, pe.chunk_size, p.HV, p.K, p.V
    dt = torch.bfloat16 if p.dtype == GDR_BF16 else torch.float32
    es = 2 if p.dtype == GDR_BF16 else 4

    def view(off, shape, dtype, esize):
        n = 1
        for s_ in shape:
            n *= s_
        return ws[off:off + n * esize].view(dtype).view(*shape)

    views.update(
        de_local=view(lay.de_local, (nt, HV, V, C), dt, es),
        qscale=view(lay.qscale, (nt, HV, C), torch.float32, 4),
        dh=view(lay.dh, (nt, HV, V, K), torch.float32, 4),   # fp32
    )
    if p.gate_per_channel:
        views.update(kt=view(lay.kt, (nt, HV, C, K), dt, es), qg=view(lay.qg, (nt, HV, C, K), dt, es),
                     dl=view(lay.dl, (nt, HV, K), torch.float32, 4))
    return views


# ---- the backward's stages one by one

def bwd_intra(p, q, k, g, do, chunk_idx, chunk_off, de_local, qscale):
    _raise(lib().gdr_bwd_intra(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(g), _ptr(do), _ptr(chunk_idx),
                               _ptr(chunk_off), _ptr(de_local), _ptr(qscale), _stream(q.device)))


def bwd_dh(p, q, k, w, do, de_local, qscale, kscale, chunk_idx, chunk_off, dht, dh, dh0):
    _raise(lib().gdr_bwd_dh(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(w), _ptr(do), _ptr(de_local),
                            _ptr(qscale), _ptr(kscale), _ptr(chunk_idx), _ptr(chunk_off), _ptr(dht),
                            _ptr(dh), _ptr(dh0), _stream(q.device)))


def bwd_dqkvg(p, q, k, v, g, beta, do, Tm, h, v_new, dh, chunk_idx, chunk_off, dq, dk, dv, dg, dbeta):
    _raise(lib().gdr_bwd_dqkvg(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(do),
                               _ptr(Tm), _ptr(h), _ptr(v_new), _ptr(dh), _ptr(chunk_idx), _ptr(chunk_off),
                               _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _stream(q.device)))
