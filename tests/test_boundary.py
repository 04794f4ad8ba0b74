"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/gdr.h declares, and rejects bad arguments on the host before
any launch (the error convention of the coverage-matrix page, section 3:
chunk_size 16 raises "chunk_size must be either 32 or 64")."""
import ctypes
import os
import re

import numpy as np
import pytest

import chunked_gated_delta_06_amd as gdr


def header_functions():
    src = open(gdr.HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z0-9_]+)\s*\(", src)))


def problem(**kw):
    base = dict(B=2, T=100, H=2, HV=4, K=64, V=128, N=2, chunk_size=64, gate_per_channel=0,
                use_qk_l2norm=1, dtype=gdr.GDR_BF16, scale=1.0)
    base.update(kw)
    return gdr.GdrProblem(**base)


def test_exports_every_declared_function():
    L = gdr.lib()
    names = header_functions()
    assert "gdr_chunk_fwd" in names and "gdr_fwd_h" in names
    assert "gdr_chunk_bwd" in names and "gdr_bwd_dqkvg" in names
    for n in names:
        assert hasattr(L, n), n
    assert L.gdr_abi_version() == 6


def test_status_strings():
    L = gdr.lib()
    assert L.gdr_status_string(2).decode() == "chunk_size must be either 32 or 64"
    for s in range(12):
        assert L.gdr_status_string(s)
    assert "backward supports" in L.gdr_status_string(10).decode()


@pytest.mark.parametrize("kw,msg", [
    (dict(chunk_size=16), "chunk_size must be either 32 or 64"),
    (dict(chunk_size=128), "chunk_size must be either 32 or 64"),
    (dict(HV=3), "unsupported shape"),
    (dict(K=300), "unsupported shape"),
    (dict(V=257), "unsupported shape"),
    (dict(H=0), "unsupported shape"),
    (dict(T=-1), "unsupported shape"),
    (dict(dtype=7), "dtype"),
    (dict(N=3), "cu_seqlens requires B == 1"),
    (dict(dtype=gdr.GDR_FP32, gate_per_channel=1, K=256), "unsupported shape"),
])
def test_check_problem_rejects(kw, msg):
    with pytest.raises(ValueError, match=msg):
        gdr.check_problem(problem(**kw))


def test_check_problem_accepts():
    gdr.check_problem(problem())
    gdr.check_problem(problem(B=1, N=5, T=1000))         # varlen
    gdr.check_problem(problem(T=0))                        # empty batch
    gdr.check_problem(problem(dtype=gdr.GDR_FP32, gate_per_channel=1, K=256, chunk_size=32))


def test_validate_cu_seqlens():
    L = gdr.lib()

    def val(arr, N, T):
        a = np.asarray(arr, dtype=np.int32)
        return L.gdr_validate_cu_seqlens(a.ctypes.data_as(ctypes.c_void_p), N, T)

    assert val([0, 5, 5, 9], 3, 9) == 0
    assert val([1, 5, 9], 2, 9) == 9
    assert val([0, 5, 4, 9], 3, 9) == 9
    assert val([0, 5, 8], 2, 9) == 9
    assert L.gdr_validate_cu_seqlens(None, 2, 9) == 1


def test_workspace_layout():
    # the separate stages (keep_states): every intermediate has its region
    p = problem(B=4, T=4096, H=16, HV=16, K=128, V=128, N=4, keep_states=1)
    lay = gdr.fwd_layout(p)
    assert lay.nt_max == 4 * 64
    offs = [lay.chunk_idx, lay.chunk_off, lay.Tm, lay.w, lay.u, lay.h, lay.v_new, lay.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    nt, C, HV, K, V = 256, 64, 16, 128, 128
    assert lay.w - lay.Tm >= nt * HV * C * C * 2
    assert lay.h - lay.u >= nt * HV * V * C * 4      # u in fp32 (the separate WY stage's)
    assert lay.total - lay.v_new >= nt * HV * V * C * 2
    blay = gdr.bwd_layout(p)
    assert blay.total - blay.dh >= nt * HV * V * K * 4   # dh in fp32
    # the fused stages (the default): no Tm, h or v_new, u in the input dtype
    pf = problem(B=4, T=4096, H=16, HV=16, K=128, V=128, N=4)
    f = gdr.fwd_layout(pf)
    assert f.Tm == f.w and f.h == f.v_new == f.kscale
    assert f.u - f.w >= nt * HV * C * K * 2 and f.kscale - f.u >= nt * HV * V * C * 2
    assert f.kscale - f.u < nt * HV * V * C * 4
    assert f.total < lay.total // 2
    # a shape without the fused scan + output stage (per-channel gate) keeps the full layout,
    # plus the WY stage's gated keys and decay for the state scan
    pc = gdr.fwd_layout(problem(B=4, T=4096, H=16, HV=16, K=128, V=128, N=4, gate_per_channel=1))
    assert pc.w - pc.Tm >= nt * HV * C * C * 2 and pc.v_new > pc.h
    assert pc.dl - pc.kt >= nt * HV * C * K * 2 and pc.total - pc.dl >= nt * HV * K * 4
    assert lay.kt == lay.dl == lay.total and f.kt == f.dl == f.total
    # per-channel gate, bf16, chunk 32, K <= 128: the per-channel fused scan + output, so no
    # Tm / h / v_new, and the fused K1 + K2's aqk and gated queries for it
    p32 = problem(B=4, T=4096, H=16, HV=16, K=128, V=128, N=4, gate_per_channel=1, chunk_size=32)
    assert gdr.lib().gdr_chunk_fwd_fused(ctypes.byref(p32)) == 2
    q = gdr.fwd_layout(p32)
    n32 = 4 * 128
    offs = [q.chunk_idx, q.Tm, q.w, q.u, q.h, q.kt, q.dl, q.aqk, q.qgs, q.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert q.h == q.v_new == q.kscale == q.kt and q.Tm == q.w
    assert n32 * HV * V * 32 * 2 <= q.h - q.u < n32 * HV * V * 32 * 4     # u in the input dtype
    assert q.dl - q.kt >= n32 * HV * 32 * K * 2 and q.aqk - q.dl >= n32 * HV * K * 4
    assert q.qgs - q.aqk >= n32 * HV * 32 * 32 * 4 and q.total - q.qgs >= n32 * HV * 32 * K * 2
    for kw in (dict(keep_states=1), dict(dtype=gdr.GDR_FP32), dict(K=256), dict(chunk_size=64)):
        other = problem(**{**dict(B=4, T=4096, H=16, HV=16, K=128, V=128, N=4, gate_per_channel=1,
                                  chunk_size=32), **kw})
        assert gdr.lib().gdr_chunk_fwd_fused(ctypes.byref(other)) == 0, kw
        o = gdr.fwd_layout(other)
        assert o.v_new > o.h and o.w > o.Tm, kw
        # the kept-states forward of the same shape runs the fused stages too
        # (storing Tm, h and v_new as well), so it keeps the aqk / qgs regions
        assert (o.qgs > o.aqk) == (kw == dict(keep_states=1)), kw
    # the backward keeps its own gated rows: its forward part reserves none
    bl = gdr.bwd_layout(problem(B=4, T=4096, H=16, HV=16, K=128, V=128, N=4, gate_per_channel=1, chunk_size=32))
    assert bl.fwd.kt == bl.fwd.dl and bl.dl > bl.kt
    # varlen bound floor(T / C) + N
    pv = problem(B=1, T=25344, H=16, HV=32, K=128, V=128, N=24)
    assert gdr.fwd_layout(pv).nt_max == 25344 // 64 + 24


def test_fwd_rejects_before_launch():
    """Null, misaligned and undersized arguments come back as error codes
    without touching the device (these calls run on the CPU host)."""
    L = gdr.lib()
    p = problem()
    P = ctypes.c_void_p
    args = [P(0x1000)] * 9
    # null q
    st = L.gdr_chunk_fwd(ctypes.byref(p), None, *args[1:5], None, None, P(0x1000), None,
                         P(0x1000), ctypes.c_size_t(1 << 40), None)
    assert st == 1
    # misaligned k
    st = L.gdr_chunk_fwd(ctypes.byref(p), P(0x1000), P(0x1008), *args[2:5], None, None, P(0x1000),
                         None, P(0x1000), ctypes.c_size_t(1 << 40), None)
    assert st == 6
    # workspace too small
    st = L.gdr_chunk_fwd(ctypes.byref(p), *args[:5], None, None, P(0x1000), None, P(0x1000),
                         ctypes.c_size_t(16), None)
    assert st == 7
    # bad chunk size
    p16 = problem(chunk_size=16)
    st = L.gdr_chunk_fwd(ctypes.byref(p16), *args[:5], None, None, P(0x1000), None, P(0x1000),
                         ctypes.c_size_t(1 << 40), None)
    assert st == 2
    # cu_seqlens with B != 1
    st = L.gdr_chunk_fwd(ctypes.byref(p), *args[:5], P(0x1000), None, P(0x1000), None, P(0x1000),
                         ctypes.c_size_t(1 << 40), None)
    assert st == 4


def test_noalloc_forward_rejects_before_launch():
    """gdr_chunk_fwd_noalloc checks its arguments and the scratch limit on the
    host before it touches the device (these calls run on the CPU host)."""
    L = gdr.lib()
    P = ctypes.c_void_p
    a = [P(0x1000)] * 5
    p = problem()
    assert L.gdr_chunk_fwd_noalloc(ctypes.byref(p), None, *a[1:5], None, None, P(0x1000), None, None) == 1
    assert L.gdr_chunk_fwd_noalloc(ctypes.byref(p), P(0x1000), P(0x1008), *a[2:5], None, None, P(0x1000),
                                   None, None) == 6
    assert L.gdr_chunk_fwd_noalloc(ctypes.byref(problem(chunk_size=16)), *a, None, None, P(0x1000), None,
                                   None) == 2
    # 32768 tokens x 32 heads at K = V = 128: w, u and the token factors exceed the scratch
    big = problem(B=1, T=32768, H=32, HV=32, K=128, V=128, N=1)
    assert L.gdr_chunk_fwd_noalloc(ctypes.byref(big), *a, None, None, P(0x1000), None, None) == 11
    assert "fixed scratch" in L.gdr_status_string(11).decode()


def test_fused_stage_support_and_host_rejections():
    """Which shapes have the fused scan + output stage, and its host-side
    errors (no call here reaches a launch)."""
    L = gdr.lib()
    sup = lambda **kw: L.gdr_fwd_h_o_supported(ctypes.byref(problem(**kw)))
    assert sup(K=128, V=128) == 1                       # the dense bf16 workload's shape
    assert sup(K=64, V=256, chunk_size=32) == 1
    assert sup(K=64, dtype=gdr.GDR_FP32) == 1
    assert sup(K=128, gate_per_channel=1) == 0           # per-channel gate: separate stages
    assert sup(K=256) == 0
    assert sup(K=128, dtype=gdr.GDR_FP32) == 0          # staged tiles exceed LDS
    assert sup(chunk_size=16) == 0
    fused = lambda **kw: L.gdr_chunk_fwd_fused(ctypes.byref(problem(**kw)))
    assert fused(B=4, N=4, HV=16, H=16, K=128, V=128) == 1     # 4 * 16 * 128 / 32 = 256 tiles
    assert fused(B=4, N=4, HV=16, H=16, K=128, V=128, keep_states=1) == 0
    assert fused(B=1, N=1, HV=32, H=32, K=128, V=128) == 1     # 16-column workgroups
    assert fused(B=4, N=4, HV=16, H=16, K=256, V=128) == 0
    assert fused(B=4, N=4, HV=16, H=16, K=128, V=128, gate_per_channel=1, chunk_size=32) == 2
    assert fused(B=4, N=4, HV=16, H=16, K=128, V=128, gate_per_channel=1) == 0   # chunk 64
    P = ctypes.c_void_p
    args = [P(0x1000)] * 11
    p = problem()
    assert L.gdr_fwd_h_o(ctypes.byref(p), None, *args[1:], None) == 1       # null q
    assert L.gdr_fwd_h_o(ctypes.byref(p), *args[:5], None, *args[6:], None) == 1   # null kscale
    assert L.gdr_fwd_h_o(ctypes.byref(p), P(0x1008), *args[1:], None) == 6  # misaligned q
    pc = problem(gate_per_channel=1)
    assert L.gdr_fwd_h_o(ctypes.byref(pc), *args, None) == 10
    pk = problem(K=256)
    assert L.gdr_fwd_h_o(ctypes.byref(pk), *args, None) == 10


def test_python_wrapper_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 64, 1, 32, dtype=torch.bfloat16)
    g = torch.zeros(1, 64, 1)
    with pytest.raises(ValueError, match="GPU"):
        gdr.chunk_fwd(x, x, x, g, g)


@pytest.mark.parametrize("kw,ok", [
    (dict(), True),
    (dict(K=128, V=256, chunk_size=32), True),
    (dict(dtype=gdr.GDR_FP32, K=128, chunk_size=32), True),
    (dict(dtype=gdr.GDR_FP32, K=64, chunk_size=64), True),
    (dict(gate_per_channel=1), True),                            # per-channel: runs at chunk 32 inside
    (dict(gate_per_channel=1, chunk_size=32, K=128, V=256), True),
    (dict(gate_per_channel=1, keep_states=1), False),            # chunk 64 kept states cannot switch
    (dict(K=256), False),
    (dict(dtype=gdr.GDR_FP32, K=128, chunk_size=64), True),     # runs at chunk 32 inside
    (dict(dtype=gdr.GDR_FP32, K=128, chunk_size=64, keep_states=1), False),
])
def test_bwd_supported_shapes(kw, ok):
    p = problem(**kw)
    gdr.check_problem(p)                 # every case is a valid forward problem
    if ok:
        lay = gdr.bwd_layout(p)
        assert lay.total > 0
    else:
        with pytest.raises(ValueError, match="backward supports"):
            gdr.bwd_layout(p)


def test_bwd_layout_reports_the_chunk_size_it_runs_at():
    assert gdr.bwd_layout(problem()).chunk_size == 64
    assert gdr.bwd_layout(problem(gate_per_channel=1)).chunk_size == 32
    assert gdr.bwd_layout(problem(dtype=gdr.GDR_FP32, K=128)).chunk_size == 32
    assert gdr.bwd_layout(problem(gate_per_channel=1, chunk_size=32)).chunk_size == 32


def test_bwd_workspace_layout():
    p = problem(B=1, T=65536, H=32, HV=32, K=128, V=128, N=1)
    lay = gdr.bwd_layout(p)
    # the backward's leading part is the keep-states forward's layout
    f = gdr.fwd_layout(problem(B=1, T=65536, H=32, HV=32, K=128, V=128, N=1, keep_states=1))
    assert lay.fwd.total == f.total and lay.fwd.h == f.h
    nt, C, HV, K, V = 1024, 64, 32, 128, 128
    assert lay.fwd.nt_max == nt
    offs = [lay.fwd.total, lay.de_local, lay.qscale, lay.dh, lay.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.qscale - lay.de_local >= nt * HV * V * C * 2
    assert lay.dh - lay.qscale >= nt * HV * C * 4
    assert lay.total - lay.dh >= nt * HV * V * K * 2
    size = ctypes.c_size_t(0)
    assert gdr.lib().gdr_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(size)) == 0
    assert size.value == lay.total


def test_bwd_rejects_before_launch():
    """Backward argument errors come back as codes before any launch."""
    L = gdr.lib()
    p = problem()
    P = ctypes.c_void_p
    a = P(0x1000)
    big = ctypes.c_size_t(1 << 40)
    # q, k, v, g, beta, cu, h0, d_o, dht, dq, dk, dv, dg, dbeta, dh0, ws
    # (every call below fails a host check, so nothing is launched even where a
    # GPU is present: the fake addresses are never dereferenced)
    base = [a, a, a, a, a, None, None, a, None, a, a, a, a, a, None]
    args = list(base)
    args[7] = None                       # null d_o
    assert L.gdr_chunk_bwd(ctypes.byref(p), *args, a, big, None) == 1
    args = list(base)
    args[12] = P(0x1004)                 # misaligned dg
    assert L.gdr_chunk_bwd(ctypes.byref(p), *args, a, big, None) == 6
    assert L.gdr_chunk_bwd(ctypes.byref(p), *base, a, ctypes.c_size_t(64), None) == 7
    assert L.gdr_chunk_bwd(ctypes.byref(p), *base, None, big, None) == 7
    ppc = problem(K=256)                       # no backward instantiation: refused on the host
    assert L.gdr_chunk_bwd(ctypes.byref(ppc), *base, a, big, None) == 10
    p16 = problem(chunk_size=16)
    assert L.gdr_chunk_bwd(ctypes.byref(p16), *base, a, big, None) == 2


def test_bwd_wrapper_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 64, 1, 32, dtype=torch.bfloat16)
    g = torch.zeros(1, 64, 1)
    with pytest.raises(ValueError, match="GPU"):
        gdr.chunk_bwd(x, x, x, g, g, x)


def test_fused_recurrent_rejects_before_launch():
    """The token-by-token forward: host-side errors, and chunk_size is not read
    (no call here reaches a launch)."""
    L = gdr.lib()
    P = ctypes.c_void_p
    A = P(0x1000)
    p = problem()
    # null q
    assert L.gdr_fused_recurrent_fwd(ctypes.byref(p), None, A, A, A, A, None, None, A, None, None) == 1
    # misaligned v
    assert L.gdr_fused_recurrent_fwd(ctypes.byref(p), A, A, P(0x1004), A, A, None, None, A, None, None) == 6
    # cu_seqlens with B != 1
    assert L.gdr_fused_recurrent_fwd(ctypes.byref(p), A, A, A, A, A, A, None, A, None, None) == 4
    # shapes and dtype
    for kw, st in ((dict(HV=3), 3), (dict(K=96), 3), (dict(dtype=7), 5), (dict(N=3), 4)):
        assert L.gdr_fused_recurrent_fwd(ctypes.byref(problem(**kw)), A, A, A, A, A, None, None, A,
                                         None, None) == st, kw
    # an empty batch without a final state launches nothing; chunk_size is not read
    for cs in (0, 16, 64):
        assert L.gdr_fused_recurrent_fwd(ctypes.byref(problem(T=0, chunk_size=cs)), None, None, None,
                                         None, None, None, None, None, None, None) == 0


def test_fused_recurrent_wrapper_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 8, 1, 32, dtype=torch.bfloat16)
    g = torch.zeros(1, 8, 1)
    with pytest.raises(ValueError, match="GPU"):
        gdr.fused_recurrent_fwd(x, x, x, g, g)


def test_segmented_rejects_before_launch():
    """The segment hand-off forward needs cu_seqlens and a large enough
    workspace; errors come back before any launch."""
    L = gdr.lib()
    P = ctypes.c_void_p
    A = P(0x1000)
    p = problem(B=1, N=3, T=300)
    lay = gdr.seg_layout(p)
    assert lay.total > lay.fwd.total and lay.s_in > lay.trans > lay.s_ext
    # no cu_seqlens
    assert L.gdr_chunk_fwd_segmented(ctypes.byref(p), A, A, A, A, A, None, None, A, None, None, None, A,
                                     ctypes.c_size_t(1 << 40), None) == 1
    # workspace too small
    assert L.gdr_chunk_fwd_segmented(ctypes.byref(p), A, A, A, A, A, A, None, A, None, None, None, A,
                                     ctypes.c_size_t(lay.total - 1), None) == 7
    # chunk size and a dense batch (B != 1 with cu_seqlens)
    assert L.gdr_chunk_fwd_segmented(ctypes.byref(problem(B=1, N=3, T=300, chunk_size=16)), A, A, A, A, A, A,
                                     None, A, None, None, None, A, ctypes.c_size_t(1 << 40), None) == 2
    assert L.gdr_chunk_fwd_segmented(ctypes.byref(problem()), A, A, A, A, A, A, None, A, None, None, None, A,
                                     ctypes.c_size_t(1 << 40), None) == 4


def test_simple_gla_rejects_before_launch():
    L = gdr.lib()
    P = ctypes.c_void_p
    A = P(0x1000)
    big = ctypes.c_size_t(1 << 40)
    assert L.gdr_simple_gla_fwd(ctypes.byref(problem(gate_per_channel=1)), A, A, A, A, None, None, A, None, A,
                                big, None) == 10
    assert L.gdr_simple_gla_fwd(ctypes.byref(problem()), None, A, A, A, None, None, A, None, A, big, None) == 1
    assert L.gdr_simple_gla_fwd(ctypes.byref(problem()), A, A, A, A, None, None, A, None, A,
                                ctypes.c_size_t(16), None) == 7
    assert L.gdr_simple_gla_fwd(ctypes.byref(problem(chunk_size=16)), A, A, A, A, None, None, A, None, A, big,
                                None) == 2


def test_padded_head_dims():
    """Head dims without an instantiation (the coverage-matrix page's D = 60)
    are taken by the full forward / backward through zero padding: the problem
    check and the workspace sizes accept them (the workspace grows by the
    padded copies); a single stage, the token-by-token forward and the
    segmented / simple GLA paths still reject them."""
    L = gdr.lib()
    P = ctypes.c_void_p
    A = P(0x1000)
    p60 = problem(K=60, V=60)
    gdr.check_problem(p60)
    lay = gdr.fwd_layout(p60)
    lay64 = gdr.fwd_layout(problem(K=64, V=64))
    assert lay.total > lay64.total and lay.w == lay64.w
    assert gdr.bwd_layout(p60).total > gdr.bwd_layout(problem(K=64, V=64)).total
    assert L.gdr_fwd_kkt_solve(ctypes.byref(p60), A, A, A, A, A, A, A, None) == 3
    assert L.gdr_fused_recurrent_fwd(ctypes.byref(p60), A, A, A, A, A, None, None, A, None, None) == 3
    assert L.gdr_simple_gla_fwd(ctypes.byref(p60), A, A, A, A, None, None, A, None, A, ctypes.c_size_t(1 << 40),
                                None) == 3
    # the full forward checks the workspace against the padded size
    st = L.gdr_chunk_fwd(ctypes.byref(p60), A, A, A, A, A, None, None, A, None, A,
                         ctypes.c_size_t(lay64.total), None)
    assert st == 7
