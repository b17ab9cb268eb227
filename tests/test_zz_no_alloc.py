"""The split-row entry point that allocates nothing (fused_ar_rmsnorm_split_static), called through
the C ABI: the same bits as fused_ar_rmsnorm_split with a caller's workspace, and the oracle's
result, on calls in a row that share the static scratch (the second smaller than the first, so
the scratch still holds the first call's values where the second does not write)."""
import ctypes

import numpy as np
import pytest
import torch

import all_reduce_residual_way_amd as fa
import oracle
from all_reduce_residual_way_amd import synth
from ulp import ulp_diff

pytestmark = pytest.mark.gpu

VP = ctypes.c_void_p


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def call_both(lib, p, splits):
    """The static-scratch call and the workspace call on the same problem, through the C ABI."""
    ins = [dev(x) for x in p.inputs]
    res, w = dev(p.residual), dev(p.weight)
    arr = (VP * p.n)(*[x.data_ptr() for x in ins])
    outs = {}
    stream = torch.cuda.current_stream().cuda_stream
    ro, out = torch.empty_like(res), torch.empty_like(res)
    rc = lib.fused_ar_rmsnorm_split_static(arr, p.n, res.data_ptr(), w.data_ptr(), p.eps, p.m,
                                           p.hidden, ro.data_ptr(), out.data_ptr(), splits, stream)
    assert rc == fa.OK, fa.strerror(rc)
    outs["static"] = (ro, out)
    need = lib.fused_ar_split_workspace_bytes(p.m, p.hidden, splits)
    ws = torch.empty(need // 4, dtype=torch.float32, device="cuda")
    ro2, out2 = torch.empty_like(res), torch.empty_like(res)
    rc = lib.fused_ar_rmsnorm_split(arr, p.n, res.data_ptr(), w.data_ptr(), p.eps, p.m, p.hidden,
                                    ro2.data_ptr(), out2.data_ptr(), splits, ws.data_ptr(), need,
                                    stream)
    assert rc == fa.OK, fa.strerror(rc)
    outs["workspace"] = (ro2, out2)
    torch.cuda.synchronize()
    return {k: (host(a), host(b)) for k, (a, b) in outs.items()}


def test_static_scratch_matches_the_workspace_form_on_calls_in_a_row():
    lib = fa.library()
    # the first call fills the whole scratch (1024 rows x 64 slices), the second uses 20 slots
    cases = [(2, 1024, 8192, 64, 31), (8, 5, 7168, 0, 32), (8, 3, 32768, 0, 33)]
    assert 1024 * 64 == fa.STATIC_SCRATCH_FLOATS
    for n, m, hidden, splits, seed in cases:
        print(f"[gpu case] static-scratch split rows n={n} m={m} hidden={hidden} splits={splits}",
              flush=True)
        p = synth.make_problem(n, m, hidden, seed=seed, dist="stress" if seed == 32 else "normal",
                               name="static scratch")
        got = call_both(lib, p, splits)
        assert np.array_equal(got["static"][0], got["workspace"][0])
        assert np.array_equal(got["static"][1], got["workspace"][1])
        want_ro, want_out = oracle.fused(p.inputs, p.residual, p.weight, p.eps)
        assert np.array_equal(got["static"][0], want_ro)
        assert ulp_diff(got["static"][1], want_out).max() <= 1


def test_static_scratch_rejects_calls_beyond_it():
    lib = fa.library()
    p = synth.make_problem(2, 1025, 8192, seed=34)  # 1025 x 64 slices: one row too many
    ins = [dev(x) for x in p.inputs]
    res, w = dev(p.residual), dev(p.weight)
    ro, out = torch.zeros_like(res), torch.zeros_like(res)
    arr = (VP * p.n)(*[x.data_ptr() for x in ins])
    print("[gpu case] static-scratch split rows beyond the scratch: rejected", flush=True)
    rc = lib.fused_ar_rmsnorm_split_static(arr, p.n, res.data_ptr(), w.data_ptr(), p.eps, p.m,
                                           p.hidden, ro.data_ptr(), out.data_ptr(), 64, None)
    assert rc == fa.ERR_SCRATCH
    torch.cuda.synchronize()
    assert not ro.view(torch.int16).any() and not out.view(torch.int16).any()  # nothing launched


def test_static_scratch_under_graph_replay():
    """Calls of the static-scratch form captured in a HIP graph give the oracle's result on every
    replay, with an eager call of another shape between replays: that call overwrites the shared
    scratch, and each captured call rewrites every slot it reads before reading it."""
    lib = fa.library()

    def device_problem(p):
        ins = [dev(x) for x in p.inputs]
        res, w = dev(p.residual), dev(p.weight)
        return dict(ins=ins, arr=(VP * p.n)(*[x.data_ptr() for x in ins]), res=res, w=w,
                    ro=torch.empty_like(res), out=torch.empty_like(res))

    def call(p, d, stream):
        return lib.fused_ar_rmsnorm_split_static(d["arr"], p.n, d["res"].data_ptr(),
                                                 d["w"].data_ptr(), p.eps, p.m, p.hidden,
                                                 d["ro"].data_ptr(), d["out"].data_ptr(), 0, stream)

    p = synth.make_problem(8, 4, 7168, seed=35, name="static scratch in a graph")
    q = synth.make_problem(2, 300, 16384, seed=36, name="static scratch between replays")
    dp, dq = device_problem(p), device_problem(q)
    want_p = oracle.fused(p.inputs, p.residual, p.weight, p.eps)
    want_q = oracle.fused(q.inputs, q.residual, q.weight, q.eps)
    print("[gpu case] static-scratch split rows: eager call before capture", flush=True)
    assert call(q, dq, torch.cuda.current_stream().cuda_stream) == fa.OK
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture = torch.cuda.current_stream().cuda_stream
        for _ in range(10):
            assert call(p, dp, capture) == fa.OK
    for replay in range(3):
        print(f"[gpu case] static-scratch split rows: graph replay {replay}", flush=True)
        dp["ro"].zero_()
        dp["out"].zero_()
        dq["out"].zero_()
        assert call(q, dq, torch.cuda.current_stream().cuda_stream) == fa.OK
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (want_ro, want_out), d in ((want_p, dp), (want_q, dq)):
            assert np.array_equal(host(d["ro"]), want_ro), replay
            assert ulp_diff(host(d["out"]), want_out).max() <= 1, replay
