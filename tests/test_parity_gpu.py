"""Parity of the HIP path with the CPU oracle, element by element, through the C ABI.

Bar: `residual_out` and the reduce bit-exact; `out` within 1 bf16 ulp (the kernel's fp32 row
statistic versus the oracle's binary64 one); no NaN, except where the inputs hold +-inf and the
oracle has NaN too. Every problem is compared whole: the
full-size workloads run the unchanged single-threaded oracle on row slices across the host's
threads (rows are independent, so the slices together are the oracle's result).
"""
import os

import numpy as np
import pytest
import torch

import all_reduce_residual_way_amd as fa
import golden_cases
import oracle
from all_reduce_residual_way_amd import synth
from ulp import is_nan, ulp_diff

pytestmark = pytest.mark.gpu

OUT_ULP = 1  # tolerance on `out`, in bf16 units in the last place


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa.library()  # raises if the HIP library is not built
    yield


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def announce(what):
    print(f"[gpu case] {what}", flush=True)


def run_gpu(p, path, in_place=False):
    ins = [dev(x) for x in p.inputs]
    res = dev(p.residual)
    w = dev(p.weight)
    ro = res if in_place else torch.empty_like(res)
    out = torch.empty_like(res)
    fa.fused_ar_rmsnorm(ins, res, w, p.eps, residual_out=ro, out=out, path=path)
    torch.cuda.synchronize()
    return host(ro), host(out)


def host_threads():
    """Host threads for the oracle: those this process may run on, at most 16 (one GPU's share of
    a shared host)."""
    try:
        have = len(os.sched_getaffinity(0))
    except AttributeError:
        have = os.cpu_count() or 1
    return max(1, min(16, have))


# problems above this many elements run the oracle on row slices across host threads
THREADED_ORACLE_ELEMENTS = 1 << 22


def oracle_rows(p):
    """The oracle's (residual_out, out) for the whole problem."""
    if p.n * p.m * p.hidden > THREADED_ORACLE_ELEMENTS:
        return oracle.fused_threads(p.inputs, p.residual, p.weight, p.eps, host_threads())
    return oracle.fused(p.inputs, p.residual, p.weight, p.eps)


def assert_parity(name, got_ro, got_out, want_ro, want_out):
    bad = np.argwhere(got_ro != want_ro)
    assert bad.size == 0, (
        f"{name}: residual_out differs at {len(bad)} elements, first {tuple(bad[0])}: "
        f"gpu {got_ro[tuple(bad[0])]:#06x} oracle {want_ro[tuple(bad[0])]:#06x}")
    assert not is_nan(got_out).any(), f"{name}: NaN in out"
    d = ulp_diff(got_out, want_out)
    assert d.max() <= OUT_ULP, (
        f"{name}: out differs by {d.max()} ulp at {tuple(np.argwhere(d == d.max())[0])}")


def check_problem(p, path):
    name = f"{p.name} n={p.n} m={p.m} hidden={p.hidden} path={path}"
    announce(name)
    ro, out = run_gpu(p, path)
    want_ro, want_out = oracle_rows(p)
    assert_parity(name, ro, out, want_ro, want_out)
    return ro, out


# ------------------------------------------------------------------------- the workloads

def workload_cases():
    cases = []
    for wname, w in synth.WORKLOADS.items():
        ms = w["ms"] if w["ms"] is not None else synth.stress_m_values(0)
        paths = sorted(set(w["paths"]) | {1, 2})  # every workload on both paths, and its own
        for m in ms:
            for path in paths:
                cases.append(pytest.param(wname, m, path, id=f"{wname}-m{m}-p{path}"))
    return cases


@pytest.mark.parametrize("wname,m,path", workload_cases())
def test_workload(wname, m, path):
    w = synth.WORKLOADS[wname]
    seed = 1000 + m
    p = synth.make_problem(w["n"], m, w["hidden"], seed=seed, eps=w["eps"], dist=w["dist"],
                           name=wname)
    check_problem(p, path)


def test_paths_agree_bit_for_bit():
    """Path 1 and path 2 give identical residual_out (the reduce order is the same) and, since
    stage 2 is the same row kernel over the same bf16 values, identical out."""
    for n, m, hidden in [(8, 16, 7168), (4, 100, 4096), (8, 17, 2880), (3, 7, 520)]:
        p = synth.make_problem(n, m, hidden, seed=7)
        announce(f"paths agree n={n} m={m} hidden={hidden}")
        r1 = run_gpu(p, 1)
        r2 = run_gpu(p, 2)
        assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])


def test_auto_path_matches_explicit():
    """The automatic path gives the bits of the path the rule names, on either side of the rule's
    corners (two-stage only for a few rows of wide, many-input rows), and the oracle's result."""
    for n, m, hidden in [(8, 16, 2880), (4, 33, 2880), (8, 48, 32768), (8, 49, 32768),
                         (6, 16, 24576), (6, 17, 24576), (4, 3, 32768)]:
        p = synth.make_problem(n, m, hidden, seed=8)
        announce(f"auto n={n} m={m} hidden={hidden} -> path {fa.auto_path(n, m, hidden)}")
        r0 = run_gpu(p, 0)
        r = run_gpu(p, fa.auto_path(n, m, hidden))
        assert np.array_equal(r0[0], r[0]) and np.array_equal(r0[1], r[1])
        want_ro, want_out = oracle_rows(p)
        assert_parity(f"auto n={n} m={m} hidden={hidden}", r0[0], r0[1], want_ro, want_out)
    assert fa.auto_path(8, 48, 32768) == fa.PATH_TWOSTAGE
    assert fa.auto_path(8, 49, 32768) == fa.PATH_ONESTAGE


# ------------------------------------------------------------------------- the reduce alone

@pytest.mark.parametrize("n,m,hidden", [(1, 3, 8), (2, 5, 24), (3, 7, 520), (4, 64, 7168),
                                        (5, 33, 2880), (6, 1, 32768), (7, 9, 1000),
                                        (8, 257, 7168), (8, 4096, 7168),
                                        (3, 2, 65544)])  # rows wider than any row kernel takes
def test_reduce_bit_exact(n, m, hidden):
    p = synth.make_problem(n, m, hidden, seed=n * 100 + m)
    announce(f"reduce n={n} m={m} hidden={hidden}")
    red = fa.fused_ar_reduce([dev(x) for x in p.inputs])
    torch.cuda.synchronize()
    assert np.array_equal(host(red), oracle.reduce(p.inputs))


def test_reduce_full_exponent_range():
    """Random finite bf16 bits across the whole exponent range (subnormals included): the fp32
    sums, their overflow to infinity and their subnormal results match the oracle exactly."""
    rng = np.random.default_rng(5)
    for n in (2, 5, 8):
        ins = []
        for _ in range(n):
            b = rng.integers(0, 0x10000, (16, 512), dtype=np.uint32).astype(np.uint16)
            b[(b & 0x7F80) == 0x7F80] &= 0xBFFF   # no Inf/NaN inputs
            ins.append(b)
        announce(f"reduce exponent range n={n}")
        red = fa.fused_ar_reduce([dev(x) for x in ins])
        torch.cuda.synchronize()
        assert np.array_equal(host(red), oracle.reduce(ins))


def test_reduce_subnormal_sums():
    """Tiny inputs whose fp32 sums are subnormal: kept, not flushed to zero."""
    rng = np.random.default_rng(6)
    ins = [(rng.integers(0, 0x80, (4, 256)) | (rng.integers(0, 2, (4, 256)) << 15)).astype(np.uint16)
           for _ in range(4)]  # bf16 subnormals: exponent field 0
    announce("reduce subnormals")
    red = fa.fused_ar_reduce([dev(x) for x in ins])
    torch.cuda.synchronize()
    want = oracle.reduce(ins)
    assert np.array_equal(host(red), want)
    assert (want & 0x7FFF).any()


def test_non_finite_partial_sums():
    """Partial sums holding +-inf: the fp32 sums (inf, and inf - inf = NaN), residual_out, and the
    rows whose square-sum is infinite (out = +-0, NaN where residual_out is infinite) or NaN (the
    whole row NaN) match the oracle on every path and in the reduce alone, NaN for NaN (a NaN's
    sign and payload are not compared: the binary32 oracle takes the host's default NaN)."""
    base = synth.make_problem(4, 6, 1024, seed=71, name="non-finite")
    ins = [x.copy() for x in base.inputs]
    ins[1][0, 5] = 0x7F80                            # row 0: +inf in one input
    ins[0][1, 9], ins[3][1, 9] = 0x7F80, 0xFF80      # row 1: +inf + -inf = NaN
    ins[2][2, 100], ins[3][2, 100] = 0xFF80, 0xFF80  # row 2: -inf twice
    p = synth.Problem(ins, base.residual, base.weight, base.eps)
    want_red = oracle.reduce(ins)
    want_ro, want_out = oracle.fused(ins, p.residual, p.weight, p.eps)
    assert is_nan(want_out[1]).all() and is_nan(want_out[0]).sum() == 1  # what the case is for

    def same(got, want, what):
        gn, wn = is_nan(got), is_nan(want)
        assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
        assert np.array_equal(got[~gn], want[~wn]), f"{what}: values differ"

    announce("non-finite partial sums: reduce")
    red = fa.fused_ar_reduce([dev(x) for x in ins])
    torch.cuda.synchronize()
    same(host(red), want_red, "reduce")
    for path in (1, 2, fa.PATH_UNFUSED):
        announce(f"non-finite partial sums: path {path}")
        if path == fa.PATH_UNFUSED:
            ro_t, out_t = fa.fused_ar_unfused_rmsnorm([dev(x) for x in ins], dev(p.residual),
                                                      dev(p.weight), p.eps)
            torch.cuda.synchronize()
            ro, out = host(ro_t), host(out_t)
        else:
            ro, out = run_gpu(p, path)
        same(ro, want_ro, f"path {path} residual_out")
        same(out[:3], want_out[:3], f"path {path} out, non-finite rows")
        assert ulp_diff(out[3:], want_out[3:]).max() <= 1, f"path {path} out, finite rows"


# ------------------------------------------------------------------------- hand-worked cases

@pytest.mark.parametrize("fixture", ["reduce_hidden8.txt", "rmsnorm_hidden8.txt"])
@pytest.mark.parametrize("path", [1, 2])
def test_golden_cases_on_gpu(fixture, path):
    for case in golden_cases.load(fixture):
        announce(f"golden {case['name']} path={path}")
        p = synth.Problem(case["inputs"], case["residual"], case["weight"], case["eps"])
        ro, out = run_gpu(p, path)
        assert np.array_equal(ro, case["expect_residual_out"]), case["name"]
        if "expect_out" in case:
            assert np.array_equal(out, case["expect_out"]), (case["name"], out)
        if "expect_reduced" in case:
            red = fa.fused_ar_reduce([dev(x) for x in case["inputs"]])
            torch.cuda.synchronize()
            assert np.array_equal(host(red), case["expect_reduced"]), case["name"]


# ------------------------------------------------------------------------- edge cases

@pytest.mark.parametrize("n,m,hidden", [
    (1, 1, 8),        # one pack per row: a 64-thread workgroup with 63 idle lanes
    (2, 3, 16),
    (8, 2, 520),      # 65 packs: two waves, the second with one active lane
    (3, 5, 8184),     # 1023 packs
    (8, 4, 8192),     # exactly 1024 packs
    (4, 3, 8200),     # 1025 packs: two packs per thread
    (5, 2, 16392),    # 2049 packs: four packs per thread, ragged
    (8, 2, 32768),    # the largest row
    (7, 11, 2880),    # 360 packs, ragged against 64-lane waves
])
@pytest.mark.parametrize("path", [1, 2])
def test_edge_shapes(n, m, hidden, path):
    p = synth.make_problem(n, m, hidden, seed=hidden + n, name="edge")
    check_problem(p, path)


@pytest.mark.parametrize("path", [1, 2])
def test_in_place_residual(path):
    p = synth.make_problem(8, 24, 7168, seed=9, name="in-place")
    announce(f"in place path={path}")
    ro, out = run_gpu(p, path, in_place=True)
    want_ro, want_out = oracle_rows(p)
    assert_parity("in-place", ro, out, want_ro, want_out)


def test_zero_rows_and_eps():
    p = synth.make_problem(8, 40, 2880, seed=10, name="zero rows")
    for x in p.inputs:
        x[[0, 13, 39]] = 0
    p.residual[13] = 0  # a row that is zero all the way through: out = +-0 (sign of the weight)
    for path in (1, 2):
        announce(f"zero rows path={path}")
        ro, out = run_gpu(p, path)
        want_ro, want_out = oracle_rows(p)
        assert_parity("zero rows", ro, out, want_ro, want_out)
        assert np.array_equal(ro[0], p.residual[0]) and np.array_equal(ro[39], p.residual[39])
        assert np.array_equal(out[13], p.weight & np.uint16(0x8000))


@pytest.mark.parametrize("eps", [0.0, 1e-2, 1.0, 100.0])
def test_eps_values(eps):
    """eps from 0 (no zero rows here) to far above the mean square."""
    p = synth.make_problem(8, 9, 2880, seed=21, eps=eps, name=f"eps={eps}")
    for path in (1, 2):
        check_problem(p, path)


@pytest.mark.parametrize("eps", [0.0, 1e-44, 2.0 ** -126])
def test_tiny_rows_with_subnormal_mean_square(eps):
    """Rows scaled by 2^-60 .. 2^-120, so that mean(x^2) falls from the normal range (1e-36) through
    fp32's subnormals to far below them, with eps = 0 or subnormal: the kernels sum such rows'
    squares again at a 2^100 scale (squares below 2^-126 lose bits, below 2^-149 vanish), so out
    stays within 1 ulp of the oracle instead of turning into +-inf. With eps = 2^-126, the smallest
    normal value, eps dominates mean + eps and the kernel takes its unscaled form. Every path and
    the split-row form."""
    rng = np.random.default_rng(31)
    scales = [2.0 ** -60, 2.0 ** -63, 2.0 ** -66, 2.0 ** -68, 2.0 ** -72, 2.0 ** -80,
              2.0 ** -100, 2.0 ** -120]
    inputs = [synth.to_bf16_bits(np.array([rng.standard_normal(64) * s for s in scales],
                                          dtype=np.float32)) for _ in range(2)]
    residual = np.zeros((len(scales), 64), dtype=np.uint16)
    weight = synth.to_bf16_bits((1 + 0.1 * rng.standard_normal(64)).astype(np.float32))
    p = synth.Problem(inputs, residual, weight, eps, name=f"tiny rows eps={eps}")
    for path in (1, 2, fa.PATH_UNFUSED):
        check_problem(p, path)
    want_ro, want_out = oracle_rows(p)
    for splits in (1, 3):
        announce(f"tiny rows eps={eps} split rows splits={splits}")
        ro, out = run_split(p, splits)
        assert_parity(f"tiny rows split {splits}", ro, out, want_ro, want_out)


def test_large_values_and_ties():
    """The stress mix: +-3e4 rows, whose sums land on bf16 rounding ties."""
    p = synth.make_problem(8, 300, 2880, seed=11, dist="stress", name="stress ties")
    for path in (1, 2):
        check_problem(p, path)


@pytest.mark.parametrize("m", [256, 257, 1024, 1025])
def test_both_row_geometries(m):
    """Either side of the row counts where the row kernel switches between one and two packs per
    thread (hidden = 7168)."""
    p = synth.make_problem(8, m, 7168, seed=16, name="geometry")
    for path in (1, 2):
        check_problem(p, path)


def test_rows_beyond_the_grid():
    """More rows than one launch takes (2^20 workgroups): the rows come in two launches."""
    m = (1 << 20) + 3
    p = synth.make_problem(2, m, 8, seed=12, name="row stride")
    want_ro, want_out = oracle_rows(p)
    for path in (1, 2):
        announce(f"row stride path={path}")
        ro, out = run_gpu(p, path)
        assert_parity("row stride", ro, out, want_ro, want_out)


def test_flat_packs_beyond_one_launch():
    """More packs than one flat launch takes (2^30): the reduce comes in two launches, the second
    starting 2^30 packs into every buffer. With one input the reduce is the identity on finite
    values, so every element of the 16 GiB plane is checked, on the GPU."""
    m, hidden = (1 << 18) + 1, 32768   # 2^30 + 4096 packs of 8 elements
    assert fa.describe_launch(1, m, hidden, 2)["kernels"][0]["launches"] == 2
    announce(f"flat launches: reduce n=1 m={m} hidden={hidden}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(17)
    x = torch.randint(0, 0x7F80, (m, hidden), dtype=torch.int16, device="cuda", generator=gen)
    red = fa.fused_ar_reduce([x.view(torch.bfloat16)])
    torch.cuda.synchronize()
    red = red.view(torch.int16)
    for r in range(0, m, 8192):
        assert torch.equal(red[r:r + 8192], x[r:r + 8192]), r
    del x, red
    torch.cuda.empty_cache()


def test_empty_problem():
    x = torch.empty(0, 4096, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(4096, dtype=torch.bfloat16, device="cuda")
    ro, out = fa.fused_ar_rmsnorm([x, x], x, w, 1e-6)
    assert ro.shape == (0, 4096) and out.shape == (0, 4096)


def test_rejects_aliasing_out_on_gpu_tensors():
    p = synth.make_problem(2, 4, 64, seed=13)
    ins = [dev(x) for x in p.inputs]
    with pytest.raises(fa.FusedArError) as e:
        fa.fused_ar_rmsnorm(ins, dev(p.residual), dev(p.weight), 1e-6, out=ins[0])
    assert e.value.status == fa.ERR_ALIAS


@pytest.mark.parametrize("path", [1, 2])
def test_read_only_buffers_may_alias(path):
    """Read-only buffers may be the same memory: one tensor passed as three of the four partial
    sums and as the residual gives the oracle's result for those repeated arrays."""
    p = synth.make_problem(2, 37, 4096, seed=14, name="aliased inputs")
    x, y = dev(p.inputs[0]), dev(p.inputs[1])
    announce(f"aliased read-only buffers path={path}")
    ro, out = fa.fused_ar_rmsnorm([x, x, y, x], x, dev(p.weight), p.eps, path=path)
    torch.cuda.synchronize()
    a, b = p.inputs
    want_ro, want_out = oracle.fused([a, a, b, a], a, p.weight, p.eps)
    assert_parity(f"aliased path={path}", host(ro), host(out), want_ro, want_out)


# ------------------------------------------------------------------------- invariants

@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("n,m,hidden", [(8, 37, 7168), (4, 300, 2880)])
def test_row_permutation_equivariance(n, m, hidden, path):
    """Rows are independent: permuting the rows of every input and of the residual permutes both
    outputs, bit for bit (a mistake in the row indexing of any kernel fails this)."""
    p = synth.make_problem(n, m, hidden, seed=41, name="rows")
    perm = np.random.default_rng(41).permutation(m)
    announce(f"row permutation n={n} m={m} hidden={hidden} path={path}")
    ro, out = run_gpu(p, path)
    q = synth.Problem([x[perm] for x in p.inputs], p.residual[perm], p.weight, p.eps)
    ro_q, out_q = run_gpu(q, path)
    assert np.array_equal(ro_q, ro[perm])
    assert np.array_equal(out_q, out[perm])


@pytest.mark.parametrize("path", [1, 2])
def test_input_order_irrelevant_when_sums_are_exact(path):
    """Inputs that are multiples of 2^-4 with |value| <= 8 make every fp32 partial sum exact, so the
    reduce result, and with it both outputs, cannot depend on the order of the inputs: reversing or
    rotating them leaves the bits unchanged (an input dropped or read twice changes them)."""
    rng = np.random.default_rng(43)
    n, m, hidden = 8, 24, 7168
    ins = [synth.to_bf16_bits(rng.integers(-128, 129, (m, hidden)).astype(np.float32) / 16)
           for _ in range(n)]
    residual = synth.to_bf16_bits(rng.standard_normal((m, hidden), dtype=np.float32))
    weight = synth.to_bf16_bits((1 + 0.1 * rng.standard_normal(hidden)).astype(np.float32))
    p = synth.Problem(ins, residual, weight, 1e-6, name="exact sums")
    ro, out = check_problem(p, path)
    for order in (ins[::-1], ins[3:] + ins[:3]):
        announce(f"input order path={path}")
        ro_q, out_q = run_gpu(synth.Problem(order, residual, weight, 1e-6), path)
        assert np.array_equal(ro_q, ro)
        assert np.array_equal(out_q, out)


def _bf16_values(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("k", [-20, 7])
def test_power_of_two_scaling(k, path):
    """Scaling every input and the residual by 2^k scales residual_out by exactly 2^k (fp32 sums
    and the rounding to bf16 commute with it while nothing overflows or turns subnormal), and with
    eps = 0 the normalised row is unchanged: out stays within the 1-ulp band of the unscaled call."""
    p = synth.make_problem(8, 16, 7168, seed=47, eps=0.0, name="scale")
    announce(f"power-of-two scaling k={k} path={path}")
    ro, out = run_gpu(p, path)
    s = np.float32(2.0 ** k)
    q = synth.Problem([synth.to_bf16_bits(_bf16_values(x) * s) for x in p.inputs],
                      synth.to_bf16_bits(_bf16_values(p.residual) * s), p.weight, 0.0)
    ro_k, out_k = run_gpu(q, path)
    assert np.array_equal(ro_k, synth.to_bf16_bits(_bf16_values(ro) * s))
    assert ulp_diff(out_k, out).max() <= OUT_ULP


# ------------------------------------------------------------------------- repeatability

def test_deterministic():
    p = synth.make_problem(8, 64, 7168, seed=14)
    for path in (1, 2):
        announce(f"determinism path={path}")
        a = run_gpu(p, path)
        b = run_gpu(p, path)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_graph_replay_matches_eager():
    """A chain of calls captured into one graph gives the eager result on every replay, with eager
    work and synchronisations between replays."""
    p = synth.make_problem(8, 16, 7168, seed=15)
    ins = [dev(x) for x in p.inputs]
    res, w = dev(p.residual), dev(p.weight)
    pages_split = fa.Options()
    pages_split.residual_stage = fa.RESIDUAL_STAGE2
    calls = [  # path 1, path 2, the pages' residual split, the unfused sequence
        lambda ro, out: fa.fused_ar_rmsnorm(ins, res, w, p.eps, residual_out=ro, out=out, path=1),
        lambda ro, out: fa.fused_ar_rmsnorm(ins, res, w, p.eps, residual_out=ro, out=out, path=2),
        lambda ro, out: fa.fused_ar_rmsnorm(ins, res, w, p.eps, residual_out=ro, out=out, path=2,
                                            options=pages_split),
        lambda ro, out: fa.fused_ar_unfused_rmsnorm(ins, res, w, p.eps, residual_out=ro, out=out),
    ]
    eager = [call(torch.empty_like(res), torch.empty_like(res)) for call in calls]
    torch.cuda.synchronize()
    bufs = [(torch.empty_like(res), torch.empty_like(res)) for _ in calls]
    ro, out = bufs[0]
    announce("graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(10):
            for call, (r, o) in zip(calls, bufs):
                call(r, o)
    for replay in range(4):
        for r, o in bufs:
            r.zero_()
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, ((r, o), (r_e, o_e)) in enumerate(zip(bufs, eager)):
            assert torch.equal(r.view(torch.int16), r_e.view(torch.int16)), (replay, k)
            assert torch.equal(o.view(torch.int16), o_e.view(torch.int16)), (replay, k)
    want_ro, want_out = oracle_rows(p)
    assert_parity("graph", host(ro), host(out), want_ro, want_out)


def test_concurrent_calls_on_two_streams():
    """The library keeps no state, so calls enqueued on two streams at once, on separate buffers
    and on every path, each give the oracle's result."""
    probs = [synth.make_problem(8, 300, 7168, seed=16), synth.make_problem(4, 17, 2880, seed=17)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    bufs = []
    for p in probs:
        ins = [dev(x) for x in p.inputs]
        res, w = dev(p.residual), dev(p.weight)
        outs = {path: (torch.empty_like(res), torch.empty_like(res)) for path in (1, 2, "split")}
        bufs.append((ins, res, w, outs))
    torch.cuda.synchronize()
    announce("two streams, 10 rounds of every path")
    def enqueue(ins, res, w, outs, p, stream):
        for path, (ro, out) in outs.items():
            if path == "split":  # the workspace is allocated by the binding
                fa.fused_ar_rmsnorm_split(ins, res, w, p.eps, residual_out=ro, out=out,
                                          stream=stream)
            else:
                fa.fused_ar_rmsnorm(ins, res, w, p.eps, residual_out=ro, out=out, path=path,
                                    stream=stream)

    for _ in range(10):
        with torch.cuda.stream(streams[0]):  # the first problem: the current stream
            enqueue(*bufs[0], probs[0], None)
        enqueue(*bufs[1], probs[1], streams[1])  # the second: an explicit stream argument
    torch.cuda.synchronize()
    for (ins, res, w, outs), p in zip(bufs, probs):
        want_ro, want_out = oracle_rows(p)
        for path, (ro, out) in outs.items():
            assert_parity(f"stream n={p.n} path={path}", host(ro), host(out), want_ro, want_out)


def test_outputs_allocated_for_a_side_stream_are_not_reused_early():
    """Outputs the binding allocates for work on a side stream are recorded on that stream: the
    caller dropping them at once must not let the current stream's next allocation take their
    memory while the side stream has not yet run the kernels that write them."""
    p = synth.make_problem(8, 64, 7168, seed=24, name="side stream")
    ins = [dev(x) for x in p.inputs]
    res, w = dev(p.residual), dev(p.weight)
    side = torch.cuda.Stream()  # default priority
    torch.cuda.synchronize()
    announce("outputs recorded on a side stream")
    for path in (1, 2):
        with torch.cuda.stream(side):
            torch.cuda._sleep(20_000_000)  # keep the side stream busy for a few milliseconds
        ro, out = fa.fused_ar_rmsnorm(ins, res, w, p.eps, path=path, stream=side)
        taken = {ro.data_ptr(), out.data_ptr()}
        del ro, out
        fresh = [torch.empty_like(res) for _ in range(2)]  # the current stream's next blocks
        assert not taken & {t.data_ptr() for t in fresh}, path
        torch.cuda.synchronize()
        del fresh


# ------------------------------------------------------------------------- unfused baseline

@pytest.mark.parametrize("n,m,hidden", [(8, 16, 7168), (4, 300, 7168), (8, 33, 2880), (3, 5, 520),
                                        (8, 2048, 7168)])
def test_unfused_matches_fused_bit_for_bit(n, m, hidden):
    """The unfused three-kernel sequence gives the fused result exactly: same reduce order, same
    bf16 roundings, and its RMSNorm kernel has the one-stage kernel's reduction tree."""
    p = synth.make_problem(n, m, hidden, seed=17, name="unfused")
    ins = [dev(x) for x in p.inputs]
    res, w = dev(p.residual), dev(p.weight)
    announce(f"unfused n={n} m={m} hidden={hidden}")
    ro_u, out_u = fa.fused_ar_unfused_rmsnorm(ins, res, w, p.eps)
    ro_f, out_f = fa.fused_ar_rmsnorm(ins, res, w, p.eps, path=1)
    torch.cuda.synchronize()
    assert torch.equal(ro_u.view(torch.int16), ro_f.view(torch.int16))
    assert torch.equal(out_u.view(torch.int16), out_f.view(torch.int16))
    want_ro, want_out = oracle_rows(p)
    assert_parity("unfused", host(ro_u), host(out_u), want_ro, want_out)


def test_unfused_in_place_residual():
    p = synth.make_problem(8, 40, 2880, seed=18, name="unfused in place")
    ins = [dev(x) for x in p.inputs]
    res, w = dev(p.residual), dev(p.weight)
    announce("unfused in place")
    ro, out = fa.fused_ar_unfused_rmsnorm(ins, res, w, p.eps, residual_out=res)
    torch.cuda.synchronize()
    want_ro, want_out = oracle_rows(p)
    assert_parity("unfused in place", host(ro), host(out), want_ro, want_out)


# ------------------------------------------------------------------------- design options

OPTION_SETS = [
    (fa.WAVE_BPERMUTE, fa.STAGE1_FLAT, 0, 0, 0),
    (fa.WAVE_DPP, fa.STAGE1_LDS, 0, 0, 0),
    (fa.WAVE_BPERMUTE, fa.STAGE1_LDS, 512, 0, fa.LOAD_STREAM),
    (fa.WAVE_DPP, fa.STAGE1_FLAT, 512, 0, fa.LOAD_CACHED),
    (fa.WAVE_DPP, fa.STAGE1_FLAT, 64, 0, fa.LOAD_STREAM),
    (fa.WAVE_DPP, fa.STAGE1_FLAT, 1024, 0, 0),
    (fa.WAVE_DPP, fa.STAGE1_FLAT, 0, 0, fa.LOAD_STREAM),
    # the two-stage path in chunks of 7 rows (ragged last chunk), sequential and pipelined
    (fa.WAVE_DPP, fa.STAGE1_FLAT, 0, 0, 0, 7, fa.CHUNKS_SEQUENTIAL),
    (fa.WAVE_DPP, fa.STAGE1_FLAT, 0, 0, 0, 7, fa.CHUNKS_PIPELINED),
    (fa.WAVE_BPERMUTE, fa.STAGE1_LDS, 0, 0, fa.LOAD_STREAM, 2, fa.CHUNKS_SEQUENTIAL),
    (fa.WAVE_DPP, fa.STAGE1_FLAT, 256, 0, fa.LOAD_STREAM, 1, fa.CHUNKS_PIPELINED),
    # where the two-stage path adds the residual: the pages' split (stage 2, through the scratch)
    # or stage 1 (the default)
    (fa.WAVE_DPP, fa.STAGE1_FLAT, 0, 0, 0, 0, 0, fa.RESIDUAL_STAGE2),
    (fa.WAVE_BPERMUTE, fa.STAGE1_FLAT, 512, 0, fa.LOAD_STREAM, 0, 0, fa.RESIDUAL_STAGE2),
    (fa.WAVE_DPP, fa.STAGE1_FLAT, 256, 0, fa.LOAD_CACHED, -1, 0, fa.RESIDUAL_STAGE1),
]


def _option_id(o):
    o = tuple(o) + (0,) * (8 - len(o))
    return "w{}-s{}-b{}-p{}-l{}-r{}-c{}-x{}".format(*o)


@pytest.mark.parametrize("opt", OPTION_SETS, ids=_option_id)
@pytest.mark.parametrize("n,m,hidden", [(8, 37, 7168), (3, 11, 520), (5, 300, 2880), (1, 9, 64)])
def test_design_options_are_bit_identical(opt, n, m, hidden):
    """The ds_bpermute wave reduction, the LDS-staged stage 1, other stage-1 workgroup sizes and
    the two-stage path in chunks of rows give exactly the default kernels' bits on every path
    (and so the oracle's)."""
    p = synth.make_problem(n, m, hidden, seed=19, name="options")
    ins = [dev(x) for x in p.inputs]
    res, w = dev(p.residual), dev(p.weight)
    announce(f"options {opt} n={n} m={m} hidden={hidden}")
    for path in (1, 2, fa.PATH_UNFUSED):
        ro_d, out_d = fa.fused_ar_rmsnorm(ins, res, w, p.eps, path=path)
        ro_o, out_o = fa.fused_ar_rmsnorm(ins, res, w, p.eps, path=path, options=fa.Options(*opt))
        torch.cuda.synchronize()
        assert torch.equal(ro_o.view(torch.int16), ro_d.view(torch.int16)), path
        assert torch.equal(out_o.view(torch.int16), out_d.view(torch.int16)), path
    want_ro, want_out = oracle_rows(p)
    assert_parity("options", host(ro_o), host(out_o), want_ro, want_out)


@pytest.mark.parametrize("variant", ["sequential", "pipelined", "residual in stage 1",
                                     "pages' split"])
def test_two_stage_variants_on_a_long_streaming_call(variant):
    """The two-stage path in chunks of 512 rows, with the residual add in stage 1 (the default) or
    in stage 2 (the pages' split), on a call that streams and caps its row workgroups (two packs
    per thread), also in place: the oracle's result, and path 1's bits."""
    opts = {"sequential": fa.Options(0, 0, 0, 0, 0, 512, fa.CHUNKS_SEQUENTIAL),
            "pipelined": fa.Options(0, 0, 0, 0, 0, 512, fa.CHUNKS_PIPELINED),
            "residual in stage 1": fa.Options(0, 0, 0, 0, 0, 0, 0, fa.RESIDUAL_STAGE1),
            "pages' split": fa.Options(0, 0, 0, 0, 0, 0, 0, fa.RESIDUAL_STAGE2)}
    p = synth.make_problem(4, 2100, 7168, seed=23, name="chunks")
    ins = [dev(x) for x in p.inputs]
    res, w = dev(p.residual), dev(p.weight)
    announce(f"two-stage {variant} n=4 m=2100 hidden=7168")
    ro1, out1 = fa.fused_ar_rmsnorm(ins, res, w, p.eps, path=1)
    ro, out = fa.fused_ar_rmsnorm(ins, res, w, p.eps, path=2, options=opts[variant])
    torch.cuda.synchronize()
    assert torch.equal(ro.view(torch.int16), ro1.view(torch.int16))
    assert torch.equal(out.view(torch.int16), out1.view(torch.int16))
    want_ro, want_out = oracle_rows(p)
    assert_parity(variant, host(ro), host(out), want_ro, want_out)
    # in place: residual_out is the residual's own buffer
    res_in_place = res.clone()
    ro, out = fa.fused_ar_rmsnorm(ins, res_in_place, w, p.eps, residual_out=res_in_place, path=2,
                                  options=opts[variant])
    torch.cuda.synchronize()
    assert_parity(f"{variant} in place", host(ro), host(out), want_ro, want_out)


@pytest.mark.parametrize("ppt", [1, 2, 4])
def test_forced_packs_per_thread(ppt):
    """Every row geometry is within the oracle's bar (out may move within its 1-ulp band)."""
    for n, m, hidden in [(8, 20, 7168), (4, 7, 2880), (2, 3, 8200)]:
        if (hidden // 8 + ppt - 1) // ppt > 1024:
            continue
        p = synth.make_problem(n, m, hidden, seed=20 + ppt, name="ppt")
        announce(f"ppt={ppt} n={n} m={m} hidden={hidden}")
        for path in (1, 2):
            ins = [dev(x) for x in p.inputs]
            ro, out = fa.fused_ar_rmsnorm(ins, dev(p.residual), dev(p.weight), p.eps, path=path,
                                          options=fa.Options(0, 0, 0, ppt))
            torch.cuda.synchronize()
            want_ro, want_out = oracle_rows(p)
            assert_parity(f"ppt={ppt}", host(ro), host(out), want_ro, want_out)


# ------------------------------------------------------------------------- randomized sweep

def test_randomized_shapes_paths_and_options():
    """80 seeded random cases: n in 1..8, m in 1..300, hidden any multiple of 8 up to 9600, every
    path (auto, one-stage, two-stage, unfused), random design options (chunked two-stage
    schedules included) and eps, normal or stress values; each compared whole with the oracle."""
    rng = np.random.default_rng(2024)
    for case in range(80):
        n = int(rng.integers(1, 9))
        m = int(rng.integers(1, 301))
        hidden = 8 * int(rng.integers(1, 1201))
        path = int(rng.choice([0, 1, 2, fa.PATH_UNFUSED]))
        ppt = int(rng.choice([0, 1, 2, 4]))
        if (hidden // 8 + max(ppt, 1) - 1) // max(ppt, 1) > 1024:
            ppt = 0
        opt = fa.Options(int(rng.integers(0, 2)), int(rng.integers(0, 2)),
                         int(rng.choice([0, 64, 256, 512, 1024])), ppt, int(rng.integers(0, 3)),
                         int(rng.choice([0, 0, 1, 13, 64])), int(rng.integers(0, 3)))
        opt.residual_stage = int(rng.integers(0, 3))
        if opt.residual_stage == fa.RESIDUAL_STAGE1 and (opt.stage1 == fa.STAGE1_LDS
                                                          or opt.stage_rows > 0):
            opt.residual_stage = fa.RESIDUAL_AUTO  # stage 1 has no LDS-staged or chunked form
        eps = float(rng.choice([1e-6, 1e-5, 0.1]))
        dist = "stress" if rng.random() < 0.3 else "normal"
        p = synth.make_problem(n, m, hidden, seed=5000 + case, eps=eps, dist=dist, name="random")
        name = (f"random case {case}: n={n} m={m} hidden={hidden} path={path} "
                f"options=({opt.wave_reduce},{opt.stage1},{opt.stage1_block},{opt.packs_per_thread},"
                f"{opt.load_policy},{opt.stage_rows},{opt.schedule},{opt.residual_stage}) "
                f"eps={eps} {dist}")
        announce(name)
        ins = [dev(x) for x in p.inputs]
        ro, out = fa.fused_ar_rmsnorm(ins, dev(p.residual), dev(p.weight), eps, path=path,
                                      options=opt)
        torch.cuda.synchronize()
        want_ro, want_out = oracle_rows(p)
        assert_parity(name, host(ro), host(out), want_ro, want_out)


# ------------------------------------------------------------------------- split rows

def run_split(p, splits, in_place=False, workspace=None):
    ins = [dev(x) for x in p.inputs]
    res = dev(p.residual)
    w = dev(p.weight)
    ro = res if in_place else torch.empty_like(res)
    out = torch.empty_like(res)
    fa.fused_ar_rmsnorm_split(ins, res, w, p.eps, splits=splits, workspace=workspace,
                              residual_out=ro, out=out)
    torch.cuda.synchronize()
    return host(ro), host(out)


@pytest.mark.parametrize("n,m,hidden,splits", [
    (8, 1, 7168, 0),      # 4 slices of 224 packs
    (8, 1, 7168, 1),      # one slice: the one-stage row
    (8, 3, 7168, 4),
    (8, 32, 7168, 7),     # 128 packs per slice, the last one short
    (4, 8, 4096, 0),
    (8, 2, 32768, 0),     # 16 slices of 256 packs
    (8, 1, 32768, 4),     # 4 slices of 1024 packs: full 1024-thread workgroups
    (5, 17, 520, 3),      # 65 packs: slices of 22, 22, 21
    (1, 5, 2880, 0),
    (2, 4, 8, 3),         # one pack per row: capped at one slice
    (8, 9, 2880, 64),     # 360 packs in slices of 6: the last four slices are empty
])
def test_split_rows_match_the_oracle(n, m, hidden, splits):
    p = synth.make_problem(n, m, hidden, seed=7000 + m + splits, name="split")
    announce(f"split rows n={n} m={m} hidden={hidden} splits={splits}")
    ro, out = run_split(p, splits)
    want_ro, want_out = oracle_rows(p)
    assert_parity(f"split n={n} m={m} hidden={hidden} splits={splits}", ro, out, want_ro, want_out)
    one_ro, _ = run_gpu(p, 1)
    assert np.array_equal(ro, one_ro)  # the same residual_out bits as the one-stage path
    again = run_split(p, splits)
    assert np.array_equal(ro, again[0]) and np.array_equal(out, again[1])  # deterministic


def test_split_rows_stress_in_place_and_reused_workspace():
    """Zero rows, +-3e4 rows and ties, in place (residual_out == residual), one workspace reused
    by calls of different sizes."""
    ws = torch.empty(64 * 64, dtype=torch.float32, device="cuda")
    for m, splits in ((40, 0), (7, 5), (64, 3)):
        p = synth.make_problem(8, m, 2880, seed=7100 + m, dist="stress", name="split stress")
        announce(f"split rows stress in place m={m} splits={splits}")
        ro, out = run_split(p, splits, in_place=True, workspace=ws)
        want_ro, want_out = oracle_rows(p)
        assert_parity(f"split stress m={m}", ro, out, want_ro, want_out)


def test_split_rows_graph_replay():
    p = synth.make_problem(8, 4, 7168, seed=7200)
    ins = [dev(x) for x in p.inputs]
    res, w = dev(p.residual), dev(p.weight)
    ro_e, out_e = fa.fused_ar_rmsnorm_split(ins, res, w, p.eps)
    ws = torch.empty(fa.split_workspace_bytes(4, 7168) // 4, dtype=torch.float32, device="cuda")
    ro, out = torch.empty_like(res), torch.empty_like(res)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(10):
            fa.fused_ar_rmsnorm_split(ins, res, w, p.eps, workspace=ws, residual_out=ro, out=out)
    for replay in range(3):
        announce(f"split rows graph replay {replay}")
        ro.zero_()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ro.view(torch.int16), ro_e.view(torch.int16)), replay
        assert torch.equal(out.view(torch.int16), out_e.view(torch.int16)), replay


def test_split_rows_randomized():
    """30 seeded random split-row cases: n in 1..8, m in 1..96, hidden any multiple of 8 up to
    32768, slices 0 (automatic) or 1..64 where a slice fits 1024 threads, eps and value mix at
    random; each compared whole with the oracle."""
    rng = np.random.default_rng(2025)
    for case in range(30):
        n = int(rng.integers(1, 9))
        m = int(rng.integers(1, 97))
        hidden = 8 * int(rng.integers(1, 4097))
        splits = int(rng.choice([0, int(rng.integers(1, 65))]))
        if fa.split_workspace_bytes(m, hidden, splits) == 0:
            splits = 0  # too few slices for one pack per thread: let the library choose
        eps = float(rng.choice([1e-6, 1e-5, 0.1]))
        dist = "stress" if rng.random() < 0.3 else "normal"
        p = synth.make_problem(n, m, hidden, seed=6000 + case, eps=eps, dist=dist, name="random split")
        name = f"random split case {case}: n={n} m={m} hidden={hidden} splits={splits} eps={eps} {dist}"
        announce(name)
        ro, out = run_split(p, splits)
        want_ro, want_out = oracle_rows(p)
        assert_parity(name, ro, out, want_ro, want_out)


def test_long_streaming_calls_randomized():
    """8 seeded random calls long enough to stream from HBM (over 128 MiB read, over 1024 rows),
    where the row kernels are capped at two workgroups per CU and take 1, 2 or 4 packs per thread
    by row width: path 1 whole against the oracle, and paths 1 and 2 and the unfused sequence
    bit-identical to each other."""
    rng = np.random.default_rng(2026)
    for case in range(8):
        n = int(rng.integers(2, 9))
        hidden = 8 * int(rng.integers(200, 4097))
        m = (128 << 20) // (2 * (n + 1) * hidden) + int(rng.integers(1, 600))
        m = max(m, 1025)
        plan = fa.describe_launch(n, m, hidden, 1)["kernels"][0]
        assert plan["streaming"] == 1 and plan["lds_bytes"] > 0, plan
        p = synth.make_problem(n, m, hidden, seed=8000 + case, name="long streaming")
        name = (f"long streaming case {case}: n={n} m={m} hidden={hidden} "
                f"packs/thread={plan['per_thread']} block={plan['block']}")
        announce(name)
        ins = [dev(x) for x in p.inputs]
        res, w = dev(p.residual), dev(p.weight)
        got = {}
        for path in (1, 2, fa.PATH_UNFUSED):
            ro, out = fa.fused_ar_rmsnorm(ins, res, w, p.eps, path=path)
            torch.cuda.synchronize()
            got[path] = (ro.view(torch.int16), out.view(torch.int16))
        for path in (2, fa.PATH_UNFUSED):
            assert torch.equal(got[path][0], got[1][0]) and torch.equal(got[path][1], got[1][1]), path
        want_ro, want_out = oracle_rows(p)
        assert_parity(name, host(got[1][0].view(torch.bfloat16)),
                      host(got[1][1].view(torch.bfloat16)), want_ro, want_out)
        del ins, res, got
        torch.cuda.empty_cache()
