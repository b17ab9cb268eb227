"""Property tests of the argument checks (CPU only, no kernel is launched): random buffer layouts
and scalars against a plain Python statement of the rules in include/fused_ar.h. Every layout
that the model accepts is only passed to fused_ar_rmsnorm_check, which never launches."""
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import all_reduce_residual_way_amd as fa  # noqa: E402

BASE = 0x7F0000000000
UNIT = 4096  # buffer offsets are multiples of 16 bytes, spread over a few units


def model(n, m, hidden, eps, path, ins, res, w, ro, out):
    """The documented checks, in the documented order."""
    if not (1 <= n <= 8) or m < 0 or hidden <= 0 or not (eps >= 0) or eps == float("inf"):
        return fa.ERR_INVALID
    if path not in (0, 1, 2):
        return fa.ERR_INVALID
    if hidden % 8 or hidden > fa.MAX_HIDDEN:
        return fa.ERR_SHAPE
    if m == 0:
        return fa.OK
    ptrs = list(ins) + [res, w, ro, out]
    if any(p == 0 for p in ptrs):
        return fa.ERR_INVALID
    if any(p % 16 for p in ptrs):
        return fa.ERR_ALIGN
    plane = m * hidden * 2
    span = lambda p, size: (p, p + size)  # noqa: E731
    ov = lambda a, b: a[0] < b[1] and b[0] < a[1]  # noqa: E731
    s_in = [span(p, plane) for p in ins]
    s_res, s_w, s_ro, s_out = span(res, plane), span(w, hidden * 2), span(ro, plane), span(out, plane)
    for si in s_in:
        if ov(s_out, si) or ov(s_ro, si):
            return fa.ERR_ALIAS
    if ov(s_out, s_res) or ov(s_out, s_w) or ov(s_out, s_ro) or ov(s_ro, s_w):
        return fa.ERR_ALIAS
    if ov(s_ro, s_res) and ro != res:
        return fa.ERR_ALIAS
    return fa.OK


offsets = st.integers(min_value=0, max_value=64).map(lambda k: BASE + k * UNIT)
# at most one faulty pointer per example: none (most often), a null, or a misaligned one, on any of
# the n inputs or the four single buffers
faults = st.one_of(st.just(None),
                   st.tuples(st.sampled_from(["null", "skew"]), st.integers(min_value=0, max_value=12),
                             st.integers(min_value=1, max_value=15)))


@settings(max_examples=4000, deadline=None)
@given(n=st.integers(min_value=0, max_value=9), m=st.integers(min_value=-1, max_value=3),
       hidden=st.sampled_from([8, 16, 24, 512, 1000, 1024, 12, 0, -8, 32768, 32776]),
       eps=st.sampled_from([0.0, -0.0, 1e-6, -1e-6, float("nan"), float("inf")]),
       path=st.integers(min_value=-1, max_value=3),
       ins=st.lists(offsets, min_size=9, max_size=9), res=offsets, w=offsets, ro=offsets,
       out=offsets, fault=st.one_of(st.just(None), faults))
def test_checks_follow_the_documented_rules(n, m, hidden, eps, path, ins, res, w, ro, out, fault):
    ptrs = ins[:max(n, 0)] + [res, w, ro, out]
    if fault is not None:
        kind, index, delta = fault
        index %= len(ptrs)
        ptrs[index] = 0 if kind == "null" else ptrs[index] + delta
    ins, (res, w, ro, out) = ptrs[:-4], ptrs[-4:]
    want = model(n, m, hidden, eps, path, ins, res, w, ro, out)
    got = fa.fused_ar_rmsnorm_check_ptrs(ins, res, w, eps, m, hidden, ro, out, path)
    assert got == want, (n, m, hidden, eps, path, [hex(p) for p in ins], hex(res), hex(w),
                         hex(ro), hex(out))


# ------------------------------------------------------------------------- launch plans

ROWS_PER_LAUNCH = 1 << 20
FLAT_PACKS_PER_LAUNCH = 1 << 30


def expected_streaming(n, m, hidden, policy):
    """Load policy: forced, or streaming when a call reads more than 128 MiB (inputs + residual)."""
    if policy != fa.LOAD_AUTO:
        return policy == fa.LOAD_STREAM
    return 2 * (n + 1) * m * hidden > (128 << 20)


def expected_rows(packs, m, forced, capped):
    """Packs per thread and threads of the row kernel, or None where a forced value does not fit."""
    if forced:
        k = forced
        if (packs + k - 1) // k > 1024:
            return None
    else:
        if capped:
            k = 4 if packs > 1024 else (2 if packs >= 512 else 1)
        else:
            k = 2 if (257 <= m <= 1024 and packs > 512) else 1
        while k < 4 and (packs + k - 1) // k > 1024:
            k *= 2
    t = (packs + k - 1) // k
    return k, (t + 63) // 64 * 64


@settings(max_examples=3000, deadline=None)
@given(n=st.integers(min_value=1, max_value=8),
       m=st.one_of(st.sampled_from([0, 1, 16, 17, 32, 33, 256, 257, 1024, 1025, 4096]),
                   st.integers(min_value=0, max_value=40), st.integers(min_value=0, max_value=5000),
                   st.integers(min_value=(1 << 20) - 2, max_value=(1 << 20) + 2),
                   st.integers(min_value=0, max_value=1 << 22)),
       packs=st.one_of(st.integers(min_value=1, max_value=4096),
                       st.sampled_from([360, 511, 512, 896, 1024, 1025, 2048, 4096])),
       path=st.integers(min_value=0, max_value=3),
       wave=st.integers(min_value=0, max_value=1), stage1=st.integers(min_value=0, max_value=1),
       block=st.sampled_from([0, 64, 256, 512, 1024]), ppt=st.sampled_from([0, 1, 2, 4]),
       policy=st.integers(min_value=0, max_value=2),
       rows=st.one_of(st.sampled_from([0, -1, 1, 2, 7, 512, 1024, 1 << 20]),
                      st.integers(min_value=1, max_value=5000)),
       sched=st.integers(min_value=0, max_value=2))
def test_launch_plans_follow_the_geometry_rules(n, m, packs, path, wave, stage1, block, ppt,
                                                policy, rows, sched):
    check_plan(n, m, packs, path, wave, stage1, block, ppt, policy, rows, sched)


def test_launch_plans_on_the_rule_boundaries():
    """Every combination of the values where a rule changes, so that each boundary is checked
    whatever the random examples above happen to draw."""
    import itertools
    for n, m, packs, path, stage1, block, ppt, policy in itertools.product(
            (1, 4, 5, 8), (0, 1, 16, 17, 32, 33, 256, 257, 1024, 1025, 2048, 4096, 9000),
            (1, 360, 511, 512, 513, 896, 1024, 1025, 2048, 4096), (0, 1, 2, 3), (0, 1),
            (0, 256), (0, 1, 2, 4), (0, 1, 2)):
        check_plan(n, m, packs, path, 0, stage1, block, ppt, policy)
    for n, m, packs, rows, sched, stage1, policy in itertools.product(
            (1, 8), (1, 2, 1024, 1025, 4096, 9000), (1, 896, 2048), (0, -1, 1, 2, 1023, 1024, 4096),
            (0, 1, 2), (0, 1), (0, 2)):
        check_plan(n, m, packs, 2, 0, stage1, 0, 0, policy, rows, sched)


def expected_flat(n, packs_total, block, stage1):
    """Workgroup and first-launch grid of a flat kernel over packs_total packs."""
    if stage1:
        want_block = 64 * n
    elif block:
        want_block = block
    else:
        want_block = 512 if packs_total >= (1 << 20) else 256
    first = min(packs_total, FLAT_PACKS_PER_LAUNCH)
    return want_block, -(-first // want_block)


def check_plan(n, m, packs, path, wave, stage1, block, ppt, policy, rows=0, sched=0):
    hidden = 8 * packs
    opt = fa.Options(wave, stage1, block, ppt, policy, rows, sched)
    stream = expected_streaming(n, m, hidden, policy)
    capped = stream and m > 1024
    rows_geometry = expected_rows(packs, m, ppt, capped)
    if m > 0 and rows_geometry is None:
        with pytest.raises(fa.FusedArError) as e:
            fa.describe_launch(n, m, hidden, path, opt)
        assert e.value.status == fa.ERR_SHAPE
        return
    plan = fa.describe_launch(n, m, hidden, path, opt)
    # automatic: two-stage for a few rows that each read a lot (R = 2 (n + 1) hidden bytes): up
    # to 48 rows from R = 512 KiB, 40 from 432 KiB, 16 from 336 KiB; else one-stage
    r = 2 * (n + 1) * hidden
    limit = 48 if r >= 512 * 1024 else 40 if r >= 432 * 1024 else 16 if r >= 336 * 1024 else -1
    want_path = path if path else (2 if m <= limit else 1)
    assert plan["path"] == want_path
    if m == 0:
        assert plan["kernels"] == []
        return
    ks = plan["kernels"]
    s1 = "stage1_reduce_lds" if stage1 else "stage1_reduce"
    chunk = m if rows in (0, -1) else min(rows, m)  # two-stage rows per chunk (auto: one chunk)
    if want_path == 2 and chunk < m:
        check_chunked_plan(ks, n, m, packs, stage1, block, rows=chunk, pipelined=sched == 2,
                           geometry=rows_geometry, stream=stream, capped=capped, s1=s1)
        return
    # two-stage: the residual add in stage 1 unless the LDS-staged stage 1 or chunks ask for the
    # pages' split (stage 1 into the scratch, stage 2 adds the residual)
    in_stage1 = not stage1 and rows <= 0
    two = ["stage1_reduce_residual", "stage2_rmsnorm"] if in_stage1 else [s1, "stage2_norm"]
    assert [k["name"] for k in ks] == {
        1: ["onestage"],
        2: two,
        3: [s1, "residual_add", "rmsnorm"]}[want_path]
    # the row kernel: one workgroup per row, whole waves, every pack of a row covered once
    k_rows = ks[-1]
    assert (k_rows["per_thread"], k_rows["block"]) == rows_geometry
    assert k_rows["grid"] == min(m, ROWS_PER_LAUNCH)
    assert k_rows["launches"] == -(-m // ROWS_PER_LAUNCH)
    assert k_rows["lds_bytes"] == (64 * 1024 if capped else 0)
    assert k_rows["streaming"] == int(stream)
    # the flat kernels: one pack per thread over all m * packs packs
    total = m * packs
    for k in ks[:-1]:
        want_block, want_grid = expected_flat(n, total, block, k["name"] == "stage1_reduce_lds")
        assert k["block"] == want_block and k["per_thread"] == 1
        assert k["grid"] == want_grid
        assert k["launches"] == -(-total // FLAT_PACKS_PER_LAUNCH)
        assert k["lds_bytes"] == 0 and k["streaming"] == int(stream)


def check_chunked_plan(ks, n, m, packs, stage1, block, rows, pipelined, geometry, stream, capped,
                       s1):
    """The two-stage path in chunks of `rows` rows (fewer than m): sequential, a flat reduce and a
    row launch per chunk; pipelined, the first chunk's reduce, one launch per chunk boundary
    holding the next chunk's reduce and this chunk's normalisation, and the last chunk's
    normalisation."""
    chunks = -(-m // rows)
    last = m - (chunks - 1) * rows
    flat_launches = lambda p: -(-p // FLAT_PACKS_PER_LAUNCH)  # noqa: E731
    names = [s1, "stage_pipe", "stage2_norm"] if pipelined else [s1, "stage2_norm"]
    assert [k["name"] for k in ks] == names
    want_block, want_grid = expected_flat(n, rows * packs, block, stage1)
    f = ks[0]
    assert (f["block"], f["grid"], f["per_thread"], f["lds_bytes"]) == (want_block, want_grid, 1, 0)
    assert f["streaming"] == int(stream)
    if pipelined:
        assert f["launches"] == flat_launches(rows * packs)
    else:
        assert f["launches"] == (chunks - 1) * flat_launches(rows * packs) + flat_launches(last * packs)
    for k in ks[1:]:
        assert (k["per_thread"], k["block"]) == geometry
        assert k["lds_bytes"] == (64 * 1024 if capped else 0) and k["streaming"] == int(stream)
    norm = ks[-1]
    if pipelined:
        pipe = ks[1]
        assert pipe["grid"] == rows + (last if chunks == 2 else rows)
        assert pipe["launches"] == chunks - 1
        assert (norm["grid"], norm["launches"]) == (last, 1)
    else:
        assert (norm["grid"], norm["launches"]) == (rows, chunks)
