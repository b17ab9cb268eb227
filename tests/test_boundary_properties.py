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
