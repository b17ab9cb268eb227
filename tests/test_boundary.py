"""The C-ABI boundary on the CPU: the library loads, exports every function include/fused_ar.h
declares, and rejects bad arguments with the documented codes before any HIP call (so none of
these tests needs a GPU; no test here launches a kernel)."""
import ctypes
import os
import re

import pytest

import all_reduce_residual_way_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fused_ar.h")

# Fake, 16-byte-aligned, non-overlapping "device addresses". Validation only compares them.
MB = 1 << 20


def addr(i):
    return 0x7F0000000000 + i * 1024 * MB


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fused_ar_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert {"fused_ar_rmsnorm", "fused_ar_rmsnorm_ex", "fused_ar_unfused_rmsnorm",
            "fused_ar_rmsnorm_check", "fused_ar_reduce", "fused_ar_auto_path",
            "fused_ar_auto_path_tp",
            "fused_ar_describe_launch", "fused_ar_describe_launch_ex",
            "fused_ar_strerror"} <= set(names)


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(fa.LIBRARY_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in fused_ar.h but not exported"


def test_header_constants_match_binding():
    with open(HEADER) as f:
        text = f.read()
    for name, value in [("FUSED_AR_OK", fa.OK), ("FUSED_AR_ERR_INVALID", fa.ERR_INVALID),
                        ("FUSED_AR_ERR_SHAPE", fa.ERR_SHAPE), ("FUSED_AR_ERR_ALIGN", fa.ERR_ALIGN),
                        ("FUSED_AR_ERR_ALIAS", fa.ERR_ALIAS), ("FUSED_AR_ERR_SCRATCH", fa.ERR_SCRATCH), ("FUSED_AR_PATH_AUTO", fa.PATH_AUTO),
                        ("FUSED_AR_PATH_ONESTAGE", fa.PATH_ONESTAGE),
                        ("FUSED_AR_PATH_TWOSTAGE", fa.PATH_TWOSTAGE),
                        ("FUSED_AR_PATH_UNFUSED", fa.PATH_UNFUSED),
                        ("FUSED_AR_WAVE_DPP", fa.WAVE_DPP), ("FUSED_AR_WAVE_BPERMUTE", fa.WAVE_BPERMUTE),
                        ("FUSED_AR_STAGE1_FLAT", fa.STAGE1_FLAT), ("FUSED_AR_STAGE1_LDS", fa.STAGE1_LDS),
                        ("FUSED_AR_LOAD_AUTO", fa.LOAD_AUTO), ("FUSED_AR_LOAD_CACHED", fa.LOAD_CACHED),
                        ("FUSED_AR_LOAD_STREAM", fa.LOAD_STREAM),
                        ("FUSED_AR_CHUNKS_AUTO", fa.CHUNKS_AUTO),
                        ("FUSED_AR_CHUNKS_SEQUENTIAL", fa.CHUNKS_SEQUENTIAL),
                        ("FUSED_AR_CHUNKS_PIPELINED", fa.CHUNKS_PIPELINED),
                        ("FUSED_AR_RESIDUAL_AUTO", fa.RESIDUAL_AUTO),
                        ("FUSED_AR_RESIDUAL_STAGE2", fa.RESIDUAL_STAGE2),
                        ("FUSED_AR_RESIDUAL_STAGE1", fa.RESIDUAL_STAGE1)]:
        assert re.search(rf"\b{name}\s*=\s*{value}\b", text), name
    assert re.search(rf"#define FUSED_AR_MAX_INPUTS {fa.MAX_INPUTS}\b", text)
    assert re.search(rf"#define FUSED_AR_MAX_HIDDEN {fa.MAX_HIDDEN}\b", text)
    assert re.search(rf"#define FUSED_AR_STATIC_SCRATCH_FLOATS {fa.STATIC_SCRATCH_FLOATS}\b", text)


def call(n=4, m=8, hidden=4096, eps=1e-6, path=1, inputs=None, residual=None, weight=None,
         residual_out=None, out=None, check_only=False):
    ins = inputs if inputs is not None else [addr(i) for i in range(n)]
    args = (ins, addr(10) if residual is None else residual, addr(11) if weight is None else weight,
            eps, m, hidden, addr(12) if residual_out is None else residual_out,
            addr(13) if out is None else out, path)
    if check_only:
        return fa.fused_ar_rmsnorm_check_ptrs(*args)
    return fa.fused_ar_rmsnorm_ptrs(*args, 0)


BAD_CALLS = [
    (dict(n=0), fa.ERR_INVALID),
    (dict(n=9), fa.ERR_INVALID),
    (dict(m=-1), fa.ERR_INVALID),
    (dict(hidden=0), fa.ERR_INVALID),
    (dict(hidden=-8), fa.ERR_INVALID),
    (dict(eps=-1e-6), fa.ERR_INVALID),
    (dict(eps=float("nan")), fa.ERR_INVALID),
    (dict(eps=float("inf")), fa.ERR_INVALID),
    (dict(path=3), fa.ERR_INVALID),
    (dict(path=-1), fa.ERR_INVALID),
    (dict(residual=0), fa.ERR_INVALID),
    (dict(weight=0), fa.ERR_INVALID),
    (dict(residual_out=0), fa.ERR_INVALID),
    (dict(out=0), fa.ERR_INVALID),
    (dict(inputs=[addr(0), 0, addr(2)]), fa.ERR_INVALID),
    (dict(hidden=4100), fa.ERR_SHAPE),
    (dict(hidden=32776), fa.ERR_SHAPE),
    (dict(inputs=[addr(0) + 8]), fa.ERR_ALIGN),
    (dict(residual=addr(10) + 2), fa.ERR_ALIGN),
    (dict(weight=addr(11) + 4), fa.ERR_ALIGN),
    (dict(residual_out=addr(12) + 8), fa.ERR_ALIGN),
    (dict(out=addr(13) + 1), fa.ERR_ALIGN),
    (dict(out=addr(1)), fa.ERR_ALIAS),                       # out == an input
    (dict(out=addr(10) + 4096), fa.ERR_ALIAS),               # out overlaps residual
    (dict(out=addr(11)), fa.ERR_ALIAS),                      # out overlaps weight
    (dict(out=addr(12)), fa.ERR_ALIAS),                      # out == residual_out
    (dict(residual_out=addr(2)), fa.ERR_ALIAS),              # residual_out == an input
    (dict(residual_out=addr(11) - 16), fa.ERR_ALIAS),        # residual_out overlaps weight
    (dict(residual_out=addr(10) + 16), fa.ERR_ALIAS),        # partial overlap with residual
    (dict(inputs=[0xFFFFFFFFFFFF0000]), fa.ERR_INVALID),     # range wraps the address space
]


@pytest.mark.parametrize("kwargs,code", BAD_CALLS)
def test_rejected_before_launch(kwargs, code):
    kwargs = dict(kwargs)
    kwargs.setdefault("n", len(kwargs["inputs"]) if "inputs" in kwargs else 4)
    assert call(**kwargs) == code
    assert call(check_only=True, **kwargs) == code


def test_valid_arguments_pass_the_check():
    assert call(check_only=True) == fa.OK
    for path in (0, 1, 2):
        assert call(check_only=True, n=8, m=8192, hidden=8192, path=path) == fa.OK
    # Allowed overlaps: inputs equal to each other, the weight inside an input (all read only),
    # and residual_out == residual (in place).
    assert call(check_only=True, n=3, inputs=[addr(0), addr(0), addr(1)], weight=addr(0),
                residual_out=addr(10)) == fa.OK
    # hidden at the maximum, eps == 0.
    assert call(check_only=True, hidden=32768, eps=0.0) == fa.OK


def test_m_zero_launches_nothing():
    # m == 0 returns success before any pointer is looked at (all null here).
    assert fa.fused_ar_rmsnorm_ptrs([0, 0], 0, 0, 1e-6, 0, 4096, 0, 0, fa.PATH_AUTO, 0) == fa.OK
    assert fa.fused_ar_reduce_ptrs([0, 0, 0], 0, 4096, 0, 0) == fa.OK


def test_reduce_checks():
    ins = [addr(i) for i in range(4)]
    assert fa.fused_ar_reduce_ptrs(ins, 8, 12, addr(20), 0) == fa.ERR_SHAPE
    assert fa.fused_ar_reduce_ptrs(ins, -1, 16, addr(20), 0) == fa.ERR_INVALID
    assert fa.fused_ar_reduce_ptrs([], 8, 16, addr(20), 0) == fa.ERR_INVALID
    assert fa.fused_ar_reduce_ptrs(ins, 8, 16, 0, 0) == fa.ERR_INVALID
    assert fa.fused_ar_reduce_ptrs(ins, 8, 16, addr(20) + 8, 0) == fa.ERR_ALIGN
    assert fa.fused_ar_reduce_ptrs(ins, 8, 16, addr(3), 0) == fa.ERR_ALIAS


def one_gpu_path(n, m, hidden):
    """The documented one-GPU rule: with R = 2 (n + 1) hidden bytes read per row, two-stage for
    m <= 48 when R >= 512 KiB, m <= 40 when R >= 432 KiB, m <= 16 when R >= 336 KiB; else
    one-stage."""
    r = 2 * (n + 1) * hidden
    limit = 48 if r >= 512 * 1024 else 40 if r >= 432 * 1024 else 16 if r >= 336 * 1024 else -1
    return fa.PATH_TWOSTAGE if m <= limit else fa.PATH_ONESTAGE


def test_auto_path_rule():
    for n in range(1, 9):
        for hidden in (8, 2880, 4096, 7168, 16384, 19112, 19120, 21496, 21504, 24568, 24576,
                       27648, 28672, 29120, 29128, 32768):
            for m in (0, 1, 15, 16, 17, 31, 32, 33, 39, 40, 41, 47, 48, 49, 4096):
                assert fa.auto_path(n, m, hidden) == one_gpu_path(n, m, hidden), (n, m, hidden)
    # the rule's corners at n = 8: 24576 reads exactly 432 KiB, 29128 is the first width over 512
    assert fa.auto_path(8, 40, 24576) == fa.PATH_TWOSTAGE
    assert fa.auto_path(8, 41, 24576) == fa.PATH_ONESTAGE
    assert fa.auto_path(8, 40, 24568) == fa.PATH_ONESTAGE
    assert fa.auto_path(8, 16, 24568) == fa.PATH_TWOSTAGE
    assert fa.auto_path(8, 48, 32768) == fa.PATH_TWOSTAGE
    assert fa.auto_path(8, 49, 32768) == fa.PATH_ONESTAGE
    assert fa.auto_path(4, 1, 32768) == fa.PATH_ONESTAGE    # 320 KiB per row
    assert fa.auto_path(8, 1, 7168) == fa.PATH_ONESTAGE
    for bad in ((0, 1, 4096), (9, 1, 4096), (4, -1, 4096), (4, 1, 0), (4, 1, -8)):
        assert fa.auto_path(*bad) == fa.ERR_INVALID, bad


def test_pages_path_rule_for_tensor_parallel_groups():
    # One-stage up to m = 32 for n <= 4 and up to m = 16 for n > 4, whatever the row width.
    for n in range(1, 9):
        limit = 32 if n <= 4 else 16
        for hidden in (4096, 32768):
            assert fa.auto_path_tp(n, 0, hidden) == fa.PATH_ONESTAGE
            assert fa.auto_path_tp(n, limit, hidden) == fa.PATH_ONESTAGE
            assert fa.auto_path_tp(n, limit + 1, hidden) == fa.PATH_TWOSTAGE
    assert fa.auto_path_tp(0, 1, 4096) == fa.ERR_INVALID
    assert fa.auto_path_tp(9, 1, 4096) == fa.ERR_INVALID
    assert fa.auto_path_tp(4, -1, 4096) == fa.ERR_INVALID


@pytest.mark.parametrize("hidden", [8, 512, 520, 2880, 4096, 7168, 8192, 8200, 16384, 32768])
def test_launch_geometry_covers_each_row(hidden):
    packs = hidden // 8
    for path in (1, 2):
        plan = fa.describe_launch(8, 100, hidden, path)
        rows = plan["kernels"][-1]
        assert rows["name"] == ("onestage" if path == 1 else "stage2_rmsnorm")
        assert rows["grid"] == 100
        assert rows["block"] % 64 == 0 and 64 <= rows["block"] <= 1024
        assert rows["block"] * rows["per_thread"] >= packs
        assert rows["block"] * rows["per_thread"] - packs < 64 * rows["per_thread"]
        if path == 2:
            flat = plan["kernels"][0]
            assert flat["name"] == "stage1_reduce_residual" and flat["block"] == 256
            assert flat["grid"] * flat["block"] * flat["per_thread"] >= 100 * packs


def test_launch_geometry_by_row_count():
    # calls from the caches: one pack per thread, except two for 256 < m <= 1024 on rows wider
    # than 512 packs; long streaming calls (two workgroups per CU): one pack per thread below 512
    # packs, two up to 1024, four above; rows come in launches of at most 2^20 workgroups
    k = fa.describe_launch(8, 256, 7168, 1)["kernels"][0]
    assert (k["per_thread"], k["block"], k["launches"]) == (1, 896, 1)
    k = fa.describe_launch(8, 257, 7168, 1)["kernels"][0]
    assert (k["per_thread"], k["block"]) == (2, 448)
    k = fa.describe_launch(8, 1024, 7168, 1)["kernels"][0]
    assert (k["per_thread"], k["block"]) == (2, 448)
    k = fa.describe_launch(8, 1025, 7168, 1)["kernels"][0]
    assert (k["per_thread"], k["block"]) == (1, 896)
    k = fa.describe_launch(8, 4096, 16384, 1)["kernels"][0]
    assert (k["per_thread"], k["block"], k["lds_bytes"]) == (4, 512, 64 * 1024)
    k = fa.describe_launch(8, 4096, 2880, 1)["kernels"][0]
    assert (k["per_thread"], k["block"], k["lds_bytes"]) == (1, 384, 64 * 1024)
    for m, hidden, want in ((4096, 7168, (2, 448)), (2048, 7168, (2, 448)), (4096, 4096, (2, 256)),
                            (8192, 8192, (2, 512)), (4096, 3584, (1, 448)), (4096, 32768, (4, 1024))):
        k = fa.describe_launch(8, m, hidden, 1)["kernels"][0]
        assert (k["per_thread"], k["block"]) == want, (m, hidden)
    # the same call forced to ordinary loads reads as a cached call: not capped, one pack
    k = fa.describe_launch(8, 4096, 7168, 1, fa.Options(0, 0, 0, 0, fa.LOAD_CACHED))["kernels"][0]
    assert (k["per_thread"], k["block"], k["lds_bytes"]) == (1, 896, 0)
    k = fa.describe_launch(2, (1 << 20) + 3, 8, 2)["kernels"][1]
    assert (k["grid"], k["launches"]) == (1 << 20, 2)


def test_launch_geometry_auto_and_empty():
    assert fa.describe_launch(8, 17, 7168)["path"] == 1
    assert fa.describe_launch(8, 48, 32768)["path"] == 2
    assert fa.describe_launch(8, 49, 32768)["path"] == 1
    assert fa.describe_launch(4, 0, 7168, 1)["kernels"] == []
    with pytest.raises(fa.FusedArError):
        fa.describe_launch(4, 8, 12, 1)


def test_strerror():
    assert fa.strerror(fa.OK) == "success"
    for code in (fa.ERR_INVALID, fa.ERR_SHAPE, fa.ERR_ALIGN, fa.ERR_ALIAS, fa.ERR_SCRATCH):
        assert fa.strerror(code) and fa.strerror(code) != "unknown status"
    assert fa.strerror(-99) == "unknown status"


def test_binding_rejects_bad_tensors_without_a_gpu():
    import torch
    x = torch.zeros(4, 16, dtype=torch.bfloat16)  # CPU tensors: rejected before any call
    with pytest.raises(ValueError):
        fa.fused_ar_rmsnorm([x], x, torch.zeros(16, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        fa.fused_ar_rmsnorm([x.float()], x, torch.zeros(16, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fa.fused_ar_rmsnorm([], x, x[0])
    for call in (fa.fused_ar_unfused_rmsnorm, fa.fused_ar_rmsnorm_split):
        with pytest.raises(ValueError):
            call([x], x, torch.zeros(16, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fa.fused_ar_reduce([x])


def test_stream_of_another_device_rejected():
    # the kernels run on the stream's device, so a stream of another device than the tensors' is
    # refused before anything is enqueued (checked here with stand-ins: no GPU is needed)
    import types

    import torch
    cuda0, cuda1 = torch.device("cuda", 0), torch.device("cuda", 1)
    fa._check_stream(None, cuda0)
    fa._check_stream(types.SimpleNamespace(device=torch.device("cuda:0")), cuda0)
    with pytest.raises(ValueError, match="stream is on cuda:1"):
        fa._check_stream(types.SimpleNamespace(device=cuda1), cuda0)


def test_options_struct_matches_header():
    with open(HEADER) as f:
        text = f.read()
    body = re.search(r"typedef struct \{(.*?)\} fused_ar_options;", text, re.S).group(1)
    fields = re.findall(r"int (\w+);", body)
    assert fields == [name for name, _ in fa.Options._fields_]


@pytest.mark.parametrize("opts", [
    fa.Options(2, 0, 0, 0), fa.Options(-1, 0, 0, 0), fa.Options(0, 2, 0, 0),
    fa.Options(0, 0, 32, 0), fa.Options(0, 0, 100, 0), fa.Options(0, 0, 2048, 0),
    fa.Options(0, 0, 0, 3), fa.Options(0, 0, 0, 8), fa.Options(0, 0, 0, 0, 3),
    fa.Options(0, 0, 0, 0, -1), fa.Options(0, 0, 0, 0, 0, -2), fa.Options(0, 0, 0, 0, 0, (1 << 20) + 1),
    fa.Options(0, 0, 0, 0, 0, 0, 3), fa.Options(0, 0, 0, 0, 0, 0, -1),
    fa.Options(0, 0, 0, 0, 0, 0, 0, 3), fa.Options(0, 0, 0, 0, 0, 0, 0, -1),
    fa.Options(0, fa.STAGE1_LDS, 0, 0, 0, 0, 0, fa.RESIDUAL_STAGE1),
    fa.Options(0, 0, 0, 0, 0, 512, 0, fa.RESIDUAL_STAGE1)])
def test_bad_options_rejected_before_launch(opts):
    ins = [addr(i) for i in range(4)]
    rc = fa.fused_ar_rmsnorm_ex_ptrs(ins, addr(10), addr(11), 1e-6, 8, 4096, addr(12), addr(13),
                                     1, opts, 0)
    assert rc == fa.ERR_INVALID
    with pytest.raises(fa.FusedArError):
        fa.describe_launch(4, 8, 4096, 1, opts)


def test_option_plans():
    k = fa.describe_launch(8, 100, 7168, 2, fa.Options(0, fa.STAGE1_LDS, 0, 0))["kernels"]
    assert k[0]["name"] == "stage1_reduce_lds" and k[0]["block"] == 512
    assert k[0]["grid"] * 512 >= 100 * 896
    k = fa.describe_launch(4, 100, 7168, 2, fa.Options(0, 0, 512, 0))["kernels"]
    assert k[0]["block"] == 512 and k[0]["grid"] == (100 * 896 + 511) // 512
    k = fa.describe_launch(8, 100, 7168, 1, fa.Options(0, 0, 0, 4))["kernels"]
    assert (k[0]["per_thread"], k[0]["block"]) == (4, 256)
    # a forced packs-per-thread that leaves the row needing more than 1024 threads
    with pytest.raises(fa.FusedArError) as e:
        fa.describe_launch(8, 100, 16384, 1, fa.Options(0, 0, 0, 1))
    assert e.value.status == fa.ERR_SHAPE


def test_chunked_two_stage_plans():
    """The two-stage path in chunks of rows: per chunk a flat reduce and a row launch
    (sequential), or the first chunk's reduce, one launch per chunk boundary, the last chunk's
    normalisation (pipelined). The one-stage path ignores the chunk options."""
    def plan(m, rows, schedule, n=4, hidden=7168, path=2):
        ks = fa.describe_launch(n, m, hidden, path,
                                fa.Options(0, 0, 0, 0, 0, rows, schedule))["kernels"]
        return [(k["name"], k["grid"], k["block"], k["per_thread"], k["launches"]) for k in ks]
    seq, pipe = fa.CHUNKS_SEQUENTIAL, fa.CHUNKS_PIPELINED
    # 4096 rows of 896 packs: 448 threads, two packs each (a long streaming call)
    assert plan(4096, 512, seq) == [("stage1_reduce", 512 * 896 // 256, 256, 1, 8),
                                    ("stage2_norm", 512, 448, 2, 8)]
    assert plan(4096, 512, pipe) == [("stage1_reduce", 512 * 896 // 256, 256, 1, 1),
                                     ("stage_pipe", 1024, 448, 2, 7),
                                     ("stage2_norm", 512, 448, 2, 1)]
    # a ragged last chunk: 4096 = 3000 + 1096
    assert plan(4096, 3000, seq)[1] == ("stage2_norm", 3000, 448, 2, 2)
    assert plan(4096, 3000, pipe)[1:] == [("stage_pipe", 4096, 448, 2, 1),
                                          ("stage2_norm", 1096, 448, 2, 1)]
    # chunks of 2^20 packs and more take the larger flat workgroup
    assert plan(8192, 1024, seq, n=8, hidden=8192)[0] == ("stage1_reduce", 2048, 512, 1, 8)
    # one chunk (rows >= m) is the plain two-stage plan in the pages' split (chunks exist only in
    # it; -1 asks for one chunk and leaves the split to the library); path 1 ignores the options
    pages = [(k["name"], k["grid"], k["block"], k["per_thread"], k["launches"])
             for k in fa.describe_launch(4, 4096, 7168, 2,
                                         fa.Options(0, 0, 0, 0, 0, 0, 0, fa.RESIDUAL_STAGE2))["kernels"]]
    assert plan(4096, 4096, pipe) == pages
    assert [k[0] for k in pages] == ["stage1_reduce", "stage2_norm"]
    assert [k[0] for k in plan(4096, -1, seq)] == ["stage1_reduce_residual", "stage2_rmsnorm"]
    whole = plan(4096, 0, 0)
    assert plan(4096, 512, pipe, path=1) == plan(4096, 0, 0, path=1)


def test_residual_stage_plans():
    """Where the two-stage path adds the residual: by default (and asked) in stage 1, a flat
    reduce + residual kernel over all packs then the plain RMSNorm row kernel; in the pages' split
    a flat reduce into the scratch then the row kernel that adds the residual; the same grids and
    geometry either way. The LDS-staged stage 1 and chunks of rows take the pages' split; other
    paths ignore the option."""
    stage1 = fa.Options(0, 0, 0, 0, 0, 0, 0, fa.RESIDUAL_STAGE1)
    pages = fa.Options(0, 0, 0, 0, 0, 0, 0, fa.RESIDUAL_STAGE2)
    k = fa.describe_launch(8, 4096, 7168, 2, stage1)["kernels"]
    assert [x["name"] for x in k] == ["stage1_reduce_residual", "stage2_rmsnorm"]
    assert fa.describe_launch(8, 4096, 7168, 2)["kernels"] == k
    assert [x["name"] for x in fa.describe_launch(8, 4096, 7168, 2, fa.Options(0, fa.STAGE1_LDS, 0, 0))["kernels"]] == \
        ["stage1_reduce_lds", "stage2_norm"]
    whole = fa.describe_launch(8, 4096, 7168, 2, pages)["kernels"]
    assert [x["name"] for x in whole] == ["stage1_reduce", "stage2_norm"]
    for a, b in zip(k, whole):
        assert (a["grid"], a["block"], a["per_thread"], a["launches"], a["lds_bytes"]) == \
            (b["grid"], b["block"], b["per_thread"], b["launches"], b["lds_bytes"])
    for opt in (stage1, pages):
        assert fa.describe_launch(8, 4096, 7168, 1, opt) == fa.describe_launch(8, 4096, 7168, 1)
        assert fa.describe_launch(4, 100, 2880, fa.PATH_UNFUSED, opt) == \
            fa.describe_launch(4, 100, 2880, fa.PATH_UNFUSED)


def test_unfused_plan_and_checks():
    plan = fa.describe_launch(8, 4096, 7168, fa.PATH_UNFUSED)
    assert plan["path"] == fa.PATH_UNFUSED
    assert [k["name"] for k in plan["kernels"]] == ["stage1_reduce", "residual_add", "rmsnorm"]
    # the row geometry of the RMSNorm kernel is the one-stage kernel's (identical reduction tree)
    one = fa.describe_launch(8, 4096, 7168, 1)["kernels"][0]
    assert (plan["kernels"][2]["block"], plan["kernels"][2]["per_thread"]) == \
        (one["block"], one["per_thread"])
    ins = [addr(i) for i in range(4)]
    assert fa.fused_ar_unfused_rmsnorm_ptrs(ins, addr(10), addr(11), 1e-6, 8, 4100, addr(12),
                                            addr(13)) == fa.ERR_SHAPE
    assert fa.fused_ar_unfused_rmsnorm_ptrs(ins, addr(10), addr(11), 1e-6, 8, 4096, addr(12),
                                            addr(1)) == fa.ERR_ALIAS
    assert fa.fused_ar_unfused_rmsnorm_ptrs([0], 0, 0, 1e-6, 0, 4096, 0, 0) == fa.OK
    # the plain entry point does not take the unfused path id
    assert fa.fused_ar_rmsnorm_ptrs(ins, addr(10), addr(11), 1e-6, 8, 4096, addr(12), addr(13),
                                    fa.PATH_UNFUSED, 0) == fa.ERR_INVALID


def test_automatic_load_policy():
    """Ordinary loads while a call reads at most 128 MiB (inputs + residual), non-temporal above;
    the same choice for every kernel of a call; forced by the option."""
    def streaming(n, m, hidden, path=1, opt=None):
        return [k["streaming"] for k in fa.describe_launch(n, m, hidden, path, opt)["kernels"]]
    limit = 128 << 20
    for n, hidden in [(8, 7168), (4, 7168), (8, 2880), (1, 8192)]:
        per_row = 2 * (n + 1) * hidden
        m_max = limit // per_row
        assert streaming(n, m_max, hidden) == [0]
        assert streaming(n, m_max + 1, hidden) == [1]
        assert streaming(n, m_max + 1, hidden, 2) == [1, 1]
        assert streaming(n, m_max, hidden, fa.PATH_UNFUSED) == [0, 0, 0]
    assert streaming(8, 4096, 7168, 1, fa.Options(0, 0, 0, 0, fa.LOAD_CACHED)) == [0]
    assert streaming(8, 8, 7168, 1, fa.Options(0, 0, 0, 0, fa.LOAD_STREAM)) == [1]


def split_call(n=4, m=8, hidden=4096, eps=1e-6, inputs=None, residual=None, weight=None,
               residual_out=None, out=None, splits=0, workspace=None, workspace_bytes=None):
    ins = inputs if inputs is not None else [addr(i) for i in range(n)]
    need = fa.split_workspace_bytes(m, hidden, splits)
    return fa.fused_ar_rmsnorm_split_ptrs(
        ins, addr(10) if residual is None else residual, addr(11) if weight is None else weight,
        eps, m, hidden, addr(12) if residual_out is None else residual_out,
        addr(13) if out is None else out, splits, addr(14) if workspace is None else workspace,
        need if workspace_bytes is None else workspace_bytes, 0)


@pytest.mark.parametrize("kwargs,code", [c for c in BAD_CALLS if "path" not in c[0]] + [
    (dict(splits=65), fa.ERR_INVALID),
    (dict(splits=-1), fa.ERR_INVALID),
    (dict(hidden=16384, splits=1), fa.ERR_SHAPE),             # 2048 packs in one slice
    (dict(workspace=0), fa.ERR_INVALID),
    (dict(workspace_bytes=8 * 2 * 4 - 4), fa.ERR_INVALID),   # one float short (2 slices of 256)
    (dict(workspace=addr(14) + 4), fa.ERR_ALIGN),
    (dict(workspace=addr(13) + 64), fa.ERR_ALIAS),           # inside out
    (dict(workspace=addr(2)), fa.ERR_ALIAS),                 # inside an input
    (dict(workspace=addr(11)), fa.ERR_ALIAS),                # the weight
    (dict(workspace=addr(10) + 4096), fa.ERR_ALIAS),         # inside the residual
    (dict(workspace=addr(12)), fa.ERR_ALIAS),                # residual_out
])
def test_split_rejected_before_launch(kwargs, code):
    kwargs = dict(kwargs)
    kwargs.setdefault("n", len(kwargs["inputs"]) if "inputs" in kwargs else 4)
    assert split_call(**kwargs) == code


def test_split_workspace_and_slices():
    # one slice per 256 packs unless given; never more slices than packs; at most 64
    assert fa.split_workspace_bytes(1, 7168) == 4 * 4
    assert fa.split_workspace_bytes(5, 32768) == 5 * 16 * 4
    assert fa.split_workspace_bytes(3, 520) == 3 * 1 * 4
    assert fa.split_workspace_bytes(2, 7168, 7) == 2 * 7 * 4
    assert fa.split_workspace_bytes(1, 8, 3) == 4          # one pack: one slice
    assert fa.split_workspace_bytes(1, 7168, 64) == 64 * 4
    assert fa.split_workspace_bytes(1, 7168, 65) == 0
    assert fa.split_workspace_bytes(0, 7168) == 0
    assert fa.split_workspace_bytes(1, 16384, 1) == 0      # a slice would need 2048 threads
    assert fa.split_workspace_bytes(1, 12) == 0            # hidden not a multiple of 8
    # m == 0: success before any pointer is looked at
    assert fa.fused_ar_rmsnorm_split_ptrs([0], 0, 0, 1e-6, 0, 4096, 0, 0, 0, 0, 0, 0) == fa.OK


def static_split_call(n=4, m=8, hidden=4096, eps=1e-6, splits=0, **bufs):
    ins = bufs.get("inputs", [addr(i) for i in range(n)])
    return fa.fused_ar_rmsnorm_split_static_ptrs(
        ins, bufs.get("residual", addr(10)), bufs.get("weight", addr(11)), eps, m, hidden,
        bufs.get("residual_out", addr(12)), bufs.get("out", addr(13)), splits, 0)


@pytest.mark.parametrize("kwargs,code", [
    (dict(m=16385, hidden=7168), fa.ERR_SCRATCH),        # 4 slices: 65540 square-sums
    (dict(m=1025, hidden=8192, splits=64), fa.ERR_SCRATCH),
    (dict(m=4097, hidden=32768), fa.ERR_SCRATCH),        # 16 slices
    (dict(m=(1 << 31) - 1, hidden=32768, splits=64), fa.ERR_ALIAS),  # planes overlap first
    (dict(splits=65), fa.ERR_INVALID),
    (dict(hidden=16384, splits=1), fa.ERR_SHAPE),
    (dict(n=0), fa.ERR_INVALID),
    (dict(eps=-1.0), fa.ERR_INVALID),
    (dict(hidden=4100), fa.ERR_SHAPE),
    (dict(out=addr(2)), fa.ERR_ALIAS),
    (dict(residual_out=addr(12) + 8), fa.ERR_ALIGN),
    (dict(weight=0), fa.ERR_INVALID),
])
def test_static_split_rejected_before_launch(kwargs, code):
    """The static-scratch split call checks like the workspace form, then rejects calls whose slice
    square-sums exceed the static scratch, all before any HIP call."""
    assert static_split_call(**kwargs) == code


def test_static_split_limit_and_empty_call():
    # m == 0: success with nothing looked at; the limit is m * slices, slices as the workspace
    # form counts them
    assert static_split_call(m=0, inputs=[0], residual=0, weight=0, residual_out=0, out=0) == fa.OK
    assert fa.split_workspace_bytes(16384, 7168) == 4 * fa.STATIC_SCRATCH_FLOATS
    assert fa.split_workspace_bytes(4096, 32768) == 4 * fa.STATIC_SCRATCH_FLOATS
    assert "static scratch" in fa.strerror(fa.ERR_SCRATCH)


def test_launch_plan_struct_matches_header():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    body = re.search(r"typedef struct \{(.*?)\} fused_ar_kernel_launch;", text, re.S).group(1)
    fields = re.findall(r"(?:unsigned|char) (\w+)", body)
    assert fields == [name for name, _ in fa._KernelLaunch._fields_]


def test_row_workgroups_capped_on_long_streaming_calls():
    # LDS reserved on the row kernel (two workgroups per CU) only when the call streams from HBM
    # and has more rows than the two-pack band; never on the flat kernels
    def lds(n, m, hidden, path=1, opt=None):
        return [k["lds_bytes"] for k in fa.describe_launch(n, m, hidden, path, opt)["kernels"]]
    assert lds(8, 4096, 7168) == [64 * 1024]
    assert lds(8, 24576, 2880) == [64 * 1024]
    assert lds(8, 4096, 7168, 2) == [0, 64 * 1024]
    assert lds(8, 4096, 7168, fa.PATH_UNFUSED) == [0, 0, 64 * 1024]
    assert lds(8, 1000, 2880) == [0]                      # reads under 128 MiB: cached, no cap
    assert lds(8, 1024, 8192) == [0]                      # streams, but within the two-pack band
    assert lds(8, 1025, 8192) == [64 * 1024]
    assert lds(8, 32, 7168) == [0]
    assert lds(8, 4096, 7168, 1, fa.Options(0, 0, 0, 0, fa.LOAD_CACHED)) == [0]


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every entry point raises; nothing falls back to other code."""
    import torch
    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(fa, "LIBRARY_PATH", str(tmp_path / "libfused_ar.so"))
    with pytest.raises(RuntimeError, match="not built"):
        fa.library()
    with pytest.raises(RuntimeError, match="not built"):
        fa.auto_path(8, 1, 7168)
    x = torch.zeros(4, 16, dtype=torch.bfloat16)
    with pytest.raises((RuntimeError, ValueError)):  # CPU tensors: rejected, never computed
        fa.fused_ar_rmsnorm([x], x, torch.zeros(16, dtype=torch.bfloat16))


def test_one_hip_runtime_per_process():
    """Loading the library in a fresh process that has not imported torch, then using torch, leaves
    a single HIP runtime mapped (torch's): two runtimes in one process cannot both open the GPU."""
    import ast
    import subprocess
    import sys
    code = ("import all_reduce_residual_way_amd as fa; fa.library(); import torch; "
            "maps = open('/proc/self/maps').read(); "
            "print(sorted({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr
    runtimes = ast.literal_eval(r.stdout.strip().splitlines()[-1])
    assert len(runtimes) == 1, runtimes
