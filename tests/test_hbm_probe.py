"""The HBM ceiling probes of the benchmark (libhbm_probe.so): argument checks on the CPU (no kernel is
launched), and on the GPU that each probe moves exactly the bytes it claims to (copy, XOR/add mix,
a mix's reads alone and its writes alone), so the ceilings the benchmark reports are measured on
correct streaming kernels."""
import ctypes
import os

import pytest
import torch  # before the probe library, so that it binds to torch's HIP runtime

import hbm_probe

VP = ctypes.c_void_p
FAKE = 0x7F0000000000  # aligned, never dereferenced: every call below is rejected before a launch


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(hbm_probe.LIBRARY):
        pytest.fail(f"{hbm_probe.LIBRARY} is not built")
    return hbm_probe.load()


def test_probe_arguments_rejected_before_launch(probe):
    assert probe.hbm_probe_read(None, 16, FAKE, 1, 8, 64, None) == -1
    assert probe.hbm_probe_read(FAKE, 0, FAKE, 1, 8, 64, None) == -1
    assert probe.hbm_probe_read(FAKE + 8, 16, FAKE, 1, 8, 64, None) == -1
    assert probe.hbm_probe_read(FAKE, 16, FAKE, 1, 3, 64, None) == -1   # unroll not 1, 4 or 8
    assert probe.hbm_probe_read(FAKE, 16, FAKE, 0, 8, 0, None) == -1    # empty grid
    assert probe.hbm_probe_read(FAKE, 16, FAKE, 4, 8, 64, None) == -1   # cache policy 0..3
    assert probe.hbm_probe_copy(FAKE, FAKE, 16, -1, 64, None) == -1
    assert probe.hbm_probe_copy(FAKE, None, 16, 1, 64, None) == -1
    assert probe.hbm_probe_copy(FAKE, FAKE, 16, 1, (1 << 20) + 1, None) == -1
    ins = (VP * 9)(*([FAKE] * 8 + [None]))
    outs = (VP * 2)(FAKE, FAKE)
    assert probe.hbm_probe_mix(ins, outs, 16, 1, 64, None) == -1
    ins = (VP * 9)(*([FAKE] * 9))
    outs = (VP * 2)(FAKE, FAKE + 4)
    assert probe.hbm_probe_mix(ins, outs, 16, 1, 64, None) == -1
    outs = (VP * 2)(FAKE, FAKE)
    assert probe.hbm_probe_mix_rw(ins, 4, outs, 1, 16, 1, 64, None) == -1   # 5 or 9 reads only
    assert probe.hbm_probe_mix_rw(ins, 9, outs, 3, 16, 1, 64, None) == -1   # 1 or 2 writes
    assert probe.hbm_probe_mix_rw(ins, 5, outs, 0, 16, 1, 64, None) == -1
    assert probe.hbm_probe_mix_rw(ins, 9, outs, 1, 0, 1, 64, None) == -1    # no packs
    ins = (VP * 9)(*([FAKE] * 4 + [None] + [FAKE] * 4))
    assert probe.hbm_probe_mix_rw(ins, 5, outs, 1, 16, 1, 64, None) == -1   # a null read stream
    ins = (VP * 9)(*([FAKE] * 9))
    assert probe.hbm_probe_reads(ins, 4, 16, FAKE, 1, 64, None) == -1       # 5 or 9 reads only
    assert probe.hbm_probe_reads(ins, 9, 16, None, 1, 64, None) == -1       # no sink
    assert probe.hbm_probe_reads(ins, 9, 16, FAKE + 4, 1, 64, None) == -1   # misaligned sink
    assert probe.hbm_probe_reads(ins, 9, 0, FAKE, 1, 64, None) == -1        # no packs
    assert probe.hbm_probe_reads(None, 9, 16, FAKE, 1, 64, None) == -1
    assert probe.hbm_probe_writes(outs, 0, 16, 2, 64, None) == -1           # 1 or 2 writes
    assert probe.hbm_probe_writes(outs, 3, 16, 2, 64, None) == -1
    assert probe.hbm_probe_writes(None, 2, 16, 2, 64, None) == -1
    assert probe.hbm_probe_writes(outs, 2, 16, 4, 64, None) == -1           # cache policy 0..3
    assert probe.hbm_probe_writes((VP * 2)(FAKE, FAKE + 8), 2, 16, 2, 64, None) == -1


@pytest.mark.gpu
def test_probes_move_the_bytes_they_claim(probe):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    print("[gpu case] HBM probes: read, copy, mix on 1 MiB streams", flush=True)
    stream = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device="cpu").manual_seed(11)
    packs = (1 << 20) // 16 + 3  # a ragged tail for the grid-stride loops
    words = packs * 4

    def rand_words():
        return torch.randint(-2**31, 2**31, (words,), generator=g, dtype=torch.int64) \
            .to(torch.int32).cuda()

    src = rand_words()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for nt in (0, 1):
        for unroll in (1, 4, 8):
            assert probe.hbm_probe_read(src.data_ptr(), packs, sink.data_ptr(), nt, unroll, 37,
                                        stream) == 0
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0  # random data never hits the fold's fixed pattern

    for nt in range(4):
        dst = torch.zeros_like(src)
        assert probe.hbm_probe_copy(src.data_ptr(), dst.data_ptr(), packs, nt, 37, stream) == 0
        torch.cuda.synchronize()
        assert torch.equal(dst, src)

    ins_t = [rand_words() for _ in range(9)]
    x = ins_t[0].clone()
    for t in ins_t[1:]:
        x = torch.bitwise_xor(x, t)
    want1 = (x.to(torch.int64) + ins_t[0].to(torch.int64)).remainder(2**32)
    for nt in range(4):
        outs_t = [torch.zeros_like(src) for _ in range(2)]
        ins = (VP * 9)(*[t.data_ptr() for t in ins_t])
        outs = (VP * 2)(*[t.data_ptr() for t in outs_t])
        assert probe.hbm_probe_mix(ins, outs, packs, nt, 37, stream) == 0
        torch.cuda.synchronize()
        assert torch.equal(outs_t[0], x)
        assert torch.equal(outs_t[1].to(torch.int64).remainder(2**32), want1)

    for reads in (5, 9):
        xr = ins_t[0].clone()
        for t in ins_t[1:reads]:
            xr = torch.bitwise_xor(xr, t)
        for writes in (1, 2):
            for nt in (1, 3):
                outs_t = [torch.zeros_like(src) for _ in range(2)]
                ins = (VP * reads)(*[t.data_ptr() for t in ins_t[:reads]])
                outs = (VP * writes)(*[t.data_ptr() for t in outs_t[:writes]])
                assert probe.hbm_probe_mix_rw(ins, reads, outs, writes, packs, nt, 37, stream) == 0
                torch.cuda.synchronize()
                assert torch.equal(outs_t[0], xr)
                if writes == 2:
                    want = (xr.to(torch.int64) + ins_t[0].to(torch.int64)).remainder(2**32)
                    assert torch.equal(outs_t[1].to(torch.int64).remainder(2**32), want)
                else:
                    assert not outs_t[1].any()  # the second stream is not written

    # a mix's reads alone write nothing; its writes alone write pack i of stream k as
    # {i, i >> 32, k, ~i}
    for reads in (5, 9):
        for nt in (0, 1):
            ins = (VP * reads)(*[t.data_ptr() for t in ins_t[:reads]])
            assert probe.hbm_probe_reads(ins, reads, packs, sink.data_ptr(), nt, 37, stream) == 0
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
    idx = torch.arange(packs, dtype=torch.int64)
    for writes in (1, 2):
        for nt in (0, 2):
            outs_t = [torch.zeros_like(src) for _ in range(2)]
            outs = (VP * writes)(*[t.data_ptr() for t in outs_t[:writes]])
            assert probe.hbm_probe_writes(outs, writes, packs, nt, 37, stream) == 0
            torch.cuda.synchronize()
            for k in range(2):
                got = outs_t[k].cpu().view(packs, 4).to(torch.int64).remainder(2**32)
                if k >= writes:
                    assert not got.any()  # a stream past `writes` is not touched
                    continue
                assert torch.equal(got[:, 0], idx)
                assert not got[:, 1].any()
                assert torch.equal(got[:, 2], torch.full_like(idx, k))
                assert torch.equal(got[:, 3], (~idx).remainder(2**32))
