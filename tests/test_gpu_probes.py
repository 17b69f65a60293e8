"""The two measurement helpers the benchmark times its kernels against:
mla_stream_read (a plain read that writes nothing unless its fold equals a
value the data never folds to) and mla_copy_probe (the partition kernels'
LDS copies alone). They return no result, so the checks are that every
launch shape the benchmark uses runs to completion, leaves its inputs
unchanged, and that the stream read's sink is never written.
"""
import pytest

import absorbed_mla_paged_amd as mla

from gpu_helpers import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (37 << 20) + 48])
def test_stream_read_leaves_sink(nbytes):
    import torch
    log(f"[case] stream read of {nbytes} bytes")
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 1 << 30, (nbytes // 4,), dtype=torch.int32, device="cuda",
                        generator=g)
    before = src.clone()
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    mla.mla_stream_read(src, sink)
    torch.cuda.synchronize()
    # Every word is below 2^30, so every XOR fold of them is too and never
    # equals 0xA5A5A5A5: nothing may have been written.
    assert int(src.max().item()) < (1 << 30)
    assert sink.cpu().tolist() == [7, 7, 7, 7]
    assert torch.equal(src, before)


# (rows, blocks per row, groups, waves, inflight): the benchmark's shapes at
# a small byte count, plus a row count that is not a multiple of 8 and
# four workgroups per row.
SHAPES = [(256, 2, 1, 8, 8), (128, 4, 2, 8, 8), (128, 4, 2, 4, 4), (256, 2, 1, 4, 16),
          (13, 3, 2, 8, 16), (5, 2, 4, 4, 8)]


@pytest.mark.parametrize("rows,blocks,groups,waves,inflight", SHAPES,
                         ids=[f"r{r}b{b}g{g}w{w}i{i}" for r, b, g, w, i in SHAPES])
def test_copy_probe_runs(rows, blocks, groups, waves, inflight):
    import torch
    log(f"[case] copy probe rows={rows} blocks={blocks} groups={groups} waves={waves} "
        f"inflight={inflight}")
    nblk = rows * blocks + 3
    g = torch.Generator(device="cuda").manual_seed(rows * 100 + blocks)
    ckv = torch.randn((nblk, 32, 512), device="cuda", generator=g).to(torch.bfloat16)
    kpe = torch.randn((nblk, 32, 64), device="cuda", generator=g).to(torch.bfloat16)
    table = torch.randperm(nblk, device="cuda", generator=g)[:rows * blocks].to(torch.int32)
    c0, k0 = ckv.clone(), kpe.clone()
    mla.mla_copy_probe(ckv, kpe, table, rows, blocks, groups, waves=waves, inflight=inflight)
    torch.cuda.synchronize()
    assert torch.equal(ckv, c0) and torch.equal(kpe, k0)
