"""Decode captured in a HIP graph and replayed: every replay must equal the
eager result, with eager work and synchronisations between replays. The
launches record no memset, and the fused launch's hand-off state carries
over from one replay to the next with nothing cleared in between, so these
replays are the test that it does."""
import numpy as np
import pytest

import absorbed_mla_paged_amd as mla
import mla_synth

from gpu_helpers import check_sync_quiet, log, to_device, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,fused,q_len", [("v2lite_32k", False, 1), ("v2lite_32k", True, 1),
                                              ("two_req_32k_20k", True, 1),
                                              ("v3_81k", False, 1), ("tiny", False, 2)])
def test_graph_replays_equal_eager(name, fused, q_len):
    import torch
    case = mla_synth.make_workload(name, q_len=q_len) if q_len > 1 else mla_synth.make_workload(name)
    dev = to_device(case)
    plan = mla.DecodePlan(case.context_lens, case.heads, mla.PlanParams(force_partitions=2)
                          if name == "tiny" else None, q_len=q_len)
    rows = q_len * case.heads
    out = torch.empty((case.batch, rows, 512), dtype=torch_dtype(case.dtype), device="cuda")
    lse = torch.empty((case.batch, rows), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def step():
        mla.decode(plan, dev["q_absorbed"], dev["q_pe"], dev["ckv_cache"], dev["kpe_cache"],
                   dev["block_table"], dev["context_lens"], case.scale, out, lse,
                   stream=stream, fused=fused)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    eager_out, eager_lse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(7.0)
        lse.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out) and torch.equal(lse, eager_lse), (name, fused, i)
        # eager work between replays, on the same plan and buffers
        with torch.cuda.stream(stream):
            step()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out)
    if fused:
        check_sync_quiet(plan, name)
    log(f"[graph] {name} fused={fused} q_len={q_len}: 4 replays equal the eager result")


@pytest.mark.parametrize("name,block_size,fp8", [("v2lite_32k", 16, False), ("v3_81k", 16, False),
                                                 ("v2lite_32k", 32, True),
                                                 ("two_req_32k_20k", 16, True),
                                                 ("v3_81k", 32, True)])
def test_graph_replays_equal_eager_cache_layouts(name, block_size, fp8):
    # 16-token blocks and E4M3 byte caches (16- and 64-head workgroups),
    # captured and replayed the same way.
    import torch
    kw = dict(kv_dtype="fp8_e4m3", kv_scale=2.0 ** -5) if fp8 else {}
    case = mla_synth.make_workload(name, block_size=block_size, **kw)
    dev = to_device(case)
    if fp8:
        dev["ckv_cache"] = torch.from_numpy(case.ckv_pool).cuda()
        dev["kpe_cache"] = torch.from_numpy(case.kpe_pool).cuda()
    plan = mla.DecodePlan(case.context_lens, case.heads, None, block_size=block_size)
    out = torch.empty((case.batch, case.heads, 512), dtype=torch_dtype(case.dtype), device="cuda")
    lse = torch.empty((case.batch, case.heads), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def step():
        mla.decode(plan, dev["q_absorbed"], dev["q_pe"], dev["ckv_cache"], dev["kpe_cache"],
                   dev["block_table"], dev["context_lens"], case.scale, out, lse,
                   stream=stream, kv_scale=case.kv_scale)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    eager_out, eager_lse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(7.0)
        lse.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out) and torch.equal(lse, eager_lse), (name, i)
        with torch.cuda.stream(stream):
            step()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_out)
    log(f"[graph] {name} block {block_size} fp8={fp8}: 4 replays equal the eager result")
