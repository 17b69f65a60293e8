"""mla_decode_noalloc (partials in the library's fixed device scratch)
against the two-launch path with caller workspace (mla_decode_partition +
mla_decode_reduce): bit-identical output and LSE, on consecutive calls whose
second input is smaller than the first, so the second call runs over what
the first left in the scratch.
"""
import numpy as np
import pytest

import absorbed_mla_paged_amd as mla
import mla_synth

from gpu_helpers import log, to_device, torch_dtype

pytestmark = pytest.mark.gpu


def both_paths(case, params=None):
    import torch
    dev = to_device(case)
    plan = mla.DecodePlan(case.context_lens, case.heads, params)
    shape = (case.batch, case.heads, 512)
    ref_out = torch.empty(shape, dtype=torch_dtype(case.dtype), device="cuda")
    ref_lse = torch.empty(shape[:2], dtype=torch.float32, device="cuda")
    mla.decode(plan, dev["q_absorbed"], dev["q_pe"], dev["ckv_cache"], dev["kpe_cache"],
               dev["block_table"], dev["context_lens"], case.scale, ref_out, ref_lse)
    out = torch.full(shape, 3.0, dtype=torch_dtype(case.dtype), device="cuda")
    lse = torch.full(shape[:2], 3.0, dtype=torch.float32, device="cuda")
    mla.mla_decode_noalloc(dev["q_absorbed"], dev["q_pe"], dev["ckv_cache"], dev["kpe_cache"],
                           dev["block_table"], dev["context_lens"], case.scale, plan.partitions,
                           plan.splits, plan.row_indptr, plan.total_rows,
                           plan.info["max_rows_per_req"], plan.info["heads_per_wg"], out, lse)
    torch.cuda.synchronize()
    log(f"[noalloc] B={case.batch} H={case.heads} rows={plan.total_rows} "
        f"scratch={mla.mla_noalloc_scratch_bytes(plan.total_rows, case.heads)} bytes")
    return (ref_out.cpu(), ref_lse.cpu()), (out.cpu(), lse.cpu()), plan


def assert_identical(ref, got):
    import torch
    assert torch.equal(ref[0].view(torch.int16), got[0].view(torch.int16))
    assert torch.equal(ref[1], got[1])


def test_noalloc_matches_workspace_path_on_consecutive_calls():
    # First call: 128 heads (64-head workgroups), 81920 tokens, 128 rows.
    big = mla_synth.make_workload("v3_81k", poison=True)
    ref, got, plan = both_paths(big)
    assert plan.total_rows > 1
    assert_identical(ref, got)
    # Second call, smaller: two requests of 16 heads (16-head workgroups),
    # fewer rows, over the scratch the first call filled.
    small = mla_synth.make_workload("two_req_32k_20k", poison=True)
    ref2, got2, plan2 = both_paths(small)
    assert 1 < plan2.total_rows * small.heads < plan.total_rows * big.heads
    assert_identical(ref2, got2)
    # And the first shape again, after the smaller one.
    ref3, got3, _ = both_paths(big)
    assert_identical(ref3, got3)
    assert_identical(ref, ref3)


def test_noalloc_single_pass_and_empty_requests():
    case = mla_synth.make_case(seed=404, batch=3, heads=16, contexts=[0, 700, 33],
                               dtype="f16", poison=True)
    ref, got, plan = both_paths(case, mla.PlanParams(force_partitions=1, force_splits=1))
    assert plan.total_rows == 3
    assert_identical(ref, got)
    ref, got, plan = both_paths(case, mla.PlanParams(force_partitions=4))
    assert plan.total_rows > 3
    assert_identical(ref, got)
    assert np.all(got[1][0].numpy() == -np.inf)


def test_noalloc_refuses_plans_beyond_its_scratch():
    import torch
    case = mla_synth.make_case(seed=405, batch=1, heads=128, contexts=[4096], dtype="bf16")
    dev = to_device(case)
    plan = mla.DecodePlan(case.context_lens, case.heads,
                          mla.PlanParams(force_partitions=8, force_splits=64, min_tile_blocks=1))
    assert mla.mla_noalloc_scratch_bytes(plan.total_rows, 128) > mla.NOALLOC_SCRATCH_BYTES
    out = torch.zeros((1, 128, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_noalloc(dev["q_absorbed"], dev["q_pe"], dev["ckv_cache"],
                               dev["kpe_cache"], dev["block_table"], dev["context_lens"],
                               case.scale, plan.partitions, plan.splits, plan.row_indptr,
                               plan.total_rows, plan.info["max_rows_per_req"],
                               plan.info["heads_per_wg"], out)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert torch.all(out == 0)
