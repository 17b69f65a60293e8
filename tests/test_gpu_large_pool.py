"""Cache pools larger than 4 GiB: every block a request reads sits past the
first 4 GiB of the pool, so the kernels' block addressing must be 64-bit.

The small seeded case gives the oracle's answer. On the device its blocks are
copied to block indices from BASE on, in a pool of BASE + pool blocks (the
rest of the pool is left unwritten and is never read), and the block table
is shifted by BASE. Both partition kernels (16 and 64 heads), both block
sizes and the E4M3 cache (in both kernels) are covered. A second test runs launches of several
hundred requests, more workgroups than the chip holds at once.
"""
import numpy as np
import pytest
import torch

import absorbed_mla_paged_amd as mla
import mla_synth
import oracle

from gpu_helpers import compare, log, run_case, to_device

pytestmark = pytest.mark.gpu

GIB = 1 << 30


@pytest.mark.parametrize("heads,block_size,fp8", [(16, 32, False), (128, 32, False),
                                                  (64, 16, False), (32, 32, True),
                                                  (128, 16, True)])
def test_blocks_past_4_gib(heads, block_size, fp8):
    kw = dict(kv_dtype="fp8_e4m3", kv_scale=2.0 ** -5) if fp8 else {}
    case = mla_synth.make_case(seed=901, batch=2, heads=heads, contexts=[5000, 2999],
                               dtype="bf16", block_size=block_size, poison=True, **kw)
    elem = 1 if fp8 else 2
    block_bytes = block_size * 512 * elem
    base = (4 * GIB) // block_bytes + 1000          # first block past 4 GiB
    nblk = base + case.num_blocks
    log(f"[case] large pool H={heads} bs={block_size} fp8={fp8}: {nblk} blocks, "
        f"{nblk * block_bytes / GIB:.2f} GiB of ckv")
    dev = to_device(case)
    small_ckv = torch.from_numpy(case.ckv_pool).cuda() if fp8 else dev["ckv_cache"]
    small_kpe = torch.from_numpy(case.kpe_pool).cuda() if fp8 else dev["kpe_cache"]
    ckv = torch.empty((nblk,) + tuple(small_ckv.shape[1:]), dtype=small_ckv.dtype, device="cuda")
    kpe = torch.empty((nblk,) + tuple(small_kpe.shape[1:]), dtype=small_kpe.dtype, device="cuda")
    ckv[base:] = small_ckv
    kpe[base:] = small_kpe
    assert ckv[base:].data_ptr() - ckv.data_ptr() > 4 * GIB
    dev["ckv_cache"], dev["kpe_cache"] = ckv, kpe
    dev["block_table"] = torch.from_numpy(case.block_table.astype(np.int64) + base).to(
        torch.int32).cuda()
    if fp8:
        dev["kv_scale"] = case.kv_scale
    prm = mla.PlanParams(force_partitions=2, heads_per_wg=16 if fp8 and heads % 64 else 0)
    out, lse2, plan, _ = run_case(case, prm, dev=dev)
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    compare(case, out, lse2, ref, lref, f"large pool H={heads} bs={block_size} fp8={fp8}", moments=mom)
    del ckv, kpe
    torch.cuda.empty_cache()


@pytest.mark.parametrize("batch,heads,block_size,fp8", [(600, 16, 32, False), (160, 128, 16, False),
                                                        (300, 32, 32, True)])
def test_large_batch(batch, heads, block_size, fp8):
    # Many requests: the launch is not small, so the policy splits nothing
    # (P = 1), and the grid holds more workgroups than the chip runs at once.
    kw = dict(kv_dtype="fp8_e4m3", kv_scale=2.0 ** -5) if fp8 else {}
    case = mla_synth.make_case(seed=902 + batch, batch=batch, heads=heads,
                               context_range=(0, 2000), dtype="f16", block_size=block_size,
                               poison=True, **kw)
    log(f"[case] large batch B={batch} H={heads} bs={block_size} fp8={fp8}")
    dev = to_device(case)
    if fp8:
        dev["ckv_cache"] = torch.from_numpy(case.ckv_pool).cuda()
        dev["kpe_cache"] = torch.from_numpy(case.kpe_pool).cuda()
        dev["kv_scale"] = case.kv_scale
    prm = mla.PlanParams(heads_per_wg=16 if fp8 else 0)
    out, lse2, plan, _ = run_case(case, prm, dev=dev)
    workgroups = plan.total_rows * plan.info["groups"]
    log(f"[plan] P max {max(plan.info['P'])}, rows {plan.total_rows}, {workgroups} workgroups")
    assert max(plan.info["P"]) == 1 and workgroups > 256
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    compare(case, out, lse2, ref, lref, f"large batch B={batch} H={heads} bs={block_size}", moments=mom)
