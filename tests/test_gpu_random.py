"""GPU parity over seeded random configurations against the f64 oracle.

Each case draws, from one fixed seed: the batch (1-4), the head count (16 to
128, a multiple of 16), per-request contexts (zero, 16- and 32-token block
edges, or uniform up to 12K), new tokens per request (1-4), the cache block
size (16 or 32), the 16-bit type, the cache storage (16-bit or E4M3 bytes),
the plan (chooser, forced P and S, a workspace limit) and, for 16-bit caches
with 16-head workgroups, the fused launch. Every case is checked at the
acceptance bounds and its row ranges bit for bit; the cases complement the
hand-picked ones in the other files with combinations nobody chose.
"""
import numpy as np
import pytest
import torch

import absorbed_mla_paged_amd as mla
import mla_synth
import oracle

from gpu_helpers import check_sync_quiet, compare, log, rows_of_plan, run_case, to_device

pytestmark = pytest.mark.gpu

N_CASES = 96


def draw_case(i):
    rng = np.random.default_rng(9000 + i)
    batch = int(rng.integers(1, 5))
    heads = int(rng.choice([16, 32, 48, 64, 128]))
    bs = int(rng.choice([16, 32]))
    q_len = int(rng.choice([1, 1, 1, 2, 4]))
    dtype = str(rng.choice(["f16", "bf16"]))
    fp8 = bool(rng.random() < 0.3)
    ctx = []
    for _ in range(batch):
        kind = rng.integers(0, 4)
        if kind == 0:
            ctx.append(int(rng.choice([0, 1, 15, 16, 17, 31, 32, 33])))
        elif kind == 1:
            ctx.append(int(rng.integers(1, 40)) * 16 + int(rng.choice([-1, 0, 1])))
        else:
            ctx.append(int(rng.integers(1, 12288)))
    ctx = [max(0, c) for c in ctx]
    prm = {}
    mode = rng.integers(0, 4)
    if mode == 1:
        prm = dict(force_partitions=int(rng.integers(1, 9)), force_splits=int(rng.integers(1, 6)))
    elif mode == 2:
        prm = dict(workspace_limit_bytes=int(rng.choice([1 << 20, 8 << 20])))
    elif mode == 3:
        prm = dict(num_cus=int(rng.choice([64, 512, 2048])), min_tile_blocks=1)
    if fp8:
        # E4M3 runs in both workgroup shapes: 64 heads where 64 divides the
        # head count in every other case, else 16.
        prm["heads_per_wg"] = 64 if heads % 64 == 0 and i % 2 == 0 else 16
    elif rng.random() < 0.3:
        prm["heads_per_wg"] = 16
    fused = (not fp8 and prm.get("heads_per_wg", 16 if heads % 64 else 64) == 16
             and q_len * heads <= 128 and rng.random() < 0.4)
    kw = dict(kv_dtype="fp8_e4m3", kv_scale=float(2.0 ** -int(rng.integers(3, 7)))) if fp8 else {}
    case = mla_synth.make_case(seed=9000 + i, batch=batch, heads=heads, contexts=ctx, dtype=dtype,
                               q_len=q_len, block_size=bs, poison=True, **kw)
    return case, prm, fused


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    case, prm, fused = draw_case(i)
    what = (f"random {i}: B={case.batch} H={case.heads} ctx={list(case.context_lens)} "
            f"q_len={case.q_len} bs={case.block_size} {case.dtype} kv={case.kv_dtype} "
            f"{prm} fused={fused}")
    log(f"[case] {what}")
    dev = to_device(case)
    if case.kv_dtype:
        dev["ckv_cache"] = torch.from_numpy(case.ckv_pool).cuda()
        dev["kpe_cache"] = torch.from_numpy(case.kpe_pool).cuda()
        dev["kv_scale"] = case.kv_scale
    out, lse2, plan, ranges = run_case(case, mla.PlanParams(**prm), dev=dev, want_ranges=True,
                                       fused=fused)
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    compare(case, out, lse2, ref, lref, what, moments=mom)
    if plan.total_rows > case.batch:
        want = rows_of_plan(case, plan)
        got = [tuple(r) for r in ranges[:plan.total_rows]]
        assert got == [(lo, hi) for _, lo, hi in want]
    if fused and plan.info["needs_reduce"]:
        check_sync_quiet(plan, what)
