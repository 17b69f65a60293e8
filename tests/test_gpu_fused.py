"""GPU parity of the fused launch (mla_decode_fused: partition and merge in
one launch) against the f64 oracle, at the same bounds as the two-launch
path, plus the hand-off state it leaves behind.

The cases cover: the workloads with 16-head workgroups; requests whose rows
are all empty; many empty rows; head groups G > 1; grids larger than the
device (workgroups that start late cannot wait, so the last arrival merges
their pieces); more rows per request than the merge's 64 row lanes x 4
(two-batch pieces); the same hand-off buffer reused by different plans.
"""
import numpy as np
import pytest

import absorbed_mla_paged_amd as mla
import mla_synth
import oracle
from oracle import reference

from gpu_helpers import check_sync_quiet, compare, log, rows_of_plan, run_case, to_device

pytestmark = pytest.mark.gpu


def small(seed, contexts, heads=16, dtype="f16", **kw):
    return mla_synth.make_case(seed=seed, batch=len(contexts), heads=heads, contexts=contexts,
                               dtype=dtype, **kw)


FUSED_WORKLOADS = [
    ("tiny", dict(force_partitions=2, force_splits=1)),
    ("tiny", dict(force_partitions=2)),
    ("v2lite_32k", {}),
    ("v2lite_32k", dict(force_partitions=1, force_splits=1)),   # single pass: no merge
    ("two_req_32k_32k", {}),
    ("two_req_32k_20k", {}),
    # 8 requests x 128 heads as eight 16-head groups each, bounded workspace.
    ("mixed_b8", dict(heads_per_wg=16, workspace_limit_bytes=64 << 20)),
]


@pytest.mark.parametrize("name,prm", FUSED_WORKLOADS,
                         ids=[f"{n}-{'-'.join(f'{k}{v}' for k, v in p.items()) or 'chooser'}"
                              for n, p in FUSED_WORKLOADS])
def test_fused_workload_parity(name, prm):
    log(f"[case] fused workload {name} {prm}")
    case = mla_synth.make_workload(name, poison=True)
    out, lse2, plan, ranges = run_case(case, mla.PlanParams(**prm), want_ranges=True, fused=True)
    log(f"[plan] P={plan.info['P']} S={plan.info['S']} rows={plan.total_rows}")
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    compare(case, out, lse2, ref, lref, f"fused {name} {prm}", moments=mom)
    want = rows_of_plan(case, plan)
    got = [tuple(r) for r in ranges[:plan.total_rows]]
    assert got == [(lo, hi) for _, lo, hi in want]
    check_sync_quiet(plan, name)


FUSED_EDGE = [
    ([1], 16, "f16", dict(force_partitions=2)),                     # one token, one empty row
    ([31, 32, 33], 16, "bf16", dict(force_partitions=2)),
    ([0, 100, 0], 16, "f16", dict(force_partitions=2)),              # requests with nothing visible
    ([33], 16, "f16", dict(force_partitions=8, force_splits=16)),    # 128 rows, most empty
    ([1000], 32, "bf16", dict(force_partitions=3, heads_per_wg=16)),  # two head groups
    ([4097, 1, 300], 48, "bf16", dict(num_cus=4096, min_tile_blocks=1)),   # grid > device
    ([32768], 16, "f16", dict(force_partitions=8, force_splits=75)),  # 600 rows per request
    ([65536 + 17], 16, "bf16", {}),
]


@pytest.mark.parametrize("contexts,heads,dtype,prm", FUSED_EDGE,
                         ids=[f"{c}-H{h}-{d}-{p}" for c, h, d, p in FUSED_EDGE])
def test_fused_edge_cases(contexts, heads, dtype, prm):
    log(f"[case] fused edge {contexts} H={heads} {dtype} {prm}")
    case = small(700 + sum(contexts) % 89, contexts, heads, dtype, poison=True)
    out, lse2, plan, ranges = run_case(case, mla.PlanParams(**prm), want_ranges=True, fused=True)
    log(f"[plan] P={plan.info['P']} S={plan.info['S']} rows={plan.total_rows}")
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    compare(case, out, lse2, ref, lref, f"fused edge {contexts} H={heads} {prm}", moments=mom)
    want = rows_of_plan(case, plan)
    got = [tuple(r) for r in ranges[:plan.total_rows]]
    assert got == [(lo, hi) for _, lo, hi in want]
    check_sync_quiet(plan, f"{contexts}")


def plant(case, b, t, h):
    phys = case.block_table[b, t // 32]
    sign = np.sign(reference.decode16(case.q_absorbed[b, h], case.dtype))
    sign[sign == 0] = 1
    case.ckv_pool[phys, t % 32] = mla_synth.encode16((6.0 * sign).astype(np.float32), case.dtype)
    case.kpe_pool[phys, t % 32] = mla_synth.encode16(np.zeros(64, np.float32), case.dtype)


def test_fused_needles_at_row_boundaries():
    # A dominant token at the first and last position of each row must come
    # through the in-launch merge exactly.
    n = 4000
    prm = mla.PlanParams(force_partitions=3, force_splits=4)
    plan_rows = oracle.row_ranges([n], [3], [4])
    spots = sorted({lo for _, lo, hi in plan_rows if hi > lo} |
                   {hi - 1 for _, lo, hi in plan_rows if hi > lo})
    for i, t in enumerate(spots):
        case = small(79, [n], 16, "bf16", poison=True)
        h = (5 * i) % 16
        plant(case, 0, t, h)
        out, _, plan, _ = run_case(case, prm, fused=True)
        needle = reference.decode16(case.ckv_pool[case.block_table[0, t // 32], t % 32], "bf16")
        assert np.max(np.abs(out[0, h] - needle)) < 1e-2, (t, h)
        check_sync_quiet(plan, f"needle {t}")


def test_fused_run_to_run_bit_identical_and_close_to_two_launches():
    case = mla_synth.make_workload("two_req_32k_20k")
    dev = to_device(case)
    a = run_case(case, None, dev, fused=True)
    b = run_case(case, None, dev, fused=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = run_case(case, None, dev)   # partition + reduce launches
    d = np.abs(a[0] - c[0])
    log(f"[fused vs two launches] max {d.max():.3e}")
    assert d.max() <= 1e-2 and np.max(np.abs(a[1] - c[1])) <= 1e-5


def test_fused_sync_buffer_reused_across_plans():
    # One hand-off buffer, three plans of different row counts in a row: each
    # result matches the oracle and the records are left consistent.
    import torch
    case = small(83, [9000, 2500], 16, "f16", poison=True)
    dev = to_device(case)
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    plans = [mla.DecodePlan(case.context_lens, 16, mla.PlanParams(**p)) for p in
             (dict(force_partitions=2, force_splits=7), dict(force_partitions=5),
              dict(force_partitions=2, force_splits=7))]
    shared = plans[0].sync
    for i, plan in enumerate(plans):
        plan.sync = shared
        out = torch.empty((2, 16, 512), dtype=torch.float16, device="cuda")
        lse2 = torch.empty((2, 16), dtype=torch.float32, device="cuda")
        mla.decode(plan, dev["q_absorbed"], dev["q_pe"], dev["ckv_cache"], dev["kpe_cache"],
                   dev["block_table"], dev["context_lens"], case.scale, out, lse2, fused=True)
        torch.cuda.synchronize()
        compare(case, out.float().cpu().numpy().astype(np.float64),
                lse2.cpu().numpy().astype(np.float64), ref, lref, f"plan {i} rows {plan.total_rows}",
                moments=mom)
        check_sync_quiet(plan, f"plan {i}")


def test_fused_path_counters():
    case = small(5, [40000], 16, "f16")
    dev = to_device(case)
    mla.mla_reset_counters()
    run_case(case, None, dev, fused=True)
    c = mla.mla_get_counters()
    assert c[0] == 0 and c[1] == 1 and c[2] == 0 and c[3] >= 2
