"""GPU parity of decoding several new tokens per request (q_len > 1) against
the f64 oracle, at the same bounds as one-token decode.

New token j of a window of q_len sits at position n - q_len + j and sees
positions 0 .. n - q_len + j (the oracle's visible_len; pinned on the CPU by
brute force with an explicit mask, by closed-form counts and by needles).
Query rows are token-major (row j * H + h). The chooser keeps the policy split
at P = 1 for these requests (pure decode only) and tiles them for the device;
forced plans cover P > 1, and single pass covers the direct write.
"""
import numpy as np
import pytest

import absorbed_mla_paged_amd as mla
import mla_synth
import oracle
from oracle import reference

from gpu_helpers import check_sync_quiet, compare, log, rows_of_plan, run_case, to_device

pytestmark = pytest.mark.gpu


def small(seed, contexts, heads, dtype, q_len, **kw):
    return mla_synth.make_case(seed=seed, batch=len(contexts), heads=heads, contexts=contexts,
                               dtype=dtype, q_len=q_len, **kw)


def check(case, prm, fused=False, what=""):
    out, lse2, plan, ranges = run_case(case, mla.PlanParams(**prm), want_ranges=True, fused=fused)
    log(f"[plan] {what} q_len={case.q_len} P={plan.info['P']} S={plan.info['S']} "
        f"rows={plan.total_rows} groups={plan.info['groups']}")
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    compare(case, out, lse2, ref, lref, what, moments=mom)
    if plan.info["needs_reduce"] or plan.total_rows > case.batch:
        want = rows_of_plan(case, plan)
        got = [tuple(r) for r in ranges[:plan.total_rows]]
        assert got == [(lo, hi) for _, lo, hi in want]
    if fused:
        check_sync_quiet(plan, what)
    return plan


WORKLOADS = [
    ("v2lite_32k_q2", {}),
    ("v2lite_32k_q4", {}),
    ("v2lite_32k_q2", dict(force_partitions=2)),
    ("v2lite_32k_q2", dict(force_partitions=1, force_splits=1)),   # single pass, direct write
    ("v3_131k_q2", {}),
]


@pytest.mark.parametrize("name,prm", WORKLOADS,
                         ids=[f"{n}-{'-'.join(f'{k}{v}' for k, v in p.items()) or 'chooser'}"
                              for n, p in WORKLOADS])
def test_multitoken_workloads(name, prm):
    log(f"[case] multi-token workload {name} {prm}")
    case = mla_synth.make_workload(name, poison=True)
    plan = check(case, prm, what=f"{name} {prm}")
    if not prm:
        assert plan.info["P"] == [1]          # no policy split with several new tokens


EDGE = [
    ([2], 16, "f16", 4, dict(force_partitions=2)),          # first new tokens see nothing
    ([33, 1, 70], 32, "bf16", 3, dict(heads_per_wg=16)),
    ([31, 4000], 64, "f16", 3, {}),                          # 64-head workgroups
    ([5000], 128, "bf16", 2, dict(force_partitions=3, force_splits=2)),
    ([64], 16, "bf16", 8, dict(force_partitions=2, force_splits=2)),   # window = the last block
    ([3000], 128, "bf16", 8, {}),                            # the largest window: 1024 query rows
    ([1500, 700], 128, "f16", 8, dict(heads_per_wg=16)),     # the same in 16-head workgroups
]


@pytest.mark.parametrize("contexts,heads,dtype,q_len,prm", EDGE,
                         ids=[f"{c}-H{h}-{d}-q{q}-{p}" for c, h, d, q, p in EDGE])
def test_multitoken_edge_cases(contexts, heads, dtype, q_len, prm):
    log(f"[case] multi-token edge {contexts} H={heads} q_len={q_len} {prm}")
    case = small(900 + sum(contexts) % 83, contexts, heads, dtype, q_len, poison=True)
    check(case, prm, what=f"edge {contexts} H={heads} q={q_len}")


@pytest.mark.parametrize("heads,prm", [(16, dict(force_partitions=2, force_splits=3)),
                                       (64, dict(heads_per_wg=16, force_partitions=2))])
def test_multitoken_fused(heads, prm):
    case = small(950, [3000], heads, "f16", 2, poison=True)
    check(case, prm, fused=True, what=f"fused H={heads}")


def plant(case, b, t, row):
    phys = case.block_table[b, t // 32]
    sign = np.sign(reference.decode16(case.q_absorbed[b, row], case.dtype))
    sign[sign == 0] = 1
    case.ckv_pool[phys, t % 32] = mla_synth.encode16((6.0 * sign).astype(np.float32), case.dtype)
    case.kpe_pool[phys, t % 32] = mla_synth.encode16(np.zeros(64, np.float32), case.dtype)
    return reference.decode16(case.ckv_pool[phys, t % 32], case.dtype)


@pytest.mark.parametrize("heads,q_len", [(16, 3), (64, 2)])
def test_multitoken_window_boundary_needles(heads, q_len):
    # The token at position n - q_len + j is seen by new token j (found
    # exactly) and not by new token j - 1 (its output is unchanged).
    n = 2000
    prm = mla.PlanParams(force_partitions=2, force_splits=2)
    for j in range(1, q_len):
        t = n - q_len + j
        for row, seen in ((j * heads + 3, True), ((j - 1) * heads + 3, False)):
            case = small(960, [n], heads, "bf16", q_len)
            before, _, _, _ = run_case(case, prm)
            needle = plant(case, 0, t, row)
            after, _, _, _ = run_case(case, prm)
            if seen:
                assert np.max(np.abs(after[0, row] - needle)) < 1e-2, (j, row)
            else:
                assert np.array_equal(before[0, row], after[0, row]), (j, row)
