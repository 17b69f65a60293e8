"""GPU parity of the 64-head workgroups (head counts that 64 divides).

Same bounds as test_gpu_parity: max |gpu - ref| <= 1e-2, mean <= 1e-3, the
base-2 LSE within the derived bound, and the index math bit-exact. Also:
the second pass the kernel takes when a later block's maximum outgrows the
first block's by more than 2^15 (forced here by planting dominant tokens),
run-to-run and block-permutation bit identity, and the 16-head path forced
at 128 heads.
"""
import numpy as np
import pytest

import absorbed_mla_paged_amd as mla
import mla_synth
import oracle
from oracle import reference

from gpu_helpers import compare, compare_beyond_rounding, log, rows_of_plan, run_case, to_device

pytestmark = pytest.mark.gpu


def small(seed, contexts, heads=128, dtype="bf16", **kw):
    return mla_synth.make_case(seed=seed, batch=len(contexts), heads=heads, contexts=contexts,
                               dtype=dtype, **kw)


CASES = [
    ([1], 64, "f16", {}),
    ([31, 32, 33], 128, "bf16", {}),
    ([0, 100, 0], 128, "f16", {}),
    ([1000], 128, "bf16", dict(force_partitions=3)),
    ([5000, 70], 64, "bf16", dict(force_partitions=8, force_splits=3)),
    ([33], 128, "f16", dict(force_partitions=8, force_splits=16)),   # mostly empty rows
    ([4097, 1, 300], 128, "bf16", dict(num_cus=4096, min_tile_blocks=1)),
    ([20000], 128, "bf16", dict(force_partitions=1, force_splits=1)),  # one long row
    ([3000], 128, "bf16", dict(heads_per_wg=16)),                      # 16-head path
    ([3000, 129], 128, "f16", dict(heads_per_wg=64)),
]


@pytest.mark.parametrize("contexts,heads,dtype,prm", CASES,
                         ids=[f"{c}-H{h}-{d}-{p}" for c, h, d, p in CASES])
def test_wide_cases(contexts, heads, dtype, prm):
    log(f"[case] wide {contexts} H={heads} {dtype} {prm}")
    case = small(700 + sum(contexts) % 89, contexts, heads, dtype, poison=True)
    out, lse2, plan, ranges = run_case(case, mla.PlanParams(**prm), want_ranges=True)
    assert plan.info["heads_per_wg"] == prm.get("heads_per_wg", 64)
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    compare(case, out, lse2, ref, lref, f"wide {contexts} H={heads} {prm}", moments=mom)
    want = rows_of_plan(case, plan)
    if plan.total_rows > len(contexts) or any(p * s > 1 for p, s in zip(plan.info["P"],
                                                                      plan.info["S"])):
        got = [tuple(r) for r in ranges[:plan.total_rows]]
        assert got == [(lo, hi) for _, lo, hi in want]


def plant(case, b, t, h):
    phys = case.block_table[b, t // 32]
    sign = np.sign(reference.decode16(case.q_absorbed[b, h], case.dtype))
    sign[sign == 0] = 1
    case.ckv_pool[phys, t % 32] = mla_synth.encode16((6.0 * sign).astype(np.float32), case.dtype)
    case.kpe_pool[phys, t % 32] = mla_synth.encode16(np.zeros(64, np.float32), case.dtype)


@pytest.mark.parametrize("dtype,heads", [("bf16", 128), ("f16", 64)])
def test_wide_needles_and_second_pass(dtype, heads):
    # A dominant token at the first and last position of each row and at the
    # last visible token. Inside a row's first block it sets the reference;
    # in a later block it outgrows the reference by far more than 2^15 and
    # forces the second pass, for every head of the workgroup. The whole
    # output (not only the needle's head) must match the oracle.
    n = 4000
    prm = mla.PlanParams(force_partitions=3, force_splits=4)
    rows = oracle.row_ranges([n], [3], [4])
    spots = sorted({lo for _, lo, hi in rows if hi > lo} | {hi - 1 for _, lo, hi in rows if hi > lo})
    for i, t in enumerate(spots):
        case = small(81, [n], heads, dtype, poison=True)
        h = (37 * i) % heads
        plant(case, 0, t, h)
        out, lse2, _, _ = run_case(case, prm)
        needle = reference.decode16(case.ckv_pool[case.block_table[0, t // 32], t % 32], dtype)
        assert np.max(np.abs(out[0, h] - needle)) < 1e-2, (t, h)
        ref, lref = oracle.latent_f64(case)
        compare_beyond_rounding(case, out, lse2, ref, lref, f"needle t={t} h={h}")


def test_wide_run_to_run_and_permutation_bit_identical():
    case = small(93, [7000, 333], 128, "bf16")
    dev = to_device(case)
    prm = mla.PlanParams(force_partitions=2)
    a = run_case(case, prm, dev)
    b = run_case(case, prm, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    rng = np.random.default_rng(4)
    perm = rng.permutation(case.num_blocks)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    case.ckv_pool = np.ascontiguousarray(case.ckv_pool[inv])
    case.kpe_pool = np.ascontiguousarray(case.kpe_pool[inv])
    case.block_table = perm[case.block_table].astype(np.int32)
    c = run_case(case, prm)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])
