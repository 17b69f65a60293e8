"""GPU parity with 16-token cache blocks (the "block16" layout the review of
vllm-metal pull request 601 asks to see covered) against the f64 oracle, at
the same bounds as the 32-token layout.

Both partition kernels take the cache block size as a template parameter;
with 16-token blocks a 32-token segment of a row spans two blocks, looked
up separately in the table. Covered: the workloads stored in 16-token blocks
(16-head and 64-head workgroups, chooser and forced plans, single pass), the
kernel's row ranges bit for bit, edge cases around 16-token boundaries,
needles at every row boundary, several new tokens per request, the fused
launch, and bit-identity with the 32-token layout of the same tokens.
"""
import numpy as np
import pytest

import absorbed_mla_paged_amd as mla
import mla_synth
import oracle
from oracle import reference

from gpu_helpers import check_sync_quiet, compare, log, rows_of_plan, run_case

pytestmark = pytest.mark.gpu


def small(seed, contexts, heads=16, dtype="f16", **kw):
    return mla_synth.make_case(seed=seed, batch=len(contexts), heads=heads, contexts=contexts,
                               dtype=dtype, block_size=16, **kw)


def check(case, prm, fused=False, what=""):
    assert case.ckv_pool.shape[1] == 16
    out, lse2, plan, ranges = run_case(case, mla.PlanParams(**prm), want_ranges=True, fused=fused)
    log(f"[plan] {what} P={plan.info['P']} S={plan.info['S']} rows={plan.total_rows} "
        f"hpw={plan.info['heads_per_wg']} tile={plan.info['tile_blocks']}")
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    compare(case, out, lse2, ref, lref, what, moments=mom)
    if plan.total_rows > case.batch:
        want = rows_of_plan(case, plan)
        got = [tuple(r) for r in ranges[:plan.total_rows]]
        assert got == [(lo, hi) for _, lo, hi in want]
        assert all(lo % 16 == 0 for lo, hi in got if hi > lo)
    if fused:
        check_sync_quiet(plan, what)
    return out, lse2, plan


WORKLOADS = [
    ("tiny", dict(force_partitions=2, force_splits=1)),
    ("tiny", dict(force_partitions=2)),
    ("v2lite_32k", {}),
    ("v2lite_32k", dict(force_partitions=1, force_splits=1)),   # single pass
    ("two_req_32k_20k", {}),
    ("v3_81k", {}),                                             # 64-head workgroups
    ("mixed_b8", dict(workspace_limit_bytes=64 << 20)),
]


@pytest.mark.parametrize("name,prm", WORKLOADS,
                         ids=[f"{n}-{'-'.join(f'{k}{v}' for k, v in p.items()) or 'chooser'}"
                              for n, p in WORKLOADS])
def test_block16_workloads(name, prm):
    log(f"[case] block16 workload {name} {prm}")
    case = mla_synth.make_workload(name, poison=True, block_size=16)
    _, _, plan = check(case, prm, what=f"block16 {name} {prm}")
    if name == "v2lite_32k" and not prm:
        assert plan.info["P"] == [2]
    if name == "v3_81k":
        assert plan.info["P"] == [5] and plan.info["heads_per_wg"] == 64


EDGE = [
    ([1], 16, "f16", {}),
    ([15, 16, 17], 16, "bf16", {}),
    ([31, 32, 33, 47, 48, 49], 16, "f16", dict(force_partitions=3)),
    ([0, 100, 0], 16, "f16", dict(force_partitions=2)),
    ([33], 16, "f16", dict(force_partitions=8, force_splits=16)),    # many empty rows
    ([1000], 32, "bf16", dict(force_partitions=3, force_splits=5)),
    ([16], 64, "bf16", {}),
    ([17], 128, "f16", {}),
    ([40, 5000], 128, "bf16", dict(force_partitions=8, force_splits=3)),
    ([2000, 70], 64, "f16", dict(force_partitions=8)),
    ([4097, 1, 300], 128, "bf16", dict(num_cus=4096, min_tile_blocks=1)),
]


@pytest.mark.parametrize("contexts,heads,dtype,prm", EDGE,
                         ids=[f"{c}-H{h}-{d}-{p}" for c, h, d, p in EDGE])
def test_block16_edge_cases(contexts, heads, dtype, prm):
    log(f"[case] block16 edge {contexts} H={heads} {dtype} {prm}")
    case = small(700 + sum(contexts) % 89, contexts, heads, dtype, poison=True)
    check(case, prm, what=f"block16 edge {contexts} H={heads} {prm}")


def plant(case, b, t, h):
    phys = case.block_table[b, t // 16]
    sign = np.sign(reference.decode16(case.q_absorbed[b, h], case.dtype))
    sign[sign == 0] = 1
    case.ckv_pool[phys, t % 16] = mla_synth.encode16((6.0 * sign).astype(np.float32), case.dtype)
    case.kpe_pool[phys, t % 16] = mla_synth.encode16(np.zeros(64, np.float32), case.dtype)
    return reference.decode16(case.ckv_pool[phys, t % 16], case.dtype)


@pytest.mark.parametrize("heads,dtype", [(32, "f16"), (64, "bf16")])
def test_block16_needles_at_row_boundaries(heads, dtype):
    # A dominant token at the first and last position of every row must be
    # found; the rows start at 16-token boundaries that are not 32-aligned.
    n = 3000
    prm = mla.PlanParams(force_partitions=3, force_splits=5)
    rows = oracle.row_ranges([n], [3], [5], block_size=16)
    spots = sorted({lo for _, lo, hi in rows if hi > lo} | {hi - 1 for _, lo, hi in rows if hi > lo})
    assert any(t % 32 == 16 for t in spots)
    for i, t in enumerate(spots):
        case = small(79, [n], heads, dtype, poison=True)
        h = (7 * i) % heads
        needle = plant(case, 0, t, h)
        out, _, _, _ = run_case(case, prm)
        assert np.max(np.abs(out[0, h] - needle)) < 1e-2, (t, h)


@pytest.mark.parametrize("heads", [16, 128])
def test_block16_needle_past_context_end_is_ignored(heads):
    case = small(80, [1000], heads, "bf16")
    out0, l0, _, _ = run_case(case, mla.PlanParams(force_partitions=2))
    plant(case, 0, 1005, 3)   # 1000 % 16 = 8 visible rows in the last block
    out1, l1, _, _ = run_case(case, mla.PlanParams(force_partitions=2))
    assert np.array_equal(out0, out1) and np.array_equal(l0, l1)


@pytest.mark.parametrize("heads,q_len", [(16, 2), (16, 4), (128, 2)])
def test_block16_multitoken(heads, q_len):
    case = mla_synth.make_case(seed=81, batch=2, heads=heads, contexts=[3000, 49],
                               dtype="bf16", q_len=q_len, block_size=16, poison=True)
    check(case, {}, what=f"block16 q_len={q_len} H={heads}")
    check(case, dict(force_partitions=2), what=f"block16 q_len={q_len} H={heads} P=2")


@pytest.mark.parametrize("name,prm", [("v2lite_32k", {}), ("two_req_32k_20k", {}),
                                      ("tiny", dict(force_partitions=2))])
def test_block16_fused(name, prm):
    case = mla_synth.make_workload(name, poison=True, block_size=16)
    check(case, prm, fused=True, what=f"block16 fused {name} {prm}")


def relayout_16(case):
    """The same tokens stored as 16-token blocks: half i of 32-token block k
    moves to a fresh random position, and the table is rewritten."""
    pool32 = case.num_blocks
    ckv = case.ckv_pool.reshape(pool32 * 2, 16, 512)
    kpe = case.kpe_pool.reshape(pool32 * 2, 16, 64)
    perm = np.random.default_rng(9).permutation(pool32 * 2)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    table = np.empty((case.batch, case.max_blocks * 2), dtype=np.int32)
    table[:, 0::2] = perm[2 * case.block_table]
    table[:, 1::2] = perm[2 * case.block_table + 1]
    return mla_synth.Case(dtype=case.dtype, batch=case.batch, heads=case.heads,
                          context_lens=case.context_lens.copy(), block_table=table,
                          ckv_pool=np.ascontiguousarray(ckv[inv]),
                          kpe_pool=np.ascontiguousarray(kpe[inv]), q_absorbed=case.q_absorbed,
                          q_pe=case.q_pe, scale=case.scale, seed=case.seed, q_len=case.q_len,
                          block_size=16)


@pytest.mark.parametrize("heads,contexts,prm", [
    (16, [1024], dict(force_partitions=2, force_splits=1)),   # the same rows in both layouts
    (16, [5000, 333], dict(force_partitions=1, force_splits=1)),   # single pass
    (128, [4096], dict(force_partitions=4, force_splits=2)),
    (64, [777], dict(force_partitions=1, force_splits=1)),
])
def test_block16_bit_identical_to_block32(heads, contexts, prm):
    # Where both layouts give the same rows, each kernel reads the same
    # tokens in the same order, so the outputs are bit for bit the same.
    case = mla_synth.make_case(seed=82, batch=len(contexts), heads=heads, contexts=contexts,
                               dtype="bf16")
    c16 = relayout_16(case)
    r32 = oracle.row_ranges(case.context_lens, [prm["force_partitions"]] * case.batch,
                            [prm["force_splits"]] * case.batch)
    r16 = oracle.row_ranges(case.context_lens, [prm["force_partitions"]] * case.batch,
                            [prm["force_splits"]] * case.batch, block_size=16)
    assert r32 == r16
    a = run_case(case, mla.PlanParams(**prm))
    b = run_case(c16, mla.PlanParams(**prm))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
