"""GPU parity: the HIP path through the C ABI against the f64 oracle.

Bounds: max |gpu - ref| <= 1e-2 and mean |gpu - ref| <= 1e-3 on the 512-wide
latent output; the base-2 LSE within the bound derived in gpu_helpers; the
partition index math bit-exact (debug ranges written by the kernel).
"""
import numpy as np
import pytest

import absorbed_mla_paged_amd as mla
import mla_synth
import oracle
from oracle import reference

from gpu_helpers import compare, device_cus, log, rows_of_plan, run_case, to_device

pytestmark = pytest.mark.gpu


def small(seed, contexts, heads=16, dtype="f16", **kw):
    return mla_synth.make_case(seed=seed, batch=len(contexts), heads=heads, contexts=contexts,
                               dtype=dtype, **kw)


# --- the five workloads (full size; chooser plans) ---------------------------

WORKLOAD_PLANS = [
    ("tiny", dict(force_partitions=2, force_splits=1)),   # 2 partitions of 512 tokens
    ("tiny", dict(force_partitions=2)),                    # 2 partitions, device-tiled
    ("v2lite_32k", {}),                                    # chooser (P = 2)
    ("v2lite_32k", dict(force_partitions=1, force_splits=1)),  # single pass
    ("two_req_32k_32k", {}),
    ("two_req_32k_20k", {}),
    ("v3_81k", {}),                                        # P = 5
    ("v3_131k", {}),                                       # P = 8
    ("mixed_b8", dict(workspace_limit_bytes=64 << 20)),    # P_b in 1..8, bounded workspace
]


@pytest.mark.parametrize("name,prm", WORKLOAD_PLANS,
                         ids=[f"{n}-{'-'.join(f'{k}{v}' for k, v in p.items()) or 'chooser'}"
                              for n, p in WORKLOAD_PLANS])
def test_workload_parity(name, prm):
    log(f"[case] workload {name} {prm}")
    case = mla_synth.make_workload(name, poison=True)
    out, lse2, plan, ranges = run_case(case, mla.PlanParams(**prm), want_ranges=True)
    log(f"[plan] P={plan.info['P']} S={plan.info['S']} rows={plan.total_rows}")
    if name == "tiny" and prm.get("force_splits") == 1:
        assert plan.info["P"] == [2] and plan.info["S"] == [1]
    if name == "v2lite_32k" and not prm:
        assert plan.info["P"] == [2]
    if name == "v3_81k":
        assert plan.info["P"] == [5]
    if name == "v3_131k":
        assert plan.info["P"] == [8]
    if name == "mixed_b8":
        assert all(1 <= p <= 8 for p in plan.info["P"])
        assert plan.info["partial_out_bytes"] + plan.info["partial_lse_bytes"] <= 64 << 20
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    compare(case, out, lse2, ref, lref, f"{name} {prm}", moments=mom)
    want = rows_of_plan(case, plan)
    got = [tuple(r) for r in ranges[:plan.total_rows]]
    assert got == [(lo, hi) for _, lo, hi in want]


# --- edge cases ----------------------------------------------------------------

EDGE = [
    ([1], 16, "f16", {}),
    ([31, 32, 33], 16, "bf16", {}),
    ([0, 100, 0], 16, "f16", {}),
    ([0], 16, "bf16", {}),
    ([1000], 32, "bf16", dict(force_partitions=3)),
    ([2000, 70], 64, "f16", dict(force_partitions=8)),
    ([40, 5000], 128, "bf16", dict(force_partitions=8, force_splits=3)),
    ([33], 16, "f16", dict(force_partitions=8, force_splits=16)),   # many empty rows
    ([4097, 1, 300], 48, "bf16", dict(num_cus=4096, min_tile_blocks=1)),
    ([65536 + 17], 16, "bf16", {}),
]


@pytest.mark.parametrize("contexts,heads,dtype,prm", EDGE,
                         ids=[f"{c}-H{h}-{d}-{p}" for c, h, d, p in EDGE])
def test_edge_cases(contexts, heads, dtype, prm):
    log(f"[case] edge {contexts} H={heads} {dtype} {prm}")
    case = small(500 + sum(contexts) % 97, contexts, heads, dtype, poison=True)
    out, lse2, plan, ranges = run_case(case, mla.PlanParams(**prm), want_ranges=True)
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    compare(case, out, lse2, ref, lref, f"edge {contexts} H={heads} {prm}", moments=mom)
    want = rows_of_plan(case, plan)
    if plan.total_rows > len(contexts) or any(p * s > 1 for p, s in zip(plan.info["P"], plan.info["S"])):
        got = [tuple(r) for r in ranges[:plan.total_rows]]
        assert got == [(lo, hi) for _, lo, hi in want]


# --- needles at every range boundary -------------------------------------------

def plant(case, b, t, h):
    phys = case.block_table[b, t // 32]
    sign = np.sign(reference.decode16(case.q_absorbed[b, h], case.dtype))
    sign[sign == 0] = 1
    case.ckv_pool[phys, t % 32] = mla_synth.encode16((6.0 * sign).astype(np.float32), case.dtype)
    case.kpe_pool[phys, t % 32] = mla_synth.encode16(np.zeros(64, np.float32), case.dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_needles_at_row_boundaries(dtype):
    # A dominant token at the first and last position of each row (and the
    # last visible token) must be found exactly; one just past the context
    # end must not show.
    n = 4000
    prm = mla.PlanParams(force_partitions=3, force_splits=4)
    base = small(77, [n], 32, dtype, poison=True)
    plan_rows = oracle.row_ranges([n], [3], [4])
    spots = sorted({lo for _, lo, hi in plan_rows if hi > lo} |
                   {hi - 1 for _, lo, hi in plan_rows if hi > lo})
    dev = None
    for i, t in enumerate(spots):
        case = small(77, [n], 32, dtype, poison=True)
        h = (7 * i) % 32
        plant(case, 0, t, h)
        out, lse2, _, _ = run_case(case, prm)
        needle = reference.decode16(case.ckv_pool[case.block_table[0, t // 32], t % 32], dtype)
        assert np.max(np.abs(out[0, h] - needle)) < 1e-2, (t, h)
    del base, dev


def test_needle_past_context_end_is_ignored():
    case = small(78, [1000], 16, "f16")
    out0, l0, _, _ = run_case(case, mla.PlanParams(force_partitions=2))
    # token 1000 lives in the last block's tail (1000 % 32 = 8 visible rows)
    plant(case, 0, 1005, 3)
    out1, l1, _, _ = run_case(case, mla.PlanParams(force_partitions=2))
    assert np.array_equal(out0, out1) and np.array_equal(l0, l1)


# --- determinism and layout independence -------------------------------------

def test_run_to_run_bit_identical():
    case = mla_synth.make_workload("two_req_32k_20k")
    dev = to_device(case)
    a = run_case(case, None, dev)
    b = run_case(case, None, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_block_permutation_bit_identical():
    case = small(91, [5000, 333], 32, "bf16")
    out, lse2, _, _ = run_case(case, mla.PlanParams(force_partitions=2))
    rng = np.random.default_rng(3)
    perm = rng.permutation(case.num_blocks)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    case.ckv_pool = np.ascontiguousarray(case.ckv_pool[inv])
    case.kpe_pool = np.ascontiguousarray(case.kpe_pool[inv])
    case.block_table = perm[case.block_table].astype(np.int32)
    out2, lse22, _, _ = run_case(case, mla.PlanParams(force_partitions=2))
    assert np.array_equal(out, out2) and np.array_equal(lse2, lse22)


# --- the reduce on its own, with oracle partials --------------------------------

def test_reduce_matches_oracle_merge_and_rejects_ln_lse():
    import torch
    case = small(121, [1024], 16, "f16")
    blocks = case.block_table[0, :8]
    hot = reference.decode16(case.ckv_pool[blocks], case.dtype) * 1.5
    case.ckv_pool[blocks] = mla_synth.encode16(hot.astype(np.float32), case.dtype)
    ref, lref, *mom = oracle.latent_f64(case, moments=True)
    ranges = oracle.row_ranges(case.context_lens, [4], [1])
    po, pl = oracle.partials_f64(case, ranges, [0, 4])
    ind = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    out = torch.empty((1, 16, 512), dtype=torch.float16, device="cuda")
    lse = torch.empty((1, 16), dtype=torch.float32, device="cuda")
    po_d = torch.tensor(po, dtype=torch.float32, device="cuda")
    for units, lse_in in (("log2", pl), ("ln", pl * np.log(2.0))):
        pl_d = torch.tensor(lse_in, dtype=torch.float32, device="cuda")
        mla.mla_decode_reduce(po_d, pl_d, ind, 1, 16, 4, out, lse)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        err = np.max(np.abs(got - ref))
        log(f"[reduce] {units}: max err {err:.3e}")
        if units == "log2":
            assert err < 1e-2
            assert np.max(np.abs(lse.cpu().numpy() - lref)) < 1e-4
        else:
            assert err > 10 * 1e-2


@pytest.mark.parametrize("hot_tail", [False, True])
def test_reduce_many_rows_online_merge(hot_tail):
    # 600 rows for one request: each row lane of the reduce takes its rows in
    # three batches of eight, keeping a running maximum. With the latent
    # values of the last 16 blocks scaled up, the largest LSEs sit in the
    # last rows, so the running sums are rescaled in the later batches. The
    # first 40 rows are emptied (LSE -inf, zero partial): lanes start from a
    # maximum of -inf.
    import torch
    case = small(131, [32768], 16, "f16")
    if hot_tail:
        blocks = case.block_table[0, 1024 - 16:1024]
        hot = reference.decode16(case.ckv_pool[blocks], case.dtype) * 1.5
        case.ckv_pool[blocks] = mla_synth.encode16(hot.astype(np.float32), case.dtype)
    ranges = oracle.row_ranges(case.context_lens, [12], [50])
    assert len(ranges) == 600
    po, pl = oracle.partials_f64(case, ranges, [0, 600])
    po[:40] = 0.0
    pl[:40] = -np.inf
    ref, lref = reference.merge_log2_f64(po, pl, [0, 600])
    ind = torch.tensor([0, 600], dtype=torch.int32, device="cuda")
    out = torch.empty((1, 16, 512), dtype=torch.float16, device="cuda")
    lse = torch.empty((1, 16), dtype=torch.float32, device="cuda")
    po_d = torch.tensor(po, dtype=torch.float32, device="cuda")
    pl_d = torch.tensor(pl, dtype=torch.float32, device="cuda")
    mla.mla_decode_reduce(po_d, pl_d, ind, 1, 16, 600, out, lse)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    err = np.abs(got - ref)
    log(f"[reduce] 600 rows hot_tail={hot_tail}: max err {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= 1e-2 and err.mean() <= 1e-3
    assert np.max(np.abs(lse.cpu().numpy() - lref)) < 1e-4
    a = out.clone()
    mla.mla_decode_reduce(po_d, pl_d, ind, 1, 16, 600, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(a, out)


def test_reduce_all_empty_rows_give_zero():
    import torch
    po = torch.zeros((3, 16, 512), dtype=torch.float32, device="cuda")
    pl = torch.full((3, 16), float("-inf"), dtype=torch.float32, device="cuda")
    ind = torch.tensor([0, 3], dtype=torch.int32, device="cuda")
    out = torch.full((1, 16, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 16), dtype=torch.float32, device="cuda")
    mla.mla_decode_reduce(po, pl, ind, 1, 16, 3, out, lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == float("-inf"))


@pytest.mark.parametrize("batch,heads,max_rows", [(1, 128, 200), (2, 64, 200), (8, 16, 200),
                                                   (1, 112, 200), (4, 16, 200), (8, 128, 32),
                                                   (64, 16, 33), (16, 16, 32)])
def test_reduce_slice_widths(batch, heads, max_rows):
    # The reduce launch takes 64-dim slices when batch x heads x 8 reaches
    # 1024 workgroups, else 32-dim ones, and 256-dim ones when requests hold
    # 32 rows or fewer on average and batch x heads x 2 reaches 256: cases
    # on every side of those thresholds, with random partials of uneven row
    # counts, some rows empty (LSE -inf, zero partial) and a hot last row per
    # request, against the oracle's merge.
    import torch
    rng = np.random.default_rng(140 + batch * heads + max_rows)
    rows = rng.integers(1, max_rows, size=batch)
    rows[0] = 257 if max_rows > 32 else max_rows
    ind = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    total = int(ind[-1])
    po = rng.standard_normal((total, heads, 512)).astype(np.float32)
    pl = rng.uniform(-4.0, 12.0, size=(total, heads)).astype(np.float32)
    empty = rng.random((total, heads)) < 0.1
    pl[empty] = -np.inf
    po[empty] = 0.0
    pl[ind[1:] - 1] += 20.0
    ref, lref = reference.merge_log2_f64(po, pl, ind)
    out = torch.empty((batch, heads, 512), dtype=torch.float16, device="cuda")
    lse = torch.empty((batch, heads), dtype=torch.float32, device="cuda")
    mla.mla_decode_reduce(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                          torch.from_numpy(ind).cuda(), batch, heads, total, out, lse)
    torch.cuda.synchronize()
    err = np.abs(out.float().cpu().numpy() - ref)
    log(f"[reduce] B={batch} H={heads} rows={total}: max err {err.max():.3e} "
        f"mean {err.mean():.3e}")
    assert err.max() <= 1e-2 and err.mean() <= 1e-3
    got_l = lse.cpu().numpy()
    fin = np.isfinite(lref)      # a head whose rows are all empty merges to -inf
    assert np.max(np.abs(got_l[fin] - lref[fin])) < 1e-4
    assert np.all(got_l[~fin] == -np.inf)


# --- the path taken is provable ---------------------------------------------------

def test_path_counters():
    case = small(5, [40000], 16, "f16")
    dev = to_device(case)
    mla.mla_reset_counters()
    run_case(case, None, dev)
    c = mla.mla_get_counters()
    assert c[0] == 0 and c[1] == 1 and c[2] == 1 and c[3] >= 2
    run_case(case, mla.PlanParams(force_partitions=1, force_splits=1), dev)
    c2 = mla.mla_get_counters()
    assert c2[0] == 1 and c2[1] == 1 and c2[2] == 1


def test_chooser_uses_the_device():
    p = mla.mla_choose_partitions(1, 16, 1, [32768])
    assert device_cus() >= 1
    assert p["P"] == [2] and p["total_rows"] >= 2
