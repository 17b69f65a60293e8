"""Pins of the plan mirror (chooser + index math) on the CPU.

The chooser's gates come from vllm-metal pull request 601 "[kernel] Wire MLA
split-KV decode", "What changed" (pure decode, long enough context, small
launch, 2 to 8 partitions, bounded temporary memory) and the note before the
wrapper grid that the split path starts at 32K+ context. Its printed choices
are in the "Wrapper benchmark" table.
"""
import itertools

import pytest

from oracle import plan


def test_ranges_tile_the_context_exactly():
    # Every token in [0, n) is covered once, in order, by block-aligned tiles.
    for n in list(range(0, 200)) + [1023, 1024, 1025, 4096, 32768, 81920]:
        for P in range(1, 9):
            for S in (1, 2, 3, 5, 16):
                pos = 0
                for p in range(P):
                    for s in range(S):
                        lo, hi = plan.partition_range(n, P, S, p, s)
                        assert lo <= hi
                        if hi > lo:
                            assert lo == pos and lo % 32 == 0
                            assert hi == n or hi % 32 == 0
                            pos = hi
                assert pos == n, (n, P, S)


def test_tiny_workload_forced_two_partitions():
    # 1024 tokens in 2 partitions of 512 tokens.
    r = plan.choose_partitions(1, 16, 1, [1024],
                               plan.PlanParams(force_partitions=2, force_splits=1))
    assert r["P"] == [2] and r["S"] == [1] and r["row_indptr"] == [0, 2]
    assert [plan.partition_range(1024, 2, 1, p, 0) for p in range(2)] == [(0, 512), (512, 1024)]
    assert r["needs_reduce"] == 1
    assert r["workspace_bytes"] == 2 * 16 * 513 * 4


@pytest.mark.parametrize("n,expect", [(32768, 2), (81920, 5), (98304, 6), (131072, 8),
                                      (32767, 1), (20000, 1)])
def test_policy_partition_counts(n, expect):
    # 32K -> 2, 81K -> 5 and 98K -> 6 match the wrapper table's selected
    # splits; 49K -> 2, 65K -> 2 and 131K -> 4 in that table are not
    # monotone in the context and no context-only rule reproduces them.
    r = plan.choose_partitions(1, 16, 1, [n], plan.PlanParams())
    assert r["P"] == [expect]


def test_pure_decode_gate():
    # Two new tokens: no policy split (pure decode only), but the device
    # tiling still spreads the 2 x 16 query rows' head groups over the CUs.
    r = plan.choose_partitions(1, 16, 2, [131072], plan.PlanParams())
    assert r["P"] == [1] and r["groups"] == 2
    assert r["S"] == [128] and r["tile_blocks"] == 32     # 2 * 4096 blocks / 256 CUs
    assert r["workspace_bytes"] == 128 * 2 * 16 * 513 * 4
    r1 = plan.choose_partitions(1, 16, 1, [131072], plan.PlanParams())
    assert r1["P"] == [8]
    with pytest.raises(ValueError):
        plan.choose_partitions(1, 16, 9, [1000], plan.PlanParams())


def test_small_launch_gate():
    # A launch that already fills the device is not split by policy.
    prm = plan.PlanParams(num_cus=8)
    r = plan.choose_partitions(8, 16, 1, [65536] * 8, prm)
    assert r["P"] == [1] * 8
    r = plan.choose_partitions(7, 16, 1, [65536] * 7, prm)
    assert r["P"] == [4] * 7


def test_device_tiling_fills_the_device():
    r = plan.choose_partitions(1, 16, 1, [32768], plan.PlanParams(num_cus=256))
    assert r["P"] == [2]
    assert r["tile_blocks"] == 4
    assert r["S"] == [128]
    assert r["total_rows"] == 256


def test_workspace_shedding_order():
    heads = 128
    ctx = [131072, 4096, 40000, 90000]
    row = heads * 513 * 4
    free = plan.choose_partitions(4, heads, 1, ctx, plan.PlanParams(heads_per_wg=64))
    assert free["workspace_bytes"] == free["total_rows"] * row
    # Step 1: tiles grow until S is 1 everywhere.
    lim = sum(free["P"]) * row
    r = plan.choose_partitions(4, heads, 1, ctx,
                               plan.PlanParams(heads_per_wg=64, workspace_limit_bytes=lim))
    assert r["S"] == [1, 1, 1, 1] and r["P"] == free["P"]
    # Step 2: the largest P comes down first, not below 2.
    lim2 = (sum(free["P"]) - 3) * row
    r = plan.choose_partitions(4, heads, 1, ctx,
                               plan.PlanParams(heads_per_wg=64, workspace_limit_bytes=lim2))
    assert sum(r["P"]) == sum(free["P"]) - 3 and min(p for p in r["P"]) >= 1
    assert r["workspace_bytes"] <= lim2
    # Step 3: down to single pass, which needs no workspace at all.
    r = plan.choose_partitions(4, heads, 1, ctx,
                               plan.PlanParams(heads_per_wg=64, workspace_limit_bytes=1))
    assert r["P"] == [1] * 4 and r["S"] == [1] * 4 and r["workspace_bytes"] == 0


def test_workspace_limit_with_forced_values_errors():
    with pytest.raises(ValueError):
        plan.choose_partitions(1, 16, 1, [4096],
                               plan.PlanParams(force_partitions=4, force_splits=4,
                                               workspace_limit_bytes=1000))


@pytest.mark.parametrize("heads", [0, 8, 24, 144])
def test_unsupported_heads(heads):
    with pytest.raises(ValueError):
        plan.choose_partitions(1, heads, 1, [100])


def test_rows_are_request_major():
    ctx = [40000, 5, 0, 70000]
    r = plan.choose_partitions(4, 16, 1, ctx, plan.PlanParams(num_cus=64))
    rows = plan.row_ranges(ctx, r["P"], r["S"])
    assert len(rows) == r["total_rows"]
    for b in range(4):
        span = rows[r["row_indptr"][b]:r["row_indptr"][b + 1]]
        assert all(x[0] == b for x in span)
        covered = sum(hi - lo for _, lo, hi in span)
        assert covered == ctx[b]


def test_exhaustive_small_grid_is_consistent():
    # Mirror self-consistency over a small grid: P in [1, 8], S >= 1, rows sum.
    for ctx in itertools.product([0, 1, 33, 5000, 40000], repeat=2):
        r = plan.choose_partitions(2, 32, 1, list(ctx), plan.PlanParams(num_cus=16))
        assert all(1 <= p <= 8 for p in r["P"]) and all(s >= 1 for s in r["S"])
        assert r["row_indptr"][-1] == sum(p * s for p, s in zip(r["P"], r["S"]))


def test_device_tiling_fits_one_wave_81k_64_head_groups():
    # 81920 tokens, P = 5 (512 blocks per partition), 128 heads in 64-head
    # workgroups (G = 2): the first tile, ceil(2 * 2560 / 256) = 20 blocks,
    # gives 5 * 26 rows = 260 workgroups, four past one wave of 256; 21
    # blocks gives 5 * 25 rows = 250.
    r = plan.choose_partitions(1, 128, 1, [81920], plan.PlanParams(num_cus=256))
    assert r["heads_per_wg"] == 64 and r["groups"] == 2
    assert r["P"] == [5] and r["tile_blocks"] == 21 and r["S"] == [25]
    assert r["groups"] * r["total_rows"] == 250


def test_device_tiling_fit_is_the_smallest_fitting_tile():
    # Brute force: whenever the fit step moved the tile, no smaller tile at
    # or above the first estimate fits, and the chosen one does (or gives
    # S_b = 1 everywhere).
    import random
    rnd = random.Random(7)
    for _ in range(400):
        batch = rnd.choice([1, 2, 3, 5, 8])
        heads = rnd.choice([16, 64, 128])
        ctx = [rnd.choice([0, 33, 4096, 20000, 32768, 81920, 131072, rnd.randint(0, 131072)])
               for _ in range(batch)]
        cus = rnd.choice([8, 64, 256, 304])
        r = plan.choose_partitions(batch, heads, 1, ctx, plan.PlanParams(num_cus=cus))
        nblk = [-(-n // 32) for n in ctx]
        G = r["groups"]
        first = max(4, -(-G * sum(nblk) // cus))

        def wgs(t):
            return G * sum(p * max(1, -(-(-(-nb // p)) // t)) for nb, p in zip(nblk, r["P"]))
        t = r["tile_blocks"]
        assert t >= first
        if t > first:
            assert all(wgs(u) > cus for u in range(first, t))
            assert wgs(t) <= cus or all(s == 1 for s in r["S"])
        assert r["S"] == [max(1, -(-(-(-nb // p)) // t)) for nb, p in zip(nblk, r["P"])]
