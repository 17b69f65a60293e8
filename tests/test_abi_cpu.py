"""The C-ABI library on the CPU: symbols, chooser, index math, host checks.

No kernel is launched here. The chooser and the index math are compared bit
for bit with the independent mirror in oracle.plan.
"""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import absorbed_mla_paged_amd as mla
from oracle import plan as mirror

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="session", autouse=True)
def built_library():
    if not os.path.exists(mla.LIB_PATH):
        from absorbed_mla_paged_amd import _build
        _build.build()
    return mla.load_library()


def declared_functions():
    with open(os.path.join(ROOT, "include", "mla_decode.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(built_library):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(built_library, n), n
    assert sorted(mla.EXPORTS) == names


def test_status_strings():
    for code in mla.STATUS:
        assert mla.mla_status_string(code)
    assert mla.mla_status_string(12345) == "unknown status"


def test_default_params_match_header_and_mirror():
    d = mla.mla_default_plan_params()
    m = mirror.PlanParams()
    for f in ("min_split_ctx", "tokens_per_partition", "min_partitions", "max_partitions",
              "min_tile_blocks", "wgs_per_cu", "force_partitions", "force_splits",
              "workspace_limit_bytes"):
        assert getattr(d, f) == getattr(m, f), f
    assert d.num_cus == 0 and d.heads_per_wg == 0


def _both(batch, heads, q_len, ctx, block_size=32, **kw):
    c_params = mla.PlanParams(**kw)
    m_params = mirror.PlanParams(**kw)
    try:
        ref = mirror.choose_partitions(batch, heads, q_len, ctx, m_params, block_size=block_size)
    except ValueError:
        ref = None
    try:
        got = mla.mla_choose_partitions(batch, heads, q_len, ctx, c_params,
                                        block_size=block_size)
    except mla.MlaError:
        got = None
    return ref, got


def _same(ref, got):
    assert (ref is None) == (got is None)
    if ref is None:
        return
    for k in ("P", "S", "row_indptr", "total_rows", "max_rows_per_req", "tile_blocks",
              "heads_per_wg", "groups", "needs_reduce"):
        assert ref[k] == got[k], (k, ref[k], got[k])
    assert ref["workspace_bytes"] == got["partial_out_bytes"] + got["partial_lse_bytes"]


@pytest.mark.parametrize("block_size", [32, 16])
@pytest.mark.parametrize("heads", [16, 32, 64, 128])
def test_chooser_matches_mirror_on_a_grid(heads, block_size):
    rng = np.random.default_rng(heads + block_size)
    ctx_pool = [0, 1, 31, 32, 33, 1000, 4096, 20000, 32767, 32768, 49152, 65536, 81920,
                98304, 131072]
    for batch in (1, 2, 3, 8):
        for trial in range(12):
            ctx = [int(c) for c in rng.choice(ctx_pool, size=batch)]
            for num_cus, tile, limit, fp, fs, hpw in itertools.product(
                    (8, 256), (1, 4), (0, 1 << 20, 64 << 20), (0, 3), (0, 2), (0, 16, heads)):
                ref, got = _both(batch, heads, 1, ctx, block_size, num_cus=num_cus,
                                 min_tile_blocks=tile,
                                 workspace_limit_bytes=limit, force_partitions=fp,
                                 force_splits=fs, heads_per_wg=hpw)
                _same(ref, got)


def test_chooser_matches_mirror_on_workloads():
    import mla_synth
    for name, spec in mla_synth.WORKLOADS.items():
        if "context_range" in spec:
            rng = np.random.Generator(np.random.PCG64(spec["seed"]))
            lo, hi = spec["context_range"]
            ctx = [int(c) for c in rng.integers(lo, hi, size=spec["batch"], endpoint=True)]
        else:
            ctx = spec["contexts"]
        for limit, bs in itertools.product((0, 64 << 20), (32, 16)):
            ref, got = _both(spec["batch"], spec["heads"], 1, ctx, bs, num_cus=256,
                             workspace_limit_bytes=limit)
            _same(ref, got)
            assert got is not None


def test_chooser_pure_decode_and_errors():
    _same(*_both(2, 16, 3, [70000, 5], num_cus=256))
    for bad in [dict(batch=1, heads=24), dict(batch=1, heads=0), dict(batch=1, heads=144)]:
        ref, got = _both(bad["batch"], bad["heads"], 1, [10], num_cus=256)
        assert ref is None and got is None
    ref, got = _both(1, 16, 1, [-1], num_cus=256)
    assert ref is None and got is None
    ref, got = _both(1, 16, 0, [10], num_cus=256)
    assert ref is None and got is None
    ref, got = _both(1, 16, 9, [10], num_cus=256)
    assert ref is None and got is None
    for q in (2, 4, 8):
        _same(*_both(3, 32, q, [40000, 7, 3000], num_cus=256))
        _same(*_both(1, 128, q, [131072], num_cus=256))
    for bs in (8, 24, 64):
        with pytest.raises(mla.MlaError) as e:
            mla.mla_choose_partitions(1, 16, 1, [10], mla.PlanParams(num_cus=256), block_size=bs)
        assert e.value.status == -6
        ref, got = _both(1, 16, 1, [10], bs, num_cus=256)
        assert ref is None and got is None
    with pytest.raises(mla.MlaError) as e:
        mla.mla_choose_partitions(1, 16, 1, [4096], mla.PlanParams(
            num_cus=256, force_partitions=4, force_splits=4, workspace_limit_bytes=1000))
    assert e.value.status == -5 and "workspace" in mla.mla_last_error()


@pytest.mark.parametrize("block_size", [32, 16])
def test_index_math_matches_mirror_exhaustively_small(block_size):
    # Every context up to 300 tokens, every P <= 8, S <= 16, every (p, s).
    lib = mla.load_library()
    lo, hi = ctypes.c_int32(), ctypes.c_int32()
    for n in range(0, 301):
        for P in range(1, 9):
            for S in range(1, 17):
                for p in range(P):
                    for s in range(S):
                        assert lib.mla_partition_range(n, block_size, P, S, p, s,
                                                       ctypes.byref(lo), ctypes.byref(hi)) == 0
                        assert (lo.value, hi.value) == \
                            mirror.partition_range(n, P, S, p, s, block_size)


def test_index_math_matches_mirror_at_long_contexts():
    rng = np.random.default_rng(1)
    ns = [1023, 1024, 1025, 32767, 32768, 32769, 81920, 131071, 131072] + \
        [int(x) for x in rng.integers(0, 1 << 20, size=40)]
    for n in ns:
        for P in range(1, 9):
            for S in (1, 2, 3, 7, 64, 128, 1000):
                for p in range(P):
                    for s in sorted({0, 1, S // 2, S - 1}):
                        if s < S:
                            for bs in (32, 16):
                                assert mla.mla_partition_range(n, P, S, p, s, bs) == \
                                    mirror.partition_range(n, P, S, p, s, bs)


def test_index_math_errors():
    for args in [(-1, 1, 1, 0, 0), (10, 0, 1, 0, 0), (10, 2, 1, 2, 0), (10, 1, 2, 0, 2)]:
        with pytest.raises(mla.MlaError) as e:
            mla.mla_partition_range(*args)
        assert e.value.status == -3


def test_decode_partition_host_checks_launch_nothing():
    # Invalid calls are refused on the host, before any HIP call.
    lib = mla.load_library()
    vp = ctypes.c_void_p
    good = vp(0x10000)
    odd = vp(0x10008)

    def call(**kw):
        a = dict(qa=good, qp=good, ckv=good, kpe=good, nblk=4, bs=32, tbl=good, maxb=4, ctx=good,
                 batch=1, heads=16, qlen=1, scale=0.07, dtype=0, P=good, S=good, ind=good, rows=2,
                 maxr=2, hpw=0, po=good, pl=good, out=good, lo=None, dbg=None, stream=None)
        a.update(kw)
        return lib.mla_decode_partition(a["qa"], a["qp"], a["ckv"], a["kpe"], a["nblk"], a["bs"],
                                        a["tbl"],
                                        a["maxb"], a["ctx"], a["batch"], a["heads"], a["qlen"],
                                        a["scale"],
                                        a["dtype"], a["P"], a["S"], a["ind"], a["rows"], a["maxr"],
                                        a["hpw"], a["po"], a["pl"], a["out"], a["lo"], a["dbg"],
                                        a["stream"])
    assert call(heads=24) == -6
    assert call(heads=160) == -6
    assert call(qlen=0) == -6
    assert call(qlen=9) == -6
    assert call(dtype=7) == -6
    assert call(bs=64) == -6             # cache blocks of 16 or 32 tokens only
    assert call(bs=8) == -6
    assert call(hpw=32) == -6
    assert call(heads=128, hpw=128) == -6   # no 128-head layout
    assert call(heads=96, hpw=64) == -6     # 64 must divide H
    assert call(scale=float("nan")) == -3
    assert call(scale=0.0) == -3          # the scale must be > 0: the 64-head kernel
    assert call(scale=-0.07) == -3        # tracks unscaled maxima
    assert call(qa=None) == -1
    assert call(po=None) == -1          # split plan without workspace
    assert call(rows=1, out=None) == -1  # single pass without out
    assert call(qa=odd) == -4
    assert call(po=odd) == -4
    assert call(rows=0) == -2
    assert call(rows=5, maxr=2) == -2
    assert call(nblk=0) == -2
    assert call(batch=-1) == -2
    assert call(batch=0) == 0            # nothing to do
    assert "heads" in mla.mla_last_error() or mla.mla_last_error() == ""


def test_decode_fused_host_checks_launch_nothing():
    lib = mla.load_library()
    vp = ctypes.c_void_p
    good = vp(0x10000)

    def call(**kw):
        a = dict(qa=good, qp=good, ckv=good, kpe=good, nblk=4, bs=32, tbl=good, maxb=4, ctx=good,
                 batch=1, heads=16, qlen=1, scale=0.07, dtype=0, P=good, S=good, ind=good, rows=2,
                 maxr=2, hpw=0, po=good, pl=good, out=good, lo=None, sync=good, dbg=None,
                 stream=None)
        a.update(kw)
        return lib.mla_decode_fused(a["qa"], a["qp"], a["ckv"], a["kpe"], a["nblk"], a["bs"],
                                    a["tbl"],
                                    a["maxb"], a["ctx"], a["batch"], a["heads"], a["qlen"],
                                    a["scale"],
                                    a["dtype"], a["P"], a["S"], a["ind"], a["rows"], a["maxr"],
                                    a["hpw"], a["po"], a["pl"], a["out"], a["lo"], a["sync"],
                                    a["dbg"], a["stream"])
    assert call(sync=None) == -1             # split plan without hand-off state
    assert call(out=None) == -1              # split plan without out
    assert call(sync=vp(0x10020)) == -4      # sync must be 64-byte aligned
    assert call(heads=128, hpw=16, qlen=2) == -6   # 16 head groups: more than the record holds
    assert call(heads=24) == -6
    assert call(bs=48) == -6
    assert call(po=None) == -1
    assert call(batch=0) == 0


def test_head_products_host_checks():
    lib = mla.load_library()
    vp = ctypes.c_void_p
    g = vp(0x10000)
    for fn in (lib.mla_absorb_query, lib.mla_unabsorb_output):
        assert fn(None, g, g, 2, 16, 0, None) == -1
        assert fn(g, g, vp(0x10008), 2, 16, 0, None) == -4
        assert fn(g, g, g, 2, 0, 0, None) == -2
        assert fn(g, g, g, -1, 16, 0, None) == -2
        assert fn(g, g, g, 2, 16, 5, None) == -6
        assert fn(None, None, None, 0, 16, 0, None) == 0   # nothing to do


def test_decode_reduce_host_checks():
    lib = mla.load_library()
    vp = ctypes.c_void_p
    g = vp(0x10000)
    assert lib.mla_decode_reduce(g, g, g, 1, 24, 2, 0, g, None, None) == -6
    assert lib.mla_decode_reduce(g, g, g, 1, 16, 2, 9, g, None, None) == -6
    assert lib.mla_decode_reduce(None, g, g, 1, 16, 2, 0, g, None, None) == -1
    assert lib.mla_decode_reduce(g, g, g, 1, 16, 2, 0, vp(0x10002), None, None) == -4
    assert lib.mla_decode_reduce(g, g, g, 0, 16, 0, 0, g, None, None) == 0


def test_decode_noalloc_host_checks_launch_nothing():
    # Plans whose partials exceed the fixed scratch, and a missing or
    # misaligned `out`, are refused before any HIP call.
    lib = mla.load_library()
    vp = ctypes.c_void_p
    g = vp(0x10000)

    def call(rows=2, out=g, batch=1, heads=128, lo=None):
        return lib.mla_decode_noalloc(g, g, g, g, 4, 32, g, 4, g, batch, heads, 1, 0.07, 1, g, g,
                                      g, rows, max(1, rows), 0, out, lo, None)
    limit = mla.NOALLOC_SCRATCH_BYTES
    assert mla.mla_noalloc_scratch_bytes(2, 128) == 2 * 128 * 513 * 4
    rows_fit = limit // (128 * 513 * 4)
    assert mla.mla_noalloc_scratch_bytes(rows_fit, 128) <= limit
    assert mla.mla_noalloc_scratch_bytes(rows_fit + 1, 128) > limit
    assert call(rows=rows_fit + 1) == -5
    assert "scratch" in mla.mla_last_error()
    assert call(out=None) == -1
    assert call(out=vp(0x10008)) == -4
    assert call(lo=vp(0x10002)) == -4
    assert call(batch=0, rows=0) == 0
    assert call(batch=-1) == -2


def test_stream_read_host_checks():
    lib = mla.load_library()
    vp = ctypes.c_void_p
    g = vp(0x10000)
    assert lib.mla_stream_read(None, 1024, g, 5, None) == -1
    assert lib.mla_stream_read(g, 1024, None, 5, None) == -1
    assert lib.mla_stream_read(vp(0x10008), 1024, g, 5, None) == -4
    assert lib.mla_stream_read(g, 1000, g, 5, None) == -4
    assert lib.mla_stream_read(None, 0, None, 5, None) == 0


def test_copy_probe_host_checks():
    lib = mla.load_library()
    vp = ctypes.c_void_p
    g = vp(0x10000)
    assert lib.mla_copy_probe(None, g, 8, g, 2, 4, 1, 8, 8, None) == -1
    assert lib.mla_copy_probe(g, g, 8, g, 0, 4, 1, 8, 8, None) == -2
    assert lib.mla_copy_probe(g, g, 8, g, 2, 4, 3, 8, 8, None) == -2
    assert lib.mla_copy_probe(g, g, 8, g, 2, 4, 1, 6, 8, None) == -6
    assert lib.mla_copy_probe(g, g, 8, g, 2, 4, 1, 8, 32, None) == -6


def test_counters_reset():
    mla.mla_reset_counters()
    assert mla.mla_get_counters() == [0, 0, 0, 0]


def test_decode_partition_fp8_host_checks_launch_nothing():
    lib = mla.load_library()
    vp = ctypes.c_void_p
    good = vp(0x10000)

    def call(**kw):
        a = dict(qa=good, qp=good, ckv=good, kpe=good, ks=0.03125, nblk=4, bs=32, tbl=good,
                 maxb=4, ctx=good, batch=1, heads=16, qlen=1, scale=0.07, dtype=0, P=good,
                 S=good, ind=good, rows=2, maxr=2, hpw=16, po=good, pl=good, out=good, lo=None,
                 dbg=None, stream=None)
        a.update(kw)
        return lib.mla_decode_partition_fp8(
            a["qa"], a["qp"], a["ckv"], a["kpe"], a["ks"], a["nblk"], a["bs"], a["tbl"],
            a["maxb"], a["ctx"], a["batch"], a["heads"], a["qlen"], a["scale"], a["dtype"],
            a["P"], a["S"], a["ind"], a["rows"], a["maxr"], a["hpw"], a["po"], a["pl"],
            a["out"], a["lo"], a["dbg"], a["stream"])
    assert call(hpw=64, heads=48) == -6       # 64 does not divide 48 heads
    assert call(ks=0.0) == -3
    assert call(ks=-2.0) == -3
    assert call(ks=float("inf")) == -3
    assert call(bs=48) == -6
    assert call(ckv=vp(0x10008)) == -4
    assert call(kpe=None) == -1
    assert call(dtype=3) == -6
    assert call(batch=0) == 0
