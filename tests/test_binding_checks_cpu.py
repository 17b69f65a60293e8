"""The binding refuses, before any pointer reaches the library, every tensor
that would be read or written out of bounds: wrong element type, wrong
shape, non-contiguous, or on another device. CPU tensors only: with every
argument valid the last check (device tensors required) is the one that
fires, so each mutated case proves its own check ran first.
"""
import os

import pytest
import torch

import absorbed_mla_paged_amd as mla

B, H, NB, BS, MB = 2, 16, 8, 32, 3
ROWS = 4


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(mla.LIB_PATH):
        from absorbed_mla_paged_amd import _build
        _build.build()
    return mla.load_library()


def valid(dtype=torch.bfloat16):
    i32 = torch.int32
    return dict(
        q_absorbed=torch.zeros((B, H, 512), dtype=dtype),
        q_pe=torch.zeros((B, H, 64), dtype=dtype),
        ckv_cache=torch.zeros((NB, BS, 512), dtype=dtype),
        kpe_cache=torch.zeros((NB, BS, 64), dtype=dtype),
        block_table=torch.zeros((B, MB), dtype=i32),
        context_lens=torch.full((B,), 40, dtype=i32),
        scale=0.07,
        partitions=torch.full((B,), 2, dtype=i32),
        splits=torch.ones((B,), dtype=i32),
        row_indptr=torch.tensor([0, 2, 4], dtype=i32),
        total_rows=ROWS, max_rows_per_req=2, heads_per_wg=16,
        partial_out=torch.zeros((ROWS, H, 512), dtype=torch.float32),
        partial_lse2=torch.zeros((ROWS, H), dtype=torch.float32),
        out=torch.zeros((B, H, 512), dtype=dtype),
        lse2_out=torch.zeros((B, H), dtype=torch.float32),
        debug_ranges=torch.zeros((ROWS, 2), dtype=torch.int32))


def call(args):
    mla.mla_decode_partition(**args)


def status_of(args, fn=call):
    with pytest.raises(mla.MlaError) as e:
        fn(args)
    return e.value.status


def test_valid_cpu_arguments_reach_the_device_check():
    assert status_of(valid()) == -1


def noncontig(t):
    big = torch.zeros(t.shape[:-1] + (2 * t.shape[-1],), dtype=t.dtype)
    return big[..., ::2]


BAD = [
    ("kpe with fewer blocks", "kpe_cache", lambda a: torch.zeros((NB - 1, BS, 64), dtype=a.dtype), -2),
    ("kpe of another block size", "kpe_cache", lambda a: torch.zeros((NB, 16, 64), dtype=a.dtype), -2),
    ("kpe of another type", "kpe_cache", lambda a: a.to(torch.float16), -6),
    ("ckv non-contiguous", "ckv_cache", noncontig, -2),
    ("ckv of another type than q", "ckv_cache", lambda a: a.to(torch.float16), -6),
    ("q_pe too short", "q_pe", lambda a: torch.zeros((B, H, 32), dtype=a.dtype), -2),
    ("q_pe of another type", "q_pe", lambda a: a.to(torch.float16), -6),
    ("q_pe non-contiguous", "q_pe", noncontig, -2),
    ("q_absorbed float32", "q_absorbed", lambda a: a.to(torch.float32), -6),
    ("q_absorbed width 256", "q_absorbed", lambda a: torch.zeros((B, H, 256), dtype=a.dtype), -2),
    ("int64 block table", "block_table", lambda a: a.to(torch.int64), -6),
    ("block table of another batch", "block_table", lambda a: torch.zeros((B + 1, MB), dtype=a.dtype), -2),
    ("int64 context lengths", "context_lens", lambda a: a.to(torch.int64), -6),
    ("context lengths too short", "context_lens", lambda a: a[:1].clone(), -2),
    ("int64 plan array", "partitions", lambda a: a.to(torch.int64), -6),
    ("row_indptr too short", "row_indptr", lambda a: a[:2].clone(), -2),
    ("partials of too few rows", "partial_out", lambda a: a[:ROWS - 1].clone(), -2),
    ("partials in bf16", "partial_out", lambda a: a.to(torch.bfloat16), -6),
    ("partial LSEs non-contiguous", "partial_lse2", noncontig, -2),
    ("lse2_out too small", "lse2_out", lambda a: a[:1].clone(), -2),
    ("debug ranges too small", "debug_ranges", lambda a: a[:1].clone(), -2),
]


@pytest.mark.parametrize("what,key,mutate,status", BAD, ids=[w for w, _, _, _ in BAD])
def test_partition_refuses(what, key, mutate, status):
    args = valid()
    args[key] = mutate(args[key])
    assert status_of(args) == status, what


def test_single_pass_out_is_checked():
    args = valid()
    args.update(total_rows=B, max_rows_per_req=1, partitions=None, splits=None,
                row_indptr=None, partial_out=None, partial_lse2=None)
    assert status_of(args) == -1                       # valid single pass
    args["out"] = torch.zeros((B, H, 256), dtype=torch.bfloat16)
    assert status_of(args) == -2
    args["out"] = torch.zeros((B, H, 512), dtype=torch.float16)
    assert status_of(args) == -6


def test_split_plan_needs_its_buffers():
    args = valid()
    args["partial_out"] = None
    assert status_of(args) == -1 and "partial_out" in str(
        pytest.raises(mla.MlaError, call, args).value)


def test_fp8_partition_refuses_16bit_caches():
    args = valid()
    args["kv_scale"] = 1.0
    assert status_of(args, lambda a: mla.mla_decode_partition_fp8(**a)) == -6
    args["ckv_cache"] = torch.zeros((NB, BS, 512), dtype=torch.uint8)
    args["kpe_cache"] = torch.zeros((NB - 1, BS, 64), dtype=torch.uint8)
    assert status_of(args, lambda a: mla.mla_decode_partition_fp8(**a)) == -2
    args["kpe_cache"] = torch.zeros((NB, BS, 64), dtype=torch.uint8)
    assert status_of(args, lambda a: mla.mla_decode_partition_fp8(**a)) == -1


def reduce_args():
    return dict(partial_out=torch.zeros((ROWS, H, 512)), partial_lse2=torch.zeros((ROWS, H)),
                row_indptr=torch.tensor([0, 2, 4], dtype=torch.int32), batch=B, num_heads=H,
                total_rows=ROWS, out=torch.zeros((B, H, 512), dtype=torch.float16),
                lse2_out=torch.zeros((B, H)))


REDUCE_BAD = [
    ("partials short", "partial_out", lambda a: a[:ROWS - 1].clone(), -2),
    ("partials of fewer heads", "partial_out", lambda a: torch.zeros((ROWS, H - 16, 512)), -2),
    ("LSEs in float64", "partial_lse2", lambda a: a.double(), -6),
    ("int64 row_indptr", "row_indptr", lambda a: a.long(), -6),
    ("out float32", "out", lambda a: a.float(), -6),
    ("out non-contiguous", "out", noncontig, -2),
    ("lse2_out short", "lse2_out", lambda a: a[:1].clone(), -2),
]


def test_reduce_valid_reaches_device_check():
    assert status_of(reduce_args(), lambda a: mla.mla_decode_reduce(**a)) == -1


@pytest.mark.parametrize("what,key,mutate,status", REDUCE_BAD, ids=[w for w, _, _, _ in REDUCE_BAD])
def test_reduce_refuses(what, key, mutate, status):
    args = reduce_args()
    args[key] = mutate(args[key])
    assert status_of(args, lambda a: mla.mla_decode_reduce(**a)) == status, what


def test_head_products_refuse_mismatched_tensors():
    w = torch.zeros((H, 128, 512), dtype=torch.bfloat16)
    x = torch.zeros((3, H, 128), dtype=torch.bfloat16)
    y = torch.zeros((3, H, 512), dtype=torch.bfloat16)
    assert status_of(None, lambda _: mla.mla_absorb_query(x, w, y)) == -1
    assert status_of(None, lambda _: mla.mla_absorb_query(x.half(), w, y)) == -6
    assert status_of(None, lambda _: mla.mla_absorb_query(x, w, y[:2].clone())) == -2
    assert status_of(None, lambda _: mla.mla_absorb_query(torch.zeros((3, H, 64), dtype=w.dtype),
                                                          w, y)) == -2
    assert status_of(None, lambda _: mla.mla_absorb_query(noncontig(x), w, y)) == -2


def test_fused_sync_buffer_is_checked():
    args = valid()
    args["sync"] = torch.zeros(8, dtype=torch.int64)      # needs 64 words per request
    assert status_of(args, lambda a: mla.mla_decode_fused(**a)) == -2
    args["sync"] = torch.zeros(B * 64, dtype=torch.int64)
    assert status_of(args, lambda a: mla.mla_decode_fused(**a)) == -1


def test_fused_single_pass_needs_no_workspace():
    args = valid()
    args.update(total_rows=B, max_rows_per_req=1, partitions=None, splits=None,
                row_indptr=None, partial_out=None, partial_lse2=None, sync=None,
                debug_ranges=None)
    assert status_of(args, lambda a: mla.mla_decode_fused(**a)) == -1
    args["out"] = None
    assert status_of(args, lambda a: mla.mla_decode_fused(**a)) == -1 and \
        "out" in str(pytest.raises(mla.MlaError, mla.mla_decode_fused, **args).value)
