"""Python binding of libmla_decode.so: split-KV, matrix-absorbed MLA decode
over a paged latent KV cache on MI355X (gfx950).

The functions here carry the C ABI's names (include/mla_decode.h) and only
marshal arguments: every step of the decode runs in the HIP kernels of the
library. torch is used for device memory and the current stream. If the
library is not built, importing works but every call raises; build it with
``python -m absorbed_mla_paged_amd._build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_decode.so")

MLA_F16, MLA_BF16 = 0, 1
KV_LORA_RANK, ROPE_DIM, BLOCK_SIZE = 512, 64, 32
BLOCK_SIZES = (16, 32)   # cache block sizes the kernels are built for
FUSED_SYNC_BYTES_PER_REQUEST = 512
NOALLOC_SCRATCH_BYTES = 64 << 20   # MLA_NOALLOC_SCRATCH_BYTES
STATUS = {0: "MLA_OK", -1: "MLA_E_NULL", -2: "MLA_E_SHAPE", -3: "MLA_E_RANGE",
          -4: "MLA_E_ALIGN", -5: "MLA_E_WORKSPACE", -6: "MLA_E_UNSUPPORTED",
          -7: "MLA_E_HIP"}

# Every function include/mla_decode.h declares.
EXPORTS = ["mla_default_plan_params", "mla_choose_partitions", "mla_partition_range",
           "mla_decode_partition", "mla_decode_partition_fp8", "mla_decode_reduce",
           "mla_decode_fused", "mla_decode_noalloc", "mla_noalloc_scratch_bytes",
           "mla_stream_read", "mla_copy_probe",
           "mla_absorb_query",
           "mla_unabsorb_output", "mla_status_string",
           "mla_last_error", "mla_get_counters", "mla_reset_counters"]


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class _PlanParams(ctypes.Structure):
    _fields_ = [("min_split_ctx", ctypes.c_int32), ("tokens_per_partition", ctypes.c_int32),
                ("min_partitions", ctypes.c_int32), ("max_partitions", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("heads_per_wg", ctypes.c_int32),
                ("min_tile_blocks", ctypes.c_int32), ("wgs_per_cu", ctypes.c_int32),
                ("force_partitions", ctypes.c_int32), ("force_splits", ctypes.c_int32),
                ("workspace_limit_bytes", ctypes.c_int64)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [("total_rows", ctypes.c_int32), ("max_rows_per_req", ctypes.c_int32),
                ("heads_per_wg", ctypes.c_int32), ("groups", ctypes.c_int32),
                ("tile_blocks", ctypes.c_int32), ("needs_reduce", ctypes.c_int32),
                ("partial_out_bytes", ctypes.c_int64), ("partial_lse_bytes", ctypes.c_int64)]


_lib = None


def library_path() -> str:
    return LIB_PATH


def load_library(path: str | None = None):
    """Load (once) and return the ctypes handle; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise MlaError(-7, f"{path} is not built; run python -m absorbed_mla_paged_amd._build")
    lib = ctypes.CDLL(path, mode=ctypes.RTLD_LOCAL)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    pi32 = ctypes.POINTER(ctypes.c_int32)
    lib.mla_default_plan_params.argtypes = [ctypes.POINTER(_PlanParams)]
    lib.mla_default_plan_params.restype = None
    lib.mla_choose_partitions.argtypes = [i32, i32, i32, pi32, i32, ctypes.POINTER(_PlanParams),
                                          pi32, pi32, pi32, ctypes.POINTER(_PlanInfo)]
    lib.mla_choose_partitions.restype = ctypes.c_int
    lib.mla_partition_range.argtypes = [i32, i32, i32, i32, i32, i32, pi32, pi32]
    lib.mla_partition_range.restype = ctypes.c_int
    lib.mla_decode_partition.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, i32, i32, i32,
                                         ctypes.c_float, i32, vp, vp, vp, i32, i32, i32,
                                         vp, vp, vp, vp, vp, vp]
    lib.mla_decode_partition.restype = ctypes.c_int
    lib.mla_decode_partition_fp8.argtypes = [vp, vp, vp, vp, ctypes.c_float, i32, i32, vp, i32,
                                             vp, i32, i32, i32, ctypes.c_float, i32, vp, vp, vp,
                                             i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.mla_decode_partition_fp8.restype = ctypes.c_int
    lib.mla_decode_reduce.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
    lib.mla_decode_reduce.restype = ctypes.c_int
    lib.mla_decode_fused.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, i32, i32, i32,
                                     ctypes.c_float, i32, vp, vp, vp, i32, i32, i32,
                                     vp, vp, vp, vp, vp, vp, vp]
    lib.mla_decode_fused.restype = ctypes.c_int
    lib.mla_decode_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, i32, i32, i32,
                                       ctypes.c_float, i32, vp, vp, vp, i32, i32, i32, vp, vp,
                                       vp]
    lib.mla_decode_noalloc.restype = ctypes.c_int
    lib.mla_noalloc_scratch_bytes.argtypes = [i32, i32, i32]
    lib.mla_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.mla_copy_probe.argtypes = [vp, vp, i32, vp, i32, i32, i32, i32, i32, vp]
    lib.mla_copy_probe.restype = ctypes.c_int
    lib.mla_stream_read.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_uint32, vp]
    lib.mla_stream_read.restype = ctypes.c_int
    for name in ("mla_absorb_query", "mla_unabsorb_output"):
        getattr(lib, name).argtypes = [vp, vp, vp, i32, i32, i32, vp]
        getattr(lib, name).restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_get_counters.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
    lib.mla_get_counters.restype = None
    lib.mla_reset_counters.argtypes = []
    lib.mla_reset_counters.restype = None
    del i64
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().mla_last_error().decode(errors="replace")
        raise MlaError(status, msg)


@dataclasses.dataclass
class PlanParams:
    """Mirror of mla_plan_params (defaults from mla_default_plan_params)."""
    min_split_ctx: int = 32768
    tokens_per_partition: int = 16384
    min_partitions: int = 2
    max_partitions: int = 8
    num_cus: int = 0
    heads_per_wg: int = 0
    min_tile_blocks: int = 4
    wgs_per_cu: int = 1
    force_partitions: int = 0
    force_splits: int = 0
    workspace_limit_bytes: int = 0

    def _c(self) -> _PlanParams:
        return _PlanParams(**dataclasses.asdict(self))


def mla_default_plan_params() -> PlanParams:
    lib = load_library()
    p = _PlanParams()
    lib.mla_default_plan_params(ctypes.byref(p))
    return PlanParams(**{f: getattr(p, f) for f, _ in _PlanParams._fields_})


def _i32_array(values):
    values = [int(v) for v in values]
    return (ctypes.c_int32 * max(1, len(values)))(*values)


def mla_choose_partitions(batch: int, num_heads: int, q_len: int, context_lens,
                          params: PlanParams | None = None, block_size: int = BLOCK_SIZE) -> dict:
    """Host chooser: returns P, S, row_indptr (lists) and the plan info."""
    lib = load_library()
    ctx = _i32_array(context_lens)
    P = (ctypes.c_int32 * max(1, batch))()
    S = (ctypes.c_int32 * max(1, batch))()
    ind = (ctypes.c_int32 * (batch + 1))()
    info = _PlanInfo()
    prm = params._c() if params is not None else None
    _check(lib.mla_choose_partitions(batch, num_heads, q_len, ctx, block_size,
                                     ctypes.byref(prm) if prm is not None else None,
                                     P, S, ind, ctypes.byref(info)))
    out = {f: getattr(info, f) for f, _ in _PlanInfo._fields_}
    out.update(P=list(P)[:batch], S=list(S)[:batch], row_indptr=list(ind))
    return out


def mla_partition_range(ctx: int, P: int, S: int, p: int, s: int,
                        block_size: int = BLOCK_SIZE):
    lib = load_library()
    lo, hi = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.mla_partition_range(ctx, block_size, P, S, p, s, ctypes.byref(lo), ctypes.byref(hi)))
    return lo.value, hi.value


def mla_status_string(status: int) -> str:
    return load_library().mla_status_string(status).decode()


def mla_last_error() -> str:
    return load_library().mla_last_error().decode(errors="replace")


def mla_get_counters():
    arr = (ctypes.c_uint64 * 4)()
    load_library().mla_get_counters(arr)
    return list(arr)


def mla_reset_counters():
    load_library().mla_reset_counters()


# ---------------------------------------------------------------------------
# Device-side calls (torch tensors in, pointers out).
# ---------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return MLA_F16
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    raise MlaError(-6, f"16-bit tensors must be float16 or bfloat16, got {t.dtype}")


def _query_shape(q_absorbed, q_len):
    """(batch, heads per new token, q_len) of [B, Q, H, 512] or [B, Q*H, 512]."""
    if q_absorbed.dim() == 4:
        return int(q_absorbed.shape[0]), int(q_absorbed.shape[2]), int(q_absorbed.shape[1])
    q = int(q_len or 1)
    return int(q_absorbed.shape[0]), int(q_absorbed.shape[1]) // q, q


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise MlaError(-1, "device tensors are required (torch CUDA/HIP tensors)")


# Argument checks made before any pointer crosses the ABI: the library sees
# only pointers and sizes, so a tensor that is non-contiguous, of the wrong
# element type or smaller than its declared shape would be read or written
# out of bounds on the device. Every check raises MlaError: -2 (MLA_E_SHAPE)
# for layout and shape, -6 (MLA_E_UNSUPPORTED) for element types.

def _tensor(t, name, dtypes, shape=None, numel=None, optional=False, min_numel=None):
    """Check one tensor: present (unless optional), contiguous, of one of
    `dtypes` (torch dtypes), and of `shape` (None entries are free), of
    `numel` elements, or of at least `min_numel`."""
    if t is None:
        if optional:
            return
        raise MlaError(-1, f"{name} is required")
    if t.dtype not in dtypes:
        raise MlaError(-6, f"{name}: dtype {t.dtype}, need {' or '.join(str(d) for d in dtypes)}")
    if not t.is_contiguous():
        raise MlaError(-2, f"{name} must be contiguous")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(g) != int(w)
                                        for g, w in zip(t.shape, shape)):
            want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
            raise MlaError(-2, f"{name}: shape {list(t.shape)}, need {want}")
    if numel is not None and t.numel() != int(numel):
        raise MlaError(-2, f"{name}: {t.numel()} elements, need {int(numel)}")
    if min_numel is not None and t.numel() < int(min_numel):
        raise MlaError(-2, f"{name}: {t.numel()} elements, need at least {int(min_numel)}")


def _same_device(*ts):
    devs = {str(t.device) for t in ts if t is not None}
    if len(devs) > 1:
        raise MlaError(-2, f"tensors on different devices: {sorted(devs)}")


def _f16_types():
    import torch
    return (torch.float16, torch.bfloat16)


def _check_decode_args(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table, context_lens,
                       partitions, splits, row_indptr, total_rows, partial_out, partial_lse2,
                       out, lse2_out, debug_ranges, q_len, cache_dtypes,
                       caller_workspace=True):
    """Shapes and types of a partition launch; returns (B, H, Q). Without
    caller workspace (the library's own scratch) `out` is always needed."""
    import torch
    f16 = _f16_types()
    i32 = (torch.int32,)
    f32 = (torch.float32,)
    if q_absorbed is None:
        raise MlaError(-1, "q_absorbed is required")
    if q_absorbed.dim() not in (3, 4) or int(q_absorbed.shape[-1]) != KV_LORA_RANK:
        raise MlaError(-2, f"q_absorbed: shape {list(q_absorbed.shape)}, need [B, Q*H, 512] "
                           f"or [B, Q, H, 512]")
    B, H, Q = _query_shape(q_absorbed, q_len)
    if Q < 1 or (q_absorbed.dim() == 3 and int(q_absorbed.shape[1]) != Q * H):
        raise MlaError(-2, f"q_absorbed: {int(q_absorbed.shape[1])} rows is not q_len "
                           f"{Q} x heads")
    _tensor(q_absorbed, "q_absorbed", f16)
    qd = (q_absorbed.dtype,)
    _tensor(q_pe, "q_pe", qd, numel=B * Q * H * ROPE_DIM)
    if q_pe.shape[0] != B or int(q_pe.shape[-1]) != ROPE_DIM:
        raise MlaError(-2, f"q_pe: shape {list(q_pe.shape)}, need [B, Q*H, 64] or [B, Q, H, 64]")
    _tensor(ckv_cache, "ckv_cache", cache_dtypes, shape=(None, None, KV_LORA_RANK))
    nb, bs = int(ckv_cache.shape[0]), int(ckv_cache.shape[1])
    _tensor(kpe_cache, "kpe_cache", (ckv_cache.dtype,), shape=(nb, bs, ROPE_DIM))
    _tensor(block_table, "block_table", i32, shape=(B, None))
    _tensor(context_lens, "context_lens", i32, shape=(B,))
    rows = int(total_rows)
    split = rows != B
    _tensor(partitions, "partitions", i32, shape=(B,), optional=not split)
    _tensor(splits, "splits", i32, shape=(B,), optional=not split)
    _tensor(row_indptr, "row_indptr", i32, shape=(B + 1,), optional=not split)
    if caller_workspace:
        _tensor(partial_out, "partial_out", f32, shape=(rows, Q * H, KV_LORA_RANK),
                optional=not split)
        _tensor(partial_lse2, "partial_lse2", f32, shape=(rows, Q * H), optional=not split)
    _tensor(out, "out", qd, numel=B * Q * H * KV_LORA_RANK,
            optional=split and caller_workspace)
    if out is not None and int(out.shape[0]) != B:
        raise MlaError(-2, f"out: shape {list(out.shape)}, need [B, Q*H, 512]")
    _tensor(lse2_out, "lse2_out", f32, numel=B * Q * H, optional=True)
    _tensor(debug_ranges, "debug_ranges", i32, min_numel=2 * rows, optional=True)
    _same_device(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table, context_lens, partitions,
                 splits, row_indptr, partial_out, partial_lse2, out, lse2_out, debug_ranges)
    return B, H, Q


def mla_decode_partition(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table, context_lens,
                         scale: float, partitions, splits, row_indptr, total_rows: int,
                         max_rows_per_req: int, heads_per_wg: int, partial_out, partial_lse2,
                         out, lse2_out=None, debug_ranges=None, stream=None, q_len=None):
    """Launch the partition kernel (see include/mla_decode.h). q_absorbed is
    [B, H, 512], or [B, q_len, H, 512] / [B, q_len*H, 512] for several new
    tokens per request. The cache block size is ckv_cache.shape[1] (16 or
    32), and must be the one the plan was chosen for."""
    lib = load_library()
    B, H, Q = _check_decode_args(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table,
                                 context_lens, partitions, splits, row_indptr, total_rows,
                                 partial_out, partial_lse2, out, lse2_out, debug_ranges, q_len,
                                 _f16_types())
    if ckv_cache.dtype != q_absorbed.dtype:
        raise MlaError(-6, f"ckv_cache dtype {ckv_cache.dtype} differs from q_absorbed's")
    _need_cuda(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table, context_lens)
    _check(lib.mla_decode_partition(
        _ptr(q_absorbed), _ptr(q_pe), _ptr(ckv_cache), _ptr(kpe_cache), int(ckv_cache.shape[0]),
        int(ckv_cache.shape[1]), _ptr(block_table), int(block_table.shape[1]), _ptr(context_lens), B, H, Q,
        float(scale), _dtype_code(q_absorbed), _ptr(partitions), _ptr(splits), _ptr(row_indptr),
        int(total_rows), int(max_rows_per_req), int(heads_per_wg), _ptr(partial_out),
        _ptr(partial_lse2), _ptr(out), _ptr(lse2_out), _ptr(debug_ranges), _stream(stream)))


def mla_decode_partition_fp8(q_absorbed, q_pe, ckv_cache, kpe_cache, kv_scale: float,
                             block_table, context_lens, scale: float, partitions, splits,
                             row_indptr, total_rows: int, max_rows_per_req: int,
                             heads_per_wg: int, partial_out, partial_lse2, out, lse2_out=None,
                             debug_ranges=None, stream=None, q_len=None):
    """The partition kernel over an E4M3 byte cache (uint8 tensors
    [num_blocks, block_size, 512] and [.., 64]) times kv_scale (see
    include/mla_decode.h), with 16 or 64 heads per workgroup."""
    import torch
    lib = load_library()
    B, H, Q = _check_decode_args(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table,
                                 context_lens, partitions, splits, row_indptr, total_rows,
                                 partial_out, partial_lse2, out, lse2_out, debug_ranges, q_len,
                                 (torch.uint8,))
    _need_cuda(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table, context_lens)
    _check(lib.mla_decode_partition_fp8(
        _ptr(q_absorbed), _ptr(q_pe), _ptr(ckv_cache), _ptr(kpe_cache), float(kv_scale),
        int(ckv_cache.shape[0]), int(ckv_cache.shape[1]), _ptr(block_table),
        int(block_table.shape[1]), _ptr(context_lens), B, H, Q, float(scale),
        _dtype_code(q_absorbed), _ptr(partitions), _ptr(splits), _ptr(row_indptr),
        int(total_rows), int(max_rows_per_req), int(heads_per_wg), _ptr(partial_out),
        _ptr(partial_lse2), _ptr(out), _ptr(lse2_out), _ptr(debug_ranges), _stream(stream)))


def mla_decode_fused(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table, context_lens,
                     scale: float, partitions, splits, row_indptr, total_rows: int,
                     max_rows_per_req: int, heads_per_wg: int, partial_out, partial_lse2,
                     out, lse2_out, sync, debug_ranges=None, stream=None, q_len=None):
    """Partition and merge in one launch (see include/mla_decode.h)."""
    import torch
    lib = load_library()
    B, H, Q = _check_decode_args(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table,
                                 context_lens, partitions, splits, row_indptr, total_rows,
                                 partial_out, partial_lse2, out, lse2_out, debug_ranges, q_len,
                                 _f16_types())
    if ckv_cache.dtype != q_absorbed.dtype:
        raise MlaError(-6, f"ckv_cache dtype {ckv_cache.dtype} differs from q_absorbed's")
    _tensor(out, "out", (q_absorbed.dtype,), numel=B * Q * H * KV_LORA_RANK)
    if int(total_rows) != B:
        _tensor(sync, "sync", (torch.int64,),
                numel=max(1, B) * FUSED_SYNC_BYTES_PER_REQUEST // 8)
    _same_device(q_absorbed, out, sync)
    _need_cuda(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table, context_lens, out)
    _check(lib.mla_decode_fused(
        _ptr(q_absorbed), _ptr(q_pe), _ptr(ckv_cache), _ptr(kpe_cache), int(ckv_cache.shape[0]),
        int(ckv_cache.shape[1]), _ptr(block_table), int(block_table.shape[1]), _ptr(context_lens), B, H, Q,
        float(scale), _dtype_code(q_absorbed), _ptr(partitions), _ptr(splits), _ptr(row_indptr),
        int(total_rows), int(max_rows_per_req), int(heads_per_wg), _ptr(partial_out),
        _ptr(partial_lse2), _ptr(out), _ptr(lse2_out), _ptr(sync), _ptr(debug_ranges),
        _stream(stream)))


def mla_noalloc_scratch_bytes(total_rows: int, num_heads: int, q_len: int = 1) -> int:
    """Scratch bytes mla_decode_noalloc needs for a plan (see the header)."""
    return int(load_library().mla_noalloc_scratch_bytes(int(total_rows), int(num_heads),
                                                        int(q_len)))


def mla_decode_noalloc(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table, context_lens,
                       scale: float, partitions, splits, row_indptr, total_rows: int,
                       max_rows_per_req: int, heads_per_wg: int, out, lse2_out=None,
                       stream=None, q_len=None):
    """The split decode with its partials in the library's fixed device
    scratch instead of caller memory (see include/mla_decode.h): nothing is
    allocated. Calls that overlap on one GPU race."""
    lib = load_library()
    B, H, Q = _check_decode_args(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table,
                                 context_lens, partitions, splits, row_indptr, total_rows,
                                 None, None, out, lse2_out, None, q_len, _f16_types(),
                                 caller_workspace=False)
    if ckv_cache.dtype != q_absorbed.dtype:
        raise MlaError(-6, f"ckv_cache dtype {ckv_cache.dtype} differs from q_absorbed's")
    _need_cuda(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table, context_lens, out)
    _check(lib.mla_decode_noalloc(
        _ptr(q_absorbed), _ptr(q_pe), _ptr(ckv_cache), _ptr(kpe_cache), int(ckv_cache.shape[0]),
        int(ckv_cache.shape[1]), _ptr(block_table), int(block_table.shape[1]), _ptr(context_lens),
        B, H, Q, float(scale), _dtype_code(q_absorbed), _ptr(partitions), _ptr(splits),
        _ptr(row_indptr), int(total_rows), int(max_rows_per_req), int(heads_per_wg), _ptr(out),
        _ptr(lse2_out), _stream(stream)))


def mla_stream_read(src, sink, stream=None):
    """Measurement helper: one plain contiguous read of the bytes of `src`
    (a contiguous device tensor of 16-byte multiple size); `sink` is a
    device int32/uint32 tensor of at least one element that stays
    untouched as long as no thread's XOR fold of the words it reads is
    0xA5A5A5A5: data whose 4-byte words all keep bit 31 clear qualifies
    (see include/mla_decode.h)."""
    lib = load_library()
    if not src.is_contiguous() or sink.numel() < 1:
        raise MlaError(-2, "src must be contiguous and sink non-empty")
    _need_cuda(src, sink)
    nbytes = src.numel() * src.element_size()
    _check(lib.mla_stream_read(_ptr(src), nbytes, _ptr(sink), 0xA5A5A5A5, _stream(stream)))


def mla_copy_probe(ckv_cache, kpe_cache, table, rows: int, blocks_per_row: int, groups: int,
                   waves: int = 8, inflight: int = 8, stream=None):
    """Measurement helper: copy paged rows' KV into LDS only (see
    include/mla_decode.h); `table` is an int32 device tensor of
    rows * blocks_per_row block indices."""
    import torch
    lib = load_library()
    _tensor(ckv_cache, "ckv_cache", _f16_types(), shape=(None, BLOCK_SIZE, KV_LORA_RANK))
    _tensor(kpe_cache, "kpe_cache", (ckv_cache.dtype,),
            shape=(int(ckv_cache.shape[0]), BLOCK_SIZE, ROPE_DIM))
    _tensor(table, "table", (torch.int32,), numel=int(rows) * int(blocks_per_row))
    _need_cuda(ckv_cache, kpe_cache, table)
    _check(lib.mla_copy_probe(_ptr(ckv_cache), _ptr(kpe_cache), int(ckv_cache.shape[0]),
                              _ptr(table), int(rows), int(blocks_per_row), int(groups),
                              int(waves), int(inflight), _stream(stream)))


def fused_sync_errors(sync) -> int:
    """Waits that ran out in a fused hand-off buffer: the sum of word 4 of
    every 64-byte record (see mla_decode_fused in include/mla_decode.h).
    Non-zero means a merge piece was skipped and `out` is unspecified for
    the requests concerned. Reads the buffer back, so it waits for the
    launches that use it to finish."""
    words = sync.detach().to("cpu").view(-1)
    return int(words.view(-1, 8)[:, 4].sum().item())


def mla_decode_reduce(partial_out, partial_lse2, row_indptr, batch: int, num_heads: int,
                      total_rows: int, out, lse2_out=None, stream=None):
    """Launch the LSE-weighted reduce (see include/mla_decode.h)."""
    import torch
    lib = load_library()
    rows, B, H = int(total_rows), int(batch), int(num_heads)
    _tensor(partial_out, "partial_out", (torch.float32,), shape=(rows, H, KV_LORA_RANK))
    _tensor(partial_lse2, "partial_lse2", (torch.float32,), shape=(rows, H))
    _tensor(row_indptr, "row_indptr", (torch.int32,), shape=(B + 1,))
    _tensor(out, "out", _f16_types(), numel=B * H * KV_LORA_RANK)
    _tensor(lse2_out, "lse2_out", (torch.float32,), numel=B * H, optional=True)
    _same_device(partial_out, partial_lse2, row_indptr, out, lse2_out)
    _need_cuda(partial_out, partial_lse2, row_indptr, out)
    _check(lib.mla_decode_reduce(_ptr(partial_out), _ptr(partial_lse2), _ptr(row_indptr),
                                 int(batch), int(num_heads), int(total_rows), _dtype_code(out),
                                 _ptr(out), _ptr(lse2_out), _stream(stream)))


def _head_product(name, x, w, y, stream):
    lib = load_library()
    _tensor(w, "weights", _f16_types(), shape=(None, None, None))
    heads, din, dout = (int(v) for v in w.shape)
    _tensor(x, "input", (w.dtype,))
    if x.dim() < 2 or int(x.shape[-1]) != din or int(x.shape[-2]) != heads:
        raise MlaError(-2, f"input: shape {list(x.shape)}, need [..., {heads}, {din}]")
    rows = x.numel() // (heads * din) if x.numel() else 0
    _tensor(y, "output", (w.dtype,), numel=rows * heads * dout)
    _same_device(x, w, y)
    _need_cuda(x, w, y)
    _check(getattr(lib, name)(_ptr(x), _ptr(w), _ptr(y), rows, heads, _dtype_code(x),
                              _stream(stream)))


def mla_absorb_query(q_nope, w_uk, q_absorbed, stream=None):
    """q_absorbed[..., h, :] = q_nope[..., h, :] @ w_uk[h] (see include/mla_decode.h)."""
    _head_product("mla_absorb_query", q_nope, w_uk, q_absorbed, stream)


def mla_unabsorb_output(out_latent, w_uv_t, o, stream=None):
    """o[..., h, :] = out_latent[..., h, :] @ w_uv_t[h] (see include/mla_decode.h)."""
    _head_product("mla_unabsorb_output", out_latent, w_uv_t, o, stream)


class DecodePlan:
    """A chooser result with its arrays and workspace on the device."""

    def __init__(self, context_lens, num_heads: int, params: PlanParams | None = None,
                 device="cuda", q_len: int = 1, block_size: int = BLOCK_SIZE):
        import torch
        ctx = [int(c) for c in context_lens]
        self.batch = len(ctx)
        self.heads = num_heads
        self.q_len = int(q_len)
        self.block_size = int(block_size)
        self.info = mla_choose_partitions(self.batch, num_heads, q_len, ctx, params,
                                          block_size=self.block_size)
        i32 = torch.int32
        self.partitions = torch.tensor(self.info["P"], dtype=i32, device=device)
        self.splits = torch.tensor(self.info["S"], dtype=i32, device=device)
        self.row_indptr = torch.tensor(self.info["row_indptr"], dtype=i32, device=device)
        rows = max(1, self.info["total_rows"])
        if self.info["needs_reduce"]:
            qrows = self.q_len * num_heads
            self.partial_out = torch.empty((rows, qrows, KV_LORA_RANK), dtype=torch.float32,
                                           device=device)
            self.partial_lse2 = torch.empty((rows, qrows), dtype=torch.float32, device=device)
        else:
            self.partial_out = self.partial_lse2 = None
        # Hand-off state of the fused launch: zero-filled once, left ready
        # by every completed call.
        self.sync = torch.zeros(max(1, self.batch) * FUSED_SYNC_BYTES_PER_REQUEST // 8,
                                dtype=torch.int64, device=device)

    @property
    def total_rows(self) -> int:
        return self.info["total_rows"]


def decode(plan: DecodePlan, q_absorbed, q_pe, ckv_cache, kpe_cache, block_table, context_lens,
           scale: float, out, lse2_out=None, debug_ranges=None, stream=None, fused=False,
           kv_scale: float | None = None, check_fused: bool = False):
    """Partition launch, then the reduce launch when the plan needs one; with
    fused=True, one launch that merges too (check_fused=True then waits for
    it and raises if a hand-off wait ran out). uint8 caches are E4M3 bytes
    times kv_scale (mla_decode_partition_fp8)."""
    if int(ckv_cache.shape[1]) != plan.block_size:
        raise MlaError(-2, f"cache blocks of {int(ckv_cache.shape[1])} tokens, plan chosen for "
                           f"{plan.block_size}")
    import torch
    if ckv_cache.dtype == torch.uint8:
        if fused:
            raise MlaError(-6, "the fused launch takes 16-bit caches only")
        mla_decode_partition_fp8(q_absorbed, q_pe, ckv_cache, kpe_cache,
                                 1.0 if kv_scale is None else kv_scale, block_table,
                                 context_lens, scale, plan.partitions, plan.splits,
                                 plan.row_indptr, plan.total_rows, plan.info["max_rows_per_req"],
                                 plan.info["heads_per_wg"], plan.partial_out, plan.partial_lse2,
                                 out, lse2_out if not plan.info["needs_reduce"] else None,
                                 debug_ranges, stream, q_len=plan.q_len)
        if plan.info["needs_reduce"]:
            mla_decode_reduce(plan.partial_out, plan.partial_lse2, plan.row_indptr, plan.batch,
                              plan.q_len * plan.heads, plan.total_rows, out, lse2_out, stream)
        return
    if fused:
        mla_decode_fused(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table, context_lens, scale,
                         plan.partitions, plan.splits, plan.row_indptr, plan.total_rows,
                         plan.info["max_rows_per_req"], plan.info["heads_per_wg"],
                         plan.partial_out, plan.partial_lse2, out, lse2_out, plan.sync,
                         debug_ranges, stream, q_len=plan.q_len)
        if check_fused and plan.info["needs_reduce"]:
            missed = fused_sync_errors(plan.sync)
            if missed:
                raise MlaError(-7, f"{missed} fused hand-off waits ran out; out is unspecified")
        return
    mla_decode_partition(q_absorbed, q_pe, ckv_cache, kpe_cache, block_table, context_lens, scale,
                         plan.partitions, plan.splits, plan.row_indptr, plan.total_rows,
                         plan.info["max_rows_per_req"], plan.info["heads_per_wg"],
                         plan.partial_out, plan.partial_lse2, out,
                         lse2_out if not plan.info["needs_reduce"] else None,
                         debug_ranges, stream, q_len=plan.q_len)
    if plan.info["needs_reduce"]:
        mla_decode_reduce(plan.partial_out, plan.partial_lse2, plan.row_indptr, plan.batch,
                          plan.q_len * plan.heads, plan.total_rows, out, lse2_out, stream)
