"""Python binding of the reshard C ABI (``include/reshard.h``).

Argument marshalling only: every function here forwards to the function of the
same name in ``libreshard.so``, which does all planning on the host and all data
movement in its gfx950 kernel.  There is no fallback: if the library is not
built, every call raises.

Placements are ints: ``REPLICATE`` (-1) or a tensor dim ``k`` for Shard(k).
Pointers are plain ints (device addresses, e.g. ``tensor.data_ptr()``); 0 or
None stands for an empty shard.  ``stream`` is a ``hipStream_t`` as an int (for
torch: ``torch.cuda.current_stream().cuda_stream``) or None for the default
stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libreshard.so")

REPLICATE = -1
PARTIAL = -2  # Partial (sum): source layouts only
MAX_NDIM = 8

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_LAYOUT_MISMATCH = 2
ERR_NULL_SHARD = 3
ERR_OUT_OF_MEMORY = 4
ERR_HIP = 5
ERR_DEVICE_MISMATCH = 6

DTYPE_U8, DTYPE_I8, DTYPE_BOOL, DTYPE_FP8_E4M3, DTYPE_FP8_E5M2 = 0, 1, 2, 3, 4
DTYPE_BF16, DTYPE_F16, DTYPE_I16 = 5, 6, 7
DTYPE_F32, DTYPE_I32 = 8, 9
DTYPE_F64, DTYPE_I64 = 10, 11

DESC_ITEMS = 0       # rows of items of `unit` bytes
DESC_DST_CHUNKS = 1  # rows cut into destination-aligned 16-byte chunks
DESC_WINDOW = 2      # a band of rows staged through an LDS window
DESC_CONVERT = 3     # rows of elements converted to another float format (run in elements)
DESC_GATHER_ROWS = 4  # whole destination rows gathered from wide source column segments
DESC_REDUCE = 5      # rows of elements summed over Partial contributions (run in elements)

# conversions: the `unit` of a DESC_CONVERT descriptor
CONVERT_F32_BF16 = 1
CONVERT_F32_F16 = 2
CONVERT_BF16_F32 = 3
CONVERT_F16_F32 = 4

EXPORTED = (
    "reshard_dtype_size", "reshard_layout_create", "reshard_layout_destroy",
    "reshard_layout_create_strided", "reshard_layout_shard_runs",
    "reshard_layout_num_ranks", "reshard_layout_shard_box", "reshard_plan_create",
    "reshard_plan_create_batched", "reshard_plan_upload", "reshard_execute", "reshard_execute_noalloc",
    "reshard_plan_stats", "reshard_plan_src_load", "reshard_plan_pieces", "reshard_plan_piece_sources",
    "reshard_plan_device_refs", "reshard_plan_device_segments",
    "reshard_plan_piece_fanout",
    "reshard_plan_descriptors", "reshard_plan_segments", "reshard_plan_destroy",
    "reshard_last_error",
)


class ReshardError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"reshard status {status}: {message}")
        self.status = status


class PlanStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "n_tensors", "n_src_ptrs", "n_dst_ptrs", "n_pieces", "n_dst_writes", "global_bytes",
        "bytes_read", "bytes_written", "n_descriptors", "table_bytes", "n_workgroups", "n_launches")] + [
        ("plan_host_us", ctypes.c_double)]


class Piece(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int64), ("src_rank", ctypes.c_int64),
                ("src_group", ctypes.c_int64), ("dst_group", ctypes.c_int64),
                ("fanout", ctypes.c_int64), ("lo", ctypes.c_int64 * MAX_NDIM),
                ("hi", ctypes.c_int64 * MAX_NDIM), ("src_local", ctypes.c_int64 * MAX_NDIM),
                ("dst_local", ctypes.c_int64 * MAX_NDIM)]


class Descriptor(ctypes.Structure):
    _fields_ = [("src_offset", ctypes.c_int64), ("dst_offset", ctypes.c_int64),
                ("src_stride", ctypes.c_int64 * 3), ("dst_stride", ctypes.c_int64 * 3),
                ("extent", ctypes.c_uint32 * 3), ("run_bytes", ctypes.c_uint32),
                ("row_items", ctypes.c_uint32), ("unit", ctypes.c_uint16), ("mode", ctypes.c_uint16),
                ("src_ptr", ctypes.c_uint32), ("dst_ref_begin", ctypes.c_uint32),
                ("fanout", ctypes.c_uint32), ("magic", (ctypes.c_uint32 * 2) * 3),
                ("piece", ctypes.c_uint32)]


assert ctypes.sizeof(Descriptor) == 128


class Segment(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("row_stride", ctypes.c_int64), ("col", ctypes.c_uint32),
                ("width", ctypes.c_uint32), ("ptr", ctypes.c_uint32), ("fanout", ctypes.c_uint32)]


assert ctypes.sizeof(Segment) == 32

_lib = None
_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_I64P = ctypes.POINTER(ctypes.c_int64)


def library_path() -> str:
    return LIB_PATH


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m dtensor_layout_movement_amd.build` "
            "(the reshard path has no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int
    sig = {
        "reshard_dtype_size": (_I64, [ctypes.c_int]),
        "reshard_layout_create": (st, [ctypes.c_int, _I64P, ctypes.c_int, ctypes.c_int, _I64P,
                                       ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(_VP)]),
        "reshard_layout_create_strided": (st, [ctypes.c_int, _I64P, ctypes.c_int, ctypes.c_int, _I64P,
                                               ctypes.POINTER(ctypes.c_int32), _I64P, ctypes.POINTER(_VP)]),
        "reshard_layout_shard_runs": (st, [_VP, _I64, ctypes.c_int, _I64, _I64P, _I64P]),
        "reshard_layout_destroy": (None, [_VP]),
        "reshard_layout_num_ranks": (st, [_VP, _I64P]),
        "reshard_layout_shard_box": (st, [_VP, _I64, _I64P, _I64P]),
        "reshard_plan_create": (st, [_VP, _VP, ctypes.POINTER(_VP)]),
        "reshard_plan_create_batched": (st, [ctypes.c_int, ctypes.POINTER(_VP), ctypes.POINTER(_VP),
                                             ctypes.POINTER(_VP)]),
        "reshard_plan_upload": (st, [_VP, _VP]),
        "reshard_execute": (st, [_VP, ctypes.POINTER(_VP), ctypes.POINTER(_VP), _VP]),
        "reshard_execute_noalloc": (st, [_VP, ctypes.POINTER(_VP), ctypes.POINTER(_VP), _VP]),
        "reshard_plan_stats": (st, [_VP, ctypes.POINTER(PlanStats)]),
        "reshard_plan_src_load": (st, [_VP, _I64, _I64P, _I64P]),
        "reshard_plan_pieces": (st, [_VP, _I64, ctypes.POINTER(Piece), _I64P]),
        "reshard_plan_piece_fanout": (st, [_VP, _I64, _I64, _I64P, _I64P]),
        "reshard_plan_piece_sources": (st, [_VP, _I64, _I64, _I64P, _I64P]),
        "reshard_plan_device_refs": (st, [_VP, _I64, ctypes.POINTER(ctypes.c_uint32), _I64P]),
        "reshard_plan_device_segments": (st, [_VP, _I64, ctypes.POINTER(Segment), _I64P]),
        "reshard_plan_descriptors": (st, [_VP, _I64, ctypes.POINTER(Descriptor), _I64P, _I64,
                                          ctypes.POINTER(ctypes.c_uint32), _I64P]),
        "reshard_plan_segments": (st, [_VP, _I64, ctypes.POINTER(Segment), _I64P]),
        "reshard_plan_destroy": (None, [_VP]),
        "reshard_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != OK:
        raise ReshardError(status, (_load().reshard_last_error() or b"").decode())


def _i64s(xs: Sequence[int]):
    return (ctypes.c_int64 * max(1, len(xs)))(*[int(x) for x in xs])


def dtype_code(dtype) -> int:
    """Map a torch dtype (or a name such as "bf16") to a reshard dtype code."""
    import torch
    table = {
        torch.uint8: DTYPE_U8, torch.int8: DTYPE_I8, torch.bool: DTYPE_BOOL,
        torch.float8_e4m3fn: DTYPE_FP8_E4M3, torch.float8_e5m2: DTYPE_FP8_E5M2,
        torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16, torch.int16: DTYPE_I16,
        torch.float32: DTYPE_F32, torch.int32: DTYPE_I32,
        torch.float64: DTYPE_F64, torch.int64: DTYPE_I64,
    }
    return table[dtype]


def reshard_dtype_size(dtype: int) -> int:
    return int(_load().reshard_dtype_size(int(dtype)))


def reshard_layout_create(global_shape: Sequence[int], dtype: int, mesh_shape: Sequence[int],
                          placements: Sequence[int]) -> int:
    out = _VP()
    pl = (ctypes.c_int32 * max(1, len(placements)))(*[int(p) for p in placements])
    _check(_load().reshard_layout_create(len(global_shape), _i64s(global_shape), int(dtype),
                                         len(mesh_shape), _i64s(mesh_shape), pl, ctypes.byref(out)))
    return out.value


def reshard_layout_create_strided(global_shape: Sequence[int], dtype: int, mesh_shape: Sequence[int],
                                  placements: Sequence[int], split_factors: Sequence[int]) -> int:
    out = _VP()
    pl = (ctypes.c_int32 * max(1, len(placements)))(*[int(p) for p in placements])
    _check(_load().reshard_layout_create_strided(len(global_shape), _i64s(global_shape), int(dtype),
                                                 len(mesh_shape), _i64s(mesh_shape), pl, _i64s(split_factors),
                                                 ctypes.byref(out)))
    return out.value


def reshard_layout_shard_runs(layout: int, rank: int, dim: int) -> list[tuple[int, int]]:
    """The runs ``(lo, hi)`` of global indices ``rank`` holds along ``dim``."""
    n = ctypes.c_int64()
    _check(_load().reshard_layout_shard_runs(layout, int(rank), int(dim), 0, None, ctypes.byref(n)))
    buf = (ctypes.c_int64 * max(2, 2 * n.value))()
    _check(_load().reshard_layout_shard_runs(layout, int(rank), int(dim), n.value, buf, ctypes.byref(n)))
    return [(buf[2 * i], buf[2 * i + 1]) for i in range(n.value)]


def layout_create(global_shape: Sequence[int], dtype: int, mesh_shape: Sequence[int], placements: Sequence[int],
                  split_factors: Sequence[int] | None = None) -> int:
    """reshard_layout_create, or reshard_layout_create_strided when some split
    factor is above 1 (None: all 1)."""
    if split_factors is not None and any(int(f) != 1 for f in split_factors):
        return reshard_layout_create_strided(global_shape, dtype, mesh_shape, placements, split_factors)
    return reshard_layout_create(global_shape, dtype, mesh_shape, placements)


def local_shape(layout: int, rank: int, ndim: int) -> list[int]:
    """Shape of ``rank``'s local shard (any layout): per dim, the total length
    of its runs."""
    return [sum(b - a for a, b in reshard_layout_shard_runs(layout, rank, k)) for k in range(ndim)]


def reshard_layout_destroy(layout: int) -> None:
    _load().reshard_layout_destroy(layout)


def reshard_layout_num_ranks(layout: int) -> int:
    out = ctypes.c_int64()
    _check(_load().reshard_layout_num_ranks(layout, ctypes.byref(out)))
    return out.value


def reshard_layout_shard_box(layout: int, rank: int, ndim: int):
    """Return ``(offset, extent)`` of ``rank``'s box (ndim = tensor rank)."""
    off = (ctypes.c_int64 * MAX_NDIM)()
    ext = (ctypes.c_int64 * MAX_NDIM)()
    _check(_load().reshard_layout_shard_box(layout, int(rank), off, ext))
    return list(off[:ndim]), list(ext[:ndim])


def reshard_plan_create(src_layout: int, dst_layout: int) -> int:
    out = _VP()
    _check(_load().reshard_plan_create(src_layout, dst_layout, ctypes.byref(out)))
    return out.value


def reshard_plan_create_batched(src_layouts: Sequence[int], dst_layouts: Sequence[int]) -> int:
    n = len(src_layouts)
    if len(dst_layouts) != n:
        raise ValueError("need as many destination layouts as source layouts")
    out = _VP()
    s = (_VP * max(1, n))(*src_layouts)
    d = (_VP * max(1, n))(*dst_layouts)
    _check(_load().reshard_plan_create_batched(n, s, d, ctypes.byref(out)))
    return out.value


def reshard_plan_upload(plan: int, stream: int | None = None) -> None:
    _check(_load().reshard_plan_upload(plan, stream or None))


def pointer_array(ptrs: Sequence[int | None]):
    """Build the ctypes pointer array reshard_execute takes (reusable across calls)."""
    return (_VP * max(1, len(ptrs)))(*[p or None for p in ptrs])


def reshard_execute(plan: int, src_ptrs, dst_ptrs, stream: int | None = None) -> None:
    """Launch the reshard on ``stream``.  ``src_ptrs``/``dst_ptrs`` are sequences of
    device addresses or arrays made by ``pointer_array``."""
    if not isinstance(src_ptrs, ctypes.Array):
        src_ptrs = pointer_array(src_ptrs)
    if not isinstance(dst_ptrs, ctypes.Array):
        dst_ptrs = pointer_array(dst_ptrs)
    _check(_load().reshard_execute(plan, src_ptrs, dst_ptrs, stream or None))


def reshard_execute_noalloc(plan: int, src_ptrs, dst_ptrs, stream: int | None = None) -> None:
    """reshard_execute with the plan's table in the library's static device array
    (no allocation; calls that overlap on one GPU race)."""
    if not isinstance(src_ptrs, ctypes.Array):
        src_ptrs = pointer_array(src_ptrs)
    if not isinstance(dst_ptrs, ctypes.Array):
        dst_ptrs = pointer_array(dst_ptrs)
    _check(_load().reshard_execute_noalloc(plan, src_ptrs, dst_ptrs, stream or None))


NOALLOC_SCRATCH_BYTES = 2 << 20


def reshard_plan_stats(plan: int) -> dict:
    out = PlanStats()
    _check(_load().reshard_plan_stats(plan, ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in PlanStats._fields_}


def reshard_plan_src_load(plan: int) -> list[int]:
    """Bytes read from each source pointer slot by one execute (src_ptrs order)."""
    n = ctypes.c_int64()
    _check(_load().reshard_plan_src_load(plan, 0, None, ctypes.byref(n)))
    arr = (ctypes.c_int64 * max(1, n.value))()
    _check(_load().reshard_plan_src_load(plan, n.value, arr, ctypes.byref(n)))
    return list(arr[:n.value])


def reshard_plan_pieces(plan: int) -> list[dict]:
    n = ctypes.c_int64()
    _check(_load().reshard_plan_pieces(plan, 0, None, ctypes.byref(n)))
    arr = (Piece * max(1, n.value))()
    _check(_load().reshard_plan_pieces(plan, n.value, arr, ctypes.byref(n)))
    return [{"tensor": p.tensor, "src_rank": p.src_rank, "src_group": p.src_group,
             "dst_group": p.dst_group, "fanout": p.fanout, "lo": list(p.lo), "hi": list(p.hi),
             "src_local": list(p.src_local), "dst_local": list(p.dst_local)}
            for p in arr[:n.value]]


def reshard_plan_device_refs(plan: int) -> list[int]:
    """The fan-out list as the kernel reads it from the device table: absolute
    slots of the pointer array (sources, then destinations)."""
    n = ctypes.c_int64()
    _check(_load().reshard_plan_device_refs(plan, 0, None, ctypes.byref(n)))
    arr = (ctypes.c_uint32 * max(1, n.value))()
    _check(_load().reshard_plan_device_refs(plan, n.value, arr, ctypes.byref(n)))
    return list(arr[:n.value])


def reshard_plan_device_segments(plan: int) -> list[dict]:
    """The segment table as the kernel reads it (see the C header)."""
    n = ctypes.c_int64()
    _check(_load().reshard_plan_device_segments(plan, 0, None, ctypes.byref(n)))
    arr = (Segment * max(1, n.value))()
    _check(_load().reshard_plan_device_segments(plan, n.value, arr, ctypes.byref(n)))
    return [{name: getattr(x, name) for name, _ in Segment._fields_} for x in arr[:n.value]]


def reshard_plan_piece_sources(plan: int, index: int) -> list[int]:
    """Source ranks piece ``index`` reads, in contribution order."""
    n = ctypes.c_int64()
    _check(_load().reshard_plan_piece_sources(plan, int(index), 0, None, ctypes.byref(n)))
    arr = (ctypes.c_int64 * max(1, n.value))()
    _check(_load().reshard_plan_piece_sources(plan, int(index), n.value, arr, ctypes.byref(n)))
    return list(arr[:n.value])


def reshard_plan_piece_fanout(plan: int, index: int) -> list[int]:
    n = ctypes.c_int64()
    _check(_load().reshard_plan_piece_fanout(plan, int(index), 0, None, ctypes.byref(n)))
    arr = (ctypes.c_int64 * max(1, n.value))()
    _check(_load().reshard_plan_piece_fanout(plan, int(index), n.value, arr, ctypes.byref(n)))
    return list(arr[:n.value])


def reshard_plan_descriptors(plan: int):
    """Return ``(descriptors, refs)``: the device table as a list of dicts and the
    fan-out list (indices into the destination pointer array)."""
    nd, nr = ctypes.c_int64(), ctypes.c_int64()
    _check(_load().reshard_plan_descriptors(plan, 0, None, ctypes.byref(nd), 0, None,
                                            ctypes.byref(nr)))
    descs = (Descriptor * max(1, nd.value))()
    refs = (ctypes.c_uint32 * max(1, nr.value))()
    _check(_load().reshard_plan_descriptors(plan, nd.value, descs, ctypes.byref(nd), nr.value,
                                            refs, ctypes.byref(nr)))
    out = []
    for d in descs[:nd.value]:
        out.append({
            "src_offset": d.src_offset, "dst_offset": d.dst_offset,
            "src_stride": list(d.src_stride), "dst_stride": list(d.dst_stride),
            "extent": list(d.extent), "run_bytes": d.run_bytes, "row_items": d.row_items,
            "unit": d.unit, "mode": d.mode,
            "src_ptr": d.src_ptr, "dst_ref_begin": d.dst_ref_begin, "fanout": d.fanout,
            "magic": [list(m) for m in d.magic], "piece": d.piece,
        })
    return out, list(refs[:nr.value])


def reshard_plan_segments(plan: int) -> list[dict]:
    """Segments of the plan's window descriptors (see reshard_segment_t)."""
    n = ctypes.c_int64()
    _check(_load().reshard_plan_segments(plan, 0, None, ctypes.byref(n)))
    arr = (Segment * max(1, n.value))()
    _check(_load().reshard_plan_segments(plan, n.value, arr, ctypes.byref(n)))
    return [{"offset": x.offset, "row_stride": x.row_stride, "col": x.col, "width": x.width,
             "ptr": x.ptr, "fanout": x.fanout} for x in arr[:n.value]]


def reshard_plan_destroy(plan: int) -> None:
    _load().reshard_plan_destroy(plan)


def reshard_last_error() -> str:
    return (_load().reshard_last_error() or b"").decode()
