"""CPU oracle for the DTensor reshard -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``dtensor_layout_movement_amd``) never imports, links or calls it, and it
imports nothing from the product.

The arithmetic lives in ``oracle.cpp`` (plain C++17 built with g++): the
gather-then-slice scheme that the reshard write-ups give as the usual refit path
(techfeed.io, "core problem" section; news.bpdata.com, "why is weight refit a
problem" section): rebuild the global tensor from the source shards, then cut
every destination shard out of it.  This module only marshals arguments.

Placements are ints: ``-1`` is Replicate, ``k >= 0`` is Shard(k).  Layouts with
right-to-left (strided) nesting add one split factor per mesh dim (1 = plain):
``shard_indices`` and ``reshard_indexed`` take them, on explicit per-dim index
lists.  A source mesh dim may also be Partial (``PARTIAL``, sum):
``reshard_partial``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

OK = 0
BAD_LAYOUT = 1
REPLICA_MISMATCH = 2
COVERAGE_MISMATCH = 3
NO_MEMORY = 4
NULL_BUFFER = 5

_I64P = ctypes.POINTER(ctypes.c_int64)
_I32P = ctypes.POINTER(ctypes.c_int32)


def build(out_path: str = _LIB_PATH, source: str = _SRC) -> str:
    """Compile the oracle with g++ into ``out_path`` and return that path."""
    cmd = ["g++", "-std=c++17", "-O2", "-Wall", "-fPIC", "-shared", "-pthread",
           source, "-o", out_path]
    subprocess.run(cmd, check=True)
    return out_path


def load(path: str = _LIB_PATH) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library."""
    global _lib
    if path == _LIB_PATH and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(path)
    lib = ctypes.CDLL(path)
    lib.oracle_num_ranks.argtypes = [ctypes.c_int, _I64P, ctypes.c_int, _I64P, _I32P, _I64P]
    lib.oracle_shard_box.argtypes = [ctypes.c_int, _I64P, ctypes.c_int, _I64P, _I32P,
                                     ctypes.c_int64, _I64P, _I64P]
    lib.oracle_reshard.argtypes = [ctypes.c_int, _I64P, ctypes.c_int64,
                                   ctypes.c_int, _I64P, _I32P, ctypes.POINTER(ctypes.c_void_p),
                                   ctypes.c_int, _I64P, _I32P, ctypes.POINTER(ctypes.c_void_p),
                                   ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
    lib.oracle_convert.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_int]
    lib.oracle_shard_indices.argtypes = [ctypes.c_int, _I64P, ctypes.c_int, _I64P, _I32P, _I64P,
                                         ctypes.c_int64, ctypes.c_int, _I64P, ctypes.c_int64, _I64P]
    lib.oracle_reshard_indexed.argtypes = [ctypes.c_int, _I64P, ctypes.c_int64,
                                           ctypes.c_int, _I64P, _I32P, _I64P, ctypes.POINTER(ctypes.c_void_p),
                                           ctypes.c_int, _I64P, _I32P, _I64P, ctypes.POINTER(ctypes.c_void_p),
                                           ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
    lib.oracle_reshard_partial.argtypes = [ctypes.c_int, _I64P, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, _I64P, _I32P, ctypes.POINTER(ctypes.c_void_p),
                                           ctypes.c_int, _I64P, _I32P, ctypes.POINTER(ctypes.c_void_p),
                                           ctypes.c_int, ctypes.c_int]
    for f in (lib.oracle_num_ranks, lib.oracle_shard_box, lib.oracle_reshard, lib.oracle_convert,
              lib.oracle_shard_indices, lib.oracle_reshard_indexed, lib.oracle_reshard_partial):
        f.restype = ctypes.c_int
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _i64(xs: Sequence[int]):
    return (ctypes.c_int64 * max(1, len(xs)))(*xs)


def _i32(xs: Sequence[int]):
    return (ctypes.c_int32 * max(1, len(xs)))(*xs)


class OracleError(RuntimeError):
    def __init__(self, code: int):
        names = {1: "bad layout", 2: "replica mismatch", 3: "coverage mismatch",
                 4: "out of memory", 5: "NULL buffer for a non-empty shard"}
        super().__init__(f"oracle error {code}: {names.get(code, '?')}")
        self.code = code


def num_ranks(shape, mesh, placements, lib=None) -> int:
    lib = lib or load()
    out = ctypes.c_int64(0)
    rc = lib.oracle_num_ranks(len(shape), _i64(shape), len(mesh), _i64(mesh),
                              _i32(placements), ctypes.byref(out))
    if rc:
        raise OracleError(rc)
    return out.value


def shard_box(shape, mesh, placements, rank, lib=None):
    """Return ``(lo, hi)`` lists: the half-open box that ``rank`` holds."""
    lib = lib or load()
    lo = (ctypes.c_int64 * len(shape))()
    hi = (ctypes.c_int64 * len(shape))()
    rc = lib.oracle_shard_box(len(shape), _i64(shape), len(mesh), _i64(mesh),
                              _i32(placements), rank, lo, hi)
    if rc:
        raise OracleError(rc)
    return list(lo), list(hi)


def _addr(buf) -> int | None:
    if buf is None:
        return None
    if hasattr(buf, "data_ptr"):           # torch CPU tensor
        if buf.device.type != "cpu" or not buf.is_contiguous():
            raise ValueError("oracle buffers must be contiguous CPU tensors")
        return buf.data_ptr() if buf.numel() else None
    iface = buf.__array_interface__        # numpy array
    return iface["data"][0] if buf.size else None


def reshard(shape, elem_size, src_mesh, src_pl, src_bufs, dst_mesh, dst_pl, dst_bufs,
            global_out=None, check: bool = True, threads: int = 1, lib=None) -> None:
    """Gather-then-slice: fill every ``dst_bufs[d]`` from ``src_bufs``.

    Buffers are contiguous CPU tensors / numpy arrays (or None for empty shards),
    one per rank in row-major mesh order.  Raises OracleError on a failed check.
    """
    lib = lib or load()
    srcs = (ctypes.c_void_p * max(1, len(src_bufs)))(*[_addr(b) for b in src_bufs])
    dsts = (ctypes.c_void_p * max(1, len(dst_bufs)))(*[_addr(b) for b in dst_bufs])
    rc = lib.oracle_reshard(len(shape), _i64(shape), elem_size,
                            len(src_mesh), _i64(src_mesh), _i32(src_pl), srcs,
                            len(dst_mesh), _i64(dst_mesh), _i32(dst_pl), dsts,
                            _addr(global_out), int(check), int(threads))
    if rc:
        raise OracleError(rc)


def shard_indices(shape, mesh, placements, split, rank, lib=None):
    """Per tensor dim, the list of global indices ``rank`` holds, in local
    order, under a layout whose mesh dims have split factors ``split`` (1 for a
    plain Shard or Replicate).  The local shard is the row-major buffer over the
    product of these lists."""
    lib = lib or load()
    out = []
    for dim in range(len(shape)):
        n = ctypes.c_int64(0)
        buf = (ctypes.c_int64 * max(1, shape[dim]))()
        rc = lib.oracle_shard_indices(len(shape), _i64(shape), len(mesh), _i64(mesh), _i32(placements),
                                      _i64(split), rank, dim, buf, max(1, shape[dim]), ctypes.byref(n))
        if rc:
            raise OracleError(rc)
        out.append(list(buf[:n.value]))
    return out


def reshard_indexed(shape, elem_size, src_mesh, src_pl, src_split, src_bufs, dst_mesh, dst_pl, dst_split,
                    dst_bufs, global_out=None, check: bool = True, threads: int = 1, lib=None) -> None:
    """Gather-then-slice over explicit index lists (layouts with split factors):
    fill every ``dst_bufs[d]`` from ``src_bufs``.  Buffers as for ``reshard``;
    a shard's buffer is row-major over its ``shard_indices`` lists."""
    lib = lib or load()
    srcs = (ctypes.c_void_p * max(1, len(src_bufs)))(*[_addr(b) for b in src_bufs])
    dsts = (ctypes.c_void_p * max(1, len(dst_bufs)))(*[_addr(b) for b in dst_bufs])
    rc = lib.oracle_reshard_indexed(len(shape), _i64(shape), elem_size,
                                    len(src_mesh), _i64(src_mesh), _i32(src_pl), _i64(src_split), srcs,
                                    len(dst_mesh), _i64(dst_mesh), _i32(dst_pl), _i64(dst_split), dsts,
                                    _addr(global_out), int(check), int(threads))
    if rc:
        raise OracleError(rc)


# Float formats of oracle_convert, by name.
FORMATS = {"f32": 0, "bf16": 1, "f16": 2}

# Placement code of a Partial (sum) mesh dim in a source layout.
PARTIAL = -2


def reshard_partial(shape, src_fmt: str, dst_fmt: str, src_mesh, src_pl, src_bufs, dst_mesh, dst_pl, dst_bufs,
                    check: bool = True, threads: int = 1, lib=None) -> None:
    """Reshard from a source layout with Partial mesh dims (placement ``PARTIAL``):
    every destination element is the sum of the contributions, in contribution
    order, in binary32, rounded once to ``dst_fmt`` ("f32", "bf16", "f16").
    Buffers as for ``reshard``; the source shards hold ``src_fmt`` elements."""
    lib = lib or load()
    srcs = (ctypes.c_void_p * max(1, len(src_bufs)))(*[_addr(b) for b in src_bufs])
    dsts = (ctypes.c_void_p * max(1, len(dst_bufs)))(*[_addr(b) for b in dst_bufs])
    rc = lib.oracle_reshard_partial(len(shape), _i64(shape), FORMATS[src_fmt], FORMATS[dst_fmt],
                                    len(src_mesh), _i64(src_mesh), _i32(src_pl), srcs,
                                    len(dst_mesh), _i64(dst_mesh), _i32(dst_pl), dsts, int(check), int(threads))
    if rc:
        raise OracleError(rc)


def convert(values, from_fmt: str, to_fmt: str, threads: int = 1, lib=None):
    """Convert a contiguous CPU torch tensor of `from_fmt` elements to `to_fmt`
    ("f32", "bf16", "f16"): round to nearest, ties to even; NaN keeps its sign
    and leading payload bits and becomes quiet.  Returns a new tensor."""
    import torch
    lib = lib or load()
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
    if values.dtype != dt[from_fmt] or not values.is_contiguous() or values.device.type != "cpu":
        raise ValueError("convert needs a contiguous CPU tensor of the source format")
    out = torch.empty(values.shape, dtype=dt[to_fmt])
    if values.numel():
        rc = lib.oracle_convert(FORMATS[from_fmt], FORMATS[to_fmt], values.data_ptr(), out.data_ptr(),
                                values.numel(), int(threads))
        if rc:
            raise OracleError(rc)
    return out
