"""Test-side helpers around the reshard library: plans for workload specs, and
two host-side *interpreters* of a plan that exist only in the tests:

* ``apply_pieces``      -- applies the planned overlaps (global boxes) with torch
  slicing, checking the planner's intersections and replica choice;
* ``run_descriptors``   -- walks the device descriptor table byte by byte the way
  the kernel reads it (rows, strides, unit, fan-out), checking dim merging,
  splitting and offsets.

Neither is reachable from the product library, which has no CPU copy path.
"""
from __future__ import annotations

import numpy as np
import torch

import dtensor_layout_movement_amd as R
import oracle
from dtensor_layout_movement_amd import workloads as W


class Plan:
    """A plan for a list of TensorSpecs plus its layouts (freed on close)."""

    def __init__(self, specs):
        self.specs = list(specs)
        self.src_layouts, self.dst_layouts = [], []
        for t in self.specs:
            self.src_layouts.append(make_layout(t, "src"))
            self.dst_layouts.append(make_layout(t, "dst"))
        self.handle = R.reshard_plan_create_batched(self.src_layouts, self.dst_layouts)

    def src_boxes(self, t):
        return lib_boxes(self.src_layouts[t], self.specs[t].shape)

    def dst_boxes(self, t):
        return lib_boxes(self.dst_layouts[t], self.specs[t].shape)

    def src_shapes(self, t):
        return lib_shapes(self.src_layouts[t], self.specs[t].shape)

    def dst_shapes(self, t):
        return lib_shapes(self.dst_layouts[t], self.specs[t].shape)

    def stats(self):
        return R.reshard_plan_stats(self.handle)

    def close(self):
        if self.handle:
            R.reshard_plan_destroy(self.handle)
            self.handle = None
        for lay in self.src_layouts + self.dst_layouts:
            R.reshard_layout_destroy(lay)
        self.src_layouts, self.dst_layouts = [], []

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def make_layout(spec, side):
    """The library layout of one side of a spec (strided when it has split factors)."""
    if side == "src":
        dt, mesh, pl = spec.dtype, spec.src_mesh, spec.src_placements
    else:
        dt, mesh, pl = spec.out_dtype, spec.dst_mesh, spec.dst_placements
    split = spec.split(side)
    if any(f > 1 for f in split):
        return R.reshard_layout_create_strided(spec.shape, R.dtype_code(dt), mesh, pl, split)
    return R.reshard_layout_create(spec.shape, R.dtype_code(dt), mesh, pl)


def lib_runs(layout, shape):
    """Per rank, per dim: the library's runs of global indices."""
    return [[R.reshard_layout_shard_runs(layout, r, k) for k in range(len(shape))]
            for r in range(R.reshard_layout_num_ranks(layout))]


def lib_shapes(layout, shape):
    """Local shard shapes (sum of run lengths per dim), any layout."""
    return [[sum(b - a for a, b in runs) for runs in per_rank] for per_rank in lib_runs(layout, shape)]


def oracle_index_lists(spec, side):
    """Per rank, per dim: the oracle's global index lists."""
    mesh = spec.src_mesh if side == "src" else spec.dst_mesh
    pl = spec.src_placements if side == "src" else spec.dst_placements
    n = int(np.prod(mesh))
    return [oracle.shard_indices(list(spec.shape), list(mesh), list(pl), list(spec.split(side)), r)
            for r in range(n)]


def lib_boxes(layout, shape):
    n = R.reshard_layout_num_ranks(layout)
    out = []
    for r in range(n):
        off, ext = R.reshard_layout_shard_box(layout, r, len(shape))
        out.append(([o for o in off], [o + e for o, e in zip(off, ext)]))
    return out


def oracle_boxes(shape, mesh, placements):
    """The oracle's boxes (a Partial mesh dim splits nothing, like Replicate)."""
    n = 1
    for m in mesh:
        n *= m
    plain = [W.R if p == W.P else p for p in placements]
    return [oracle.shard_box(list(shape), list(mesh), plain, r) for r in range(n)]





def assert_boxes_agree(plan: Plan):
    """The library's boxes (runs, for a strided spec) must equal the oracle's
    before any buffer is sized."""
    for t, spec in enumerate(plan.specs):
        if spec.strided:
            for side, lay in (("src", plan.src_layouts[t]), ("dst", plan.dst_layouts[t])):
                got = [[[i for a, b in runs for i in range(a, b)] for runs in per_rank]
                       for per_rank in lib_runs(lay, spec.shape)]
                assert got == oracle_index_lists(spec, side), (spec, side)
            continue
        assert plan.src_boxes(t) == oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements), spec
        assert plan.dst_boxes(t) == oracle_boxes(spec.shape, spec.dst_mesh, spec.dst_placements), spec


def box_shape(box):
    lo, hi = box
    return [max(0, h - l) for l, h in zip(lo, hi)]


FMT = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}


def oracle_dsts(spec, srcs, threads=1):
    """Destination shards by the oracle (gather-then-slice) from given sources;
    for a converting spec, each shard is then converted by the oracle."""
    es = torch.empty((), dtype=spec.dtype).element_size()
    src_in = [s if s is not None and s.numel() else None for s in srcs]
    if spec.partial:  # the sum, rounded to the destination dtype by the oracle itself
        boxes = oracle_boxes(spec.shape, spec.dst_mesh, spec.dst_placements)
        dsts = [torch.empty(box_shape(b), dtype=spec.out_dtype) for b in boxes]
        oracle.reshard_partial(list(spec.shape), FMT[spec.dtype], FMT[spec.out_dtype], list(spec.src_mesh),
                               list(spec.src_placements), src_in, list(spec.dst_mesh), list(spec.dst_placements),
                               [d if d.numel() else None for d in dsts], threads=threads)
        return dsts
    if spec.strided:
        dsts = [torch.empty([len(ix) for ix in lists], dtype=spec.dtype) for lists in oracle_index_lists(spec, "dst")]
        oracle.reshard_indexed(list(spec.shape), es, list(spec.src_mesh), list(spec.src_placements),
                               list(spec.split("src")), src_in, list(spec.dst_mesh), list(spec.dst_placements),
                               list(spec.split("dst")), [d if d.numel() else None for d in dsts], threads=threads)
    else:
        boxes = oracle_boxes(spec.shape, spec.dst_mesh, spec.dst_placements)
        dsts = [torch.empty(box_shape(b), dtype=spec.dtype) for b in boxes]
        oracle.reshard(list(spec.shape), es, list(spec.src_mesh), list(spec.src_placements), src_in,
                       list(spec.dst_mesh), list(spec.dst_placements),
                       [d if d.numel() else None for d in dsts], threads=threads)
    if spec.out_dtype != spec.dtype:
        dsts = [oracle.convert(d, FMT[spec.dtype], FMT[spec.out_dtype], threads=threads) for d in dsts]
    return dsts


def oracle_shapes(spec, side):
    """Local shard shapes of one side by the oracle (boxes, or index lists)."""
    if spec.strided:
        return [[len(ix) for ix in lists] for lists in oracle_index_lists(spec, side)]
    mesh = spec.src_mesh if side == "src" else spec.dst_mesh
    pl = spec.src_placements if side == "src" else spec.dst_placements
    return [box_shape(b) for b in oracle_boxes(spec.shape, mesh, pl)]


def oracle_cut(spec, g):
    """Source shards of the global tensor g, cut by the oracle's boxes (index
    lists, for a strided spec).  For a Partial spec g is the list of
    contributions and each rank gets its own contribution's box."""
    if spec.partial:
        boxes = oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements)
        return [W.cut(g[W.contribution_of(spec, r)], [b])[0] for r, b in enumerate(boxes)]
    if spec.strided:
        return W.cut_indexed(g, oracle_index_lists(spec, "src"))
    return W.cut(g, oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements))


def make_inputs(spec, values, seed, t=0, device="cpu"):
    """The seeded global tensor, or for a Partial spec its contributions."""
    if spec.partial:
        return W.make_contributions(spec, values, seed, t, device=device)
    return W.make_global(spec, values, seed, t, device=device)


def sources_for(spec, values, seed, t=0):
    """Seeded global tensor and its source shards cut with the oracle's boxes
    (index lists, for a strided spec)."""
    g = make_inputs(spec, values, seed, t)
    return g, oracle_cut(spec, g)


def apply_pieces(plan: Plan, srcs_per_tensor, fill=None):
    """Destination shards built by copying every planned piece on the host, at
    the local offsets the plan reports (for a plain layout those must equal the
    piece's offset from its shard's box)."""
    out = []
    for t, spec in enumerate(plan.specs):
        out.append([torch.full(shape, 0 if fill is None else fill, dtype=spec.out_dtype)
                    for shape in plan.dst_shapes(t)])
    sboxes = [None if s.strided else plan.src_boxes(t) for t, s in enumerate(plan.specs)]
    dboxes = [None if s.strided else plan.dst_boxes(t) for t, s in enumerate(plan.specs)]
    for i, pc in enumerate(R.reshard_plan_pieces(plan.handle)):
        t = pc["tensor"]
        nd = len(plan.specs[t].shape)
        lo, hi = pc["lo"][:nd], pc["hi"][:nd]
        ext = [h - l for l, h in zip(lo, hi)]
        s_loc, d_loc = pc["src_local"][:nd], pc["dst_local"][:nd]
        if sboxes[t] is not None:
            assert s_loc == [l - o for l, o in zip(lo, sboxes[t][pc["src_rank"]][0])], pc
        spec = plan.specs[t]
        sel = tuple(slice(a, a + e) for a, e in zip(s_loc, ext))
        if spec.partial:  # binary32 sum over the contributions, in order, then one rounding
            ranks = R.reshard_plan_piece_sources(plan.handle, i)
            assert len(ranks) == spec.partial and ranks[0] == pc["src_rank"]
            assert [W.contribution_of(spec, r) for r in ranks] == list(range(len(ranks)))
            acc = None
            for r in ranks:
                x = srcs_per_tensor[t][r][sel].contiguous()
                x = x.numpy() if spec.dtype == torch.float32 else oracle.convert(x, FMT[spec.dtype], "f32").numpy()
                acc = x.astype(np.float32) if acc is None else np.add(acc, x, dtype=np.float32)
            part = torch.from_numpy(np.ascontiguousarray(acc))
            if spec.out_dtype != torch.float32:
                part = oracle.convert(part, "f32", FMT[spec.out_dtype])
        else:
            part = srcs_per_tensor[t][pc["src_rank"]][sel]
            if spec.out_dtype != spec.dtype:
                part = oracle.convert(part.contiguous(), FMT[spec.dtype], FMT[spec.out_dtype])
        for d in R.reshard_plan_piece_fanout(plan.handle, i):
            if dboxes[t] is not None:
                assert d_loc == [l - o for l, o in zip(lo, dboxes[t][d][0])], pc
            out[t][d][tuple(slice(a, a + e) for a, e in zip(d_loc, ext))] = part
    return out


def _ranges(starts, lengths):
    """Concatenation of the integer ranges [starts[i], starts[i] + lengths[i])."""
    lengths = np.asarray(lengths, dtype=np.int64)
    total = int(lengths.sum())
    if total == 0:
        return np.zeros(0, dtype=np.int64)
    offs = np.repeat(np.cumsum(lengths) - lengths, lengths)
    return np.repeat(np.asarray(starts, dtype=np.int64), lengths) + (np.arange(total) - offs)


def run_descriptors(plan: Plan, srcs_flat, dsts_flat):
    """Execute the descriptor table on host byte arrays exactly as the kernel
    addresses memory (shard bases taken as 16-byte aligned) and resolves its
    shard pointers from the device table's fan-out list.  srcs_flat /
    dsts_flat: uint8 numpy arrays (or None), in the pointer-array order of
    reshard_execute.  For DST_CHUNKS descriptors it also checks that the chunks
    of every row tile the row exactly."""
    descs, _ = R.reshard_plan_descriptors(plan.handle)
    segs = R.reshard_plan_segments(plan.handle)
    # pointers resolve as in the kernel: one array of sources then destinations,
    # indexed by source slots and by the device table's fan-out list (absolute)
    refs = R.reshard_plan_device_refs(plan.handle)
    srcs_flat = dsts_flat = list(srcs_flat) + list(dsts_flat)
    for D in descs:
        if D["mode"] == R.DESC_WINDOW:
            _run_window(D, segs, refs, srcs_flat, dsts_flat)
            continue
        if D["mode"] == R.DESC_GATHER_ROWS:
            _run_gather_rows(D, segs, refs, srcs_flat, dsts_flat)
            continue
        if D["mode"] == R.DESC_CONVERT:
            _run_convert(D, refs, srcs_flat, dsts_flat)
            continue
        if D["mode"] == R.DESC_REDUCE:
            _run_reduce(D, refs, srcs_flat, dsts_flat)
            continue
        e0, e1, e2 = D["extent"]
        i0, i1, i2 = np.meshgrid(np.arange(e0), np.arange(e1), np.arange(e2), indexing="ij")
        so = (D["src_offset"] + i0 * D["src_stride"][0] + i1 * D["src_stride"][1]
              + i2 * D["src_stride"][2]).reshape(-1)
        do = (D["dst_offset"] + i0 * D["dst_stride"][0] + i1 * D["dst_stride"][1]
              + i2 * D["dst_stride"][2]).reshape(-1)
        L, n = D["run_bytes"], D["row_items"]
        c = np.arange(n, dtype=np.int64)
        if D["mode"] == R.DESC_ITEMS:
            assert n * D["unit"] == L
            lo = do[:, None] + c[None, :] * D["unit"]
            hi = lo + D["unit"]
        else:
            assert D["mode"] == R.DESC_DST_CHUNKS and n == (L + 30) // 16
            block = (do[:, None] & ~15) + 16 * c[None, :]
            lo = np.maximum(block, do[:, None])
            hi = np.maximum(np.minimum(block + 16, do[:, None] + L), lo)
            assert ((hi - lo).sum(axis=1) == L).all()          # every byte of every row, once
        lengths = (hi - lo).reshape(-1)
        dst_idx = _ranges(lo.reshape(-1), lengths)
        shift = np.repeat(np.repeat(so - do, n), lengths)       # same place in the row
        src_idx = dst_idx + shift
        data = srcs_flat[D["src_ptr"]][src_idx]
        for r in range(D["fanout"]):
            dsts_flat[refs[D["dst_ref_begin"] + r]][dst_idx] = data


CONVERSIONS = {R.CONVERT_F32_BF16: ("f32", "bf16", 4, 2), R.CONVERT_F32_F16: ("f32", "f16", 4, 2),
               R.CONVERT_BF16_F32: ("bf16", "f32", 2, 4), R.CONVERT_F16_F32: ("f16", "f32", 2, 4)}
_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _run_convert(D, refs, srcs_flat, dsts_flat):
    """A CONVERT descriptor element by element: items of 8 elements tile each
    row of `run` elements; elements are converted by the oracle."""
    fs, fd, es, ed = CONVERSIONS[D["unit"]]
    run, n = D["run_bytes"], D["row_items"]
    assert n == (run + 7) // 8
    e0, e1, e2 = D["extent"]
    i0, i1, i2 = np.meshgrid(np.arange(e0), np.arange(e1), np.arange(e2), indexing="ij")
    so = (D["src_offset"] + i0 * D["src_stride"][0] + i1 * D["src_stride"][1]
          + i2 * D["src_stride"][2]).reshape(-1)
    do = (D["dst_offset"] + i0 * D["dst_stride"][0] + i1 * D["dst_stride"][1]
          + i2 * D["dst_stride"][2]).reshape(-1)
    # element k of item c is element c*8 + k of the row (k < 8, inside the row)
    el = np.arange(n * 8, dtype=np.int64)
    el = el[el < run]
    s_byte = (so[:, None] + el[None, :] * es).reshape(-1)
    d_byte = (do[:, None] + el[None, :] * ed).reshape(-1)
    src = srcs_flat[D["src_ptr"]]
    vals = np.stack([src[s_byte + b] for b in range(es)], axis=1).reshape(-1)
    conv = oracle.convert(torch.from_numpy(vals.copy()).view(_TORCH[fs]), fs, fd)
    out = conv.view(torch.uint8).numpy().reshape(-1, ed)
    for r in range(D["fanout"]):
        dst = dsts_flat[refs[D["dst_ref_begin"] + r]]
        for b in range(ed):
            dst[d_byte + b] = out[:, b]


_FORMATS = ("f32", "bf16", "f16")


def _run_reduce(D, refs, srcs_flat, dsts_flat):
    """A REDUCE descriptor element by element: items of 8 elements tile each row
    of `run` elements; each element is the binary32 sum of the contributions
    refs[src_ptr ...] in list order (numpy float32 additions), rounded to the
    destination format by the oracle."""
    unit = D["unit"]
    parts, fs, fd = unit & 0xFFF, _FORMATS[(unit >> 12) & 3], _FORMATS[(unit >> 14) & 3]
    es, ed = (4 if fs == "f32" else 2), (4 if fd == "f32" else 2)
    run, n = D["run_bytes"], D["row_items"]
    assert n == (run + 7) // 8 and parts >= 1
    e0, e1, e2 = D["extent"]
    i0, i1, i2 = np.meshgrid(np.arange(e0), np.arange(e1), np.arange(e2), indexing="ij")
    so = (D["src_offset"] + i0 * D["src_stride"][0] + i1 * D["src_stride"][1]
          + i2 * D["src_stride"][2]).reshape(-1)
    do = (D["dst_offset"] + i0 * D["dst_stride"][0] + i1 * D["dst_stride"][1]
          + i2 * D["dst_stride"][2]).reshape(-1)
    el = np.arange(n * 8, dtype=np.int64)
    el = el[el < run]
    s_byte = (so[:, None] + el[None, :] * es).reshape(-1)
    d_byte = (do[:, None] + el[None, :] * ed).reshape(-1)
    acc = None
    for p in range(parts):
        src = srcs_flat[refs[D["src_ptr"] + p]]
        vals = np.stack([src[s_byte + b] for b in range(es)], axis=1).reshape(-1)
        x = torch.from_numpy(vals.copy()).view(_TORCH[fs])
        x = (x if fs == "f32" else oracle.convert(x, fs, "f32")).numpy()
        acc = x.copy() if acc is None else np.add(acc, x, dtype=np.float32)
    out = torch.from_numpy(acc)
    if fd != "f32":
        out = oracle.convert(out, "f32", fd)
    out = out.view(torch.uint8).numpy().reshape(-1, ed)
    for r in range(D["fanout"]):
        dst = dsts_flat[refs[D["dst_ref_begin"] + r]]
        for b in range(ed):
            dst[d_byte + b] = out[:, b]


NARROW_WINDOW_BYTES = 18432
NARROW_BIG_WINDOW_BYTES = 36864  # bands with small destination pieces or short tiles: twice the rows


def narrow_pitch(W):
    """Window row pitch (bytes) of a narrow band: an odd number of dwords when the
    band width W is a multiple of 4, else W."""
    return W if W % 4 else 4 * ((W // 4) | 1)


def narrow_class(wb, cb, P, W):
    """How the narrow-band kernel moves a segment of width wb at column cb."""
    if P % 4 == 0 and wb % 4 == 0 and cb % 4 == 0:
        return "dwords"
    if cb == 0 and wb == W and P == W:
        return "whole"
    if wb > 16:
        return "pieces"
    return "rows" if wb in (1, 2, 4, 8, 16) else "bytes"


def _exchange_band(D, srcs, dsts):
    """A 16-byte band with four packed 4-byte or eight packed 2-byte column runs
    on one side (the quad and octet exchanges of the row mode)."""
    def runs(S, k, rw):
        return len(S) == k and all(x["width"] == rw and x["row_stride"] == rw and x["col"] == rw * i
                                   and x["fanout"] == S[0]["fanout"] for i, x in enumerate(S))
    return D["run_bytes"] == 16 and any(runs(S, k, rw) for S in (srcs, dsts) for k, rw in ((4, 4), (8, 2)))


def is_narrow_band(D, segs):
    """The host check that sends a WINDOW band to the narrow-band kernel: packed
    segments, at most 64 a side, the window within its LDS; a band of at most 16
    bytes only with a segment of one or two bytes, a source segment of the bytes
    class or a destination one over 4 bytes, or of 12-byte rows of dword
    segments, and not one of the quad or octet exchanges."""
    W = D["run_bytes"]
    if D["mode"] != R.DESC_WINDOW or W == 0 or W > 16384:
        return False
    if D["extent"][1] * narrow_pitch(W) > NARROW_BIG_WINDOW_BYTES or D["dst_ref_begin"] > 64 or D["fanout"] > 64:
        return False
    srcs = segs[D["src_ptr"]:D["src_ptr"] + D["dst_ref_begin"]]
    dsts = segs[D["src_ptr"] + D["dst_ref_begin"]:D["src_ptr"] + D["dst_ref_begin"] + D["fanout"]]
    if not all(sg["width"] > 0 and sg["row_stride"] == sg["width"] and sg["col"] + sg["width"] <= W
               for sg in srcs + dsts):
        return False
    if W <= 16:
        P = narrow_pitch(W)
        thin = any(sg["width"] <= 2 for sg in srcs + dsts)
        bytewise = any(narrow_class(sg["width"], sg["col"], P, W) == "bytes" and (i < len(srcs) or sg["width"] > 4)
                       for i, sg in enumerate(srcs + dsts))
        dwords = all(narrow_class(sg["width"], sg["col"], P, W) == "dwords" for sg in srcs + dsts)
        if _exchange_band(D, srcs, dsts) or not (thin or bytewise or (dwords and P == W)):
            return False
    return True


def _div_small(n, w):
    """The kernel's n / w (n < 2^16, 1 <= w < 2^16) by a multiply with 2^32 / w
    rounded up; n may be an array."""
    assert 1 <= w < 1 << 16 and np.all(np.asarray(n) < 1 << 16)
    if w == 1:
        return n
    return (np.asarray(n, dtype=np.uint64) * np.uint64(0xFFFFFFFF // w + 1) >> np.uint64(32)).astype(np.int64)


def narrow_segment_moves(sg, P, W, hr, phase):
    """The narrow-band kernel's addressing of one segment for one tile of hr
    rows, replayed: arrays (stream byte, window byte, bytes) of the pieces its
    lanes move, in phase 1 (source stream into the window) or phase 2 (window
    into the destination stream).  Every piece stays inside the segment's
    columns of one window row."""
    wb, cb = sg["width"], sg["col"]
    cls = narrow_class(wb, cb, P, W)
    if cls == "dwords":
        w, c, pitch, n = wb // 4, cb // 4, P // 4, hr * wb // 4
        row_lane = phase == 2 and w <= 4 and sg["fanout"] == 1  # one row a lane (also the batched reads)
        if row_lane:
            r = np.arange(hr, dtype=np.int64)
            lo, win, ln = 4 * w * r, 4 * (r * pitch + c), np.full(hr, 4 * w)
        else:
            # quads stay together in the window; otherwise the kernel still moves
            # 16 bytes of the stream a lane but places its four dwords one by one
            # (the same dword moves as below, by stream offset)
            quads = (w & 3) == 0 or (c == 0 and w == pitch)
            nq = n // 4 if quads else 0
            j = np.concatenate([4 * np.arange(nq, dtype=np.int64), np.arange(4 * nq, n, dtype=np.int64)])
            r = _div_small(j, w)
            lo, win = 4 * j, 4 * (r * pitch + c + (j - r * w))
            ln = np.where(np.arange(len(j)) < nq, 16, 4)
            # a quad stays together in the window
            jq = j[:nq]
            rq = _div_small(jq + 3, w)
            assert np.all(rq * pitch + c + (jq + 3 - rq * w) == win[:nq] // 4 + 3)
    elif cls == "whole":
        lo = 16 * np.arange(-(-hr * wb // 16), dtype=np.int64)
        win, ln = lo.copy(), np.minimum(16, hr * wb - lo)
    elif cls == "rows":  # phase 2 moves 4- and 8-byte rows 16 stream bytes a lane, one window access a row
        r = np.arange(hr, dtype=np.int64)
        lo, win, ln = r * wb, r * P + cb, np.full(hr, wb)
    elif cls == "bytes" and phase == 2:  # one row a lane, as for rows
        r = np.arange(hr, dtype=np.int64)
        lo, win, ln = r * wb, r * P + cb, np.full(hr, wb)
    elif cls == "bytes":  # 16-byte pieces byte by byte: row and column of the first, then stepping
        j0 = 16 * np.arange(-(-hr * wb // 16), dtype=np.int64)
        r0 = _div_small(j0, wb)
        b = np.arange(16, dtype=np.int64)
        lo = (j0[:, None] + b[None, :]).reshape(-1)
        step = (j0 - r0 * wb)[:, None] + b[None, :]
        win = ((r0[:, None] + step // wb) * P + cb + step % wb).reshape(-1)
        keep = lo < hr * wb
        lo, win = lo[keep], win[keep]
        ln = np.ones(len(lo), dtype=np.int64)
    else:
        j = 16 * np.arange(-(-hr * wb // 16), dtype=np.int64)
        ln = np.minimum(16, hr * wb - j)
        r = _div_small(j, wb)
        col = j - r * wb
        l1 = np.minimum(ln, wb - col)
        two = ln > l1
        lo = np.concatenate([j, j[two] + l1[two]])
        win = np.concatenate([r * P + cb + col, (r[two] + 1) * P + cb])
        ln = np.concatenate([l1, ln[two] - l1[two]])
    lo, win, ln = (np.asarray(x, dtype=np.int64) for x in (lo, win, ln))
    assert np.all(ln >= 1) and np.all(lo >= 0) and np.all(lo + ln <= hr * wb)
    if cb == 0 and wb == W == P:  # whole rows with no padding: the stream is the window
        assert np.all(win == lo)
    else:
        row = win // P
        assert np.all(row < hr) and np.all(win % P >= cb) and np.all(win % P + ln <= cb + wb)
        assert np.all((win - row * P - cb) == lo - row * wb)  # the same row and column on both sides
    return lo, win, ln


_M32 = 0xFFFFFFFF


def _rotate_bytes(v, s):
    """The kernel's rotate_bytes on four 32-bit words: byte i of the result is
    byte (i - s) mod 16 of v, built the way the kernel builds it."""
    if s & 1:
        v = [((v[0] << 8) | (v[3] >> 24)) & _M32, ((v[1] << 8) | (v[0] >> 24)) & _M32,
             ((v[2] << 8) | (v[1] >> 24)) & _M32, ((v[3] << 8) | (v[2] >> 24)) & _M32]
    if s & 2:
        v = [((v[0] << 16) | (v[3] >> 16)) & _M32, ((v[1] << 16) | (v[0] >> 16)) & _M32,
             ((v[2] << 16) | (v[1] >> 16)) & _M32, ((v[3] << 16) | (v[2] >> 16)) & _M32]
    if s & 4:
        v = [v[3], v[0], v[1], v[2]]
    if s & 8:
        v = [v[2], v[3], v[0], v[1]]
    return v


def thin_runs(side, fan_matters):
    """The kernel's runs of thin segments (1 or 2 bytes wide) of one side: lists
    of consecutive segment indices with one width, consecutive columns and (on
    the destination side) one fan-out; every other segment stands alone."""
    out, s = [], 0
    while s < len(side):
        e = s + 1
        if side[s]["width"] <= 2:
            while (e < len(side) and side[e]["width"] == side[s]["width"]
                   and side[e]["col"] == side[s]["col"] + (e - s) * side[s]["width"]
                   and (not fan_matters or side[e]["fanout"] == side[s]["fanout"])):
                e += 1
        out.append(list(range(s, e)))
        s = e
    return out


def _thin_run_bytes(run, side, P, hr, r0, window, flat, refs, is_src):
    """A run of thin segments through the kernel's thin path, byte for byte: a
    lane (item i, lane i mod 64) moves 8 rows of one segment in a rotated
    order, rows past the last whole piece one a lane."""
    wb = side[run[0]]["width"]
    nq, tail = hr // 8, hr % 8
    for i in range(len(run) * nq):
        seg, q = divmod(i, nq)
        sg = side[run[seg]]
        lane = i % 64
        rot = ((lane >> 2) ^ (lane >> 5)) & 7
        g = sg["offset"] + r0 * wb + 8 * wb * q                 # stream piece in the shard
        p = q * 8 * P + side[run[0]]["col"] + seg * wb          # window byte of row 8q
        assert p - q * 8 * P == sg["col"]
        at = [p + ((j + rot) & 7) * P for j in range(8)]         # slot j -> row (j + rot) mod 8
        if is_src:
            data = flat[sg["ptr"]][g:g + 8 * wb]
            if wb == 2:
                w = [int(x) for x in data.view(np.uint32)]
                w = _rotate_bytes(w, (16 - 2 * rot) & 15)
                slots = np.array(w, dtype=np.uint32).view(np.uint8)
            else:
                x = int(data.view(np.uint64)[0])
                y = ((x >> (8 * rot)) | (x << (64 - 8 * rot))) & (2 ** 64 - 1) if rot else x
                slots = np.array([y], dtype=np.uint64).view(np.uint8)
            for j in range(8):
                window[at[j]:at[j] + wb] = slots[j * wb:(j + 1) * wb]
        else:
            slots = np.concatenate([window[a:a + wb] for a in at])
            if wb == 2:
                w = [int(x) for x in slots.view(np.uint32)]
                v = np.array(_rotate_bytes(w, 2 * rot), dtype=np.uint32).view(np.uint8)
            else:
                x = int(slots.view(np.uint64)[0])
                y = ((x << (8 * rot)) | (x >> (64 - 8 * rot))) & (2 ** 64 - 1) if rot else x
                v = np.array([y], dtype=np.uint64).view(np.uint8)
            for k in range(sg["fanout"]):
                flat[refs[sg["ptr"] + k]][g:g + 8 * wb] = v
    for i in range(len(run) * tail):
        seg, t = divmod(i, tail)
        sg = side[run[seg]]
        r = 8 * nq + t
        g, a = sg["offset"] + (r0 + r) * wb, r * P + sg["col"]
        if is_src:
            window[a:a + wb] = flat[sg["ptr"]][g:g + wb]
        else:
            for k in range(sg["fanout"]):
                flat[refs[sg["ptr"] + k]][g:g + wb] = window[a:a + wb]


def _run_narrow(D, segs, refs, srcs_flat, dsts_flat):
    """A narrow band tile by tile, as the narrow-band kernel addresses it; checks
    that phase 1 writes every window byte of the tile's rows once and phase 2
    writes every destination stream byte once."""
    rows, per_tile, W = D["extent"][0], D["extent"][1], D["run_bytes"]
    P = narrow_pitch(W)
    assert per_tile * P <= NARROW_BIG_WINDOW_BYTES
    srcs = segs[D["src_ptr"]:D["src_ptr"] + D["dst_ref_begin"]]
    dsts = segs[D["src_ptr"] + D["dst_ref_begin"]:D["src_ptr"] + D["dst_ref_begin"] + D["fanout"]]
    for tile in range(-(-rows // per_tile)):
        r0 = tile * per_tile
        hr = min(per_tile, rows - r0)
        window = np.zeros(per_tile * P, dtype=np.uint8)
        written = np.zeros(per_tile * P, dtype=np.int32)
        # a single source segment is read through the scalar path, never as a run
        for run in thin_runs(srcs, False) if len(srcs) > 1 else [[0]]:
            for s_i in run:
                lo, win, ln = narrow_segment_moves(srcs[s_i], P, W, hr, 1)
                written[_ranges(win, ln)] += 1
            if srcs[run[0]]["width"] <= 2:
                _thin_run_bytes(run, srcs, P, hr, r0, window, srcs_flat, refs, True)
                continue
            sg = srcs[run[0]]
            lo, win, ln = narrow_segment_moves(sg, P, W, hr, 1)
            si, wi = _ranges(lo, ln), _ranges(win, ln)
            assert len(np.unique(si)) == len(si) == hr * sg["width"]
            window[wi] = srcs_flat[sg["ptr"]][sg["offset"] + r0 * sg["width"] + si]
        used = (np.arange(hr)[:, None] * P + np.arange(W)[None, :]).reshape(-1)
        assert np.all(written[used] == 1) and written.sum() == hr * W
        for run in thin_runs(dsts, True):
            if dsts[run[0]]["width"] <= 2:
                _thin_run_bytes(run, dsts, P, hr, r0, window, dsts_flat, refs, False)
                continue
            sg = dsts[run[0]]
            lo, win, ln = narrow_segment_moves(sg, P, W, hr, 2)
            di, wi = _ranges(lo, ln), _ranges(win, ln)
            assert len(np.unique(di)) == len(di) == hr * sg["width"]
            for k in range(sg["fanout"]):
                dsts_flat[refs[sg["ptr"] + k]][sg["offset"] + r0 * sg["width"] + di] = window[wi]


def _run_window(D, segs, refs, srcs_flat, dsts_flat):
    """A window band row by row: sources into a window row, window row out to
    every destination replica.  Also checks that the sources and the
    destinations each tile the window row exactly.  Narrow bands go through
    the narrow-band kernel's addressing (_run_narrow) after the same check."""
    rows, width = D["extent"][0], D["run_bytes"]
    window = np.zeros((rows, width), dtype=np.uint8)
    srcs = segs[D["src_ptr"]:D["src_ptr"] + D["dst_ref_begin"]]
    dsts = segs[D["src_ptr"] + D["dst_ref_begin"]:D["src_ptr"] + D["dst_ref_begin"] + D["fanout"]]
    for side in (srcs, dsts):
        cover = np.zeros(width, dtype=np.int32)
        for sg in side:
            cover[sg["col"]:sg["col"] + sg["width"]] += 1
        assert (cover == 1).all()
    if is_narrow_band(D, segs):
        _run_narrow(D, segs, refs, srcs_flat, dsts_flat)
        return
    r = np.arange(rows, dtype=np.int64)[:, None]
    for sg in srcs:
        assert sg["fanout"] == 0
        idx = sg["offset"] + r * sg["row_stride"] + np.arange(sg["width"])[None, :]
        window[:, sg["col"]:sg["col"] + sg["width"]] = srcs_flat[sg["ptr"]][idx]
    for sg in dsts:
        idx = sg["offset"] + r * sg["row_stride"] + np.arange(sg["width"])[None, :]
        for k in range(sg["fanout"]):
            dsts_flat[refs[sg["ptr"] + k]][idx] = window[:, sg["col"]:sg["col"] + sg["width"]]


def gather_lane_blocks(D, segs):
    """The gather-rows kernel's addressing, replayed per 16-byte destination
    block: (destination offset, bytes, [(segment, source byte offset, bytes)]).
    Waves of 64 blocks place their span the way the kernel does (the segment
    holding the wave's first byte and the next one, wrapping to the next row's
    first segment), and every block reads inside its segments' rows."""
    W, rows, nseg = D["run_bytes"], D["extent"][0], D["extent"][1]
    S = segs[D["src_ptr"]:D["src_ptr"] + nseg]
    band = rows * W
    out = []
    for a_w in range(0, band, 1024):
        row_w, col_w = divmod(a_w, W)
        assert magic_div(a_w, *D["magic"][0]) == row_w
        i0 = max(i for i in range(nseg) if S[i]["col"] <= col_w)
        if D["row_items"] == 1:  # the kernel's lookup, read the way it reads it, gives the same segment
            raw = np.array([D["src_offset"], D["dst_offset"], *D["src_stride"], *D["dst_stride"]],
                           dtype=np.int64).view(np.uint32)         # descriptor words 0 .. 15
            w = col_w >> 11
            word = int(raw[w if w < 2 else w + 2])
            e = word >> 16 if col_w & 1024 else word & 0xFFFF
            assert (e & 63) + (1 if (e >> 6) and (col_w & 1023) >= (e >> 6) else 0) == i0, (D, a_w)
        wrap = i0 + 1 == nseg
        s0, s1 = S[i0], S[0 if wrap else i0 + 1]
        B1 = s0["col"] + s0["width"]
        E1 = W + s1["width"] if wrap else s1["col"] + s1["width"]
        for lane in range(64):
            pos, a = col_w + 16 * lane, a_w + 16 * lane
            n = max(0, min(16, band - a))
            if n == 0:
                continue
            seg, row, start, end = (s1, row_w + 1 if wrap else row_w, W if wrap else s1["col"], E1) \
                if pos >= B1 else (s0, row_w, s0["col"], B1)
            at = min(pos, end - 16)
            assert start <= at and at + 16 <= end, (D, a)      # the 16-byte load stays in the row
            L1 = min(pos + n, end) - pos
            parts = [(seg, seg["offset"] + row * seg["row_stride"] + (pos - start), L1)]
            if L1 < n:
                assert pos < B1 and n - L1 <= 16
                r1 = row_w + 1 if wrap else row_w
                parts.append((s1, s1["offset"] + r1 * s1["row_stride"], n - L1))
            out.append((D["dst_offset"] + a, n, parts))
    return out


def _run_gather_rows(D, segs, refs, srcs_flat, dsts_flat):
    """A gather-rows band block by block, as the kernel addresses it; also
    checks that the segments tile the row."""
    W, nseg = D["run_bytes"], D["extent"][1]
    S = segs[D["src_ptr"]:D["src_ptr"] + nseg]
    cover = np.zeros(W, dtype=np.int32)
    for sg in S:
        assert sg["fanout"] == 0 and sg["width"] >= 1024
        cover[sg["col"]:sg["col"] + sg["width"]] += 1
    assert (cover == 1).all()
    blocks = gather_lane_blocks(D, segs)
    assert sum(n for _, n, _ in blocks) == D["extent"][0] * W
    for d_off, n, parts in blocks:
        data = np.concatenate([srcs_flat[sg["ptr"]][o:o + k] for sg, o, k in parts])
        assert len(data) == n
        for r in range(D["fanout"]):
            dsts_flat[refs[D["dst_ref_begin"] + r]][d_off:d_off + n] = data


def shard_bytes(plan: Plan):
    """Bytes of every shard, in the src / dst pointer-array order of execute."""
    sb, db = [], []
    for t, spec in enumerate(plan.specs):
        sb += [int(np.prod(shape)) * spec.dtype.itemsize for shape in plan.src_shapes(t)]
        db += [int(np.prod(shape)) * spec.out_dtype.itemsize for shape in plan.dst_shapes(t)]
    return sb, db


def assert_descriptors_in_bounds(plan: Plan):
    """Every byte a descriptor touches lies inside its shards (checked before
    any launch)."""
    sb, db = shard_bytes(plan)
    descs, refs = R.reshard_plan_descriptors(plan.handle)
    segs = R.reshard_plan_segments(plan.handle)
    # the device table's fan-out list: absolute slots, destinations after the
    # sources, a REDUCE descriptor's contributions among the sources
    drefs = R.reshard_plan_device_refs(plan.handle)
    n_src = len(sb)
    reduce_slots = {D["src_ptr"] + q for D in descs if D["mode"] == R.DESC_REDUCE for q in range(D["unit"] & 0xFFF)}
    for i, (a, b) in enumerate(zip(drefs, refs)):
        if i in reduce_slots:
            assert a == b < n_src, (i, a, b)
        else:
            assert a == n_src + b < n_src + len(db), (i, a, b)
    for D in descs:
        ext = D["extent"]
        if D["mode"] == R.DESC_GATHER_ROWS:
            rows, nseg, W = ext[0], ext[1], D["run_bytes"]
            assert rows >= 1 and nseg >= 1 and rows * W < 2 ** 31 and D["dst_offset"] >= 0
            # the segment lookup the kernel reads: the segment holding each KiB's
            # first byte and where inside the KiB the next one starts
            lut = np.array([D["src_offset"], *D["src_stride"], *D["dst_stride"]], dtype=np.int64).view(np.uint16)
            S = segs[D["src_ptr"]:D["src_ptr"] + nseg]
            if D["row_items"] == 1:
                assert W <= 28 * 1024 and nseg <= 64
                for k in range(-(-W // 1024)):
                    c = 1024 * k
                    i = max(j for j in range(nseg) if S[j]["col"] <= c)
                    nxt = [S[j]["col"] for j in range(nseg) if c < S[j]["col"] < c + 1024]
                    assert len(nxt) <= 1
                    assert lut[k] == i | ((nxt[0] - c if nxt else 0) << 6), (D, k)
            else:
                assert D["row_items"] == 0 and (W > 28 * 1024 or nseg > 64)
            for sg in segs[D["src_ptr"]:D["src_ptr"] + nseg]:
                assert sg["offset"] >= 0 and sg["row_stride"] >= sg["width"] >= 1024
                assert sg["offset"] + (rows - 1) * sg["row_stride"] + sg["width"] <= sb[sg["ptr"]], sg
            for r in range(D["fanout"]):
                assert D["dst_offset"] + rows * W <= db[refs[D["dst_ref_begin"] + r]], D
            continue
        if D["mode"] == R.DESC_WINDOW:
            rows, per_tile, pitch, width = ext[0], ext[1], D["row_items"], D["run_bytes"]
            assert rows >= 1 and per_tile >= 1 and pitch % 16 == 0 and pitch >= width
            # the all-modes LDS window, or the row mode, or a narrow band's window (twice
            # the rows for small destination pieces)
            assert (per_tile * pitch <= 16384 or (width <= 16 and per_tile % 256 == 0)
                    or (is_narrow_band(D, segs) and per_tile * narrow_pitch(width) <= NARROW_BIG_WINDOW_BYTES))
            first = D["src_ptr"]
            for i, sg in enumerate(segs[first:first + D["dst_ref_begin"] + D["fanout"]]):
                assert sg["col"] + sg["width"] <= width and sg["offset"] >= 0 and sg["row_stride"] >= 0
                last = sg["offset"] + (rows - 1) * sg["row_stride"] + sg["width"]
                if i < D["dst_ref_begin"]:
                    assert last <= sb[sg["ptr"]], sg
                else:
                    for k in range(sg["fanout"]):
                        assert last <= db[refs[sg["ptr"] + k]], sg
            continue
        assert D["run_bytes"] >= 1 and D["row_items"] >= 1 and all(e >= 1 for e in ext)
        assert ext[0] * ext[1] * ext[2] * D["row_items"] < 2 ** 31
        s_span = d_span = D["run_bytes"]
        if D["mode"] == R.DESC_CONVERT:
            _, _, es, ed = CONVERSIONS[D["unit"]]
            s_span, d_span = D["run_bytes"] * es, D["run_bytes"] * ed
        src_slots = [D["src_ptr"]]
        if D["mode"] == R.DESC_REDUCE:  # every contribution's slot, all at the same offsets
            unit = D["unit"]
            es, ed = (4 if (unit >> 12) & 3 == 0 else 2), (4 if (unit >> 14) & 3 == 0 else 2)
            s_span, d_span = D["run_bytes"] * es, D["run_bytes"] * ed
            src_slots = [refs[D["src_ptr"] + p] for p in range(unit & 0xFFF)]
            assert len(src_slots) >= 1
        s_last = D["src_offset"] + sum((e - 1) * st for e, st in zip(ext, D["src_stride"])) + s_span
        d_last = D["dst_offset"] + sum((e - 1) * st for e, st in zip(ext, D["dst_stride"])) + d_span
        assert D["src_offset"] >= 0 and D["dst_offset"] >= 0
        assert all(st >= 0 for st in D["src_stride"] + D["dst_stride"])
        for slot in src_slots:
            assert s_last <= sb[slot], D
        for r in range(D["fanout"]):
            assert d_last <= db[refs[D["dst_ref_begin"] + r]], D


def magic_div(n, m, s):
    """The kernel's quotient formula for n < 2^31."""
    return ((n * m >> 32) + n) >> s
