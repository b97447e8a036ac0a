"""Hybrid refit routing: the feed-forward projections go through the reshard,
every other weight through gather-then-slice.

This is the split the NeMo RL integration makes (NVIDIA blog summaries, the
"NeMo RL" benchmark sections of the techfeed.io and news.bpdata.com write-ups):
the FFN projection weights carry about 95% of a dense model's refit payload, so
they take the reshard path; the smaller weights (attention projections, norms)
keep the gather path.  On one GPU the gather path is the same library used twice:
sources -> one full copy of the tensor (a 1-rank replicated layout), then full
copy -> destination shards.  Every byte is moved by the library's kernel.
"""
from __future__ import annotations

from . import reshard as R

FFN_NAMES = ("gate", "up", "down", "gate_proj", "up_proj", "down_proj", "w1", "w2", "w3")


def ffn_route(spec) -> bool:
    """True when the tensor is a feed-forward projection (taken by the reshard)."""
    return spec.name.rsplit(".", 1)[-1] in FFN_NAMES


class HybridPlan:
    """Plans for a list of tensors split by `use_reshard(spec)`.

    specs: objects with name, shape, dtype, src_mesh, src_placements, dst_mesh,
    dst_placements and optionally src_split / dst_split (e.g.
    workloads.TensorSpec).  Tensors routed to the gather path
    need one full-size buffer each (`global_shapes()`), owned by the caller.
    """

    def __init__(self, specs, use_reshard=ffn_route):
        self.specs = list(specs)
        self.direct = [t for t, s in enumerate(self.specs) if use_reshard(s)]
        self.gather = [t for t, s in enumerate(self.specs) if not use_reshard(s)]
        self._layouts = []
        src, dst, glob = {}, {}, {}
        for t, spec in enumerate(self.specs):
            code = R.dtype_code(spec.dtype)
            out = R.dtype_code(getattr(spec, "out_dtype", spec.dtype))
            src[t] = R.layout_create(spec.shape, code, spec.src_mesh, spec.src_placements,
                                     getattr(spec, "src_split", None))
            dst[t] = R.layout_create(spec.shape, out, spec.dst_mesh, spec.dst_placements,
                                     getattr(spec, "dst_split", None))
            self._layouts += [src[t], dst[t]]
            if t in self.gather:
                glob[t] = R.reshard_layout_create(spec.shape, code, (1,), (R.REPLICATE,))
                self._layouts.append(glob[t])
        self.plan_direct = self.plan_gather = self.plan_slice = None
        if self.direct:
            self.plan_direct = R.reshard_plan_create_batched([src[t] for t in self.direct],
                                                             [dst[t] for t in self.direct])
        if self.gather:
            self.plan_gather = R.reshard_plan_create_batched([src[t] for t in self.gather],
                                                             [glob[t] for t in self.gather])
            self.plan_slice = R.reshard_plan_create_batched([glob[t] for t in self.gather],
                                                            [dst[t] for t in self.gather])

    def plans(self):
        return [p for p in (self.plan_direct, self.plan_gather, self.plan_slice) if p is not None]

    def global_shapes(self):
        """Shapes of the full-size buffers, one per gather-routed tensor, in order."""
        return [tuple(self.specs[t].shape) for t in self.gather]

    def bytes_moved(self) -> int:
        total = 0
        for p in self.plans():
            st = R.reshard_plan_stats(p)
            total += st["bytes_read"] + st["bytes_written"]
        return total

    def reshard_share(self) -> float:
        """Fraction of the tensors' bytes that the reshard path carries."""
        size = lambda t: R.reshard_dtype_size(R.dtype_code(self.specs[t].dtype)) * _numel(self.specs[t].shape)
        whole = sum(size(t) for t in range(len(self.specs)))
        return sum(size(t) for t in self.direct) / whole if whole else 0.0

    def pointer_arrays(self, src_ptrs, dst_ptrs, global_ptrs):
        """(direct, gather, slice) pairs of pointer arrays, None for an unused
        path.  src_ptrs / dst_ptrs: per-tensor lists of device addresses;
        global_ptrs: one address per gather-routed tensor, in `gather` order."""
        direct = gather = slice_ = None
        if self.plan_direct is not None:
            direct = (R.pointer_array([p for t in self.direct for p in src_ptrs[t]]),
                      R.pointer_array([p for t in self.direct for p in dst_ptrs[t]]))
        if self.plan_gather is not None:
            g = R.pointer_array(list(global_ptrs))
            gather = (R.pointer_array([p for t in self.gather for p in src_ptrs[t]]), g)
            slice_ = (g, R.pointer_array([p for t in self.gather for p in dst_ptrs[t]]))
        return direct, gather, slice_

    def execute(self, arrays, stream: int):
        """Gather, then slice, then the reshard of the FFN tensors, all on one
        stream (a raw hipStream_t address; 0 = the null stream)."""
        direct, gather, slice_ = arrays
        if gather is not None:
            R.reshard_execute(self.plan_gather, gather[0], gather[1], stream)
            R.reshard_execute(self.plan_slice, slice_[0], slice_[1], stream)
        if direct is not None:
            R.reshard_execute(self.plan_direct, direct[0], direct[1], stream)

    def close(self):
        for p in self.plans():
            R.reshard_plan_destroy(p)
        for h in self._layouts:
            R.reshard_layout_destroy(h)
        self.plan_direct = self.plan_gather = self.plan_slice = None
        self._layouts = []


def _numel(shape) -> int:
    n = 1
    for s in shape:
        n *= s
    return n
