"""Two-stage reshard: send each contribution once, then replicate inside the
destination domain -- the transport the Reshard write-ups describe for NCCL M2N
Reshard (techfeed.io write-up, "NVIDIA's NVLink implementation" section:
received data is spread as evenly as possible over the replicas of a domain,
which then exchange it; news.bpdata.com write-up, "the Reshard collective"
section: network and NVLink stages are pipelined).  On one GPU both stages run
in HBM, so this is an emulation of the structure, measured beside the direct
reshard; every byte is moved by the library's kernel.

Stage 1 ("network"): every destination box is delivered exactly once, cut along
tensor dim 0 into one slice per replica, each slice landing in a staging buffer
of the replica that owns it.  Its layout is the destination layout with the
Replicate mesh dims moved last and turned into Shard(0): nested ceil splits of
dim 0 inside each box, so the replicas' slices tile the box.

Stage 2 ("in-domain exchange"): every replica assembles its full box from all
slices of its box (a reshard from the stage-1 layout to the destination layout).

Tensors are cut into chunks; stage 2 of chunk c runs on a second stream while
stage 1 of chunk c + 1 runs on the first.
"""
from __future__ import annotations

from . import reshard as R


def stage1_layout(mesh, placements, split=None):
    """(mesh, placements, split factors) of the stage-1 layout: the
    destination's non-Replicate mesh dims in order (with their split factors),
    then its Replicate dims turned into Shard(0) (factor 1)."""
    split = tuple(split) if split is not None else (1,) * len(mesh)
    non = [i for i, p in enumerate(placements) if p != R.REPLICATE]
    rep = [i for i, p in enumerate(placements) if p == R.REPLICATE]
    mesh1 = [mesh[i] for i in non] + [mesh[i] for i in rep]
    pl1 = [placements[i] for i in non] + [0] * len(rep)
    sp1 = [split[i] for i in non] + [1] * len(rep)
    return tuple(mesh1), tuple(pl1), tuple(sp1)


class TwoStagePlan:
    """Stage-1 and stage-2 plans for a list of tensors, `chunks` tensor chunks.

    specs: objects with shape, dtype, src_mesh, src_placements, dst_mesh,
    dst_placements and optionally src_split / dst_split (e.g.
    workloads.TensorSpec).
    """

    def __init__(self, specs, chunks: int = 1):
        self.specs = list(specs)
        n = len(self.specs)
        chunks = max(1, min(chunks, n))
        self.bounds = [n * c // chunks for c in range(chunks + 1)]
        self._layouts = []
        self.src_l, self.mid_l, self.dst_l = [], [], []
        for spec in self.specs:
            code = R.dtype_code(spec.dtype)
            out = R.dtype_code(getattr(spec, "out_dtype", spec.dtype))  # a conversion happens in stage 1
            m1, p1, f1 = stage1_layout(spec.dst_mesh, spec.dst_placements, getattr(spec, "dst_split", None))
            s = R.layout_create(spec.shape, code, spec.src_mesh, spec.src_placements, getattr(spec, "src_split", None))
            m = R.layout_create(spec.shape, out, m1, p1, f1)
            d = R.layout_create(spec.shape, out, spec.dst_mesh, spec.dst_placements, getattr(spec, "dst_split", None))
            self._layouts += [s, m, d]
            self.src_l.append(s)
            self.mid_l.append(m)
            self.dst_l.append(d)
        self.stage1, self.stage2 = [], []
        for c in range(chunks):
            a, b = self.bounds[c], self.bounds[c + 1]
            self.stage1.append(R.reshard_plan_create_batched(self.src_l[a:b], self.mid_l[a:b]))
            self.stage2.append(R.reshard_plan_create_batched(self.mid_l[a:b], self.dst_l[a:b]))

    def staging_shapes(self):
        """Per tensor, the local shapes of the stage-1 (staging) shards."""
        out = []
        for t, spec in enumerate(self.specs):
            n = R.reshard_layout_num_ranks(self.mid_l[t])
            out.append([R.local_shape(self.mid_l[t], r, len(spec.shape)) for r in range(n)])
        return out

    def bytes_moved(self) -> int:
        total = 0
        for p in self.stage1 + self.stage2:
            st = R.reshard_plan_stats(p)
            total += st["bytes_read"] + st["bytes_written"]
        return total

    def pointer_arrays(self, src_ptrs, staging_ptrs, dst_ptrs):
        """Per chunk (stage-1 src, stage-1 dst = staging, stage-2 dst) pointer
        arrays; inputs are per-tensor lists of device addresses."""
        out = []
        for c in range(len(self.stage1)):
            a, b = self.bounds[c], self.bounds[c + 1]
            s = [p for t in range(a, b) for p in src_ptrs[t]]
            m = [p for t in range(a, b) for p in staging_ptrs[t]]
            d = [p for t in range(a, b) for p in dst_ptrs[t]]
            out.append((R.pointer_array(s), R.pointer_array(m), R.pointer_array(d)))
        return out

    def execute(self, arrays, stream_a, stream_b, events):
        """Stage 1 of every chunk on stream_a; stage 2 of chunk c on stream_b once
        stage 1 of chunk c is done (events: one torch.cuda.Event per chunk).
        Streams are torch.cuda.Stream objects; returns after enqueueing."""
        for c, (s, m, d) in enumerate(arrays):
            R.reshard_execute(self.stage1[c], s, m, stream_a.cuda_stream)
            events[c].record(stream_a)
            stream_b.wait_event(events[c])
            R.reshard_execute(self.stage2[c], m, d, stream_b.cuda_stream)

    def close(self):
        for p in self.stage1 + self.stage2:
            R.reshard_plan_destroy(p)
        for h in self._layouts:
            R.reshard_layout_destroy(h)
        self.stage1, self.stage2, self._layouts = [], [], []
