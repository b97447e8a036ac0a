"""Benchmark of the reshard execute on one MI355X.

A step is one reshard_execute of the workload's plan: the fused launch(es) that
read every source byte once and write every destination shard.  The plan
(boxes, replica groups, intersections, replica choice, descriptors) is built
once per layout pair and reused for every refit; its host time is reported
separately as ``plan_us``.

The headline workload is the 32-layer FFN refit (96 tensors in one launch).
The other configurations of the same benchmark family are measured in the same
run and reported in ``per_config``: the pages' 8x8 worked example (parity only),
one FFN up-projection, an MoE expert stack and the uneven fp32 nested split.
Each row carries its own cold timing, roofline fraction, counter traffic and CPU
baseline.

Inputs are resident in HBM before timing starts.  To keep every step cold in
the 256 MB Infinity Cache, steps rotate over several independent sets of
source and destination buffers whose total size is at least 2 GB.

After the timed region (and outside it) the same inputs are also moved by the
pages' baseline scheme, gather-then-slice, built from two plans of the same
library (sources -> one global buffer -> destinations); its step time and the
reshard's speed-up over it are reported as ``gather_then_slice_gpu``.

``contiguous_same_bytes`` is the same kernel moving the same bytes as one
contiguous buffer with the same fan-out: the practical ceiling for the
workload's read:write mix on this GPU.  ``copy_reference`` (per config:
``torch_copy_half_bytes_gbps``) is the runtime's own device copy (torch
``copy_``) of half the algorithmic bytes, rotated over buffer pairs the same
way: the 1:1 read:write ceiling at that size, and the size calibration of the
rocprofv3 byte counters.

The two-stage transport of the pages (each destination box delivered once,
split over its replicas, then assembled by every replica; pipelined over
tensor chunks on two streams) is timed the same way as ``two_stage_gpu``, and
the pages' hybrid refit (FFN projections by the reshard, other weights by
gather-then-slice) as ``hybrid_gpu`` where the workload has both kinds.

``cpu_baseline`` times the oracle (the pages' gather-then-slice scheme, run on
the host) on the same input bytes the GPU consumed and checks that its output
equals the GPU's, byte for byte.

Prints one JSON line.  ``value`` = algorithmic bytes (global bytes read once +
every destination shard written once) per second over the timed steps;
``roofline.achieved`` = the same bytes over the kernel's mean launch duration:
HIP events on the launch stream around the K back-to-back launches of the timed
region, divided by K (one launch per step for the headline plan).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, decimal GB/s
METRIC = "reshard execute GB/s (bytes read+written) and % of MI355X HBM peak; plan time us"
DEFAULT_WORKLOAD = "ffn_refit_32_layers"
# the benchmark family, in order: the worked example (parity only), one FFN
# up-projection, an MoE expert stack, the uneven fp32 nested split, the 32-layer refit
CONFIGS = ["worked_example_8x8", "ffn_up_14336x4096", "moe_experts_64x2048x7168", "uneven_5000x3001",
           "ffn_refit_32_layers"]
KERNEL_SOURCES = [os.path.join(ROOT, "dtensor_layout_movement_amd", "csrc", f)
                  for f in ("kernel.hip", "kernel.h", "plan.h", "plan.cpp", "reshard.hip")]
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_NAME = "reshard_copy_kernel"


def kernel_source_sha() -> str:
    """Hash of the sources that fix what the copy kernel reads and writes."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def dtype_name(dt) -> str:
    return {"bfloat16": "bf16", "float32": "f32", "float16": "f16", "float64": "f64",
            "uint8": "u8"}.get(str(dt).replace("torch.", ""), str(dt).replace("torch.", ""))


def layout_str(mesh, placements, split=None) -> str:
    """(mesh)[placements]; a strided shard with split factor f prints as S<dim>/f."""
    split = split or (1,) * len(mesh)
    pl = ",".join("R" if p < 0 else f"S{p}" + (f"/{f}" if f > 1 else "") for p, f in zip(placements, split))
    return f"({','.join(str(m) for m in mesh)})[{pl}]"


def traffic_from_profile(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    if there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"{KERNEL_NAME}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_sha():
        return None
    try:
        return int(vals["fetch_bytes_per_launch"]) + int(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def build_plan(R, wl):
    srcs, dsts = [], []
    for t in wl.tensors:
        srcs.append(R.layout_create(t.shape, R.dtype_code(t.dtype), t.src_mesh, t.src_placements, t.src_split))
        dsts.append(R.layout_create(t.shape, R.dtype_code(t.out_dtype), t.dst_mesh, t.dst_placements, t.dst_split))
    plan = R.reshard_plan_create_batched(srcs, dsts)
    return plan, srcs, dsts


def plan_timing(R, wl, reps: int) -> dict:
    host, wall = [], []
    for _ in range(reps):
        t0 = time.perf_counter()
        plan, srcs, dsts = build_plan(R, wl)
        wall.append((time.perf_counter() - t0) * 1e6)
        host.append(R.reshard_plan_stats(plan)["plan_host_us"])
        R.reshard_plan_destroy(plan)
        for h in srcs + dsts:
            R.reshard_layout_destroy(h)
    up = []
    for _ in range(max(3, reps // 10)):
        plan, srcs, dsts = build_plan(R, wl)
        t0 = time.perf_counter()
        R.reshard_plan_upload(plan, None)
        up.append((time.perf_counter() - t0) * 1e6)
        R.reshard_plan_destroy(plan)
        for h in srcs + dsts:
            R.reshard_layout_destroy(h)
    return {"host_median": round(statistics.median(host), 2),
            "with_layouts_and_binding_median": round(statistics.median(wall), 2),
            "upload_median": round(statistics.median(up), 2), "reps": reps}


def source_shards(R, W, spec, layout, values: str, seed: int, t: int, dev) -> list:
    """Seeded source shards of one tensor, one per rank (None when empty): boxes
    of the global tensor, runs of it for a strided layout, or for a Partial
    source each rank's box of its own contribution."""
    nd = len(spec.shape)
    ranks = range(R.reshard_layout_num_ranks(layout))

    def box(r):
        off, ext = R.reshard_layout_shard_box(layout, r, nd)
        return off, [o + e for o, e in zip(off, ext)]
    if spec.partial:
        contribs = W.make_contributions(spec, values, seed, t, device=dev)
        return [W.cut(contribs[W.contribution_of(spec, r)], [box(r)])[0] for r in ranks]
    g = W.make_global(spec, values, seed, t, device=dev)
    if spec.strided:
        lists = [[[i for a, b in R.reshard_layout_shard_runs(layout, r, k) for i in range(a, b)] for k in range(nd)]
                 for r in ranks]
        return W.cut_indexed(g, lists)
    return W.cut(g, [box(r) for r in ranks])


def alloc_set(torch, R, wl, lay_src, lay_dst, dev, seed):
    """One set of source shards (seeded values) and destination shards."""
    from dtensor_layout_movement_amd import workloads as W
    src_bufs, dst_bufs = [], []
    for t, spec in enumerate(wl.tensors):
        src_bufs += source_shards(R, W, spec, lay_src[t], wl.values, seed, t, dev)
        for r in range(R.reshard_layout_num_ranks(lay_dst[t])):
            shape = R.local_shape(lay_dst[t], r, len(spec.shape))
            dst_bufs.append(torch.empty(shape, dtype=spec.out_dtype, device=dev) if all(shape) else None)
    sp = R.pointer_array([b.data_ptr() if b is not None else 0 for b in src_bufs])
    dp = R.pointer_array([b.data_ptr() if b is not None else 0 for b in dst_bufs])
    return src_bufs, dst_bufs, sp, dp


def contiguous_reference(torch, R, st, dev, stream, steps: int, min_footprint_gb: float):
    """The same kernel moving the same bytes with no layout structure: one
    contiguous byte buffer of `bytes_read` bytes replicated to `fan` destinations,
    (1,)[R] -> (fan,)[R], fan = bytes_written / bytes_read when that is whole.
    Timed cold like the main step: its rate is what this kernel reaches on this
    read:write mix, the practical ceiling for the workload."""
    n, w = st["bytes_read"], st["bytes_written"]
    if n == 0 or w % n:
        return None
    fan = w // n
    lay_s = R.reshard_layout_create((n,), R.DTYPE_U8, (1,), (R.REPLICATE,))
    lay_d = R.reshard_layout_create((n,), R.DTYPE_U8, (fan,), (R.REPLICATE,))
    plan = R.reshard_plan_create(lay_s, lay_d)
    try:
        R.reshard_plan_upload(plan, stream.cuda_stream)
        n_sets = max(1, min(16, int(-(-min_footprint_gb * 1e9 // (n * (1 + fan))))))
        bufs = [[torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(1 + fan)] for _ in range(n_sets)]
        arrays = [(R.pointer_array([b[0].data_ptr()]), R.pointer_array([x.data_ptr() for x in b[1:]]))
                  for b in bufs]
        for i in range(3):
            R.reshard_execute(plan, *arrays[i % n_sets], stream.cuda_stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            R.reshard_execute(plan, *arrays[i % n_sets], stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        gbps = (n + w) / (ms * 1e-3) / 1e9
        return {"gbps": round(gbps, 1), "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
                "fanout": fan, "steps": steps, "buffer_sets_rotated": n_sets}
    finally:
        R.reshard_plan_destroy(plan)
        R.reshard_layout_destroy(lay_s)
        R.reshard_layout_destroy(lay_d)


def gather_then_slice(torch, R, wl, lay_src, lay_dst, sets, stream, steps: int, reshard_ms: float) -> dict:
    """The pages' baseline scheme on the same GPU, built from two plans of the same
    library: every source shard into one global buffer (gather), then every
    destination shard out of it (slice).  It moves twice the reshard's bytes."""
    g_lay, plans_g, plans_s = [], None, None
    for t, spec in enumerate(wl.tensors):
        g_lay.append(R.reshard_layout_create(spec.shape, R.dtype_code(spec.dtype), (1,), (R.REPLICATE,)))
    plans_g = R.reshard_plan_create_batched(lay_src, g_lay)
    plans_s = R.reshard_plan_create_batched(g_lay, lay_dst)
    R.reshard_plan_upload(plans_g, stream.cuda_stream)
    R.reshard_plan_upload(plans_s, stream.cuda_stream)
    n_sets = len(sets)
    globals_ = [[torch.empty(spec.shape, dtype=spec.dtype, device="cuda") for spec in wl.tensors]
                for _ in range(n_sets)]
    gp = [R.pointer_array([g.data_ptr() for g in gl]) for gl in globals_]
    for i in range(3):
        _, _, sp, dp = sets[i % n_sets]
        R.reshard_execute(plans_g, sp, gp[i % n_sets], stream.cuda_stream)
        R.reshard_execute(plans_s, gp[i % n_sets], dp, stream.cuda_stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        _, _, sp, dp = sets[i % n_sets]
        R.reshard_execute(plans_g, sp, gp[i % n_sets], stream.cuda_stream)
        R.reshard_execute(plans_s, gp[i % n_sets], dp, stream.cuda_stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    st_g, st_s = R.reshard_plan_stats(plans_g), R.reshard_plan_stats(plans_s)
    traffic = st_g["bytes_read"] + st_g["bytes_written"] + st_s["bytes_read"] + st_s["bytes_written"]
    R.reshard_plan_destroy(plans_g)
    R.reshard_plan_destroy(plans_s)
    for h in g_lay:
        R.reshard_layout_destroy(h)
    del globals_
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 5), "bytes_moved": traffic, "steps": steps,
            "reshard_speedup": round(ms / reshard_ms, 3)}


def two_stage(torch, wl, sets_boxes, steps: int, reshard_ms: float, chunks: int = 4) -> dict:
    """The pages' two-stage transport emulated on the same GPU: each destination
    box delivered once, split over its replicas, then assembled by every
    replica; pipelined over tensor chunks on two streams."""
    from dtensor_layout_movement_amd.two_stage import TwoStagePlan
    ts = TwoStagePlan(wl.tensors, chunks=chunks)
    try:
        staging = [[torch.empty(sh, dtype=spec.out_dtype, device="cuda") if all(sh) else None
                    for sh in shapes] for spec, shapes in zip(wl.tensors, ts.staging_shapes())]
        stag_ptrs = [[x.data_ptr() if x is not None else 0 for x in row] for row in staging]
        arrays = [ts.pointer_arrays(sp, stag_ptrs, dp) for sp, dp in sets_boxes]
        a, b = torch.cuda.Stream(), torch.cuda.Stream()
        events = [torch.cuda.Event() for _ in range(chunks)]
        torch.cuda.synchronize()
        for i in range(3):
            ts.execute(arrays[i % len(arrays)], a, b, events)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(a)
        for i in range(steps):
            b.wait_stream(a)
            a.wait_stream(b)
            ts.execute(arrays[i % len(arrays)], a, b, events)
        a.wait_stream(b)
        e1.record(a)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        return {"ms_per_step": round(ms, 5), "bytes_moved": ts.bytes_moved(), "steps": steps,
                "chunks": len(ts.stage1), "reshard_speedup": round(ms / reshard_ms, 3)}
    finally:
        ts.close()


def hybrid(torch, wl, sets_boxes, stream, steps: int, reshard_ms: float):
    """The pages' hybrid refit on the same GPU: FFN projections by the reshard,
    the other weights by gather-then-slice, one stream.  None when the routing
    does not split the workload."""
    from dtensor_layout_movement_amd.hybrid import HybridPlan
    hp = HybridPlan(wl.tensors)
    try:
        if not hp.direct or not hp.gather:
            return None
        n_sets = len(sets_boxes)
        glob = [[torch.empty(sh, dtype=wl.tensors[t].dtype, device="cuda")
                 for t, sh in zip(hp.gather, hp.global_shapes())] for _ in range(n_sets)]
        arrays = [hp.pointer_arrays(sp, dp, [g.data_ptr() for g in glob[i]])
                  for i, (sp, dp) in enumerate(sets_boxes)]
        for i in range(3):
            hp.execute(arrays[i % n_sets], stream.cuda_stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            hp.execute(arrays[i % n_sets], stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        return {"ms_per_step": round(ms, 5), "bytes_moved": hp.bytes_moved(), "steps": steps,
                "reshard_tensors": len(hp.direct), "gather_tensors": len(hp.gather),
                "reshard_share_of_bytes": round(hp.reshard_share(), 4),
                "reshard_speedup": round(ms / reshard_ms, 3)}
    finally:
        hp.close()


def cpu_info() -> dict:
    """Host threads this process may use and the CPU model string."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cores": len(os.sched_getaffinity(0)), "cpu_model": model}


def tensor_slices(R, lay_src, lay_dst):
    """Per tensor, its ranges in the flat source and destination buffer lists."""
    out, i_s, i_d = [], 0, 0
    for ls, ld in zip(lay_src, lay_dst):
        ns, nd = R.reshard_layout_num_ranks(ls), R.reshard_layout_num_ranks(ld)
        out.append(((i_s, i_s + ns), (i_d, i_d + nd)))
        i_s += ns
        i_d += nd
    return out


def cpu_baseline(torch, R, wl, lay_src, lay_dst, gpu_set, reps: int, single_core_tensors: int | None,
                 algo_bytes: int) -> dict:
    """The oracle (the pages' gather-then-slice scheme on the host) timed on this
    host's cores over the input bytes of one GPU buffer set, tensor by tensor; its
    output is compared byte for byte with what the GPU wrote into that set.
    All-cores time: median of `reps` passes over every tensor.  One-core time:
    median of `reps` passes over the first `single_core_tensors` tensors (all
    when None).  Rates are GB/s over the reshard's algorithmic bytes of the
    tensors timed."""
    import oracle
    info = cpu_info()
    src_bufs, dst_bufs, _, _ = gpu_set
    spans = tensor_slices(R, lay_src, lay_dst)
    one_n = len(wl.tensors) if single_core_tensors is None else min(single_core_tensors, len(wl.tensors))
    all_s, one_s = [], []
    matches = True
    algo_one = 0
    for rep in range(reps):
        t_all = t_one = 0.0
        for t, spec in enumerate(wl.tensors):
            (s0, s1), (d0, d1) = spans[t]
            srcs = [b.cpu().contiguous() if b is not None else None for b in src_bufs[s0:s1]]
            es = torch.empty((), dtype=spec.dtype).element_size()
            dsts = [torch.empty(b.shape, dtype=spec.dtype) if b is not None else None for b in dst_bufs[d0:d1]]
            src_in = [x if x is not None and x.numel() else None for x in srcs]
            dst_in = [x if x is not None and x.numel() else None for x in dsts]
            if spec.partial:  # the oracle's Partial sum, rounded to the destination dtype
                fmt = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}
                fn = oracle.reshard_partial
                dsts = [torch.empty(b.shape, dtype=spec.out_dtype) if b is not None else None
                        for b in dst_bufs[d0:d1]]
                dst_in = [x if x is not None and x.numel() else None for x in dsts]
                args = (list(spec.shape), fmt[spec.dtype], fmt[spec.out_dtype], list(spec.src_mesh),
                        list(spec.src_placements), src_in, list(spec.dst_mesh), list(spec.dst_placements), dst_in)
            elif spec.strided:  # the oracle's index-list form
                fn = oracle.reshard_indexed
                args = (list(spec.shape), es, list(spec.src_mesh), list(spec.src_placements), list(spec.split("src")),
                        src_in, list(spec.dst_mesh), list(spec.dst_placements), list(spec.split("dst")), dst_in)
            else:
                fn = oracle.reshard
                args = (list(spec.shape), es, list(spec.src_mesh), list(spec.src_placements), src_in,
                        list(spec.dst_mesh), list(spec.dst_placements), dst_in)
            t0 = time.perf_counter()
            fn(*args, threads=info["cores"])
            t_all += time.perf_counter() - t0
            if t < one_n:
                t0 = time.perf_counter()
                fn(*args, threads=1)
                t_one += time.perf_counter() - t0
                if rep == 0:
                    algo_one += sum(x.numel() for x in srcs if x is not None) // max(1, _src_replicas(spec)) * es
                    algo_one += sum(x.numel() for x in dsts if x is not None) * es
            if rep == 0:  # the GPU's bytes of this set
                for g, c in zip(dst_bufs[d0:d1], dsts):
                    if g is not None and not torch.equal(g.cpu().view(torch.uint8), c.view(torch.uint8)):
                        matches = False
            del srcs, dsts
        all_s.append(t_all)
        one_s.append(t_one)
    t_all, t_one = statistics.median(all_s), statistics.median(one_s)
    names = wl.name if one_n == len(wl.tensors) else f"the first {one_n} of {len(wl.tensors)} tensors of {wl.name}"
    return {"value": round(algo_bytes / t_all / 1e9, 3), "unit": "GB/s", "cores": info["cores"], "kind": "oracle",
            "cpu_model": info["cpu_model"], "seconds_all_cores": round(t_all, 6),
            "single_core_value": round(algo_one / t_one / 1e9, 3), "seconds_single_core": round(t_one, 6),
            "matches_gpu": matches,
            "sample": f"gather-then-slice of every tensor of {wl.name} (replica and coverage checks on), median of "
                      f"{reps} pass(es) on {info['cores']} threads; single core: {names}, median of {reps}; "
                      f"GB/s over the reshard's algorithmic bytes"}


def _src_replicas(spec) -> int:
    """Replicas of each source box (product of the Replicate mesh sizes)."""
    n = 1
    for m, p in zip(spec.src_mesh, spec.src_placements):
        if p < 0:
            n *= m
    return n


def steps_for(algo_bytes: int) -> int:
    """Timed steps of a per-config row: about 1e11 bytes, between 50 and 1000."""
    return max(50, min(1000, int(1e11 // max(1, algo_bytes))))


def measure(torch, R, wl, dev, stream, steps: int, warmup: int, min_footprint_gb: float):
    """Plan, allocate rotating buffer sets and time `steps` cold executes.
    Returns (row dict, plan, layouts, sets)."""
    plan, lay_src, lay_dst = build_plan(R, wl)
    R.reshard_plan_upload(plan, stream.cuda_stream)
    st = R.reshard_plan_stats(plan)
    algo = st["bytes_read"] + st["bytes_written"]
    n_sets = max(1, min(16, int(-(-min_footprint_gb * 1e9 // algo))))
    sets = [alloc_set(torch, R, wl, lay_src, lay_dst, dev, seed=s) for s in range(n_sets)]
    torch.cuda.synchronize()
    for i in range(warmup):
        _, _, sp, dp = sets[i % n_sets]
        R.reshard_execute(plan, sp, dp, stream.cuda_stream)
    torch.cuda.synchronize()
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_begin.record(stream)
    for i in range(steps):
        _, _, sp, dp = sets[i % n_sets]
        R.reshard_execute(plan, sp, dp, stream.cuda_stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_begin.elapsed_time(t_end) / steps
    gbps = algo / (ms * 1e-3) / 1e9
    st = R.reshard_plan_stats(plan)
    row = {
        "workload": wl.name, "tensors": len(wl.tensors), "bytes_read": st["bytes_read"],
        "bytes_written": st["bytes_written"], "algorithmic_bytes": algo, "pieces": st["n_pieces"],
        "descriptors": st["n_descriptors"], "grid_workgroups": st["n_workgroups"],
        "launches_per_step": st["n_launches"], "steps": steps, "buffer_sets_rotated": n_sets,
        "ms_per_step": round(ms, 5), "gbps": round(gbps, 2), "frac": round(gbps / HBM_PEAK_GBPS, 4),
        # one launch per step: the mean launch duration on the launch stream;
        # several: the step time of all of them, gaps included
        ("kernel_mean_us" if st["n_launches"] == 1 else "step_us_all_launches"): round(ms * 1e3, 3),
        "traffic": traffic_from_profile(wl.name), "wall_s": round(wall, 4), "plan_host_us": st["plan_host_us"],
    }
    return row, plan, lay_src, lay_dst, sets


def release(R, plan, lay_src, lay_dst):
    R.reshard_plan_destroy(plan)
    for h in lay_src + lay_dst:
        R.reshard_layout_destroy(h)


def worked_example_row(torch, R, dev, stream, reps: int) -> dict:
    """The pages' 8x8 example: parity only.  Destination c must hold
    v[i][2c + k] = 8 i + 2 c + k (the example's closed form for v[i][j] = 8 i + j),
    and the oracle must produce the same bytes."""
    from dtensor_layout_movement_amd import workloads as W
    wl = W.worked_example_8x8()
    row, plan, lay_src, lay_dst, sets = measure(torch, R, wl, dev, stream, 5, 1, 0.0)
    _, dst_bufs, _, _ = sets[0]
    closed = all(torch.equal(d.cpu().float(), torch.tensor([[8 * i + 2 * c + k for k in range(2)]
                                                             for i in range(8)], dtype=torch.float32))
                 for c, d in enumerate(dst_bufs))
    cpu = cpu_baseline(torch, R, wl, lay_src, lay_dst, sets[0], reps, None, row["algorithmic_bytes"])
    release(R, plan, lay_src, lay_dst)
    return {"workload": wl.name, "parity": "bit-exact" if closed and cpu["matches_gpu"] else "MISMATCH",
            "closed_form": closed, "launches_per_step": row["launches_per_step"], "cpu_baseline": cpu}


def torch_copy_reference(torch, dev, stream, algo_bytes: int, min_footprint_gb: float) -> dict:
    """A plain device copy (torch copy_, the runtime's own blit kernel) of half
    the algorithmic bytes, rotated over buffer pairs of at least
    min_footprint_gb like the reshard: context for the read:write mix 1:1, and
    the size calibration of rocprofv3's FETCH_SIZE / WRITE_SIZE counters."""
    half = min(algo_bytes // 2, 1 << 30)
    n_pairs = max(2, min(16, int(-(-min_footprint_gb * 1e9 // (2 * half)))))
    pairs = [(torch.empty(half, dtype=torch.uint8, device=dev), torch.empty(half, dtype=torch.uint8, device=dev))
             for _ in range(n_pairs)]
    for i in range(3):
        pairs[i % n_pairs][1].copy_(pairs[i % n_pairs][0])
    n_copy = max(20, n_pairs)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for i in range(n_copy):
        pairs[i % n_pairs][1].copy_(pairs[i % n_pairs][0])
    c1.record(stream)
    torch.cuda.synchronize()
    ms = c0.elapsed_time(c1) / n_copy
    del pairs
    torch.cuda.empty_cache()
    return {"bytes_each_way": half, "gbps": round(2 * half / (ms * 1e-3) / 1e9, 1), "buffer_pairs_rotated": n_pairs}


def config_row(torch, R, name, dev, stream, min_footprint_gb: float, cpu: bool) -> dict:
    """One configuration of the benchmark family, measured cold like the headline."""
    from dtensor_layout_movement_amd import workloads as W
    wl = W.WORKLOADS[name]()
    plan, lay_src, lay_dst = build_plan(R, wl)
    st = R.reshard_plan_stats(plan)
    release(R, plan, lay_src, lay_dst)
    steps = steps_for(st["bytes_read"] + st["bytes_written"])
    row, plan, lay_src, lay_dst, sets = measure(torch, R, wl, dev, stream, steps, 10, min_footprint_gb)
    ref = contiguous_reference(torch, R, st, dev, stream, max(20, steps // 4), min_footprint_gb)
    if ref:
        row["contiguous_same_bytes_gbps"] = ref["gbps"]
    row["torch_copy_half_bytes_gbps"] = torch_copy_reference(torch, dev, stream, row["algorithmic_bytes"],
                                                             min_footprint_gb)["gbps"]
    if cpu:
        _, _, sp, dp = sets[0]
        R.reshard_execute(plan, sp, dp, stream.cuda_stream)
        torch.cuda.synchronize()
        row["cpu_baseline"] = cpu_baseline(torch, R, wl, lay_src, lay_dst, sets[0], 3, None,
                                           row["algorithmic_bytes"])
        row["parity"] = "bit-exact" if row["cpu_baseline"]["matches_gpu"] else "MISMATCH"
    release(R, plan, lay_src, lay_dst)
    del sets
    torch.cuda.empty_cache()
    return row


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--min-footprint-gb", type=float, default=2.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-comparator", action="store_true",
                    help="skip the gather-then-slice, two-stage, hybrid and contiguous comparators")
    ap.add_argument("--no-per-config", action="store_true",
                    help="measure only --workload (profiling runs)")
    ap.add_argument("--plan-reps", type=int, default=200)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the reshard's source and destination ranks are "
              "simulated as separate buffers in one MI355X's HBM; there is no multi-GPU path "
              "in this build.", file=sys.stderr)
        return 2

    import torch
    import dtensor_layout_movement_amd as R
    from dtensor_layout_movement_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    wl = W.WORKLOADS[args.workload]()
    print(f"[bench] {wl.name}: {len(wl.tensors)} tensors", file=sys.stderr, flush=True)

    head, plan, lay_src, lay_dst, sets = measure(torch, R, wl, dev, stream, args.steps, args.warmup,
                                                 args.min_footprint_gb)
    st = R.reshard_plan_stats(plan)
    algo_bytes = head["algorithmic_bytes"]
    n_sets = head["buffer_sets_rotated"]
    ms_per_step = head["ms_per_step"]
    K = args.steps
    value = head["gbps"]
    achieved = value  # one launch per step (the headline plan): mean launch = step time

    # outside the timed region: per-launch event distribution, and warm steps on
    # one buffer set (inputs partly cache-resident)
    n_dist = min(50, K)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dist)]
    for i in range(n_dist):
        _, _, sp, dp = sets[i % n_sets]
        ev[i][0].record(stream)
        R.reshard_execute(plan, sp, dp, stream.cuda_stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_launch = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    _, _, sp0, dp0 = sets[0]
    for _ in range(3):
        R.reshard_execute(plan, sp0, dp0, stream.cuda_stream)
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(n_dist):
        R.reshard_execute(plan, sp0, dp0, stream.cuda_stream)
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / n_dist

    copy_ref = torch_copy_reference(torch, dev, stream, algo_bytes, args.min_footprint_gb)

    reference = comparator = two = mixed = None
    if not args.no_comparator:
        print("[bench] comparators", file=sys.stderr, flush=True)
        reference = contiguous_reference(torch, R, st, dev, stream, max(5, K // 4), args.min_footprint_gb)
        if reference:
            reference["workload_vs_reference"] = round(value / reference["gbps"], 4)
        comparator = gather_then_slice(torch, R, wl, lay_src, lay_dst, sets, stream, max(5, K // 4), ms_per_step)
        per_tensor = []
        for src_bufs, dst_bufs, _, _ in sets:
            sp, dp = [], []
            for (s0, s1), (d0, d1) in tensor_slices(R, lay_src, lay_dst):
                sp.append([b.data_ptr() if b is not None else 0 for b in src_bufs[s0:s1]])
                dp.append([b.data_ptr() if b is not None else 0 for b in dst_bufs[d0:d1]])
            per_tensor.append((sp, dp))
        two = two_stage(torch, wl, per_tensor, max(5, K // 4), ms_per_step)
        mixed = hybrid(torch, wl, per_tensor, stream, max(5, K // 4), ms_per_step)
        torch.cuda.empty_cache()
    plan_us = plan_timing(R, wl, args.plan_reps if algo_bytes < 2e10 else max(5, args.plan_reps // 20))
    spec0 = wl.tensors[0]
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name(spec0.dtype) + ("" if spec0.out_dtype == spec0.dtype else "->" + dtype_name(spec0.out_dtype)),
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "tensors": len(wl.tensors),
            "global_shape": list(spec0.shape) if len(wl.tensors) == 1 else None,
            "src_layout": layout_str(spec0.src_mesh, spec0.src_placements, spec0.src_split),
            "dst_layout": layout_str(spec0.dst_mesh, spec0.dst_placements, spec0.dst_split),
            "bytes_read": st["bytes_read"],
            "bytes_written": st["bytes_written"],
            "pieces": st["n_pieces"],
            "descriptors": st["n_descriptors"],
            "grid_workgroups": st["n_workgroups"],
            "launches_per_step": st["n_launches"],
            "buffer_sets_rotated": n_sets,
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        },
        "plan_us": plan_us,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": head["traffic"],
            "kernel": KERNEL_NAME,
            ("kernel_mean_us" if st["n_launches"] == 1 else "step_us_all_launches"): round(ms_per_step * 1e3, 3),
        },
        "launch_us_cold": {"p10": round(per_launch[len(per_launch) // 10], 2),
                           "p50": round(per_launch[len(per_launch) // 2], 2),
                           "p90": round(per_launch[(9 * len(per_launch)) // 10], 2), "n": n_dist},
        "warm_same_buffers_gbps": round(algo_bytes / (warm_ms * 1e-3) / 1e9, 1),
        "copy_reference": copy_ref,
        "contiguous_same_bytes": reference,
        "gather_then_slice_gpu": comparator,
        "two_stage_gpu": two,
        "hybrid_gpu": mixed,
        "wall_s": head["wall_s"],
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        R.reshard_execute(plan, sp0, dp0, stream.cuda_stream)
        torch.cuda.synchronize()
        many = len(wl.tensors) > 3
        out["cpu_baseline"] = cpu_baseline(torch, R, wl, lay_src, lay_dst, sets[0], 1 if many else 3,
                                           12 if many else None, algo_bytes)
    release(R, plan, lay_src, lay_dst)
    del sets
    torch.cuda.empty_cache()

    if not args.no_per_config:
        rows = {}
        for i, name in enumerate(CONFIGS):
            if name == wl.name:
                rows[name] = {"config_index": i, "headline": True}
                continue
            print(f"[bench] per-config {name}", file=sys.stderr, flush=True)
            try:
                if name == "worked_example_8x8":
                    row = worked_example_row(torch, R, dev, stream, 3)
                else:
                    row = config_row(torch, R, name, dev, stream, args.min_footprint_gb, not args.no_cpu_baseline)
            except Exception as e:  # a failing row is reported, not fatal to the headline
                row = {"error": f"{type(e).__name__}: {e}"}
            row["config_index"] = i
            rows[name] = row
        out["per_config"] = rows
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
