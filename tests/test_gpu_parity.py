"""GPU parity: the fused gfx950 copy kernel, called through the C ABI, against
the CPU oracle, bit for bit, on guarded shard buffers.  Full-size workloads run
in the same launch configuration as the benchmark (the plan's own grid)."""
import numpy as np
import pytest
import torch

import dtensor_layout_movement_amd as R
import oracle_pins as P
from dtensor_layout_movement_amd import workloads as W
from gpu_harness import GuardedShards, run_parity, shard_nbytes
from reshard_harness import Plan, assert_boxes_agree, assert_descriptors_in_bounds, box_shape, oracle_boxes
from test_planner import narrow_random_specs, random_specs, small_specs, strided_random_specs

pytestmark = pytest.mark.gpu

T = W.TensorSpec
RR = W.R


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def test_worked_example_golden():
    """The pages' 8x8 example on the GPU against the golden fixture."""
    wl = W.worked_example_8x8()
    spec = wl.tensors[0]
    gold = P.read_golden()
    with Plan([spec]) as plan:
        assert_boxes_agree(plan)
        g = W.make_global(spec, "arange", 0)
        srcs = W.cut(g, oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements))
        src_d = [s.cuda() for s in srcs]
        dst_d = [torch.full((8, 2), -1.0, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
        R.reshard_execute(plan.handle, [t.data_ptr() for t in src_d], [t.data_ptr() for t in dst_d],
                          torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for c, d in enumerate(dst_d):
            got = d.cpu().float().numpy().astype(np.int64)
            assert np.array_equal(got, gold[("dst", c)])


SMALL_FULL = ["worked_example_8x8", "ffn_up_14336x4096", "moe_experts_64x2048x7168", "uneven_5000x3001",
              "narrow_columns_4194304x8", "narrow_columns_tp8_2097152x16", "narrow_columns_64b_tp8_1048576x32",
              "narrow_columns_64b_tp4_1048576x32", "narrow_columns_32b_tp4_2097152x16",
              "narrow_columns_16b_tp8_4194304x8",
              "ffn_up_f32_to_bf16_14336x4096", "ffn_up_fsdp2_tp_14336x4096", "ffn_up_partial_14336x4096",
              "narrow_columns_8b_tp2_8388608x4", "narrow_columns_64b_tp16_1048576x32",
              "narrow_columns_ragged_tp4_2396745x14", "narrow_columns_2b_tp16_2097152x16"]


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", SMALL_FULL)
def test_workload_parity_full_size(name, seed):
    wl = W.WORKLOADS[name]()
    run_parity(wl.tensors, wl.values, seed)


@pytest.mark.parametrize("name", SMALL_FULL)
def test_workload_parity_raw_bits(name):
    """Random bytes (NaN payloads, infinities, -0.0, subnormals) arrive unchanged."""
    wl = W.WORKLOADS[name]()
    run_parity(wl.tensors, "raw", 7)


@pytest.mark.parametrize("values,seed", [("normal", 0), ("normal", 1), ("normal", 2), ("raw", 0)])
def test_ffn_refit_32_layers_one_launch(values, seed):
    """All 96 tensors of the 32-layer refit in one fused launch (pointer table
    too large for kernel arguments: uploaded into a device slot)."""
    wl = W.ffn_refit()
    st = run_parity(wl.tensors, values, seed, threads=16)
    assert st["n_tensors"] == 96 and st["n_pieces"] == 384
    assert st["n_launches"] == 1


def test_dense_layer_refit_32_layers_one_launch():
    """Every weight of 32 dense layers (attention, FFN, replicated norm vectors
    read from one of two source replicas and written to 8 destinations) in one
    fused launch."""
    wl = W.dense_layer_refit()
    st = run_parity(wl.tensors, "raw", 0, threads=16)
    assert st["n_tensors"] == 32 * 9
    assert st["n_launches"] == 1


def test_replan_after_rank_loss():
    """Plans destroyed and rebuilt on shrinking meshes (the image of a refit whose
    communication groups are recreated after ranks leave), each executed on the
    GPU and compared with the oracle; every rebuilt plan runs twice, so a stale
    pointer slot or table from the destroyed plan would show."""
    from test_planner import rank_loss_sequence
    for i, spec in enumerate(rank_loss_sequence(4480, 3200)):
        run_parity([spec], "raw", 20 + i, executes=2)


@pytest.mark.parametrize("spec", small_specs(), ids=lambda s: s.name)
def test_small_layouts(spec):
    run_parity([spec], "normal" if spec.partial else "raw", 3)


def _narrow_shapes_at_scale():
    """Narrow layouts of a million rows and more that take the narrow-band paths
    the small cases cover only in a few tiles: 24- and 40-byte rows into 8-byte
    shards (16-byte stream pieces split over window rows), 10-byte rows into
    4/4/2-byte shards (4-byte rows 16 stream bytes a lane), 12-byte rows gathered
    from 3-byte shards (a band of at most 16 bytes on the narrow path), and
    32-byte rows read from replicated row shards in row parts."""
    return [T("f32_in24", ((1 << 20) + 3, 6), torch.float32, (2,), (0,), (3,), (1,)),
            T("bf16_in40", ((1 << 19) + 7, 20), torch.bfloat16, (2,), (0,), (5,), (1,)),
            T("bf16_in10", ((1 << 20) + 5, 5), torch.bfloat16, (2,), (0,), (3,), (1,)),
            T("u8_r3_gather", ((1 << 20) + 1, 12), torch.uint8, (4,), (1,), (2,), (0,)),
            T("rep_rows_in32", ((1 << 20) + 9, 16), torch.bfloat16, (2, 3), (RR, 0), (16,), (1,))]


@pytest.mark.parametrize("spec", _narrow_shapes_at_scale(), ids=lambda s: s.name)
def test_narrow_shapes_at_scale(spec):
    """Bit-exact against the oracle, every destination byte."""
    run_parity([spec], "raw", 7)


@pytest.mark.parametrize("name", ["partial_tp2", "partial_rep", "partial_two_dims", "partial_f32_f16"])
def test_partial_sums_of_raw_bits(name):
    """Partial sums over random bytes: infinities, NaN payloads, subnormals and
    signed zeros in every contribution.  Every element that is not NaN matches
    the oracle bit for bit; NaN positions match."""
    spec = {s.name: s for s in small_specs()}[name]
    run_parity([spec], "raw", 5)


@pytest.mark.parametrize("misalign", [1, 2, 4, 8, "mixed"])
def test_misaligned_shard_pointers(misalign):
    """Shard pointers off the 16-byte grid (all by the same offset, or 'mixed':
    each shard at its own phase, replicas included) take the bytewise or
    unaligned paths; results and guard bands must be unaffected."""
    specs = [W.uneven(50, 31).tensors[0], W.ffn_up(112, 64).tensors[0]] + \
        [s for s in small_specs() if s.name in ("conv_f32_bf16", "conv_bf16_f32_ragged", "strips_fanout",
                                                "strips_rep_src", "chunked_bf16", "strips_nine",
                                                "narrow_rep", "narrow_scatter", "narrow_gather_rep", "narrow_bf16_cols",
                                                "runs_scatter_rep", "runs_gather", "runs64_scatter_rep",
                                                "runs64_gather", "bands16_rep", "bands16_gather", "runs32_scatter_rep",
                                                "runs32_gather", "octets_gather", "octets_scatter_rep", "bands16_96",
                                                "bands16_80_rep", "pairs_gather", "pairs_rep", "narrow_8byte_rows",
                                                "gather_uneven", "gather_fanout", "gather_rep_src",
                                                "gather_row_cuts", "bytes_r2_in32", "bytes_r2_rep",
                                                "bytes_ragged13", "bytes_ragged13_gather", "bytes_u8_odd_rows",
                                                "bytes_pieces18", "bytes_pieces18_gather", "bytes_w512",
                                                "thin_u8_16", "thin_u8_gather", "thin_f16_rep", "thin_bf16_6",
                                                "rows12_f32", "rows12_gather", "rows12_rep", "bytes_r6_gather",
                                                "bytes_u8_r7_rep", "dwords24_scatter", "dwords40_rep",
                                                "dwords24_gather", "rows4_w10", "rows4_w10_gather",
                                                "bytes_u8_r3_gather", "bytes_r6_in12", "rep_src_u8",
                                                "rep_src_bf16_rows", "thin32_gather_rep")]
    for spec in specs:
        run_parity([spec], "raw", 4, misalign=misalign)


@pytest.mark.parametrize("name", ["narrow_scatter_rep", "runs_scatter", "runs64_scatter", "runs32_scatter",
                                  "bands16_scatter", "octets_gather", "bytes_r2_rep", "bytes_ragged13_gather"])
def test_band_builds_with_pointer_table(name):
    """Narrow band layouts (quad rows, narrow bands, 2-byte column runs) with
    their shard pointers in the device table (a batch of copies of one narrow
    layout, more pointers than the kernel arguments hold), so every pointer
    lookup goes through the table."""
    spec = {s.name: s for s in small_specs()}[name]
    per_copy = int(np.prod(spec.src_mesh)) + int(np.prod(spec.dst_mesh))
    copies = 120 // per_copy + 1
    st = run_parity([spec] * copies, "raw", 9)
    assert st["n_src_ptrs"] + st["n_dst_ptrs"] > 120


def test_batched_mixed_dtypes():
    specs = list(W.ffn_refit(2, 64, 224).tensors) + [W.uneven(77, 53).tensors[0]] + \
        [s for s in small_specs() if s.name in ("u8_odd", "i64", "five_d", "rep_src", "conv_f32_f16_ragged",
                                                "conv_f16_f32_nested", "narrow_scatter", "narrow_gather_rep",
                                                "narrow_bf16_cols", "wide_window")]
    run_parity(specs, "raw", 5)


def _narrowing_patterns():
    """f32 bit patterns: every upper half with lower halves at and around each
    place a bf16 or f16 rounding decision (normal or subnormal) is taken."""
    lows = [0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2001, 0x3000, 0x3FFF, 0x4000,
            0x4001, 0x5000, 0x6000, 0x7000, 0x7FFF, 0x8000, 0x8001, 0x9000, 0xA000, 0xBFFF, 0xC000,
            0xC001, 0xE000, 0xF000, 0xFFFE, 0xFFFF, 0x0800, 0x1800, 0x2800, 0x5555, 0xAAAA]
    hi = torch.arange(1 << 16, dtype=torch.int64) << 16
    bits = (hi[:, None] | torch.tensor(lows, dtype=torch.int64)[None, :]).reshape(-1)
    return bits.to(torch.int32).view(torch.float32)   # wraps to the signed pattern, same bits


@pytest.mark.parametrize("layout", ["ragged", "aligned"])
@pytest.mark.parametrize("conv", ["f32_bf16", "f32_f16", "bf16_f32", "f16_f32"])
def test_conversion_bit_patterns(conv, layout):
    """Every rounding case of the formats through the kernel's conversion:
    all 2^16 upper halves of an f32 with 32 lower halves around each rounding
    point (ties, one below, one above; normal and subnormal targets, overflow,
    NaN payloads), or all 2^16 patterns of a 16-bit format, each four times.
    'ragged': (2,)[S0] -> (3,)[S0], shard rows off the 16-byte grid (element
    path at the edges); 'aligned': (2,)[S0] -> (2,)[S0] (16-byte path)."""
    src_dt, dst_dt = {"f32_bf16": (torch.float32, torch.bfloat16), "f32_f16": (torch.float32, torch.float16),
                      "bf16_f32": (torch.bfloat16, torch.float32), "f16_f32": (torch.float16, torch.float32)}[conv]
    if src_dt == torch.float32:
        g = _narrowing_patterns()
    else:
        g = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16).view(src_dt).repeat(4)
    n = g.numel()
    if layout == "ragged":
        spec = W.TensorSpec(f"bits_{conv}", (n - 3,), src_dt, (2,), (0,), (3,), (0,), dst_dt)
        g = g[:n - 3].contiguous()
    else:
        spec = W.TensorSpec(f"bits_{conv}", (n,), src_dt, (2,), (0,), (2,), (0,), dst_dt)
    run_parity([spec], "given", 0, globals_=[g])


def test_pointer_slot_ring():
    """More pointers than kernel arguments hold: each execute with a new pointer
    set goes through the slot ring (wrapping it), repeats reuse the slot."""
    specs = list(W.ffn_refit(16, 64, 96).tensors)  # 48 tensors x 10 ranks = 480 pointers
    with Plan(specs) as plan:
        assert_boxes_agree(plan)
        assert_descriptors_in_bounds(plan)
        srcs_all, want_all = [], []
        src_sets = []
        for t, spec in enumerate(specs):
            g = W.make_global(spec, "raw", 9, t)
            sb = oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements)
            srcs = W.cut(g, sb)
            srcs_all.append(srcs)
            from reshard_harness import oracle_dsts
            want_all.append(oracle_dsts(spec, srcs))
            gs = GuardedShards(shard_nbytes(sb, spec.dtype), "cuda")
            for i, s in enumerate(srcs):
                gs.region(i).copy_(s.reshape(-1).view(torch.uint8).cuda())
            src_sets.append(gs)
        src_ptrs = [p for s in src_sets for p in s.ptrs]
        stream = torch.cuda.current_stream().cuda_stream
        rounds = []
        for k in range(11):  # 11 distinct destination sets > 8 slots
            dsts = [GuardedShards(shard_nbytes(oracle_boxes(s.shape, s.dst_mesh, s.dst_placements),
                                               s.dtype), "cuda") for s in specs]
            dst_ptrs = [p for d in dsts for p in d.ptrs]
            R.reshard_execute(plan.handle, src_ptrs, dst_ptrs, stream)
            if k == 3:  # the same pointers again: slot reuse without a copy
                R.reshard_execute(plan.handle, src_ptrs, dst_ptrs, stream)
            rounds.append(dsts)
        torch.cuda.synchronize()
        for dsts in rounds:
            for t, spec in enumerate(specs):
                for i, w in enumerate(want_all[t]):
                    assert torch.equal(dsts[t].region(i).cpu(), w.reshape(-1).view(torch.uint8))
                    assert dsts[t].guards_intact(i)


def test_pointer_slot_reused_from_another_stream():
    """A pointer set just copied into a device slot on a busy stream, executed
    again on another stream: the second launch must wait for the copy that
    fills the slot.  Every slot first holds a valid older set, and the set the
    slot held before (set 0) had its destinations overwritten with a canary: a
    launch that read the slot too early would copy set 0 again and destroy it."""
    from reshard_harness import oracle_dsts
    specs = list(W.ffn_refit(16, 64, 96).tensors)  # 480 pointers: device slots
    with Plan(specs) as plan:
        sets = []
        for seed in (31, 32, 33):  # three source sets with different values
            want, srcs_d = [], []
            for t, spec in enumerate(specs):
                g = W.make_global(spec, "raw", seed, t)
                sb = oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements)
                srcs = W.cut(g, sb)
                want.append(oracle_dsts(spec, srcs))
                gs = GuardedShards(shard_nbytes(sb, spec.dtype), "cuda")
                for i, x in enumerate(srcs):
                    gs.region(i).copy_(x.reshape(-1).view(torch.uint8).cuda())
                srcs_d.append(gs)
            dsts = [GuardedShards(shard_nbytes(oracle_boxes(s.shape, s.dst_mesh, s.dst_placements), s.dtype),
                                  "cuda") for s in specs]
            sets.append((want, srcs_d, dsts))
        ptrs = [([p for g in sd for p in g.ptrs], [p for d in dd for p in d.ptrs]) for _, sd, dd in sets]
        a, b = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        for k in range(8):  # every slot of the ring holds set 0 or set 1; slot 0 holds set 0
            R.reshard_execute(plan.handle, *ptrs[k % 2], a.cuda_stream)
        torch.cuda.synchronize()
        for d in sets[0][2]:
            for i in range(len(d.nbytes)):
                if d.nbytes[i]:
                    d.region(i).fill_(0x5A)
        busy = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(a):
            for _ in range(20):  # keep stream a busy ahead of the next copy
                busy.add_(1)
        R.reshard_execute(plan.handle, *ptrs[2], a.cuda_stream)  # slot 0, copied on a
        R.reshard_execute(plan.handle, *ptrs[2], b.cuda_stream)  # same pointers, on b
        torch.cuda.synchronize()
        for d in sets[0][2]:
            for i in range(len(d.nbytes)):
                if d.nbytes[i]:
                    assert bool((d.region(i) == 0x5A).all().item()), "set 0 was copied again"
        for k in (1, 2):
            want, _, dsts = sets[k]
            for t in range(len(specs)):
                for i, w in enumerate(want[t]):
                    assert torch.equal(dsts[t].region(i).cpu(), w.reshape(-1).view(torch.uint8))
                    assert dsts[t].guards_intact(i)


def test_two_streams_concurrently():
    spec = W.ffn_up(1024, 512).tensors[0]
    with Plan([spec]) as plan:
        assert_boxes_agree(plan)
        g = W.make_global(spec, "raw", 11)
        sb = oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements)
        db = oracle_boxes(spec.shape, spec.dst_mesh, spec.dst_placements)
        srcs = W.cut(g, sb)
        from reshard_harness import oracle_dsts
        want = oracle_dsts(spec, srcs)
        src = GuardedShards(shard_nbytes(sb, spec.dtype), "cuda")
        for i, s in enumerate(srcs):
            src.region(i).copy_(s.reshape(-1).view(torch.uint8).cuda())
        torch.cuda.synchronize()
        outs = []
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for st in streams:
            d = GuardedShards(shard_nbytes(db, spec.dtype), "cuda")
            torch.cuda.synchronize()
            with torch.cuda.stream(st):
                for _ in range(3):
                    R.reshard_execute(plan.handle, src.ptrs, d.ptrs, st.cuda_stream)
            outs.append(d)
        torch.cuda.synchronize()
        for d in outs:
            for i, w in enumerate(want):
                assert torch.equal(d.region(i).cpu(), w.reshape(-1).view(torch.uint8))
                assert d.guards_intact(i)


def test_empty_plan_launches_nothing():
    spec = T("zero", (0, 6), torch.float32, (2,), (0,), (3,), (1,))
    with Plan([spec]) as plan:
        R.reshard_execute(plan.handle, [0, 0], [0, 0, 0], torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert plan.stats()["n_workgroups"] == 0


def test_upload_and_stats_after_execute():
    with Plan(W.ffn_up().tensors) as plan:
        R.reshard_plan_upload(plan.handle, torch.cuda.current_stream().cuda_stream)
        st = plan.stats()
        tiles = -(-117440512 // 4096)  # one workgroup per 4 KiB source tile
        per_xcd = -(-(-(-tiles // 8)) // 64) * 64  # whole groups of 64 tiles per XCD
        assert st["n_workgroups"] == 8 * per_xcd
    with Plan(W.worked_example_8x8().tensors) as plan:  # fewer tiles than one group round
        R.reshard_plan_upload(plan.handle, torch.cuda.current_stream().cuda_stream)
        assert plan.stats()["n_workgroups"] == 2
        R.reshard_plan_upload(plan.handle, None)  # second upload is a no-op


def test_gather_then_slice_two_plans_match_oracle():
    """The comparator the benchmark times (sources -> one global buffer ->
    destinations, two plans of the same library) produces the oracle's bytes."""
    from reshard_harness import oracle_dsts
    for spec in (W.uneven(301, 257).tensors[0], W.ffn_up(448, 320).tensors[0]):
        code = R.dtype_code(spec.dtype)
        with Plan([spec]) as plan:
            g_lay = R.reshard_layout_create(spec.shape, code, (1,), (R.REPLICATE,))
            p_g = R.reshard_plan_create(plan.src_layouts[0], g_lay)
            p_s = R.reshard_plan_create(g_lay, plan.dst_layouts[0])
            g = W.make_global(spec, "raw", 12)
            srcs = W.cut(g, oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements))
            want = oracle_dsts(spec, srcs)
            src_d = [s.cuda() for s in srcs]
            glob = torch.empty(spec.shape, dtype=spec.dtype, device="cuda")
            dst_d = [torch.empty_like(w, device="cuda") for w in want]
            stream = torch.cuda.current_stream().cuda_stream
            R.reshard_execute(p_g, [t.data_ptr() for t in src_d], [glob.data_ptr()], stream)
            R.reshard_execute(p_s, [glob.data_ptr()], [t.data_ptr() for t in dst_d], stream)
            torch.cuda.synchronize()
            assert torch.equal(glob.cpu().view(torch.uint8), g.view(torch.uint8))
            for got, w in zip(dst_d, want):
                assert torch.equal(got.cpu().view(torch.uint8), w.view(torch.uint8))
            R.reshard_plan_destroy(p_g)
            R.reshard_plan_destroy(p_s)
            R.reshard_layout_destroy(g_lay)


@pytest.mark.parametrize("layers", [1, 16], ids=["kernel_arg_pointers", "slot_ring_pointers"])
def test_execute_from_many_threads(layers):
    """One plan executed concurrently from several host threads, each on its own
    stream with its own destination buffers; with more pointers than kernel
    arguments hold, every call goes through the shared slot ring.  Plan stats
    are read between the calls, racing the first call's upload."""
    import threading
    from reshard_harness import oracle_dsts
    specs = list(W.ffn_refit(layers, 64, 96).tensors)
    with Plan(specs) as plan:
        assert_boxes_agree(plan)
        assert_descriptors_in_bounds(plan)
        want, src_sets = [], []
        for t, spec in enumerate(specs):
            g = W.make_global(spec, "raw", 21, t)
            sb = oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements)
            srcs = W.cut(g, sb)
            want.append(oracle_dsts(spec, srcs))
            gs = GuardedShards(shard_nbytes(sb, spec.dtype), "cuda")
            for i, s in enumerate(srcs):
                gs.region(i).copy_(s.reshape(-1).view(torch.uint8).cuda())
            src_sets.append(gs)
        src_ptrs = [p for s in src_sets for p in s.ptrs]
        outs = [[GuardedShards(shard_nbytes(oracle_boxes(s.shape, s.dst_mesh, s.dst_placements), s.dtype),
                               "cuda") for s in specs] for _ in range(4)]
        torch.cuda.synchronize()
        errors, seen, after = [], [], []

        def work(k):
            try:
                st = torch.cuda.Stream()
                dst_ptrs = [p for d in outs[k] for p in d.ptrs]
                with torch.cuda.stream(st):
                    for _ in range(5):
                        seen.append(R.reshard_plan_stats(plan.handle)["n_launches"])  # racing the upload
                        R.reshard_execute(plan.handle, src_ptrs, dst_ptrs, st.cuda_stream)
                        after.append(R.reshard_plan_stats(plan.handle)["n_launches"])
                st.synchronize()
            except Exception as e:  # noqa: BLE001
                errors.append(e)
        threads = [threading.Thread(target=work, args=(k,)) for k in range(4)]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        torch.cuda.synchronize()
        assert not errors, errors
        final = plan.stats()["n_launches"]
        assert final >= 1 and set(after) == {final} and set(seen) <= {0, final}
        for dsts in outs:
            for t in range(len(specs)):
                for i, w in enumerate(want[t]):
                    assert torch.equal(dsts[t].region(i).cpu(), w.reshape(-1).view(torch.uint8))
                    assert dsts[t].guards_intact(i)


@pytest.mark.parametrize("chunks", [1, 4])
def test_two_stage_send_once_then_exchange(chunks):
    """The two-stage transport (each box delivered once, split over its replicas,
    then assembled by every replica; pipelined over tensor chunks on two
    streams) reaches the oracle's bytes."""
    from dtensor_layout_movement_amd.two_stage import TwoStagePlan
    from reshard_harness import oracle_dsts
    from reshard_harness import oracle_cut
    strided = {s.name: s for s in small_specs()}
    specs = list(W.ffn_refit(3, 64, 224).tensors) + [W.ffn_up(448, 320).tensors[0], W.uneven(301, 257).tensors[0],
                                                      strided["strided_dst"], strided["strided_both"]]
    ts = TwoStagePlan(specs, chunks=chunks)
    try:
        srcs_d, dsts_d, stag_d, wants = [], [], [], []
        for t, spec in enumerate(specs):
            g = W.make_global(spec, "raw", 31, t)
            srcs = oracle_cut(spec, g)
            wants.append(oracle_dsts(spec, srcs))
            srcs_d.append([s.cuda() if s is not None else None for s in srcs])
            dsts_d.append([torch.full_like(w, 0, device="cuda") for w in wants[-1]])
        for t, shapes in enumerate(ts.staging_shapes()):
            stag_d.append([torch.empty(sh, dtype=specs[t].dtype, device="cuda") if all(sh) else None
                           for sh in shapes])
        ptr = lambda lst: [[x.data_ptr() if x is not None and x.numel() else 0 for x in row] for row in lst]
        arrays = ts.pointer_arrays(ptr(srcs_d), ptr(stag_d), ptr(dsts_d))
        a, b = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        events = [torch.cuda.Event() for _ in arrays]
        ts.execute(arrays, a, b, events)
        torch.cuda.synchronize()
        for t in range(len(specs)):
            for got, w in zip(dsts_d[t], wants[t]):
                assert torch.equal(got.cpu().view(torch.uint8), w.view(torch.uint8)), specs[t].name
    finally:
        ts.close()


def test_hybrid_routing_matches_oracle():
    """FFN projections by the reshard, the other weights by gather-then-slice,
    all on one stream: every destination shard equals the oracle's."""
    from dtensor_layout_movement_amd.hybrid import HybridPlan
    from reshard_harness import oracle_dsts
    specs = W.dense_layer_refit(2, 256, 64, 512).tensors
    hp = HybridPlan(specs)
    try:
        srcs_d, dsts_d, wants = [], [], []
        for t, spec in enumerate(specs):
            g = W.make_global(spec, "raw", 41, t)
            srcs = W.cut(g, oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements))
            wants.append(oracle_dsts(spec, srcs))
            srcs_d.append([s.cuda() if s is not None else None for s in srcs])
            dsts_d.append([torch.zeros_like(w, device="cuda") for w in wants[-1]])
        glob = [torch.empty(sh, dtype=specs[t].dtype, device="cuda")
                for t, sh in zip(hp.gather, hp.global_shapes())]
        ptr = lambda lst: [[x.data_ptr() if x is not None and x.numel() else 0 for x in row] for row in lst]
        arrays = hp.pointer_arrays(ptr(srcs_d), ptr(dsts_d), [g.data_ptr() for g in glob])
        stream = torch.cuda.current_stream()
        hp.execute(arrays, stream.cuda_stream)
        torch.cuda.synchronize()
        for t in range(len(specs)):
            for got, w in zip(dsts_d[t], wants[t]):
                assert torch.equal(got.cpu().view(torch.uint8), w.view(torch.uint8)), specs[t].name
    finally:
        hp.close()


@pytest.mark.parametrize("batch", range(5))
def test_random_layouts_batched(batch):
    """Seeded random layout pairs of moderate size (1-4 dims, up to three mesh
    dims, nested / replicated / empty shards, several dtypes and conversions),
    six per fused launch."""
    specs = random_specs(100 + batch, 6)
    run_parity(specs, "raw", batch)


@pytest.mark.parametrize("batch", range(3))
def test_random_strided_layouts_batched(batch):
    """Seeded random layout pairs with right-to-left (strided) nesting on either
    side, six per plan, together with three plain random pairs in the same
    fused launch."""
    specs = strided_random_specs(700 + batch, 6) + random_specs(800 + batch, 3)
    run_parity(specs, "raw", batch)


@pytest.mark.parametrize("batch", range(4))
def test_narrow_random_layouts(batch):
    """Seeded random narrow layouts (rows of at most 32 bytes; whole rows against
    4-byte runs, replicas, ragged row counts), one plan each, so that each runs
    the build its descriptors select: row bands, quad and 8-lane exchanges, LDS
    windows, items or chunks."""
    for spec in narrow_random_specs(300 + batch, 10):
        run_parity([spec], "raw", 8)


def test_graph_capture_replays_match_oracle():
    """An execute captured into a HIP graph (torch.cuda.CUDAGraph on a side
    stream) replays the reshard: three replays, each after eager work that
    clears the destinations and changes the sources, each checked against the
    oracle for the sources of that replay."""
    from reshard_harness import oracle_dsts
    spec = W.uneven(301, 257).tensors[0]
    with Plan([spec]) as plan:
        stream = torch.cuda.Stream()
        R.reshard_plan_upload(plan.handle, stream.cuda_stream)
        sboxes = oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements)
        srcs = [s.cuda() for s in W.cut(W.make_global(spec, "raw", 0, 0), sboxes)]
        dsts = [torch.zeros(box_shape(b), dtype=spec.dtype, device="cuda")
                for b in oracle_boxes(spec.shape, spec.dst_mesh, spec.dst_placements)]
        sp = R.pointer_array([s.data_ptr() for s in srcs])
        dp = R.pointer_array([d.data_ptr() for d in dsts])
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            R.reshard_execute(plan.handle, sp, dp, stream.cuda_stream)
        torch.cuda.synchronize()
        for rep in range(3):
            fresh = W.cut(W.make_global(spec, "raw", 10 + rep, 0), sboxes)
            for s, f in zip(srcs, fresh):
                s.copy_(f)          # eager work between replays: new sources ...
            for d in dsts:
                d.zero_()           # ... and cleared destinations (fill kernels)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            want = oracle_dsts(spec, fresh)
            for got, w in zip(dsts, want):
                assert torch.equal(got.cpu().view(torch.uint8), w.view(torch.uint8)), rep


def test_graph_capture_refused_for_pointer_table_plans():
    """A plan whose pointers need the device slot ring refuses to be captured
    and records nothing; it still runs eagerly afterwards."""
    specs = W.ffn_refit(16, 64, 224).tensors      # 48 tensors x 10 ranks > 120 pointers
    with Plan(specs) as plan:
        stream = torch.cuda.Stream()
        R.reshard_plan_upload(plan.handle, stream.cuda_stream)
        st = plan.stats()
        assert st["n_src_ptrs"] + st["n_dst_ptrs"] > 120
        graph = torch.cuda.CUDAGraph()
        with pytest.raises(R.ReshardError) as e:
            with torch.cuda.graph(graph, stream=stream):
                R.reshard_execute(plan.handle, [0x1000] * st["n_src_ptrs"], [0x2000] * st["n_dst_ptrs"],
                                  stream.cuda_stream)
        assert e.value.status == R.ERR_INVALID_ARGUMENT and "captured" in str(e.value)
        torch.cuda.synchronize()
    run_parity(list(W.ffn_refit(16, 64, 224).tensors), "raw", 9)


def _mixed_kind_specs():
    """A batch that mixes descriptor kinds: 16-byte items of a 32 MiB projection,
    narrow bands of 64 MiB of 8-byte column slices, destination chunks, a small
    band of 2-byte column runs and gather-rows bands (8002-byte rows from three
    column strips)."""
    small = {s.name: s for s in small_specs()}
    return [T("mix_rows", (4096, 4096), torch.bfloat16, (4,), (0,), (2, 2), (RR, 1)),
            W.narrow_columns_64b_tp8(1 << 20).tensors[0],
            W.uneven(301, 257).tensors[0], small["narrow_bf16_cols"], small["wide_window"]]


def test_mixed_kinds_one_launch_per_group():
    """The descriptors that are not bands share one launch, and each band kind
    (narrow bands, 2-byte column runs, gather rows) runs in a launch of its
    own build; bit-exact.  Items with chunks, or one band kind alone, stay one
    launch."""
    specs = _mixed_kind_specs()
    assert run_parity(specs, "raw", 12)["n_launches"] == 4
    assert run_parity([specs[1]], "raw", 13)["n_launches"] == 1
    assert run_parity([specs[0], specs[2]], "raw", 15)["n_launches"] == 1
    assert run_parity([specs[0], specs[2], specs[4]], "raw", 15)["n_launches"] == 2
    assert run_parity([specs[1], specs[3]], "raw", 16)["n_launches"] == 2
    # a plan smaller than one pass over the chip is split the same way
    small = [W.ffn_up(1024, 1024).tensors[0], W.narrow_columns_64b_tp8(1 << 14).tensors[0]]
    assert run_parity(small, "raw", 17)["n_launches"] == 2


def test_mixed_kinds_with_pointer_table():
    """The same groups with the shard pointers in the device slot ring (small
    copies appended to pass the kernel-argument slots): every launch of the
    execute reads the same slot."""
    spec = {s.name: s for s in small_specs()}["narrow_scatter_rep"]
    specs = _mixed_kind_specs() + [spec] * 12
    st = run_parity(specs, "raw", 14, executes=2)
    assert st["n_src_ptrs"] + st["n_dst_ptrs"] > 120 and st["n_launches"] == 5  # + the quad row bands


def test_mixed_kinds_graph_capture_replays():
    """A mixed plan's launches captured into one HIP graph replay correctly:
    three replays after eager work that changes the sources and clears the
    destinations, each checked against the oracle."""
    from reshard_harness import oracle_dsts
    specs = _mixed_kind_specs()
    with Plan(specs) as plan:
        stream = torch.cuda.Stream()
        R.reshard_plan_upload(plan.handle, stream.cuda_stream)
        assert plan.stats()["n_launches"] == 4
        sboxes = [oracle_boxes(s.shape, s.src_mesh, s.src_placements) for s in specs]
        srcs = [[p.cuda() for p in W.cut(W.make_global(s, "raw", 0, t), b)] for t, (s, b) in
                enumerate(zip(specs, sboxes))]
        dsts = [[torch.zeros(box_shape(b), dtype=s.dtype, device="cuda")
                 for b in oracle_boxes(s.shape, s.dst_mesh, s.dst_placements)] for s in specs]
        sp = R.pointer_array([x.data_ptr() for xs in srcs for x in xs])
        dp = R.pointer_array([x.data_ptr() for xs in dsts for x in xs])
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            R.reshard_execute(plan.handle, sp, dp, stream.cuda_stream)
        torch.cuda.synchronize()
        for rep in range(3):
            fresh = [W.cut(W.make_global(s, "raw", 20 + rep, t), b) for t, (s, b) in enumerate(zip(specs, sboxes))]
            for xs, fs in zip(srcs, fresh):
                for x, f in zip(xs, fs):
                    x.copy_(f)
            for xs in dsts:
                for x in xs:
                    x.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for s, xs, fs in zip(specs, dsts, fresh):
                for got, w in zip(xs, oracle_dsts(s, fs, threads=8)):
                    assert torch.equal(got.cpu().view(torch.uint8), w.view(torch.uint8)), (rep, s.name)


@pytest.mark.parametrize("seed", range(3))
def test_random_mixed_launch_groups(seed):
    """Three narrow band workloads of 4096 tiles each, drawn at random, batched
    with seeded random layouts and small narrow ones in shuffled order: the plan
    runs as several launch groups (one per band build drawn, quad rows, 2-byte
    column runs or narrow bands), and every destination is bit-exact."""
    import random
    rng = random.Random(seed)
    bands = [(W.narrow_columns(1 << 21), "quad"), (W.narrow_columns_tp8(1 << 21), "narrow"),
             (W.narrow_columns_64b_tp8(1 << 20), "narrow"), (W.narrow_columns_64b_tp4(1 << 20), "narrow"),
             (W.narrow_columns_32b_tp4(1 << 21), "narrow"), (W.narrow_columns_16b_tp8(1 << 21), "octets")]
    drawn = rng.sample(bands, 3)
    specs = [w.tensors[0] for w, _ in drawn] + random_specs(400 + seed, 4) + narrow_random_specs(500 + seed, 3)
    rng.shuffle(specs)
    st = run_parity(specs, "raw", 30 + seed)
    # the descriptors that are not bands, and each band build drawn
    assert st["n_launches"] >= 1 + len({k for _, k in drawn})
