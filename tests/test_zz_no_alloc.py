"""GPU tests of reshard_execute_noalloc, the entry point that allocates nothing:
its output must equal reshard_execute's (and the oracle's) byte for byte, over
two calls in a row where the second plan is smaller than the first, with the
pointers in the kernel arguments and in the static scratch array."""
import pytest
import torch

import dtensor_layout_movement_amd as R
from dtensor_layout_movement_amd import workloads as W
from gpu_harness import GuardedShards, shard_nbytes
from reshard_harness import Plan, assert_boxes_agree, oracle_boxes, oracle_dsts

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


def run_both(specs, seed):
    """Execute one plan through both entry points into separate guarded
    destinations; both must equal the oracle byte for byte."""
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream().cuda_stream
    with Plan(specs) as plan:
        assert_boxes_agree(plan)
        srcs, dst_a, dst_b, host_srcs = [], [], [], []
        for t, spec in enumerate(plan.specs):
            sboxes = oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements)
            dboxes = oracle_boxes(spec.shape, spec.dst_mesh, spec.dst_placements)
            g = W.make_global(spec, "raw", seed, t)
            pieces = W.cut(g, sboxes)
            host_srcs.append(pieces)
            s = GuardedShards(shard_nbytes(sboxes, spec.dtype), dev)
            for i, piece in enumerate(pieces):
                if piece is not None:
                    s.region(i).copy_(piece.reshape(-1).view(torch.uint8).to(dev))
            srcs.append(s)
            dst_a.append(GuardedShards(shard_nbytes(dboxes, spec.out_dtype), dev))
            dst_b.append(GuardedShards(shard_nbytes(dboxes, spec.out_dtype), dev))
        sp = [p for s in srcs for p in s.ptrs]
        print(f"[noalloc] {specs[0].name} x{len(specs)} seed={seed} pointers={len(sp) + sum(len(d.ptrs) for d in dst_a)}",
              flush=True)
        R.reshard_execute(plan.handle, sp, [p for d in dst_a for p in d.ptrs], stream)
        R.reshard_execute_noalloc(plan.handle, sp, [p for d in dst_b for p in d.ptrs], stream)
        torch.cuda.synchronize()
        for t, spec in enumerate(plan.specs):
            want = oracle_dsts(spec, host_srcs[t])
            for i, w in enumerate(want):
                if dst_a[t].nbytes[i]:
                    a, b = dst_a[t].region(i).cpu(), dst_b[t].region(i).cpu()
                    assert torch.equal(a, b), (spec.name, t, i)
                    assert torch.equal(b, w.reshape(-1).view(torch.uint8)), (spec.name, t, i)
                assert dst_a[t].guards_intact(i) and dst_b[t].guards_intact(i), (spec.name, t, i)
        return plan.stats()


def test_noalloc_two_calls_kernel_argument_pointers():
    """A batched plan (ragged fp32 nested split + replicated bf16 projection +
    narrow columns), then the smaller worked example: the second call's table
    overwrites the first's in the scratch array."""
    big = [W.uneven(301, 257).tensors[0], W.ffn_up(448, 320).tensors[0], W.narrow_columns(4096).tensors[0]]
    st = run_both(big, 1)
    assert st["n_src_ptrs"] + st["n_dst_ptrs"] <= 120
    small = [W.worked_example_8x8().tensors[0]]
    st2 = run_both(small, 2)
    assert st2["n_descriptors"] < st["n_descriptors"]


def test_noalloc_two_calls_pointer_table():
    """More than 120 shard pointers (they go to the scratch array after the
    table), then a smaller plan that still needs the pointer table."""
    one = T("refit_small", (96, 64), torch.bfloat16, (2,), (0,), (2, 4), (RR, 1))
    st = run_both([one] * 16, 3)
    assert st["n_src_ptrs"] + st["n_dst_ptrs"] > 120
    st2 = run_both([one] * 13, 4)
    assert 120 < st2["n_src_ptrs"] + st2["n_dst_ptrs"] < st["n_src_ptrs"] + st["n_dst_ptrs"]


def test_noalloc_refuses_a_plan_beyond_the_scratch_array():
    """A plan whose table exceeds the static array is refused before anything is
    copied or launched (the pointers are real buffers all the same)."""
    n_t = 800
    spec = T("tiny", (4096,), torch.uint8, (64,), (0,), (64,), (0,))
    with Plan([spec] * n_t) as plan:
        st = plan.stats()
        assert st["n_descriptors"] * 128 > 2 * R.reshard.NOALLOC_SCRATCH_BYTES
        buf = torch.zeros(2 * 4096 * n_t, dtype=torch.uint8, device="cuda")
        base = buf.data_ptr()
        sp = [base + 64 * i for i in range(64 * n_t)]
        dp = [base + 4096 * n_t + 64 * i for i in range(64 * n_t)]
        with pytest.raises(R.ReshardError) as e:
            R.reshard_execute_noalloc(plan.handle, sp, dp, torch.cuda.current_stream().cuda_stream)
        assert e.value.status == R.ERR_INVALID_ARGUMENT and "scratch" in str(e.value)
        torch.cuda.synchronize()
        assert int(buf[4096 * n_t:].sum().item()) == 0  # nothing was written


def test_noalloc_narrow_band_windows():
    """Narrow bands in launches of both window sizes (dynamic LDS sized per
    launch): 4-byte shards of 64-byte rows (the usual window) with single u8
    columns of 16-byte rows (twice the rows), then a smaller plan of 2-byte
    shards of 64-byte rows (twice the rows)."""
    mix = [W.narrow_columns_64b_tp16(2048).tensors[0],
           T("u8_cols", (4099, 16), torch.uint8, (2,), (0,), (16,), (1,))]
    st = run_both(mix, 5)
    assert st["n_launches"] >= 2
    small = [T("bf16_cols", (1031, 32), torch.bfloat16, (2,), (0,), (32,), (1,))]
    run_both(small, 6)


def test_noalloc_then_execute_same_plan_repeatedly():
    """The two entry points alternate on one plan and one stream; every result
    is compared with the oracle."""
    spec = W.uneven(500, 301).tensors[0]
    for k in range(3):
        run_both([spec], 10 + k)
