"""GPU parity at sizes past the 32-bit limits: shards larger than 4 GiB (64-bit
byte offsets inside one shard) and a piece of more than 2^31 16-byte items (the
planner splits it over several descriptors).  Every element holds its own
global linear index (int64, or int32 wrapped modulo 2^32), so the expected
content of any destination shard is a closed form of its box; it is computed
with plain PyTorch on the GPU, chunk by chunk, and compared element by element
with what the kernel wrote.  The CPU oracle is not used here: at 10-70 GB per
case it would take minutes; the small and full-workload cases pin the same
paths against it."""
import pytest
import torch

import dtensor_layout_movement_amd as R
from dtensor_layout_movement_amd import workloads as W
from reshard_harness import Plan, assert_boxes_agree, assert_descriptors_in_bounds, box_shape, oracle_boxes

pytestmark = pytest.mark.gpu

T = W.TensorSpec
RR = W.R
CHUNK = 1 << 26  # elements per generated or compared chunk
MAX_LAUNCH_BLOCKS = (0xFFFFFFFF // 256) & ~7  # workgroups of one launch at most


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def index_block(lo, hi, ncols, r0, r1, dtype):
    """Global linear indices of rows [r0, r1) of the 2-d box [lo, hi), as dtype
    (int32: wrapped to two's complement modulo 2^32)."""
    rows = torch.arange(lo[0] + r0, lo[0] + r1, device="cuda", dtype=torch.int64)
    cols = torch.arange(lo[1], hi[1], device="cuda", dtype=torch.int64)
    idx = rows[:, None] * ncols + cols[None, :]
    if dtype == torch.int32:
        idx = torch.remainder(idx + (1 << 31), 1 << 32) - (1 << 31)
    return idx.to(dtype)


def row_chunks(box):
    n_rows, width = box_shape(box)
    step = max(1, CHUNK // max(1, width))
    for r0 in range(0, n_rows, step):
        yield r0, min(n_rows, r0 + step)


def check_large(spec):
    assert len(spec.shape) == 2
    ncols = spec.shape[1]
    with Plan([spec]) as plan:
        assert_boxes_agree(plan)
        assert_descriptors_in_bounds(plan)
        sboxes = oracle_boxes(spec.shape, spec.src_mesh, spec.src_placements)
        dboxes = oracle_boxes(spec.shape, spec.dst_mesh, spec.dst_placements)
        srcs = []
        for box in sboxes:
            t = torch.empty(box_shape(box), dtype=spec.dtype, device="cuda")
            for r0, r1 in row_chunks(box):
                t[r0:r1] = index_block(box[0], box[1], ncols, r0, r1, spec.dtype)
            srcs.append(t)
        dsts = [torch.full(box_shape(box), -1, dtype=spec.dtype, device="cuda") for box in dboxes]
        st = plan.stats()
        print(f"[large] {spec.name} shape={spec.shape} {spec.dtype} descriptors={st['n_descriptors']} "
              f"bytes_read={st['bytes_read']} largest_shard={max(s.numel() * s.element_size() for s in srcs + dsts)}",
              flush=True)
        R.reshard_execute(plan.handle, [s.data_ptr() for s in srcs], [d.data_ptr() for d in dsts],
                          torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        del srcs
        for i, (box, d) in enumerate(zip(dboxes, dsts)):
            for r0, r1 in row_chunks(box):
                want = index_block(box[0], box[1], ncols, r0, r1, spec.dtype)
                got = d[r0:r1]
                if not torch.equal(got, want):
                    bad = (got != want).nonzero()[0].tolist()
                    pytest.fail(f"{spec.name}: destination {i} differs at row {r0 + bad[0]}, col {bad[1]}: "
                                f"{got[bad[0], bad[1]].item()} != {want[bad[0], bad[1]].item()}")
        del dsts
        torch.cuda.empty_cache()
        return st


def test_piece_over_2_31_items():
    """One 32 GiB piece (2^31 16-byte items) copied whole: split over several
    descriptors, each indexing fewer than 2^31 items; byte offsets past 2^32."""
    st = check_large(T("big_copy", (1 << 31, 2), torch.int64, (1,), (RR,), (1,), (RR,)))
    assert st["n_descriptors"] > 1


def test_launch_split_over_2_24_workgroups():
    """A 69 GB copy needs more workgroups than one dispatch can count in 32-bit
    work-items: the execute goes out as two launches, the second continuing the
    plan's block numbering."""
    spec = T("big_split", ((1 << 32) + (1 << 24), 2), torch.int64, (1,), (RR,), (1,), (RR,))
    check_large(spec)
    with Plan([spec]) as plan:  # the same plan's grid, after an upload
        R.reshard_plan_upload(plan.handle, torch.cuda.current_stream().cuda_stream)
        assert plan.stats()["n_workgroups"] > MAX_LAUNCH_BLOCKS


def test_item_path_shards_over_4_gib():
    """16-byte items with fan-out 2 from 4.6 GB source shards (row offsets past
    2^32 bytes inside a shard)."""
    check_large(T("big_items", (65536, 34816), torch.int32, (2,), (0,), (2, 2), (RR, 1)))


def test_quad_row_bands_over_4_gib():
    """16-byte rows cut into four 4-byte column runs (the quad exchange) from
    4.3 GB source shards: band row offsets past 2^32 bytes."""
    check_large(T("big_quad", ((1 << 29) + (1 << 20), 4), torch.int32, (2,), (0,), (4,), (1,)))


def test_destination_chunks_over_4_gib():
    """The uneven config's layouts (misaligned column strips, destination
    chunks) at 2.2 M rows: 4.4 GB source shards, 3.8 GB destination shards."""
    check_large(T("big_strips", (2200000, 3001), torch.int32, (3, 2), (1, 1), (7,), (0,)))
