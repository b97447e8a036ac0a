"""Seeded synthetic reshard workloads.

This module only describes inputs: global shapes, dtypes, source and
destination layouts, and seeded value generators.  It holds none of the
reshard's arithmetic (no shard boxes, no intersections): code that needs a
rank's box asks either the product library or, in tests, the oracle, and hands
the boxes to ``cut``.

Workloads (all synthetic; the pages publish no dataset and no per-tensor
numbers, only an 8x8 example and multi-node refit latencies):

* ``worked_example_8x8`` -- the pages' example: an 8x8 matrix row-sharded over
  two training GPUs and column-sharded over four inference GPUs, so that every
  destination receives one 4x2 block from each source (techfeed.io write-up,
  "reformulation" section; news.bpdata.com write-up, "the approach" section).
  Values 0..63, exact in bf16.
* ``ffn_up_14336x4096`` -- one feed-forward up-projection (the FFN projections
  carry about 95% of the refit payload: techfeed.io, "results" section):
  TP4 row split -> DP2 x TP2 column split.
* ``moe_experts_64x2048x7168`` -- an MoE expert stack: EP8 x TP2 -> DP2 x TP8.
* ``uneven_5000x3001`` -- odd fp32 shape with a nested split of one dim into
  ragged chunks -> seven row shards.
* ``ffn_refit_32_layers`` -- 32 layers x (gate, up, down) moved by one fused
  launch: 4 pipeline stages x TP2 -> DP2 x TP4.
* ``ffn_up_fsdp2_tp_14336x4096`` -- the up-projection trained under FSDP2 x TP
  (right-to-left nesting, DTensor's _StridedShard) -> DP2 x TP2.
* ``ffn_up_partial_14336x4096`` -- the up-projection held as two Partial (sum)
  contributions, rows split over 4 -> DP2 x TP2; contribution q of tensor t
  under seed s draws from generator seed 1000 s + t + 7919 (q + 1).

Values: bf16 tensors are N(0, 0.02) drawn in fp32 and rounded to nearest-even;
fp32 tensors are U[-1, 1); "raw" fills every byte uniformly at random (NaN
payloads, infinities, signed zeros and subnormals included).  Tensor t of a
workload under seed s draws from ``torch.Generator().manual_seed(1000*s + t)``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence

import torch

R = -1  # Replicate placement code (Shard(k) is k)
P = -2  # Partial (sum) placement code, source layouts only


@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: tuple
    dtype: torch.dtype
    src_mesh: tuple
    src_placements: tuple
    dst_mesh: tuple
    dst_placements: tuple
    dst_dtype: torch.dtype | None = None  # another float format: a converting reshard
    src_split: tuple | None = None  # split factor per source mesh dim (right-to-left nesting)
    dst_split: tuple | None = None  # the same for the destination; None: all 1

    @property
    def out_dtype(self) -> torch.dtype:
        """Element type of the destination shards."""
        return self.dst_dtype if self.dst_dtype is not None else self.dtype

    @property
    def partial(self) -> int:
        """Contributions of a Partial (sum) source: the product of the sizes of
        its Partial mesh dims (0 for a source without any)."""
        n = 0
        for m, p in zip(self.src_mesh, self.src_placements):
            if p == P:
                n = (n or 1) * m
        return n

    @property
    def strided(self) -> bool:
        """Whether either layout nests right to left (a split factor above 1)."""
        return any(f > 1 for f in (self.src_split or ()) + (self.dst_split or ()))

    def split(self, side: str) -> tuple:
        """Split factors of the "src" or "dst" layout, one per mesh dim."""
        mesh = self.src_mesh if side == "src" else self.dst_mesh
        f = self.src_split if side == "src" else self.dst_split
        return tuple(f) if f is not None else (1,) * len(mesh)


@dataclass(frozen=True)
class Workload:
    name: str
    tensors: tuple
    values: str  # "arange" | "normal" | "uniform"
    description: str

    @property
    def global_bytes(self) -> int:
        return sum(_numel(t.shape) * _esize(t.dtype) for t in self.tensors)


def _numel(shape) -> int:
    n = 1
    for s in shape:
        n *= s
    return n


def _esize(dtype: torch.dtype) -> int:
    return torch.empty((), dtype=dtype).element_size()


def worked_example_8x8() -> Workload:
    t = TensorSpec("w", (8, 8), torch.bfloat16, (2,), (0,), (4,), (1,))
    return Workload("worked_example_8x8", (t,), "arange",
                    "8x8 bf16 0..63, (2,)[S0] -> (4,)[S1]")


def ffn_up(rows: int = 14336, cols: int = 4096) -> Workload:
    t = TensorSpec("up_proj", (rows, cols), torch.bfloat16, (4,), (0,), (2, 2), (R, 1))
    return Workload(f"ffn_up_{rows}x{cols}", (t,), "normal",
                    f"{rows}x{cols} bf16 N(0,0.02), (4,)[S0] -> (2,2)[R,S1]")


def ffn_up_fsdp2_tp(rows: int = 14336, cols: int = 4096) -> Workload:
    """The up-projection trained under FSDP2 (2) x TP (4): TP splits the rows
    first and FSDP each TP slice, which DTensor writes as [_StridedShard(0,
    split_factor=4), Shard(0)] on the (dp, tp) mesh -> DP2 x TP2 column split."""
    t = TensorSpec("up_proj", (rows, cols), torch.bfloat16, (2, 4), (0, 0), (2, 2), (R, 1), src_split=(4, 1))
    return Workload(f"ffn_up_fsdp2_tp_{rows}x{cols}", (t,), "normal",
                    f"{rows}x{cols} bf16 N(0,0.02), (2,4)[S0 strided by 4, S0] -> (2,2)[R,S1]")


def ffn_up_partial(rows: int = 14336, cols: int = 4096) -> Workload:
    """The up-projection held as two partial sums (a Partial mesh dim of 2, rows
    split over 4) -> DP2 x TP2 column split of the summed weight."""
    t = TensorSpec("up_proj", (rows, cols), torch.bfloat16, (2, 4), (P, 0), (2, 2), (R, 1))
    return Workload(f"ffn_up_partial_{rows}x{cols}", (t,), "normal",
                    f"{rows}x{cols} bf16 N(0,0.02) x 2 contributions, (2,4)[P,S0] -> (2,2)[R,S1]")


def moe_experts(experts: int = 64, hidden: int = 2048, ffn: int = 7168) -> Workload:
    t = TensorSpec("experts", (experts, hidden, ffn), torch.bfloat16, (8, 2), (0, 1), (2, 8), (R, 2))
    return Workload(f"moe_experts_{experts}x{hidden}x{ffn}", (t,), "normal",
                    f"[{experts},{hidden},{ffn}] bf16 N(0,0.02), (8,2)[S0,S1] -> (2,8)[R,S2]")


def uneven(rows: int = 5000, cols: int = 3001) -> Workload:
    t = TensorSpec("uneven", (rows, cols), torch.float32, (3, 2), (1, 1), (7,), (0,))
    return Workload(f"uneven_{rows}x{cols}", (t,), "uniform",
                    f"{rows}x{cols} fp32 U[-1,1), (3,2)[S1,S1] -> (7,)[S0]")


def ffn_refit(layers: int = 32, hidden: int = 4096, ffn: int = 14336, stages: int = 4) -> Workload:
    """Per layer gate [ffn, hidden], up [ffn, hidden], down [hidden, ffn].  Each
    tensor lives on its pipeline stage's 2-rank mesh; tensors are ordered
    layer-major (gate, up, down)."""
    ts = []
    for layer in range(layers):
        for name in ("gate", "up", "down"):
            if name == "down":
                shape, sp, dp = (hidden, ffn), (1,), (R, 1)
            else:
                shape, sp, dp = (ffn, hidden), (0,), (R, 0)
            ts.append(TensorSpec(f"layer{layer}.{name}", shape, torch.bfloat16, (2,), sp, (2, 4), dp))
    return Workload(f"ffn_refit_{layers}_layers", tuple(ts), "normal",
                    f"{layers} layers x (gate {ffn}x{hidden}, up {ffn}x{hidden}, down {hidden}x{ffn}) "
                    f"bf16, PP{stages} x (2,)[S0|S1] -> (2,4)[R,S0|S1], one fused launch")


def dense_layer_refit(layers: int = 32, hidden: int = 4096, kv: int = 1024, ffn: int = 14336,
                      stages: int = 4) -> Workload:
    """Every weight of `layers` dense transformer layers in one fused launch:
    q [hidden, hidden], k and v [kv, hidden] (grouped-query attention), o
    [hidden, hidden], gate/up [ffn, hidden], down [hidden, ffn], and two norm
    vectors [hidden].  Training side: a pipeline stage's 2-rank mesh, matrices
    split on their output dim (row) except o and down, split on the input dim;
    the norm vectors replicated on both ranks.  Inference side: (2, 4) = DP2 x
    TP4 with the same split dims; the norm vectors replicated on all 8 ranks."""
    ts = []
    for layer in range(layers):
        for name, shape, d in (("q", (hidden, hidden), 0), ("k", (kv, hidden), 0), ("v", (kv, hidden), 0),
                               ("o", (hidden, hidden), 1), ("gate", (ffn, hidden), 0),
                               ("up", (ffn, hidden), 0), ("down", (hidden, ffn), 1)):
            ts.append(TensorSpec(f"layer{layer}.{name}", shape, torch.bfloat16, (2,), (d,), (2, 4), (R, d)))
        for name in ("input_norm", "post_norm"):
            ts.append(TensorSpec(f"layer{layer}.{name}", (hidden,), torch.bfloat16, (2,), (R,), (2, 4), (R, R)))
    return Workload(f"dense_layer_refit_{layers}_layers", tuple(ts), "normal",
                    f"{layers} layers x (q, k, v, o, gate, up, down, 2 norms) bf16, PP{stages} x (2,) -> (2,4), "
                    f"one fused launch")


def ffn_up_f32_to_bf16(rows: int = 14336, cols: int = 4096) -> Workload:
    """The ffn_up layouts with a precision change on the way: fp32 training
    weights, TP4 over rows, to bf16 inference weights, DP2 x TP2 over columns
    (each element converted once per destination replica)."""
    t = TensorSpec("up_proj", (rows, cols), torch.float32, (4,), (0,), (2, 2), (R, 1), torch.bfloat16)
    return Workload(f"ffn_up_f32_to_bf16_{rows}x{cols}", (t,), "normal",
                    f"{rows}x{cols} fp32 N(0,0.02) (4,)[S0] -> bf16 (2,2)[R,S1]")


def stage_of_layer(layer: int, layers: int = 32, stages: int = 4) -> int:
    """Pipeline stage holding `layer` (contiguous blocks of layers per stage)."""
    return layer * stages // layers


def narrow_columns(rows: int = 1 << 22) -> Workload:
    """The worked example's layouts on a tall matrix: 8 bf16 columns, rows split
    over two sources, columns over four destinations, so every destination row is
    a 2-element (4-byte) slice of a 16-byte source row."""
    t = TensorSpec("narrow", (rows, 8), torch.bfloat16, (2,), (0,), (4,), (1,))
    return Workload(f"narrow_columns_{rows}x8", (t,), "normal",
                    f"{rows}x8 bf16 N(0,0.02), (2,)[S0] -> (4,)[S1]: 2-element column slices")


def narrow_columns_tp8(rows: int = 1 << 21) -> Workload:
    """16 bf16 columns (32-byte rows: the shape of a rank-16 low-rank factor),
    rows split over two sources, columns over eight destinations: every
    destination row is a 2-element (4-byte) slice of a 32-byte source row (the
    8-lane word exchange)."""
    t = TensorSpec("narrow16", (rows, 16), torch.bfloat16, (2,), (0,), (8,), (1,))
    return Workload(f"narrow_columns_tp8_{rows}x16", (t,), "normal",
                    f"{rows}x16 bf16 N(0,0.02), (2,)[S0] -> (8,)[S1]: 2-element slices of 32-byte rows")


def narrow_columns_64b_tp8(rows: int = 1 << 20) -> Workload:
    """32 bf16 columns (64-byte rows: a rank-32 low-rank factor), rows split over
    two sources, columns over eight destinations: every destination row is a
    4-element (8-byte) slice of a 64-byte source row, moved through an LDS
    window."""
    t = TensorSpec("narrow32", (rows, 32), torch.bfloat16, (2,), (0,), (8,), (1,))
    return Workload(f"narrow_columns_64b_tp8_{rows}x32", (t,), "normal",
                    f"{rows}x32 bf16 N(0,0.02), (2,)[S0] -> (8,)[S1]: 4-element slices of 64-byte rows")


def narrow_columns_64b_tp4(rows: int = 1 << 20) -> Workload:
    """32 bf16 columns (64-byte rows), rows split over two sources, columns over
    four destinations: every destination row is an 8-element (16-byte) slice of
    a 64-byte source row, moved as 16-byte chunks."""
    t = TensorSpec("narrow32q", (rows, 32), torch.bfloat16, (2,), (0,), (4,), (1,))
    return Workload(f"narrow_columns_64b_tp4_{rows}x32", (t,), "normal",
                    f"{rows}x32 bf16 N(0,0.02), (2,)[S0] -> (4,)[S1]: 8-element slices of 64-byte rows")


def narrow_columns_32b_tp4(rows: int = 1 << 21) -> Workload:
    """16 bf16 columns (32-byte rows: a rank-16 factor), rows split over two
    sources, columns over four destinations: every destination row is a
    4-element (8-byte) slice of a 32-byte source row (half and quad exchanges)."""
    t = TensorSpec("narrow16q", (rows, 16), torch.bfloat16, (2,), (0,), (4,), (1,))
    return Workload(f"narrow_columns_32b_tp4_{rows}x16", (t,), "normal",
                    f"{rows}x16 bf16 N(0,0.02), (2,)[S0] -> (4,)[S1]: 4-element slices of 32-byte rows")


def narrow_columns_16b_tp8(rows: int = 1 << 22) -> Workload:
    """8 bf16 columns (16-byte rows: a rank-8 factor), rows split over two
    sources, columns over eight destinations: every destination row is one
    element (2 bytes) of a 16-byte source row (halfword octet exchange)."""
    t = TensorSpec("narrow8o", (rows, 8), torch.bfloat16, (2,), (0,), (8,), (1,))
    return Workload(f"narrow_columns_16b_tp8_{rows}x8", (t,), "normal",
                    f"{rows}x8 bf16 N(0,0.02), (2,)[S0] -> (8,)[S1]: single columns of 16-byte rows")


def narrow_columns_8b_tp2(rows: int = 1 << 23) -> Workload:
    """4 bf16 columns (8-byte rows), rows split over two sources, columns over
    two destinations: every destination row is a 2-element (4-byte) half of an
    8-byte source row."""
    t = TensorSpec("narrow4", (rows, 4), torch.bfloat16, (2,), (0,), (2,), (1,))
    return Workload(f"narrow_columns_8b_tp2_{rows}x4", (t,), "normal",
                    f"{rows}x4 bf16 N(0,0.02), (2,)[S0] -> (2,)[S1]: 4-byte halves of 8-byte rows")


def narrow_columns_64b_tp16(rows: int = 1 << 20) -> Workload:
    """32 bf16 columns (64-byte rows), rows split over two sources, columns over
    sixteen destinations: every destination row is a 2-element (4-byte) slice
    of a 64-byte source row."""
    t = TensorSpec("narrow32s", (rows, 32), torch.bfloat16, (2,), (0,), (16,), (1,))
    return Workload(f"narrow_columns_64b_tp16_{rows}x32", (t,), "normal",
                    f"{rows}x32 bf16 N(0,0.02), (2,)[S0] -> (16,)[S1]: 4-byte slices of 64-byte rows")


def narrow_columns_ragged_tp4(rows: int = 2396745) -> Workload:
    """14 bf16 columns (28-byte rows) over four destinations: ceil-split column
    shards of 4, 4, 4 and 2 elements (8-, 8-, 8- and 4-byte runs)."""
    t = TensorSpec("narrow14", (rows, 14), torch.bfloat16, (2,), (0,), (4,), (1,))
    return Workload(f"narrow_columns_ragged_tp4_{rows}x14", (t,), "normal",
                    f"{rows}x14 bf16 N(0,0.02), (2,)[S0] -> (4,)[S1]: ragged 8/8/8/4-byte column shards")


def narrow_columns_2b_tp16(rows: int = 1 << 21) -> Workload:
    """16 bf16 columns (32-byte rows, a rank-16 low-rank factor) over sixteen
    destinations: every destination row is a single 2-byte column."""
    t = TensorSpec("narrow16t", (rows, 16), torch.bfloat16, (2,), (0,), (16,), (1,))
    return Workload(f"narrow_columns_2b_tp16_{rows}x16", (t,), "normal",
                    f"{rows}x16 bf16 N(0,0.02), (2,)[S0] -> (16,)[S1]: single bf16 columns of 32-byte rows")


WORKLOADS = {
    "worked_example_8x8": worked_example_8x8,
    "ffn_up_14336x4096": ffn_up,
    "moe_experts_64x2048x7168": moe_experts,
    "uneven_5000x3001": uneven,
    "ffn_refit_32_layers": ffn_refit,
    "narrow_columns_4194304x8": narrow_columns,
    "narrow_columns_tp8_2097152x16": narrow_columns_tp8,
    "narrow_columns_64b_tp8_1048576x32": narrow_columns_64b_tp8,
    "narrow_columns_64b_tp4_1048576x32": narrow_columns_64b_tp4,
    "narrow_columns_32b_tp4_2097152x16": narrow_columns_32b_tp4,
    "narrow_columns_16b_tp8_4194304x8": narrow_columns_16b_tp8,
    "ffn_up_f32_to_bf16_14336x4096": ffn_up_f32_to_bf16,
    "dense_layer_refit_32_layers": dense_layer_refit,
    "ffn_up_fsdp2_tp_14336x4096": ffn_up_fsdp2_tp,
    "ffn_up_partial_14336x4096": ffn_up_partial,
    "narrow_columns_8b_tp2_8388608x4": narrow_columns_8b_tp2,
    "narrow_columns_64b_tp16_1048576x32": narrow_columns_64b_tp16,
    "narrow_columns_ragged_tp4_2396745x14": narrow_columns_ragged_tp4,
    "narrow_columns_2b_tp16_2097152x16": narrow_columns_2b_tp16,
}


def generator(seed: int, tensor_index: int, device="cpu") -> torch.Generator:
    return torch.Generator(device=device).manual_seed(1000 * seed + tensor_index)


def make_global(spec: TensorSpec, values: str, seed: int, tensor_index: int = 0,
                device="cpu") -> torch.Tensor:
    """The seeded global tensor (contiguous) of one workload tensor.  The CPU and
    GPU generators are different streams: a given (seed, device) is reproducible."""
    g = generator(seed, tensor_index, device)
    if values == "arange":
        n = _numel(spec.shape)
        return torch.arange(n, dtype=torch.float32, device=device).reshape(spec.shape).to(spec.dtype)
    if values == "normal":
        x = torch.randn(spec.shape, generator=g, dtype=torch.float32, device=device)
        return (x * 0.02).to(spec.dtype)
    if values == "uniform":
        x = torch.rand(spec.shape, generator=g, dtype=torch.float32, device=device)
        return (x * 2 - 1).to(spec.dtype)
    if values == "raw":
        nbytes = _numel(spec.shape) * _esize(spec.dtype)
        raw = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g, device=device)
        return raw.view(spec.dtype).reshape(spec.shape)
    raise ValueError(f"unknown value kind {values!r}")


def contribution_of(spec: TensorSpec, rank: int) -> int:
    """The contribution a source rank of a Partial spec holds: its coordinates
    on the Partial mesh dims, row-major (ranks are row-major over the mesh)."""
    coords = []
    for m in reversed(spec.src_mesh):
        coords.append(rank % m)
        rank //= m
    q = 0
    for c, m, p in zip(reversed(coords), spec.src_mesh, spec.src_placements):
        if p == P:
            q = q * m + c
    return q


def make_contributions(spec: TensorSpec, values: str, seed: int, tensor_index: int = 0, device="cpu") -> list:
    """The seeded contributions of a Partial source, one global-shaped tensor
    each (contribution q draws from tensor index tensor_index + 7919 (q + 1))."""
    return [make_global(spec, values, seed, tensor_index + 7919 * (q + 1), device=device)
            for q in range(spec.partial)]


def cut_indexed(global_tensor: torch.Tensor, index_lists: Sequence) -> list:
    """Contiguous copies of the global tensor restricted, along every dim, to a
    list of global indices (one list of per-dim lists per rank); None for an
    empty shard."""
    out = []
    for lists in index_lists:
        if any(len(ix) == 0 for ix in lists):
            out.append(None)
            continue
        x = global_tensor
        for k, ix in enumerate(lists):
            x = x.index_select(k, torch.as_tensor(list(ix), dtype=torch.int64, device=x.device))
        out.append(x.contiguous())
    return out


def cut(global_tensor: torch.Tensor, boxes: Sequence) -> list:
    """Contiguous copies of ``global_tensor[lo:hi, ...]`` for each ``(lo, hi)`` box;
    None for empty boxes."""
    out = []
    for lo, hi in boxes:
        if any(h <= l for l, h in zip(lo, hi)):
            out.append(None)
            continue
        idx = tuple(slice(l, h) for l, h in zip(lo, hi))
        out.append(global_tensor[idx].contiguous())
    return out
