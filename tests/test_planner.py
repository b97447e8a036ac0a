"""Host planner of the reshard library, on the CPU (no GPU needed: planning is
host-only).  The plan is checked three ways against the oracle: by applying its
pieces, by walking its device descriptor table byte by byte, and by the plan
invariants I1-I6 (coverage, byte totals, containment, replica balance,
determinism)."""
import ctypes
import os
import random
import re
import subprocess

import numpy as np
import pytest
import torch

import dtensor_layout_movement_amd as R
import oracle_pins as P
from dtensor_layout_movement_amd import workloads as W
from reshard_harness import (Plan, apply_pieces, assert_boxes_agree, assert_descriptors_in_bounds,
                             box_shape, is_narrow_band, lib_runs, magic_div, narrow_pitch,
                             oracle_dsts, run_descriptors, sources_for)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "reshard.h")

T = W.TensorSpec
RR = W.R


def small_specs():
    """Reduced versions of every workload plus supplemental layouts."""
    specs = [
        W.worked_example_8x8().tensors[0],
        W.ffn_up(112, 64).tensors[0],
        W.moe_experts(16, 64, 448).tensors[0],
        W.uneven(500, 301).tensors[0],
        *W.ffn_refit(2, 64, 224).tensors,
        T("rep_src", (37, 29), torch.float32, (2, 2), (RR, 0), (3,), (1,)),
        T("rep_both", (40, 24), torch.bfloat16, (3, 2), (RR, 1), (2, 2), (0, RR)),
        T("fanout8", (33, 17), torch.float32, (3,), (0,), (4, 2), (RR, RR)),
        T("empty_src", (5, 3), torch.bfloat16, (4,), (0,), (2,), (1,)),
        T("empty_both", (3, 2), torch.float32, (5,), (1,), (4, 2), (0, 1)),
        T("zero_dim", (0, 6), torch.float32, (2,), (0,), (3,), (1,)),
        T("u8_odd", (13, 7, 5), torch.uint8, (2, 3), (0, 2), (3,), (1,)),
        T("i64", (9, 11), torch.int64, (2,), (1,), (3, 2), (0, 1)),
        T("five_d", (3, 4, 5, 6, 7), torch.bfloat16, (2, 2), (1, 3), (3, 2), (4, 0)),
        T("eight_d", (2, 3, 2, 3, 2, 3, 2, 3), torch.float32, (2, 3), (1, 7), (3, 2), (3, 0)),
        T("nested", (9, 4, 10), torch.bfloat16, (2, 3), (0, 0), (2, 2, 2), (2, 0, 2)),
        T("one_elem", (1,), torch.float32, (3,), (0,), (2,), (RR,)),
        T("peel_outer", (3, 5, 5, 5, 6), torch.float32, (2, 2, 2), (1, 2, 3), (2,), (4,)),
        T("chunked_bf16", (37, 301), torch.bfloat16, (3,), (1,), (2, 2), (RR, 0)),
        T("chunked_u8", (9, 1000), torch.uint8, (3,), (1,), (2,), (0,)),
        T("chunked_f64", (11, 45), torch.float64, (2,), (1,), (3,), (0,)),
        T("narrow_scatter", (4099, 8), torch.bfloat16, (2,), (0,), (4,), (1,)),
        T("narrow_gather", (4099, 8), torch.bfloat16, (4,), (1,), (2,), (0,)),
        T("narrow_fp8_3d", (6, 7, 24), torch.uint8, (2, 3), (0, 2), (4,), (2,)),
        T("narrow_rep", (301, 12), torch.float32, (3,), (1,), (2, 3), (RR, 1)),
        # 16-byte rows cut into four 4-byte column runs (quad transposes), row
        # counts that leave partial quads
        T("narrow_scatter_rep", (1031, 8), torch.bfloat16, (2,), (0,), (2, 4), (RR, 1)),
        T("narrow_f32_cols", (2053, 4), torch.float32, (3,), (0,), (4,), (1,)),
        T("narrow_gather_rep", (1029, 8), torch.bfloat16, (2, 4), (RR, 1), (3,), (0,)),
        # 32-byte rows cut into eight 4-byte column runs (8-lane exchange), row
        # counts that leave partial groups of eight
        T("runs_scatter", (1043, 16), torch.bfloat16, (2,), (0,), (8,), (1,)),
        T("runs_gather", (1043, 16), torch.bfloat16, (8,), (1,), (3,), (0,)),
        T("runs_scatter_rep", (517, 16), torch.bfloat16, (2,), (0,), (2, 8), (RR, 1)),
        T("runs_f32_cols", (1029, 8), torch.float32, (3,), (0,), (8,), (1,)),
        # 64-byte rows cut into eight 8-byte column runs (quarter and 8-lane
        # exchanges), row counts that leave partial pairs and short waves
        T("runs64_scatter", (1043, 32), torch.bfloat16, (2,), (0,), (8,), (1,)),
        T("runs64_gather", (1037, 32), torch.bfloat16, (8,), (1,), (3,), (0,)),
        T("runs64_scatter_rep", (517, 16), torch.float32, (3,), (0,), (2, 8), (RR, 1)),
        T("runs64_tiny", (3, 32), torch.bfloat16, (1,), (0,), (8,), (1,)),
        # bands of packed 16-byte-aligned segments (16-byte chunks, no LDS):
        # 16-byte runs in 64-byte rows, 32-byte runs in 128- and 256-byte rows,
        # gather, fan-out, ragged tails
        T("bands16_scatter", (1043, 32), torch.bfloat16, (2,), (0,), (4,), (1,)),
        T("bands16_gather", (1037, 64), torch.bfloat16, (4,), (1,), (3,), (0,)),
        T("bands16_rep", (517, 32), torch.float32, (3,), (0,), (2, 8), (RR, 1)),
        T("bands16_256", (1029, 128), torch.bfloat16, (2,), (0,), (8,), (1,)),
        T("bands16_tiny", (2, 16), torch.float32, (1,), (0,), (2,), (1,)),
        # chunks per row not a power of two: 96-, 48- and 80-byte rows
        T("bands16_96", (1031, 48), torch.bfloat16, (2,), (0,), (3,), (1,)),
        T("bands16_48_gather", (1033, 24), torch.bfloat16, (3,), (1,), (2,), (0,)),
        T("bands16_80_rep", (517, 20), torch.float32, (1,), (0,), (2, 5), (RR, 1)),
        # 32-byte rows cut into four 8-byte column runs (half and quad exchanges)
        T("runs32_scatter", (1043, 16), torch.bfloat16, (2,), (0,), (4,), (1,)),
        T("runs32_gather", (1037, 8), torch.float32, (4,), (1,), (3,), (0,)),
        T("runs32_scatter_rep", (517, 16), torch.bfloat16, (3,), (0,), (2, 4), (RR, 1)),
        T("runs32_tiny", (3, 16), torch.bfloat16, (1,), (0,), (4,), (1,)),
        # 16-byte rows cut into eight 2-byte column runs (halfword octet exchange)
        T("octets_gather", (1041, 8), torch.bfloat16, (8,), (1,), (3,), (0,)),
        T("octets_scatter_rep", (523, 8), torch.float16, (3,), (0,), (2, 8), (RR, 1)),
        T("octets_tiny", (5, 8), torch.bfloat16, (1,), (0,), (8,), (1,)),
        # single bf16 or fp16 columns of 32-byte rows over sixteen shards
        # gathered (thin runs on the source side), with destination replicas, tiny
        T("thin32_gather", (1041, 16), torch.float16, (16,), (1,), (3,), (0,)),
        T("thin32_gather_rep", (1029, 16), torch.bfloat16, (16,), (1,), (2, 3), (RR, 0)),
        T("thin32_tiny", (5, 16), torch.bfloat16, (1,), (0,), (16,), (1,)),
        # narrow bands at 2- and 1-byte granularity and past 256 bytes: single
        # bf16 columns of 32- and 64-byte rows (scatter, gather, replicas),
        # ragged 8/8/8/2-byte shards of 26-byte rows (a pitch of one row), 6-,
        # 5- and 1-byte shards, odd row widths, 18-byte shards whose 16-byte
        # pieces straddle rows, 512-byte rows of 64-byte shards, a tiny band
        T("bytes_r2_in32", (1037, 16), torch.bfloat16, (2,), (0,), (16,), (1,)),
        T("bytes_r2_in64_gather", (1043, 32), torch.bfloat16, (32,), (1,), (3,), (0,)),
        T("bytes_r2_rep", (523, 16), torch.float16, (3,), (0,), (2, 16), (RR, 1)),
        T("bytes_ragged13", (2053, 13), torch.bfloat16, (2,), (0,), (4,), (1,)),
        T("bytes_ragged13_gather", (2053, 13), torch.bfloat16, (4,), (1,), (3,), (0,)),
        T("bytes_r6_in24", (1031, 12), torch.bfloat16, (3,), (0,), (4,), (1,)),
        T("bytes_u8_r5", (1029, 40), torch.uint8, (2,), (0,), (8,), (1,)),
        T("bytes_u8_r1", (1033, 24), torch.uint8, (2,), (0,), (24,), (1,)),
        T("bytes_u8_odd_rows", (1031, 19), torch.uint8, (3,), (0,), (2,), (1,)),
        T("bytes_pieces18", (1039, 18), torch.bfloat16, (2,), (0,), (2,), (1,)),
        T("bytes_pieces18_gather", (1039, 18), torch.bfloat16, (2,), (1,), (3,), (0,)),
        T("bytes_w512", (301, 256), torch.bfloat16, (2,), (0,), (8,), (1,)),
        T("bytes_w512_gather", (301, 256), torch.bfloat16, (8,), (1,), (2,), (0,)),
        T("bytes_tiny", (3, 13), torch.bfloat16, (1,), (0,), (4,), (1,)),
        # rows of at most 16 bytes with 1- or 2-byte shards (narrow bands too):
        # sixteen u8 columns, four bf16 columns, a gather of u8 columns, f16
        # pairs with replicas, three bf16 columns (a pitch of one row), tiny
        T("thin_u8_16", (1037, 16), torch.uint8, (2,), (0,), (16,), (1,)),
        T("thin_bf16_8", (2053, 4), torch.bfloat16, (3,), (0,), (4,), (1,)),
        T("thin_u8_gather", (1031, 8), torch.uint8, (8,), (1,), (3,), (0,)),
        T("thin_f16_rep", (1029, 2), torch.float16, (2,), (0,), (2, 2), (RR, 1)),
        T("thin_bf16_6", (2049, 3), torch.bfloat16, (2,), (0,), (3,), (1,)),
        T("thin_tiny", (5, 16), torch.uint8, (1,), (0,), (16,), (1,)),
        # 2-byte shards of 19-byte rows (an odd pitch: 2-byte window accesses at
        # odd addresses), scatter and gather
        T("thin_u8_odd_pitch", (1033, 19), torch.uint8, (2,), (0,), (10,), (1,)),
        T("thin_u8_odd_gather", (1033, 19), torch.uint8, (10,), (1,), (2,), (0,)),
        # 12-byte rows of 4-byte shards (narrow bands with rows back to back):
        # scatter, gather, replicas
        T("rows12_f32", (2053, 3), torch.float32, (2,), (0,), (3,), (1,)),
        T("rows12_gather", (1031, 6), torch.bfloat16, (3,), (1,), (2,), (0,)),
        T("rows12_rep", (517, 3), torch.float32, (3,), (0,), (2, 3), (RR, 1)),
        # shards of 3 to 15 bytes moved byte by byte in 16-byte pieces: gathers
        # of 6-byte and 5-byte shards, 7-byte shards with replicas
        T("bytes_r6_gather", (1031, 12), torch.bfloat16, (4,), (1,), (3,), (0,)),
        T("bytes_u8_r5_gather", (1029, 20), torch.uint8, (4,), (1,), (2,), (0,)),
        T("bytes_u8_r7_rep", (523, 28), torch.uint8, (2,), (0,), (2, 4), (RR, 1)),
        # rows of 24 and 40 bytes (a window pitch one dword wider): 16-byte
        # stream pieces whose dwords fall in two window rows, scattered,
        # scattered to replicas and gathered
        T("dwords24_scatter", (1031, 6), torch.float32, (2,), (0,), (3,), (1,)),
        T("dwords40_rep", (1029, 10), torch.float32, (3,), (0,), (2, 5), (RR, 1)),
        T("dwords24_gather", (1033, 6), torch.float32, (3,), (1,), (2,), (0,)),
        # 4-byte shards at an odd window pitch (10-byte rows): 16 stream bytes
        # a lane cover four rows, scattered and gathered
        T("rows4_w10", (1031, 5), torch.bfloat16, (2,), (0,), (3,), (1,)),
        T("rows4_w10_gather", (1029, 5), torch.bfloat16, (3,), (1,), (2,), (0,)),
        # rows of at most 16 bytes gathered from 3-byte shards or scattered into
        # 5- to 7-byte ones (narrow bands, not the row mode)
        T("bytes_u8_r3_gather", (1029, 12), torch.uint8, (4,), (1,), (3,), (0,)),
        T("bytes_r6_in12", (1033, 6), torch.bfloat16, (3,), (0,), (2,), (1,)),
        T("bytes_u8_r5_rep", (517, 15), torch.uint8, (2,), (0,), (2, 3), (RR, 1)),
        # replicated sources: each replica reads its own part of the rows
        T("rep_src_u8", (515, 40), torch.uint8, (3,), (RR,), (5,), (1,)),
        T("rep_src_bf16_rows", (1027, 24), torch.bfloat16, (2, 3), (RR, 0), (4,), (1,)),
        # 8-byte rows cut into two 4-byte column runs (register row mode)
        T("pairs_gather", (1029, 4), torch.bfloat16, (2,), (1,), (3,), (0,)),
        T("pairs_rep", (517, 2), torch.float32, (3,), (0,), (2, 2), (RR, 1)),
        T("pairs_tiny", (3, 4), torch.bfloat16, (1,), (0,), (2,), (1,)),
        # row mode without the quad exchange: single bf16 columns, 8-byte rows
        T("narrow_bf16_cols", (1037, 8), torch.bfloat16, (2,), (0,), (8,), (1,)),
        T("narrow_8byte_rows", (2051, 4), torch.bfloat16, (3,), (0,), (2,), (1,)),
        T("wide_window", (37, 4001), torch.bfloat16, (3,), (1,), (5,), (0,)),
        # misaligned column strips (destination-aligned chunks): row cuts inside a
        # destination shard, destination replicas, source replicas, nine strips,
        # a split middle dim; and a 4-byte piece in rows too wide for a window
        T("strips_row_cuts", (50, 301), torch.float32, (2, 2), (0, 1), (3,), (0,)),
        T("strips_fanout", (50, 301), torch.float32, (2, 2), (0, 1), (2, 3), (RR, 0)),
        T("strips_rep_src", (61, 301), torch.float32, (2, 3), (RR, 1), (4,), (0,)),
        T("strips_nine", (20, 333), torch.float32, (9,), (1,), (2,), (0,)),
        T("strips_mid_split", (6, 10, 301), torch.bfloat16, (2, 3), (1, 2), (3,), (2,)),
        T("narrow_wide_rows", (5, 4201), torch.float32, (4,), (1,), (2,), (1,)),
        # gather-rows bands (whole destination rows from source column strips of
        # at least 1 KiB that meet off the 16-byte grid): ragged nested split,
        # destination replicas, source replicas, row cuts inside destination
        # shards (bands that start mid-shard), rows that end inside a wave, a
        # split middle dim, and strips of exactly 1 KiB
        T("gather_uneven", (301, 1543), torch.float32, (3, 2), (1, 1), (7,), (0,)),
        T("gather_fanout", (256, 1030), torch.bfloat16, (2,), (1,), (2, 3), (RR, 0)),
        T("gather_rep_src", (100, 2049), torch.uint8, (2, 2), (RR, 1), (3,), (0,)),
        T("gather_row_cuts", (500, 1031), torch.float32, (3, 2), (0, 1), (4,), (0,)),
        T("gather_short_rows", (77, 1545), torch.uint8, (3,), (1,), (5,), (0,)),
        T("gather_mid_dim", (6, 4, 2051), torch.bfloat16, (2, 2), (0, 2), (3,), (0,)),
        T("gather_1k", (129, 2049), torch.uint8, (2,), (1,), (2,), (0,)),
        T("gather_17_strips", (40, 4384), torch.float32, (17,), (1,), (3,), (0,)),  # past the 14 column slots
        # converting reshards: ragged rows (not a multiple of 8 elements), fan-out,
        # nesting, peeled outer dims, empty shards
        T("conv_f32_bf16", (112, 64), torch.float32, (4,), (0,), (2, 2), (RR, 1), torch.bfloat16),
        T("conv_f32_f16_ragged", (37, 29), torch.float32, (2, 2), (RR, 0), (3,), (1,), torch.float16),
        T("conv_bf16_f32_ragged", (50, 31), torch.bfloat16, (3,), (1,), (2, 2), (0, RR), torch.float32),
        T("conv_f16_f32_nested", (9, 4, 10), torch.float16, (2, 3), (0, 0), (2, 2, 2), (2, 0, 2),
          torch.float32),
        T("conv_peel", (3, 5, 5, 5, 6), torch.float32, (2, 2, 2), (1, 2, 3), (2,), (4,), torch.bfloat16),
        T("conv_empty", (5, 3), torch.float32, (4,), (0,), (2,), (1,), torch.float16),
        T("conv_narrow", (4099, 8), torch.float32, (2,), (0,), (4,), (1,), torch.bfloat16),
    ]
    return specs + strided_specs() + partial_specs()


def partial_specs():
    """Partial (sum) sources: contributions over one or two mesh dims, replicas
    of a contribution, row and column splits, empty shards, conversions, a
    single contribution and ragged rows."""
    S = W.TensorSpec
    PP = W.P
    return [
        S("partial_tp2", (96, 40), torch.bfloat16, (2, 2), (PP, 0), (2, 2), (RR, 1)),
        S("partial_f32", (50, 31), torch.float32, (3,), (PP,), (2,), (0,)),
        S("partial_rep", (40, 24), torch.float32, (2, 2, 2), (RR, PP, 1), (4,), (0,), torch.bfloat16),
        S("partial_two_dims", (33, 17), torch.float16, (2, 3), (PP, PP), (2,), (1,)),
        S("partial_bf16_f32", (64, 48), torch.bfloat16, (4,), (PP,), (2, 2), (0, 1), torch.float32),
        S("partial_f32_f16", (31, 9), torch.float32, (2, 2), (PP, 0), (3,), (RR,), torch.float16),
        S("partial_empty", (5, 3), torch.float32, (2, 4), (PP, 0), (2,), (0,)),
        S("partial_nested", (3, 40, 12), torch.bfloat16, (2, 2, 2), (1, PP, 1), (2, 2), (2, RR)),
        S("partial_single", (20, 8), torch.float32, (1,), (PP,), (2,), (0,)),
        S("partial_ragged", (7, 13), torch.bfloat16, (3, 2), (PP, 1), (2,), (0,)),
    ]


def strided_specs():
    """Right-to-left (strided) nesting on either side: FSDP2 x TP training
    layouts, holdings of several runs per dim, empty shards, replicas, nesting
    over three mesh dims, narrow runs and a converting case."""
    S = W.TensorSpec
    return [
        S("strided_fsdp_tp", (96, 40), torch.bfloat16, (2, 4), (0, 0), (2, 2), (RR, 1), src_split=(4, 1)),
        S("strided_runs", (50, 31), torch.float32, (2, 2), (0, 0), (3,), (1,), src_split=(3, 1)),
        S("strided_dst", (64, 24), torch.bfloat16, (4,), (1,), (2, 2, 2), (RR, 1, 1), dst_split=(1, 2, 1)),
        S("strided_both", (3, 40, 12), torch.float32, (2, 3), (1, 1), (2, 2), (1, 2), src_split=(3, 1),
          dst_split=(2, 1)),
        S("strided_empty", (5, 7), torch.int16, (4,), (0,), (2,), (1,), src_split=(4,)),
        S("strided_three", (40, 6), torch.uint8, (2, 2, 2), (0, 0, 0), (2, 2), (1, 0), src_split=(2, 2, 1),
          dst_split=(1, 3)),
        S("strided_rep_src", (30, 20), torch.float64, (2, 3), (RR, 0), (2,), (1,), src_split=(1, 3)),
        S("strided_narrow", (1031, 8), torch.bfloat16, (2,), (0,), (4,), (1,), dst_split=(2,)),
        S("strided_same", (60, 16), torch.float32, (2, 3), (0, 0), (3, 2), (0, 0), src_split=(3, 1),
          dst_split=(2, 1)),
        S("strided_convert", (48, 36), torch.float32, (2, 2), (1, 1), (2, 2), (RR, 0), torch.bfloat16,
          src_split=(2, 1)),
    ]


def values_for(spec):
    """Random bytes, except for Partial sums: there a NaN's payload is the
    adder's to choose, so their bit-exact tests use normal values (NaN-ness is
    tested on its own)."""
    return "normal" if spec.partial else "raw"


@pytest.mark.parametrize("spec", small_specs(), ids=lambda s: s.name)
def test_pieces_and_descriptors_match_oracle(spec):
    with Plan([spec]) as plan:
        assert_boxes_agree(plan)
        g, srcs = sources_for(spec, values_for(spec), seed=0)
        want = oracle_dsts(spec, srcs)
        got = apply_pieces(plan, [srcs])[0]
        for d, (a, b) in enumerate(zip(got, want)):
            assert a.view(torch.uint8).numpy().tobytes() == b.view(torch.uint8).numpy().tobytes(), d
        # byte-level walk of the device table
        sflat = [None if s is None else s.contiguous().view(torch.uint8).reshape(-1).numpy()
                 for s in srcs]
        dflat = [np.full(int(np.prod(sh)) * spec.out_dtype.itemsize, 0xA5, dtype=np.uint8)
                 for sh in plan.dst_shapes(0)]
        run_descriptors(plan, sflat, dflat)
        for d, (a, b) in enumerate(zip(dflat, want)):
            assert a.tobytes() == b.view(torch.uint8).numpy().tobytes(), d


def test_batched_plan_matches_oracle():
    specs = W.ffn_refit(3, 64, 224).tensors + (W.uneven(50, 31).tensors[0],
                                                W.moe_experts(8, 32, 64).tensors[0])
    with Plan(specs) as plan:
        assert_boxes_agree(plan)
        srcs, wants = [], []
        for t, spec in enumerate(specs):
            _, s = sources_for(spec, "raw", seed=1, t=t)
            srcs.append(s)
            wants.append(oracle_dsts(spec, s))
        got = apply_pieces(plan, srcs)
        for t in range(len(specs)):
            for a, b in zip(got[t], wants[t]):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
        sflat = [None if s is None else s.view(torch.uint8).reshape(-1).numpy()
                 for ss in srcs for s in ss]
        dflat = [np.zeros(int(np.prod(box_shape(b))) * specs[t].dtype.itemsize, dtype=np.uint8)
                 for t in range(len(specs)) for b in plan.dst_boxes(t)]
        run_descriptors(plan, sflat, dflat)
        want_flat = [w.view(torch.uint8).reshape(-1).numpy() for ww in wants for w in ww]
        for a, b in zip(dflat, want_flat):
            assert a.tobytes() == b.tobytes()


def test_brute_force_random_layout_pairs():
    rng = random.Random(3)
    n = 0
    while n < 250:
        (shape, smesh, spl), = P.small_layouts(rng, 1)
        (_, dmesh, dpl), = P.small_layouts(rng, 1)
        dpl = tuple(p if p == RR else p % len(shape) for p in dpl)
        dtype = rng.choice([torch.uint8, torch.bfloat16, torch.float32, torch.float64])
        spec = T("bf", shape, dtype, smesh, spl, dmesh, dpl)
        with Plan([spec]) as plan:
            assert_boxes_agree(plan)
            _, srcs = sources_for(spec, "raw", seed=n)
            want = oracle_dsts(spec, srcs)
            got = apply_pieces(plan, [srcs])[0]
            for a, b in zip(got, want):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), spec
            sflat = [None if s is None else s.view(torch.uint8).reshape(-1).numpy() for s in srcs]
            dflat = [np.zeros(b.numel() * b.element_size(), dtype=np.uint8) for b in want]
            run_descriptors(plan, sflat, dflat)
            for a, b in zip(dflat, want):
                assert a.tobytes() == b.view(torch.uint8).reshape(-1).numpy().tobytes(), spec
        n += 1


def test_brute_force_random_strided_pairs():
    """Random small layout pairs with split factors on either side (DTensor's
    right-to-left placement): runs, pieces and the byte-level descriptor walk
    against the oracle's index lists."""
    rng = random.Random(5)
    for n in range(220):
        (shape, smesh, spl, ssp), = P.strided_layouts(rng, 1)
        (_, dmesh, dpl, dsp), = P.strided_layouts(rng, 1)
        dpl = tuple(p if p == RR else p % len(shape) for p in dpl)
        dtype = rng.choice([torch.uint8, torch.bfloat16, torch.float32, torch.float64])
        spec = T("sbf", shape, dtype, smesh, spl, dmesh, dpl, src_split=ssp, dst_split=dsp)
        with Plan([spec]) as plan:
            assert_boxes_agree(plan)
            assert_descriptors_in_bounds(plan)
            _, srcs = sources_for(spec, "raw", seed=n)
            want = oracle_dsts(spec, srcs)
            got = apply_pieces(plan, [srcs])[0]
            for a, b in zip(got, want):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), spec
            sflat = [None if s is None else s.view(torch.uint8).reshape(-1).numpy() for s in srcs]
            dflat = [np.zeros(b.numel() * b.element_size(), dtype=np.uint8) for b in want]
            run_descriptors(plan, sflat, dflat)
            for a, b in zip(dflat, want):
                assert a.tobytes() == b.view(torch.uint8).reshape(-1).numpy().tobytes(), spec
            st = plan.stats()
            assert st["bytes_read"] == int(np.prod(shape)) * dtype.itemsize


def strided_random_specs(seed, count, max_numel=300_000):
    """Seeded random layout pairs of moderate size with split factors 1-4 on
    either side (1-3 dims, meshes of up to three dims, several dtypes)."""
    rng = random.Random(seed)
    caps = {1: 200_000, 2: 1500, 3: 120}
    out = []
    while len(out) < count:
        nd = rng.randint(1, 3)
        shape = tuple(rng.choice([rng.randint(1, 9), rng.randint(1, caps[nd])]) for _ in range(nd))
        if int(np.prod(shape)) > max_numel:
            continue
        def layout():
            md = rng.randint(1, 3)
            mesh = tuple(rng.randint(1, 4) for _ in range(md))
            pl = tuple(rng.choice([RR] + list(range(nd))) for _ in range(md))
            return mesh, pl, tuple(1 if p == RR else rng.choice([1, 2, 3, 4]) for p in pl)
        (sm, sp, ss), (dm, dp, ds) = layout(), layout()
        dtype = rng.choice([torch.uint8, torch.bfloat16, torch.float32, torch.int16])
        out.append(T(f"srand{seed}_{len(out)}", shape, dtype, sm, sp, dm, dp, src_split=ss, dst_split=ds))
    return out


def test_strided_layout_calls_and_errors():
    # a split factor on a Replicate mesh dim, or below 1, is refused
    with pytest.raises(R.ReshardError) as e:
        R.reshard_layout_create_strided((8, 4), R.DTYPE_F32, (2, 2), (RR, 0), (2, 1))
    assert e.value.status == R.ERR_INVALID_ARGUMENT
    with pytest.raises(R.ReshardError):
        R.reshard_layout_create_strided((8, 4), R.DTYPE_F32, (2,), (0,), (0,))
    lay = R.reshard_layout_create_strided((8, 4), R.DTYPE_F32, (2, 2), (0, 0), (2, 1))
    try:
        # DTensor's documented example: rows {0,1}, {4,5}, {2,3}, {6,7}
        assert [R.reshard_layout_shard_runs(lay, r, 0) for r in range(4)] == [[(0, 2)], [(4, 6)], [(2, 4)], [(6, 8)]]
        assert R.reshard_layout_shard_runs(lay, 3, 1) == [(0, 4)]
        with pytest.raises(R.ReshardError):  # not a box
            R.reshard_layout_shard_box(lay, 0, 2)
        with pytest.raises(R.ReshardError):
            R.reshard_layout_shard_runs(lay, 4, 0)
        with pytest.raises(R.ReshardError):
            R.reshard_layout_shard_runs(lay, 0, 2)
    finally:
        R.reshard_layout_destroy(lay)
    # several runs in one shard, and an empty one
    lay = R.reshard_layout_create_strided((5,), R.DTYPE_U8, (4,), (0,), (4,))
    try:
        assert [R.reshard_layout_shard_runs(lay, r, 0) for r in range(4)] == [[(0, 1), (2, 3), (4, 5)],
                                                                              [(1, 2), (3, 4)], [], []]
    finally:
        R.reshard_layout_destroy(lay)
    # all factors 1: the plain layout, boxes and runs agree
    lay = R.reshard_layout_create_strided((9, 7), R.DTYPE_F32, (2, 3), (1, 0), (1, 1))
    try:
        for r in range(6):
            off, ext = R.reshard_layout_shard_box(lay, r, 2)
            for k in range(2):
                runs = R.reshard_layout_shard_runs(lay, r, k)
                assert runs == ([(off[k], off[k] + ext[k])] if ext[k] else [])
    finally:
        R.reshard_layout_destroy(lay)


def test_fsdp2_tp_layout_moves_as_plain_boxes():
    """FSDP2 x TP right-to-left sharding of an FFN projection gives every rank
    one run per dim, so the plan is the 16-byte item path of plain boxes."""
    wl = W.ffn_up_fsdp2_tp()
    with Plan(wl.tensors) as plan:
        assert_boxes_agree(plan)
        assert_descriptors_in_bounds(plan)
        for r in range(8):
            assert len(R.reshard_layout_shard_runs(plan.src_layouts[0], r, 0)) == 1
        descs, _ = R.reshard_plan_descriptors(plan.handle)
        assert all(D["mode"] == R.DESC_ITEMS and D["unit"] == 16 for D in descs)
        st = plan.stats()
        assert st["bytes_read"] == 14336 * 4096 * 2 and st["bytes_written"] == 2 * st["bytes_read"]


def random_specs(seed, count, max_numel=400_000):
    """Seeded random layout pairs of moderate size: 1-4 dims, meshes of up to
    three dims, any placements (nested, replicated, empty shards), several
    dtypes and the supported conversions."""
    rng = random.Random(seed)
    caps = {1: 200_000, 2: 1500, 3: 120, 4: 40}
    out = []
    while len(out) < count:
        nd = rng.randint(1, 4)
        shape = tuple(rng.choice([rng.randint(1, 7), rng.randint(1, caps[nd])]) for _ in range(nd))
        if int(np.prod(shape)) > max_numel:
            continue
        def layout():
            md = rng.randint(1, 3)
            mesh = tuple(rng.randint(1, 5) for _ in range(md))
            if int(np.prod(mesh)) > 32:
                mesh = mesh[:1]
            return mesh, tuple(rng.choice([RR] + list(range(nd))) for _ in range(len(mesh)))
        (sm, sp), (dm, dp) = layout(), layout()
        pair = rng.choice([(torch.uint8, None), (torch.bfloat16, None), (torch.float32, None),
                           (torch.float64, None), (torch.int16, None), (torch.float32, torch.bfloat16),
                           (torch.float32, torch.float16), (torch.bfloat16, torch.float32),
                           (torch.float16, torch.float32)])
        out.append(T(f"rand{seed}_{len(out)}", shape, pair[0], sm, sp, dm, dp, pair[1]))
    return out


def narrow_random_specs(seed, count):
    """Seeded random 2-d layouts whose rows are at most 512 bytes (odd widths
    included) and whose column splits, even or ragged, give shards of 1 to 256
    bytes: the register row mode, the quad and octet exchanges, the narrow
    bands of every segment class (thin runs of up to 32 segments among them)
    and the LDS windows, with ragged row counts (partial groups of four and
    eight rows, short last tiles), row splits on either side, replicas on either
    side (of column shards, of row shards, of the whole tensor) and every
    element size."""
    rng = random.Random(seed)
    out = []
    while len(out) < count:
        dtype = rng.choice([torch.uint8, torch.bfloat16, torch.float32, torch.float64])
        es = torch.tensor([], dtype=dtype).element_size()
        width = rng.choice([b for b in (4, 5, 6, 8, 10, 12, 13, 16, 19, 24, 26, 32, 48, 64, 96, 128, 256, 512)
                            if b >= es and b % es == 0])
        cols = width // es
        rows = rng.choice([rng.randint(1, 40), rng.randint(500, 1100), rng.randint(2000, 5000)])
        # runs the register exchanges move: four or eight 4-byte runs, eight 8-byte runs
        runs4 = 8 if width == 64 else width // 4 if width in (16, 32) and es <= 4 else 0
        def layout():
            k = rng.choice([c for c in (1, 2, 3, 4, 8, 16, 32) if c <= cols])
            if runs4 and rng.random() < 0.5:
                k = runs4
            r = rng.choice([1, 2, 3])
            kind = rng.randint(0, 5)
            if kind == 0:
                return (k,), (1,)
            if kind == 1:
                return (r,), (0,)
            if kind == 2:
                return (r, k), (0, 1)
            if kind == 3:
                return (2, k), (RR, 1)
            if kind == 4:  # replicated row shards (a source reads them in row parts, one per replica)
                return (rng.choice([2, 3]), r), (RR, 0)
            return (rng.choice([2, 3]),), (RR,)
        (sm, sp), (dm, dp) = layout(), layout()
        if runs4 and rng.random() < 0.4:  # whole rows on one side, 4-byte runs on the other
            rows_side = ((rng.choice([1, 2, 3]),), (0,))
            runs_side = rng.choice([((runs4,), (1,)), ((2, runs4), (RR, 1))])
            (sm, sp), (dm, dp) = (rows_side, runs_side) if rng.random() < 0.5 else (runs_side, rows_side)
        out.append(T(f"nrand{seed}_{len(out)}", (rows, cols), dtype, sm, sp, dm, dp))
    return out


def test_narrow_random_layouts_descriptor_walk():
    """40 seeded random narrow layouts: planned pieces and the byte-level walk of
    the descriptor table both equal the oracle."""
    for spec in narrow_random_specs(21, 40):
        with Plan([spec]) as plan:
            assert_boxes_agree(plan)
            assert_descriptors_in_bounds(plan)
            _, srcs = sources_for(spec, "raw", seed=6)
            want = oracle_dsts(spec, srcs)
            sflat = [None if s is None else s.contiguous().view(torch.uint8).reshape(-1).numpy() for s in srcs]
            dflat = [np.zeros(b.numel() * b.element_size(), dtype=np.uint8) for b in want]
            run_descriptors(plan, sflat, dflat)
            for a, b in zip(dflat, want):
                assert a.tobytes() == b.view(torch.uint8).reshape(-1).numpy().tobytes(), spec


def test_random_moderate_layouts_descriptor_walk():
    """40 seeded random layout pairs of moderate size: planned pieces and the
    byte-level walk of the descriptor table both equal the oracle."""
    for spec in random_specs(11, 40):
        with Plan([spec]) as plan:
            assert_boxes_agree(plan)
            assert_descriptors_in_bounds(plan)
            _, srcs = sources_for(spec, "raw", seed=5)
            want = oracle_dsts(spec, srcs)
            sflat = [None if s is None else s.contiguous().view(torch.uint8).reshape(-1).numpy() for s in srcs]
            dflat = [np.zeros(b.numel() * b.element_size(), dtype=np.uint8) for b in want]
            run_descriptors(plan, sflat, dflat)
            for a, b in zip(dflat, want):
                assert a.tobytes() == b.view(torch.uint8).reshape(-1).numpy().tobytes(), spec


def assert_in_runs(runs, lo, hi, local):
    """[lo, hi) lies inside one run of every dim, and local is its offset in the
    shard's buffer (the run's position plus the offset inside the run)."""
    for k, (a, b) in enumerate(zip(lo, hi)):
        pos = 0
        for ra, rb in runs[k]:
            if ra <= a and b <= rb:
                assert local[k] == pos + (a - ra), (k, runs[k], a, b, local)
                break
            pos += rb - ra
        else:
            raise AssertionError(f"dim {k}: [{a}, {b}) in no run of {runs[k]}")


def full_workload_plans():
    return [mk() for mk in W.WORKLOADS.values()]


@pytest.mark.parametrize("wl", full_workload_plans(), ids=lambda w: w.name)
def test_invariants_full_size(wl):
    """I1 coverage, I2/I3 byte totals, I4 containment, I5 balance, I6 determinism,
    on the full-size workload plans (no data needed)."""
    with Plan(wl.tensors) as plan:
        st = plan.stats()
        pieces = R.reshard_plan_pieces(plan.handle)
        dst_bytes = 0
        for t, spec in enumerate(wl.tensors):
            es = spec.out_dtype.itemsize
            for sh in plan.dst_shapes(t):
                dst_bytes += int(np.prod(sh)) * es
        # I2, I3: write bytes = destination bytes, read bytes = global bytes (no 2x inflation)
        assert st["global_bytes"] == wl.global_bytes
        # a Partial source is read once per contribution
        assert st["bytes_read"] == sum(int(np.prod(s.shape)) * s.dtype.itemsize * max(1, s.partial)
                                       for s in wl.tensors)
        assert st["bytes_written"] == dst_bytes
        # I4: each piece lies in its source shard and in every destination shard it
        # feeds (inside one run per dim, at the local offset the plan reports);
        # I1: per destination rank, the pieces tile its shard exactly once
        src_runs = [lib_runs(plan.src_layouts[t], s.shape) for t, s in enumerate(wl.tensors)]
        dst_runs = [lib_runs(plan.dst_layouts[t], s.shape) for t, s in enumerate(wl.tensors)]
        covered = {}
        for i, pc in enumerate(pieces):
            t = pc["tensor"]
            nd = len(wl.tensors[t].shape)
            lo, hi = pc["lo"][:nd], pc["hi"][:nd]
            assert_in_runs(src_runs[t][pc["src_rank"]], lo, hi, pc["src_local"][:nd])
            vol = int(np.prod([h - l for l, h in zip(lo, hi)]))
            for d in R.reshard_plan_piece_fanout(plan.handle, i):
                assert_in_runs(dst_runs[t][d], lo, hi, pc["dst_local"][:nd])
                covered[(t, d)] = covered.get((t, d), 0) + vol
        for t, spec in enumerate(wl.tensors):
            for d, sh in enumerate(plan.dst_shapes(t)):
                assert covered.get((t, d), 0) == int(np.prod(sh))
        # I6: the same layouts give a byte-identical table
        with Plan(wl.tensors) as again:
            assert R.reshard_plan_descriptors(plan.handle) == R.reshard_plan_descriptors(again.handle)


def test_pairwise_disjoint_pieces_small():
    """I1 element by element on small layouts: every destination element is
    written by exactly one piece."""
    for spec in small_specs():
        with Plan([spec]) as plan:
            counts = [np.zeros(sh, dtype=np.int32) for sh in plan.dst_shapes(0)]
            nd = len(spec.shape)
            for i, pc in enumerate(R.reshard_plan_pieces(plan.handle)):
                for d in R.reshard_plan_piece_fanout(plan.handle, i):
                    idx = tuple(slice(a, a + h - l) for a, l, h in zip(pc["dst_local"][:nd], pc["lo"][:nd],
                                                                      pc["hi"][:nd]))
                    counts[d][idx] += 1
            for c in counts:
                assert (c == 1).all(), spec.name


def test_worked_example_plan():
    """The pages' example: 8 transfers, each a 4x2 block from source s to
    destination c at rows 4s, columns 2c."""
    with Plan(W.worked_example_8x8().tensors) as plan:
        pieces = R.reshard_plan_pieces(plan.handle)
        assert len(pieces) == 8
        got = sorted((pc["src_rank"], R.reshard_plan_piece_fanout(plan.handle, i)[0],
                      pc["lo"][:2], pc["hi"][:2]) for i, pc in enumerate(pieces))
        want = sorted((s, c, [4 * s, 2 * c], [4 * s + 4, 2 * c + 2]) for s in range(2) for c in range(4))
        assert got == want


def test_piece_counts_of_workloads():
    counts = {"worked_example_8x8": 8, "ffn_up_14336x4096": 8, "moe_experts_64x2048x7168": 128,
              "uneven_5000x3001": 42, "ffn_refit_32_layers": 384, "narrow_columns_4194304x8": 8, "ffn_up_f32_to_bf16_14336x4096": 8,
              "narrow_columns_tp8_2097152x16": 16, "narrow_columns_64b_tp8_1048576x32": 16, "narrow_columns_64b_tp4_1048576x32": 8,
              "narrow_columns_32b_tp4_2097152x16": 8, "narrow_columns_16b_tp8_4194304x8": 16,
              "dense_layer_refit_32_layers": 32 * (7 * 4 + 2 * 1), "ffn_up_fsdp2_tp_14336x4096": 16,
              "ffn_up_partial_14336x4096": 8, "narrow_columns_8b_tp2_8388608x4": 4,
              "narrow_columns_64b_tp16_1048576x32": 32, "narrow_columns_ragged_tp4_2396745x14": 8,
              "narrow_columns_2b_tp16_2097152x16": 32}
    for wl in full_workload_plans():
        with Plan(wl.tensors) as plan:
            assert plan.stats()["n_pieces"] == counts[wl.name]


def test_source_replica_balance():
    """I5: within each set of source replicas, bytes read per replica differ by at
    most the largest piece; here the choice is spread over all replicas."""
    spec = T("rep", (4096, 512), torch.bfloat16, (4, 2), (RR, 0), (8,), (1,))
    with Plan([spec]) as plan:
        loads, largest = {}, 0
        for pc in R.reshard_plan_pieces(plan.handle):
            b = int(np.prod([h - l for l, h in zip(pc["lo"][:2], pc["hi"][:2])])) * 2
            loads.setdefault(pc["src_group"], {}).setdefault(pc["src_rank"], 0)
            loads[pc["src_group"]][pc["src_rank"]] += b
            largest = max(largest, b)
        for group, per_rank in loads.items():
            assert len(per_rank) == 4, per_rank  # all four replicas used
            assert max(per_rank.values()) - min(per_rank.values()) <= largest
        # the same bound read through the C ABI's per-slot load: replicas of one
        # source box are the slots 2 r + c for the four values of r
        load = R.reshard_plan_src_load(plan.handle)
        assert len(load) == 8 and sum(load) == plan.stats()["bytes_read"]
        for c in range(2):
            per = [load[2 * r + c] for r in range(4)]
            assert min(per) > 0 and max(per) - min(per) <= largest, per
            assert per == [loads[c][2 * r + c] for r in range(4)]


def test_source_load_per_slot():
    """reshard_plan_src_load: one entry per source pointer slot of a batched
    plan, summing to bytes_read; slots whose shard is empty, and replicas that
    the choice leaves unread, hold 0."""
    specs = [T("a", (5, 3), torch.float32, (4,), (0,), (2,), (1,)),           # rank 3 of 4 is empty
             T("b", (64, 64), torch.bfloat16, (3, 1), (RR, 0), (2,), (0,)),   # three replicas of one box
             T("c", (64, 64), torch.bfloat16, (2,), (RR,), (4,), (1,))]       # two replicas, four pieces
    with Plan(specs) as plan:
        load = R.reshard_plan_src_load(plan.handle)
        st = plan.stats()
        assert len(load) == st["n_src_ptrs"] == 4 + 3 + 2
        assert sum(load) == st["bytes_read"]
        assert load[3] == 0 and all(x > 0 for x in load[:3])
        assert sum(load[4:7]) == 64 * 64 * 2 and sum(1 for x in load[4:7] if x) == 2  # two pieces, two replicas
        assert load[7] == load[8] == 64 * 64 * 2 // 2
        for i, pc in enumerate(R.reshard_plan_pieces(plan.handle)):
            assert load[[0, 4, 7][pc["tensor"]] + pc["src_rank"]] > 0


def test_replicated_source_bands():
    """A replicated source box is read in row parts, one per replica: every
    band takes each box's rows from one replica, so a narrow band's sources stay
    packed (one segment per box and band) and take the narrow path, and the
    replicas of a box read equal shares to within a row."""
    cases = {"rep_src": [(0, 2), (1, 3)], "rep_src_u8": [(0, 1, 2)],
             "rep_src_bf16_rows": [(0, 3), (1, 4), (2, 5)], "narrow_gather_rep": [(j, 4 + j) for j in range(4)]}
    specs = {s.name: s for s in small_specs()}
    for name, boxes in cases.items():
        spec = specs[name]
        width = spec.shape[-1] * torch.empty((), dtype=spec.dtype).element_size()
        with Plan([spec]) as plan:
            descs, _ = R.reshard_plan_descriptors(plan.handle)
            segs = R.reshard_plan_segments(plan.handle)
            load = R.reshard_plan_src_load(plan.handle)
        bands = [D for D in descs if D["mode"] == R.DESC_WINDOW]
        assert bands, name
        for D in bands:
            src = segs[D["src_ptr"]:D["src_ptr"] + D["dst_ref_begin"]]
            assert len({s["ptr"] for s in src}) == len(src), name  # one replica per box and band
            if width > 16:
                assert is_narrow_band(D, segs), name
        for box in boxes:
            shares = [load[r] for r in box]
            assert max(shares) - min(shares) <= width and min(shares) > 0, (name, shares)


def rank_loss_sequence(rows=448, cols=320):
    """The single-GPU image of a refit whose communication groups are torn down
    and rebuilt when ranks leave: the same weight planned again and again on
    shrinking meshes (training ranks lost: fewer row shards; inference ranks
    lost: fewer data-parallel replicas or tensor-parallel column shards, some
    splits ragged)."""
    layouts = [((4,), (0,), (2, 4), (RR, 1)), ((3,), (0,), (2, 4), (RR, 1)), ((3,), (0,), (2, 3), (RR, 1)),
               ((3,), (0,), (1, 3), (RR, 1)), ((2,), (0,), (3,), (1,)), ((1,), (RR,), (2,), (1,))]
    return [T(f"rank_loss_{i}", (rows, cols), torch.bfloat16, sm, sp, dm, dp)
            for i, (sm, sp, dm, dp) in enumerate(layouts)]


def test_replan_after_rank_loss():
    """Destroy a plan, plan the same tensor again on a smaller mesh, and check
    each new plan against the oracle: the planned pieces applied on the host and
    the descriptor table walked byte by byte."""
    prev = None
    for spec in rank_loss_sequence():
        plan = Plan([spec])
        try:
            assert_boxes_agree(plan)
            _, srcs = sources_for(spec, "raw", seed=5)
            want = oracle_dsts(spec, srcs)
            got = apply_pieces(plan, [srcs])[0]
            for a, b in zip(got, want):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), spec.name
            sflat = [None if x is None else x.contiguous().view(torch.uint8).reshape(-1).numpy() for x in srcs]
            dflat = [np.full(int(np.prod(box_shape(b))) * 2, 0xA5, dtype=np.uint8) for b in plan.dst_boxes(0)]
            run_descriptors(plan, sflat, dflat)
            for a, b in zip(dflat, want):
                assert a.tobytes() == b.view(torch.uint8).numpy().tobytes(), spec.name
            st = plan.stats()
            assert st["bytes_read"] == 448 * 320 * 2
            assert st["bytes_written"] == sum(int(np.prod(box_shape(b))) * 2 for b in plan.dst_boxes(0))
            if prev is not None:
                assert st["n_dst_ptrs"] <= prev["n_dst_ptrs"] and st["n_src_ptrs"] <= prev["n_src_ptrs"]
            prev = st
        finally:
            plan.close()


def test_gather_rows_selection():
    """The uneven fp32 split runs as one gather-rows band per destination shard
    (six source segments each); strips narrower than 1 KiB, and 16-byte aligned
    strips, keep the per-piece descriptors."""
    with Plan(W.uneven().tensors) as plan:
        descs, _ = R.reshard_plan_descriptors(plan.handle)
        segs = R.reshard_plan_segments(plan.handle)
        assert [d["mode"] for d in descs] == [R.DESC_GATHER_ROWS] * 7
        assert [d["extent"][:2] for d in descs] == [[715, 6]] * 6 + [[710, 6]]
        assert all(d["dst_offset"] == 0 and d["run_bytes"] == 3001 * 4 for d in descs)
        assert [s["width"] for s in segs[:6]] == [2004, 2000, 2004, 2000, 2000, 1996]
        assert [s["col"] for s in segs[:6]] == [0, 2004, 4004, 6008, 8008, 10008]
    with Plan(W.uneven(500, 301).tensors) as plan:     # 500-byte strips: chunks
        assert {d["mode"] for d in R.reshard_plan_descriptors(plan.handle)[0]} == {R.DESC_DST_CHUNKS}
    with Plan(W.uneven(5000, 3072).tensors) as plan:   # 16-byte aligned strips: items
        assert {d["mode"] for d in R.reshard_plan_descriptors(plan.handle)[0]} == {R.DESC_ITEMS}
    spec = {s.name: s for s in small_specs()}["gather_row_cuts"]
    with Plan([spec]) as plan:                         # bands cut where source row boxes end
        descs, _ = R.reshard_plan_descriptors(plan.handle)
        assert {d["mode"] for d in descs} == {R.DESC_GATHER_ROWS} and len(descs) == 6
        assert any(d["dst_offset"] > 0 for d in descs)


def test_gather_rows_long_band_is_split():
    """Bands longer than the kernel's 31-bit byte index are split by rows; the
    pieces still cover every row once (checked on the descriptors, no data)."""
    spec = T("long", (600000, 4099), torch.float32, (2,), (1,), (3,), (0,))
    with Plan([spec]) as plan:
        descs, _ = R.reshard_plan_descriptors(plan.handle)
        segs = R.reshard_plan_segments(plan.handle)
        assert {d["mode"] for d in descs} == {R.DESC_GATHER_ROWS}
        W_ = 4099 * 4
        for dst in range(3):
            mine = sorted((d["dst_offset"], d["extent"][0]) for d in descs
                          if R.reshard_plan_descriptors(plan.handle)[1][d["dst_ref_begin"]] == dst)
            at = 0
            for off, rows in mine:
                assert off == at * W_ and rows * W_ < 2 ** 31
                at += rows
            assert at == 200000
        for d in descs:
            first = d["src_ptr"]
            rows = d["extent"][0]
            for sg in segs[first:first + d["extent"][1]]:
                assert sg["offset"] % sg["row_stride"] == 0  # starts at a row of the source strip


def test_dim_merging():
    """Contiguous dims merge into one run; strided dims stay outer dims."""
    with Plan(W.ffn_refit(1, 4096, 14336).tensors) as plan:
        descs, _ = R.reshard_plan_descriptors(plan.handle)
        gate = descs[0]  # gate piece: rows of a row split -> one contiguous run
        assert gate["extent"] == [1, 1, 1] and gate["unit"] == 16
        assert gate["run_bytes"] == 3584 * 4096 * 2 and gate["mode"] == R.DESC_ITEMS
        down = [d for d in descs if d["run_bytes"] == 3584 * 2]
        assert down and all(d["extent"][2] == 4096 for d in down)
    with Plan(W.moe_experts().tensors) as plan:
        d = R.reshard_plan_descriptors(plan.handle)[0][0]
        assert d["extent"][1:] == [8, 1024] and d["run_bytes"] == 1792 and d["unit"] == 16


def test_big_tensor_is_split_within_31_bit_items():
    """A plan whose pieces exceed 2^31 items is split; the descriptors of each
    piece still cover it exactly (checked analytically, no data)."""
    n = (1 << 33) + 6  # bytes of a 1-d uint8 tensor
    spec = T("big", (n,), torch.uint8, (3,), (0,), (2,), (0,))
    with Plan([spec]) as plan:
        descs, _ = R.reshard_plan_descriptors(plan.handle)
        pieces = R.reshard_plan_pieces(plan.handle)
        assert len(descs) > len(pieces)
        for d in descs:
            items = d["extent"][0] * d["extent"][1] * d["extent"][2] * d["row_items"]
            assert items < 2 ** 31 and d["run_bytes"] <= 2 ** 30
        for i, pc in enumerate(pieces):
            mine = sorted((d["src_offset"], d["run_bytes"]) for d in descs if d["piece"] == i)
            size = pc["hi"][0] - pc["lo"][0]
            pos = mine[0][0]
            for off, length in mine:
                assert off == pos
                pos += length
            assert pos - mine[0][0] == size


def test_magic_constants_exact():
    rng = random.Random(5)
    with Plan(small_specs()) as plan:
        descs, _ = R.reshard_plan_descriptors(plan.handle)
    divisors = {}
    for d in descs:
        if d["mode"] == R.DESC_WINDOW:  # windows divide nothing
            continue
        if d["mode"] == R.DESC_GATHER_ROWS:  # gather-rows bands divide by the row width only
            divisors[d["run_bytes"]] = tuple(d["magic"][0])
            continue
        divisors[d["row_items"]] = tuple(d["magic"][0])
        divisors[d["extent"][2]] = tuple(d["magic"][1])
        divisors[d["extent"][1]] = tuple(d["magic"][2])
    assert len(divisors) > 5
    for dv, (m, s) in divisors.items():
        ns = [0, 1, dv - 1, dv, dv + 1, 2 ** 31 - 1, 2 ** 31 - 2] + [rng.randrange(2 ** 31) for _ in range(2000)]
        for n in ns:
            assert magic_div(n, m, s) == n // dv, (dv, n)


def test_descriptor_modes():
    """16-byte aligned rows copy as 16-byte items; whole destination rows from
    misaligned source strips of at least 1 KiB as gather-rows bands; other long
    misaligned rows as destination-aligned 16-byte chunks; short misaligned rows
    item by item;
    narrow rows of a 2-d view through windows, unless the rows are wider than a
    window."""
    def modes(specs):
        with Plan(specs) as plan:
            return {(d["mode"], d["unit"]) for d in R.reshard_plan_descriptors(plan.handle)[0]}
    small = {s.name: s for s in small_specs()}
    assert modes(W.ffn_up().tensors) == {(R.DESC_ITEMS, 16)}
    assert modes(W.uneven().tensors) == {(R.DESC_GATHER_ROWS, 4)}      # 12004-byte rows of ~2000-byte strips
    assert modes(W.uneven(500, 301).tensors) == {(R.DESC_DST_CHUNKS, 4)}  # strips narrower than 1 KiB
    assert {m for m, _ in modes(W.worked_example_8x8().tensors)} == {R.DESC_WINDOW}  # 4-byte rows
    for name in ("strips_row_cuts", "strips_fanout", "strips_rep_src", "strips_nine", "strips_mid_split"):
        assert modes([small[name]]) == {(R.DESC_DST_CHUNKS, 4 if small[name].dtype == torch.float32 else 2)}, name
    # a 4-byte piece in 16804-byte rows: too wide for a window, so per piece
    assert {m for m, _ in modes([small["narrow_wide_rows"]])} == {R.DESC_DST_CHUNKS, R.DESC_ITEMS}


def test_narrow_band_window_per_band():
    """Narrow bands take twice the rows per tile (a window of up to 36 KiB)
    when a destination segment would get less than 1 KiB a tile or is one or
    two bytes wide, or a tile fewer than 64 rows, and keep the usual rows
    otherwise; every band but the row-mode one stays a narrow band."""
    cases = [
        (T("u8_16", (4099, 16), torch.uint8, (2,), (0,), (16,), (1,)), 1024),     # 1-byte columns, 512 -> 1024
        (T("bf16_64", (1031, 32), torch.bfloat16, (2,), (0,), (32,), (1,)), 512),  # 2-byte columns, 256 -> 512
        (T("rows512", (301, 256), torch.bfloat16, (2,), (0,), (8,), (1,)), 64),   # 32-row tiles -> 64
        (T("bf16_32", (2053, 16), torch.bfloat16, (2,), (0,), (16,), (1,)), 1024),  # 1 KiB of a 2-byte column: 512 -> 1024
        (T("bf16_24", (2053, 12), torch.bfloat16, (2,), (0,), (12,), (1,)), 1024),
        (T("u8_8", (4099, 8), torch.uint8, (2,), (0,), (8,), (1,)), 2048),        # 1 KiB of a 1-byte column: 1024 -> 2048
        (T("bf16_8", (4099, 4), torch.bfloat16, (2,), (0,), (4,), (1,)), 2048),   # 2 KiB of a 2-byte column: 1024 -> 2048
        (T("f32_8", (4099, 2), torch.float32, (2,), (0,), (2,), (1,)), 1024),     # 4-byte columns of 8-byte rows: row mode
        (W.narrow_columns_64b_tp16(2048).tensors[0], 256),                         # 4-byte columns, 1 KiB pieces
        (W.narrow_columns_tp8(4096).tensors[0], 512),
    ]
    for spec, rows in cases:
        with Plan([spec]) as plan:
            descs, _ = R.reshard_plan_descriptors(plan.handle)
            segs = R.reshard_plan_segments(plan.handle)
        assert {d["extent"][1] for d in descs} == {rows}, spec.name
        assert all(is_narrow_band(d, segs) == (spec.name != "f32_8") for d in descs), spec.name
        assert all(d["extent"][1] * narrow_pitch(d["run_bytes"]) <= 36864 for d in descs), spec.name


def test_row_mode_tile_rows():
    """Row-mode bands (at most 16 bytes wide) take 1024 rows per tile, or 512 when
    one side is four packed 4-byte column runs (quad exchange); wider bands as
    many rows as fit a 16 KiB LDS window (512 for the 32-byte bands of eight
    4-byte runs that the 8-lane exchange moves)."""
    small = {s.name: s for s in small_specs()}
    want = {"narrow_scatter": 512, "narrow_gather": 512, "narrow_f32_cols": 512, "narrow_scatter_rep": 512,
            "narrow_gather_rep": 512, "narrow_bf16_cols": 512, "narrow_8byte_rows": 1024,
            "narrow_fp8_3d": 16384 // 32, "runs_scatter": 512, "runs_gather": 512, "runs_scatter_rep": 512,
            "runs_f32_cols": 512, "runs64_scatter": 256, "runs64_gather": 256, "runs64_scatter_rep": 256,
            "bands16_scatter": 256, "bands16_gather": 128, "bands16_rep": 128, "bands16_256": 64,
            "runs32_scatter": 512, "runs32_gather": 512, "runs32_scatter_rep": 512,
            "octets_gather": 512, "octets_scatter_rep": 512, "thin32_gather": 512, "thin32_gather_rep": 512,
            "bytes_r2_in32": 1024, "bytes_r2_rep": 1024, "bands16_96": 170, "bands16_48_gather": 341,
            "bands16_80_rep": 204}
    for name, rows in want.items():
        with Plan([small[name]]) as plan:
            descs, _ = R.reshard_plan_descriptors(plan.handle)
        assert {d["mode"] for d in descs} == {R.DESC_WINDOW}, name
        assert {d["extent"][1] for d in descs} == {rows}, name


@pytest.mark.parametrize("name", ["w", "up_proj", "layer0.down", "rep_src", "rep_both", "empty_src", "nested",
                                  "narrow_scatter", "narrow_gather", "narrow_scatter_rep", "narrow_gather_rep",
                                  "narrow_f32_cols", "narrow_bf16_cols", "narrow_8byte_rows", "narrow_fp8_3d",
                                  "runs_scatter", "runs_gather", "runs_scatter_rep", "runs_f32_cols",
                                  "runs64_scatter", "runs64_gather", "runs64_scatter_rep"])
def test_window_segments_in_column_order(name):
    """Every window band lists its source segments, and its destination segments,
    by column and without overlap, covering the band's full width on each side
    (the register paths take lane j's 4-byte run to be segment j)."""
    spec = {s.name: s for s in small_specs()}[name]
    with Plan([spec]) as plan:
        descs, _ = R.reshard_plan_descriptors(plan.handle)
        segs = R.reshard_plan_segments(plan.handle)
        windows = [D for D in descs if D["mode"] == R.DESC_WINDOW]
        assert windows, name
        for D in windows:
            first = D["src_ptr"]
            for side in (segs[first:first + D["dst_ref_begin"]],
                         segs[first + D["dst_ref_begin"]:first + D["dst_ref_begin"] + D["fanout"]]):
                cols = [(sg["col"], sg["col"] + sg["width"]) for sg in side]
                assert cols == sorted(cols), (name, cols)
                assert cols[0][0] == 0 and cols[-1][1] == D["run_bytes"], (name, cols)
                assert all(a[1] == b[0] for a, b in zip(cols, cols[1:])), (name, cols)


def test_window_segments_worked_example():
    """The pages' example as one window band per source shard: one source segment
    (the whole 16-byte rows, merged across the four pieces) and four destination
    segments of 4-byte rows."""
    with Plan(W.worked_example_8x8().tensors) as plan:
        descs, _ = R.reshard_plan_descriptors(plan.handle)
        segs = R.reshard_plan_segments(plan.handle)
        assert [d["mode"] for d in descs] == [R.DESC_WINDOW, R.DESC_WINDOW]
        for d in descs:
            assert d["extent"][0] == 4 and d["run_bytes"] == 16
            assert d["dst_ref_begin"] == 1 and d["fanout"] == 4
            src = segs[d["src_ptr"]]
            assert src["width"] == 16 and src["row_stride"] == 16
            dsts = segs[d["src_ptr"] + 1:d["src_ptr"] + 5]
            assert [x["col"] for x in dsts] == [0, 4, 8, 12] and all(x["width"] == 4 for x in dsts)


def test_outer_dims_beyond_three_are_peeled():
    spec = [s for s in small_specs() if s.name == "peel_outer"][0]
    with Plan([spec]) as plan:
        st = plan.stats()
        assert st["n_descriptors"] > st["n_pieces"]


@pytest.mark.parametrize("wl", full_workload_plans(), ids=lambda w: w.name)
def test_descriptors_in_bounds_full_size(wl):
    with Plan(wl.tensors) as plan:
        assert_descriptors_in_bounds(plan)


def test_descriptors_in_bounds_small():
    for spec in small_specs():
        with Plan([spec]) as plan:
            assert_descriptors_in_bounds(plan)


def test_errors():
    with pytest.raises(R.ReshardError) as e:
        R.reshard_layout_create((4, 4), R.DTYPE_F32, (2,), (2,))  # no dim 2
    assert e.value.status == R.ERR_INVALID_ARGUMENT
    with pytest.raises(R.ReshardError):
        R.reshard_layout_create((4, 4), R.DTYPE_F32, (0,), (0,))  # empty mesh dim
    with pytest.raises(R.ReshardError):
        R.reshard_layout_create((4, -1), R.DTYPE_F32, (2,), (0,))
    with pytest.raises(R.ReshardError):
        R.reshard_layout_create((4,), 99, (2,), (0,))  # unknown dtype
    with pytest.raises(R.ReshardError):
        R.reshard_layout_create(tuple([2] * 9), R.DTYPE_F32, (2,), (0,))  # ndim 9
    a = R.reshard_layout_create((4, 4), R.DTYPE_F32, (2,), (0,))
    b = R.reshard_layout_create((4, 5), R.DTYPE_F32, (2,), (0,))
    c = R.reshard_layout_create((4, 4), R.DTYPE_I32, (2,), (0,))     # same size, no conversion
    c2 = R.reshard_layout_create((4, 4), R.DTYPE_F64, (2,), (0,))    # no f32 -> f64 conversion
    bf = R.reshard_layout_create((4, 4), R.DTYPE_BF16, (2,), (0,))
    hf = R.reshard_layout_create((4, 4), R.DTYPE_F16, (2,), (0,))
    for other in (b, c, c2):
        with pytest.raises(R.ReshardError) as e:
            R.reshard_plan_create(a, other)
        assert e.value.status == R.ERR_LAYOUT_MISMATCH
    with pytest.raises(R.ReshardError) as e:
        R.reshard_plan_create(bf, hf)  # bf16 -> f16 is not a supported conversion
    assert e.value.status == R.ERR_LAYOUT_MISMATCH
    for x, y in ((a, bf), (a, hf), (bf, a), (hf, a)):  # the supported conversions plan
        R.reshard_plan_destroy(R.reshard_plan_create(x, y))
    for h in (c2, bf, hf):
        R.reshard_layout_destroy(h)
    with pytest.raises(R.ReshardError):
        R.reshard_layout_shard_box(a, 2, 2)  # rank out of range
    plan = R.reshard_plan_create(a, a)
    # a NULL pointer for a non-empty shard is refused before anything is launched
    with pytest.raises(R.ReshardError) as e:
        R.reshard_execute(plan, [0x1000, 0], [0x2000, 0x3000])
    assert e.value.status == R.ERR_NULL_SHARD
    assert "src_ptrs[1]" in R.reshard_last_error()
    R.reshard_plan_destroy(plan)
    for h in (a, b, c):
        R.reshard_layout_destroy(h)
    R.reshard_plan_destroy(None)
    R.reshard_layout_destroy(None)


def test_device_segments_of_narrow_bands():
    """The device table's segments equal the planned ones, except that each
    destination segment of a narrow band carries its first replica's absolute
    pointer slot in row_stride (all of a band's segments, or none)."""
    specs = [W.narrow_columns_64b_tp16(4096).tensors[0], W.narrow_columns_ragged_tp4(3001).tensors[0],
             W.narrow_columns(2048).tensors[0], W.uneven(301, 257).tensors[0],
             W.narrow_columns_2b_tp16(4096).tensors[0]]
    specs += [s for s in small_specs() if s.name in ("wide_window", "narrow_scatter_rep", "strips_fanout",
                                                     "bytes_r2_rep", "thin_u8_16")]
    rewritten_bands = 0
    for spec in specs:
        with Plan([spec]) as plan:
            st = plan.stats()
            host = R.reshard_plan_segments(plan.handle)
            dev = R.reshard_plan_device_segments(plan.handle)
            _, refs = R.reshard_plan_descriptors(plan.handle)
            descs, _ = R.reshard_plan_descriptors(plan.handle)
            assert len(host) == len(dev)
            for D in descs:
                if D["mode"] != R.DESC_WINDOW:
                    continue
                first = D["src_ptr"]
                for k in range(D["dst_ref_begin"]):  # sources: unchanged
                    assert dev[first + k] == host[first + k]
                dst = range(first + D["dst_ref_begin"], first + D["dst_ref_begin"] + D["fanout"])
                if is_narrow_band(D, host):
                    rewritten_bands += 1
                    for i in dst:
                        h, d = host[i], dev[i]
                        assert h["row_stride"] == h["width"]
                        assert d["row_stride"] == st["n_src_ptrs"] + refs[h["ptr"]]
                        assert {k: v for k, v in d.items() if k != "row_stride"} == \
                            {k: v for k, v in h.items() if k != "row_stride"}
                else:
                    assert all(dev[i] == host[i] for i in dst)
    assert rewritten_bands >= 6


def test_partial_errors():
    """Partial only on a source, only for float elements, never with split factors."""
    src = R.reshard_layout_create((8, 4), R.DTYPE_F32, (2, 2), (R.PARTIAL, 0))
    dst = R.reshard_layout_create((8, 4), R.DTYPE_F32, (2,), (1,))
    isrc = R.reshard_layout_create((8, 4), R.DTYPE_I32, (2, 2), (R.PARTIAL, 0))
    idst = R.reshard_layout_create((8, 4), R.DTYPE_I32, (2,), (1,))
    sdst = R.reshard_layout_create_strided((8, 4), R.DTYPE_F32, (2,), (0,), (2,))
    try:
        for a, b in ((dst, src), (isrc, idst), (src, sdst)):
            with pytest.raises(R.ReshardError) as e:
                R.reshard_plan_create(a, b)
            assert e.value.status == R.ERR_LAYOUT_MISMATCH
        with pytest.raises(R.ReshardError) as e:  # no split factor on a Partial dim
            R.reshard_layout_create_strided((8, 4), R.DTYPE_F32, (2,), (R.PARTIAL,), (2,))
        assert e.value.status == R.ERR_INVALID_ARGUMENT
        plan = R.reshard_plan_create(src, dst)
        st = R.reshard_plan_stats(plan)
        assert st["bytes_read"] == 2 * 8 * 4 * 4 and st["bytes_written"] == 8 * 4 * 4
        descs, refs = R.reshard_plan_descriptors(plan)
        assert all(D["mode"] == R.DESC_REDUCE and D["unit"] & 0xFFF == 2 for D in descs)
        assert R.reshard_plan_piece_sources(plan, 0) == [0, 2]  # contribution 0, then 1
        R.reshard_plan_destroy(plan)
    finally:
        for h in (src, dst, isrc, idst, sdst):
            R.reshard_layout_destroy(h)


def test_dtype_sizes():
    sizes = {R.DTYPE_U8: 1, R.DTYPE_FP8_E4M3: 1, R.DTYPE_BF16: 2, R.DTYPE_F16: 2, R.DTYPE_F32: 4,
             R.DTYPE_I32: 4, R.DTYPE_F64: 8, R.DTYPE_I64: 8}
    for code, size in sizes.items():
        assert R.reshard_dtype_size(code) == size
    assert R.reshard_dtype_size(42) == 0


def test_library_exports_every_declared_symbol():
    declared = set(re.findall(r"\b(reshard_\w+)\s*\(", open(HEADER).read()))
    declared -= {"reshard_status", "reshard_dtype"}
    assert declared == set(R.reshard.EXPORTED)
    lib = ctypes.CDLL(R.library_path())
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", R.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (reshard_\w+)$", out, flags=re.M))
    assert declared <= exported


def test_plan_stats_fields():
    with Plan(W.ffn_up().tensors) as plan:
        st = plan.stats()
        assert st["n_src_ptrs"] == 4 and st["n_dst_ptrs"] == 4
        assert st["n_dst_writes"] == 16 and st["n_descriptors"] == 8
        assert st["n_workgroups"] == 0 and st["n_launches"] == 0  # not uploaded: no device touched
        assert st["plan_host_us"] > 0


def test_plans_from_many_threads():
    """Planning is host-only and re-entrant: plans built concurrently from
    several threads equal the one built alone."""
    import threading
    wl = W.dense_layer_refit(4, 256, 64, 512)
    with Plan(wl.tensors) as ref_plan:
        ref = R.reshard_plan_descriptors(ref_plan.handle)
    results, errors = [], []

    def work():
        try:
            for _ in range(5):
                with Plan(wl.tensors) as p:
                    results.append(R.reshard_plan_descriptors(p.handle))
        except Exception as e:  # noqa: BLE001
            errors.append(e)
    threads = [threading.Thread(target=work) for _ in range(6)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors and len(results) == 30
    assert all(r == ref for r in results)


def test_device_calls_fail_cleanly_without_a_gpu():
    """With no visible GPU, upload and execute return RESHARD_ERR_HIP (no crash);
    planning and inspection keep working."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with Plan(W.ffn_up(64, 32).tensors) as plan:
        with pytest.raises(R.ReshardError) as e:
            R.reshard_plan_upload(plan.handle, None)
        assert e.value.status == R.ERR_HIP
        with pytest.raises(R.ReshardError) as e:
            R.reshard_execute(plan.handle, [0x1000] * 4, [0x2000] * 4, None)
        assert e.value.status == R.ERR_HIP
        with pytest.raises(R.ReshardError) as e:
            R.reshard_execute_noalloc(plan.handle, [0x1000] * 4, [0x2000] * 4, None)
        assert e.value.status == R.ERR_HIP
        with pytest.raises(R.ReshardError) as e:  # argument checks come before any device call
            R.reshard_execute_noalloc(plan.handle, [0x1000, 0, 0x1000, 0x1000], [0x2000] * 4, None)
        assert e.value.status == R.ERR_NULL_SHARD
        assert plan.stats()["n_pieces"] == 8


@pytest.mark.parametrize("wl", full_workload_plans() + [W.dense_layer_refit(2, 256, 64, 512)],
                         ids=lambda w: w.name)
def test_two_stage_layout_slices_tile_each_box(wl):
    """Stage 1 of the two-stage transport gives every destination replica one
    slice of its box; the slices of a box's replicas tile it exactly (checked
    with the oracle's box function)."""
    import oracle
    from dtensor_layout_movement_amd.two_stage import stage1_layout
    for spec in wl.tensors[:9]:
        mesh1, pl1, _ = stage1_layout(spec.dst_mesh, spec.dst_placements)
        n1 = int(np.prod(mesh1))
        # stage-1 rank r1 has the coordinates of the destination rank that owns its
        # slice, listed in stage-1 mesh order (non-Replicate dims, then Replicate)
        order = [i for i, p in enumerate(spec.dst_placements) if p != R.REPLICATE] + \
                [i for i, p in enumerate(spec.dst_placements) if p == R.REPLICATE]
        rank_map = []
        for r1 in range(n1):
            c1 = np.unravel_index(r1, mesh1)
            cd = [0] * len(spec.dst_mesh)
            for j, i in enumerate(order):
                cd[i] = int(c1[j])
            rank_map.append(int(np.ravel_multi_index(cd, spec.dst_mesh)))
        covered = {}
        for r1 in range(n1):
            lo, hi = oracle.shard_box(list(spec.shape), list(mesh1), list(pl1), r1)
            dlo, dhi = oracle.shard_box(list(spec.shape), list(spec.dst_mesh), list(spec.dst_placements),
                                        rank_map[r1])
            assert all(a <= l and h <= b for l, h, a, b in zip(lo, hi, dlo, dhi) if h > l)
            vol = int(np.prod([max(0, h - l) for l, h in zip(lo, hi)]))
            key = (tuple(dlo), tuple(dhi))
            covered[key] = covered.get(key, 0) + vol
        for (dlo, dhi), vol in covered.items():
            assert vol == int(np.prod([max(0, h - l) for l, h in zip(dlo, dhi)]))
        assert sorted(rank_map) == list(range(int(np.prod(spec.dst_mesh))))


def test_two_stage_strided_destination_slices_tile_each_shard():
    """With split factors on the destination, the stage-1 layout keeps them on
    its non-Replicate mesh dims: every stage-1 slice lies in the shard of the
    destination rank that owns it, and a shard's replica slices tile it (index
    sets from the oracle)."""
    import itertools
    import oracle
    from dtensor_layout_movement_amd.two_stage import stage1_layout
    for spec in strided_specs():
        if spec.dst_split is None:
            continue
        mesh1, pl1, sp1 = stage1_layout(spec.dst_mesh, spec.dst_placements, spec.dst_split)
        order = [i for i, p in enumerate(spec.dst_placements) if p != R.REPLICATE] + \
                [i for i, p in enumerate(spec.dst_placements) if p == R.REPLICATE]
        owned = {}
        for r1 in range(int(np.prod(mesh1))):
            c1 = np.unravel_index(r1, mesh1)
            cd = [0] * len(spec.dst_mesh)
            for j, i in enumerate(order):
                cd[i] = int(c1[j])
            d = int(np.ravel_multi_index(cd, spec.dst_mesh))
            mid = oracle.shard_indices(list(spec.shape), list(mesh1), list(pl1), list(sp1), r1)
            dst = oracle.shard_indices(list(spec.shape), list(spec.dst_mesh), list(spec.dst_placements),
                                       list(spec.dst_split), d)
            cells = set(itertools.product(*mid))
            assert cells <= set(itertools.product(*dst)), spec.name
            key = tuple(tuple(x) for x in dst)
            assert not (owned.get(key, set()) & cells), spec.name  # slices of one shard are disjoint
            owned[key] = owned.get(key, set()) | cells
        for key, cells in owned.items():
            assert cells == set(itertools.product(*key)), spec.name


def test_hybrid_routing_bytes():
    """Hybrid refit: FFN projections by the reshard (G(1+R) bytes each), the
    rest by gather-then-slice (source reads + one full write, then a full read
    per destination box plus every destination write)."""
    from dtensor_layout_movement_amd.hybrid import HybridPlan
    wl = W.dense_layer_refit(2, 256, 64, 512)
    hp = HybridPlan(wl.tensors)
    try:
        names = [wl.tensors[t].name.split(".")[1] for t in hp.direct]
        assert sorted(set(names)) == ["down", "gate", "up"] and len(hp.direct) == 6
        assert len(hp.gather) == 12
        want = 0
        for t, spec in enumerate(wl.tensors):
            g = int(np.prod(spec.shape)) * 2
            if t in hp.direct:
                want += g * (1 + 2)                # read once, written to both replicas
            else:
                unique = 1 if len(spec.shape) == 1 else 4
                r = 8 // unique
                want += 2 * g + g + g * r          # gather: read + write G; slice: read G, write G*R
        assert hp.bytes_moved() == want
        ffn = sum(int(np.prod(wl.tensors[t].shape)) for t in hp.direct)
        allb = sum(int(np.prod(s.shape)) for s in wl.tensors)
        assert abs(hp.reshard_share() - ffn / allb) < 1e-12
    finally:
        hp.close()
