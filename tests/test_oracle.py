"""The CPU oracle against its pins (CPU only), and proof that the pins catch
plausible mistakes: each mutant below plants one mistake in a copy of
oracle.cpp, and at least one pin must fail against it."""
import os
import subprocess
import sys

import pytest
import torch

import oracle
import oracle_pins as P
from dtensor_layout_movement_amd import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_pin_worked_example(oracle_lib):
    P.pin_worked_example(oracle_lib)


def test_pin_box_vs_dtensor(oracle_lib):
    P.pin_box_vs_dtensor(oracle_lib)


def test_pin_box_vs_chunk(oracle_lib):
    P.pin_box_vs_chunk(oracle_lib)


def test_pin_end_to_end_chunk(oracle_lib):
    P.pin_end_to_end_chunk(oracle_lib)


def test_pin_gather_and_checks(oracle_lib):
    P.pin_gather(oracle_lib)


def test_pin_raw_bits(oracle_lib):
    P.pin_raw_bits(oracle_lib)


def test_pin_convert_library(oracle_lib):
    P.pin_convert_library(oracle_lib)


def test_pin_convert_nan_payloads(oracle_lib):
    P.pin_convert_nan_payloads(oracle_lib)


def test_pin_convert_closed(oracle_lib):
    P.pin_convert_closed(oracle_lib)


def test_pin_strided_vs_dtensor(oracle_lib):
    P.pin_strided_vs_dtensor(oracle_lib)


def test_pin_strided_closed(oracle_lib):
    P.pin_strided_closed(oracle_lib)


def test_pin_end_to_end_strided(oracle_lib):
    P.pin_end_to_end_strided(oracle_lib)


def test_pin_partial_vs_numpy(oracle_lib):
    P.pin_partial_vs_numpy(oracle_lib)


def test_pin_partial_closed(oracle_lib):
    P.pin_partial_closed(oracle_lib)


def test_partial_threads_give_same_bytes(oracle_lib):
    g = torch.Generator().manual_seed(9)
    contribs = [torch.randn(64, 48, generator=g).to(torch.bfloat16) for _ in range(4)]
    a = P.run_partial(oracle_lib, (64, 48), "bf16", "bf16", (2, 2, 2), (0, oracle.PARTIAL, oracle.PARTIAL), (3,),
                      (1,), contribs, threads=1)
    b = P.run_partial(oracle_lib, (64, 48), "bf16", "bf16", (2, 2, 2), (0, oracle.PARTIAL, oracle.PARTIAL), (3,),
                      (1,), contribs, threads=8)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_indexed_threads_give_same_bytes(oracle_lib):
    shape, smesh, spl, ssp = (96, 40), (2, 4), (0, 0), (4, 1)
    g = torch.randn(shape)
    srcs = [g.reshape(-1)[P.dtensor_split_local(shape, smesh, spl, ssp, s)].contiguous() for s in range(8)]
    outs = []
    for threads in (1, 8):
        dsts = [torch.empty(48, 40), torch.empty(48, 40)]
        oracle.reshard_indexed(list(shape), 4, list(smesh), list(spl), list(ssp), srcs, [2], [0], [1], dsts,
                               threads=threads, lib=oracle_lib)
        outs.append(dsts)
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    assert torch.equal(torch.cat(outs[0]), g)


def test_convert_threads_and_errors(oracle_lib):
    x = torch.randn(100_003, dtype=torch.float32)
    a = oracle.convert(x, "f32", "bf16", threads=1, lib=oracle_lib)
    b = oracle.convert(x, "f32", "bf16", threads=8, lib=oracle_lib)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert oracle_lib.oracle_convert(0, 3, None, None, 0, 1) == oracle.BAD_LAYOUT
    assert oracle.convert(torch.empty(0), "f32", "f16", lib=oracle_lib).numel() == 0


def test_nested_split_reading(oracle_lib):
    # Nested Shard on one dim splits the interval left by the outer mesh dim
    # (DTensor's rule), which differs from a flat 6-way split at rank (0, 1).
    shape, mesh, pl = (5000, 3001), (3, 2), (1, 1)
    cols = [oracle.shard_box(shape, mesh, pl, r, lib=oracle_lib) for r in range(6)]
    assert [(lo[1], hi[1]) for lo, hi in cols] == [
        (0, 501), (501, 1001), (1001, 1502), (1502, 2002), (2002, 2502), (2502, 3001)]


def test_threads_give_same_bytes(oracle_lib):
    spec = W.moe_experts(16, 64, 448).tensors[0]
    g = W.make_global(spec, "normal", seed=1)
    one, _ = P.run_oracle(oracle_lib, spec, g, threads=1)
    many, _ = P.run_oracle(oracle_lib, spec, g, threads=8)
    for a, b in zip(one, many):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("spec_fn", [W.ffn_up, W.uneven])
def test_full_size_slices(oracle_lib, spec_fn):
    """Full-size configs: every destination shard equals the generated global
    sliced by PyTorch DTensor's boxes (no oracle arithmetic on that side)."""
    wl = spec_fn()
    spec = wl.tensors[0]
    g = W.make_global(spec, wl.values, seed=0)
    dsts, _ = P.run_oracle(oracle_lib, spec, g, threads=4)
    for d, got in enumerate(dsts):
        off, ext = P.dtensor_box(spec.shape, spec.dst_mesh, spec.dst_placements, d)
        idx = tuple(slice(o, o + e) for o, e in zip(off, ext))
        assert torch.equal(got.view(torch.uint8), g[idx].contiguous().view(torch.uint8))


# Each mutant plants one plausible mistake in the oracle's source.
MUTANTS = {
    "floor_split": ("int64_t chunk = (n + L.mesh[m] - 1) / L.mesh[m];",
                    "int64_t chunk = n / L.mesh[m] + (n % L.mesh[m] != 0 && coord[m] == 0);"),
    "column_major_mesh": ("for (int m = L.mesh_ndim - 1; m >= 0; --m) {  // row-major mesh order",
                          "for (int m = 0; m < L.mesh_ndim; ++m) {"),
    "flat_nesting": ("int64_t a = lo[p] + coord[m] * chunk;", "int64_t a = coord[m] * chunk;"),
    "stride_from_box": ("    stride *= shape[k];", "    stride *= ext[k];"),
    "dropped_column_offset": ("  off += lo[ndim - 1];", "  off += 0;"),
    "swapped_row_index": ("    int64_t i = row % ext[k];\n    row /= ext[k];",
                          "    int64_t i = row / ext[k] % ext[k];\n    row %= ext[k];"),
    "short_run": ("std::memcpy(shard + (size_t)(row * run) * es, X + (size_t)g * es, (size_t)run * es);",
                  "std::memcpy(shard + (size_t)(row * run) * es, X + (size_t)g * es, (size_t)(run - (run > 1)) * es);"),
    "coverage_all_dims": ("if (S.placements[m] == kReplicate) r_src *= S.mesh[m];",
                          "r_src *= S.mesh[m];"),
    "no_replica_compare": ("} else if (std::memcmp(to + j * es, from + j * es, es) != 0) {",
                           "} else if (false) {"),
    "replicate_splits": ("if (p == kReplicate) continue;\n    int64_t n",
                         "if (p == kReplicate) p = 0;\n    int64_t n"),
    # float conversion
    "round_toward_zero": ("if (d > 0.5 || (d == 0.5 && std::fmod(r, 2.0) != 0)) r += 1;", "if (false) r += 1;"),
    "ties_away_from_zero": ("(d == 0.5 && std::fmod(r, 2.0) != 0)", "(d == 0.5)"),
    "no_subnormal_spacing": ("  if (E < 1 - f.bias) E = 1 - f.bias;   // subnormal range: fixed spacing", "  (void)0;"),
    "no_overflow_to_inf": ("  if (y > max_finite(f)) y = INFINITY;", "  (void)0;"),
    "f16_bias_16": ("    {16, 10, 15},   // 2: IEEE binary16", "    {16, 10, 16},   // 2: IEEE binary16"),
    "nan_not_quiet": ("    m |= 1u << (to.frac - 1);  // quiet", "    m |= 0;"),
    "nan_payload_dropped": ("    m |= 1u << (to.frac - 1);  // quiet", "    m = 1u << (to.frac - 1);"),
    "nan_payload_low_bits": ("m = to.frac >= from.frac ? m << (to.frac - from.frac) : m >> (from.frac - to.frac);",
                             "m = to.frac >= from.frac ? m << (to.frac - from.frac) : m & ((1u << to.frac) - 1);"),
    "nan_sign_dropped": ("return (sign << (to.bits - 1)) | (exp_all_ones(to) << to.frac) | m;",
                         "return (exp_all_ones(to) << to.frac) | m;"),
    # strided nesting and the indexed gather-then-slice
    "strided_factor_ignored": ("    const int64_t f = split[m];", "    const int64_t f = 1;"),
    "strided_pieces_reversed": ("    for (int64_t j = 0; j < f; ++j) {\n      const int64_t start = j * piece;",
                                "    for (int64_t jj = 0; jj < f; ++jj) {\n      const int64_t j = f - 1 - jj;\n"
                                "      const int64_t start = j * piece;"),
    "strided_parts_floor": ("const int64_t part = (len + L.mesh[m] - 1) / L.mesh[m];",
                            "const int64_t part = len / L.mesh[m] > 0 ? len / L.mesh[m] : 1;"),
    "strided_flat_nesting": ("        kept.push_back(cur[start + p]);", "        kept.push_back(start + p);"),
    "indexed_row_order": ("      off += idx[k][row % len] * gstride[k];\n      row /= len;",
                          "      off += idx[k][row / len % len] * gstride[k];\n      row %= len;"),
    "indexed_no_replica_compare": ("if (std::memcmp(X + (size_t)g * es, from, es) != 0) mismatch.store(1);",
                                   "if (false) mismatch.store(1);"),
    # partial (sum) sources
    "partial_reverse_order": ("if (src_pl[m] == kPartial) q = q * src_mesh[m] + coord[m];",
                              "if (src_pl[m] == kPartial) q = q * src_mesh[m] + (src_mesh[m] - 1 - coord[m]);"),
    "partial_starts_from_zero": ("  std::vector<float> sum(X[0]);\n  for (int64_t q = 1; q < contributions; ++q) {",
                                 "  std::vector<float> sum((size_t)numel, 0.0f);\n"
                                 "  for (int64_t q = 0; q < contributions; ++q) {"),
    "partial_drops_last": ("  for (int64_t q = 1; q < contributions; ++q) {",
                           "  for (int64_t q = 1; q < contributions - 1; ++q) {"),
    "partial_bf16_truncates": ("const uint32_t out = dst_fmt == 0 ? f32 : convert_one(kFormats[0], T, f32);",
                               "const uint32_t out = dst_fmt == 0 ? f32 : (T.frac == 7 ? f32 >> 16 : "
                               "convert_one(kFormats[0], T, f32));"),
    "partial_no_replica_compare": ("if (std::memcmp(&Xq[g + j], &v, 4) != 0) mismatch.store(1);",
                                   "if (false) mismatch.store(1);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "oracle.cpp")).read()
    find, repl = MUTANTS[name]
    assert src.count(find) == 1, f"mutation anchor for {name} not found exactly once"
    mutant = tmp_path / "oracle_mutant.cpp"
    mutant.write_text(src.replace(find, repl))
    lib = oracle.build(str(tmp_path / "liboracle_mutant.so"), str(mutant))
    # run the pins in a child process: a mutant may also crash, which counts as caught
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([ROOT, HERE]))
    res = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), lib],
                         capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode != 0, f"no pin caught mutant {name}:\n{res.stdout}\n{res.stderr}"
