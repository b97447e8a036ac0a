// Host planner: layouts -> boxes -> replica groups -> overlaps -> descriptors.
// Plain C++17; the device side lives in kernel.hip, the C ABI in reshard.hip.
#include "plan.h"

#include <algorithm>
#include <chrono>
#include <cstring>
#include <map>
#include <unordered_map>
#include <utility>

namespace rs {

namespace {

int64_t elem_size_of(int dtype) {
  switch (dtype) {
    case RESHARD_DTYPE_U8:
    case RESHARD_DTYPE_I8:
    case RESHARD_DTYPE_BOOL:
    case RESHARD_DTYPE_FP8_E4M3:
    case RESHARD_DTYPE_FP8_E5M2:
      return 1;
    case RESHARD_DTYPE_BF16:
    case RESHARD_DTYPE_F16:
    case RESHARD_DTYPE_I16:
      return 2;
    case RESHARD_DTYPE_F32:
    case RESHARD_DTYPE_I32:
      return 4;
    case RESHARD_DTYPE_F64:
    case RESHARD_DTYPE_I64:
      return 8;
    default:
      return 0;
  }
}

}  // namespace

int conversion_of(int src_dtype, int dst_dtype) {
  if (src_dtype == dst_dtype) return 0;
  if (src_dtype == RESHARD_DTYPE_F32 && dst_dtype == RESHARD_DTYPE_BF16) return RESHARD_CONVERT_F32_BF16;
  if (src_dtype == RESHARD_DTYPE_F32 && dst_dtype == RESHARD_DTYPE_F16) return RESHARD_CONVERT_F32_F16;
  if (src_dtype == RESHARD_DTYPE_BF16 && dst_dtype == RESHARD_DTYPE_F32) return RESHARD_CONVERT_BF16_F32;
  if (src_dtype == RESHARD_DTYPE_F16 && dst_dtype == RESHARD_DTYPE_F32) return RESHARD_CONVERT_F16_F32;
  return -1;
}

namespace {

bool same_box(int ndim, const Box& a, const Box& b) {
  for (int k = 0; k < ndim; ++k)
    if (a.lo[k] != b.lo[k] || a.hi[k] != b.hi[k]) return false;
  return true;
}

// Groups the non-empty boxes of one tensor's layout by equality.  Groups come
// out ordered by their lowest rank.  Ranks that share a box differ only in the
// coordinates of Replicate mesh dims (and of mesh dims whose chunks are empty),
// so a rank is compared with the groups already formed, most recent first.
void group_ranks(const Layout& L, int64_t tensor, std::vector<Group>* groups) {
  const size_t first = groups->size();
  std::map<std::vector<int64_t>, size_t> index;  // used only for big meshes
  const bool use_index = L.nranks > 256;
  for (int64_t r = 0; r < L.nranks; ++r) {
    Box b;
    shard_box(L, r, &b);
    if (box_empty(L.ndim, b)) continue;
    size_t found = SIZE_MAX;
    if (use_index) {
      std::vector<int64_t> key(2 * L.ndim);
      for (int k = 0; k < L.ndim; ++k) {
        key[2 * k] = b.lo[k];
        key[2 * k + 1] = b.hi[k];
      }
      auto it = index.find(key);
      if (it != index.end()) found = it->second;
      else index.emplace(std::move(key), groups->size());
    } else {
      for (size_t g = groups->size(); g-- > first;)
        if (same_box(L.ndim, (*groups)[g].box, b)) {
          found = g;
          break;
        }
    }
    if (found == SIZE_MAX) groups->push_back(Group{tensor, b, {r}, {}});
    else (*groups)[found].ranks.push_back(r);
  }
}

// Unique source boxes of one tensor seen as a grid.  Along each tensor dim the
// distinct non-empty source intervals are disjoint and cover the dim, and every
// combination of them is some rank's box (each tensor dim's interval depends
// only on the coordinates of the mesh dims that shard it).
struct SourceGrid {
  int ndim = 0;
  std::vector<std::vector<std::pair<int64_t, int64_t>>> iv;  // per dim, sorted by lo
  std::vector<int64_t> cell_stride;
  std::vector<int64_t> dense;                      // cell -> group, when the grid is small
  std::unordered_map<int64_t, int64_t> sparse;     // cell -> group otherwise
  int64_t group_of(int64_t cell) const {
    if (!dense.empty()) return dense[size_t(cell)];
    auto it = sparse.find(cell);
    return it == sparse.end() ? -1 : it->second;
  }
};

int64_t interval_index(const std::vector<std::pair<int64_t, int64_t>>& v, int64_t lo) {
  auto it = std::lower_bound(v.begin(), v.end(), std::make_pair(lo, INT64_MIN));
  return int64_t(it - v.begin());
}

SourceGrid make_grid(int ndim, const std::vector<Group>& groups, size_t g_begin, size_t g_end) {
  SourceGrid G;
  G.ndim = ndim;
  G.iv.resize(ndim);
  for (int d = 0; d < ndim; ++d) {
    auto& v = G.iv[d];
    for (size_t g = g_begin; g < g_end; ++g) v.emplace_back(groups[g].box.lo[d], groups[g].box.hi[d]);
    std::sort(v.begin(), v.end());
    v.erase(std::unique(v.begin(), v.end()), v.end());
  }
  G.cell_stride.assign(ndim, 1);
  for (int d = ndim - 2; d >= 0; --d) G.cell_stride[d] = G.cell_stride[d + 1] * int64_t(G.iv[d + 1].size());
  const int64_t cells = G.cell_stride[0] * int64_t(G.iv[0].size());
  if (cells <= (int64_t(1) << 20)) G.dense.assign(size_t(cells), -1);
  for (size_t g = g_begin; g < g_end; ++g) {
    int64_t cell = 0;
    for (int d = 0; d < ndim; ++d) cell += interval_index(G.iv[d], groups[g].box.lo[d]) * G.cell_stride[d];
    if (!G.dense.empty()) G.dense[size_t(cell)] = int64_t(g);
    else G.sparse.emplace(cell, int64_t(g));
  }
  return G;
}

// Calls fn(box, source group) for every cell of the source grid that
// overlaps dbox (the overlap as box), in row-major cell order.
template <class Fn>
reshard_status_t for_each_cell(const SourceGrid& grid, const Box& dbox, int nd, std::string* err, Fn fn) {
  // per dim, the range of source intervals that overlap the destination box
  int64_t first[kMaxDims], last[kMaxDims], idx[kMaxDims];
  for (int k = 0; k < nd; ++k) {
    const auto& v = grid.iv[k];
    auto lo_it = std::upper_bound(v.begin(), v.end(), std::make_pair(dbox.lo[k], INT64_MAX));
    first[k] = std::max<int64_t>(0, int64_t(lo_it - v.begin()) - 1);
    last[k] = first[k];
    while (last[k] + 1 < int64_t(v.size()) && v[last[k] + 1].first < dbox.hi[k]) ++last[k];
    idx[k] = first[k];
  }
  for (;;) {  // every cell in the product of those ranges
    int64_t cell = 0;
    Box box;
    bool empty = false;
    for (int k = 0; k < nd; ++k) {
      cell += idx[k] * grid.cell_stride[k];
      box.lo[k] = std::max(dbox.lo[k], grid.iv[k][idx[k]].first);
      box.hi[k] = std::min(dbox.hi[k], grid.iv[k][idx[k]].second);
      if (box.hi[k] <= box.lo[k]) empty = true;
    }
    if (!empty) {
      const int64_t sg = grid.group_of(cell);
      if (sg < 0) {
        *err = "internal: source grid cell without a rank";
        return RESHARD_ERR_INVALID_ARGUMENT;
      }
      fn(box, sg);
    }
    int k = nd - 1;
    while (k >= 0 && idx[k] == last[k]) {
      idx[k] = first[k];
      --k;
    }
    if (k < 0) break;
    ++idx[k];
  }
  return RESHARD_OK;
}

struct Dim {
  int64_t e;   // extent
  int64_t ss;  // source stride, bytes
  int64_t sd;  // destination stride, bytes
};

// Outer dims of a run, inner -> outer (at most one per tensor dim).
struct Dims {
  Dim d[kMaxDims];
  int n = 0;
  size_t size() const { return size_t(n); }
  bool empty() const { return n == 0; }
  Dim& operator[](size_t i) { return d[i]; }
  const Dim& operator[](size_t i) const { return d[i]; }
  Dim& back() { return d[n - 1]; }
  void push_back(const Dim& x) { d[n++] = x; }
  void pop_back() { --n; }
  const Dim* begin() const { return d; }
  const Dim* end() const { return d + n; }
};

uint32_t unit_for(int64_t bits) {
  uint32_t u = 16;
  while (u > 1 && (bits & int64_t(u - 1))) u >>= 1;
  return u;
}

// Emits descriptors for a run of `run_bytes` contiguous bytes repeated over the
// outer dims (inner -> outer order), splitting where the kernel's 31-bit item
// indexing or its three outer dims would be exceeded.
void emit(HostPlan* P, uint32_t piece, uint32_t src_ptr, uint32_t ref_begin, uint32_t fanout,
          int64_t src_off, int64_t dst_off, int64_t run_bytes, Dims outer) {
  if (outer.size() > 3) {  // peel the outermost dim into separate descriptors
    Dim top = outer.back();
    outer.pop_back();
    for (int64_t i = 0; i < top.e; ++i)
      emit(P, piece, src_ptr, ref_begin, fanout, src_off + i * top.ss, dst_off + i * top.sd,
           run_bytes, outer);
    return;
  }
  if (run_bytes > kMaxRunBytes) {  // split every row into column ranges
    for (int64_t c = 0; c < run_bytes; c += kMaxRunBytes) {
      const int64_t n = std::min<int64_t>(kMaxRunBytes, run_bytes - c);
      emit(P, piece, src_ptr, ref_begin, fanout, src_off + c, dst_off + c, n, outer);
    }
    return;
  }
  int64_t bits = src_off | dst_off | run_bytes;
  for (const Dim& d : outer) bits |= d.ss | d.sd;
  const uint32_t unit = unit_for(bits);
  const bool chunked = unit < 16 && run_bytes >= kChunkedMinRun;
  const uint64_t row_items = chunked ? uint64_t(run_bytes + 30) / 16 : uint64_t(run_bytes) / unit;
  uint64_t rows = 1;
  for (const Dim& d : outer) rows *= uint64_t(d.e);

  if (rows * row_items > kMaxItems) {  // halve the outermost dim with extent > 1
    for (int k = int(outer.size()) - 1; k >= 0; --k) {
      if (outer[k].e < 2) continue;
      Dims a = outer, b = outer;
      int64_t h = outer[k].e / 2;
      a[k].e = h;
      b[k].e = outer[k].e - h;
      emit(P, piece, src_ptr, ref_begin, fanout, src_off, dst_off, run_bytes, a);
      emit(P, piece, src_ptr, ref_begin, fanout, src_off + h * outer[k].ss, dst_off + h * outer[k].sd,
           run_bytes, b);
      return;
    }
  }

  reshard_descriptor_t D;
  std::memset(&D, 0, sizeof(D));
  D.src_offset = src_off;
  D.dst_offset = dst_off;
  // descriptor order: extent[0] outermost, extent[2] the fastest outer dim;
  // `outer` is listed inner -> outer, so outer[j] goes to slot 2 - j.
  for (int j = 0; j < 3; ++j) {
    const int slot = 2 - j;
    if (j < int(outer.size())) {
      D.extent[slot] = uint32_t(outer[j].e);
      D.src_stride[slot] = outer[j].ss;
      D.dst_stride[slot] = outer[j].sd;
    } else {
      D.extent[slot] = 1;
    }
  }
  D.run_bytes = uint32_t(run_bytes);
  D.row_items = uint32_t(row_items);
  D.unit = uint16_t(unit);
  D.mode = chunked ? RESHARD_DESC_DST_CHUNKS : RESHARD_DESC_ITEMS;
  D.src_ptr = src_ptr;
  D.dst_ref_begin = ref_begin;
  D.fanout = fanout;
  magic_u31(D.row_items, &D.magic[0][0], &D.magic[0][1]);
  magic_u31(D.extent[2], &D.magic[1][0], &D.magic[1][1]);
  magic_u31(D.extent[1], &D.magic[2][0], &D.magic[2][1]);
  D.piece = piece;
  P->descs.push_back(D);
}

// RESHARD_DESC_CONVERT (or RESHARD_DESC_REDUCE) descriptors for rows of `run`
// elements (outer dims inner -> outer, byte strides of each side), split like
// emit() does; `unit` is the descriptor's conversion (or contributions and
// formats) field.
void emit_convert(HostPlan* P, uint32_t piece, uint32_t src_ptr, uint32_t ref_begin, uint32_t fanout,
                  int64_t src_off, int64_t dst_off, int64_t run, Dims outer, uint32_t unit, int64_t es_s,
                  int64_t es_d, uint16_t mode = RESHARD_DESC_CONVERT) {
  if (outer.size() > 3) {
    Dim top = outer.back();
    outer.pop_back();
    for (int64_t i = 0; i < top.e; ++i)
      emit_convert(P, piece, src_ptr, ref_begin, fanout, src_off + i * top.ss, dst_off + i * top.sd,
                   run, outer, unit, es_s, es_d, mode);
    return;
  }
  const int64_t max_run = kMaxRunBytes / 4;  // elements: every row stays under kMaxRunBytes per side
  if (run > max_run) {
    for (int64_t c = 0; c < run; c += max_run)
      emit_convert(P, piece, src_ptr, ref_begin, fanout, src_off + c * es_s, dst_off + c * es_d,
                   std::min<int64_t>(max_run, run - c), outer, unit, es_s, es_d, mode);
    return;
  }
  const uint64_t row_items = uint64_t(run + kConvertElems - 1) / kConvertElems;
  uint64_t rows = 1;
  for (const Dim& d : outer) rows *= uint64_t(d.e);
  if (rows * row_items > kMaxItems) {  // halve the outermost dim with extent > 1
    for (int k = int(outer.size()) - 1; k >= 0; --k) {
      if (outer[k].e < 2) continue;
      Dims a = outer, b = outer;
      const int64_t h = outer[k].e / 2;
      a[k].e = h;
      b[k].e = outer[k].e - h;
      emit_convert(P, piece, src_ptr, ref_begin, fanout, src_off, dst_off, run, a, unit, es_s, es_d, mode);
      emit_convert(P, piece, src_ptr, ref_begin, fanout, src_off + h * outer[k].ss,
                   dst_off + h * outer[k].sd, run, b, unit, es_s, es_d, mode);
      return;
    }
  }
  reshard_descriptor_t D;
  std::memset(&D, 0, sizeof(D));
  D.src_offset = src_off;
  D.dst_offset = dst_off;
  for (int j = 0; j < 3; ++j) {
    const int slot = 2 - j;
    if (j < int(outer.size())) {
      D.extent[slot] = uint32_t(outer[j].e);
      D.src_stride[slot] = outer[j].ss;
      D.dst_stride[slot] = outer[j].sd;
    } else {
      D.extent[slot] = 1;
    }
  }
  D.run_bytes = uint32_t(run);
  D.row_items = uint32_t(row_items);
  D.unit = uint16_t(unit);
  D.mode = mode;
  D.src_ptr = src_ptr;
  D.dst_ref_begin = ref_begin;
  D.fanout = fanout;
  magic_u31(D.row_items, &D.magic[0][0], &D.magic[0][1]);
  magic_u31(D.extent[2], &D.magic[1][0], &D.magic[1][1]);
  magic_u31(D.extent[1], &D.magic[2][0], &D.magic[2][1]);
  D.piece = piece;
  P->descs.push_back(D);
}

// Turns one overlap into descriptors: local offsets in the source and
// destination shards, then adjacent dims are merged wherever both sides are
// contiguous across them, and size-1 dims are dropped.  Merging works in
// elements; strides become bytes of each side's dtype (they differ only for a
// converting reshard, conv != 0).
void describe_piece(HostPlan* P, uint32_t piece_idx, uint32_t src_ptr, uint32_t ref_begin,
                    uint32_t fanout, const Box& piece, const Box& sbox, const Box& dbox, int ndim,
                    int64_t es_s, int64_t es_d, int conv, uint32_t reduce_unit = 0) {
  int64_t s_stride[kMaxDims], d_stride[kMaxDims];  // elements
  int64_t ss = 1, sd = 1;
  for (int k = ndim - 1; k >= 0; --k) {
    s_stride[k] = ss;
    d_stride[k] = sd;
    ss *= sbox.hi[k] - sbox.lo[k];
    sd *= dbox.hi[k] - dbox.lo[k];
  }
  int64_t src_off = 0, dst_off = 0;
  for (int k = 0; k < ndim; ++k) {
    src_off += (piece.lo[k] - sbox.lo[k]) * s_stride[k];
    dst_off += (piece.lo[k] - dbox.lo[k]) * d_stride[k];
  }
  // Fold dims from the innermost outwards into the contiguous run while both
  // sides stay contiguous; the rest become outer dims.
  bool in_run = true;
  int64_t run = 1;  // elements
  Dims outer;       // inner -> outer
  for (int k = ndim - 1; k >= 0; --k) {
    int64_t e = piece.hi[k] - piece.lo[k];
    if (e == 1) continue;
    if (in_run && s_stride[k] == run && d_stride[k] == run) {
      run *= e;
      continue;
    }
    in_run = false;
    if (!outer.empty() && s_stride[k] == outer.back().e * outer.back().ss &&
        d_stride[k] == outer.back().e * outer.back().sd) {
      outer.back().e *= e;
      continue;
    }
    outer.push_back(Dim{e, s_stride[k], d_stride[k]});
  }
  for (int j = 0; j < outer.n; ++j) {
    outer[j].ss *= es_s;
    outer[j].sd *= es_d;
  }
  if (reduce_unit != 0)
    emit_convert(P, piece_idx, src_ptr, ref_begin, fanout, src_off * es_s, dst_off * es_d, run, outer,
                 reduce_unit, es_s, es_d, RESHARD_DESC_REDUCE);
  else if (conv == 0)
    emit(P, piece_idx, src_ptr, ref_begin, fanout, src_off * es_s, dst_off * es_d, run * es_s, outer);
  else
    emit_convert(P, piece_idx, src_ptr, ref_begin, fanout, src_off * es_s, dst_off * es_d, run, outer,
                 uint32_t(conv), es_s, es_d);
}

// Float format code of a REDUCE descriptor: 0 binary32, 1 bfloat16, 2 binary16.
uint32_t float_format(int dtype) {
  return dtype == RESHARD_DTYPE_BF16 ? 1u : dtype == RESHARD_DTYPE_F16 ? 2u : 0u;
}

// Copy descriptors of every piece of one tensor, in piece order.
void emit_pieces(HostPlan* P, int t, size_t pc0, size_t pc1) {
  const int nd = P->src[t].ndim;
  const int64_t es_s = P->src[t].elem_size, es_d = P->dst[t].elem_size;
  const int conv = P->conv[t];
  for (size_t i = pc0; i < pc1; ++i) {
    const Piece& pc = P->pieces[i];
    const Group& dgrp = P->dst_groups[pc.dst_group];
    const uint32_t ref_begin = uint32_t(P->refs.size());
    for (int64_t r : dgrp.ranks) P->refs.push_back(uint32_t(P->dst_base[t] + r));
    if (!pc.src_ranks.empty()) {  // Partial: the contributions' source slots follow the fan-out
      const uint32_t list = uint32_t(P->refs.size());
      for (int64_t r : pc.src_ranks) P->refs.push_back(uint32_t(P->src_base[t] + r));
      const uint32_t unit = uint32_t(pc.src_ranks.size()) | (float_format(P->src[t].dtype) << 12) |
                            (float_format(P->dst[t].dtype) << 14);
      describe_piece(P, uint32_t(i), list, ref_begin, uint32_t(dgrp.ranks.size()), pc.box, pc.sframe,
                     pc.dframe, nd, es_s, es_d, conv, unit);
      continue;
    }
    describe_piece(P, uint32_t(i), uint32_t(P->src_base[t] + pc.src_rank), ref_begin,
                   uint32_t(dgrp.ranks.size()), pc.box, pc.sframe, pc.dframe, nd, es_s, es_d, conv);
  }
}

// 2-d view of a tensor for windows: rows = dims 0..nd-2 flattened, columns =
// the last dim.  Valid when no box splits dims 1..nd-2.
struct View2d {
  int64_t row_mult = 1;  // flattened rows per unit of dim 0
  int64_t cols = 1;
};

bool view_2d(const HostPlan& P, int t, size_t pc0, size_t pc1, View2d* v) {
  const Layout& S = P.src[t];
  const int nd = S.ndim;
  if (nd < 2) return false;
  v->cols = S.shape[nd - 1];
  v->row_mult = 1;
  for (int k = 1; k < nd - 1; ++k) v->row_mult *= S.shape[k];
  for (size_t i = pc0; i < pc1; ++i) {
    const Box* boxes[2] = {&P.src_groups[P.pieces[i].src_group].box, &P.dst_groups[P.pieces[i].dst_group].box};
    for (const Box* b : boxes)
      for (int k = 1; k < nd - 1; ++k)
        if (b->lo[k] != 0 || b->hi[k] != S.shape[k]) return false;
  }
  return true;
}

// Window bands of one tensor.  Rows are cut wherever a source or destination
// box starts or ends; each band lists the pieces that cover it as source
// segments (merged where one shard continues across pieces) and the
// destination boxes that cover it as destination segments.
bool emit_windows(HostPlan* P, int t, size_t pc0, size_t pc1, const View2d& v, std::vector<int64_t>& load) {
  const int nd = P->src[t].ndim;
  const int64_t es = P->src[t].elem_size;
  const int64_t width = v.cols * es;
  const int64_t pitch = (width + 15) / 16 * 16;
  if (width <= 0 || pitch > int64_t(kWindowBytes)) return false;
  const int64_t window_rows = int64_t(kWindowBytes) / pitch;  // rows per tile of an LDS window
  auto rlo = [&](const Box& b) { return b.lo[0] * v.row_mult; };
  auto rhi = [&](const Box& b) { return b.hi[0] * v.row_mult; };
  // A replicated source box is read in k row parts, part j from its j-th
  // replica: a band then reads whole source rows from one replica (its
  // segments of that box merge into one packed run), and the replicas share
  // the reads evenly.
  auto part_cut = [&](const Group& g, int64_t j) {
    const int64_t k = int64_t(g.ranks.size());
    return rlo(g.box) + (rhi(g.box) - rlo(g.box)) * j / k;
  };
  auto replica = [&](const Group& g, int64_t row) {
    int64_t j = int64_t(g.ranks.size()) - 1;
    while (j > 0 && part_cut(g, j) > row) --j;
    return g.ranks[size_t(j)];
  };
  std::vector<int64_t> cuts;
  for (size_t i = pc0; i < pc1; ++i) {
    cuts.push_back(rlo(P->pieces[i].box));
    cuts.push_back(rhi(P->pieces[i].box));
    const Group& sg = P->src_groups[P->pieces[i].src_group];
    for (int64_t j = 1; j < int64_t(sg.ranks.size()); ++j) {
      const int64_t cut = part_cut(sg, j);
      if (cut > rlo(P->pieces[i].box) && cut < rhi(P->pieces[i].box)) cuts.push_back(cut);
    }
  }
  std::sort(cuts.begin(), cuts.end());
  cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
  struct Pending {
    reshard_descriptor_t d;
    std::vector<reshard_segment_t> src, dst;
    std::vector<std::vector<uint32_t>> dst_refs;
  };
  std::vector<Pending> bands;
  for (size_t c = 0; c + 1 < cuts.size(); ++c) {
    const int64_t ra = cuts[c], rb = cuts[c + 1];
    Pending b;
    std::vector<int64_t> dst_seen;
    int64_t bits = width;
    for (size_t i = pc0; i < pc1; ++i) {
      const Piece& pc = P->pieces[i];
      if (rlo(pc.box) > ra || rhi(pc.box) < rb) continue;
      const Box& sb = P->src_groups[pc.src_group].box;
      const int64_t s_cols = sb.hi[nd - 1] - sb.lo[nd - 1];
      reshard_segment_t s;
      s.offset = ((ra - rlo(sb)) * s_cols + (pc.box.lo[nd - 1] - sb.lo[nd - 1])) * es;
      s.row_stride = s_cols * es;
      s.col = uint32_t(pc.box.lo[nd - 1] * es);
      s.width = uint32_t((pc.box.hi[nd - 1] - pc.box.lo[nd - 1]) * es);
      s.ptr = uint32_t(P->src_base[t] + replica(P->src_groups[pc.src_group], ra));
      s.fanout = 0;
      b.src.push_back(s);
      if (std::find(dst_seen.begin(), dst_seen.end(), pc.dst_group) == dst_seen.end()) {
        dst_seen.push_back(pc.dst_group);
        const Group& dg = P->dst_groups[pc.dst_group];
        const int64_t d_cols = dg.box.hi[nd - 1] - dg.box.lo[nd - 1];
        reshard_segment_t d;
        d.offset = (ra - rlo(dg.box)) * d_cols * es;
        d.row_stride = d_cols * es;
        d.col = uint32_t(dg.box.lo[nd - 1] * es);
        d.width = uint32_t(d_cols * es);
        d.ptr = 0;
        d.fanout = uint32_t(dg.ranks.size());
        b.dst.push_back(d);
        std::vector<uint32_t> refs;
        for (int64_t r : dg.ranks) refs.push_back(uint32_t(P->dst_base[t] + r));
        b.dst_refs.push_back(refs);
      }
    }
    // sources in column order; merge neighbours that continue in the same shard
    std::sort(b.src.begin(), b.src.end(),
              [](const reshard_segment_t& x, const reshard_segment_t& y) { return x.col < y.col; });
    std::vector<reshard_segment_t> merged;
    for (const reshard_segment_t& s : b.src) {
      if (!merged.empty()) {
        reshard_segment_t& m = merged.back();
        if (m.ptr == s.ptr && m.row_stride == s.row_stride && m.col + m.width == s.col &&
            m.offset + int64_t(m.width) == s.offset) {
          m.width += s.width;
          continue;
        }
      }
      merged.push_back(s);
    }
    b.src = merged;
    // destinations in column order too (with their fan-out lists)
    std::vector<size_t> order(b.dst.size());
    for (size_t k = 0; k < order.size(); ++k) order[k] = k;
    std::sort(order.begin(), order.end(), [&](size_t x, size_t y) { return b.dst[x].col < b.dst[y].col; });
    std::vector<reshard_segment_t> dst_sorted;
    std::vector<std::vector<uint32_t>> refs_sorted;
    for (size_t k : order) {
      dst_sorted.push_back(b.dst[k]);
      refs_sorted.push_back(std::move(b.dst_refs[k]));
    }
    b.dst = std::move(dst_sorted);
    b.dst_refs = std::move(refs_sorted);
    if (b.src.size() > kWindowMaxSegs || b.dst.size() > kWindowMaxSegs) return false;
    for (const auto& s : b.src) bits |= s.offset | s.row_stride | s.col | s.width;
    for (const auto& d : b.dst) bits |= d.offset | d.row_stride | d.col | d.width;
    std::memset(&b.d, 0, sizeof(b.d));
    b.d.mode = RESHARD_DESC_WINDOW;
    b.d.unit = uint16_t(unit_for(bits));
    b.d.run_bytes = uint32_t(width);
    b.d.row_items = uint32_t(pitch);
    b.d.extent[0] = uint32_t(rb - ra);
    const bool quad = width == kRowModeBytes && (quad_side(b.src) || quad_side(b.dst) || octet_side(b.src) ||
                                                 octet_side(b.dst));
    // a segment of one or two bytes, a source segment of the bytes class or a
    // destination one over 4 bytes: a band the narrow kernel takes from the row mode
    bool bytewise = false;
    for (const auto* side : {&b.src, &b.dst})
      for (const auto& x : *side)
        bytewise |= x.width <= 2 || (narrow_class(x.width, x.col, narrow_pitch(uint32_t(width)), uint32_t(width)) ==
                                         kSegBytes && (side == &b.src || x.width > 4));
    int64_t rows_per_tile = width > kRowModeBytes ? window_rows
                            : int64_t(kTileThreads) * (quad ? kQuadRowsPerLane : kRowsPerLane);
    if (width <= kRowModeBytes && bytewise && !quad)
      while (rows_per_tile * narrow_pitch(uint32_t(width)) > int64_t(kNarrowWindowBytes)) rows_per_tile /= 2;
    // a narrow band with small destination pieces, a thin destination segment or
    // short tiles: twice the rows
    if (narrow_band(uint32_t(width), uint64_t(rows_per_tile), b.src.data(), uint32_t(b.src.size()), b.dst.data(),
                    uint32_t(b.dst.size()))) {
      bool small = rows_per_tile < kNarrowShortTile;
      for (const auto& x : b.dst) {
        const int64_t piece = rows_per_tile * int64_t(x.width);
        small |= piece < kNarrowSmallPiece || x.width <= 2;
      }
      if (small &&
          2 * rows_per_tile * narrow_pitch(uint32_t(width)) <= int64_t(kNarrowBigWindowBytes))
        rows_per_tile *= 2;
    }
    b.d.extent[1] = uint32_t(rows_per_tile);
    b.d.extent[2] = 1;
    b.d.piece = uint32_t(pc0);
    if (rb - ra > int64_t(kMaxItems)) return false;
    // Tiles of a band end where its segments' lines end only if the band starts
    // on the line grid: otherwise two tiles (often on different XCDs) write
    // parts of each line a tile boundary cuts.  Take the head rows up to the
    // row that puts the most segment starts on the grid (a destination counts
    // twice: a line written in part costs more than one read twice) into a
    // band of their own, when at least one full tile follows.
    const int64_t tile = b.d.extent[1];
    int64_t head = 0;
    bool tiles_keep_grid = true;
    for (const auto* side : {&b.src, &b.dst})
      for (const auto& x : *side) tiles_keep_grid &= (tile * x.row_stride) % kLineBytes == 0;
    if (tiles_keep_grid) {
      auto score = [&](int64_t h) {
        int64_t n = 0;
        for (const auto& x : b.src) n += (x.offset + h * x.row_stride) % kLineBytes == 0;
        for (const auto& x : b.dst) n += 2 * ((x.offset + h * x.row_stride) % kLineBytes == 0);
        return n;
      };
      int64_t best = score(0);
      for (int64_t h = 1; h < kLineBytes && h + tile <= rb - ra; ++h)
        if (score(h) > best) best = score(h), head = h;
    }
    if (head > 0) {
      Pending rest = b;
      b.d.extent[0] = uint32_t(head);
      rest.d.extent[0] = uint32_t(rb - ra - head);
      for (auto* side : {&rest.src, &rest.dst})
        for (auto& x : *side) x.offset += head * x.row_stride;
      int64_t rest_bits = width;
      for (const auto& x : rest.src) rest_bits |= x.offset | x.row_stride | x.col | x.width;
      for (const auto& x : rest.dst) rest_bits |= x.offset | x.row_stride | x.col | x.width;
      rest.d.unit = uint16_t(unit_for(rest_bits));
      bands.push_back(std::move(b));
      bands.push_back(std::move(rest));
      continue;
    }
    bands.push_back(std::move(b));
  }
  for (Pending& b : bands) {
    b.d.src_ptr = uint32_t(P->segs.size());
    b.d.dst_ref_begin = uint32_t(b.src.size());
    b.d.fanout = uint32_t(b.dst.size());
    for (const auto& s : b.src) P->segs.push_back(s);
    for (size_t k = 0; k < b.dst.size(); ++k) {
      reshard_segment_t d = b.dst[k];
      d.ptr = uint32_t(P->refs.size());
      for (uint32_t r : b.dst_refs[k]) P->refs.push_back(r);
      P->segs.push_back(d);
    }
    P->descs.push_back(b.d);
  }
  // source reads by the bands in place of the pieces' own replica choice
  for (size_t i = pc0; i < pc1; ++i) load[size_t(P->src_base[t] + P->pieces[i].src_rank)] -= P->pieces[i].bytes;
  for (const Pending& b : bands)
    for (const auto& s : b.src) load[s.ptr] += int64_t(b.d.extent[0]) * s.width;
  return true;
}

// Gather-rows bands of one tensor whose destination boxes are whole rows of
// the 2-d view and whose source pieces are column strips, each at least
// kGatherMinSeg bytes wide.  Rows are cut wherever a source or destination box
// starts or ends; each band holds the source segments that tile its rows (in
// column order, merged where one shard continues) and the one destination box
// that holds them.  Returns false, emitting nothing it keeps, when the pieces
// do not have that shape.
bool emit_gather_rows(HostPlan* P, int t, size_t pc0, size_t pc1, const View2d& v) {
  const int nd = P->src[t].ndim;
  const int64_t es = P->src[t].elem_size;
  const int64_t W = v.cols * es;
  if (W < kGatherMinSeg) return false;
  auto rlo = [&](const Box& b) { return b.lo[0] * v.row_mult; };
  auto rhi = [&](const Box& b) { return b.hi[0] * v.row_mult; };
  for (size_t i = pc0; i < pc1; ++i) {
    const Box& db = P->dst_groups[P->pieces[i].dst_group].box;
    if (db.lo[nd - 1] != 0 || db.hi[nd - 1] != v.cols) return false;  // destination rows must be whole
  }
  // A replicated source box is read in k row parts, part j from its j-th
  // replica: a band then reads whole source rows from one replica (its
  // segments of that box merge into one packed run), and the replicas share
  // the reads evenly.
  auto part_cut = [&](const Group& g, int64_t j) {
    const int64_t k = int64_t(g.ranks.size());
    return rlo(g.box) + (rhi(g.box) - rlo(g.box)) * j / k;
  };
  auto replica = [&](const Group& g, int64_t row) {
    int64_t j = int64_t(g.ranks.size()) - 1;
    while (j > 0 && part_cut(g, j) > row) --j;
    return g.ranks[size_t(j)];
  };
  std::vector<int64_t> cuts;
  for (size_t i = pc0; i < pc1; ++i) {
    cuts.push_back(rlo(P->pieces[i].box));
    cuts.push_back(rhi(P->pieces[i].box));
    const Group& sg = P->src_groups[P->pieces[i].src_group];
    for (int64_t j = 1; j < int64_t(sg.ranks.size()); ++j) {
      const int64_t cut = part_cut(sg, j);
      if (cut > rlo(P->pieces[i].box) && cut < rhi(P->pieces[i].box)) cuts.push_back(cut);
    }
  }
  std::sort(cuts.begin(), cuts.end());
  cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
  struct Band {
    int64_t ra, rb;
    int64_t dst_group;
    std::vector<reshard_segment_t> src;
  };
  std::vector<Band> bands;
  for (size_t c = 0; c + 1 < cuts.size(); ++c) {
    Band b{cuts[c], cuts[c + 1], -1, {}};
    for (size_t i = pc0; i < pc1; ++i) {
      const Piece& pc = P->pieces[i];
      if (rlo(pc.box) > b.ra || rhi(pc.box) < b.rb) continue;
      if (b.dst_group >= 0 && b.dst_group != pc.dst_group) return false;
      b.dst_group = pc.dst_group;
      const Box& sb = P->src_groups[pc.src_group].box;
      const int64_t s_cols = sb.hi[nd - 1] - sb.lo[nd - 1];
      reshard_segment_t sg;
      sg.offset = ((b.ra - rlo(sb)) * s_cols + (pc.box.lo[nd - 1] - sb.lo[nd - 1])) * es;
      sg.row_stride = s_cols * es;
      sg.col = uint32_t(pc.box.lo[nd - 1] * es);
      sg.width = uint32_t((pc.box.hi[nd - 1] - pc.box.lo[nd - 1]) * es);
      sg.ptr = uint32_t(P->src_base[t] + pc.src_rank);
      sg.fanout = 0;
      b.src.push_back(sg);
    }
    std::sort(b.src.begin(), b.src.end(),
              [](const reshard_segment_t& x, const reshard_segment_t& y) { return x.col < y.col; });
    std::vector<reshard_segment_t> merged;
    for (const reshard_segment_t& sg : b.src) {
      if (!merged.empty()) {
        reshard_segment_t& m = merged.back();
        if (m.ptr == sg.ptr && m.row_stride == sg.row_stride && m.col + m.width == sg.col &&
            m.offset + int64_t(m.width) == sg.offset) {
          m.width += sg.width;
          continue;
        }
      }
      merged.push_back(sg);
    }
    b.src = std::move(merged);
    int64_t next = 0;  // the segments must tile [0, W)
    for (const reshard_segment_t& sg : b.src) {
      if (int64_t(sg.col) != next || int64_t(sg.width) < kGatherMinSeg) return false;
      next += sg.width;
    }
    if (next != W || b.dst_group < 0) return false;
    bands.push_back(std::move(b));
  }
  const int64_t max_rows = kGatherMaxBand / W;
  for (const Band& b : bands) {
    const Group& dg = P->dst_groups[b.dst_group];
    const uint32_t ref_begin = uint32_t(P->refs.size());
    for (int64_t r : dg.ranks) P->refs.push_back(uint32_t(P->dst_base[t] + r));
    for (int64_t r0 = b.ra; r0 < b.rb; r0 += max_rows) {
      const int64_t rows = std::min(max_rows, b.rb - r0);
      reshard_descriptor_t D;
      std::memset(&D, 0, sizeof(D));
      D.mode = RESHARD_DESC_GATHER_ROWS;
      D.dst_offset = (r0 - rlo(dg.box)) * W;
      D.run_bytes = uint32_t(W);
      D.extent[0] = uint32_t(rows);
      D.extent[1] = uint32_t(b.src.size());
      D.extent[2] = 1;
      D.src_ptr = uint32_t(P->segs.size());
      D.dst_ref_begin = ref_begin;
      D.fanout = uint32_t(dg.ranks.size());
      // the segment lookup, in the fields this mode leaves unused
      uint16_t lut[kGatherLutKiB] = {};
      static_assert(sizeof(lut) == sizeof(D.src_offset) + sizeof(D.src_stride) + sizeof(D.dst_stride),
                    "lookup slots");
      if (W <= int64_t(kGatherLutKiB) * 1024 && b.src.size() <= kGatherLutSegs) {
        size_t i = 0;
        for (uint32_t k = 0; int64_t(k) * 1024 < W; ++k) {
          const uint32_t c = k * 1024;
          while (i + 1 < b.src.size() && b.src[i + 1].col <= c) ++i;
          const uint32_t next = i + 1 < b.src.size() ? b.src[i + 1].col : uint32_t(W);
          const uint32_t off = next < c + 1024 && next < uint32_t(W) ? next - c : 0u;
          lut[k] = uint16_t(i | (off << 6));
        }
        D.row_items = 1;
      }
      std::memcpy(&D.src_offset, lut, sizeof(D.src_offset));
      std::memcpy(D.src_stride, lut + 4, sizeof(D.src_stride));
      std::memcpy(D.dst_stride, lut + 16, sizeof(D.dst_stride));
      int64_t bits = W | D.dst_offset;
      for (reshard_segment_t sg : b.src) {
        sg.offset += (r0 - b.ra) * sg.row_stride;
        bits |= sg.offset | sg.row_stride | sg.col;
        P->segs.push_back(sg);
      }
      D.unit = uint16_t(unit_for(bits));
      magic_u31(D.run_bytes, &D.magic[0][0], &D.magic[0][1]);
      D.piece = uint32_t(pc0);
      P->descs.push_back(D);
    }
  }
  return true;
}

// Descriptors of one tensor: windows when some piece has narrow rows and the
// tensor has a 2-d view that fits; gather-rows bands when whole destination
// rows are assembled from wide source column strips that meet off the 16-byte
// grid (the per-piece path would write the lines where strips meet in part,
// from two workgroups); per-piece descriptors otherwise.
void emit_tensor(HostPlan* P, int t, size_t pc0, size_t pc1, std::vector<int64_t>& load) {
  if (pc0 == pc1) return;
  const size_t d0 = P->descs.size(), r0 = P->refs.size();
  emit_pieces(P, t, pc0, pc1);
  if (P->conv[t] != 0) return;  // converting rows always go element-group by element-group
  if (P->src[t].strided || P->dst[t].strided) return;  // bands assume one box per rank
  if (P->src[t].partial) return;                         // sums go element group by element group
  bool narrow = false, chunked = false;
  for (size_t i = d0; i < P->descs.size(); ++i) {
    const reshard_descriptor_t& D = P->descs[i];
    const uint64_t rows = uint64_t(D.extent[0]) * D.extent[1] * D.extent[2];
    if (rows > 1 && int64_t(D.run_bytes) < kWindowMaxRun) narrow = true;
    if (rows > 1 && D.mode == RESHARD_DESC_DST_CHUNKS) chunked = true;
  }
  View2d v;
  if ((!narrow && !chunked) || !view_2d(*P, t, pc0, pc1, &v)) return;
  const size_t s0 = P->segs.size();
  std::vector<reshard_descriptor_t> saved(P->descs.begin() + d0, P->descs.end());
  std::vector<uint32_t> saved_refs(P->refs.begin() + r0, P->refs.end());
  P->descs.resize(d0);
  P->refs.resize(r0);
  const bool done = narrow ? emit_windows(P, t, pc0, pc1, v, load) : emit_gather_rows(P, t, pc0, pc1, v);
  if (!done) {  // keep the per-piece descriptors
    P->descs.resize(d0);
    P->refs.resize(r0);
    P->segs.resize(s0);
    P->descs.insert(P->descs.end(), saved.begin(), saved.end());
    P->refs.insert(P->refs.end(), saved_refs.begin(), saved_refs.end());
  }
}

// Groups the non-empty shards of a strided layout by equal runs along every
// dim, in order of their lowest rank.
void group_ranks_runs(const Layout& L, int64_t tensor, std::vector<Group>* groups) {
  std::map<std::vector<int64_t>, size_t> index;
  for (int64_t r = 0; r < L.nranks; ++r) {
    Group g;
    g.tensor = tensor;
    std::vector<int64_t> key;
    bool empty = false;
    for (int k = 0; k < L.ndim; ++k) {
      g.runs[k] = shard_runs(L, r, k);
      if (g.runs[k].empty()) {
        empty = true;
        break;
      }
      g.box.lo[k] = g.runs[k].front().first;
      g.box.hi[k] = g.runs[k].back().second;
      key.push_back(int64_t(g.runs[k].size()));
      for (const auto& [a, b] : g.runs[k]) {
        key.push_back(a);
        key.push_back(b);
      }
    }
    if (empty) continue;
    auto it = index.find(key);
    if (it != index.end()) {
      (*groups)[it->second].ranks.push_back(r);
      continue;
    }
    index.emplace(std::move(key), groups->size());
    g.ranks.push_back(r);
    groups->push_back(std::move(g));
  }
}

// Position, in a shard's local buffer along one dim, of the run starting at
// global index lo (runs holds it).
int64_t run_origin(const Runs& runs, int64_t lo) {
  int64_t pos = 0;
  for (const auto& [a, b] : runs) {
    if (a == lo) return pos;
    pos += b - a;
  }
  return -1;
}

int64_t runs_length(const Runs& runs) {
  int64_t n = 0;
  for (const auto& [a, b] : runs) n += b - a;
  return n;
}

// Pieces and descriptors of one tensor whose source or destination layout is
// strided.  Along each dim the runs of all source groups are either equal or
// disjoint (a rank's runs depend only on its coordinates in the mesh dims that
// split that dim), and together they cover the dim: they form a grid as the
// boxes of a plain layout do.  Every run of a destination group is cut by the
// grid; each cell is one piece, read from the least-loaded replica of the
// source group that holds the cell and placed in both shard buffers by frames.
reshard_status_t plan_runs_tensor(HostPlan* P, int t, std::vector<int64_t>& load, std::string* err) {
  const Layout& S = P->src[t];
  const Layout& D = P->dst[t];
  const int nd = S.ndim;
  const int64_t es = S.elem_size;
  const size_t sg0 = P->src_groups.size();
  group_ranks_runs(S, t, &P->src_groups);
  const size_t sg1 = P->src_groups.size();
  const size_t dg0 = P->dst_groups.size();
  group_ranks_runs(D, t, &P->dst_groups);
  const size_t dg1 = P->dst_groups.size();
  for (size_t g = sg0; g < sg1; ++g)
    for (int64_t r : P->src_groups[g].ranks) P->src_needed[P->src_base[t] + r] = 1;
  for (size_t g = dg0; g < dg1; ++g)
    for (int64_t r : P->dst_groups[g].ranks) P->dst_needed[P->dst_base[t] + r] = 1;
  if (sg0 == sg1) return RESHARD_OK;

  std::vector<Runs> iv(nd);  // per dim: every source run, sorted
  for (int k = 0; k < nd; ++k) {
    for (size_t g = sg0; g < sg1; ++g)
      iv[k].insert(iv[k].end(), P->src_groups[g].runs[k].begin(), P->src_groups[g].runs[k].end());
    std::sort(iv[k].begin(), iv[k].end());
    iv[k].erase(std::unique(iv[k].begin(), iv[k].end()), iv[k].end());
    for (size_t i = 0; i + 1 < iv[k].size(); ++i)
      if (iv[k][i].second > iv[k][i + 1].first) {
        *err = "internal: overlapping source runs";
        return RESHARD_ERR_INVALID_ARGUMENT;
      }
  }
  std::vector<int64_t> stride(nd, 1);
  for (int k = nd - 2; k >= 0; --k) stride[k] = stride[k + 1] * int64_t(iv[k + 1].size());
  std::unordered_map<int64_t, int64_t> cell_group;
  for (size_t g = sg0; g < sg1; ++g) {
    const Group& G = P->src_groups[g];
    std::vector<size_t> j(nd, 0);
    for (;;) {
      int64_t cell = 0;
      for (int k = 0; k < nd; ++k) cell += interval_index(iv[k], G.runs[k][j[k]].first) * stride[k];
      cell_group[cell] = int64_t(g);
      int k = nd - 1;
      while (k >= 0 && j[k] + 1 == G.runs[k].size()) j[k--] = 0;
      if (k < 0) break;
      ++j[k];
    }
  }

  const size_t pc0 = P->pieces.size();
  for (size_t g = dg0; g < dg1; ++g) {
    const Group& dgrp = P->dst_groups[g];
    int64_t dext[kMaxDims];
    for (int k = 0; k < nd; ++k) dext[k] = runs_length(dgrp.runs[k]);
    std::vector<size_t> dj(nd, 0);
    std::vector<int64_t> dorig(nd, 0);  // local position of run dj[k]
    for (;;) {  // every destination sub-box: one run per dim
      int64_t first[kMaxDims], last[kMaxDims], idx[kMaxDims];
      for (int k = 0; k < nd; ++k) {
        const auto& run = dgrp.runs[k][dj[k]];
        const auto& v = iv[k];
        auto lo_it = std::upper_bound(v.begin(), v.end(), std::make_pair(run.first, INT64_MAX));
        first[k] = std::max<int64_t>(0, int64_t(lo_it - v.begin()) - 1);
        last[k] = first[k];
        while (last[k] + 1 < int64_t(v.size()) && v[last[k] + 1].first < run.second) ++last[k];
        idx[k] = first[k];
      }
      for (;;) {  // every source cell overlapping it
        int64_t cell = 0;
        Box box;
        bool empty = false;
        for (int k = 0; k < nd; ++k) {
          const auto& run = dgrp.runs[k][dj[k]];
          cell += idx[k] * stride[k];
          box.lo[k] = std::max(run.first, iv[k][idx[k]].first);
          box.hi[k] = std::min(run.second, iv[k][idx[k]].second);
          if (box.hi[k] <= box.lo[k]) empty = true;
        }
        if (!empty) {
          auto it = cell_group.find(cell);
          if (it == cell_group.end()) {
            *err = "internal: source grid cell without a rank";
            return RESHARD_ERR_INVALID_ARGUMENT;
          }
          const int64_t sg = it->second;
          const Group& sgrp = P->src_groups[sg];
          int64_t best = sgrp.ranks[0];
          for (int64_t r : sgrp.ranks)
            if (load[P->src_base[t] + r] < load[P->src_base[t] + best]) best = r;
          Box sframe, dframe;
          for (int k = 0; k < nd; ++k) {
            const int64_t so = run_origin(sgrp.runs[k], iv[k][idx[k]].first);
            sframe.lo[k] = iv[k][idx[k]].first - so;
            sframe.hi[k] = sframe.lo[k] + runs_length(sgrp.runs[k]);
            dframe.lo[k] = dgrp.runs[k][dj[k]].first - dorig[k];
            dframe.hi[k] = dframe.lo[k] + dext[k];
          }
          const int64_t bytes = box_numel(nd, box) * es;
          load[P->src_base[t] + best] += bytes;
          P->pieces.push_back(Piece{t, best, sg, int64_t(g), box, bytes, sframe, dframe});
          const int64_t fanout = int64_t(dgrp.ranks.size());
          P->bytes_read += bytes;
          P->bytes_written += box_numel(nd, box) * D.elem_size * fanout;
          P->n_dst_writes += fanout;
        }
        int k = nd - 1;
        while (k >= 0 && idx[k] == last[k]) {
          idx[k] = first[k];
          --k;
        }
        if (k < 0) break;
        ++idx[k];
      }
      int k = nd - 1;
      while (k >= 0 && dj[k] + 1 == dgrp.runs[k].size()) {
        dj[k] = 0;
        dorig[k] = 0;
        --k;
      }
      if (k < 0) break;
      dorig[k] += dgrp.runs[k][dj[k]].second - dgrp.runs[k][dj[k]].first;
      ++dj[k];
    }
  }
  emit_tensor(P, t, pc0, P->pieces.size(), load);
  return RESHARD_OK;
}

}  // namespace

void fill_tile_groups(const uint32_t* tb, uint32_t n_desc, uint32_t n_tiles, uint32_t* out) {
  const uint64_t n_groups = tile_groups(n_tiles);
  uint32_t d = 0;  // descriptor of the group's first tile: the last one starting at or before it
  for (uint64_t g = 0; g < n_groups; ++g) {
    const uint32_t t0 = uint32_t(g * kTileGroup);
    const uint32_t t1 = uint32_t(std::min<uint64_t>(uint64_t(t0) + kTileGroup, n_tiles));  // exclusive
    while (d + 1 < n_desc && tb[d + 1] <= t0) ++d;
    uint32_t e = d;  // descriptor of the group's last tile
    while (e + 1 < n_desc && tb[e + 1] <= t1 - 1) ++e;
    if (n_desc >= (1u << 24)) out[g] = kTileGroupSearch << 24;
    else if (e == d) out[g] = d | (kTileGroup << 24);
    else if (e == d + 1) out[g] = d | ((tb[d + 1] - t0) << 24);
    else out[g] = kTileGroupSearch << 24;
  }
}

void magic_u31(uint32_t d, uint32_t* m, uint32_t* s) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;  // l = ceil(log2 d)
  uint64_t mm = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  *m = uint32_t(mm);
  *s = l;
}

bool make_layout(int ndim, const int64_t* shape, int dtype, int mesh_ndim, const int64_t* mesh,
                 const int32_t* placements, Layout* out, std::string* err, const int64_t* split) {
  if (ndim < 1 || ndim > kMaxDims) {
    *err = "ndim must be in [1, " + std::to_string(kMaxDims) + "]";
    return false;
  }
  if (mesh_ndim < 1 || mesh_ndim > kMaxMeshDims) {
    *err = "mesh_ndim must be in [1, " + std::to_string(kMaxMeshDims) + "]";
    return false;
  }
  if (!shape || !mesh || !placements) {
    *err = "NULL shape, mesh or placements";
    return false;
  }
  Layout L;
  L.ndim = ndim;
  L.dtype = dtype;
  L.elem_size = elem_size_of(dtype);
  if (L.elem_size == 0) {
    *err = "unknown dtype " + std::to_string(dtype);
    return false;
  }
  for (int k = 0; k < ndim; ++k) {
    if (shape[k] < 0 || shape[k] > (int64_t(1) << 40)) {
      *err = "global_shape[" + std::to_string(k) + "] out of range";
      return false;
    }
    L.shape[k] = shape[k];
  }
  L.mesh_ndim = mesh_ndim;
  L.nranks = 1;
  for (int m = 0; m < mesh_ndim; ++m) {
    if (mesh[m] < 1 || mesh[m] > (int64_t(1) << 20)) {
      *err = "mesh_shape[" + std::to_string(m) + "] must be in [1, 2^20]";
      return false;
    }
    if (placements[m] != RESHARD_REPLICATE && placements[m] != RESHARD_PARTIAL &&
        (placements[m] < 0 || placements[m] >= ndim)) {
      *err = "placements[" + std::to_string(m) + "] must be RESHARD_REPLICATE, RESHARD_PARTIAL or a tensor dim";
      return false;
    }
    L.mesh[m] = mesh[m];
    L.place[m] = placements[m];
    L.split[m] = split ? split[m] : 1;
    if (L.split[m] < 1 || L.split[m] > (int64_t(1) << 20)) {
      *err = "split_factors[" + std::to_string(m) + "] must be in [1, 2^20]";
      return false;
    }
    if (L.split[m] > 1 && placements[m] < 0) {
      *err = "split_factors[" + std::to_string(m) + "] > 1 on a Replicate or Partial mesh dim";
      return false;
    }
    if (L.split[m] > 1) L.strided = true;
    if (placements[m] == RESHARD_PARTIAL) {
      L.partial = true;
      L.n_partial *= mesh[m];
    }
    L.nranks *= mesh[m];
    if (L.nranks > (int64_t(1) << 24)) {
      *err = "mesh has more than 2^24 ranks";
      return false;
    }
  }
  *out = L;
  return true;
}

void shard_box(const Layout& L, int64_t rank, Box* out) {
  int64_t coord[kMaxMeshDims];
  for (int m = L.mesh_ndim - 1; m >= 0; --m) {
    coord[m] = rank % L.mesh[m];
    rank /= L.mesh[m];
  }
  for (int k = 0; k < L.ndim; ++k) {
    out->lo[k] = 0;
    out->hi[k] = L.shape[k];
  }
  for (int m = 0; m < L.mesh_ndim; ++m) {
    if (L.place[m] < 0) continue;  // Replicate or Partial: no split
    const int k = L.place[m];
    const int64_t lo = out->lo[k], hi = out->hi[k];
    const int64_t chunk = (hi - lo + L.mesh[m] - 1) / L.mesh[m];
    out->lo[k] = std::min(hi, lo + coord[m] * chunk);
    out->hi[k] = std::min(hi, lo + (coord[m] + 1) * chunk);
  }
}

int64_t partial_index(const Layout& L, int64_t rank) {
  int64_t coord[kMaxMeshDims];
  for (int m = L.mesh_ndim - 1; m >= 0; --m) {
    coord[m] = rank % L.mesh[m];
    rank /= L.mesh[m];
  }
  int64_t q = 0;
  for (int m = 0; m < L.mesh_ndim; ++m)
    if (L.place[m] == RESHARD_PARTIAL) q = q * L.mesh[m] + coord[m];
  return q;
}

int narrow_band(uint32_t W, uint64_t rows_per_tile, const reshard_segment_t* src, uint32_t ns,
                const reshard_segment_t* dst, uint32_t nd) {
  if (W == 0 || W > kWindowBytes || ns > 64 || nd > 64) return 0;  // one segment per lane
  const uint32_t P = narrow_pitch(W);
  if (rows_per_tile * P > kNarrowBigWindowBytes) return 0;
  int kind = 1;
  bool thin = false, bytes = false;  // bytes: a source segment of the bytes class, or a destination one over 4 bytes
  for (const auto& side : {std::make_pair(src, ns), std::make_pair(dst, nd)})
    for (uint32_t i = 0; i < side.second; ++i) {
      const reshard_segment_t& x = side.first[i];
      if (x.width == 0 || uint64_t(x.row_stride) != x.width || uint64_t(x.col) + x.width > W) return 0;
      const uint32_t cls = narrow_class(x.width, x.col, P, W);
      if (cls != kSegDwords) kind = 2;
      thin |= x.width <= 2;
      bytes |= cls == kSegBytes && (side.first == src || x.width > 4);
    }
  // the row mode measured faster on 8- and 16-byte rows of dword segments, and
  // on rows scattered into 3-byte shards
  if (W <= uint32_t(kRowModeBytes)) {
    if (W == uint32_t(kRowModeBytes) &&
        (runs_side(src, ns, 4, 4) || runs_side(dst, nd, 4, 4) || runs_side(src, ns, 8, 2) || runs_side(dst, nd, 8, 2)))
      return 0;
    if (!thin && !bytes && (kind != 1 || P != W)) return 0;
  }
  return kind;
}

Runs shard_runs(const Layout& L, int64_t rank, int dim) {
  int64_t coord[kMaxMeshDims];
  for (int m = L.mesh_ndim - 1; m >= 0; --m) {
    coord[m] = rank % L.mesh[m];
    rank /= L.mesh[m];
  }
  Runs cur;
  if (L.shape[dim] > 0) cur.emplace_back(0, L.shape[dim]);
  int64_t n = L.shape[dim];  // length of cur
  for (int m = 0; m < L.mesh_ndim; ++m) {
    if (L.place[m] != dim) continue;
    const int64_t f = L.split[m];
    const int64_t piece = (n + f - 1) / f;
    // local positions kept, in order: part coord[m] of each of the f pieces
    Runs keep;
    for (int64_t j = 0; j < f && j * piece < n; ++j) {
      const int64_t start = j * piece, len = std::min(piece, n - start);
      const int64_t part = (len + L.mesh[m] - 1) / L.mesh[m];
      const int64_t a = std::min(len, coord[m] * part), b = std::min(len, (coord[m] + 1) * part);
      if (a < b) keep.emplace_back(start + a, start + b);
    }
    // map the kept local positions through cur to global runs (both lists
    // are increasing, so one forward walk over cur serves every kept range)
    Runs next;
    int64_t kept = 0;
    size_t r = 0;
    int64_t pos = 0;  // local position where cur[r] starts
    for (const auto& [a, b] : keep) {
      kept += b - a;
      for (int64_t x = a; x < b;) {
        const int64_t in_run = cur[r].second - cur[r].first;
        if (pos + in_run <= x) {  // x lies past cur[r]
          pos += in_run;
          ++r;
          continue;
        }
        const int64_t hi = std::min(b, pos + in_run);
        const int64_t g0 = cur[r].first + (x - pos), g1 = cur[r].first + (hi - pos);
        if (!next.empty() && next.back().second == g0) next.back().second = g1;
        else next.emplace_back(g0, g1);
        x = hi;
      }
    }
    cur = std::move(next);
    n = kept;
  }
  return cur;
}

bool box_empty(int ndim, const Box& b) {
  for (int k = 0; k < ndim; ++k)
    if (b.hi[k] <= b.lo[k]) return true;
  return false;
}

int64_t box_numel(int ndim, const Box& b) {
  int64_t n = 1;
  for (int k = 0; k < ndim; ++k) n *= std::max<int64_t>(0, b.hi[k] - b.lo[k]);
  return n;
}

reshard_status_t build_plan(int n, const Layout* const* src, const Layout* const* dst, HostPlan* P,
                            std::string* err) {
  auto t0 = std::chrono::steady_clock::now();
  if (n < 1) {
    *err = "a plan needs at least one tensor";
    return RESHARD_ERR_INVALID_ARGUMENT;
  }
  P->n_tensors = n;
  for (int t = 0; t < n; ++t) {
    if (!src[t] || !dst[t]) {
      *err = "NULL layout for tensor " + std::to_string(t);
      return RESHARD_ERR_INVALID_ARGUMENT;
    }
    const Layout& S = *src[t];
    const Layout& D = *dst[t];
    if (S.ndim != D.ndim || !std::equal(S.shape, S.shape + S.ndim, D.shape)) {
      *err = "tensor " + std::to_string(t) + ": source and destination differ in global shape";
      return RESHARD_ERR_LAYOUT_MISMATCH;
    }
    const int conv = conversion_of(S.dtype, D.dtype);
    if (conv < 0) {
      *err = "tensor " + std::to_string(t) + ": no conversion from dtype " + std::to_string(S.dtype) +
             " to dtype " + std::to_string(D.dtype);
      return RESHARD_ERR_LAYOUT_MISMATCH;
    }
    if (D.partial) {
      *err = "tensor " + std::to_string(t) + ": a destination layout cannot be Partial";
      return RESHARD_ERR_LAYOUT_MISMATCH;
    }
    if (S.partial) {
      const bool fp = S.dtype == RESHARD_DTYPE_F32 || S.dtype == RESHARD_DTYPE_BF16 || S.dtype == RESHARD_DTYPE_F16;
      if (!fp || S.strided || D.strided || S.n_partial > kMaxPartials) {
        *err = "tensor " + std::to_string(t) +
               ": a Partial source needs F32, BF16 or F16 elements, no split factors on either side and at most " +
               std::to_string(kMaxPartials) + " contributions";
        return RESHARD_ERR_LAYOUT_MISMATCH;
      }
    }
    P->conv.push_back(conv);
    P->src.push_back(S);
    P->dst.push_back(D);
    P->src_base.push_back(P->n_src_ptrs);
    P->dst_base.push_back(P->n_dst_ptrs);
    P->n_src_ptrs += S.nranks;
    P->n_dst_ptrs += D.nranks;
  }
  if (P->n_src_ptrs + P->n_dst_ptrs > (int64_t(1) << 31)) {
    *err = "too many ranks in the plan";
    return RESHARD_ERR_INVALID_ARGUMENT;
  }
  P->src_needed.assign(P->n_src_ptrs, 0);
  P->dst_needed.assign(P->n_dst_ptrs, 0);

  std::vector<int64_t> load(P->n_src_ptrs, 0);  // bytes read from each source slot
  for (int t = 0; t < n; ++t) {
    const Layout& S = P->src[t];
    const Layout& D = P->dst[t];
    const int nd = S.ndim;
    const int64_t es = S.elem_size;
    int64_t numel = 1;
    for (int k = 0; k < nd; ++k) numel *= S.shape[k];
    P->global_bytes += numel * es;

    if (S.strided || D.strided) {
      const reshard_status_t st = plan_runs_tensor(P, t, load, err);
      if (st != RESHARD_OK) return st;
      continue;
    }
    const size_t sg0 = P->src_groups.size();
    group_ranks(S, t, &P->src_groups);
    const size_t sg1 = P->src_groups.size();
    const size_t dg0 = P->dst_groups.size();
    group_ranks(D, t, &P->dst_groups);
    const size_t dg1 = P->dst_groups.size();
    for (size_t g = sg0; g < sg1; ++g)
      for (int64_t r : P->src_groups[g].ranks) P->src_needed[P->src_base[t] + r] = 1;
    for (size_t g = dg0; g < dg1; ++g)
      for (int64_t r : P->dst_groups[g].ranks) P->dst_needed[P->dst_base[t] + r] = 1;
    if (sg0 == sg1) continue;  // empty tensor

    SourceGrid grid = make_grid(nd, P->src_groups, sg0, sg1);
    if (S.partial)  // every contribution of a box in the same group, split by contribution
      for (size_t g = sg0; g < sg1; ++g) {
        Group& G = P->src_groups[g];
        G.parts.assign(size_t(S.n_partial), {});
        for (int64_t r : G.ranks) G.parts[size_t(partial_index(S, r))].push_back(r);
      }
    const size_t pc0 = P->pieces.size();
    for (size_t g = dg0; g < dg1; ++g) {
      const Group& dgrp = P->dst_groups[g];
      const reshard_status_t st = for_each_cell(grid, dgrp.box, nd, err, [&](const Box& box, int64_t sg) {
        const Group& sgrp = P->src_groups[sg];
        // least-loaded replica of this source box; ties go to the lowest rank
        auto least_loaded = [&](const std::vector<int64_t>& ranks) {
          int64_t best = ranks[0];
          for (int64_t r : ranks)
            if (load[P->src_base[t] + r] < load[P->src_base[t] + best]) best = r;
          return best;
        };
        const int64_t bytes = box_numel(nd, box) * es;
        Piece pc{t, 0, sg, int64_t(g), box, bytes, sgrp.box, dgrp.box, {}};
        if (S.partial) {  // one replica of every contribution, in contribution order
          for (const auto& part : sgrp.parts) {
            const int64_t r = least_loaded(part);
            load[P->src_base[t] + r] += bytes;
            pc.src_ranks.push_back(r);
          }
          pc.src_rank = pc.src_ranks[0];
        } else {
          pc.src_rank = least_loaded(sgrp.ranks);
          load[P->src_base[t] + pc.src_rank] += bytes;
        }
        const int64_t fanout = int64_t(dgrp.ranks.size());
        P->bytes_read += bytes * S.n_partial;
        P->bytes_written += box_numel(nd, box) * D.elem_size * fanout;
        P->n_dst_writes += fanout;
        P->pieces.push_back(std::move(pc));
      });
      if (st != RESHARD_OK) return st;
    }
    emit_tensor(P, t, pc0, P->pieces.size(), load);
  }
  // tiles: each descriptor gets desc_tiles() consecutive tiles
  P->tile_begin.assign(1, 0);
  for (const reshard_descriptor_t& D : P->descs) {
    P->n_tiles += desc_tiles(D);
    if (P->n_tiles >= (uint64_t(1) << 31)) {
      *err = "plan needs more than 2^31 tiles";
      return RESHARD_ERR_INVALID_ARGUMENT;
    }
    P->tile_begin.push_back(uint32_t(P->n_tiles));
  }
  P->src_load = std::move(load);
  auto t1 = std::chrono::steady_clock::now();
  P->plan_host_us = std::chrono::duration<double, std::micro>(t1 - t0).count();
  return RESHARD_OK;
}

}  // namespace rs
