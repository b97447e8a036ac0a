// Host planner of the reshard library: plain C++17, no HIP.
//
// From two DTensor layouts (global shape + device mesh + placements) it finds
// every overlap between a source shard and a destination shard and turns each
// overlap into copy descriptors for the fused gfx950 copy kernel.  The pages
// that describe the Reshard collective fix the principle -- compute the exact
// intersections of source and destination shards, then move only those
// (news.bpdata.com write-up, "the Reshard collective" section; techfeed.io
// write-up, "reformulation" section and its 8x8 example) -- and the
// send-once-then-replicate treatment of destination replicas (techfeed.io,
// "NVIDIA's NVLink implementation" section).
#pragma once

#include <cstdint>
#include <string>
#include <utility>
#include <vector>

#include "reshard.h"

namespace rs {

constexpr int kMaxDims = RESHARD_MAX_NDIM;
constexpr int kMaxMeshDims = RESHARD_MAX_MESH_NDIM;

struct Layout {
  int ndim = 0;
  int64_t shape[kMaxDims] = {};
  int dtype = 0;
  int64_t elem_size = 0;
  int mesh_ndim = 0;
  int64_t mesh[kMaxMeshDims] = {};
  int32_t place[kMaxMeshDims] = {};
  int64_t split[kMaxMeshDims] = {};  // split factor of each mesh dim (1 = plain Shard / Replicate)
  bool strided = false;              // some split factor above 1
  int64_t n_partial = 1;             // contributions: product of the Partial mesh dims' sizes
  bool partial = false;              // some mesh dim is Partial (sum)
  int64_t nranks = 0;
};

// Contribution number of `rank` under a layout with Partial mesh dims: its
// coordinates on those dims, row-major (0 for a layout without them).
int64_t partial_index(const Layout& L, int64_t rank);

// Contributions one REDUCE descriptor can sum (12 bits of its unit field).
constexpr int64_t kMaxPartials = 4095;

struct Box {
  int64_t lo[kMaxDims];
  int64_t hi[kMaxDims];
};

// Ordered runs [lo, hi) of global indices along one tensor dim: what a rank of
// a strided layout holds, stored in this order (increasing, not touching).
using Runs = std::vector<std::pair<int64_t, int64_t>>;

// Conversion code (RESHARD_CONVERT_*) from src_dtype to dst_dtype: 0 when the
// dtypes are equal, -1 when the pair is not supported.
int conversion_of(int src_dtype, int dst_dtype);

// Validates and fills a layout; returns false with a message on bad input.
// split: one split factor per mesh dim, or NULL for all 1.
bool make_layout(int ndim, const int64_t* shape, int dtype, int mesh_ndim, const int64_t* mesh,
                 const int32_t* placements, Layout* out, std::string* err, const int64_t* split = nullptr);

// Box of `rank` (row-major mesh coordinates, nested ceil-chunk splitting).
// Layouts without split factors only.
void shard_box(const Layout& L, int64_t rank, Box* out);

// Runs of global indices that `rank` holds along tensor dim `dim`, for any
// layout.  A mesh dim with split factor f that shards `dim` cuts the rank's
// current index list (what the mesh dims to its left left it, length n) into f
// ceil-chunks, cuts each of those into mesh-size ceil-chunks, and keeps part
// coord of each, in order (DTensor's right-to-left _StridedShard placement;
// f = 1 is a plain Shard).
Runs shard_runs(const Layout& L, int64_t rank, int dim);
bool box_empty(int ndim, const Box& b);
int64_t box_numel(int ndim, const Box& b);

// A set of ranks of one tensor that hold the same non-empty box (or, for a
// strided layout, the same runs along every dim; box is then their bounding box).
struct Group {
  int64_t tensor;
  Box box;
  std::vector<int64_t> ranks;  // ascending
  Runs runs[kMaxDims];         // strided layouts only
  std::vector<std::vector<int64_t>> parts;  // Partial layouts only: ranks by contribution
};

// One overlap of a unique source box and a unique destination box.  A frame
// places the shard buffer in global coordinates: local index = global - lo,
// buffer extents = hi - lo.  For a plain layout it is the group's box; for a
// strided one it is shifted per run, so that the piece's run lands at its
// position in the buffer.
struct Piece {
  int64_t tensor;
  int64_t src_rank;   // replica chosen to read from
  int64_t src_group;  // index into HostPlan::src_groups
  int64_t dst_group;  // index into HostPlan::dst_groups
  Box box;            // global coordinates
  int64_t bytes;
  Box sframe, dframe;
  std::vector<int64_t> src_ranks;  // Partial sources: the rank read for each contribution
};

// Tiling.  One workgroup of kTileThreads threads copies one tile of one
// descriptor: kTileItems consecutive items, one per thread (4 KiB of source for
// 16-byte items and 16-byte destination chunks).
constexpr uint32_t kTileThreads = 256;
constexpr uint32_t kItemsPerThread = 1;
constexpr uint32_t kTileItems = kTileThreads * kItemsPerThread;

// Rows at least this long whose alignment is below 16 bytes are copied as
// destination-aligned 16-byte chunks; shorter ones item by item.
constexpr int64_t kChunkedMinRun = 128;
// Longest row a descriptor holds (longer rows are split into column ranges).
constexpr int64_t kMaxRunBytes = int64_t(1) << 30;

// LDS window of a RESHARD_DESC_WINDOW tile, and the most segments one band may
// have on each side.  A tensor's pieces go through windows when rows are at most
// kWindowBytes wide, only the first and the last tensor dims are split, and some
// piece has rows shorter than kWindowMaxRun bytes (narrow column runs).
constexpr uint32_t kWindowBytes = 16384;
constexpr uint32_t kWindowMaxSegs = 64;
constexpr int64_t kWindowMaxRun = 128;
// Bands at most kRowModeBytes wide skip LDS: each lane assembles whole rows in a
// 16-byte register, kRowsPerLane rows per lane and tile.  A 16-byte band whose
// source or destination side is four packed 4-byte column runs (the four lanes
// of a quad exchange words) takes kQuadRowsPerLane rows per lane and tile.
constexpr int64_t kRowModeBytes = 16;
constexpr uint32_t kRowsPerLane = 4;
constexpr uint32_t kQuadRowsPerLane = 2;
// LDS window of a narrow band (a packed window band that the narrow-band
// kernel moves), and its row pitch for a band W bytes wide: an odd number of
// dwords when W is a multiple of 4, else W.  A band of at most kRowModeBytes
// with segments of one or two bytes goes there too (its rows per tile are the
// largest power of two up to kTileThreads * kRowsPerLane whose window fits), and
// so does one of 12-byte rows of dword segments.
constexpr uint32_t kNarrowWindowBytes = 18432;
constexpr uint32_t narrow_pitch(uint32_t W) { return W % 4 ? W : 4 * ((W / 4) | 1u); }
// A narrow band whose destination pieces per tile would be small (under
// kNarrowSmallPiece bytes in some destination segment), that has a destination
// segment of one or two bytes (whose lanes move eight rows each), or whose
// tiles would be
// short (under kNarrowShortTile rows) takes twice the rows, in a window of up
// to kNarrowBigWindowBytes; such bands run in launches of their own, with half
// as many workgroups per CU.
constexpr uint32_t kNarrowBigWindowBytes = 2 * kNarrowWindowBytes;
constexpr int64_t kNarrowSmallPiece = 1024;
constexpr int64_t kNarrowShortTile = 64;

// How the narrow-band kernel moves a segment wb bytes wide at window column cb
// of a band W bytes wide at pitch P (see the kernel).
enum NarrowClass : uint32_t { kSegDwords = 0, kSegWhole = 1, kSegRows = 2, kSegPieces = 3, kSegBytes = 4 };
constexpr uint32_t narrow_class(uint32_t wb, uint32_t cb, uint32_t P, uint32_t W) {
  return P % 4 == 0 && wb % 4 == 0 && cb % 4 == 0 ? kSegDwords
         : cb == 0 && wb == W && P == W          ? kSegWhole
         : wb > 16                               ? kSegPieces
         : wb <= 2 || wb == 4 || wb == 8 || wb == 16 ? kSegRows
                                                     : kSegBytes;
}

// Whether segments [0, n) of a band side are k packed rw-byte column runs in
// column order (run s at column rw * s) with one fan-out.
inline bool runs_side(const reshard_segment_t* S, uint32_t n, uint32_t k, uint32_t rw) {
  if (n != k) return false;
  for (uint32_t s = 0; s < n; ++s)
    if (S[s].width != rw || uint64_t(S[s].row_stride) != rw || S[s].col != rw * s || S[s].fanout != S[0].fanout)
      return false;
  return true;
}

// Whether a WINDOW band (run_bytes W wide, `rows_per_tile` rows a tile, source
// segments src[0, ns), destination segments dst[0, nd)) is one the narrow-band
// kernel builds move: 0 no, 1 with dword segments only, 2 with segments of
// other classes too.  Every segment packed (row stride = width), at most 64 a
// side, the window (rows_per_tile rows at the band's pitch) within
// kNarrowBigWindowBytes; a band of at most kRowModeBytes only with a segment of
// one or two bytes, a source segment of the bytes class or a destination one
// over 4 bytes, or of 12-byte rows of dword segments, and not one with four
// 4-byte or eight 2-byte column runs on a side (the row mode's exchanges).
int narrow_band(uint32_t W, uint64_t rows_per_tile, const reshard_segment_t* src, uint32_t ns,
                const reshard_segment_t* dst, uint32_t nd);
// Cache line of the L2: a band whose tiles would start off the line grid in
// its segments gives up to kLineBytes / row_stride rows to a head band of its
// own, so that the tiles after it start on the grid (destination lines first).
constexpr int64_t kLineBytes = 128;

// Whether the segments of one side of a 16-byte band are four packed 4-byte
// column runs with one fan-out (the kernel's quad exchange applies).
inline bool quad_side(const std::vector<reshard_segment_t>& segs) {
  if (segs.size() != 4) return false;
  for (const reshard_segment_t& s : segs)
    if (s.width != 4 || s.row_stride != 4 || s.fanout != segs[0].fanout) return false;
  return true;
}

// The same for eight packed 2-byte column runs (single bf16 or fp16 columns over
// eight shards): the eight lanes of a group exchange halfwords.
inline bool octet_side(const std::vector<reshard_segment_t>& segs) {
  if (segs.size() != 8) return false;
  for (const reshard_segment_t& s : segs)
    if (s.width != 2 || s.row_stride != 2 || s.fanout != segs[0].fanout) return false;
  return true;
}

// RESHARD_DESC_GATHER_ROWS bands: a tile is kGatherTileBytes of destination (16
// bytes a lane, 1 KiB a wave), and every source segment is at least
// kGatherMinSeg bytes wide, so that one wave's 1 KiB touches at most two
// segments (or the end of one row and the start of the next).
constexpr uint32_t kGatherTileBytes = 16 * kTileThreads;
constexpr int64_t kGatherMinSeg = 1024;
// Bytes of one band at most (the kernel indexes a band in 31 bits).
constexpr int64_t kGatherMaxBand = (int64_t(1) << 31) - 2 * int64_t(kGatherTileBytes);

// Elements per item of a RESHARD_DESC_CONVERT row.
constexpr uint32_t kConvertElems = RESHARD_CONVERT_ELEMS;

// Tiles of one descriptor.
inline uint64_t desc_tiles(const reshard_descriptor_t& D) {
  if (D.mode == RESHARD_DESC_WINDOW) return (uint64_t(D.extent[0]) + D.extent[1] - 1) / D.extent[1];
  if (D.mode == RESHARD_DESC_GATHER_ROWS)
    return (uint64_t(D.extent[0]) * D.run_bytes + kGatherTileBytes - 1) / kGatherTileBytes;
  const uint64_t items = uint64_t(D.extent[0]) * D.extent[1] * D.extent[2] * D.row_items;
  return (items + kTileItems - 1) / kTileItems;
}

struct HostPlan {
  int n_tensors = 0;
  std::vector<Layout> src, dst;
  std::vector<int> conv;                     // per tensor: RESHARD_CONVERT_* or 0
  std::vector<int64_t> src_base, dst_base;  // first pointer-array slot of each tensor
  int64_t n_src_ptrs = 0, n_dst_ptrs = 0;
  std::vector<uint8_t> src_needed, dst_needed;  // 1 if that pointer slot holds a non-empty shard
  std::vector<int64_t> src_load;                // bytes read from each source pointer slot
  std::vector<Group> src_groups, dst_groups;
  std::vector<Piece> pieces;
  std::vector<reshard_descriptor_t> descs;
  std::vector<uint32_t> refs;       // fan-out: destination pointer slots (0-based in dst_ptrs)
  std::vector<reshard_segment_t> segs;  // segments of RESHARD_DESC_WINDOW descriptors
  std::vector<uint32_t> tile_begin; // first tile of each descriptor; n_desc + 1 entries
  uint64_t n_tiles = 0;
  int64_t global_bytes = 0, bytes_read = 0, bytes_written = 0, n_dst_writes = 0;
  double plan_host_us = 0.0;
};

// Builds the host plan of n tensors.  Returns RESHARD_OK or an error code with
// a message in *err.
reshard_status_t build_plan(int n, const Layout* const* src, const Layout* const* dst,
                            HostPlan* out, std::string* err);

// Division by an invariant 32-bit divisor d >= 1 for numerators below 2^31:
// q = (mulhi(n, m) + n) >> s.  Granlund & Montgomery, "Division by invariant
// integers using multiplication" (PLDI 1994), round-up multiplier.
void magic_u31(uint32_t d, uint32_t* m, uint32_t* s);

// Tile-group lookup of a launch group: one u32 per kTileGroup consecutive tiles,
// stored after the group's tile_begin list, so that a workgroup can find its
// descriptor with one load instead of a search.  Entry g describes tiles
// [64 g, 64 g + 64): its low 24 bits are the index d of the descriptor holding
// tile 64 g and its high 8 bits a split s in 1..64: the group's tiles from
// 64 g + s on belong to descriptor d + 1 (s = 64: none do).  kTileGroupSearch
// in the high bits marks a group that touches three or more descriptors; its
// tiles search tile_begin instead.  (Only the gather-rows build reads it: for
// the other builds a search over tile_begin measured as fast.)
constexpr uint32_t kTileGroup = 64;
constexpr uint32_t kTileGroupSearch = 255;
inline uint64_t tile_groups(uint64_t n_tiles) { return (n_tiles + kTileGroup - 1) / kTileGroup; }
// Fills the tile_groups(n_tiles) entries at out from tile_begin[0 .. n_desc].
void fill_tile_groups(const uint32_t* tile_begin, uint32_t n_desc, uint32_t n_tiles, uint32_t* out);

// A gather-rows descriptor keeps a segment lookup in the 56 bytes of src_offset
// and the strides, which that mode does not use: uint16 entry k describes row
// columns [1024 k, 1024 k + 1024) -- the index of the segment holding column
// 1024 k in its low 6 bits and, in its high 10 bits, the offset inside the KiB
// where the next segment starts (0: none starts there; segments are at least
// 1 KiB wide, so at most one does).  Rows up to kGatherLutKiB KiB wide with at
// most kGatherLutSegs segments have one (row_items = 1); other bands search.
constexpr uint32_t kGatherLutKiB = 28;
constexpr uint32_t kGatherLutSegs = 64;

// Largest item count a descriptor may hold (items are indexed in 31 bits).
constexpr uint64_t kMaxItems = (uint64_t(1) << 31) - 1;

}  // namespace rs
