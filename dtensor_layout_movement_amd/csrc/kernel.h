// Launch interface of the gfx950 copy kernel (kernel.hip), used by the host
// code of the C ABI (reshard.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "reshard.h"

namespace rs {

constexpr uint32_t kXcds = 8;       // MI355X: workgroups go round-robin over 8 XCDs
constexpr uint32_t kXcdGroup = 64;  // consecutive tiles one XCD takes at a time
constexpr int kKargPtrs = 120;      // pointer slots passed in kernel arguments

// Shard pointers passed by value in the kernel arguments (plans with at most
// kKargPtrs of them).
struct KargPtrs {
  const void* p[kKargPtrs];
};

// Bits of the kernel's `flags` argument.
constexpr uint32_t kAllAligned16 = 1;  // every shard pointer of this execute is 16-byte aligned

// The kernel variant of a plan: the smallest build that covers its descriptors
// (and their window segments).
int kernel_kind(const std::vector<reshard_descriptor_t>& descs, const std::vector<reshard_segment_t>& segs);

// The kernel variant that moves RESHARD_DESC_GATHER_ROWS bands.
int kernel_kind_gather_rows();

// Whether a kernel variant is one that moves narrow bands (packed WINDOW bands
// more than 16 bytes wide).  In the device table, a destination segment of a
// band in a launch of such a variant holds, in row_stride, the absolute pointer
// slot of its first replica (the band is packed: its row stride is its width).
bool kernel_kind_narrow(int kind);

// Workgroups of one launch at most: a dispatch counts its work-items in 32
// bits.  A multiple of kXcds, so that every launch starts on XCD 0's turn.
constexpr uint32_t kMaxLaunchBlocks = (0xffffffffu / 256u) & ~(kXcds - 1);

// Descriptors of one launch that all span `tiles` tiles (the last ones may
// leave some of theirs idle): tile t belongs to descriptor t / tiles, found with
// the multiplier (m, s) and no table load.  tiles = 0: the tiles are looked up.
// Only the gather-rows build reads it.
struct TileStride {
  uint32_t tiles = 0, m = 0, s = 0;
};

// Variant `kind` over workgroups [0, n_wg) on `stream`, as one launch, or as
// several back-to-back launches of at most kMaxLaunchBlocks workgroups each
// when n_wg is larger.  Shard pointers come from `karg` when `table` is NULL,
// else from the device table.  The narrow-band variants take `lds_bytes` of
// dynamic LDS for their window (the largest of the launch's bands).
// Returns the first launch error.
hipError_t launch_copy(int kind, uint32_t n_wg, hipStream_t stream, const reshard_descriptor_t* descs,
                       uint32_t n_desc, const uint32_t* tile_begin, const uint32_t* refs,
                       const reshard_segment_t* segs, const void* const* table, const KargPtrs& karg,
                       uint32_t n_tiles, uint32_t per_xcd, uint32_t flags, TileStride stride, uint32_t lds_bytes);

}  // namespace rs
