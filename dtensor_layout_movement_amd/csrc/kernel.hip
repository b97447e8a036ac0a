// The gfx950 copy kernel of the reshard library and its launch.
//
// Execute = one launch of reshard_copy_kernel.  The plan's descriptor table
// sits in device memory together with the first tile of every descriptor.  One
// workgroup copies one tile (4 KiB of source for 16-byte items): it finds its
// descriptor by a binary search over the tile prefix, then every thread loads
// its item(s) once and stores them to each destination replica (the single-GPU
// form of "send each contribution once, replicate locally": techfeed.io
// write-up, "NVIDIA's NVLink implementation" section).  Many small workgroups
// let the dispatcher balance the load; groups of consecutive tiles are kept on
// one XCD so that rows straddling tile edges merge in that XCD's L2.  Data only moves
// through integer registers, so the copy is bit-exact for every dtype.
#include "kernel.h"

#include <cstddef>
#include <cstdint>
#include <vector>

#include "plan.h"

namespace rs {
namespace {

constexpr int kBlock = int(kTileThreads);  // threads per workgroup (4 wave64s)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

// q = n / d for n < 2^31 with the planner's round-up multiplier (m, s).
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t m, uint32_t s) {
  return (__umulhi(n, m) + n) >> s;
}

// Row origin offsets (relative to the shard pointers) and item index of item f.
struct ItemPos {
  uint64_t src, dst;  // byte offsets of the row origin
  uint32_t col;       // item index inside the row
};

__device__ __forceinline__ ItemPos item_pos(const reshard_descriptor_t& D, uint32_t f) {
  const uint32_t row = div_magic(f, D.magic[0][0], D.magic[0][1]);
  const uint32_t t = div_magic(row, D.magic[1][0], D.magic[1][1]);
  const uint32_t i2 = row - t * D.extent[2];
  const uint32_t i0 = div_magic(t, D.magic[2][0], D.magic[2][1]);
  const uint32_t i1 = t - i0 * D.extent[1];
  ItemPos o;
  o.col = f - row * D.row_items;
  o.src = uint64_t(D.src_offset) + uint64_t(i0) * uint64_t(D.src_stride[0]) +
          uint64_t(i1) * uint64_t(D.src_stride[1]) + uint64_t(i2) * uint64_t(D.src_stride[2]);
  o.dst = uint64_t(D.dst_offset) + uint64_t(i0) * uint64_t(D.dst_stride[0]) +
          uint64_t(i1) * uint64_t(D.dst_stride[1]) + uint64_t(i2) * uint64_t(D.dst_stride[2]);
  return o;
}

template <typename V>
__device__ __forceinline__ V load_item(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
}

template <typename V>
__device__ __forceinline__ void store_item(uint8_t* p, V v) {
  __builtin_nontemporal_store(v, reinterpret_cast<V*>(p));
}

// Global-memory (address space 1) pointer from an address computed as an
// integer, so that accesses compile to global_* rather than flat_* instructions.
template <typename T>
using global_ptr = __attribute__((address_space(1))) T*;
template <typename T>
__device__ __forceinline__ global_ptr<T> as_global(uintptr_t a) {
  return reinterpret_cast<global_ptr<T>>(a);
}

// 16 bytes from any byte address (gfx950 global loads need no alignment).
typedef uint32_t u32x4_u __attribute__((ext_vector_type(4), aligned(1)));
__device__ __forceinline__ u32x4 load_16_unaligned(uintptr_t a) {
  return __builtin_nontemporal_load(as_global<const u32x4_u>(a));
}

// Shard pointers of one descriptor.  kKarg: the pointer array sits in the kernel
// arguments; otherwise in a device table.  Either way every lookup is a scalar
// load from a known address space.
template <bool kKarg>
struct Shards {
  const void* const* table;
  const KargPtrs* karg;
  const uint32_t* refs;  // this descriptor's fan-out list
  __device__ __forceinline__ uintptr_t ptr(uint32_t i) const {
    if constexpr (kKarg) return reinterpret_cast<uintptr_t>(karg->p[i]);
    else return reinterpret_cast<uintptr_t>(table[i]);
  }
  __device__ __forceinline__ uintptr_t dst(uint32_t r) const { return ptr(refs[r]); }
};

// ITEMS mode: items [lo, hi) (at most kBlock * U of them) with V-sized accesses.
// All loads are issued before the stores; each item is stored to every replica.
template <typename V, int U, class Sh>
__device__ __forceinline__ void copy_items(const reshard_descriptor_t& D, const uint8_t* src,
                                           const Sh& sh, uint32_t lo, uint32_t hi) {
  V v[U];
  uint64_t doff[U];
  bool ok[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const uint32_t f = lo + uint32_t(k * kBlock) + threadIdx.x;
    ok[k] = f < hi;
    const ItemPos o = item_pos(D, ok[k] ? f : lo);
    const uint64_t c = uint64_t(o.col) * sizeof(V);
    doff[k] = o.dst + c;
    if (ok[k]) v[k] = load_item<V>(src + o.src + c);
  }
  for (uint32_t r = 0; r < D.fanout; ++r) {
    uint8_t* dst = reinterpret_cast<uint8_t*>(sh.dst(r));
#pragma unroll
    for (int k = 0; k < U; ++k)
      if (ok[k]) store_item<V>(dst + doff[k], v[k]);
  }
}

// Byte range [lo, hi) of the destination row starting at `row` (absolute address
// of replica 0) that chunk `col` covers: the row's part of the col-th 16-byte
// aligned block it touches.
__device__ __forceinline__ void chunk_range(uintptr_t row, uint32_t run, uint32_t col,
                                            uintptr_t* lo, uintptr_t* hi) {
  const uintptr_t block = (row & ~uintptr_t(15)) + uintptr_t(col) * 16;
  *lo = block > row ? block : row;
  *hi = block + 16 < row + run ? block + 16 : row + run;
  if (*hi < *lo) *hi = *lo;  // a block past the row's end: empty
}

typedef uint64_t u64_u __attribute__((aligned(1)));
typedef uint32_t u32_u __attribute__((aligned(1)));
typedef uint16_t u16_u __attribute__((aligned(1)));

// v >> (8 * s) as a 128-bit little-endian value, 1 <= s <= 15.
__device__ __forceinline__ u32x4 shift_right_bytes(u32x4 v, uint32_t s) {
  uint64_t lo = (uint64_t(v.y) << 32) | v.x, hi = (uint64_t(v.w) << 32) | v.z;
  const uint32_t b = 8 * s;
  if (b >= 64) {
    lo = hi >> (b - 64);
    hi = 0;
  } else {
    lo = (lo >> b) | (hi << (64 - b));
    hi >>= b;
  }
  return u32x4{uint32_t(lo), uint32_t(lo >> 32), uint32_t(hi), uint32_t(hi >> 32)};
}

// The first n < 16 bytes of v to address d, with at most four stores.  They are
// streaming (non-temporal) like the full 16-byte stores around them: a partial
// chunk shares its destination line with full chunks, and mixing temporal and
// streaming stores on one line measured 5% slower on misaligned column strips.
__device__ __forceinline__ void store_head_bytes(uintptr_t d, u32x4 v, uint32_t n) {
  uint64_t lo = (uint64_t(v.y) << 32) | v.x;
  const uint64_t hi = (uint64_t(v.w) << 32) | v.z;
  if (n & 8) {
    __builtin_nontemporal_store(lo, as_global<u64_u>(d));
    d += 8;
    lo = hi;
  }
  if (n & 4) {
    __builtin_nontemporal_store(uint32_t(lo), as_global<u32_u>(d));
    d += 4;
    lo >>= 32;
  }
  if (n & 2) {
    __builtin_nontemporal_store(uint16_t(lo), as_global<u16_u>(d));
    d += 2;
    lo >>= 16;
  }
  if (n & 1) __builtin_nontemporal_store(uint8_t(lo), as_global<uint8_t>(d));
}

// DST_CHUNKS mode: chunks [lo, hi).  Every non-empty chunk is one 16-byte load
// that stays inside its source row: at the chunk's own bytes for a full chunk,
// at the row start for the head chunk and at the row end minus 16 for the tail
// chunk (rows are at least kChunkedMinRun bytes).  A full chunk is then one
// aligned 16-byte store per replica; a partial one (fewer than 16 bytes) at most
// four.  All loads are issued before any store.  Replicas share replica 0's
// 16-byte phase.
template <int U, class Sh>
__device__ __forceinline__ void copy_chunks(const reshard_descriptor_t& D, const uint8_t* src,
                                            const Sh& sh, uint32_t lo, uint32_t hi) {
  const uintptr_t d0 = sh.dst(0);
  const uint32_t run = D.run_bytes;
  u32x4 v[U];
  uintptr_t clo[U];  // first covered destination byte, replica-0 address
  uint32_t n[U];     // covered bytes: 16 (full), 1..15 (partial) or 0
  uint32_t skip[U];  // leading bytes of the load that precede the chunk (tail chunk only)
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const uint32_t f = lo + uint32_t(k * kBlock) + threadIdx.x;
    const ItemPos o = item_pos(D, f < hi ? f : lo);
    const uintptr_t row = d0 + o.dst;
    uintptr_t chi;
    chunk_range(row, run, o.col, &clo[k], &chi);
    n[k] = f < hi ? uint32_t(chi - clo[k]) : 0u;
    const uint32_t off = uint32_t(clo[k] - row);            // chunk's first byte within the row
    const uint32_t load_off = off < run - 16 ? off : run - 16;
    skip[k] = off - load_off;
    if (n[k] != 0) v[k] = load_16_unaligned(reinterpret_cast<uintptr_t>(src) + o.src + load_off);
  }
#pragma unroll
  for (int k = 0; k < U; ++k)
    if (n[k] != 0 && skip[k] != 0) v[k] = shift_right_bytes(v[k], skip[k]);
  for (uint32_t r = 0; r < D.fanout; ++r) {
    const uintptr_t shift = sh.dst(r) - d0;
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const uintptr_t d = clo[k] + shift;
      if (n[k] == 16) __builtin_nontemporal_store(v[k], as_global<u32x4>(d));
      else if (n[k] != 0) store_head_bytes(d, v[k], n[k]);
    }
  }
}

// ---------------------------------------------------------------- windows
//
// A RESHARD_DESC_WINDOW tile moves rows [r0, r0 + hr) of a band through an LDS
// window (row r at r * pitch).  Phase 1 reads every source segment into the
// window, phase 2 writes every destination segment from it to each replica.
// Global accesses are 16-byte chunks aligned to the global address; the LDS side
// takes whatever alignment that leaves.  A segment whose rows are packed in its
// shard (row stride == width) is handled as one contiguous run, so narrow column
// runs still move in 16-byte global accesses.

typedef uint32_t u32x4_u1 __attribute__((ext_vector_type(4), aligned(1)));
typedef uint32_t u32x2_u1 __attribute__((ext_vector_type(2), aligned(1)));

__device__ __forceinline__ u32x4 shift_left_bytes(u32x4 v, uint32_t s) {  // s in [0, 15]
  if (s == 0) return v;
  uint64_t lo = (uint64_t(v.y) << 32) | v.x, hi = (uint64_t(v.w) << 32) | v.z;
  const uint32_t b = 8 * s;
  if (b >= 64) {
    hi = lo << (b - 64);
    lo = 0;
  } else {
    hi = (hi << b) | (lo >> (64 - b));
    lo <<= b;
  }
  return u32x4{uint32_t(lo), uint32_t(lo >> 32), uint32_t(hi), uint32_t(hi >> 32)};
}

// Bytes [0, n) of v (n <= 16) into LDS at p, with at most four writes.
__device__ __forceinline__ void lds_put(uint8_t* p, u32x4 v, uint32_t n) {
  if (n == 16) {
    *reinterpret_cast<u32x4_u1*>(p) = v;
    return;
  }
  uint64_t lo = (uint64_t(v.y) << 32) | v.x;
  const uint64_t hi = (uint64_t(v.w) << 32) | v.z;
  if (n & 8) {
    *reinterpret_cast<u64_u*>(p) = lo;
    p += 8;
    lo = hi;
  }
  if (n & 4) {
    *reinterpret_cast<u32_u*>(p) = uint32_t(lo);
    p += 4;
    lo >>= 32;
  }
  if (n & 2) {
    *reinterpret_cast<u16_u*>(p) = uint16_t(lo);
    p += 2;
    lo >>= 16;
  }
  if (n & 1) *p = uint8_t(lo);
}

// n <= 16 bytes from LDS at p into bytes [0, n) of the result.
__device__ __forceinline__ u32x4 lds_get(const uint8_t* p, uint32_t n) {
  if (n == 16) return *reinterpret_cast<const u32x4_u1*>(p);
  uint64_t lo = 0, hi = 0;
  uint32_t at = 0;  // bytes gathered so far
  if (n & 8) {
    lo = *reinterpret_cast<const u64_u*>(p);
    at = 8;
  }
  if (n & 4) {
    const uint64_t x = *reinterpret_cast<const u32_u*>(p + at);
    if (at < 8) lo |= x << (8 * at); else hi |= x;
    at += 4;
  }
  if (n & 2) {
    const uint64_t x = *reinterpret_cast<const u16_u*>(p + at);
    if (at < 8) lo |= x << (8 * at); else hi |= x << (8 * (at - 8));
    at += 2;
  }
  if (n & 1) {
    const uint64_t x = p[at];
    if (at < 8) lo |= x << (8 * at); else hi |= x << (8 * (at - 8));
  }
  return u32x4{uint32_t(lo), uint32_t(lo >> 32), uint32_t(hi), uint32_t(hi >> 32)};
}

// The len <= 16 bytes at global address lo of a run [base, base + n): bytes
// [0, len) of the result.  Reads stay inside the run: one 16-byte load when the
// run is at least 16 bytes long, else pieces of `unit` bytes.
__device__ __forceinline__ u32x4 load_in_run(uintptr_t base, uint32_t n, uintptr_t lo, uint32_t len,
                                             uint32_t unit) {
  if (n >= 16) {
    const uint32_t off = uint32_t(lo - base);
    const uint32_t at = off < n - 16 ? off : n - 16;
    u32x4 v = load_16_unaligned(base + at);
    return off > at ? shift_right_bytes(v, off - at) : v;
  }
  uint64_t w[2] = {0, 0};
  for (uint32_t b = 0; b < len; b += unit) {
    uint64_t x;
    if (unit >= 8) x = *as_global<const u64_u>(lo + b);
    else if (unit == 4) x = *as_global<const u32_u>(lo + b);
    else if (unit == 2) x = *as_global<const u16_u>(lo + b);
    else x = *as_global<const uint8_t>(lo + b);
    w[b / 8] |= x << (8 * (b % 8));
  }
  return u32x4{uint32_t(w[0]), uint32_t(w[0] >> 32), uint32_t(w[1]), uint32_t(w[1] >> 32)};
}

// Bytes [0, len) of v to global address d (len < 16: at most four stores), all
// streaming.
__device__ __forceinline__ void store_chunk(uintptr_t d, u32x4 v, uint32_t len) {
  if (len == 16) __builtin_nontemporal_store(v, as_global<u32x4_u>(d));
  else store_head_bytes(d, v, len);
}

// Where chunk j of a segment's tile lies.  Packed segments: one run of hr*w
// bytes at g.  Otherwise row r of the tile starts at g + r*stride and has
// chunks_per_row chunk slots.
struct SegChunk {
  uintptr_t lo;      // first global byte (replica-0 address for destinations)
  uint32_t len;      // bytes, 0 if the slot is empty
  uint32_t run_off;  // packed: offset of lo in the run; else offset of lo in its row
  uint32_t row;      // row of lo inside the tile
  uintptr_t base;    // start of the run (packed) or of the row
  uint32_t n;        // bytes of the run (packed) or of the row
};

__device__ __forceinline__ SegChunk seg_chunk(uintptr_t g, uint64_t stride, uint32_t w, uint32_t hr,
                                              bool packed, uint32_t chunks_per_row, uint32_t j) {
  SegChunk c;
  if (packed) {
    c.base = g;
    c.n = hr * w;
    c.row = 0;
  } else {
    c.row = j / chunks_per_row;
    j -= c.row * chunks_per_row;
    c.base = g + c.row * stride;
    c.n = w;
  }
  const uintptr_t block = (c.base & ~uintptr_t(15)) + uintptr_t(j) * 16;
  const uintptr_t lo = block > c.base ? block : c.base;
  const uintptr_t end = c.base + c.n;
  const uintptr_t hi = block + 16 < end ? block + 16 : end;
  c.lo = lo;
  c.len = hi > lo ? uint32_t(hi - lo) : 0u;
  c.run_off = uint32_t(lo - c.base);
  return c;
}

__device__ __forceinline__ uint32_t seg_chunks(uintptr_t g, uint32_t w, uint32_t hr, bool packed,
                                               uint32_t* chunks_per_row) {
  *chunks_per_row = (w + 30) / 16;
  if (packed) return uint32_t(((g & 15) + uint64_t(hr) * w + 15) / 16);
  return hr * *chunks_per_row;
}

// LDS address of byte `off` of a packed run (rows of w bytes, window column col).
__device__ __forceinline__ uint8_t* run_lds(uint8_t* lds, uint32_t pitch, uint32_t col, uint32_t w,
                                           uint32_t off) {
  const uint32_t r = off / w;
  return lds + r * pitch + col + (off - r * w);
}

constexpr int kWindowBatch = 4;  // chunks per thread with loads in flight together

template <class Sh>
__device__ __forceinline__ void window_tile(const reshard_descriptor_t& D, const reshard_segment_t* __restrict__ segs,
                            const uint32_t* __restrict__ refs, const Sh& sh, uint32_t tile,
                            uint8_t* lds) {
  const uint32_t rows = D.extent[0], per_tile = D.extent[1], pitch = D.row_items;
  const uint32_t r0 = tile * per_tile;
  const uint32_t hr = min(per_tile, rows - r0);
  const uint32_t unit = D.unit;
  const reshard_segment_t* src_segs = segs + D.src_ptr;
  const reshard_segment_t* dst_segs = src_segs + D.dst_ref_begin;

  // phase 1: source segments -> window
  for (uint32_t s = 0; s < D.dst_ref_begin; ++s) {
    const reshard_segment_t S = src_segs[s];
    const uintptr_t g = sh.ptr(S.ptr) + uint64_t(S.offset) + uint64_t(r0) * uint64_t(S.row_stride);
    const bool packed = uint64_t(S.row_stride) == S.width;
    uint32_t cpr;
    const uint32_t n = seg_chunks(g, S.width, hr, packed, &cpr);
    for (uint32_t base = 0; base < n; base += kBlock * kWindowBatch) {
      u32x4 v[kWindowBatch];
      SegChunk c[kWindowBatch];
#pragma unroll
      for (int k = 0; k < kWindowBatch; ++k) {
        const uint32_t j = base + uint32_t(k * kBlock) + threadIdx.x;
        c[k] = seg_chunk(g, uint64_t(S.row_stride), S.width, hr, packed, cpr, j < n ? j : 0);
        if (j >= n) c[k].len = 0;
        if (c[k].len) v[k] = load_in_run(c[k].base, c[k].n, c[k].lo, c[k].len, unit);
      }
#pragma unroll
      for (int k = 0; k < kWindowBatch; ++k) {
        if (!c[k].len) continue;
        if (!packed) {
          lds_put(lds + c[k].row * pitch + S.col + c[k].run_off, v[k], c[k].len);
          continue;
        }
        // a packed chunk may cover several window rows
        uint32_t off = c[k].run_off, left = c[k].len;
        u32x4 x = v[k];
        while (left) {
          const uint32_t in_row = S.width - off % S.width;
          const uint32_t take = left < in_row ? left : in_row;
          lds_put(run_lds(lds, pitch, S.col, S.width, off), x, take);
          left -= take;
          off += take;
          if (left) x = shift_right_bytes(x, take);
        }
      }
    }
  }
  __syncthreads();

  // phase 2: window -> destination segments, every replica
  for (uint32_t s = 0; s < D.fanout; ++s) {
    const reshard_segment_t S = dst_segs[s];
    const uint64_t row_off = uint64_t(S.offset) + uint64_t(r0) * uint64_t(S.row_stride);
    const uintptr_t g = sh.ptr(refs[S.ptr]) + row_off;
    const bool packed = uint64_t(S.row_stride) == S.width;
    uint32_t cpr;
    const uint32_t n = seg_chunks(g, S.width, hr, packed, &cpr);
    for (uint32_t j = threadIdx.x; j < n; j += kBlock) {
      const SegChunk c = seg_chunk(g, uint64_t(S.row_stride), S.width, hr, packed, cpr, j);
      if (!c.len) continue;
      u32x4 v;
      if (!packed) {
        v = lds_get(lds + c.row * pitch + S.col + c.run_off, c.len);
      } else {
        uint32_t off = c.run_off, got = 0;
        v = u32x4{0, 0, 0, 0};
        while (got < c.len) {
          const uint32_t in_row = S.width - off % S.width;
          const uint32_t take = c.len - got < in_row ? c.len - got : in_row;
          const u32x4 part = lds_get(run_lds(lds, pitch, S.col, S.width, off), take);
          const u32x4 sh_part = shift_left_bytes(part, got);
          v = u32x4{v.x | sh_part.x, v.y | sh_part.y, v.z | sh_part.z, v.w | sh_part.w};
          got += take;
          off += take;
        }
      }
      for (uint32_t r = 0; r < S.fanout; ++r) {
        const uintptr_t d = sh.ptr(refs[S.ptr + r]) + row_off + (c.lo - g);
        store_chunk(d, v, c.len);
      }
    }
  }
}

// n <= 16 bytes from global address a into bytes [0, n) of the result (any
// alignment: gfx950 global accesses need none).  Streaming (non-temporal).
__device__ __forceinline__ u32x4 load_bytes(uintptr_t a, uint32_t n) {
  if (n == 16) return load_16_unaligned(a);
  uint64_t lo = 0, hi = 0;
  uint32_t at = 0;
  if (n & 8) {
    lo = __builtin_nontemporal_load(as_global<const u64_u>(a));
    at = 8;
  }
  if (n & 4) {
    const uint64_t x = __builtin_nontemporal_load(as_global<const u32_u>(a + at));
    if (at < 8) lo |= x << (8 * at); else hi |= x;
    at += 4;
  }
  if (n & 2) {
    const uint64_t x = *as_global<const u16_u>(a + at);
    if (at < 8) lo |= x << (8 * at); else hi |= x << (8 * (at - 8));
    at += 2;
  }
  if (n & 1) {
    const uint64_t x = *as_global<const uint8_t>(a + at);
    if (at < 8) lo |= x << (8 * at); else hi |= x << (8 * (at - 8));
  }
  return u32x4{uint32_t(lo), uint32_t(lo >> 32), uint32_t(hi), uint32_t(hi >> 32)};
}

// Bytes [0, n) of v (n <= 16) to global address d, streaming stores for the
// whole-word widths, at most four stores otherwise.
__device__ __forceinline__ void store_bytes(uintptr_t d, u32x4 v, uint32_t n) {
  if (n == 16) __builtin_nontemporal_store(v, as_global<u32x4_u>(d));
  else if (n == 8) __builtin_nontemporal_store((uint64_t(v.y) << 32) | v.x, as_global<u64_u>(d));
  else if (n == 4) __builtin_nontemporal_store(v.x, as_global<u32_u>(d));
  else store_head_bytes(d, v, n);
}

// Narrow bands: a WINDOW band whose segments all hold their rows back to back
// in their shards (row stride = width), more than 16 bytes wide, or at most 16
// with a segment of one or two bytes, or of 12-byte rows of dword segments
// (narrow_band on the host has the details).  Every side is
// then a contiguous stream of bytes: stream byte j of a segment w bytes wide is
// row j / w, byte j % w of the segment.  The window keeps rows at a pitch of P
// bytes: an odd number of dwords when the band width W is a multiple of 4 (lanes
// that touch one column of consecutive rows, or consecutive dwords of one row,
// then hit distinct LDS banks), W otherwise (a segment of whole rows is then the
// window itself).  The window is dynamic LDS, sized at launch for the launch's
// largest band: kNarrowWindowBytes, or kNarrowBigWindowBytes for bands with
// small destination pieces (checked on the host).  Each segment
// moves in one of five ways:
//   dwords  P, column and width multiples of 4: a lane moves one dword of the
//           stream, or four where they stay together in the window;
//   whole   the whole row, P = W: 16-byte pieces of the stream are 16-byte
//           pieces of the window;
//   rows    4, 8 or 16 bytes wide (or 1 or 2: thin_run): a lane moves one row;
//   bytes   another width below 16: on the source side a lane moves a
//           16-byte piece of the stream byte by byte (one global access
//           instead of two or more a row); on the destination side, one row
//           a lane as for rows;
//   pieces  wider: a lane moves a 16-byte piece of the stream, which meets at
//           most two rows.
using rs::kNarrowWindowBytes;
using rs::narrow_pitch;
constexpr uint32_t kNarrowWindowWords = kNarrowWindowBytes / 4;
constexpr int kNarrowBatch = 4;  // dword pieces per lane with loads in flight together
constexpr int kBytesBatch = 2;   // other pieces
// (the segment classes kSeg* and narrow_class sit with the planner, which
// checks and sizes the bands)

// 2^32 / d rounded up, for div_small by d (its unit: dwords for a dword segment,
// bytes otherwise); 0 for d = 1.
__device__ __forceinline__ uint32_t narrow_magic(uint32_t wb, uint32_t cb, uint32_t P, uint32_t W) {
  const uint32_t d = narrow_class(wb, cb, P, W) == kSegDwords ? wb / 4 : wb;
  return d > 1 ? 0xffffffffu / d + 1u : 0u;
}

// n / w for n < 2^16 and 1 <= w < 2^16, with m = 2^32 / w rounded up (w > 1).
__device__ __forceinline__ uint32_t div_small(uint32_t n, uint32_t w, uint32_t m) {
  return w == 1 ? n : __umulhi(n, m);
}

// Whether four consecutive stream dwords of a segment (from a multiple of 4)
// stay consecutive in the window: the segment is a whole number of 16 bytes
// wide, or it is the whole row and the pitch adds no padding (odd width).
__device__ __forceinline__ bool dword_quads(uint32_t w, uint32_t c, uint32_t pitch) {
  return (w & 3u) == 0 || (c == 0 && w == pitch);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, uint32_t lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(v), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(v >> 32), lane);
  return uint64_t(lo) | (uint64_t(hi) << 32);
}

// Lane `lane`'s value of v (a per-lane value; lane may differ between lanes).
__device__ __forceinline__ uint32_t lane_value(uint32_t v, uint32_t lane) {
  return uint32_t(__builtin_amdgcn_ds_bpermute(int(lane * 4), int(v)));
}
__device__ __forceinline__ uint64_t lane_value64(uint64_t v, uint32_t lane) {
  return uint64_t(lane_value(uint32_t(v), lane)) | (uint64_t(lane_value(uint32_t(v >> 32), lane)) << 32);
}

// v rotated toward higher bytes by s (0 <= s < 16): byte i of the result is
// byte (i - s) mod 16 of v.  Four selects a stage, s may differ between lanes.
__device__ __forceinline__ u32x4 rotate_bytes(u32x4 v, uint32_t s) {
  u32x4 t = u32x4{(v.x << 8) | (v.w >> 24), (v.y << 8) | (v.x >> 24), (v.z << 8) | (v.y >> 24),
                  (v.w << 8) | (v.z >> 24)};
  v = (s & 1) ? t : v;
  t = u32x4{(v.x << 16) | (v.w >> 16), (v.y << 16) | (v.x >> 16), (v.z << 16) | (v.y >> 16), (v.w << 16) | (v.z >> 16)};
  v = (s & 2) ? t : v;
  t = u32x4{v.w, v.x, v.y, v.z};
  v = (s & 4) ? t : v;
  t = u32x4{v.z, v.w, v.x, v.y};
  return (s & 8) ? t : v;
}

// A run of m thin segments (kWb = 1 or 2 bytes wide, columns cb0, cb0 + kWb,
// ..., the same fan-out) of one side of a narrow band, for one tile of hr rows.
// A lane moves 8 consecutive rows of one segment, 8 kWb contiguous bytes of
// its stream, in one global access; the (segment, piece) pairs of the run are
// spread over the whole workgroup, and a lane finds its segment's address in
// the lane holding that segment (lane_addr: segment s in lane s).  The rows'
// LDS accesses go in an order rotated per lane so that the lanes of one access
// touch distinct banks (at 32 or 64 banks of 4 bytes and an odd dword pitch);
// the piece's bytes are rotated to match.  Rows past the last whole piece go
// one row a lane.  kIn: source side (stream -> window), else destination side
// (window -> stream, to every replica).
template <uint32_t kWb, bool kIn, class Sh>
__device__ __forceinline__ void thin_run(uint32_t s0, uint32_t m, uint32_t cb0, uint32_t fan, uint64_t lane_addr,
                                         uint64_t lane_off, uint32_t lane_ref, const uint32_t* __restrict__ refs,
                                         const Sh& sh, uint32_t hr, uint32_t P, uint8_t* lds) {
  constexpr uint32_t k = 8, kBytes = 8 * kWb;  // rows and bytes per piece
  const uint32_t nq = hr / k, tail = hr - nq * k;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x - lane);  // the wave's first thread
  const uint32_t rot = ((lane >> 2) ^ (lane >> 5)) & (k - 1);
  const uint32_t mq = nq > 1 ? 0xffffffffu / nq + 1u : 0u;
  // The trip counts are the same for every lane of a wave, and a lane past the
  // last item repeats it: every lane takes part in the lane lookups, whose
  // source lane must be active.
  const uint32_t items = m * nq;
  for (uint32_t base = wave0; base < items; base += kBlock) {
    const uint32_t i = base + lane, ic = min(i, items - 1);
    const uint32_t seg = nq == 1 ? ic : div_small(ic, nq, mq), q = ic - seg * nq;
    const uint64_t g = lane_value64(lane_addr, s0 + seg) + kBytes * uint64_t(q);
    const uint64_t o = !kIn && fan > 1 ? lane_value64(lane_off, s0 + seg) + kBytes * uint64_t(q) : 0u;
    const uint32_t ref = !kIn && fan > 1 ? lane_value(lane_ref, s0 + seg) : 0u;
    if (i >= items) continue;
    uint8_t* p = lds + q * k * P + cb0 + seg * kWb;
    if constexpr (kIn) {
      // slot j of the rotated piece is row (j + rot) mod 8
      uint32_t w[4];
      if constexpr (kWb == 2) {
        const u32x4 v = rotate_bytes(load_16_unaligned(g), (16 - 2 * rot) & 15u);
        w[0] = v.x, w[1] = v.y, w[2] = v.z, w[3] = v.w;
      } else {
        const uint64_t x = __builtin_nontemporal_load(as_global<const u64_u>(g));
        const uint64_t y = rot ? (x >> (8 * rot)) | (x << (64 - 8 * rot)) : x;
        w[0] = uint32_t(y), w[1] = uint32_t(y >> 32);
      }
#pragma unroll
      for (uint32_t j = 0; j < k; ++j) {
        uint8_t* at = p + ((j + rot) & (k - 1)) * P;
        if constexpr (kWb == 2) *reinterpret_cast<u16_u*>(at) = uint16_t(w[j / 2] >> (16 * (j % 2)));
        else *at = uint8_t(w[j / 4] >> (8 * (j % 4)));
      }
    } else {
      uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
      for (uint32_t j = 0; j < k; ++j) {
        const uint8_t* at = p + ((j + rot) & (k - 1)) * P;
        if constexpr (kWb == 2) w[j / 2] |= uint32_t(*reinterpret_cast<const u16_u*>(at)) << (16 * (j % 2));
        else w[j / 4] |= uint32_t(*at) << (8 * (j % 4));
      }
      if constexpr (kWb == 2) {
        const u32x4 v = rotate_bytes(u32x4{w[0], w[1], w[2], w[3]}, 2 * rot);
        __builtin_nontemporal_store(v, as_global<u32x4_u>(g));
        for (uint32_t f = 1; f < fan; ++f) __builtin_nontemporal_store(v, as_global<u32x4_u>(sh.ptr(refs[ref + f]) + o));
      } else {
        const uint64_t x = uint64_t(w[0]) | (uint64_t(w[1]) << 32);
        const uint64_t v = rot ? (x << (8 * rot)) | (x >> (64 - 8 * rot)) : x;
        __builtin_nontemporal_store(v, as_global<u64_u>(g));
        for (uint32_t f = 1; f < fan; ++f) __builtin_nontemporal_store(v, as_global<u64_u>(sh.ptr(refs[ref + f]) + o));
      }
    }
  }
  if (tail == 0) return;
  const uint32_t mt = tail > 1 ? 0xffffffffu / tail + 1u : 0u;
  const uint32_t tail_items = m * tail;
  for (uint32_t base = wave0; base < tail_items; base += kBlock) {  // as above
    const uint32_t i = base + lane, ic = min(i, tail_items - 1);
    const uint32_t seg = div_small(ic, tail, mt), r = nq * k + (ic - seg * tail);
    const uint64_t o = uint64_t(r) * kWb;
    const uint64_t g = lane_value64(lane_addr, s0 + seg) + o;
    const uint64_t off = kIn ? 0u : lane_value64(lane_off, s0 + seg) + o;
    const uint32_t ref = kIn ? 0u : lane_value(lane_ref, s0 + seg);
    if (i >= tail_items) continue;
    uint8_t* p = lds + r * P + cb0 + seg * kWb;
    if constexpr (kIn) {
      if constexpr (kWb == 2) *reinterpret_cast<u16_u*>(p) = *as_global<const u16_u>(g);
      else *p = *as_global<const uint8_t>(g);
    } else {
      const uint32_t x = kWb == 2 ? uint32_t(*reinterpret_cast<const u16_u*>(p)) : uint32_t(*p);
      for (uint32_t f = 0; f < fan; ++f) {
        const uintptr_t d = f == 0 ? g : sh.ptr(refs[ref + f]) + off;
        if constexpr (kWb == 2) *as_global<u16_u>(d) = uint16_t(x);
        else *as_global<uint8_t>(d) = uint8_t(x);
      }
    }
  }
}

// The end of the run of thin segments that starts at segment s of one side
// (lane t of wc / fan holding segment t's width | column << 16 and fan-out):
// the following segments of the same width, the next columns, the same fan-out.
__device__ __forceinline__ uint32_t thin_run_end(uint32_t s, uint32_t n, uint32_t wc, uint32_t fan) {
  const uint32_t w0 = __builtin_amdgcn_readlane(wc, s);
  const uint32_t wb = w0 & 0xffffu, f0 = __builtin_amdgcn_readlane(fan, s);
  uint32_t e = s + 1;
  while (e < n && __builtin_amdgcn_readlane(wc, e) == w0 + ((e - s) * wb << 16) &&
         __builtin_amdgcn_readlane(fan, e) == f0)
    ++e;
  return e;
}

// Phase 1 of a narrow band for one dword source stream: loads into the window
// (w, c and pitch in dwords).
__device__ __forceinline__ void dword_stream_in(uintptr_t g, uint32_t w, uint32_t c, uint32_t m, uint32_t hr,
                                                uint32_t pitch, uint32_t* lds) {
  const uint32_t n = hr * w;
  uint32_t done = 0;  // stream dwords moved as quads
  if (dword_quads(w, c, pitch)) {
    const uint32_t nq = n / 4;
    for (uint32_t base = threadIdx.x; base < nq; base += kBlock * kNarrowBatch) {
      u32x4 v[kNarrowBatch];
#pragma unroll
      for (int k = 0; k < kNarrowBatch; ++k) {
        const uint32_t q = base + uint32_t(k) * kBlock;
        if (q < nq) v[k] = load_16_unaligned(g + 16 * uint64_t(q));
      }
#pragma unroll
      for (int k = 0; k < kNarrowBatch; ++k) {
        const uint32_t q = base + uint32_t(k) * kBlock;
        if (q >= nq) break;
        const uint32_t j = 4 * q, r = div_small(j, w, m);
        *reinterpret_cast<u32x4_u1*>(lds + r * pitch + c + (j - r * w)) = v[k];
      }
    }
    done = 4 * nq;
  } else {  // 16-byte loads too, their four dwords placed one by one (a row may end inside)
    const uint32_t nq = n / 4;
    for (uint32_t base = threadIdx.x; base < nq; base += kBlock * kNarrowBatch) {
      u32x4 v[kNarrowBatch];
#pragma unroll
      for (int k = 0; k < kNarrowBatch; ++k) {
        const uint32_t q = base + uint32_t(k) * kBlock;
        if (q < nq) v[k] = load_16_unaligned(g + 16 * uint64_t(q));
      }
#pragma unroll
      for (int k = 0; k < kNarrowBatch; ++k) {
        const uint32_t q = base + uint32_t(k) * kBlock;
        if (q >= nq) break;
        const uint32_t j = 4 * q, r = div_small(j, w, m);
        uint32_t col = j - r * w;
        uint32_t* a = lds + r * pitch + c + col;
        const uint32_t x[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {  // stream dword j + b: the next column, or the next row's first
          *a = x[b];
          ++a;
          if (++col == w) col = 0, a += pitch - w;
        }
      }
    }
    done = 4 * nq;
  }
  for (uint32_t base = done + threadIdx.x; base < n; base += kBlock * kNarrowBatch) {
    uint32_t v[kNarrowBatch];
#pragma unroll
    for (int k = 0; k < kNarrowBatch; ++k) {
      const uint32_t j = base + uint32_t(k) * kBlock;
      if (j < n) v[k] = __builtin_nontemporal_load(as_global<const u32_u>(g + 4 * uint64_t(j)));
    }
#pragma unroll
    for (int k = 0; k < kNarrowBatch; ++k) {
      const uint32_t j = base + uint32_t(k) * kBlock;
      if (j >= n) break;
      const uint32_t r = div_small(j, w, m);
      lds[r * pitch + c + (j - r * w)] = v[k];
    }
  }
}

// Phase 1 of a narrow band for one source stream of any other class (wb, cb
// and P in bytes).
__device__ __forceinline__ void bytes_stream_in(uintptr_t g, uint32_t wb, uint32_t cb, uint32_t m, uint32_t cls,
                                                uint32_t hr, uint32_t P, uint8_t* lds) {
  if (cls == kSegBytes) {
    const uint32_t nb = hr * wb;
    for (uint32_t base = threadIdx.x; 16 * base < nb; base += kBlock * kBytesBatch) {
      u32x4 v[kBytesBatch];
#pragma unroll
      for (int k = 0; k < kBytesBatch; ++k) {
        const uint32_t j = 16 * (base + uint32_t(k) * kBlock);
        if (j < nb) v[k] = load_bytes(g + j, min(16u, nb - j));
      }
#pragma unroll
      for (int k = 0; k < kBytesBatch; ++k) {
        const uint32_t j = 16 * (base + uint32_t(k) * kBlock);
        if (j >= nb) break;
        const uint32_t len = min(16u, nb - j);
        uint32_t r = div_small(j, wb, m), col = j - r * wb;
        uint8_t* a = lds + r * P + cb + col;
        const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (uint32_t b = 0; b < 16; ++b) {  // stream byte j + b: the next column, or the next row's first
          if (b < len) *a = uint8_t(w[b / 4] >> (8 * (b % 4)));
          ++col, ++a;
          if (col == wb) col = 0, a += P - wb;
        }
      }
    }
    return;
  }
  if (cls == kSegRows) {
    for (uint32_t base = threadIdx.x; base < hr; base += kBlock * kBytesBatch) {
      u32x4 v[kBytesBatch];
#pragma unroll
      for (int k = 0; k < kBytesBatch; ++k) {
        const uint32_t r = base + uint32_t(k) * kBlock;
        if (r < hr) v[k] = load_bytes(g + uint64_t(r) * wb, wb);
      }
#pragma unroll
      for (int k = 0; k < kBytesBatch; ++k) {
        const uint32_t r = base + uint32_t(k) * kBlock;
        if (r >= hr) break;
        lds_put(lds + r * P + cb, v[k], wb);
      }
    }
    return;
  }
  const uint32_t nb = hr * wb;
  for (uint32_t base = threadIdx.x; 16 * base < nb; base += kBlock * kBytesBatch) {
    u32x4 v[kBytesBatch];
#pragma unroll
    for (int k = 0; k < kBytesBatch; ++k) {
      const uint32_t j = 16 * (base + uint32_t(k) * kBlock);
      if (j < nb) v[k] = load_bytes(g + j, min(16u, nb - j));
    }
#pragma unroll
    for (int k = 0; k < kBytesBatch; ++k) {
      const uint32_t j = 16 * (base + uint32_t(k) * kBlock);
      if (j >= nb) break;
      const uint32_t len = min(16u, nb - j);
      if (cls == kSegWhole) {
        lds_put(lds + j, v[k], len);
        continue;
      }
      const uint32_t r = div_small(j, wb, m), col = j - r * wb;
      const uint32_t l1 = min(len, wb - col);
      lds_put(lds + r * P + cb + col, v[k], l1);
      if (len > l1) lds_put(lds + (r + 1) * P + cb, shift_right_bytes(v[k], l1), len - l1);
    }
  }
}

// Phase 2 of a narrow band for one destination stream that is not a dword
// stream: to g0 (first replica) and, at the same offset `off`, to the other
// replicas of fan-out list refs[ref ..].
template <class Sh>
__device__ __forceinline__ void bytes_stream_out(uintptr_t g0, uint64_t off, uint32_t ref, uint32_t fan,
                                                 const uint32_t* __restrict__ refs, const Sh& sh, uint32_t wb,
                                                 uint32_t cb, uint32_t m, uint32_t cls, uint32_t hr, uint32_t P,
                                                 const uint8_t* lds) {
  if (cls == kSegRows || cls == kSegBytes) {  // one row a lane (byte by byte measured no faster here)
    uint32_t first = 0;  // rows moved 16 stream bytes a lane
    if (wb == 4 || wb == 8) {  // 16 / wb rows a lane: one window access a row, one 16-byte store
      const uint32_t k = 16 / wb, nq = hr / k;
      for (uint32_t q = threadIdx.x; q < nq; q += kBlock) {
        const uint8_t* a = lds + q * k * P + cb;
        u32x4 v;
        if (wb == 8) {
          const u32x2_u1 x = *reinterpret_cast<const u32x2_u1*>(a), y = *reinterpret_cast<const u32x2_u1*>(a + P);
          v = u32x4{x.x, x.y, y.x, y.y};
        } else {
          v = u32x4{*reinterpret_cast<const u32_u*>(a), *reinterpret_cast<const u32_u*>(a + P),
                    *reinterpret_cast<const u32_u*>(a + 2 * P), *reinterpret_cast<const u32_u*>(a + 3 * P)};
        }
        const uint64_t o = 16 * uint64_t(q);
        __builtin_nontemporal_store(v, as_global<u32x4_u1>(g0 + o));
        for (uint32_t f = 1; f < fan; ++f) __builtin_nontemporal_store(v, as_global<u32x4_u1>(sh.ptr(refs[ref + f]) + off + o));
      }
      first = nq * k;
    }
    for (uint32_t r = first + threadIdx.x; r < hr; r += kBlock) {
      const u32x4 v = lds_get(lds + r * P + cb, wb);
      const uint64_t o = uint64_t(r) * wb;
      store_bytes(g0 + o, v, wb);
      for (uint32_t f = 1; f < fan; ++f) store_bytes(sh.ptr(refs[ref + f]) + off + o, v, wb);
    }
    return;
  }
  const uint32_t nb = hr * wb;
  for (uint32_t j = 16 * threadIdx.x; j < nb; j += 16 * kBlock) {
    const uint32_t len = min(16u, nb - j);
    u32x4 v;
    if (cls == kSegWhole) {
      v = lds_get(lds + j, len);
    } else {
      const uint32_t r = div_small(j, wb, m), col = j - r * wb;
      const uint32_t l1 = min(len, wb - col);
      v = lds_get(lds + r * P + cb + col, l1);
      if (len > l1) {
        const u32x4 x = shift_left_bytes(lds_get(lds + (r + 1) * P + cb, len - l1), l1);
        v = u32x4{v.x | x.x, v.y | x.y, v.z | x.z, v.w | x.w};
      }
    }
    store_bytes(g0 + j, v, len);
    for (uint32_t f = 1; f < fan; ++f) store_bytes(sh.ptr(refs[ref + f]) + off + j, v, len);
  }
}

// kBytes: the build for bands with segments of every class; without it, every
// segment of every band is a dword segment (checked on the host), and only the
// dword paths are compiled.
template <bool kBytes, class Sh>
__device__ __forceinline__ void window_narrow(const reshard_descriptor_t& D, const reshard_segment_t* __restrict__ segs,
                                              const uint32_t* __restrict__ refs, const Sh& sh, uint32_t tile,
                                              uint32_t* lds) {
  const uint32_t rows = D.extent[0], per_tile = D.extent[1];
  const uint32_t r0 = tile * per_tile;
  const uint32_t hr = min(per_tile, rows - r0);
  const uint32_t W = D.run_bytes, P = narrow_pitch(W), pitch = P / 4;  // pitch: dwords, for dword segments
  uint8_t* lds8 = reinterpret_cast<uint8_t*>(lds);
  const uint32_t ns = D.dst_ref_begin, nd = D.fanout;  // at most 64 each
  const reshard_segment_t* src_segs = segs + D.src_ptr;
  const reshard_segment_t* dst_segs = src_segs + ns;
  // Every wave reads the destination segments once, lane s holding segment s
  // and its first replica's address (its slot sits in the segment's row_stride
  // in the device table), so that the loop of phase 2 takes them from
  // registers.  The loads go out first; phase 1 does not wait for them.
  // (Lanes past the last segment read segment 0 again.)
  const uint32_t lane = threadIdx.x & 63u;
  const reshard_segment_t SD = dst_segs[lane < nd ? lane : 0u];

  // phase 1: source streams -> window.  One source segment comes through the
  // scalar cache; several, one per lane as above.
  if (ns == 1) {
    const reshard_segment_t S = src_segs[0];
    const uintptr_t g = sh.ptr(S.ptr) + uint64_t(S.offset) + uint64_t(r0) * uint64_t(S.width);
    const uint32_t cls = narrow_class(S.width, S.col, P, W), m = narrow_magic(S.width, S.col, P, W);
    if (!kBytes || cls == kSegDwords) dword_stream_in(g, S.width / 4, S.col / 4, m, hr, pitch, lds);
    else bytes_stream_in(g, S.width, S.col, m, cls, hr, P, lds8);
  } else {
    const reshard_segment_t SS = src_segs[lane < ns ? lane : 0u];
    const uint32_t s_wc = SS.width | (SS.col << 16);  // width | col << 16 (bytes)
    const uint32_t s_m = narrow_magic(SS.width, SS.col, P, W);
    const uint64_t s_addr = sh.ptr(SS.ptr) + uint64_t(SS.offset) + uint64_t(r0) * uint64_t(SS.width);
    for (uint32_t s = 0; s < ns; ++s) {
      const uint32_t wc = __builtin_amdgcn_readlane(s_wc, s);
      const uint32_t wb = wc & 0xffffu, cb = wc >> 16, cls = narrow_class(wb, cb, P, W);
      if (kBytes && wb <= 2) {  // thin: a run of them together
        const uint32_t e = thin_run_end(s, ns, s_wc, 0u);
        if (wb == 2) thin_run<2, true>(s, e - s, cb, 1u, s_addr, 0u, 0u, refs, sh, hr, P, lds8);
        else thin_run<1, true>(s, e - s, cb, 1u, s_addr, 0u, 0u, refs, sh, hr, P, lds8);
        s = e - 1;
        continue;
      }
      const uint32_t m = __builtin_amdgcn_readlane(s_m, s);
      if (!kBytes || cls == kSegDwords) dword_stream_in(readlane64(s_addr, s), wb / 4, cb / 4, m, hr, pitch, lds);
      else bytes_stream_in(readlane64(s_addr, s), wb, cb, m, cls, hr, P, lds8);
    }
  }
  const uint32_t d_wc = SD.width | (SD.col << 16);  // bytes
  const uint32_t d_m = narrow_magic(SD.width, SD.col, P, W);
  const uint64_t d_off = uint64_t(SD.offset) + uint64_t(r0) * uint64_t(SD.width);
  const uint32_t d_ref = SD.ptr, d_fan = SD.fanout;
  const uint64_t d_addr = sh.ptr(uint32_t(SD.row_stride)) + d_off;
  __syncthreads();

  // phase 2: window -> destination streams, every replica.  A dword segment at
  // most four dwords wide goes row by row, one row a lane: one LDS read of the
  // row's dwords and one store of them (the lanes' stores are consecutive in
  // the stream); wider ones in stream order like phase 1.
  for (uint32_t s = 0; s < nd; ++s) {
    const uint32_t wc = __builtin_amdgcn_readlane(d_wc, s);
    const uint32_t wb = wc & 0xffffu, cb = wc >> 16;
    const uintptr_t g0 = readlane64(d_addr, s);
    const uint32_t fan = __builtin_amdgcn_readlane(d_fan, s);
    const uint32_t cls = narrow_class(wb, cb, P, W);
    if (kBytes && wb <= 2) {  // thin: a run of them together
      const uint32_t e = thin_run_end(s, nd, d_wc, d_fan);
      if (wb == 2) thin_run<2, false>(s, e - s, cb, fan, d_addr, d_off, d_ref, refs, sh, hr, P, lds8);
      else thin_run<1, false>(s, e - s, cb, fan, d_addr, d_off, d_ref, refs, sh, hr, P, lds8);
      s = e - 1;
      continue;
    }
    if (kBytes && cls != kSegDwords) {
      bytes_stream_out(g0, readlane64(d_off, s), __builtin_amdgcn_readlane(d_ref, s), fan, refs, sh, wb, cb,
                       __builtin_amdgcn_readlane(d_m, s), cls, hr, P, lds8);
      continue;
    }
    const uint32_t w = wb / 4, c = cb / 4, n = hr * w;
    // four one-dword segments side by side (columns c .. c + 3, one replica
    // each): one LDS read of the four dwords a row, four stores
    if (w == 1 && fan == 1 && s + 3 < nd) {
      const uint32_t wc3 = __builtin_amdgcn_readlane(d_wc, s + 3);
      const uint32_t f1 = __builtin_amdgcn_readlane(d_fan, s + 1), f2 = __builtin_amdgcn_readlane(d_fan, s + 2),
                     f3 = __builtin_amdgcn_readlane(d_fan, s + 3);
      if (wc3 == (4u | ((cb + 12) << 16)) && __builtin_amdgcn_readlane(d_wc, s + 1) == (4u | ((cb + 4) << 16)) &&
          __builtin_amdgcn_readlane(d_wc, s + 2) == (4u | ((cb + 8) << 16)) && (f1 & f2 & f3) == 1) {
        const uintptr_t g1 = readlane64(d_addr, s + 1), g2 = readlane64(d_addr, s + 2),
                        g3 = readlane64(d_addr, s + 3);
        for (uint32_t r = threadIdx.x; r < hr; r += kBlock) {
          const u32x4 v = *reinterpret_cast<const u32x4_u1*>(lds + r * pitch + c);
          const uint64_t o = 4 * uint64_t(r);
          __builtin_nontemporal_store(v.x, as_global<u32_u>(g0 + o));
          __builtin_nontemporal_store(v.y, as_global<u32_u>(g1 + o));
          __builtin_nontemporal_store(v.z, as_global<u32_u>(g2 + o));
          __builtin_nontemporal_store(v.w, as_global<u32_u>(g3 + o));
        }
        s += 3;
        continue;
      }
    }
    // two two-dword segments side by side (8-byte runs): one LDS read of the
    // four dwords a row, two stores
    if (w == 2 && fan == 1 && s + 1 < nd && __builtin_amdgcn_readlane(d_wc, s + 1) == (8u | ((cb + 8) << 16)) &&
        __builtin_amdgcn_readlane(d_fan, s + 1) == 1) {
      const uintptr_t g1 = readlane64(d_addr, s + 1);
      for (uint32_t r = threadIdx.x; r < hr; r += kBlock) {
        const u32x4 v = *reinterpret_cast<const u32x4_u1*>(lds + r * pitch + c);
        const uint64_t o = 8 * uint64_t(r);
        __builtin_nontemporal_store(u32x2_u1{v.x, v.y}, as_global<u32x2_u1>(g0 + o));
        __builtin_nontemporal_store(u32x2_u1{v.z, v.w}, as_global<u32x2_u1>(g1 + o));
      }
      s += 1;
      continue;
    }
    if (w <= 4 && fan == 1) {
      for (uint32_t r = threadIdx.x; r < hr; r += kBlock) {
        const uint32_t* src = lds + r * pitch + c;
        const uintptr_t d = g0 + uint64_t(r) * (4 * w);
        switch (w) {
          case 1: __builtin_nontemporal_store(src[0], as_global<u32_u>(d)); break;
          case 2: __builtin_nontemporal_store(*reinterpret_cast<const u32x2_u1*>(src), as_global<u32x2_u1>(d)); break;
          case 3: {
            const u32x2_u1 a = *reinterpret_cast<const u32x2_u1*>(src);
            __builtin_nontemporal_store(a, as_global<u32x2_u1>(d));
            __builtin_nontemporal_store(src[2], as_global<u32_u>(d + 8));
            break;
          }
          default: __builtin_nontemporal_store(*reinterpret_cast<const u32x4_u1*>(src), as_global<u32x4_u1>(d));
        }
      }
      continue;
    }
    const uint32_t m = __builtin_amdgcn_readlane(d_m, s);
    const uint32_t ref = __builtin_amdgcn_readlane(d_ref, s);
    const uint64_t off = readlane64(d_off, s);
    uint32_t done = 0;
    if (dword_quads(w, c, pitch)) {
      const uint32_t nq = n / 4;
      for (uint32_t q = threadIdx.x; q < nq; q += kBlock) {
        const uint32_t j = 4 * q, r = div_small(j, w, m);
        const u32x4 v = *reinterpret_cast<const u32x4_u1*>(lds + r * pitch + c + (j - r * w));
        __builtin_nontemporal_store(v, as_global<u32x4_u1>(g0 + 16 * uint64_t(q)));
        for (uint32_t f = 1; f < fan; ++f)
          __builtin_nontemporal_store(v, as_global<u32x4_u1>(sh.ptr(refs[ref + f]) + off + 16 * uint64_t(q)));
      }
      done = 4 * nq;
    } else {  // 16-byte stores too, their four dwords read one by one (a row may end inside)
      const uint32_t nq = n / 4;
      for (uint32_t q = threadIdx.x; q < nq; q += kBlock) {
        const uint32_t j = 4 * q, r = div_small(j, w, m);
        uint32_t col = j - r * w;
        const uint32_t* a = lds + r * pitch + c + col;
        uint32_t x[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          x[b] = *a;
          ++a;
          if (++col == w) col = 0, a += pitch - w;
        }
        const u32x4 v = u32x4{x[0], x[1], x[2], x[3]};
        __builtin_nontemporal_store(v, as_global<u32x4_u1>(g0 + 16 * uint64_t(q)));
        for (uint32_t f = 1; f < fan; ++f)
          __builtin_nontemporal_store(v, as_global<u32x4_u1>(sh.ptr(refs[ref + f]) + off + 16 * uint64_t(q)));
      }
      done = 4 * nq;
    }
    for (uint32_t j = done + threadIdx.x; j < n; j += kBlock) {
      const uint32_t r = div_small(j, w, m);
      const uint32_t v = lds[r * pitch + c + (j - r * w)];
      __builtin_nontemporal_store(v, as_global<u32_u>(g0 + 4 * uint64_t(j)));
      for (uint32_t f = 1; f < fan; ++f)
        __builtin_nontemporal_store(v, as_global<u32_u>(sh.ptr(refs[ref + f]) + off + 4 * uint64_t(j)));
    }
  }
}

// 4x4 transpose of 32-bit words across the four lanes of each quad: with row i
// of a 4x4 matrix in lane i of the quad, lane j ends with column j.  Two
// exchanges with DPP quad permutations: the off-diagonal words of each 2x2
// block with the neighbour lane (quad_perm 1,0,3,2), then the off-diagonal 2x2
// blocks with the lane two away (quad_perm 2,3,0,1).  Every lane of the wave
// must be active.
__device__ __forceinline__ u32x4 quad_transpose(u32x4 v) {
  const uint32_t j = threadIdx.x & 3u;
  uint32_t m[4] = {v.x, v.y, v.z, v.w};
  const bool odd = (j & 1u) != 0, upper = (j & 2u) != 0;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint32_t x = odd ? m[2 * b] : m[2 * b + 1];
    const uint32_t y = uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0xB1, 0xF, 0xF, false));
    if (odd) m[2 * b] = y;
    else m[2 * b + 1] = y;
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint32_t x = upper ? m[c] : m[2 + c];
    const uint32_t y = uint32_t(__builtin_amdgcn_mov_dpp(int(x), 0x4E, 0xF, 0xF, false));
    if (upper) m[c] = y;
    else m[2 + c] = y;
  }
  return u32x4{m[0], m[1], m[2], m[3]};
}

// Whether segments [0, n) of a 16-byte band are four packed 4-byte column runs
// (the band's row split into four 4-byte pieces, each stored contiguously) with
// one fan-out: then four consecutive rows of one segment are 16 contiguous bytes.
__device__ __forceinline__ bool quad_segments(const reshard_segment_t* __restrict__ S, uint32_t n,
                                              uint32_t* fanout) {
  if (n != 4) return false;
  // every field is read and the tests are combined with &, not &&: a
  // short-circuit chain makes each load wait for the previous test (a dozen
  // dependent scalar round trips at the start of every tile)
  bool ok = true;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    ok &= (S[s].width == 4u) & (S[s].row_stride == 4) & (S[s].fanout == S[0].fanout);
  *fanout = S[0].fanout;
  return ok;
}

// Base address (tile row 0) of the segment at column 4 * (lane & 3) of a quad
// band, replica f (source segments: f = 0 and fan-out 0).
template <class Sh>
__device__ __forceinline__ uintptr_t quad_base(const reshard_segment_t* __restrict__ S,
                                               const uint32_t* __restrict__ refs, const Sh& sh, uint32_t r0,
                                               bool dst, uint32_t f) {
  const uint32_t want = 4u * (threadIdx.x & 3u);
  uintptr_t base = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uintptr_t p = (dst ? sh.ptr(refs[S[s].ptr + f]) : sh.ptr(S[s].ptr)) + uint64_t(S[s].offset) +
                        uint64_t(r0) * 4u;
    base = S[s].col == want ? p : base;
  }
  return base;
}

// A window band at most 16 bytes wide, without LDS: each lane owns rows
// r = k * kBlock + lane of the tile, builds each row in one 16-byte register
// from every source segment (shifted to its column), then writes each
// destination segment's bytes of it to every replica.  Consecutive lanes touch
// consecutive rows, so packed segments give contiguous wave accesses.  When a
// 16-byte band is cut into four packed 4-byte column runs (a bf16 pair or an
// fp32 column per shard) on one side, the four lanes of a quad exchange words
// (quad_transpose): a lane then moves four consecutive rows of one run, 16
// contiguous bytes, in one access instead of four.
template <int kRows, class Sh>
__device__ __forceinline__ void window_rows(const reshard_descriptor_t& D, const reshard_segment_t* __restrict__ segs,
                            const uint32_t* __restrict__ refs, const Sh& sh, uint32_t tile) {
  const uint32_t rows = D.extent[0], per_tile = D.extent[1];
  const uint32_t r0 = tile * per_tile;
  const uint32_t hr = min(per_tile, rows - r0);
  const reshard_segment_t* src_segs = segs + D.src_ptr;
  const reshard_segment_t* dst_segs = src_segs + D.dst_ref_begin;
  const uint32_t quad_row = threadIdx.x & ~3u;  // first of the quad's rows (plus k * kBlock)
  const uint32_t used = (hr + kBlock - 1) / kBlock;  // row slots k of this tile that hold rows
  const bool wide = D.run_bytes == 16u;
  u32x4 v[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k) v[k] = u32x4{0, 0, 0, 0};
  uint32_t src_fan;
  if (wide && quad_segments(src_segs, D.dst_ref_begin, &src_fan)) {
    // lane j loads four rows of the run at column 4j, then the quad transposes
    const uintptr_t g = quad_base(src_segs, refs, sh, r0, false, 0);
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const uint32_t r = uint32_t(k * kBlock) + quad_row;
      if (uint32_t(k) >= used) continue;
      if (r + 4 <= hr) {
        v[k] = load_16_unaligned(g + uint64_t(r) * 4u);
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i)
          if (r + i < hr) w[i] = __builtin_nontemporal_load(as_global<const u32_u>(g + uint64_t(r + i) * 4u));
        v[k] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
#pragma unroll
    for (int k = 0; k < kRows; ++k)
      if (uint32_t(k) < used) v[k] = quad_transpose(v[k]);  // uniform: every lane takes part
  } else {
    // every slot's load is issued before any is used (a load under a per-lane
    // test would wait for the one before it): slots past the tile read its
    // last row again, in bounds, and drop it
    uint32_t rr[kRows];
#pragma unroll
    for (int k = 0; k < kRows; ++k) rr[k] = min(uint32_t(k * kBlock) + threadIdx.x, hr - 1);
    for (uint32_t s = 0; s < D.dst_ref_begin; ++s) {
      const reshard_segment_t S = src_segs[s];
      const uintptr_t g = sh.ptr(S.ptr) + uint64_t(S.offset) + uint64_t(r0) * uint64_t(S.row_stride);
      u32x4 x[kRows];
      if (S.width == 16u) {  // uniform: whole 16-byte rows
#pragma unroll
        for (int k = 0; k < kRows; ++k) x[k] = load_16_unaligned(g + uint64_t(rr[k]) * uint64_t(S.row_stride));
      } else {
#pragma unroll
        for (int k = 0; k < kRows; ++k) x[k] = load_bytes(g + uint64_t(rr[k]) * uint64_t(S.row_stride), S.width);
      }
#pragma unroll
      for (int k = 0; k < kRows; ++k) {
        const u32x4 y = shift_left_bytes(x[k], S.col);
        v[k] = u32x4{v[k].x | y.x, v[k].y | y.y, v[k].z | y.z, v[k].w | y.w};
      }
    }
  }
  uint32_t dst_fan;
  if (wide && quad_segments(dst_segs, D.fanout, &dst_fan)) {
    // the quad transposes, then lane j stores four rows of the run at column 4j
#pragma unroll
    for (int k = 0; k < kRows; ++k)
      if (uint32_t(k) < used) v[k] = quad_transpose(v[k]);  // uniform: every lane takes part
    for (uint32_t f = 0; f < dst_fan; ++f) {
      const uintptr_t g = quad_base(dst_segs, refs, sh, r0, true, f);
#pragma unroll
      for (int k = 0; k < kRows; ++k) {
        const uint32_t r = uint32_t(k * kBlock) + quad_row;
        if (uint32_t(k) >= used) continue;
        if (r + 4 <= hr) {
          store_bytes(g + uint64_t(r) * 4u, v[k], 16);
        } else {
          const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
          for (uint32_t i = 0; i < 4; ++i)
            if (r + i < hr) __builtin_nontemporal_store(w[i], as_global<u32_u>(g + uint64_t(r + i) * 4u));
        }
      }
    }
    return;
  }
  for (uint32_t s = 0; s < D.fanout; ++s) {
    const reshard_segment_t S = dst_segs[s];
    const uint64_t row_off = uint64_t(S.offset) + uint64_t(r0) * uint64_t(S.row_stride);
    u32x4 x[kRows];
#pragma unroll
    for (int k = 0; k < kRows; ++k) x[k] = S.col == 0 ? v[k] : shift_right_bytes(v[k], S.col);
    for (uint32_t f = 0; f < S.fanout; ++f) {
      const uintptr_t g = sh.ptr(refs[S.ptr + f]) + row_off;
#pragma unroll
      for (int k = 0; k < kRows; ++k) {
        const uint32_t r = uint32_t(k * kBlock) + threadIdx.x;
        if (r < hr) store_bytes(g + uint64_t(r) * uint64_t(S.row_stride), x[k], S.width);
      }
    }
  }
}

// The value of v held by lane (this lane) ^ X, for X = 1, 2 (DPP quad
// permutations) and X = 4, 8 (LDS-crossbar swizzle, bit mode: and-mask 0x1f,
// xor-mask X).  Every lane of the wave must be active.
template <int X>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (X == 1) return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xB1, 0xF, 0xF, false));
  else if constexpr (X == 2) return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x4E, 0xF, 0xF, false));
  else return uint32_t(__builtin_amdgcn_ds_swizzle(int(v), 0x1F | (X << 10)));
}

// Whether segments [0, n) of a band side are one packed run of the whole row
// of w bytes (runs_side, with the planner, tells K packed column runs).
// Host-side checks: in a plan that runs a band kernel every descriptor passed
// them, so on the device a side's segment count tells the two apart (K
// segments: runs, one: whole rows).
inline bool full_side(const reshard_segment_t* S, uint32_t n, uint32_t w) {
  return n == 1 && S[0].width == w && uint64_t(S[0].row_stride) == w;
}

// A 16-byte window band whose one side is eight packed 2-byte column runs (one
// bf16 or fp16 column per shard over eight shards) and whose other side is one
// packed run of whole rows.  No LDS: each lane holds one 16-byte row per slot
// (row k * kBlock + lane), and an 8 x 8 transpose of halfwords across each group
// of eight lanes leaves lane j of group G with run j at rows 8G .. 8G + 7 (16
// contiguous bytes; the eight lanes that hold run j cover 128 contiguous bytes
// in one access).  Transpose stages: lanes 1 apart trade halfwords (bit 0 of
// the element index), lanes 2 and 4 apart whole words (bits 1 and 2).
__device__ __forceinline__ u32x4 octet_transpose(u32x4 v) {
  const bool odd = (threadIdx.x & 1u) != 0, b1 = (threadIdx.x & 2u) != 0, b2 = (threadIdx.x & 4u) != 0;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // an odd lane's low halves for the even partner's high halves
    const uint32_t got = lane_xor<1>(odd ? (w[i] & 0xffffu) : (w[i] >> 16));
    w[i] = odd ? ((w[i] & 0xffff0000u) | got) : ((w[i] & 0xffffu) | (got << 16));
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {  // words 2p and 2p + 1 against lanes 2 apart
    const uint32_t lo = w[2 * p], up = w[2 * p + 1];
    const uint32_t got = lane_xor<2>(b1 ? lo : up);
    w[2 * p] = b1 ? got : lo;
    w[2 * p + 1] = b1 ? up : got;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {  // words p and p + 2 against lanes 4 apart
    const uint32_t lo = w[p], up = w[p + 2];
    const uint32_t got = lane_xor<4>(b2 ? lo : up);
    w[p] = b2 ? got : lo;
    w[p + 2] = b2 ? up : got;
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

template <class Sh>
__device__ __forceinline__ void window_octets(const reshard_descriptor_t& D,
                                              const reshard_segment_t* __restrict__ segs,
                                              const uint32_t* __restrict__ refs, const Sh& sh, uint32_t tile) {
  constexpr int kRows = int(rs::kQuadRowsPerLane);
  const uint32_t rows = D.extent[0], per_tile = D.extent[1];  // kRows * kBlock rows per tile
  const uint32_t r0 = tile * per_tile;
  const uint32_t hr = min(per_tile, rows - r0);
  const reshard_segment_t* src_segs = segs + D.src_ptr;
  const reshard_segment_t* dst_segs = src_segs + D.dst_ref_begin;
  const bool src_runs = D.dst_ref_begin == 8;  // else one segment of whole rows (and eight runs out)
  const uint32_t j = threadIdx.x & 7u, group_row = threadIdx.x & ~7u;
  u32x4 v[kRows];
  if (src_runs) {  // lane j loads eight rows of run j, then the group transposes
    const reshard_segment_t& seg = src_segs[j];
    const uintptr_t g = sh.ptr(seg.ptr) + uint64_t(seg.offset) + uint64_t(r0) * 2u;
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const uint32_t r = uint32_t(k * kBlock) + group_row;
      if (r + 8 <= hr) {
        v[k] = load_16_unaligned(g + uint64_t(r) * 2u);
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i)
          if (r + i < hr) w[i / 2] |= uint32_t(*as_global<const u16_u>(g + uint64_t(r + i) * 2u)) << (16 * (i & 1));
        v[k] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
#pragma unroll
    for (int k = 0; k < kRows; ++k) v[k] = octet_transpose(v[k]);  // uniform: every lane takes part
    for (uint32_t f = 0; f < dst_segs[0].fanout; ++f) {
      const uintptr_t g = sh.ptr(refs[dst_segs[0].ptr + f]) + uint64_t(dst_segs[0].offset) + uint64_t(r0) * 16u;
#pragma unroll
      for (int k = 0; k < kRows; ++k) {
        const uint32_t r = uint32_t(k * kBlock) + threadIdx.x;
        if (r < hr) store_bytes(g + uint64_t(r) * 16u, v[k], 16);
      }
    }
  } else {  // whole rows in (slots past the tile re-read its last row, never stored)
    // replica 0's run address is looked up next to the data loads, not after them
    const reshard_segment_t& seg = dst_segs[j];
    const uintptr_t gd0 = sh.ptr(refs[seg.ptr]) + uint64_t(seg.offset) + uint64_t(r0) * 2u;
    const uintptr_t g = sh.ptr(src_segs[0].ptr) + uint64_t(src_segs[0].offset) + uint64_t(r0) * 16u;
#pragma unroll
    for (int k = 0; k < kRows; ++k)
      v[k] = load_16_unaligned(g + uint64_t(min(uint32_t(k * kBlock) + threadIdx.x, hr - 1)) * 16u);
#pragma unroll
    for (int k = 0; k < kRows; ++k) v[k] = octet_transpose(v[k]);
    for (uint32_t f = 0; f < seg.fanout; ++f) {
      const uintptr_t g2 = f == 0 ? gd0 : sh.ptr(refs[seg.ptr + f]) + uint64_t(seg.offset) + uint64_t(r0) * 2u;
#pragma unroll
      for (int k = 0; k < kRows; ++k) {
        const uint32_t r = uint32_t(k * kBlock) + group_row;
        if (r + 8 <= hr) {
          store_bytes(g2 + uint64_t(r) * 2u, v[k], 16);
        } else {
          const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
          for (uint32_t i = 0; i < 8; ++i)
            if (r + i < hr)
              __builtin_nontemporal_store(uint16_t(w[i / 2] >> (16 * (i & 1))), as_global<u16_u>(g2 + uint64_t(r + i) * 2u));
        }
      }
    }
  }
}

// Bytewise copy of items [lo, hi) (either mode): taken when shard pointers are not
// aligned to the descriptor's unit, or replicas differ in 16-byte phase.
template <class Sh>
__device__ __forceinline__ void copy_bytes(const reshard_descriptor_t& D, uint32_t unit, uint32_t mode,
                           const uint8_t* src, const Sh& sh, uint32_t lo, uint32_t hi) {
  const uintptr_t d0 = sh.dst(0);
  for (uint32_t f = lo + threadIdx.x; f < hi; f += kBlock) {
    const ItemPos o = item_pos(D, f);
    uintptr_t a, b;
    if (mode == RESHARD_DESC_DST_CHUNKS) {
      chunk_range(d0 + o.dst, D.run_bytes, o.col, &a, &b);
      a -= d0;
      b -= d0;
    } else {
      a = o.dst + uint64_t(o.col) * unit;
      b = a + unit;
    }
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src) + o.src;
    for (uint32_t r = 0; r < D.fanout; ++r) {
      const uintptr_t dr = sh.dst(r);
      for (uintptr_t x = a; x < b; ++x)  // same place in the row on both sides
        *as_global<uint8_t>(dr + x) = *as_global<const uint8_t>(s0 + (x - o.dst));
    }
  }
}

// ---------------------------------------------------------------- conversion
//
// Float conversions of a RESHARD_DESC_CONVERT descriptor, on bit patterns with
// integer operations only (no dependence on the hardware's rounding mode).
// Narrowing rounds to nearest, ties to even: adding 2^(k-1) - 1 plus the last
// kept bit and dropping the k low bits rounds the magnitude that way, and a
// carry out of the fraction lands in the exponent, up to infinity.  A NaN keeps
// its sign and leading payload bits and gets the quiet bit.

__device__ __forceinline__ uint32_t f32_to_bf16(uint32_t u) {
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16(uint32_t u) {
  const uint32_t sign = (u >> 16) & 0x8000u, a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7e00u | ((a >> 13) & 0x3ffu);
  if (a >= 0x477ff000u) return sign | 0x7c00u;  // rounds past 65504: infinity
  if (a >= 0x38800000u)                         // normal binary16 (>= 2^-14): rebias 127 -> 15
    return sign | (((a + 0xfffu + ((a >> 13) & 1u)) >> 13) - (112u << 10));
  // below 2^-14: a multiple of 2^-24 (subnormal), rounded to nearest even
  const uint32_t e = a >> 23;
  if (e < 102) return sign;  // below 2^-25: rounds to zero
  const uint32_t m = (a & 0x7fffffu) | 0x800000u, sh = 126u - e;  // value = m * 2^(e - 150)
  const uint32_t q = m >> sh, rem = m & ((1u << sh) - 1u), half = 1u << (sh - 1u);
  return sign | (q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u));
}

__device__ __forceinline__ uint32_t bf16_to_f32(uint32_t h) {
  const uint32_t u = h << 16;
  return (u & 0x7fffffffu) > 0x7f800000u ? u | 0x00400000u : u;
}

__device__ __forceinline__ uint32_t f16_to_f32(uint32_t h) {
  const uint32_t sign = (h & 0x8000u) << 16, e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  if (e == 0x1fu) return sign | 0x7f800000u | (m << 13) | (m ? 0x00400000u : 0u);
  if (e != 0) return sign | ((e + 112u) << 23) | (m << 13);
  if (m == 0) return sign;
  const uint32_t p = 31u - __clz(m);  // subnormal m * 2^-24: leading bit at p < 10
  return sign | ((p + 103u) << 23) | ((m << (23u - p)) & 0x7fffffu);
}

template <int kConv>
__device__ __forceinline__ uint32_t convert_elem(uint32_t x) {
  if constexpr (kConv == RESHARD_CONVERT_F32_BF16) return f32_to_bf16(x);
  else if constexpr (kConv == RESHARD_CONVERT_F32_F16) return f32_to_f16(x);
  else if constexpr (kConv == RESHARD_CONVERT_BF16_F32) return bf16_to_f32(x);
  else return f16_to_f32(x);
}

// CONVERT mode: item f is up to 8 elements of a row.  A full item whose source
// and destination are 16-byte aligned moves as 16-byte accesses (32 bytes of
// fp32 in, 16 of 16-bit out, or the reverse); anything else element by element.
template <int kConv, class Sh>
__device__ __forceinline__ void convert_items(const reshard_descriptor_t& D, const uint8_t* src,
                                              const Sh& sh, uint32_t lo, uint32_t hi, bool aligned) {
  static_assert(rs::kItemsPerThread == 1, "a CONVERT tile holds one item per thread");
  constexpr bool kNarrow = kConv == RESHARD_CONVERT_F32_BF16 || kConv == RESHARD_CONVERT_F32_F16;
  constexpr uint32_t kEs = kNarrow ? 4 : 2, kEd = kNarrow ? 2 : 4;
  const uint32_t f = lo + threadIdx.x;
  if (f >= hi) return;
  const ItemPos o = item_pos(D, f);
  const uint32_t e0 = o.col * rs::kConvertElems;
  const uint32_t n = min(rs::kConvertElems, D.run_bytes - e0);
  const uintptr_t s = reinterpret_cast<uintptr_t>(src) + o.src + uint64_t(e0) * kEs;
  const uint64_t doff = o.dst + uint64_t(e0) * kEd;
  if (aligned && n == rs::kConvertElems && ((s | doff) & 15) == 0) {
    uint32_t x[8];
    if constexpr (kNarrow) {
      const u32x4 a = __builtin_nontemporal_load(as_global<const u32x4>(s));
      const u32x4 b = __builtin_nontemporal_load(as_global<const u32x4>(s + 16));
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
      const u32x4 a = __builtin_nontemporal_load(as_global<const u32x4>(s));
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = w[k] & 0xffffu;
        x[2 * k + 1] = w[k] >> 16;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = convert_elem<kConv>(x[k]);
    for (uint32_t r = 0; r < D.fanout; ++r) {
      const uintptr_t d = sh.dst(r) + doff;
      if constexpr (kNarrow) {
        const u32x4 v{x[0] | (x[1] << 16), x[2] | (x[3] << 16), x[4] | (x[5] << 16), x[6] | (x[7] << 16)};
        __builtin_nontemporal_store(v, as_global<u32x4>(d));
      } else {
        __builtin_nontemporal_store(u32x4{x[0], x[1], x[2], x[3]}, as_global<u32x4>(d));
        __builtin_nontemporal_store(u32x4{x[4], x[5], x[6], x[7]}, as_global<u32x4>(d + 16));
      }
    }
    return;
  }
  uint32_t x[8];
#pragma unroll
  for (uint32_t k = 0; k < 8; ++k) {
    if (k >= n) break;
    if constexpr (kNarrow) x[k] = convert_elem<kConv>(*as_global<const u32_u>(s + 4 * k));
    else x[k] = convert_elem<kConv>(*as_global<const u16_u>(s + 2 * k));
  }
  for (uint32_t r = 0; r < D.fanout; ++r) {
    const uintptr_t d = sh.dst(r) + doff;
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
      if (k >= n) break;
      if constexpr (kNarrow) *as_global<u16_u>(d + 2 * k) = uint16_t(x[k]);
      else *as_global<u32_u>(d + 4 * k) = x[k];
    }
  }
}

// ------------------------------------------------------------ partial sums
//
// REDUCE mode (Partial sources): item f is up to 8 elements of a row; each
// element is the binary32 sum, in list order, of the same element of every
// contribution (source slots refs[src_ptr ...], all at the same offsets),
// rounded once to the destination format.  The sum starts from contribution 0
// widened exactly, so that a -0.0 survives, and each addition is one v_add_f32
// (round to nearest even, denormals kept).  Formats: 0 binary32, 1 bfloat16,
// 2 binary16.

template <int kFmt>
__device__ __forceinline__ float widen_elem(uint32_t x) {
  uint32_t u;
  if constexpr (kFmt == 0) u = x;
  else if constexpr (kFmt == 1) u = bf16_to_f32(x);
  else u = f16_to_f32(x);
  return __uint_as_float(u);
}

template <int kFmt>
__device__ __forceinline__ uint32_t narrow_elem(float v) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (kFmt == 0) return u;
  else if constexpr (kFmt == 1) return f32_to_bf16(u);
  else return f32_to_f16(u);
}

// The n <= 8 elements at s as binary32 (the rest 0): 16-byte loads when vec
// (n == 8 and s 16-byte aligned), else element by element.
template <int kFmt>
__device__ __forceinline__ void load_elems(uintptr_t s, uint32_t n, bool vec, float x[8]) {
  if (vec) {
    if constexpr (kFmt == 0) {
      const u32x4 a = __builtin_nontemporal_load(as_global<const u32x4>(s));
      const u32x4 b = __builtin_nontemporal_load(as_global<const u32x4>(s + 16));
      x[0] = widen_elem<0>(a.x); x[1] = widen_elem<0>(a.y); x[2] = widen_elem<0>(a.z); x[3] = widen_elem<0>(a.w);
      x[4] = widen_elem<0>(b.x); x[5] = widen_elem<0>(b.y); x[6] = widen_elem<0>(b.z); x[7] = widen_elem<0>(b.w);
    } else {
      const u32x4 a = __builtin_nontemporal_load(as_global<const u32x4>(s));
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = widen_elem<kFmt>(w[k] & 0xffffu);
        x[2 * k + 1] = widen_elem<kFmt>(w[k] >> 16);
      }
    }
    return;
  }
#pragma unroll
  for (uint32_t k = 0; k < 8; ++k) {
    if (k < n) {
      if constexpr (kFmt == 0) x[k] = widen_elem<0>(*as_global<const u32_u>(s + 4 * k));
      else x[k] = widen_elem<kFmt>(*as_global<const u16_u>(s + 2 * k));
    } else {
      x[k] = 0.0f;
    }
  }
}

template <int kSrc, int kDst, class Sh>
__device__ __forceinline__ void reduce_items(const reshard_descriptor_t& D, const uint32_t* __restrict__ refs,
                                             const Sh& sh, uint32_t lo, uint32_t hi, bool aligned) {
  static_assert(rs::kItemsPerThread == 1, "a REDUCE tile holds one item per thread");
  constexpr uint32_t kEs = kSrc == 0 ? 4 : 2, kEd = kDst == 0 ? 4 : 2;
  const uint32_t f = lo + threadIdx.x;
  if (f >= hi) return;
  const ItemPos o = item_pos(D, f);
  const uint32_t e0 = o.col * rs::kConvertElems;
  const uint32_t n = min(rs::kConvertElems, D.run_bytes - e0);
  const uint64_t soff = o.src + uint64_t(e0) * kEs, doff = o.dst + uint64_t(e0) * kEd;
  const uint32_t parts = D.unit & 0xfffu;
  const bool vec = aligned && n == rs::kConvertElems && ((soff | doff) & 15) == 0;
  float acc[8];
  load_elems<kSrc>(sh.ptr(refs[D.src_ptr]) + soff, n, vec, acc);
#pragma unroll 2
  for (uint32_t p = 1; p < parts; ++p) {
    float x[8];
    load_elems<kSrc>(sh.ptr(refs[D.src_ptr + p]) + soff, n, vec, x);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = acc[k] + x[k];
  }
  uint32_t y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = narrow_elem<kDst>(acc[k]);
  for (uint32_t r = 0; r < D.fanout; ++r) {
    const uintptr_t d = sh.dst(r) + doff;
    if (vec) {
      if constexpr (kEd == 4) {
        __builtin_nontemporal_store(u32x4{y[0], y[1], y[2], y[3]}, as_global<u32x4>(d));
        __builtin_nontemporal_store(u32x4{y[4], y[5], y[6], y[7]}, as_global<u32x4>(d + 16));
      } else {
        const u32x4 v{y[0] | (y[1] << 16), y[2] | (y[3] << 16), y[4] | (y[5] << 16), y[6] | (y[7] << 16)};
        __builtin_nontemporal_store(v, as_global<u32x4>(d));
      }
      continue;
    }
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
      if (k >= n) break;
      if constexpr (kEd == 4) *as_global<u32_u>(d + 4 * k) = y[k];
      else *as_global<u16_u>(d + 2 * k) = uint16_t(y[k]);
    }
  }
}

// ------------------------------------------------------------ gather rows
//
// A RESHARD_DESC_GATHER_ROWS tile writes kGatherTileBytes consecutive bytes of
// a band of whole destination rows (all replicas at the same offset), 16 bytes
// a lane, so every destination line inside the band is written by one
// workgroup in whole 16-byte blocks.  A lane's block holds bytes of one source
// segment, or of two where segments meet (or where a row ends and the next
// begins).  Every segment is at least 1 KiB wide, so one wave's 1 KiB span
// touches at most two segments: the wave places its span once, in scalar
// registers -- row, column, the segment holding its first byte and the one after
// it -- and a lane only chooses between the two.  Bytes are counted from the
// start of the wave's row ("pos"); segment i covers pos [col_i, col_i + width_i)
// and the next row's first segment follows at pos >= W.

// Bytes [0, n) set, n <= 16.
__device__ __forceinline__ u32x4 low_bytes_mask(uint32_t n) {
  u32x4 m;
  m.x = n >= 4 ? 0xffffffffu : (n ? 0xffffffffu >> (32 - 8 * n) : 0u);
  m.y = n >= 8 ? 0xffffffffu : (n > 4 ? 0xffffffffu >> (32 - 8 * (n - 4)) : 0u);
  m.z = n >= 12 ? 0xffffffffu : (n > 8 ? 0xffffffffu >> (32 - 8 * (n - 8)) : 0u);
  m.w = n >= 16 ? 0xffffffffu : (n > 12 ? 0xffffffffu >> (32 - 8 * (n - 12)) : 0u);
  return m;
}

// Field words of a descriptor read as sixteen-word vectors (one 64-byte
// scalar load each), and of a segment as an eight-word one.
__device__ __forceinline__ uint64_t word64(uint32_t lo, uint32_t hi) { return uint64_t(lo) | (uint64_t(hi) << 32); }

template <class Sh>
__device__ __forceinline__ void gather_rows(const reshard_descriptor_t& D, const reshard_segment_t* __restrict__ segs,
                                            const uint32_t* __restrict__ refs, const Sh& sh, uint32_t tile) {
  // Every scalar load is issued before the first branch: the descriptor (two
  // 64-byte loads), the lookup word, both segments, then both pointers.  The
  // loads stay inside the band's tables even for a wave past the band's end.
  static_assert(offsetof(reshard_descriptor_t, dst_offset) == 8 && offsetof(reshard_descriptor_t, run_bytes) == 76 &&
                    offsetof(reshard_descriptor_t, extent) == 64 && offsetof(reshard_descriptor_t, row_items) == 80 &&
                    offsetof(reshard_descriptor_t, src_ptr) == 88 && offsetof(reshard_descriptor_t, dst_ref_begin) == 92 &&
                    offsetof(reshard_descriptor_t, fanout) == 96 && offsetof(reshard_descriptor_t, magic) == 100,
                "descriptor word layout");
  const u32x16 d0 = reinterpret_cast<const u32x16*>(&D)[0];
  const u32x16 d1 = reinterpret_cast<const u32x16*>(&D)[1];
  const uint32_t rows = d1[0], nseg = d1[1], W = d1[3], lut_ok = d1[4];
  const uint32_t src_ptr = d1[6], ref_begin = d1[7], fanout = d1[8], magic_m = d1[9], magic_s = d1[10];
  const uint64_t dst_offset = word64(d0[2], d0[3]);
  const uint32_t band = rows * W;  // < 2^31 (the planner splits longer bands)
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t a_w = tile * rs::kGatherTileBytes + wave * 1024u;
  const uint32_t row_w = div_magic(a_w, magic_m, magic_s);
  const uint32_t col_w = a_w - row_w * W;  // < W: the lookup index is in range even past the band
  const reshard_segment_t* __restrict__ S = segs + src_ptr;
  // the last segment whose column is <= col_w: one entry of the descriptor's
  // lookup (a 16-bit entry per KiB of row: the segment at the KiB's start and
  // where, inside it, the next one begins; its words 0-1 sit in src_offset,
  // 2-13 in the strides, after dst_offset), or a search for rows without one
  uint32_t i0 = 0;
  if (lut_ok) {
    const uint32_t w = col_w >> 11;
    const uint32_t word = w < 2 ? d0[w] : (w < 14 ? d0[w + 2] : 0u);
    const uint32_t e = (col_w & 1024u) ? word >> 16 : word & 0xffffu;
    const uint32_t split = e >> 6;
    i0 = (e & 63u) + (split != 0 && (col_w & 1023u) >= split ? 1u : 0u);
  } else {
    uint32_t hi = nseg;
    while (hi - i0 > 1) {
      const uint32_t mid = (i0 + hi) >> 1;
      if (S[mid].col <= col_w) i0 = mid; else hi = mid;
    }
  }
  // segments i0 and i0 + 1 in one 64-byte load (the table holds one padding
  // segment after the last), and segment 0 for a wave whose span wraps to the
  // next row
  const bool wrap = i0 + 1 == nseg;
  const u32x16 g01 = *reinterpret_cast<const u32x16*>(S + i0);
  const u32x8 gz = *reinterpret_cast<const u32x8*>(S);
  const u32x8 g0 = g01.lo;
  const u32x8 g1 = wrap ? gz : g01.hi;
  // segment words: 0-1 offset, 2-3 row_stride, 4 col, 5 width, 6 ptr
  const uint64_t p0 = sh.ptr(g0[6]), p1 = sh.ptr(g1[6]);
  asm volatile("" ::"s"(p0), "s"(p1));  // both pointer loads in flight together, not one sunk past the return
  if (a_w >= band) return;
  const uint32_t c0 = g0[4], c1 = g1[4];
  const uint32_t B1 = c0 + g0[5];                         // end of segment 0
  const uint32_t E1 = wrap ? W + g1[5] : c1 + g1[5];      // end of segment 1
  const uint64_t base0 = p0 + word64(g0[0], g0[1]) + uint64_t(row_w) * word64(g0[2], g0[3]) - c0;
  const uint64_t base1 = p1 + word64(g1[0], g1[1]) +
                         uint64_t(wrap ? row_w + 1 : row_w) * word64(g1[2], g1[3]) - (wrap ? W : c1);
  const uint32_t lane16 = 16u * (threadIdx.x & 63u);
  const uint32_t pos = col_w + lane16;
  const uint32_t left = band - a_w;
  const uint32_t n = left <= lane16 ? 0u : (left - lane16 < 16u ? left - lane16 : 16u);
  const bool in1 = pos >= B1;
  const uint64_t base = in1 ? base1 : base0;
  const uint32_t E = in1 ? E1 : B1;
  // one 16-byte load inside the segment's row (rows are >= 16 bytes wide);
  // a block that runs past the segment's end takes the rest from the start of
  // the next one
  const uint32_t at = pos < E - 16 ? pos : E - 16;
  const uint32_t L1 = (pos + n < E ? pos + n : E) - pos;
  // The second segment's first 16 bytes sit at one address for the whole wave;
  // kept in vector registers, since the compiler would read a wave-uniform
  // address with a scalar load, and scalar loads ignore the low two address bits
  // (the segment start need not be 4-byte aligned).
  uint64_t at1 = base1 + B1;
  asm volatile("" : "+v"(at1));
  u32x4 v1 = u32x4{0, 0, 0, 0}, v2 = v1;
  if (n) v1 = load_16_unaligned(base + at);
  if (L1 < n) v2 = load_16_unaligned(at1);
  if (!n) return;
  u32x4 x = pos != at ? shift_right_bytes(v1, pos - at) : v1;
  if (L1 < n) {
    const u32x4 m = low_bytes_mask(L1);
    const u32x4 y = shift_left_bytes(v2, L1);
    x = (x & m) | (y & ~m);
  }
  const uint64_t off = dst_offset + a_w + lane16;
  for (uint32_t r = 0; r < fanout; ++r) {
    const uintptr_t d = sh.ptr(refs[ref_begin + r]) + off;
    if (n == 16) __builtin_nontemporal_store(x, as_global<u32x4_u1>(d));
    else store_head_bytes(d, x, n);
  }
}

// Kernel variants.  A plan runs the smallest variant that covers the modes of
// its descriptors: short launches pay for code size, for branches in the tile
// prologue and for an LDS allocation they do not use.
enum KernelKind : int {
  kKindItems16 = 0,  // every descriptor ITEMS with 16-byte items
  kKindChunks = 1,   // every descriptor DST_CHUNKS
  kKindCopy = 2,     // ITEMS, DST_CHUNKS and CONVERT; no LDS
  kKindAll = 3,      // any mode, LDS window included
  kKindQuadRows = 4, // every descriptor a 16-byte row-mode band with the quad exchange
                     // (kQuadRowsPerLane rows per lane): no LDS, fewer registers
  kKindOctets = 9,   // every descriptor a 16-byte window band of eight 2-byte column
                     // runs (window_octets): no LDS
  kKindGatherRows = 10,  // every descriptor RESHARD_DESC_GATHER_ROWS (gather_rows)
  kKindReduce = 11,      // every descriptor RESHARD_DESC_REDUCE (reduce_items)
  kKindNarrow = 12,      // every descriptor a narrow band of dword segments (window_narrow): LDS
  kKindNarrowBytes = 13, // every descriptor a narrow band (window_narrow, every segment class): LDS
  kKindAligned = 16, // added to kKindChunks when every shard pointer is 16-byte
                     // aligned: no bytewise fallback is compiled in
};

template <bool kKarg, int kVariant>
__global__ __launch_bounds__(kBlock) void reshard_copy_kernel(
    const reshard_descriptor_t* __restrict__ descs, uint32_t n_desc,
    const uint32_t* __restrict__ tile_begin, const uint32_t* __restrict__ refs,
    const reshard_segment_t* __restrict__ segs, const void* const* __restrict__ table, KargPtrs karg,
    uint32_t n_tiles, uint32_t per_xcd, uint32_t flags, uint32_t block_base, TileStride stride) {
  constexpr int kKind = kVariant % kKindAligned;
  constexpr bool kAligned = kVariant >= kKindAligned;
  // Block b of the plan (block_base + blockIdx.x: a plan larger than one
  // launch is split into launches of a multiple of kXcds blocks) runs on XCD
  // b % kXcds.  Each XCD takes groups of kXcdGroup consecutive tiles, the
  // XCDs side by side: nearby tiles share an XCD's L2 while all XCDs stream
  // through the same region of memory.  Plans smaller than one round of groups
  // (per_xcd == 0) use block b for tile b.
  const uint32_t b = block_base + blockIdx.x;
  const uint32_t kx = b / kXcds;
  const uint32_t t = per_xcd == 0 ? b : ((kx / kXcdGroup) * kXcds + b % kXcds) * kXcdGroup + kx % kXcdGroup;
  if constexpr (kKind == kKindGatherRows) {
    if (stride.tiles) {
      // every band of the launch spans stride.tiles tiles: the band is a
      // division away, and a surplus block reads band 0's tables (in bounds)
      // and returns once its loads are issued
      const bool live = t < n_tiles;
      const uint32_t lo = live ? div_magic(t, stride.m, stride.s) : 0u;
      const Shards<kKarg> gsh{table, &karg, refs};
      gather_rows(descs[lo], segs, refs, gsh, live ? t - lo * stride.tiles : stride.tiles);
      return;
    }
  }
  if (t >= n_tiles) return;
  // the descriptor of tile t: the last one whose first tile is <= t.  The
  // gather-rows build reads the tile-group lookup behind tile_begin (one load;
  // a search only where 64 tiles touch three or more descriptors); the others
  // search tile_begin, which measured as fast for them.
  uint32_t lo = 0;
  bool search = true;
  if constexpr (kKind == kKindGatherRows) {
    const uint32_t grp = tile_begin[n_desc + 1 + t / kTileGroup];
    if ((grp >> 24) != kTileGroupSearch) {
      lo = (grp & 0xffffffu) + (t % kTileGroup >= (grp >> 24) ? 1u : 0u);
      search = false;
    }
  }
  if (search) {
    uint32_t hi = n_desc;
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) >> 1;
      if (tile_begin[mid] <= t) lo = mid; else hi = mid;
    }
  }
  const reshard_descriptor_t& D = descs[lo];
  uint32_t unit_mode;  // the two 16-bit fields as one scalar word
  __builtin_memcpy(&unit_mode, &D.unit, sizeof(unit_mode));
  const uint32_t unit = kKind == kKindItems16 ? 16u : unit_mode & 0xffffu;
  const uint32_t mode = kKind == kKindItems16 ? uint32_t(RESHARD_DESC_ITEMS)
                        : kKind == kKindChunks ? uint32_t(RESHARD_DESC_DST_CHUNKS)
                        : kKind == kKindQuadRows || kKind == kKindOctets || kKind == kKindNarrow ||
                                  kKind == kKindNarrowBytes
                            ? uint32_t(RESHARD_DESC_WINDOW)
                        : kKind == kKindGatherRows ? uint32_t(RESHARD_DESC_GATHER_ROWS)
                        : kKind == kKindReduce ? uint32_t(RESHARD_DESC_REDUCE)
                                               : unit_mode >> 16;
  if constexpr (kKind == kKindQuadRows) {
    const Shards<kKarg> wsh{table, &karg, refs};
    window_rows<int(rs::kQuadRowsPerLane)>(D, segs, refs, wsh, t - tile_begin[lo]);
    return;
  }
  if constexpr (kKind == kKindGatherRows) {
    const Shards<kKarg> gsh{table, &karg, refs};
    gather_rows(D, segs, refs, gsh, t - tile_begin[lo]);
    return;
  }
  if constexpr (kKind == kKindNarrow || kKind == kKindNarrowBytes) {
    // the window: dynamic LDS, as large as the launch's largest band needs
    extern __shared__ __attribute__((aligned(16))) uint32_t narrow_window[];
    const Shards<kKarg> wsh{table, &karg, refs};
    window_narrow<kKind == kKindNarrowBytes>(D, segs, refs, wsh, t - tile_begin[lo], narrow_window);
    return;
  }
  if constexpr (kKind == kKindReduce) {
    (void)mode;
    const uint32_t items = D.extent[0] * D.extent[1] * D.extent[2] * D.row_items;
    const uint32_t first = (t - tile_begin[lo]) * rs::kTileItems;
    const uint32_t last = min(first + rs::kTileItems, items);
    const Shards<kKarg> rsh{table, &karg, refs + D.dst_ref_begin};
    const bool aligned = (flags & kAllAligned16) != 0;
    switch (unit >> 12) {  // source format | destination format << 2
      case 0 | (0 << 2): reduce_items<0, 0>(D, refs, rsh, first, last, aligned); break;
      case 0 | (1 << 2): reduce_items<0, 1>(D, refs, rsh, first, last, aligned); break;
      case 0 | (2 << 2): reduce_items<0, 2>(D, refs, rsh, first, last, aligned); break;
      case 1 | (1 << 2): reduce_items<1, 1>(D, refs, rsh, first, last, aligned); break;
      case 1 | (0 << 2): reduce_items<1, 0>(D, refs, rsh, first, last, aligned); break;
      case 2 | (2 << 2): reduce_items<2, 2>(D, refs, rsh, first, last, aligned); break;
      default: reduce_items<2, 0>(D, refs, rsh, first, last, aligned); break;
    }
    return;
  }
  if constexpr (kKind == kKindOctets) {
    const Shards<kKarg> wsh{table, &karg, refs};
    window_octets(D, segs, refs, wsh, t - tile_begin[lo]);
    return;
  }
  if constexpr (kKind == kKindAll) {
    if (mode == RESHARD_DESC_WINDOW) {  // any alignment: global chunks follow the addresses
      __shared__ __attribute__((aligned(16))) uint8_t window[rs::kWindowBytes];
      const Shards<kKarg> wsh{table, &karg, refs};
      // one row-mode build serves every band here (a band's tile may have fewer
      // rows than its slots): a second one would raise the register count of
      // the whole kernel
      if (D.run_bytes > uint32_t(rs::kRowModeBytes))
        window_tile(D, segs, refs, wsh, t - tile_begin[lo], window);
      else
        window_rows<int(rs::kRowsPerLane)>(D, segs, refs, wsh, t - tile_begin[lo]);
      return;
    }
  }
  if constexpr (kKind == kKindItems16 || kKind == kKindChunks || kKind == kKindCopy || kKind == kKindAll) {
  const uint32_t items = D.extent[0] * D.extent[1] * D.extent[2] * D.row_items;
  const uint32_t first = (t - tile_begin[lo]) * rs::kTileItems;
  const uint32_t last = min(first + rs::kTileItems, items);
  const Shards<kKarg> sh{table, &karg, refs + D.dst_ref_begin};
  const uint8_t* src = reinterpret_cast<const uint8_t*>(sh.ptr(D.src_ptr));
  if constexpr (kKind == kKindCopy || kKind == kKindAll) {
    if (mode == RESHARD_DESC_CONVERT) {  // checks its own alignment per item
      const bool aligned = (flags & kAllAligned16) != 0;
      switch (unit) {
        case RESHARD_CONVERT_F32_BF16: convert_items<RESHARD_CONVERT_F32_BF16>(D, src, sh, first, last, aligned); break;
        case RESHARD_CONVERT_F32_F16: convert_items<RESHARD_CONVERT_F32_F16>(D, src, sh, first, last, aligned); break;
        case RESHARD_CONVERT_BF16_F32: convert_items<RESHARD_CONVERT_BF16_F32>(D, src, sh, first, last, aligned); break;
        default: convert_items<RESHARD_CONVERT_F16_F32>(D, src, sh, first, last, aligned); break;
      }
      return;
    }
  }
  if (!kAligned && !(flags & kAllAligned16)) {
    // alignment every access width relies on: the unit for ITEMS; for
    // DST_CHUNKS, replicas in the same 16-byte phase as replica 0
    const uintptr_t d0 = sh.dst(0);
    uintptr_t bits = reinterpret_cast<uintptr_t>(src) | d0, phase = 0;
    for (uint32_t r = 1; r < D.fanout; ++r) {
      bits |= sh.dst(r);
      phase |= sh.dst(r) - d0;
    }
    const bool ok = mode == RESHARD_DESC_DST_CHUNKS ? (phase & 15) == 0 : (bits & (unit - 1)) == 0;
    if (!ok) {
      copy_bytes(D, unit, mode, src, sh, first, last);
      return;
    }
  }
  if constexpr (kKind == kKindItems16) {
    copy_items<u32x4, rs::kItemsPerThread>(D, src, sh, first, last);
  } else if constexpr (kKind == kKindChunks) {
    copy_chunks<rs::kItemsPerThread>(D, src, sh, first, last);
  } else {
    if (mode == RESHARD_DESC_DST_CHUNKS) {
      copy_chunks<rs::kItemsPerThread>(D, src, sh, first, last);
      return;
    }
    switch (unit) {
      case 16: copy_items<u32x4, rs::kItemsPerThread>(D, src, sh, first, last); break;
      case 8: copy_items<u32x2, rs::kItemsPerThread>(D, src, sh, first, last); break;
      case 4: copy_items<uint32_t, rs::kItemsPerThread>(D, src, sh, first, last); break;
      case 2: copy_items<uint16_t, rs::kItemsPerThread>(D, src, sh, first, last); break;
      default: copy_items<uint8_t, rs::kItemsPerThread>(D, src, sh, first, last); break;
    }
  }
  }  // the item, chunk, copy and all-modes builds
}

template <bool kKarg, int kVariant>
hipError_t launch_kind(uint32_t n_wg, hipStream_t stream, const reshard_descriptor_t* descs, uint32_t n_desc,
                       const uint32_t* tile_begin, const uint32_t* refs, const reshard_segment_t* segs,
                       const void* const* table, const KargPtrs& karg, uint32_t n_tiles, uint32_t per_xcd,
                       uint32_t flags, TileStride stride, uint32_t lds_bytes) {
  for (uint32_t base = 0; base < n_wg; base += kMaxLaunchBlocks) {
    const uint32_t grid = n_wg - base < kMaxLaunchBlocks ? n_wg - base : kMaxLaunchBlocks;
    hipLaunchKernelGGL((reshard_copy_kernel<kKarg, kVariant>), dim3(grid), dim3(kBlock), lds_bytes, stream, descs,
                       n_desc, tile_begin, refs, segs, table, karg, n_tiles, per_xcd, flags, base, stride);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool kKarg>
hipError_t launch(int kind, uint32_t n_wg, hipStream_t stream, const reshard_descriptor_t* descs, uint32_t n_desc,
                  const uint32_t* tile_begin, const uint32_t* refs, const reshard_segment_t* segs,
                  const void* const* table, const KargPtrs& karg, uint32_t n_tiles, uint32_t per_xcd,
                  uint32_t flags, TileStride stride, uint32_t lds_bytes) {
  const bool aligned = (flags & kAllAligned16) != 0;
#define RS_LAUNCH(V) \
  launch_kind<kKarg, V>(n_wg, stream, descs, n_desc, tile_begin, refs, segs, table, karg, n_tiles, per_xcd, flags, \
                        stride, (V) == kKindNarrow || (V) == kKindNarrowBytes ? lds_bytes : 0u)
  switch (kind) {
    case kKindItems16:  // (an aligned-only build of this one measured slower on long copies)
      return RS_LAUNCH(kKindItems16);
    case kKindChunks:
      return aligned ? RS_LAUNCH(kKindChunks + kKindAligned) : RS_LAUNCH(kKindChunks);
    case kKindCopy:
      return RS_LAUNCH(kKindCopy);
    case kKindQuadRows:
      return RS_LAUNCH(kKindQuadRows);
    case kKindOctets:
      return RS_LAUNCH(kKindOctets);
    case kKindGatherRows:
      return RS_LAUNCH(kKindGatherRows);
    case kKindReduce:
      return RS_LAUNCH(kKindReduce);
    case kKindNarrow:
      return RS_LAUNCH(kKindNarrow);
    case kKindNarrowBytes:
      return RS_LAUNCH(kKindNarrowBytes);
    default:
      return RS_LAUNCH(kKindAll);
  }
#undef RS_LAUNCH
}

}  // namespace

namespace {

// Whether a descriptor is a band window_octets moves: 16 bytes wide, tiles of
// kQuadRowsPerLane * kBlock rows, one side eight 2-byte runs in column order,
// the other one packed run of whole rows.
bool octets_band(const reshard_descriptor_t& D, const std::vector<reshard_segment_t>& segs) {
  const uint32_t w = D.run_bytes;
  if (D.mode != RESHARD_DESC_WINDOW || w != 16 || D.extent[1] != rs::kQuadRowsPerLane * uint32_t(kBlock))
    return false;
  const reshard_segment_t* S = segs.data() + D.src_ptr;
  const reshard_segment_t* T = S + D.dst_ref_begin;
  const bool src_runs = runs_side(S, D.dst_ref_begin, 8, 2), dst_runs = runs_side(T, D.fanout, 8, 2);
  return (src_runs && full_side(T, D.fanout, w)) || (dst_runs && full_side(S, D.dst_ref_begin, w));
}

// Whether a descriptor is a band window_narrow moves (rs::narrow_band on its
// segments): 0 no, 1 with dword segments only, 2 with segments of other classes.
int narrow_band(const reshard_descriptor_t& D, const std::vector<reshard_segment_t>& segs) {
  if (D.mode != RESHARD_DESC_WINDOW) return 0;
  const reshard_segment_t* S = segs.data() + D.src_ptr;
  return rs::narrow_band(D.run_bytes, D.extent[1], S, D.dst_ref_begin, S + D.dst_ref_begin, D.fanout);
}

}  // namespace

int kernel_kind_gather_rows() { return kKindGatherRows; }
bool kernel_kind_narrow(int kind) { return kind == kKindNarrow || kind == kKindNarrowBytes; }

// The kernel variant of a plan's descriptors.
int kernel_kind(const std::vector<reshard_descriptor_t>& descs, const std::vector<reshard_segment_t>& segs) {
  bool items16 = true, chunks = true, quad_rows = true, octets = true, gather = true, reduce = true;
  bool window = false;
  int narrow = 1;  // the narrow build that moves every descriptor (0: none)
  for (const reshard_descriptor_t& D : descs) {
    if (D.mode != RESHARD_DESC_ITEMS || D.unit != 16) items16 = false;
    if (D.mode != RESHARD_DESC_DST_CHUNKS) chunks = false;
    if (D.mode != RESHARD_DESC_WINDOW || D.run_bytes > uint32_t(rs::kRowModeBytes) ||
        D.extent[1] != rs::kQuadRowsPerLane * uint32_t(kBlock))
      quad_rows = false;
    if (!octets_band(D, segs)) octets = false;
    if (D.mode != RESHARD_DESC_GATHER_ROWS) gather = false;
    if (D.mode != RESHARD_DESC_REDUCE) reduce = false;
    const int n = narrow_band(D, segs);
    narrow = n == 0 || narrow == 0 ? 0 : std::max(narrow, n);
    if (D.mode == RESHARD_DESC_WINDOW) window = true;
  }
  if (gather && !descs.empty()) return kKindGatherRows;
  if (reduce && !descs.empty()) return kKindReduce;
  return items16 ? kKindItems16 : chunks ? kKindChunks : octets ? kKindOctets : narrow == 1 ? kKindNarrow
         : narrow == 2 ? kKindNarrowBytes : quad_rows ? kKindQuadRows : window ? kKindAll : kKindCopy;
}

hipError_t launch_copy(int kind, uint32_t n_wg, hipStream_t stream, const reshard_descriptor_t* descs,
                       uint32_t n_desc, const uint32_t* tile_begin, const uint32_t* refs,
                       const reshard_segment_t* segs, const void* const* table, const KargPtrs& karg,
                       uint32_t n_tiles, uint32_t per_xcd, uint32_t flags, TileStride stride, uint32_t lds_bytes) {
  if (table)
    return launch<false>(kind, n_wg, stream, descs, n_desc, tile_begin, refs, segs, table, karg, n_tiles,
                         per_xcd, flags, stride, lds_bytes);
  return launch<true>(kind, n_wg, stream, descs, n_desc, tile_begin, refs, segs, table, karg, n_tiles, per_xcd,
                      flags, stride, lds_bytes);
}

}  // namespace rs
