// C ABI of the reshard library: layouts, host plans, the device descriptor
// table, the pointer slots of large plans and execute, which launches the
// gfx950 copy kernel (kernel.hip) once per launch group of the plan.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernel.h"
#include "plan.h"
#include "reshard.h"

struct reshard_layout_s {
  rs::Layout L;
};

namespace {

constexpr int kSlots = 8;  // device pointer-table slots for bigger plans

thread_local std::string g_err;

reshard_status_t fail(reshard_status_t s, const std::string& msg) {
  g_err = msg;
  return s;
}

reshard_status_t hip_fail(hipError_t e, const char* what) {
  return fail(e == hipErrorOutOfMemory ? RESHARD_ERR_OUT_OF_MEMORY : RESHARD_ERR_HIP,
              std::string(what) + ": " + hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

// ------------------------------------------------------------------ host side

struct reshard_plan_s {
  rs::HostPlan host;
  std::mutex mu;
  // One launch group: descriptors that run in one kernel variant.  Device
  // addresses are offsets into the table image (the image is placed either in
  // the plan's own allocation or in the library's static scratch array).
  struct Launch {
    int kind = 0;          // kernel variant (rs::kernel_kind of the group's descriptors)
    uint32_t n_desc = 0;
    uint32_t n_tiles = 0;
    uint32_t per_xcd = 0;  // blocks per XCD, a multiple of rs::kXcdGroup (0: one block per tile)
    uint32_t n_wg = 0;     // grid: rs::kXcds * per_xcd blocks (surplus ones exit), else n_tiles
    rs::TileStride stride; // gather-rows launches whose bands all span stride.tiles tiles
    uint32_t lds_bytes = 0;  // narrow-band launches: the window of their largest band (dynamic LDS)
    size_t desc_off = 0;   // the group's descriptors in the image
    size_t tb_off = 0;     // its first tile of each, from 0; n_desc + 1 entries
  };
  // host image of the device table, built once: descriptors by group | refs
  // (absolute pointer slots) | tile_begin by group | segments
  bool image_built = false;
  std::vector<uint8_t> image;
  std::vector<Launch> launches;
  size_t refs_off = 0, segs_off = 0;
  // the plan's own device copy of the image
  bool uploaded = false;
  int device = -1;
  int64_t table_bytes = 0;
  void* table = nullptr;
  // pointer-table slots, used when the pointers do not fit in kernel arguments
  int64_t n_ptrs = 0;
  void* d_slots = nullptr;
  void** h_slots = nullptr;  // pinned host staging, kSlots * n_ptrs entries
  hipEvent_t ev[kSlots] = {};      // recorded after the last launch that read the slot
  bool ev_live[kSlots] = {};
  hipStream_t ev_stream[kSlots] = {};  // the stream of that launch
  int next_slot = 0;
  int last_slot = -1;
};

namespace {

// Descriptors that run in one launch, in plan order, and their tiles.
struct Group {
  int kind = 0;
  bool big = false;  // narrow bands whose window exceeds rs::kNarrowWindowBytes
  std::vector<uint32_t> descs;
  uint64_t tiles = 0;

  void add(uint32_t i, const rs::HostPlan& H) {
    descs.push_back(i);
    tiles += H.tile_begin[i + 1] - H.tile_begin[i];
  }
};

// The launches of one execute.  Only the general build (rs::kKindAll) runs
// item, chunk and convert descriptors together with window bands, or bands of
// several kinds together (gather-rows bands and Partial sums run in their own
// builds only), and
// it stages bands through LDS and holds more registers, so
// a plan that mixes them would run everything slower.  Instead the descriptors
// that are not bands share one launch (the item, chunk or copy build already
// covers any mix of them), and each band kind runs in a launch of its own
// build; bands that no special build moves share the general one.  Narrow
// bands with the larger window (rs::kNarrowBigWindowBytes) run apart from those
// with the usual one, since the window sets how many workgroups share a CU.  A
// plan with only one of these groups runs its descriptors in plan order.
// LDS bytes of a narrow band's window: its rows per tile at its pitch.
uint32_t narrow_window_bytes(const reshard_descriptor_t& D) { return D.extent[1] * rs::narrow_pitch(D.run_bytes); }

std::vector<Group> launch_groups(const rs::HostPlan& H) {
  Group rows;                 // descriptors that are not bands
  std::vector<Group> bands;   // bands by kind, in order of first appearance
  std::vector<reshard_descriptor_t> one(1);
  for (uint32_t i = 0; i < uint32_t(H.descs.size()); ++i) {
    if (H.descs[i].mode != RESHARD_DESC_WINDOW && H.descs[i].mode != RESHARD_DESC_GATHER_ROWS &&
        H.descs[i].mode != RESHARD_DESC_REDUCE) {
      rows.add(i, H);
      continue;
    }
    one[0] = H.descs[i];
    const int kind = rs::kernel_kind(one, H.segs);
    const bool big = rs::kernel_kind_narrow(kind) && narrow_window_bytes(H.descs[i]) > rs::kNarrowWindowBytes;
    auto g = std::find_if(bands.begin(), bands.end(), [&](const Group& x) { return x.kind == kind && x.big == big; });
    if (g == bands.end()) g = bands.insert(bands.end(), Group{kind, big, {}, 0});
    g->add(i, H);
  }
  std::vector<Group> out;
  if (!rows.descs.empty()) out.push_back(std::move(rows));
  for (Group& g : bands) out.push_back(std::move(g));
  for (Group& g : out) {
    std::vector<reshard_descriptor_t> ds;
    for (const uint32_t i : g.descs) ds.push_back(H.descs[i]);
    g.kind = rs::kernel_kind(ds, H.segs);
  }
  return out;
}

// Builds the host image of the device table and the launch groups (host only,
// once per plan).
void build_image_locked(reshard_plan_s* p) {
  if (p->image_built) return;
  const rs::HostPlan& H = p->host;
  const std::vector<Group> groups = launch_groups(H);
  size_t n_tb = 0;  // per launch group: tile_begin (n_desc + 1 entries), then its tile-group lookup
  for (const Group& g : groups) n_tb += g.descs.size() + 1 + rs::tile_groups(g.tiles);
  const size_t desc_bytes = H.descs.size() * sizeof(reshard_descriptor_t);
  const size_t refs_off = align_up(desc_bytes, 256);
  const size_t tiles_off = align_up(refs_off + H.refs.size() * sizeof(uint32_t), 256);
  const size_t segs_off = align_up(tiles_off + n_tb * sizeof(uint32_t), 256);
  // one zero segment after the last: a gather-rows wave reads segments i and
  // i + 1 together
  const size_t total = align_up(segs_off + (H.segs.size() + 1) * sizeof(reshard_segment_t), 256);
  std::vector<uint8_t> img(total, 0);
  reshard_descriptor_t* dd = reinterpret_cast<reshard_descriptor_t*>(img.data());
  uint32_t* tb = reinterpret_cast<uint32_t*>(img.data() + tiles_off);
  std::vector<reshard_plan_s::Launch> launches;
  size_t k = 0, t = 0;
  for (const Group& g : groups) {
    reshard_plan_s::Launch L;
    L.kind = g.kind;
    L.n_desc = uint32_t(g.descs.size());
    L.n_tiles = uint32_t(g.tiles);
    if (rs::kernel_kind_narrow(g.kind))
      for (const uint32_t i : g.descs) L.lds_bytes = std::max(L.lds_bytes, narrow_window_bytes(H.descs[i]));
    // Gather-rows bands of (nearly) one size take a common tile stride, so that
    // a workgroup finds its band by a division instead of a table load: the
    // shorter bands leave their last tiles idle (at most 1/16 more tiles).
    if (g.kind == rs::kernel_kind_gather_rows()) {
      uint64_t most = 0;
      for (const uint32_t i : g.descs) most = std::max<uint64_t>(most, H.tile_begin[i + 1] - H.tile_begin[i]);
      const uint64_t padded = most * g.descs.size();
      if (padded < (uint64_t(1) << 31) && padded <= g.tiles + std::max<uint64_t>(64, g.tiles / 16)) {
        L.stride.tiles = uint32_t(most);
        rs::magic_u31(L.stride.tiles, &L.stride.m, &L.stride.s);
        L.n_tiles = uint32_t(padded);
      }
    }
    const uint64_t grid_tiles = L.n_tiles;
    // blocks per XCD, a whole number of tile groups; 0: too few tiles to group
    const uint64_t per_xcd_min = (grid_tiles + rs::kXcds - 1) / rs::kXcds;
    L.per_xcd = grid_tiles < uint64_t(rs::kXcds) * rs::kXcdGroup
                    ? 0u
                    : uint32_t((per_xcd_min + rs::kXcdGroup - 1) / rs::kXcdGroup * rs::kXcdGroup);
    L.n_wg = L.per_xcd ? L.per_xcd * rs::kXcds : L.n_tiles;
    L.desc_off = k * sizeof(reshard_descriptor_t);
    L.tb_off = tiles_off + t * sizeof(uint32_t);
    uint32_t first = 0;
    const uint32_t* local = tb + t;
    for (const uint32_t i : g.descs) {
      dd[k++] = H.descs[i];
      tb[t++] = first;
      first += H.tile_begin[i + 1] - H.tile_begin[i];
    }
    tb[t++] = first;
    rs::fill_tile_groups(local, L.n_desc, uint32_t(g.tiles), tb + t);
    t += rs::tile_groups(g.tiles);
    launches.push_back(L);
  }
  // the fan-out list in absolute slots of the pointer array (sources first,
  // then destinations); a REDUCE descriptor's list of contributions holds
  // source slots, which are absolute already
  uint32_t* r = reinterpret_cast<uint32_t*>(img.data() + refs_off);
  for (size_t i = 0; i < H.refs.size(); ++i) r[i] = uint32_t(H.n_src_ptrs) + H.refs[i];
  for (const reshard_descriptor_t& D : H.descs)
    if (D.mode == RESHARD_DESC_REDUCE)
      for (uint32_t q = 0; q < (D.unit & 0xfffu); ++q) r[D.src_ptr + q] = H.refs[D.src_ptr + q];
  // window segments as planned: a source segment indexes the source pointers,
  // which come first in the pointer array; a destination segment indexes the
  // fan-out list, whose entries were made absolute above
  reshard_segment_t* sg = reinterpret_cast<reshard_segment_t*>(img.data() + segs_off);
  for (size_t i = 0; i < H.segs.size(); ++i) sg[i] = H.segs[i];
  // narrow bands: each destination segment carries its first replica's slot
  // (the kernel then reaches the pointer in one load instead of two)
  for (const Group& g : groups) {
    if (!rs::kernel_kind_narrow(g.kind)) continue;
    for (const uint32_t i : g.descs) {
      const reshard_descriptor_t& D = H.descs[i];
      for (uint32_t k = 0; k < D.fanout; ++k) {
        reshard_segment_t& x = sg[D.src_ptr + D.dst_ref_begin + k];
        x.row_stride = int64_t(uint32_t(H.n_src_ptrs) + H.refs[x.ptr]);
      }
    }
  }
  p->image = std::move(img);
  p->launches = std::move(launches);
  p->refs_off = refs_off;
  p->segs_off = segs_off;
  p->n_ptrs = H.n_src_ptrs + H.n_dst_ptrs;
  p->image_built = true;
}

reshard_status_t upload_locked(reshard_plan_s* p, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (p->uploaded) {
    if (dev != p->device)
      return fail(RESHARD_ERR_DEVICE_MISMATCH, "plan was uploaded to device " +
                                                   std::to_string(p->device) + ", current device is " +
                                                   std::to_string(dev));
    return RESHARD_OK;
  }
  try {
    build_image_locked(p);
  } catch (const std::bad_alloc&) {
    return fail(RESHARD_ERR_OUT_OF_MEMORY, "host memory exhausted while building the descriptor table");
  }
  const size_t total = p->image.size();
  void* table = nullptr;
  e = hipMalloc(&table, total);
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(descriptor table)");
  e = hipMemcpyAsync(table, p->image.data(), total, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    (void)hipFree(table);
    return hip_fail(e, "descriptor table upload");
  }
  if (p->n_ptrs > rs::kKargPtrs) {
    const size_t bytes = size_t(kSlots) * size_t(p->n_ptrs) * sizeof(void*);
    e = hipMalloc(&p->d_slots, bytes);
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&p->h_slots), bytes, hipHostMallocDefault);
    for (int s = 0; s < kSlots && e == hipSuccess; ++s)
      e = hipEventCreateWithFlags(&p->ev[s], hipEventDisableTiming);
    if (e != hipSuccess) {
      (void)hipFree(table);
      if (p->d_slots) (void)hipFree(p->d_slots);
      if (p->h_slots) (void)hipHostFree(p->h_slots);
      for (int s = 0; s < kSlots; ++s)
        if (p->ev[s]) (void)hipEventDestroy(p->ev[s]);
      p->d_slots = nullptr;
      p->h_slots = nullptr;
      for (int s = 0; s < kSlots; ++s) p->ev[s] = nullptr;
      return hip_fail(e, "pointer-table slots");
    }
  }
  p->table = table;
  p->table_bytes = int64_t(total);
  p->device = dev;
  p->uploaded = true;
  return RESHARD_OK;
}

// Every launch group of the plan, in order on `stream`, with the table image at
// device address `base`.  Returns the first launch error.
hipError_t launch_groups_at(const reshard_plan_s* p, const uint8_t* base, const void* const* table,
                            const rs::KargPtrs& karg, uint32_t flags, hipStream_t stream) {
  const uint32_t* refs = reinterpret_cast<const uint32_t*>(base + p->refs_off);
  const reshard_segment_t* segs = reinterpret_cast<const reshard_segment_t*>(base + p->segs_off);
  for (const reshard_plan_s::Launch& L : p->launches) {
    const hipError_t e =
        rs::launch_copy(L.kind, L.n_wg, stream, reinterpret_cast<const reshard_descriptor_t*>(base + L.desc_off),
                        L.n_desc, reinterpret_cast<const uint32_t*>(base + L.tb_off), refs, segs, table, karg,
                        L.n_tiles, L.per_xcd, flags, L.stride, L.lds_bytes);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Argument checks shared by the execute entry points.
reshard_status_t check_pointers(const rs::HostPlan& H, const void* const* src_ptrs, void* const* dst_ptrs) {
  if ((H.n_src_ptrs && !src_ptrs) || (H.n_dst_ptrs && !dst_ptrs))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "pointer array is NULL");
  for (int64_t i = 0; i < H.n_src_ptrs; ++i)
    if (H.src_needed[i] && !src_ptrs[i])
      return fail(RESHARD_ERR_NULL_SHARD, "src_ptrs[" + std::to_string(i) + "] is NULL but its shard is not empty");
  for (int64_t i = 0; i < H.n_dst_ptrs; ++i)
    if (H.dst_needed[i] && !dst_ptrs[i])
      return fail(RESHARD_ERR_NULL_SHARD, "dst_ptrs[" + std::to_string(i) + "] is NULL but its shard is not empty");
  return RESHARD_OK;
}

// The kAllAligned16 flag when every shard pointer is 16-byte aligned.
uint32_t alignment_flags(const rs::HostPlan& H, const void* const* src_ptrs, void* const* dst_ptrs) {
  uintptr_t bits = 0;
  for (int64_t i = 0; i < H.n_src_ptrs; ++i) bits |= reinterpret_cast<uintptr_t>(src_ptrs[i]);
  for (int64_t i = 0; i < H.n_dst_ptrs; ++i) bits |= reinterpret_cast<uintptr_t>(dst_ptrs[i]);
  return (bits & 15) == 0 ? rs::kAllAligned16 : 0;
}

// ------------------------------------------------------------ static scratch
//
// The allocation-free execute (reshard_execute_noalloc) places the plan's
// table image, and the pointer array when it does not fit in the kernel
// arguments, in this array instead of memory the library allocates.  Host code
// never uses the array's name as an address: each device's copy is found once
// with hipGetSymbolAddress and that address is used from then on.
constexpr size_t kScratchBytes = RESHARD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

reshard_status_t scratch_of_current_device(uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(RESHARD_ERR_HIP, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return RESHARD_OK;
}

reshard_status_t make_plan(int n, const reshard_layout_t* src, const reshard_layout_t* dst,
                           reshard_plan_t* out) {
  if (!out) return fail(RESHARD_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (n < 1 || !src || !dst) return fail(RESHARD_ERR_INVALID_ARGUMENT, "need n >= 1 layouts");
  reshard_plan_s* p = nullptr;
  std::string err;
  reshard_status_t st;
  try {  // no exception may cross the C ABI
    std::vector<const rs::Layout*> s(n), d(n);
    for (int t = 0; t < n; ++t) {
      if (!src[t] || !dst[t]) return fail(RESHARD_ERR_INVALID_ARGUMENT, "NULL layout");
      s[t] = &src[t]->L;
      d[t] = &dst[t]->L;
    }
    p = new reshard_plan_s();
    st = rs::build_plan(n, s.data(), d.data(), &p->host, &err);
  } catch (const std::bad_alloc&) {
    st = RESHARD_ERR_OUT_OF_MEMORY;
    err = "host memory exhausted while planning";
  }
  if (st != RESHARD_OK) {
    delete p;
    return fail(st, err);
  }
  *out = p;
  return RESHARD_OK;
}

}  // namespace

extern "C" {

int64_t reshard_dtype_size(int dtype) {
  rs::Layout L;
  std::string err;
  const int64_t one = 1;
  const int32_t rep = RESHARD_REPLICATE;
  if (!rs::make_layout(1, &one, dtype, 1, &one, &rep, &L, &err)) return 0;
  return L.elem_size;
}

reshard_status_t reshard_layout_create(int ndim, const int64_t* global_shape, int dtype,
                                       int mesh_ndim, const int64_t* mesh_shape,
                                       const int32_t* placements, reshard_layout_t* out) {
  if (!out) return fail(RESHARD_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  rs::Layout L;
  std::string err;
  if (!rs::make_layout(ndim, global_shape, dtype, mesh_ndim, mesh_shape, placements, &L, &err))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, err);
  reshard_layout_s* h = new (std::nothrow) reshard_layout_s{L};
  if (!h) return fail(RESHARD_ERR_OUT_OF_MEMORY, "layout allocation");
  *out = h;
  return RESHARD_OK;
}

reshard_status_t reshard_layout_create_strided(int ndim, const int64_t* global_shape, int dtype,
                                               int mesh_ndim, const int64_t* mesh_shape,
                                               const int32_t* placements, const int64_t* split_factors,
                                               reshard_layout_t* out) {
  if (!out) return fail(RESHARD_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (!split_factors) return fail(RESHARD_ERR_INVALID_ARGUMENT, "split_factors is NULL");
  rs::Layout L;
  std::string err;
  if (!rs::make_layout(ndim, global_shape, dtype, mesh_ndim, mesh_shape, placements, &L, &err, split_factors))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, err);
  reshard_layout_s* h = new (std::nothrow) reshard_layout_s{L};
  if (!h) return fail(RESHARD_ERR_OUT_OF_MEMORY, "layout allocation");
  *out = h;
  return RESHARD_OK;
}

void reshard_layout_destroy(reshard_layout_t layout) { delete layout; }

reshard_status_t reshard_layout_shard_runs(reshard_layout_t layout, int64_t rank, int dim, int64_t capacity,
                                           int64_t* runs, int64_t* n_runs) {
  if (!layout || !n_runs || capacity < 0 || (capacity > 0 && !runs))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "bad argument");
  if (rank < 0 || rank >= layout->L.nranks) return fail(RESHARD_ERR_INVALID_ARGUMENT, "rank out of range");
  if (dim < 0 || dim >= layout->L.ndim) return fail(RESHARD_ERR_INVALID_ARGUMENT, "dim out of range");
  const rs::Runs r = rs::shard_runs(layout->L, rank, dim);
  *n_runs = int64_t(r.size());
  for (int64_t i = 0; i < std::min<int64_t>(capacity, *n_runs); ++i) {
    runs[2 * i] = r[size_t(i)].first;
    runs[2 * i + 1] = r[size_t(i)].second;
  }
  return RESHARD_OK;
}

reshard_status_t reshard_layout_num_ranks(reshard_layout_t layout, int64_t* out) {
  if (!layout || !out) return fail(RESHARD_ERR_INVALID_ARGUMENT, "NULL argument");
  *out = layout->L.nranks;
  return RESHARD_OK;
}

reshard_status_t reshard_layout_shard_box(reshard_layout_t layout, int64_t rank, int64_t* offset,
                                          int64_t* extent) {
  if (!layout || !offset || !extent) return fail(RESHARD_ERR_INVALID_ARGUMENT, "NULL argument");
  if (rank < 0 || rank >= layout->L.nranks)
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "rank out of range");
  if (layout->L.strided)
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "a strided layout's shard is not one box: use reshard_layout_shard_runs");
  rs::Box b;
  rs::shard_box(layout->L, rank, &b);
  for (int k = 0; k < layout->L.ndim; ++k) {
    offset[k] = b.lo[k];
    extent[k] = b.hi[k] - b.lo[k];
  }
  return RESHARD_OK;
}

reshard_status_t reshard_plan_create(reshard_layout_t src, reshard_layout_t dst, reshard_plan_t* out) {
  return make_plan(1, &src, &dst, out);
}

reshard_status_t reshard_plan_create_batched(int n, const reshard_layout_t* src,
                                             const reshard_layout_t* dst, reshard_plan_t* out) {
  return make_plan(n, src, dst, out);
}

reshard_status_t reshard_plan_upload(reshard_plan_t plan, void* stream) {
  if (!plan) return fail(RESHARD_ERR_INVALID_ARGUMENT, "plan is NULL");
  std::lock_guard<std::mutex> lock(plan->mu);
  return upload_locked(plan, static_cast<hipStream_t>(stream));
}

reshard_status_t reshard_execute(reshard_plan_t plan, const void* const* src_ptrs,
                                 void* const* dst_ptrs, void* stream_arg) {
  if (!plan) return fail(RESHARD_ERR_INVALID_ARGUMENT, "plan is NULL");
  const rs::HostPlan& H = plan->host;
  reshard_status_t st = check_pointers(H, src_ptrs, dst_ptrs);
  if (st != RESHARD_OK) return st;

  hipStream_t stream = static_cast<hipStream_t>(stream_arg);
  std::lock_guard<std::mutex> lock(plan->mu);
  // Under stream capture only the launch itself may be recorded: the table
  // upload synchronises and the pointer-slot ring copies from host memory that
  // later calls rewrite, so neither may end up in a graph.
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (stream) {
    const hipError_t ce = hipStreamIsCapturing(stream, &capture);
    if (ce != hipSuccess) return hip_fail(ce, "hipStreamIsCapturing");
  }
  if (capture != hipStreamCaptureStatusNone) {
    if (!plan->uploaded)
      return fail(RESHARD_ERR_INVALID_ARGUMENT, "call reshard_plan_upload before capturing an execute");
    if (plan->n_ptrs > rs::kKargPtrs)
      return fail(RESHARD_ERR_INVALID_ARGUMENT,
                  "a plan with more than " + std::to_string(rs::kKargPtrs) +
                      " shard pointers cannot be captured into a graph");
  }
  st = upload_locked(plan, stream);
  if (st != RESHARD_OK) return st;
  if (H.descs.empty()) return RESHARD_OK;

  rs::KargPtrs karg;
  std::memset(&karg, 0, sizeof(karg));
  const void* const* table = nullptr;
  int slot = -1;
  hipError_t e;
  const uint32_t flags = alignment_flags(H, src_ptrs, dst_ptrs);
  if (plan->n_ptrs <= rs::kKargPtrs) {
    for (int64_t i = 0; i < H.n_src_ptrs; ++i) karg.p[i] = src_ptrs[i];
    for (int64_t i = 0; i < H.n_dst_ptrs; ++i) karg.p[H.n_src_ptrs + i] = dst_ptrs[i];
  } else {
    const size_t n = size_t(plan->n_ptrs);
    auto same = [&](int s) {
      void** h = plan->h_slots + size_t(s) * n;
      for (int64_t i = 0; i < H.n_src_ptrs; ++i)
        if (h[i] != src_ptrs[i]) return false;
      for (int64_t i = 0; i < H.n_dst_ptrs; ++i)
        if (h[H.n_src_ptrs + i] != dst_ptrs[i]) return false;
      return true;
    };
    if (plan->last_slot >= 0 && same(plan->last_slot)) {
      slot = plan->last_slot;  // already on the device; no copy
      // On another stream, the copy that filled the slot (and the launches that
      // read it) must come first: the ring overwrites a slot only after its
      // latest launch, so that launch has to follow every earlier one.
      if (plan->ev_live[slot] && plan->ev_stream[slot] != stream) {
        e = hipStreamWaitEvent(stream, plan->ev[slot], 0);
        if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(pointer slot)");
      }
    } else {
      slot = plan->next_slot;
      plan->next_slot = (plan->next_slot + 1) % kSlots;
      if (plan->ev_live[slot]) {  // the slot's last user must be done with it
        e = hipEventSynchronize(plan->ev[slot]);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(pointer slot)");
      }
      void** h = plan->h_slots + size_t(slot) * n;
      for (int64_t i = 0; i < H.n_src_ptrs; ++i) h[i] = const_cast<void*>(src_ptrs[i]);
      for (int64_t i = 0; i < H.n_dst_ptrs; ++i) h[H.n_src_ptrs + i] = dst_ptrs[i];
      void* d = static_cast<void**>(plan->d_slots) + size_t(slot) * n;
      e = hipMemcpyAsync(d, h, n * sizeof(void*), hipMemcpyHostToDevice, stream);
      if (e != hipSuccess) {
        plan->last_slot = -1;
        return hip_fail(e, "pointer-table copy");
      }
      plan->last_slot = slot;
    }
    table = reinterpret_cast<const void* const*>(static_cast<void**>(plan->d_slots) + size_t(slot) * n);
  }
  const hipError_t le =
      launch_groups_at(plan, static_cast<const uint8_t*>(plan->table), table, karg, flags, stream);
  if (slot >= 0) {
    // recorded even when a launch failed: the launches of a split plan that
    // went out before it may still read the slot
    e = hipEventRecord(plan->ev[slot], stream);
    if (e == hipSuccess) {
      plan->ev_live[slot] = true;
      plan->ev_stream[slot] = stream;
    } else if (le == hipSuccess) {
      return hip_fail(e, "hipEventRecord(pointer slot)");
    }
  }
  if (le != hipSuccess) return hip_fail(le, "reshard_copy_kernel launch");
  return RESHARD_OK;
}

reshard_status_t reshard_execute_noalloc(reshard_plan_t plan, const void* const* src_ptrs,
                                         void* const* dst_ptrs, void* stream_arg) {
  if (!plan) return fail(RESHARD_ERR_INVALID_ARGUMENT, "plan is NULL");
  const rs::HostPlan& H = plan->host;
  reshard_status_t st = check_pointers(H, src_ptrs, dst_ptrs);
  if (st != RESHARD_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(stream_arg);
  uint8_t* base = nullptr;
  st = scratch_of_current_device(&base);
  if (st != RESHARD_OK) return st;
  std::lock_guard<std::mutex> lock(plan->mu);
  try {
    build_image_locked(plan);
  } catch (const std::bad_alloc&) {
    return fail(RESHARD_ERR_OUT_OF_MEMORY, "host memory exhausted while building the descriptor table");
  }
  if (H.descs.empty()) return RESHARD_OK;
  const size_t img = plan->image.size();  // a multiple of 256
  const bool in_karg = plan->n_ptrs <= rs::kKargPtrs;
  const size_t need = img + (in_karg ? 0 : size_t(plan->n_ptrs) * sizeof(void*));
  if (need > kScratchBytes)
    return fail(RESHARD_ERR_INVALID_ARGUMENT,
                "plan needs " + std::to_string(need) + " bytes of table and pointers, more than the " +
                    std::to_string(kScratchBytes) + " bytes of the static scratch array");
  // The image is plan-owned and never changes, so the copy may still be in
  // flight when this call returns.
  hipError_t e = hipMemcpyAsync(base, plan->image.data(), img, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "descriptor table copy to scratch");
  rs::KargPtrs karg;
  std::memset(&karg, 0, sizeof(karg));
  const void* const* table = nullptr;
  if (in_karg) {
    for (int64_t i = 0; i < H.n_src_ptrs; ++i) karg.p[i] = src_ptrs[i];
    for (int64_t i = 0; i < H.n_dst_ptrs; ++i) karg.p[H.n_src_ptrs + i] = dst_ptrs[i];
  } else {
    // the caller's arrays: copied on the stream, then waited for, so that the
    // call has read them before it returns
    void** d = reinterpret_cast<void**>(base + img);
    if (H.n_src_ptrs) e = hipMemcpyAsync(d, src_ptrs, size_t(H.n_src_ptrs) * sizeof(void*), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess && H.n_dst_ptrs)
      e = hipMemcpyAsync(d + H.n_src_ptrs, dst_ptrs, size_t(H.n_dst_ptrs) * sizeof(void*), hipMemcpyHostToDevice,
                         stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "pointer copy to scratch");
    table = reinterpret_cast<const void* const*>(d);
  }
  e = launch_groups_at(plan, base, table, karg, alignment_flags(H, src_ptrs, dst_ptrs), stream);
  if (e != hipSuccess) return hip_fail(e, "reshard_copy_kernel launch");
  return RESHARD_OK;
}

reshard_status_t reshard_plan_stats(reshard_plan_t plan, reshard_plan_stats_t* out) {
  if (!plan || !out) return fail(RESHARD_ERR_INVALID_ARGUMENT, "NULL argument");
  const rs::HostPlan& H = plan->host;
  std::lock_guard<std::mutex> lock(plan->mu);  // the first execute may be uploading on another thread
  std::memset(out, 0, sizeof(*out));
  out->n_tensors = H.n_tensors;
  out->n_src_ptrs = H.n_src_ptrs;
  out->n_dst_ptrs = H.n_dst_ptrs;
  out->n_pieces = int64_t(H.pieces.size());
  out->n_dst_writes = H.n_dst_writes;
  out->global_bytes = H.global_bytes;
  out->bytes_read = H.bytes_read;
  out->bytes_written = H.bytes_written;
  out->n_descriptors = int64_t(H.descs.size());
  out->table_bytes = plan->uploaded ? plan->table_bytes
                                    : int64_t(H.descs.size() * sizeof(reshard_descriptor_t) + H.refs.size() * 4 +
                                              H.tile_begin.size() * 4 + H.segs.size() * sizeof(reshard_segment_t));
  if (plan->image_built)
    for (const reshard_plan_s::Launch& L : plan->launches) {
      out->n_workgroups += L.n_wg;
      out->n_launches += (int64_t(L.n_wg) + rs::kMaxLaunchBlocks - 1) / rs::kMaxLaunchBlocks;
    }
  out->plan_host_us = H.plan_host_us;
  return RESHARD_OK;
}

reshard_status_t reshard_plan_src_load(reshard_plan_t plan, int64_t capacity, int64_t* bytes,
                                       int64_t* n_total) {
  if (!plan || !n_total || capacity < 0 || (capacity > 0 && !bytes))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "bad argument");
  const rs::HostPlan& H = plan->host;
  *n_total = H.n_src_ptrs;
  for (int64_t i = 0; i < std::min<int64_t>(capacity, H.n_src_ptrs); ++i) bytes[i] = H.src_load[size_t(i)];
  return RESHARD_OK;
}

reshard_status_t reshard_plan_pieces(reshard_plan_t plan, int64_t capacity, reshard_piece_t* out,
                                     int64_t* n_total) {
  if (!plan || !n_total || capacity < 0 || (capacity > 0 && !out))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "bad argument");
  const rs::HostPlan& H = plan->host;
  *n_total = int64_t(H.pieces.size());
  for (int64_t i = 0; i < std::min<int64_t>(capacity, *n_total); ++i) {
    const rs::Piece& pc = H.pieces[i];
    reshard_piece_t& o = out[i];
    std::memset(&o, 0, sizeof(o));
    o.tensor = pc.tensor;
    o.src_rank = pc.src_rank;
    o.src_group = pc.src_group;
    o.dst_group = pc.dst_group;
    o.fanout = int64_t(H.dst_groups[pc.dst_group].ranks.size());
    const int nd = H.src[pc.tensor].ndim;
    for (int k = 0; k < nd; ++k) {
      o.lo[k] = pc.box.lo[k];
      o.hi[k] = pc.box.hi[k];
      o.src_local[k] = pc.box.lo[k] - pc.sframe.lo[k];
      o.dst_local[k] = pc.box.lo[k] - pc.dframe.lo[k];
    }
  }
  return RESHARD_OK;
}

reshard_status_t reshard_plan_device_refs(reshard_plan_t plan, int64_t capacity, uint32_t* refs, int64_t* n_refs) {
  if (!plan || !n_refs || capacity < 0 || (capacity > 0 && !refs))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "bad argument");
  std::lock_guard<std::mutex> lock(plan->mu);
  build_image_locked(plan);
  *n_refs = int64_t(plan->host.refs.size());
  const uint32_t* r = reinterpret_cast<const uint32_t*>(plan->image.data() + plan->refs_off);
  for (int64_t i = 0; i < std::min<int64_t>(capacity, *n_refs); ++i) refs[i] = r[i];
  return RESHARD_OK;
}

reshard_status_t reshard_plan_device_segments(reshard_plan_t plan, int64_t capacity, reshard_segment_t* out,
                                              int64_t* n_total) {
  if (!plan || !n_total || capacity < 0 || (capacity > 0 && !out))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "bad argument");
  std::lock_guard<std::mutex> lock(plan->mu);
  build_image_locked(plan);
  *n_total = int64_t(plan->host.segs.size());
  const reshard_segment_t* sg = reinterpret_cast<const reshard_segment_t*>(plan->image.data() + plan->segs_off);
  for (int64_t i = 0; i < std::min<int64_t>(capacity, *n_total); ++i) out[i] = sg[i];
  return RESHARD_OK;
}

reshard_status_t reshard_plan_piece_sources(reshard_plan_t plan, int64_t index, int64_t capacity,
                                            int64_t* ranks, int64_t* n_total) {
  if (!plan || !n_total || capacity < 0 || (capacity > 0 && !ranks))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "bad argument");
  const rs::HostPlan& H = plan->host;
  if (index < 0 || index >= int64_t(H.pieces.size()))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "piece index out of range");
  const rs::Piece& pc = H.pieces[index];
  const std::vector<int64_t> one{pc.src_rank};
  const std::vector<int64_t>& rk = pc.src_ranks.empty() ? one : pc.src_ranks;
  *n_total = int64_t(rk.size());
  for (int64_t i = 0; i < std::min<int64_t>(capacity, *n_total); ++i) ranks[i] = rk[i];
  return RESHARD_OK;
}

reshard_status_t reshard_plan_piece_fanout(reshard_plan_t plan, int64_t index, int64_t capacity,
                                           int64_t* ranks, int64_t* n_total) {
  if (!plan || !n_total || capacity < 0 || (capacity > 0 && !ranks))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "bad argument");
  const rs::HostPlan& H = plan->host;
  if (index < 0 || index >= int64_t(H.pieces.size()))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "piece index out of range");
  const auto& rk = H.dst_groups[H.pieces[index].dst_group].ranks;
  *n_total = int64_t(rk.size());
  for (int64_t i = 0; i < std::min<int64_t>(capacity, *n_total); ++i) ranks[i] = rk[i];
  return RESHARD_OK;
}

reshard_status_t reshard_plan_descriptors(reshard_plan_t plan, int64_t capacity,
                                          reshard_descriptor_t* out, int64_t* n_desc,
                                          int64_t ref_capacity, uint32_t* refs, int64_t* n_refs) {
  if (!plan || !n_desc || !n_refs || capacity < 0 || ref_capacity < 0 ||
      (capacity > 0 && !out) || (ref_capacity > 0 && !refs))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "bad argument");
  const rs::HostPlan& H = plan->host;
  *n_desc = int64_t(H.descs.size());
  *n_refs = int64_t(H.refs.size());
  for (int64_t i = 0; i < std::min<int64_t>(capacity, *n_desc); ++i) out[i] = H.descs[i];
  for (int64_t i = 0; i < std::min<int64_t>(ref_capacity, *n_refs); ++i) refs[i] = H.refs[i];
  return RESHARD_OK;
}

reshard_status_t reshard_plan_segments(reshard_plan_t plan, int64_t capacity, reshard_segment_t* out,
                                       int64_t* n_total) {
  if (!plan || !n_total || capacity < 0 || (capacity > 0 && !out))
    return fail(RESHARD_ERR_INVALID_ARGUMENT, "bad argument");
  const rs::HostPlan& H = plan->host;
  *n_total = int64_t(H.segs.size());
  for (int64_t i = 0; i < std::min<int64_t>(capacity, *n_total); ++i) out[i] = H.segs[i];
  return RESHARD_OK;
}

void reshard_plan_destroy(reshard_plan_t plan) {
  if (!plan) return;
  if (plan->table) (void)hipFree(plan->table);
  if (plan->d_slots) (void)hipFree(plan->d_slots);
  if (plan->h_slots) (void)hipHostFree(plan->h_slots);
  for (int s = 0; s < kSlots; ++s)
    if (plan->ev[s]) (void)hipEventDestroy(plan->ev[s]);
  delete plan;
}

const char* reshard_last_error(void) { return g_err.c_str(); }

}  // extern "C"
