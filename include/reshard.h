/*
 * reshard.h -- C ABI of the MI355X (gfx950) DTensor-to-DTensor reshard library.
 *
 * The operation.  A tensor of a given global shape is spread over a device mesh
 * by per-mesh-dim placements (Shard(k) or Replicate): the DTensor description of
 * a layout (techfeed.io write-up, "reformulation as DTensor-to-DTensor
 * transfer" section; news.bpdata.com write-up, "the approach: refit as a
 * DTensor-to-DTensor reshard" section).  A reshard takes the shards of a source
 * layout and produces the shards of a destination layout.  It first computes
 * the exact intersection of every source shard with every destination shard
 * and then moves only those overlaps (news.bpdata.com, "the Reshard
 * collective" section; the 8x8 example in which each of four column shards
 * receives one 4x2 block from each of two row shards, techfeed.io,
 * "reformulation" section).  Each overlap is read once and written to every
 * destination replica that needs it (send once, replicate locally:
 * techfeed.io, "NVIDIA's NVLink implementation" section).
 *
 * One process, one GPU.  Every source rank and destination rank is a separate
 * shard buffer in the HBM of the GPU that is current when the plan is first
 * executed.  The library computes the plan on the host, keeps a copy-descriptor
 * table in device memory, and runs one fused copy kernel per execute (a few launches
 * when a plan mixes WINDOW bands with other descriptors: see n_launches).
 *
 * Layout semantics (readings the library fixes where the pages are silent):
 *   - placement codes: RESHARD_REPLICATE (-1) or k >= 0 for Shard(k);
 *   - ranks are numbered row-major over mesh coordinates;
 *   - Shard(k) splits like torch.chunk: chunk = ceil(n / mesh_size); trailing
 *     ranks may hold a short or an empty (zero-size) shard;
 *   - several mesh dims that shard the same tensor dim nest left to right;
 *   - each local shard is a contiguous row-major buffer whose shape is the
 *     extent of its box (reshard_layout_shard_box);
 *   - right-to-left (strided) nesting: reshard_layout_create_strided;
 *   - Partial (sum) sources: a source mesh dim with placement RESHARD_PARTIAL
 *     splits nothing; each of its coordinates holds a full-size contribution
 *     of the same box, and the tensor is their elementwise sum (DTensor's
 *     Partial("sum")).  With several Partial mesh dims the contributions are
 *     numbered q = 0, 1, ... row-major over their coordinates.  The sum is taken
 *     in binary32 in ascending q: it starts from contribution 0, widened
 *     exactly, adds each next one with one rounding to nearest even, and is
 *     rounded once more to the destination dtype.  Sources are F32, BF16 or F16;
 *     the destination dtype is the source's or one of its conversions below.
 *     A destination with Partial, or Partial with split factors, is refused
 *     (RESHARD_ERR_LAYOUT_MISMATCH).  The pages say only that the refit guide
 *     lists the supported layouts (news.bpdata.com write-up, "practical access
 *     and setup" section).
 * The copy is bytewise: bf16/fp32 NaN payloads, -0.0 and subnormals arrive
 * unchanged.  Source and destination dtypes match, or the pair is one of the
 * float conversions below.
 *
 * Converting reshard.  The pages mention that the refit supports precision
 * modes and say nothing more (the news.bpdata.com and techfeed.io write-ups,
 * closing remarks on the refit guide).  The reading taken: a destination layout
 * may hold another float format than the source (say fp32 training weights,
 * bf16 inference weights).  Supported pairs: F32 -> BF16, F32 -> F16 (round to
 * nearest, ties to even, overflow to infinity) and BF16 -> F32, F16 -> F32
 * (exact).  A NaN stays a NaN with its sign and leading payload bits and with
 * the quiet bit set.  Conversion happens in the copy kernel, element by element,
 * once per destination element; everything else is as for a plain reshard.
 *
 * Errors.  Every call returns a reshard_status_t and never throws; on failure
 * reshard_last_error() gives a message for the calling thread.
 */
#ifndef RESHARD_H_
#define RESHARD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RESHARD_MAX_NDIM 8       /* tensor dims supported */
#define RESHARD_MAX_MESH_NDIM 8  /* mesh dims supported */
#define RESHARD_REPLICATE (-1)   /* placement code for Replicate */
#define RESHARD_PARTIAL (-2)     /* placement code for Partial (sum), source layouts only */

typedef enum reshard_status {
  RESHARD_OK = 0,
  RESHARD_ERR_INVALID_ARGUMENT = 1, /* bad shape, mesh, placement, dtype, rank or NULL out-pointer */
  RESHARD_ERR_LAYOUT_MISMATCH = 2,  /* source and destination disagree on global shape, or on dtype
                                       outside the supported conversions */
  RESHARD_ERR_NULL_SHARD = 3,       /* NULL pointer passed for a non-empty shard */
  RESHARD_ERR_OUT_OF_MEMORY = 4,    /* host or device allocation failed */
  RESHARD_ERR_HIP = 5,              /* a HIP runtime call failed (no device, launch error, ...) */
  RESHARD_ERR_DEVICE_MISMATCH = 6,  /* executed on a device other than the plan's */
} reshard_status_t;

/* Element types.  Only the element size matters to a copy without conversion. */
typedef enum reshard_dtype {
  RESHARD_DTYPE_U8 = 0,
  RESHARD_DTYPE_I8 = 1,
  RESHARD_DTYPE_BOOL = 2,
  RESHARD_DTYPE_FP8_E4M3 = 3,
  RESHARD_DTYPE_FP8_E5M2 = 4,
  RESHARD_DTYPE_BF16 = 5,
  RESHARD_DTYPE_F16 = 6,
  RESHARD_DTYPE_I16 = 7,
  RESHARD_DTYPE_F32 = 8,
  RESHARD_DTYPE_I32 = 9,
  RESHARD_DTYPE_F64 = 10,
  RESHARD_DTYPE_I64 = 11,
} reshard_dtype_t;

typedef struct reshard_layout_s* reshard_layout_t; /* immutable after create */
typedef struct reshard_plan_s* reshard_plan_t;     /* immutable plan + its device table */

/* Plan statistics; all byte counts are for one execute. */
typedef struct reshard_plan_stats {
  int64_t n_tensors;      /* tensors in the plan (1 unless batched) */
  int64_t n_src_ptrs;     /* length of the src_ptrs array reshard_execute expects */
  int64_t n_dst_ptrs;     /* length of the dst_ptrs array reshard_execute expects */
  int64_t n_pieces;       /* source box x unique destination box overlaps */
  int64_t n_dst_writes;   /* sum over pieces of their destination fan-out */
  int64_t global_bytes;   /* sum over tensors of the global tensor's bytes in the source dtype (G) */
  int64_t bytes_read;     /* bytes the kernel reads  (= G: each element once; times the
                             number of contributions for a Partial source) */
  int64_t bytes_written;  /* bytes the kernel writes (= sum of destination shard bytes, in the
                             destination dtype) */
  int64_t n_descriptors;  /* device copy descriptors after dim merging / splitting */
  int64_t table_bytes;    /* size of the device-resident descriptor table (once uploaded: as
                             allocated, with padding and one tile list per launch group) */
  int64_t n_workgroups;   /* workgroups of one execute, about one per tile (0 until the first
                             upload or execute) */
  int64_t n_launches;     /* kernel launches of one execute (0 until the first upload or execute):
                             the descriptors that
                             are not WINDOW bands share one launch group and each kind of band
                             (the kernel build that moves it) is a group of its own; a group of
                             more than 16,777,208 workgroups goes out as several launches of at
                             most that many */
  double plan_host_us;    /* host time spent planning in reshard_plan_create* */
} reshard_plan_stats_t;

/* One planned overlap, in global coordinates (inspection API). */
typedef struct reshard_piece {
  int64_t tensor;                 /* tensor index inside the plan */
  int64_t src_rank;               /* source rank the replica choice picks for it (a tensor
                                     moved as window bands reads a replicated box in row
                                     parts, one per replica, instead: reshard_plan_src_load
                                     counts what is read) */
  int64_t src_group;              /* index of the unique source box it belongs to */
  int64_t dst_group;              /* index of the unique destination box it feeds */
  int64_t fanout;                 /* destination ranks written (replicas of dst_group) */
  int64_t lo[RESHARD_MAX_NDIM];   /* box [lo, hi) of the overlap, global coordinates */
  int64_t hi[RESHARD_MAX_NDIM];
  int64_t src_local[RESHARD_MAX_NDIM]; /* where the box starts in the source rank's buffer, local
                                          coordinates (lo - the box's offset for a plain layout) */
  int64_t dst_local[RESHARD_MAX_NDIM]; /* the same in every destination replica's buffer */
} reshard_piece_t;

/* Descriptor modes. */
#define RESHARD_DESC_ITEMS 0      /* rows of items of `unit` bytes (unit = 16, or short rows) */
#define RESHARD_DESC_DST_CHUNKS 1 /* rows cut into 16-byte chunks aligned to the destination */
#define RESHARD_DESC_WINDOW 2     /* a band of rows staged through LDS (see below) */
#define RESHARD_DESC_CONVERT 3    /* rows of elements converted to another float format */
#define RESHARD_DESC_GATHER_ROWS 4 /* whole destination rows gathered from column segments */
#define RESHARD_DESC_REDUCE 5     /* rows of elements summed over Partial contributions */

/* Conversions (the `unit` field of a RESHARD_DESC_CONVERT descriptor). */
#define RESHARD_CONVERT_F32_BF16 1
#define RESHARD_CONVERT_F32_F16 2
#define RESHARD_CONVERT_BF16_F32 3
#define RESHARD_CONVERT_F16_F32 4
#define RESHARD_CONVERT_ELEMS 8   /* elements per item of a RESHARD_DESC_CONVERT row */

/*
 * Device copy descriptor (the table the kernel reads; inspection API).
 * A descriptor copies rows of `run_bytes` contiguous bytes.  Rows are indexed by
 * up to three outer dims (extent[0] outermost); a row's first byte is
 *   base + offset + i0*stride[0] + i1*stride[1] + i2*stride[2]
 * on each side, base being the shard pointer.  The kernel indexes `row_items`
 * items per row:
 *   RESHARD_DESC_ITEMS       item c is bytes [c*unit, (c+1)*unit) of the row;
 *                            row_items = run_bytes / unit.
 *   RESHARD_DESC_DST_CHUNKS  item c is the part of the row inside the c-th 16-byte
 *                            aligned destination block the row touches (empty,
 *                            partial or full); row_items = ceil((run_bytes+15)/16);
 *                            `unit` is the row's natural alignment (1..8 bytes).
 *   RESHARD_DESC_WINDOW      a band of `extent[0]` rows of a 2-d view of one
 *                            tensor (rows x inner dim), `run_bytes` wide, moved
 *                            `extent[1]` rows per tile through an LDS window of
 *                            pitch `row_items`.  Its segments are
 *                            segments[src_ptr .. src_ptr + dst_ref_begin) (sources,
 *                            read into the window) followed by `fanout` destination
 *                            segments (written from it), each side in column
 *                            order; offsets and strides are ignored.  Used for
 *                            narrow or misaligned pieces.  A band more than 16
 *                            bytes wide whose segments are all packed (row
 *                            stride = width) moves in a narrow-band kernel
 *                            build, each segment's rows as one contiguous
 *                            stream on the global side, with `extent[1]` rows
 *                            per tile within an 18 KiB window (36 KiB when a
 *                            destination segment would get less than 1 KiB a
 *                            tile or is one or two bytes wide, or a tile would
 *                            have fewer than 64 rows: then twice the rows, in a
 *                            launch of its own).  So do packed bands of at most
 *                            16 bytes with a 1- or 2-byte segment, a source
 *                            segment of 3 to 15 bytes (not 4 or 8) that is not
 *                            dword-granular, or such a destination segment of 5
 *                            bytes or more.
 *                            Other bands at most 16 bytes wide skip LDS: one
 *                            lane per row assembles the row in registers,
 *                            `extent[1]` = 1024 rows per tile (512 when one
 *                            side is four packed 4-byte column runs, which the
 *                            four lanes of a quad exchange, or eight packed
 *                            2-byte runs, which eight lanes exchange; a band
 *                            of at most 16 bytes on the narrow-band build takes
 *                            the largest power of two up to 1024 whose window
 *                            fits, doubled as above).  Each band kind runs in
 *                            a launch of its own, whatever the rest of the plan
 *                            holds (n_launches counts them).
 *   RESHARD_DESC_GATHER_ROWS `extent[0]` whole rows of `run_bytes` bytes, packed in
 *                            every destination replica from byte `dst_offset`
 *                            on, gathered from `extent[1]` source segments
 *                            (segments[src_ptr ...], in column order, tiling
 *                            the row; each at least 1024 bytes wide) and
 *                            written to the `fanout` shards listed in the
 *                            fan-out list from `dst_ref_begin`.  The kernel
 *                            walks the destination rows in 16-byte blocks, so
 *                            no destination line is written in part by two
 *                            workgroups where source column strips meet at an
 *                            address that is not 16-byte aligned.  magic[0]
 *                            divides by `run_bytes`.  When row_items is 1,
 *                            src_offset, src_stride and dst_stride hold, as 28
 *                            uint16 in that order, a segment lookup: entry k
 *                            covers row bytes [1024 k, 1024 k + 1024) and holds
 *                            the index of the segment at byte 1024 k (low 6
 *                            bits) and the offset inside the KiB where the
 *                            next segment starts (high 10 bits, 0 for none).
 *                            row_items 0: no lookup, the kernel searches.
 *   RESHARD_DESC_CONVERT     rows of `run_bytes` ELEMENTS (not bytes) converted by
 *                            conversion `unit`; item c is elements
 *                            [c*8, min(c*8+8, run)) of the row; row_items =
 *                            ceil(run / 8).  Offsets and strides are in bytes of
 *                            each side's own dtype.
 *   RESHARD_DESC_REDUCE      rows and items as RESHARD_DESC_CONVERT, each element
 *                            the binary32 sum, in list order, of the same element
 *                            of n contributions (Partial sources), rounded to the
 *                            destination format.  The contributions' source
 *                            pointer slots are refs[src_ptr .. src_ptr + n) of
 *                            the fan-out list (all at the same offsets); `unit`
 *                            holds n in bits 0-11, the source format in bits
 *                            12-13 and the destination format in bits 14-15
 *                            (0 binary32, 1 bfloat16, 2 binary16).
 */
typedef struct reshard_descriptor {
  int64_t src_offset;       /* byte offset of the row origin in the source shard */
  int64_t dst_offset;       /* byte offset of the row origin in each destination shard */
  int64_t src_stride[3];    /* bytes, outer dims; unused dims have extent 1 */
  int64_t dst_stride[3];
  uint32_t extent[3];       /* outer extents; product = rows */
  uint32_t run_bytes;       /* contiguous bytes per row, both sides (CONVERT: elements) */
  uint32_t row_items;       /* items the kernel indexes per row (see the modes) */
  uint16_t unit;            /* item size (ITEMS), natural alignment (DST_CHUNKS, WINDOW) or
                               conversion (CONVERT) */
  uint16_t mode;            /* RESHARD_DESC_* */
  uint32_t src_ptr;         /* index into the execute's source pointer array */
  uint32_t dst_ref_begin;   /* first entry of this descriptor's fan-out list */
  uint32_t fanout;          /* destination pointers written */
  uint32_t magic[3][2];     /* division constants for row_items, extent[2], extent[1] */
  uint32_t piece;           /* index of the planned piece it copies (or part of) */
} reshard_descriptor_t;

/*
 * One segment of a RESHARD_DESC_WINDOW band (inspection API): rows of `width`
 * bytes at window column `col`; row r of the band is at byte
 * offset + r * row_stride of its shard.  A source segment (fanout 0) reads shard
 * `ptr` of the source pointer array; a destination segment writes the `fanout`
 * destination shards listed in the fan-out list from entry `ptr`.
 */
typedef struct reshard_segment {
  int64_t offset;      /* byte offset of the band's first row in the shard */
  int64_t row_stride;  /* bytes between consecutive rows in the shard */
  uint32_t col;        /* first byte column inside the window */
  uint32_t width;      /* bytes per row */
  uint32_t ptr;        /* source pointer index, or first fan-out entry */
  uint32_t fanout;     /* 0 for a source segment, else destination replicas */
} reshard_segment_t;

/* Bytes per element of `dtype`, or 0 if unknown. */
int64_t reshard_dtype_size(int dtype);

/*
 * Describe a layout.  global_shape[ndim] (extents >= 0, 1 <= ndim <= 8),
 * mesh_shape[mesh_ndim] (sizes >= 1, 1 <= mesh_ndim <= 8), placements[mesh_ndim]
 * (RESHARD_REPLICATE or a tensor dim).  Arrays are copied; *out receives a new
 * handle owned by the caller (free with reshard_layout_destroy).
 * Errors: RESHARD_ERR_INVALID_ARGUMENT.
 */
reshard_status_t reshard_layout_create(int ndim, const int64_t* global_shape, int dtype,
                                       int mesh_ndim, const int64_t* mesh_shape,
                                       const int32_t* placements, reshard_layout_t* out);
void reshard_layout_destroy(reshard_layout_t layout); /* NULL is a no-op */

/*
 * A layout with right-to-left ("strided") nesting.  The pages say only that
 * the refit guide lists the supported layouts (news.bpdata.com write-up,
 * "practical access and setup" section); the placement follows PyTorch
 * DTensor's _StridedShard(k, split_factor), used by FSDP2 + TP when the TP
 * mesh dim splits a tensor dim before the FSDP mesh dim does.
 *   split_factors[mesh_ndim]  one factor f >= 1 per mesh dim; f > 1 only where
 *                             placements[m] is a tensor dim (f = 1 is a plain
 *                             Shard or Replicate: with all ones this is
 *                             reshard_layout_create).
 * At mesh dim m with factor f, a rank's current index list along dim k (what
 * the mesh dims to its left left it, length n) is cut into f ceil-chunks
 * (chunk = ceil(n / f), trailing ones short or empty); each of those is cut into
 * mesh_shape[m] ceil-chunks, and coordinate c keeps part c of every one of the f
 * chunks, in order.  Mesh dims still apply left to right.  Example: 8 rows on a
 * 2x2 mesh with placements {0, 0} and split factors {2, 1} give ranks 0..3 rows
 * {0,1}, {4,5}, {2,3}, {6,7}.  A rank's shard is then, along each dim, a list of
 * runs of global indices (reshard_layout_shard_runs), and its local buffer is
 * the contiguous row-major buffer over the product of those lists, runs in
 * global order.  Other arguments, ownership and errors as reshard_layout_create.
 */
reshard_status_t reshard_layout_create_strided(int ndim, const int64_t* global_shape, int dtype,
                                               int mesh_ndim, const int64_t* mesh_shape,
                                               const int32_t* placements, const int64_t* split_factors,
                                               reshard_layout_t* out);

/* Number of ranks (product of the mesh shape). */
reshard_status_t reshard_layout_num_ranks(reshard_layout_t layout, int64_t* out);

/*
 * Runs of global indices that `rank` holds along tensor dim `dim`, any layout:
 * writes min(capacity, count) runs as (lo, hi) pairs to runs[2 * capacity] and
 * the count to *n_runs (0: the shard is empty).  The runs are increasing and do
 * not touch; the shard's local extent along `dim` is the sum of their lengths.
 * A plain layout has one run per non-empty dim.  Errors:
 * RESHARD_ERR_INVALID_ARGUMENT (NULL, rank or dim out of range).
 */
reshard_status_t reshard_layout_shard_runs(reshard_layout_t layout, int64_t rank, int dim, int64_t capacity,
                                           int64_t* runs, int64_t* n_runs);

/*
 * Box held by `rank`: offset[ndim] (global start) and extent[ndim] (local shape,
 * may contain zeros for an empty shard).  Errors: RESHARD_ERR_INVALID_ARGUMENT,
 * also for a layout with a split factor above 1 (its shards are not boxes).
 */
reshard_status_t reshard_layout_shard_box(reshard_layout_t layout, int64_t rank,
                                          int64_t* offset, int64_t* extent);

/*
 * Plan the reshard of one tensor from layout src to layout dst (same global
 * shape; same dtype or a supported conversion).  The pages define the
 * operation this plans: the transfer pattern follows from the two DTensor
 * descriptions alone, by computing every source shard's overlap with every
 * destination shard before any data moves (news.bpdata.com write-up, "the
 * Reshard collective" section; techfeed.io write-up, "reformulation" section,
 * whose 8x8 example has each of four column shards receive one 4x2 block from
 * each of two row shards).  Host-only: intersects every source box with every
 * unique destination box, picks one source replica per overlap (least-loaded
 * first: replicated weights can be read at any of their holders, news.bpdata.com,
 * "the approach" section; in a tensor moved as window bands each replica of a
 * box reads a near-equal part of its rows), merges contiguous dims and builds the descriptor
 * table.  The layouts may be destroyed afterwards.  The device table is
 * uploaded by reshard_plan_upload or by the first reshard_execute.
 * Errors: RESHARD_ERR_INVALID_ARGUMENT, RESHARD_ERR_LAYOUT_MISMATCH,
 * RESHARD_ERR_OUT_OF_MEMORY.
 */
reshard_status_t reshard_plan_create(reshard_layout_t src, reshard_layout_t dst,
                                     reshard_plan_t* out);

/*
 * Plan n tensors that are moved together by one execute (one fused kernel launch,
 * or a few when band descriptors are mixed with other descriptors: see
 * n_launches).  A refit moves every weight of a model in one collective call
 * (techfeed.io write-up, "reformulation" section: one call given the two
 * DTensor descriptions; news.bpdata.com, "integration and hybrid solution in
 * NeMo RL" section: the FFN projections, about 95% of the payload, go through
 * the reshard together).  Pointer arrays of reshard_execute are then
 * concatenated tensor-major: tensor 0's ranks first, each tensor's ranks in
 * row-major mesh order.  Errors as reshard_plan_create.
 */
reshard_status_t reshard_plan_create_batched(int n, const reshard_layout_t* src,
                                             const reshard_layout_t* dst, reshard_plan_t* out);

/*
 * Upload the descriptor table to the current HIP device (once; later calls are
 * no-ops) using `stream` (a hipStream_t; NULL = default stream).  Synchronises
 * with the upload before returning.
 * Errors: RESHARD_ERR_HIP, RESHARD_ERR_OUT_OF_MEMORY, RESHARD_ERR_DEVICE_MISMATCH.
 */
reshard_status_t reshard_plan_upload(reshard_plan_t plan, void* stream);

/*
 * Run the reshard on `stream` (hipStream_t, NULL = default stream); asynchronous.
 * Every planned overlap is read once from its source shard and written to every
 * destination replica that holds it: the single-GPU form of sending each
 * contribution once and replicating it inside the destination domain
 * (techfeed.io write-up, "NVIDIA's NVLink implementation" section;
 * news.bpdata.com, "the Reshard collective" section).  Only the overlaps move,
 * so the bytes written equal the destination shards' bytes, with no gathered
 * copy of the full tensor in between (techfeed.io, "core problem" section).
 *   src_ptrs[n_src_ptrs]  device pointers to the source shards (read only)
 *   dst_ptrs[n_dst_ptrs]  device pointers to the destination shards (written)
 * Pointers are borrowed: keep the buffers alive until the stream has passed the
 * work.  NULL is allowed only for empty shards.  Sources and destinations must
 * not overlap.  The plan's n_launches kernel launches (one unless WINDOW bands
 * are mixed with other descriptors), back to back on `stream`, move every piece
 * of every tensor; if one of them fails to launch, the ones before it may still
 * run and the error is returned.  When the
 * pointer arrays exceed the kernel-argument capacity they are first copied to a
 * plan-owned device slot with one asynchronous host-to-device copy.  Device
 * faults surface at the caller's next synchronisation, as with any HIP launch.
 * Calls on several streams may overlap.
 * Graph capture: an execute may be captured into a HIP graph (stream capture
 * on `stream`) when the plan was uploaded beforehand and its pointer arrays fit
 * in the kernel arguments (n_src_ptrs + n_dst_ptrs <= 120); the graph then holds
 * n_launches kernel nodes with the pointers given at capture time.  Otherwise a
 * capturing call records nothing and fails with RESHARD_ERR_INVALID_ARGUMENT.
 * Errors: RESHARD_ERR_INVALID_ARGUMENT, RESHARD_ERR_NULL_SHARD, RESHARD_ERR_HIP,
 * RESHARD_ERR_DEVICE_MISMATCH, RESHARD_ERR_OUT_OF_MEMORY.
 */
reshard_status_t reshard_execute(reshard_plan_t plan, const void* const* src_ptrs,
                                 void* const* dst_ptrs, void* stream);

/*
 * reshard_execute without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The same kernels run; the plan's descriptor table and,
 * when src + dst pointers exceed the kernel-argument capacity (120), the
 * pointer arrays go into a static device array of the library
 * (RESHARD_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends) instead
 * of memory the library allocates.  The table is copied there on `stream`
 * before the launches of every call; nothing in it must start at zero.
 * Arguments, pointer rules and asynchrony are those of reshard_execute, except:
 *   - every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents: calls whose work overlaps on one GPU (other streams,
 *     other threads, any plan) race and may read each other's table; calls in
 *     order on one stream are safe;
 *   - with more than 120 pointers the call waits for `stream` to finish the
 *     pointer copy (and everything enqueued before it) before returning;
 *   - a plan whose table plus pointer arrays exceed the array is refused with
 *     RESHARD_ERR_INVALID_ARGUMENT.
 * It neither uploads the plan nor uses an uploaded table.
 * Errors: RESHARD_ERR_INVALID_ARGUMENT, RESHARD_ERR_NULL_SHARD, RESHARD_ERR_HIP.
 */
#define RESHARD_NOALLOC_SCRATCH_BYTES (2u << 20)
reshard_status_t reshard_execute_noalloc(reshard_plan_t plan, const void* const* src_ptrs,
                                         void* const* dst_ptrs, void* stream);

/* Statistics of the plan (one execute's bytes, pieces, launches; see the struct). */
reshard_status_t reshard_plan_stats(reshard_plan_t plan, reshard_plan_stats_t* out);

/*
 * Inspection: bytes the kernel reads from each source pointer slot of one
 * execute (the load the replica choice balances; replicated sources share the
 * reads of their box: news.bpdata.com write-up, "the approach" section).
 * Copies up to `capacity` entries, in the order of the src_ptrs array, into
 * bytes[] and the slot count (n_src_ptrs) into *n_total.  Slots of empty or
 * unread replicas hold 0.  bytes may be NULL when capacity is 0.
 * Errors: RESHARD_ERR_INVALID_ARGUMENT.
 */
reshard_status_t reshard_plan_src_load(reshard_plan_t plan, int64_t capacity, int64_t* bytes,
                                       int64_t* n_total);

/*
 * Inspection: copy up to `capacity` pieces into out[] and the total count into
 * *n_total (out may be NULL when capacity is 0).
 */
reshard_status_t reshard_plan_pieces(reshard_plan_t plan, int64_t capacity,
                                     reshard_piece_t* out, int64_t* n_total);

/*
 * Inspection: the fan-out list as the kernel reads it from the device table,
 * host-side (builds the table image if needed; no device call).  Entries are
 * absolute slots of the pointer array the kernel indexes (src_ptrs first,
 * then dst_ptrs): n_src_ptrs + the reshard_plan_descriptors entry for a
 * destination, the entry itself for a REDUCE descriptor's contributions.
 * Writes min(capacity, count) entries and the count.  Errors:
 * RESHARD_ERR_INVALID_ARGUMENT.
 */
reshard_status_t reshard_plan_device_refs(reshard_plan_t plan, int64_t capacity, uint32_t* refs,
                                          int64_t* n_refs);

/*
 * Inspection: the segment table as the kernel reads it from the device table,
 * host-side (no device call).  It equals reshard_plan_segments except in the
 * destination segments of the bands that the narrow-band kernel builds move
 * (packed bands: every segment's row stride is its width): there row_stride
 * holds the absolute pointer slot of the segment's first replica instead.  Writes min(capacity, count) segments and the count.
 * Errors: RESHARD_ERR_INVALID_ARGUMENT.
 */
reshard_status_t reshard_plan_device_segments(reshard_plan_t plan, int64_t capacity, reshard_segment_t* out,
                                              int64_t* n_total);

/* Source ranks (within the piece's tensor) that piece `index` reads, in
 * contribution order: one for a plain source, one per contribution for a
 * Partial source (the first is the piece's src_rank).  Writes min(capacity,
 * count) ranks and the count.  Errors: RESHARD_ERR_INVALID_ARGUMENT. */
reshard_status_t reshard_plan_piece_sources(reshard_plan_t plan, int64_t index, int64_t capacity,
                                            int64_t* ranks, int64_t* n_total);

/* Destination ranks (within the piece's tensor) that piece `index` is written to. */
reshard_status_t reshard_plan_piece_fanout(reshard_plan_t plan, int64_t index, int64_t capacity,
                                           int64_t* ranks, int64_t* n_total);

/*
 * Inspection: copy the descriptor table (up to `capacity` entries) and the
 * fan-out reference list (indices into the destination pointer array, except
 * a REDUCE descriptor's list of contributions at src_ptr, which indexes the
 * source pointer array; up to `ref_capacity` entries).  Totals go to *n_desc
 * and *n_refs.
 */
reshard_status_t reshard_plan_descriptors(reshard_plan_t plan, int64_t capacity,
                                          reshard_descriptor_t* out, int64_t* n_desc,
                                          int64_t ref_capacity, uint32_t* refs,
                                          int64_t* n_refs);

/* Inspection: copy up to `capacity` window segments; the total goes to *n_total. */
reshard_status_t reshard_plan_segments(reshard_plan_t plan, int64_t capacity,
                                       reshard_segment_t* out, int64_t* n_total);

/* Free the plan and its device memory.  No execute using it may be in flight.  NULL is a no-op. */
void reshard_plan_destroy(reshard_plan_t plan);

/* Message of the calling thread's last failed call ("" if none).  Valid until its next call. */
const char* reshard_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RESHARD_H_ */
