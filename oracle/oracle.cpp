/*
 * CPU oracle for the DTensor-to-DTensor reshard.  TEST INFRASTRUCTURE ONLY:
 * the tests, the smoke check and the CPU-baseline leg of the benchmark may load
 * it; the product library never does.  It shares no code, header or constant
 * with the GPU path.
 *
 * What it computes ("gather, then keep your slice"):
 *   The reshard pages describe the usual refit path as: all-gather every full
 *   parameter from the training shards, broadcast it, and let every inference
 *   GPU keep only its own shard ("Accelerating RL Weight Refit with the Reshard
 *   Collective" write-ups: techfeed.io, "core problem" section; news.bpdata.com,
 *   "why is weight refit a problem" section).  Reshard must reach exactly the
 *   same destination bytes while moving only the overlaps.  This file runs that
 *   baseline scheme on the host:
 *     1. X[box(src, s)] = src_shard[s] for every source rank s (the gather);
 *     2. dst_shard[d]   = X[box(dst, d)] for every destination rank d (the slice).
 *
 * Layout model (DTensor: global shape + device mesh + placements; techfeed.io,
 * "reformulation" section; news.bpdata.com, "the approach" section):
 *   - a placement is Replicate (code -1) or Shard(k) (code k >= 0);
 *   - ranks are numbered row-major over mesh coordinates;
 *   - Shard uses torch.chunk ceil-splitting: chunk = ceil(n / mesh_size), so
 *     trailing ranks may get a short or empty piece;
 *   - several mesh dims sharding the same tensor dim nest left to right, each
 *     splitting the interval left by the previous one;
 *   - a local shard is stored contiguous row-major with the box's extents.
 *   The pages say only "sharded"; the split rule and the nesting order are the
 *   readings this project takes (they match PyTorch DTensor's own rule).
 *
 * Checks made while gathering: a replicated source rank must hold bytes equal
 * to what an earlier replica already put into X, and at the end every global
 * element must have been covered exactly R_src times, R_src being the product
 * of the mesh sizes of the source's Replicate dims.
 *
 * Element conversion (oracle_convert) serves a reshard whose destination dtype
 * differs from the source's; see the comment above that function.
 *
 * Strided (right-to-left) nesting is a separate, plainer path: index_list and
 * oracle_reshard_indexed keep every rank's shard as one explicit list of global
 * indices per tensor dim and move element by element; see the comment above
 * index_list.
 *
 * Partial sources (oracle_reshard_partial) sum their partial tensors; see the
 * comment above that function.
 *
 * Built with g++ (plain C++17, std::thread); no HIP.
 */
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

namespace {

constexpr int kMaxDims = 8;
constexpr int32_t kReplicate = -1;

enum OracleStatus {
  ORACLE_OK = 0,
  ORACLE_BAD_LAYOUT = 1,
  ORACLE_REPLICA_MISMATCH = 2,
  ORACLE_COVERAGE_MISMATCH = 3,
  ORACLE_NO_MEMORY = 4,
  ORACLE_NULL_BUFFER = 5,
};

struct Layout {
  int ndim;
  const int64_t* shape;
  int mesh_ndim;
  const int64_t* mesh;
  const int32_t* placements;
};

bool layout_ok(const Layout& L) {
  if (L.ndim < 1 || L.ndim > kMaxDims) return false;
  if (L.mesh_ndim < 1 || L.mesh_ndim > kMaxDims) return false;
  for (int k = 0; k < L.ndim; ++k)
    if (L.shape[k] < 0) return false;
  for (int m = 0; m < L.mesh_ndim; ++m) {
    if (L.mesh[m] < 1) return false;
    int32_t p = L.placements[m];
    if (p != kReplicate && (p < 0 || p >= L.ndim)) return false;
  }
  return true;
}

int64_t num_ranks(const Layout& L) {
  int64_t n = 1;
  for (int m = 0; m < L.mesh_ndim; ++m) n *= L.mesh[m];
  return n;
}

/* Box [lo, hi) of `rank` under layout L. */
void box_of(const Layout& L, int64_t rank, int64_t* lo, int64_t* hi) {
  int64_t coord[kMaxDims];
  int64_t r = rank;
  for (int m = L.mesh_ndim - 1; m >= 0; --m) {  // row-major mesh order
    coord[m] = r % L.mesh[m];
    r /= L.mesh[m];
  }
  for (int k = 0; k < L.ndim; ++k) {
    lo[k] = 0;
    hi[k] = L.shape[k];
  }
  for (int m = 0; m < L.mesh_ndim; ++m) {  // nest left to right
    int32_t p = L.placements[m];
    if (p == kReplicate) continue;
    int64_t n = hi[p] - lo[p];
    int64_t chunk = (n + L.mesh[m] - 1) / L.mesh[m];  // ceil(n / mesh size)
    int64_t a = lo[p] + coord[m] * chunk;
    int64_t b = a + chunk;
    int64_t end = hi[p];
    lo[p] = a < end ? a : end;
    hi[p] = b < end ? b : end;
  }
}

bool box_empty(int ndim, const int64_t* lo, const int64_t* hi) {
  for (int k = 0; k < ndim; ++k)
    if (hi[k] <= lo[k]) return true;
  return false;
}

/*
 * Strided nesting.  The reshard write-ups say only that the refit guide lists
 * the supported layouts (news.bpdata.com write-up, "practical access and setup"
 * section).  The reading taken is PyTorch DTensor's right-to-left placement
 * (_StridedShard(k, split_factor)), which FSDP2 + TP use when the TP mesh dim
 * splits a tensor dim before the FSDP mesh dim does.  At mesh dim m with split
 * factor f (f = 1 is a plain Shard(k)), a rank's current list of global indices
 * along dim k, of length n, is cut into f torch.chunk pieces (size ceil(n / f),
 * the trailing ones short or missing); each piece is cut the same way into
 * mesh[m] parts; the rank keeps part coord[m] of every piece, pieces in order.
 * Mesh dims apply left to right, each to the list the previous ones left.
 * The local shard is the row-major buffer over the product of the per-dim lists.
 */
std::vector<int64_t> index_list(const Layout& L, const int64_t* split, int64_t rank, int dim) {
  int64_t coord[kMaxDims];
  int64_t rest = rank;
  for (int m = L.mesh_ndim; m-- > 0;) {  // the last mesh dim varies fastest
    coord[m] = rest % L.mesh[m];
    rest /= L.mesh[m];
  }
  std::vector<int64_t> cur;
  for (int64_t i = 0; i < L.shape[dim]; ++i) cur.push_back(i);
  for (int m = 0; m < L.mesh_ndim; ++m) {
    if (L.placements[m] != dim) continue;
    const int64_t n = (int64_t)cur.size();
    const int64_t f = split[m];
    const int64_t piece = (n + f - 1) / f;  // ceil(n / f)
    std::vector<int64_t> kept;
    for (int64_t j = 0; j < f; ++j) {
      const int64_t start = j * piece;
      if (start >= n) break;  // torch.chunk made fewer pieces: the rest are empty
      const int64_t len = n - start < piece ? n - start : piece;
      const int64_t part = (len + L.mesh[m] - 1) / L.mesh[m];  // ceil(len / mesh size)
      for (int64_t p = coord[m] * part; p < (coord[m] + 1) * part && p < len; ++p)
        kept.push_back(cur[start + p]);
    }
    cur = kept;
  }
  return cur;
}

bool split_ok(const Layout& L, const int64_t* split) {
  for (int m = 0; m < L.mesh_ndim; ++m) {
    if (split[m] < 1) return false;
    if (split[m] > 1 && L.placements[m] == kReplicate) return false;
  }
  return true;
}

/* Run fn(row_begin, row_end) over [0, rows) split into `threads` contiguous parts. */
template <class Fn>
void parallel_rows(int64_t rows, int threads, Fn fn) {
  if (threads <= 1 || rows < 2 * (int64_t)threads) {
    fn((int64_t)0, rows);
    return;
  }
  std::vector<std::thread> pool;
  int64_t per = (rows + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    int64_t a = t * per, b = a + per < rows ? a + per : rows;
    if (a >= b) break;
    pool.emplace_back(fn, a, b);
  }
  for (auto& th : pool) th.join();
}

/*
 * Offset, in elements, of the first element of row `row` of a box inside the
 * global row-major tensor.  A "row" is one run along the last dim; rows are
 * numbered row-major over the box's other dims.
 */
int64_t global_row_offset(int ndim, const int64_t* shape, const int64_t* lo,
                          const int64_t* ext, int64_t row) {
  int64_t off = 0, stride = shape[ndim - 1];
  off += lo[ndim - 1];
  for (int k = ndim - 2; k >= 0; --k) {
    int64_t i = row % ext[k];
    row /= ext[k];
    off += (lo[k] + i) * stride;
    stride *= shape[k];
  }
  return off;
}

/*
 * Floating-point formats for oracle_convert.  The reshard pages mention that
 * the refit has precision modes and say nothing more (news.bpdata.com and
 * techfeed.io write-ups of the NVIDIA blog, closing remarks on the refit guide).
 * The reading taken here: a destination may hold a different float format than
 * the source; widening keeps the value; narrowing rounds to nearest, ties to
 * even, with overflow to infinity (IEEE 754 default rounding).
 *
 * Each format is (total bits, fraction bits, exponent bias).  A finite value is
 * decoded to a double (exact for all three formats), rounded to the target's
 * precision and exponent range by a plain floor-and-compare, and encoded.  NaN
 * has no value to round; the convention used for it is: sign kept, the leading
 * fraction bits kept (shifted to the target's width), quiet bit set.
 */
struct Format {
  int bits;  // 32 or 16
  int frac;  // fraction (stored mantissa) bits
  int bias;
};

constexpr Format kFormats[3] = {
    {32, 23, 127},  // 0: IEEE binary32
    {16, 7, 127},   // 1: bfloat16
    {16, 10, 15},   // 2: IEEE binary16
};

int exp_bits(const Format& f) { return f.bits - 1 - f.frac; }
uint32_t exp_all_ones(const Format& f) { return (1u << exp_bits(f)) - 1; }

double max_finite(const Format& f) {
  const int emax = int(exp_all_ones(f)) - 1 - f.bias;
  return std::ldexp(2.0 - std::ldexp(1.0, -f.frac), emax);
}

/* Value of a finite bit pattern. */
double decode(const Format& f, uint32_t bits) {
  const bool neg = (bits >> (f.bits - 1)) & 1;
  const uint32_t e = (bits >> f.frac) & exp_all_ones(f);
  const uint32_t m = bits & ((1u << f.frac) - 1);
  double v;
  if (e == 0) v = std::ldexp(double(m), 1 - f.bias - f.frac);  // subnormal or zero
  else v = std::ldexp(double((1u << f.frac) + m), int(e) - f.bias - f.frac);
  return neg ? -v : v;
}

/* x rounded to the nearest value of format f (ties to even); beyond the largest
   finite value after rounding: infinity.  x is finite. */
double round_to(const Format& f, double x) {
  if (x == 0) return x;
  const double a = std::fabs(x);
  int e;
  std::frexp(a, &e);        // a = m * 2^e with m in [0.5, 1): a's exponent is e - 1
  int E = e - 1;
  if (E < 1 - f.bias) E = 1 - f.bias;   // subnormal range: fixed spacing
  const int q = E - f.frac;             // weight of the last kept bit is 2^q
  const double s = std::ldexp(a, -q);   // exact
  double r = std::floor(s);
  const double d = s - r;
  if (d > 0.5 || (d == 0.5 && std::fmod(r, 2.0) != 0)) r += 1;
  double y = std::ldexp(r, q);
  if (y > max_finite(f)) y = INFINITY;
  return x < 0 ? -y : y;
}

/* Bit pattern of y, which is a value of format f (or an infinity). */
uint32_t encode(const Format& f, double y) {
  const uint32_t sign = std::signbit(y) ? 1u << (f.bits - 1) : 0u;
  const double a = std::fabs(y);
  if (std::isinf(a)) return sign | (exp_all_ones(f) << f.frac);
  if (a == 0) return sign;
  int e;
  std::frexp(a, &e);
  const int E = e - 1;
  if (E < 1 - f.bias)  // subnormal: the fraction counts units of 2^(1 - bias - frac)
    return sign | uint32_t(std::ldexp(a, f.bias - 1 + f.frac));
  const uint32_t m = uint32_t(std::ldexp(a, f.frac - E)) - (1u << f.frac);
  return sign | (uint32_t(E + f.bias) << f.frac) | m;
}

bool is_nan(const Format& f, uint32_t bits) {
  return ((bits >> f.frac) & exp_all_ones(f)) == exp_all_ones(f) && (bits & ((1u << f.frac) - 1)) != 0;
}

uint32_t convert_one(const Format& from, const Format& to, uint32_t bits) {
  if (is_nan(from, bits)) {
    const uint32_t sign = (bits >> (from.bits - 1)) & 1;
    uint32_t m = bits & ((1u << from.frac) - 1);
    m = to.frac >= from.frac ? m << (to.frac - from.frac) : m >> (from.frac - to.frac);
    m |= 1u << (to.frac - 1);  // quiet
    return (sign << (to.bits - 1)) | (exp_all_ones(to) << to.frac) | m;
  }
  const uint32_t e = (bits >> from.frac) & exp_all_ones(from);
  if (e == exp_all_ones(from)) {  // infinity
    const uint32_t sign = (bits >> (from.bits - 1)) & 1;
    return (sign << (to.bits - 1)) | (exp_all_ones(to) << to.frac);
  }
  return encode(to, round_to(to, decode(from, bits)));
}

}  // namespace

extern "C" {

int oracle_num_ranks(int ndim, const int64_t* shape, int mesh_ndim, const int64_t* mesh,
                     const int32_t* placements, int64_t* out) {
  Layout L{ndim, shape, mesh_ndim, mesh, placements};
  if (!layout_ok(L)) return ORACLE_BAD_LAYOUT;
  *out = num_ranks(L);
  return ORACLE_OK;
}

int oracle_shard_box(int ndim, const int64_t* shape, int mesh_ndim, const int64_t* mesh,
                     const int32_t* placements, int64_t rank, int64_t* lo, int64_t* hi) {
  Layout L{ndim, shape, mesh_ndim, mesh, placements};
  if (!layout_ok(L) || rank < 0 || rank >= num_ranks(L)) return ORACLE_BAD_LAYOUT;
  box_of(L, rank, lo, hi);
  return ORACLE_OK;
}

/*
 * Gather-then-slice reshard of one tensor.
 *   elem_size        bytes per element (the copy is bytewise; no conversion)
 *   src_bufs[s]      source shard of rank s (contiguous row-major box); may be
 *                    NULL only when that box is empty
 *   dst_bufs[d]      destination shard of rank d, written by this call
 *   global_out       optional caller buffer of prod(shape)*elem_size bytes that
 *                    receives X; NULL lets the oracle allocate its own
 *   check            nonzero: replica-consistency and coverage checks
 *   threads          host threads used for each box copy (>= 1)
 * Returns 0, or an OracleStatus code.
 */
int oracle_reshard(int ndim, const int64_t* shape, int64_t elem_size,
                   int src_mesh_ndim, const int64_t* src_mesh, const int32_t* src_pl,
                   const void* const* src_bufs,
                   int dst_mesh_ndim, const int64_t* dst_mesh, const int32_t* dst_pl,
                   void* const* dst_bufs,
                   void* global_out, int check, int threads) {
  Layout S{ndim, shape, src_mesh_ndim, src_mesh, src_pl};
  Layout D{ndim, shape, dst_mesh_ndim, dst_mesh, dst_pl};
  if (!layout_ok(S) || !layout_ok(D) || elem_size < 1) return ORACLE_BAD_LAYOUT;
  if (threads < 1) threads = 1;

  int64_t numel = 1;
  for (int k = 0; k < ndim; ++k) numel *= shape[k];
  const size_t es = (size_t)elem_size;

  int64_t r_src = 1;  // expected coverage of every element by the sources
  for (int m = 0; m < S.mesh_ndim; ++m)
    if (S.placements[m] == kReplicate) r_src *= S.mesh[m];
  if (check && r_src > 254) check = 0;  // uint8 counters; such meshes skip the count

  unsigned char* X = (unsigned char*)global_out;
  bool own_x = false;
  if (X == nullptr && numel > 0) {
    X = (unsigned char*)std::malloc((size_t)numel * es);
    if (!X) return ORACLE_NO_MEMORY;
    own_x = true;
  }
  unsigned char* count = nullptr;
  if (check && numel > 0) {
    count = (unsigned char*)std::calloc((size_t)numel, 1);
    if (!count) {
      if (own_x) std::free(X);
      return ORACLE_NO_MEMORY;
    }
  }
  int status = ORACLE_OK;

  // 1. Gather: X[box(src, s)] = src_shard[s].
  for (int64_t s = 0; s < num_ranks(S) && status == ORACLE_OK; ++s) {
    int64_t lo[kMaxDims], hi[kMaxDims], ext[kMaxDims];
    box_of(S, s, lo, hi);
    if (box_empty(ndim, lo, hi)) continue;
    if (src_bufs[s] == nullptr) {
      status = ORACLE_NULL_BUFFER;
      break;
    }
    int64_t rows = 1;
    for (int k = 0; k < ndim; ++k) ext[k] = hi[k] - lo[k];
    for (int k = 0; k < ndim - 1; ++k) rows *= ext[k];
    const int64_t run = ext[ndim - 1];
    const unsigned char* shard = (const unsigned char*)src_bufs[s];
    std::atomic<int> mismatch{0};
    parallel_rows(rows, threads, [&](int64_t a, int64_t b) {
      for (int64_t row = a; row < b; ++row) {
        int64_t g = global_row_offset(ndim, shape, lo, ext, row);
        const unsigned char* from = shard + (size_t)(row * run) * es;
        unsigned char* to = X + (size_t)g * es;
        if (!check) {
          std::memcpy(to, from, (size_t)run * es);
          continue;
        }
        for (int64_t j = 0; j < run; ++j) {
          if (count[g + j] == 0) {
            std::memcpy(to + j * es, from + j * es, es);
          } else if (std::memcmp(to + j * es, from + j * es, es) != 0) {
            mismatch.store(1);
          }
          count[g + j] += 1;
        }
      }
    });
    if (mismatch.load()) status = ORACLE_REPLICA_MISMATCH;
  }

  // Every element must be covered exactly R_src times.
  if (status == ORACLE_OK && check) {
    for (int64_t i = 0; i < numel; ++i)
      if (count[i] != (unsigned char)r_src) {
        status = ORACLE_COVERAGE_MISMATCH;
        break;
      }
  }

  // 2. Slice: dst_shard[d] = X[box(dst, d)].
  for (int64_t d = 0; d < num_ranks(D) && status == ORACLE_OK; ++d) {
    int64_t lo[kMaxDims], hi[kMaxDims], ext[kMaxDims];
    box_of(D, d, lo, hi);
    if (box_empty(ndim, lo, hi)) continue;
    if (dst_bufs[d] == nullptr) {
      status = ORACLE_NULL_BUFFER;
      break;
    }
    int64_t rows = 1;
    for (int k = 0; k < ndim; ++k) ext[k] = hi[k] - lo[k];
    for (int k = 0; k < ndim - 1; ++k) rows *= ext[k];
    const int64_t run = ext[ndim - 1];
    unsigned char* shard = (unsigned char*)dst_bufs[d];
    parallel_rows(rows, threads, [&](int64_t a, int64_t b) {
      for (int64_t row = a; row < b; ++row) {
        int64_t g = global_row_offset(ndim, shape, lo, ext, row);
        std::memcpy(shard + (size_t)(row * run) * es, X + (size_t)g * es, (size_t)run * es);
      }
    });
  }

  std::free(count);
  if (own_x) std::free(X);
  return status;
}

/*
 * Global indices along tensor dim `dim` that `rank` holds, in local order
 * (index_list).  split[m] is the split factor of mesh dim m (1 = Shard or
 * Replicate).  Writes min(capacity, count) of them to out and the count to *n.
 */
int oracle_shard_indices(int ndim, const int64_t* shape, int mesh_ndim, const int64_t* mesh,
                         const int32_t* placements, const int64_t* split, int64_t rank, int dim,
                         int64_t* out, int64_t capacity, int64_t* n) {
  Layout L{ndim, shape, mesh_ndim, mesh, placements};
  if (!layout_ok(L) || !split_ok(L, split) || rank < 0 || rank >= num_ranks(L) || dim < 0 || dim >= ndim)
    return ORACLE_BAD_LAYOUT;
  const std::vector<int64_t> v = index_list(L, split, rank, dim);
  for (int64_t i = 0; i < (int64_t)v.size() && i < capacity; ++i) out[i] = v[i];
  *n = (int64_t)v.size();
  return ORACLE_OK;
}

/*
 * Gather-then-slice of one tensor whose layouts may use strided nesting,
 * element by element over explicit index lists (index_list): X[idx(s, l)] =
 * src_shard[s][l] for every source rank s and local multi-index l, then
 * dst_shard[d][l] = X[idx(d, l)].  Arguments as oracle_reshard, plus the split
 * factors of each layout's mesh dims.  Checks as oracle_reshard.
 */
int oracle_reshard_indexed(int ndim, const int64_t* shape, int64_t elem_size,
                           int src_mesh_ndim, const int64_t* src_mesh, const int32_t* src_pl,
                           const int64_t* src_split, const void* const* src_bufs,
                           int dst_mesh_ndim, const int64_t* dst_mesh, const int32_t* dst_pl,
                           const int64_t* dst_split, void* const* dst_bufs,
                           void* global_out, int check, int threads) {
  Layout S{ndim, shape, src_mesh_ndim, src_mesh, src_pl};
  Layout D{ndim, shape, dst_mesh_ndim, dst_mesh, dst_pl};
  if (!layout_ok(S) || !layout_ok(D) || !split_ok(S, src_split) || !split_ok(D, dst_split) || elem_size < 1)
    return ORACLE_BAD_LAYOUT;
  if (threads < 1) threads = 1;
  int64_t numel = 1;
  for (int k = 0; k < ndim; ++k) numel *= shape[k];
  const size_t es = (size_t)elem_size;
  int64_t gstride[kMaxDims];  // row-major strides of the global tensor, elements
  int64_t st = 1;
  for (int k = ndim - 1; k >= 0; --k) {
    gstride[k] = st;
    st *= shape[k];
  }
  int64_t copies = 1;  // replicas of every element among the sources
  for (int m = 0; m < S.mesh_ndim; ++m)
    if (S.placements[m] == kReplicate) copies = copies * S.mesh[m];
  if (check && copies > 254) check = 0;

  unsigned char* X = (unsigned char*)global_out;
  bool own_x = false;
  if (X == nullptr && numel > 0) {
    X = (unsigned char*)std::malloc((size_t)numel * es);
    if (!X) return ORACLE_NO_MEMORY;
    own_x = true;
  }
  unsigned char* count = nullptr;
  if (check && numel > 0) {
    count = (unsigned char*)std::calloc((size_t)numel, 1);
    if (!count) {
      if (own_x) std::free(X);
      return ORACLE_NO_MEMORY;
    }
  }
  int status = ORACLE_OK;

  // Global element offset of local row `row` (row-major over every dim but the
  // last) of a shard with index lists idx.
  auto row_base = [&](const std::vector<std::vector<int64_t>>& idx, int64_t row) {
    int64_t off = 0;
    for (int k = ndim - 2; k >= 0; --k) {
      const int64_t len = (int64_t)idx[k].size();
      off += idx[k][row % len] * gstride[k];
      row /= len;
    }
    return off;
  };

  // 1. Gather.
  for (int64_t s = 0; s < num_ranks(S) && status == ORACLE_OK; ++s) {
    std::vector<std::vector<int64_t>> idx(ndim);
    int64_t local = 1;
    for (int k = 0; k < ndim; ++k) {
      idx[k] = index_list(S, src_split, s, k);
      local *= (int64_t)idx[k].size();
    }
    if (local == 0) continue;
    if (src_bufs[s] == nullptr) {
      status = ORACLE_NULL_BUFFER;
      break;
    }
    const std::vector<int64_t>& last = idx[ndim - 1];
    const int64_t run = (int64_t)last.size();
    const int64_t rows = local / run;
    const unsigned char* shard = (const unsigned char*)src_bufs[s];
    std::atomic<int> mismatch{0};
    parallel_rows(rows, threads, [&](int64_t a, int64_t b) {
      for (int64_t row = a; row < b; ++row) {
        const int64_t base = row_base(idx, row);
        for (int64_t j = 0; j < run; ++j) {
          const int64_t g = base + last[j];
          const unsigned char* from = shard + (size_t)(row * run + j) * es;
          if (check && count[g] != 0) {
            if (std::memcmp(X + (size_t)g * es, from, es) != 0) mismatch.store(1);
          } else {
            std::memcpy(X + (size_t)g * es, from, es);
          }
          if (check) count[g] += 1;
        }
      }
    });
    if (mismatch.load()) status = ORACLE_REPLICA_MISMATCH;
  }
  if (status == ORACLE_OK && check) {
    for (int64_t i = 0; i < numel; ++i)
      if (count[i] != (unsigned char)copies) {
        status = ORACLE_COVERAGE_MISMATCH;
        break;
      }
  }

  // 2. Slice.
  for (int64_t d = 0; d < num_ranks(D) && status == ORACLE_OK; ++d) {
    std::vector<std::vector<int64_t>> idx(ndim);
    int64_t local = 1;
    for (int k = 0; k < ndim; ++k) {
      idx[k] = index_list(D, dst_split, d, k);
      local *= (int64_t)idx[k].size();
    }
    if (local == 0) continue;
    if (dst_bufs[d] == nullptr) {
      status = ORACLE_NULL_BUFFER;
      break;
    }
    const std::vector<int64_t>& last = idx[ndim - 1];
    const int64_t run = (int64_t)last.size();
    const int64_t rows = local / run;
    unsigned char* shard = (unsigned char*)dst_bufs[d];
    parallel_rows(rows, threads, [&](int64_t a, int64_t b) {
      for (int64_t row = a; row < b; ++row) {
        const int64_t base = row_base(idx, row);
        for (int64_t j = 0; j < run; ++j)
          std::memcpy(shard + (size_t)(row * run + j) * es, X + (size_t)(base + last[j]) * es, es);
      }
    });
  }
  std::free(count);
  if (own_x) std::free(X);
  return status;
}

/*
 * Reshard of one tensor whose source layout holds partial sums.  The write-ups
 * say only that the refit guide lists the supported layouts (news.bpdata.com
 * write-up, "practical access and setup" section); the reading taken is
 * DTensor's Partial("sum") placement: along a source mesh dim marked Partial
 * (code -2) every coordinate holds a full-size contribution of the same box, and
 * the tensor is their elementwise sum.  Several Partial mesh dims number their
 * contributions q = 0, 1, ... row-major over their coordinates.  The sum is
 * taken in that order, in binary32: it starts from contribution 0 (widened
 * exactly) and adds each next one with one binary32 rounding per addition
 * (round to nearest, ties to even); the result is rounded once to the
 * destination format (as oracle_convert does).  Destination layouts are plain
 * (no Partial).  Formats as oracle_convert: 0 binary32, 1 bfloat16, 2 binary16.
 *   src_bufs[s]  shard of source rank s, row-major over its box (boxes as for
 *                a plain layout, Partial mesh dims splitting nothing)
 * Checks: replicas of one contribution must hold equal bytes; every element is
 * covered R_src times by every contribution.  Returns 0 or an OracleStatus.
 */
int oracle_reshard_partial(int ndim, const int64_t* shape, int src_fmt, int dst_fmt,
                           int src_mesh_ndim, const int64_t* src_mesh, const int32_t* src_pl,
                           const void* const* src_bufs,
                           int dst_mesh_ndim, const int64_t* dst_mesh, const int32_t* dst_pl,
                           void* const* dst_bufs, int check, int threads) {
  constexpr int32_t kPartial = -2;
  if (src_fmt < 0 || src_fmt > 2 || dst_fmt < 0 || dst_fmt > 2) return ORACLE_BAD_LAYOUT;
  if (src_mesh_ndim < 1 || src_mesh_ndim > kMaxDims) return ORACLE_BAD_LAYOUT;
  // the source's boxes: its layout with every Partial mesh dim read as Replicate
  int32_t plain_pl[kMaxDims];
  int64_t contributions = 1, copies = 1;
  for (int m = 0; m < src_mesh_ndim; ++m) {
    plain_pl[m] = src_pl[m] == kPartial ? kReplicate : src_pl[m];
    if (src_pl[m] == kPartial) contributions *= src_mesh[m];
    else if (src_pl[m] == kReplicate) copies *= src_mesh[m];
  }
  Layout S{ndim, shape, src_mesh_ndim, src_mesh, plain_pl};
  Layout D{ndim, shape, dst_mesh_ndim, dst_mesh, dst_pl};
  if (!layout_ok(S) || !layout_ok(D)) return ORACLE_BAD_LAYOUT;
  if (check && copies > 254) check = 0;
  if (threads < 1) threads = 1;
  const Format& F = kFormats[src_fmt];
  const Format& T = kFormats[dst_fmt];
  const size_t es_s = size_t(F.bits / 8), es_d = size_t(T.bits / 8);
  int64_t numel = 1;
  for (int k = 0; k < ndim; ++k) numel *= shape[k];

  // 1. Gather every contribution into its own binary32 copy of the tensor.
  std::vector<std::vector<float>> X((size_t)contributions, std::vector<float>((size_t)numel));
  std::vector<std::vector<unsigned char>> count;
  if (check) count.assign((size_t)contributions, std::vector<unsigned char>((size_t)numel, 0));
  int status = ORACLE_OK;
  for (int64_t s = 0; s < num_ranks(S) && status == ORACLE_OK; ++s) {
    // contribution index: the rank's coordinates on the Partial mesh dims, row-major
    int64_t coord[kMaxDims], r = s, q = 0;
    for (int m = src_mesh_ndim - 1; m >= 0; --m) {
      coord[m] = r % src_mesh[m];
      r /= src_mesh[m];
    }
    for (int m = 0; m < src_mesh_ndim; ++m)
      if (src_pl[m] == kPartial) q = q * src_mesh[m] + coord[m];
    int64_t lo[kMaxDims], hi[kMaxDims], ext[kMaxDims];
    box_of(S, s, lo, hi);
    if (box_empty(ndim, lo, hi)) continue;
    if (src_bufs[s] == nullptr) {
      status = ORACLE_NULL_BUFFER;
      break;
    }
    int64_t rows = 1;
    for (int k = 0; k < ndim; ++k) ext[k] = hi[k] - lo[k];
    for (int k = 0; k < ndim - 1; ++k) rows *= ext[k];
    const int64_t run = ext[ndim - 1];
    const unsigned char* shard = (const unsigned char*)src_bufs[s];
    float* Xq = X[(size_t)q].data();
    unsigned char* cq = check ? count[(size_t)q].data() : nullptr;
    std::atomic<int> mismatch{0};
    parallel_rows(rows, threads, [&](int64_t a, int64_t b) {
      for (int64_t row = a; row < b; ++row) {
        const int64_t g = global_row_offset(ndim, shape, lo, ext, row);
        for (int64_t j = 0; j < run; ++j) {
          uint32_t bits = 0;
          std::memcpy(&bits, shard + (size_t)(row * run + j) * es_s, es_s);
          // widened exactly to binary32 (oracle_convert's rules; NaN stays NaN)
          const uint32_t w = src_fmt == 0 ? bits : convert_one(F, kFormats[0], bits);
          float v;
          std::memcpy(&v, &w, 4);
          if (cq && cq[g + j] != 0) {
            if (std::memcmp(&Xq[g + j], &v, 4) != 0) mismatch.store(1);
          } else {
            Xq[g + j] = v;
          }
          if (cq) cq[g + j] += 1;
        }
      }
    });
    if (mismatch.load()) status = ORACLE_REPLICA_MISMATCH;
  }
  if (status == ORACLE_OK && check) {
    for (int64_t q = 0; q < contributions && status == ORACLE_OK; ++q)
      for (int64_t i = 0; i < numel; ++i)
        if (count[(size_t)q][(size_t)i] != (unsigned char)copies) {
          status = ORACLE_COVERAGE_MISMATCH;
          break;
        }
  }
  if (status != ORACLE_OK) return status;

  // 2. Sum the contributions in order, in binary32.
  std::vector<float> sum(X[0]);
  for (int64_t q = 1; q < contributions; ++q) {
    const std::vector<float>& Xq = X[(size_t)q];
    for (int64_t i = 0; i < numel; ++i) {
      volatile float t = sum[(size_t)i] + Xq[(size_t)i];  // one binary32 rounding
      sum[(size_t)i] = t;
    }
  }

  // 3. Slice each destination box out of the sum, rounded to the destination format.
  for (int64_t d = 0; d < num_ranks(D); ++d) {
    int64_t lo[kMaxDims], hi[kMaxDims], ext[kMaxDims];
    box_of(D, d, lo, hi);
    if (box_empty(ndim, lo, hi)) continue;
    if (dst_bufs[d] == nullptr) return ORACLE_NULL_BUFFER;
    int64_t rows = 1;
    for (int k = 0; k < ndim; ++k) ext[k] = hi[k] - lo[k];
    for (int k = 0; k < ndim - 1; ++k) rows *= ext[k];
    const int64_t run = ext[ndim - 1];
    unsigned char* shard = (unsigned char*)dst_bufs[d];
    parallel_rows(rows, threads, [&](int64_t a, int64_t b) {
      for (int64_t row = a; row < b; ++row) {
        const int64_t g = global_row_offset(ndim, shape, lo, ext, row);
        for (int64_t j = 0; j < run; ++j) {
          const float v = sum[(size_t)(g + j)];
          uint32_t f32;
          std::memcpy(&f32, &v, 4);
          const uint32_t out = dst_fmt == 0 ? f32 : convert_one(kFormats[0], T, f32);
          std::memcpy(shard + (size_t)(row * run + j) * es_d, &out, es_d);
        }
      }
    });
  }
  return ORACLE_OK;
}

/*
 * Converts n elements from format `from` to format `to` (0 = binary32,
 * 1 = bfloat16, 2 = binary16; elements are stored little-endian in 4 or 2
 * bytes).  Used after the gather-then-slice for a reshard whose destination
 * dtype differs from the source's.  Returns 0, or ORACLE_BAD_LAYOUT for an
 * unknown format.
 */
int oracle_convert(int from, int to, const void* in, void* out, int64_t n, int threads) {
  if (from < 0 || from > 2 || to < 0 || to > 2 || n < 0) return ORACLE_BAD_LAYOUT;
  const Format& F = kFormats[from];
  const Format& T = kFormats[to];
  parallel_rows(n, threads < 1 ? 1 : threads, [&](int64_t a, int64_t b) {
    for (int64_t i = a; i < b; ++i) {
      uint32_t x;
      if (F.bits == 32) std::memcpy(&x, (const unsigned char*)in + 4 * i, 4);
      else {
        uint16_t h;
        std::memcpy(&h, (const unsigned char*)in + 2 * i, 2);
        x = h;
      }
      const uint32_t y = convert_one(F, T, x);
      if (T.bits == 32) std::memcpy((unsigned char*)out + 4 * i, &y, 4);
      else {
        const uint16_t h = uint16_t(y);
        std::memcpy((unsigned char*)out + 2 * i, &h, 2);
      }
    }
  });
  return ORACLE_OK;
}

}  // extern "C"
