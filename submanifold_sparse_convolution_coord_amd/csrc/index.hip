// Coordinate index (neighbour map) and warm plan for submanifold 3x3x3 convolution.
//
// Neighbour map: the gather-scatter method starts by building a hash map of the active voxel
// coordinates and then, per kernel offset, looks up each site's neighbour (trellis-mac
// article, the gather-scatter flowchart).  The LATO.2 page ("Fleet benchmark", closing
// paragraph) reports the map build as the dominant cost once the convolution is fast (232-357
// ms of CPU numpy) and amortised only by caching per coordinate set; here it runs on the GPU:
//
//   k_table_init  fill the table with the empty key, clear the error counters
//   k_insert      one thread per site: validate, pack (b,x,y,z) into a 64-bit key, insert
//                 by linear probing with a 64-bit compare-and-swap; value = row index
//   k_query       one thread per (site, tap): probe for (b, x+dx, y+dy, z+dz); write the
//                 row or -1; consecutive threads write consecutive map entries
//
// Warm plan: the sites are reordered by their 26-bit mask of valid non-centre taps (a stable
// LSD radix sort written here: per-tile digit histograms, a digit-major exclusive scan with
// one workgroup per digit, then a stable scatter that ranks equal digits with wave ballots),
// so that the 16-row blocks the matrix
// cores consume tend to share which taps are present and empty (block, tap) pairs can be
// skipped whole.  The neighbour rows are then stored tap-major in that order.
//
// Given the coordinates, the plan also tries a spatial order: the mask order stably re-sorted
// by 128^3 brick (batch entry, then the Morton code of the brick), which keeps the rows a tile
// gathers within one region.  It is kept when it costs at most 5% more (block, tap) pairs
// than the mask order, and the k=3 kernel then gives each XCD a contiguous share of the tiles
// so that its L2 serves one region (surfaces: 25-32% faster convolutions).  Point clouds
// without spatial coherence (i.i.d. sites) lose more than 5% and keep the mask order.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "dense.h"
#include "sort.h"

namespace ssc {
namespace {

constexpr unsigned long long kEmptyKey = ~0ull;  // no valid key: fields are < 65535

__device__ __forceinline__ unsigned long long pack_key(int b, int x, int y, int z) {
  return (static_cast<unsigned long long>(static_cast<uint32_t>(b)) << 48) |
         (static_cast<unsigned long long>(static_cast<uint32_t>(x)) << 32) |
         (static_cast<unsigned long long>(static_cast<uint32_t>(y)) << 16) |
         static_cast<unsigned long long>(static_cast<uint32_t>(z));
}

// 64-bit finaliser of splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): spreads the packed coordinates over the table.
__device__ __forceinline__ unsigned long long mix64(unsigned long long z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

// One 16-byte slot holds a key and its row, so a probe that finds its key reads one cache
// line, not two.
struct alignas(16) Slot {
  unsigned long long key;
  int32_t val;
  int32_t pad;
};

struct IndexLayout {
  uint64_t cap;
  size_t off_slots, total;
};

inline IndexLayout index_layout(int64_t n) {
  IndexLayout L;
  uint64_t want = static_cast<uint64_t>(n > 0 ? n : 1) * 2;
  uint64_t cap = 64;
  while (cap < want) cap <<= 1;
  L.cap = cap;
  L.off_slots = kAlign;  // [0, 256): two uint32 error counters
  L.total = align_up(L.off_slots + sizeof(Slot) * cap);
  return L;
}

__global__ void k_table_init(Slot* __restrict__ slots, uint64_t cap,
                             uint32_t* __restrict__ counters) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < cap;
       i += stride)
    slots[i].key = kEmptyKey;
  if (blockIdx.x == 0 && threadIdx.x < 2) counters[threadIdx.x] = 0;
}

__global__ void k_insert(const int4* __restrict__ coords, int64_t n, int batch, int gx, int gy,
                         int gz, Slot* __restrict__ slots, uint64_t mask,
                         uint32_t* __restrict__ counters) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride) {
    const int4 c = coords[i];  // (b, x, y, z)
    if (c.x < 0 || c.x >= batch || c.y < 0 || c.y >= gx || c.z < 0 || c.z >= gy || c.w < 0 ||
        c.w >= gz) {
      atomicAdd(&counters[0], 1u);
      continue;
    }
    const unsigned long long key = pack_key(c.x, c.y, c.z, c.w);
    uint64_t h = mix64(key) & mask;
    // The table has at least twice as many slots as sites, so an empty slot always exists
    // and the probe ends.
    while (true) {
      const unsigned long long prev = atomicCAS(&slots[h].key, kEmptyKey, key);
      if (prev == kEmptyKey) {
        slots[h].val = static_cast<int32_t>(i);
        break;
      }
      if (prev == key) {
        atomicAdd(&counters[1], 1u);
        break;
      }
      h = (h + 1) & mask;
    }
  }
}

__global__ void k_query(const int4* __restrict__ coords, int64_t n, int batch, int gx, int gy,
                        int gz, const Slot* __restrict__ slots, uint64_t mask,
                        int32_t* __restrict__ nbr) {
  const int64_t total = n * kTaps;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += stride) {
    const int64_t i = g / kTaps;
    const int t = static_cast<int>(g - i * kTaps);
    const int4 c = coords[i];
    const int x = c.y + t / 9 - 1, y = c.z + (t / 3) % 3 - 1, z = c.w + t % 3 - 1;
    int32_t r = -1;
    if (c.x >= 0 && c.x < batch && x >= 0 && x < gx && y >= 0 && y < gy && z >= 0 && z < gz) {
      const unsigned long long key = pack_key(c.x, x, y, z);
      uint64_t h = mix64(key) & mask;
      // At least half the slots are empty, so the probe ends.
      while (true) {
        const uint4 v = *reinterpret_cast<const uint4*>(&slots[h]);  // key and row, one load
        const unsigned long long k = (static_cast<unsigned long long>(v.y) << 32) | v.x;
        if (k == key) {
          r = static_cast<int32_t>(v.z);
          break;
        }
        if (k == kEmptyKey) break;
        h = (h + 1) & mask;
      }
    }
    nbr[g] = r;
  }
}

// ------------------------------------------------------------------------------------------
// Dense rank index (dense.h): the sorted-key index map kept as an occupancy bitmap of the
// sites with running counts; the rank of a site's bit is its position in key order and
// sorted_rows[rank] its row.  The arrays take about 3/16 byte per voxel plus 4 bytes per site
// (1.2 MB at 128^3, 10 %) and stay in L2.  After dense.h's clear, mark, count and scan:
//   k_dense_rows    one thread per site: sorted_rows[rank(v)] = row
//   k_dense_query   one thread per site: per (dx, dy) one word serves the three dz taps
//                   unless they cross a word boundary; rows staged in LDS and written as
//                   whole map rows
// ------------------------------------------------------------------------------------------
struct DenseIndexLayout {
  DenseBits b;
  size_t off_rows, total;
};

// [0, 256): two uint32 error counters and the "sites not in key order" flag; the bitmap
// structure; the rows in key order.
inline DenseIndexLayout dense_index_layout(int64_t n, uint64_t voxels) {
  DenseIndexLayout L;
  L.b = dense_bits_layout(voxels, kAlign);
  L.off_rows = L.b.end;
  L.total = align_up(L.off_rows + sizeof(uint32_t) * (n > 0 ? n : 1));
  return L;
}

// rows[rank of site i] = i.  *unsorted becomes 1 if any site's rank differs from its row (the
// sites are not in ascending key order, or some are out of range); the query then maps ranks
// through rows, else a rank is the row itself.  One store per wave at most.
__global__ void k_dense_rows(const int4* __restrict__ coords, int64_t n, int batch, int gx,
                             int gy, int gz, const uint64_t* __restrict__ bits,
                             const uint16_t* __restrict__ local,
                             const uint32_t* __restrict__ super_count,
                             int32_t* __restrict__ rows, uint32_t* __restrict__ unsorted) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  bool moved = false;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride) {
    const int4 c = coords[i];
    if (!in_range(c, batch, gx, gy, gz)) {
      moved = true;
      continue;
    }
    const uint64_t v = dense_id(c.x, c.y, c.z, c.w, gx, gy, gz);
    // rank < number of set bits <= n, so the write stays inside rows[0, n)
    const uint32_t r = dense_rank(local, super_count, v, bits[v >> 6]);
    rows[r] = static_cast<int32_t>(i);
    moved = moved || static_cast<int64_t>(r) != i;
  }
  if (__ballot(moved) != 0ull && (threadIdx.x & 63) == 0) *unsorted = 1u;
}

// One thread per site (256 sites per workgroup): for each (dx, dy) one bitmap word serves the
// three dz taps unless they cross a word boundary.  The map rows are staged in LDS (stride
// 27, odd, so the lanes' writes fall in distinct banks) and the workgroup's rows leave as one
// contiguous run.  (Nine threads per site, one per (dx, dy), measured slower: 23.6 against
// 20.6 us at 128^3, 113 against 84 us at the 512^3 shell.)
constexpr int kQuerySites = 256;
__global__ __launch_bounds__(kQuerySites) void k_dense_query(
    const int4* __restrict__ coords, int64_t n, int batch, int gx, int gy, int gz,
    const uint64_t* __restrict__ bits, const uint16_t* __restrict__ local,
    const uint32_t* __restrict__ super_count, const int32_t* __restrict__ rows,
    const uint32_t* __restrict__ unsorted, int32_t* __restrict__ nbr) {
  __shared__ int32_t out[kQuerySites * kTaps];
  const bool in_order = *unsorted == 0u;  // every site's row is its rank
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kQuerySites;
  const int64_t i = i0 + threadIdx.x;
  int32_t* mine = out + threadIdx.x * kTaps;
  if (i < n) {
    const int4 c = coords[i];
    const bool ok = c.x >= 0 && c.x < batch;
    // The word of voxel z (clamped into the grid) serves every dz tap inside it.
    const int zc = c.w < 0 ? 0 : c.w >= gz ? gz - 1 : c.w;
#pragma unroll
    for (int dx = -1; dx <= 1; ++dx)
#pragma unroll
      for (int dy = -1; dy <= 1; ++dy) {
        const int x = c.y + dx, y = c.z + dy;
        const int t0 = 9 * (dx + 1) + 3 * (dy + 1);
        const bool row_ok = ok && x >= 0 && x < gx && y >= 0 && y < gy;
        const uint64_t vc = row_ok ? dense_id(c.x, x, y, zc, gx, gy, gz) : 0ull;
        const uint64_t word_c = row_ok ? bits[vc >> 6] : 0ull;
#pragma unroll
        for (int dz = -1; dz <= 1; ++dz) {
          const int z = c.w + dz;
          int32_t r = -1;
          if (row_ok && z >= 0 && z < gz) {
            const uint64_t v = vc + static_cast<uint64_t>(z - zc);
            const uint64_t word = (v >> 6) == (vc >> 6) ? word_c : bits[v >> 6];
            if ((word >> (v & 63)) & 1ull) {
              const uint32_t k = dense_rank(local, super_count, v, word);
              r = in_order ? static_cast<int32_t>(k) : rows[k];
            }
          }
          mine[t0 + dz + 1] = r;
        }
      }
  }
  __syncthreads();
  const int64_t m = (n - i0 < kQuerySites ? n - i0 : kQuerySites) * kTaps;
  int32_t* dst = nbr + i0 * kTaps;
  for (int64_t e = threadIdx.x; e < m; e += kQuerySites) dst[e] = out[e];
}


// ------------------------------------------------------------------------------------------
// Plan: stable LSD radix sort of (mask, row) pairs, then the tap-major neighbour rows.
// ------------------------------------------------------------------------------------------
constexpr int kKeyBits = 26;                     // the plan's sort key (Gray rank of the mask)
constexpr int kBrickShift = 7;                   // spatial order: bricks of 128^3 voxels
constexpr int64_t kMinBricks = 8;                // ... tried when the grid holds this many
constexpr int kCountSlots = 64;                  // (block, tap) counts: slots of partial sums

// Tile order of the mask order: whole tiles of kTileRows sites are re-sorted by their cost,
// estimated as kStageCost per tap the tile walks plus one per (16-row block, tap) pair it
// computes (the k=3 kernel pays a fixed wait, barrier and issue per tap and matrix work per
// active block; 11 is about their ratio at C = 128).  One workgroup sorts up to kOrderTiles
// tiles; above that the mask order stays as it is.
constexpr int kStageCost = 11;
constexpr int kCostBins = 1024;                  // costs < 27 * (kStageCost + 8) < 1024
constexpr int64_t kOrderTiles = 32768;
static_assert(kTaps * (kStageCost + kTileRows / kBlockRows) < kCostBins, "tile cost range");

// The plan's scratch: the mask-order sort (32-bit keys), the brick sort (64-bit keys), each
// site's tap mask, the two orders' (block, tap) counts in kCountSlots slots each (one
// counter took every wave's atomic add and serialised them: 0.46 ms at 1.2M sites), and the
// full tiles' costs and cost order.
struct PlanWork {
  SortLayout<uint32_t> g;
  SortLayout<uint64_t> b;
  int64_t full_tiles;
  size_t off_mask, off_count, off_cost, off_tiles, total;
};
inline PlanWork plan_work_layout(int64_t n) {
  PlanWork W;
  W.g = sort_layout<uint32_t>(n, 0);
  W.b = sort_layout<uint64_t>(n, W.g.total);
  W.full_tiles = n > 0 ? n / kTileRows : 0;
  W.off_mask = align_up(W.b.total);
  W.off_count = align_up(W.off_mask + sizeof(uint32_t) * (n > 0 ? n : 1));
  W.off_cost = align_up(W.off_count + 2 * kCountSlots * sizeof(unsigned long long));
  W.off_tiles = align_up(W.off_cost + sizeof(uint32_t) * (W.full_tiles > 0 ? W.full_tiles : 1));
  W.total = align_up(W.off_tiles + sizeof(int32_t) * (W.full_tiles > 0 ? W.full_tiles : 1));
  return W;
}

// Whether the brick order replaces the mask order: its (block, tap) count is at most 21/20
// of the mask order's.  Wave-uniform; every lane of the calling wave must take part.
__device__ __forceinline__ bool brick_order_wins(const unsigned long long* __restrict__ counts) {
  static_assert(kCountSlots == 64, "one slot per lane");
  const int lane = threadIdx.x & 63;
  unsigned long long g = counts[2 * lane], b = counts[2 * lane + 1];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    g += __shfl_xor(g, off, 64);
    b += __shfl_xor(b, off, 64);
  }
  return b * 20 <= g * 21;
}

// Sort key of a site: bit (t < 13 ? t : t - 1) set when non-centre tap t has a neighbour.
// With masks non-null the plain mask is kept too, and block 0 clears the count slots.
__device__ __forceinline__ void plan_header(int64_t* __restrict__ header, int64_t n, int64_t npad,
                                            int64_t nblocks, uint4* __restrict__ zero) {
  if (threadIdx.x == 0) {
    header[0] = kPlanMagic;
    header[1] = n;
    header[2] = npad;
    header[3] = nblocks;
    header[kPlanSchedWord] = kSchedInterleaved;  // k_plan_fill sets the final value
  }
  for (int i = threadIdx.x; i < static_cast<int>(kZeroBytes / sizeof(uint4)); i += blockDim.x)
    zero[i] = make_uint4(0u, 0u, 0u, 0u);
}

__global__ void k_plan_header(int64_t* __restrict__ header, int64_t n, int64_t npad,
                              int64_t nblocks, uint4* __restrict__ zero) {
  plan_header(header, n, npad, nblocks, zero);
}

// Block 0 also writes the plan's header and zero row (k_plan_header does when n = 0).
__global__ void k_mask_keys(const int32_t* __restrict__ nbr, int64_t n, uint32_t* __restrict__ keys,
                            uint32_t* __restrict__ vals, uint32_t* __restrict__ totals,
                            uint32_t* __restrict__ masks, unsigned long long* __restrict__ counts,
                            int64_t* __restrict__ header, int64_t npad, int64_t nblocks,
                            uint4* __restrict__ zero) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0) plan_header(header, n, npad, nblocks, zero);
  if (blockIdx.x == 0)
    for (int d = threadIdx.x; d < kDigits; d += blockDim.x) totals[d] = 0;
  if (masks != nullptr && blockIdx.x == 0 && threadIdx.x < 2 * kCountSlots) counts[threadIdx.x] = 0;
  if (i >= n) return;
  const int32_t* row = nbr + i * kTaps;
  uint32_t m = 0;
#pragma unroll
  for (int t = 0; t < kTaps; ++t) {
    if (t == kCentreTap) continue;
    if (row[t] >= 0) m |= 1u << (t < kCentreTap ? t : t - 1);
  }
  if (masks != nullptr) masks[i] = m;
  // Sort key: the rank of m read as a reflected Gray code (bit i of the key is the XOR of
  // bits i..25 of m).  Neighbouring ranks differ in one tap, so sites next to each other in
  // key order share more taps than in plain numeric order (fewer taps per tile, fewer
  // partly-empty 16-row blocks).
  m ^= m >> 1;
  m ^= m >> 2;
  m ^= m >> 4;
  m ^= m >> 8;
  m ^= m >> 16;
  keys[i] = m;
  vals[i] = static_cast<uint32_t>(i);
}

// Spreads the low `bits` bits of v to every third bit (bit k -> bit 3k).
__device__ __forceinline__ unsigned long long spread3(uint32_t v, int bits) {
  unsigned long long r = 0;
  for (int k = 0; k < bits; ++k) r |= static_cast<unsigned long long>((v >> k) & 1u) << (3 * k);
  return r;
}

// Brick sort input: position p of the mask order holds site r = rows[p]; its key is
// (batch entry << 3L) | Morton code of its 128^3 brick (L bits per axis).  Out-of-range
// coordinates only give meaningless keys, never an out-of-bounds access (the map already
// leaves such sites without neighbours).
__global__ void k_brick_keys(const int4* __restrict__ coords, const uint32_t* __restrict__ rows,
                             int64_t n, int axis_bits, unsigned long long* __restrict__ keys,
                             uint32_t* __restrict__ vals, uint32_t* __restrict__ totals) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0)
    for (int d = threadIdx.x; d < kDigits; d += blockDim.x) totals[d] = 0;
  if (p >= n) return;
  const uint32_t r = rows[p];
  const int4 c = coords[r];  // (b, x, y, z)
  const uint32_t bx = static_cast<uint32_t>(c.y) >> kBrickShift;
  const uint32_t by = static_cast<uint32_t>(c.z) >> kBrickShift;
  const uint32_t bz = static_cast<uint32_t>(c.w) >> kBrickShift;
  keys[p] = (static_cast<unsigned long long>(static_cast<uint32_t>(c.x) & 0xFFFFu)
             << (3 * axis_bits)) |
            (spread3(bx, axis_bits) << 2) | (spread3(by, axis_bits) << 1) | spread3(bz, axis_bits);
  vals[p] = r;
}

// (block, tap) pairs of the two candidate orders: for every 16-position block, the number of
// non-centre taps present in any of its sites.  One wave covers 4 blocks of each order; the
// workgroup's sums go to slot blockIdx % kCountSlots (counts[2 s] mask order, counts[2 s + 1]
// brick order).
__global__ __launch_bounds__(256) void k_block_taps(const uint32_t* __restrict__ rows_mask,
                                                    const uint32_t* __restrict__ rows_brick,
                                                    const uint32_t* __restrict__ masks, int64_t n,
                                                    unsigned long long* __restrict__ counts) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t mg = p < n ? masks[rows_mask[p]] : 0u;
  uint32_t mb = p < n ? masks[rows_brick[p]] : 0u;
#pragma unroll
  for (int off = 1; off < kBlockRows; off <<= 1) {
    mg |= __shfl_xor(mg, off, 64);
    mb |= __shfl_xor(mb, off, 64);
  }
  const int lane = threadIdx.x & 63;
  uint32_t cg = (lane & (kBlockRows - 1)) == 0 ? __popc(mg) : 0u;
  uint32_t cb = (lane & (kBlockRows - 1)) == 0 ? __popc(mb) : 0u;
#pragma unroll
  for (int off = kBlockRows; off < 64; off <<= 1) {
    cg += __shfl_xor(cg, off, 64);
    cb += __shfl_xor(cb, off, 64);
  }
  __shared__ uint32_t wsum[2][4];
  const int wave = threadIdx.x >> 6;
  if (lane == 0) {
    wsum[0][wave] = cg;
    wsum[1][wave] = cb;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    const uint32_t t = wsum[threadIdx.x][0] + wsum[threadIdx.x][1] + wsum[threadIdx.x][2] +
                       wsum[threadIdx.x][3];
    atomicAdd(&counts[2 * (blockIdx.x % kCountSlots) + threadIdx.x],
              static_cast<unsigned long long>(t));
  }
}

// Cost of every full tile of the mask order (nothing when the brick order wins).  A site's
// mask comes back from its sorted key (the key is the prefix XOR of the mask from the top
// bit, so mask = key ^ (key >> 1)); the centre tap, present at every site, is bit 26.  Two
// tiles per workgroup, one per pair of waves.
__global__ __launch_bounds__(256) void k_tile_cost(const uint32_t* __restrict__ keys,
                                                   int64_t full_tiles,
                                                   const unsigned long long* __restrict__ counts,
                                                   uint32_t* __restrict__ cost) {
  static_assert(kTileRows == 128, "two tiles per 256-thread workgroup");
  if (counts != nullptr && brick_order_wins(counts)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t m = 0u;
  if (p < full_tiles * kTileRows) {
    const uint32_t k = keys[p];
    m = (k ^ (k >> 1)) | (1u << (kTaps - 1));
  }
#pragma unroll
  for (int off = 1; off < kBlockRows; off <<= 1) m |= __shfl_xor(m, off, 64);
  uint32_t active = (lane & (kBlockRows - 1)) == 0 ? __popc(m) : 0u;
#pragma unroll
  for (int off = kBlockRows; off < 64; off <<= 1) {
    active += __shfl_xor(active, off, 64);
    m |= __shfl_xor(m, off, 64);
  }
  __shared__ uint32_t part[4][2];
  if (lane == 0) {
    part[wave][0] = active;
    part[wave][1] = m;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 2 + threadIdx.x;
    if (t < full_tiles) {
      const uint32_t a = part[2 * threadIdx.x][0] + part[2 * threadIdx.x + 1][0];
      const uint32_t u = part[2 * threadIdx.x][1] | part[2 * threadIdx.x + 1][1];
      cost[t] = kStageCost * __popc(u) + a;
    }
  }
}

// One workgroup: the full tiles in ascending cost, ties in tile order (a stable counting
// sort) -> order[0, full_tiles).  The k=3 kernel's interleaved schedule walks the tiles from
// the last, so the costliest start first and the cheapest fill the end.  Ranks among equal
// costs inside a wave come from intersecting the ballots of the cost bits.
__global__ __launch_bounds__(1024) void k_tile_order(const uint32_t* __restrict__ cost,
                                                     int64_t full_tiles,
                                                     const unsigned long long* __restrict__ counts,
                                                     int32_t* __restrict__ order) {
  constexpr int kThreads = 1024, kWaves = kThreads / 64, kBits = 10;
  static_assert((1 << kBits) == kCostBins && kCostBins == kThreads, "one bin per thread");
  if (counts != nullptr && brick_order_wins(counts)) return;
  __shared__ uint16_t c[kOrderTiles];
  __shared__ uint32_t running[kCostBins];
  __shared__ uint16_t wcnt[kWaves][kCostBins];
  __shared__ uint32_t wsum[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int f = static_cast<int>(full_tiles);  // <= kOrderTiles
  running[tid] = 0;
  __syncthreads();
  for (int i = tid; i < f; i += kThreads) {
    const uint32_t v = cost[i];
    c[i] = static_cast<uint16_t>(v);
    atomicAdd(&running[v], 1u);
  }
  __syncthreads();
  // Exclusive scan of the bin counts: bin b starts after every cheaper tile.
  const uint32_t cnt = running[tid];
  uint32_t incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  for (int k = 0; k < wave; ++k) before += wsum[k];
  running[tid] = before + incl - cnt;
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int base = 0; base < f; base += kThreads) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) wcnt[w][tid] = 0;
    __syncthreads();
    const int i = base + tid;
    const bool valid = i < f;
    const uint32_t d = valid ? c[i] : 0u;
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < kBits; ++b) {
      const bool bit = (d >> b) & 1u;
      const unsigned long long bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const uint32_t rank = __popcll(peers & lt);
    if (valid && rank == 0) wcnt[wave][d] = static_cast<uint16_t>(__popcll(peers));
    __syncthreads();
    if (valid) {
      uint32_t pos = running[d] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][d];
      order[pos] = i;
    }
    __syncthreads();
    uint32_t add = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) add += wcnt[w][tid];
    running[tid] += add;
    __syncthreads();
  }
}

// perm, per-block tap masks and tap-major neighbour rows in sorted order.  A workgroup owns
// 256 sorted positions: it reads their 256 map rows cooperatively (consecutive lanes read
// consecutive entries of a row, so a wave touches a few 108-byte rows instead of 64 scattered
// words), stages them in LDS, then writes each tap's 256 entries as one coalesced run.  Each
// 16-lane group of a wave is one block for the tap masks.  With counts non-null the brick
// order (brick_rows) replaces the mask order when its (block, tap) count is at most 21/20 of
// the mask order's, and the header records the matching tile schedule.  With tile_order
// non-null the mask order's full tiles are taken in that order (the tiles holding padding
// stay last).
__global__ __launch_bounds__(256) void k_plan_fill(const int32_t* __restrict__ nbr, int64_t n,
                                                   const uint32_t* __restrict__ mask_rows,
                                                   const uint32_t* __restrict__ brick_rows,
                                                   const unsigned long long* __restrict__ counts,
                                                   const int32_t* __restrict__ tile_order,
                                                   int64_t full_tiles, int64_t npad,
                                                   int64_t* __restrict__ header,
                                                   int32_t* __restrict__ perm,
                                                   uint32_t* __restrict__ bmask,
                                                   int32_t* __restrict__ gidx) {
  __shared__ int32_t rows[256 * kTaps];  // row-major [position][tap]; stride 27 is odd, so a
                                         // wave's column reads hit distinct banks
  __shared__ int32_t src[256];
  const int tid = threadIdx.x;
  const bool spatial = counts != nullptr && brick_order_wins(counts);
  const uint32_t* sorted_rows = spatial ? brick_rows : mask_rows;
  if (blockIdx.x == 0 && tid == 0)
    header[kPlanSchedWord] = spatial ? kSchedPerXcd : kSchedInterleaved;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 256;
  const int64_t r = r0 + tid;  // < npad
  int64_t from = r;
  if (!spatial && tile_order != nullptr && r < full_tiles * kTileRows)
    from = static_cast<int64_t>(tile_order[r / kTileRows]) * kTileRows + r % kTileRows;
  const int32_t i = from < n ? static_cast<int32_t>(sorted_rows[from]) : -1;
  perm[r] = i;
  src[tid] = i;
  __syncthreads();
  for (int e = tid; e < 256 * kTaps; e += 256) {
    const int p = e / kTaps, t = e - p * kTaps;
    const int32_t ii = src[p];
    rows[e] = ii >= 0 ? nbr[static_cast<int64_t>(ii) * kTaps + t] : -1;
  }
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (int t = 0; t < kTaps; ++t) {
    const int32_t j = rows[tid * kTaps + t];
    gidx[t * npad + r] = j;
    if (j >= 0) m |= 1u << t;
  }
#pragma unroll
  for (int off = 1; off < kBlockRows; off <<= 1) m |= __shfl_xor(m, off, 64);
  if ((tid & (kBlockRows - 1)) == 0) bmask[r / kBlockRows] = m;
}

}  // namespace
}  // namespace ssc

using namespace ssc;

extern "C" size_t ssc_index_workspace_bytes(int64_t n) {
  return n < 0 ? 0 : index_layout(n).total;
}

namespace {
// Whether the dense rank index builds the map: its arrays must fit in the workspace the hash
// needs for the same n (so ssc_index_workspace_bytes covers both), which keeps it to grids of
// at most about 85 voxels per hash slot; otherwise the hash does.
bool dense_fits(int64_t n, uint64_t voxels) {
  return voxels > 0 && dense_index_layout(n, voxels).total <= index_layout(n).total;
}

ssc_status build_index_hash(const int4* coords, int64_t n, int32_t batch, const int32_t* grid,
                            int32_t* nbr, char* ws, hipStream_t s) {
  const IndexLayout L = index_layout(n);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws);
  auto* slots = reinterpret_cast<Slot*>(ws + L.off_slots);
  const int bs = 256;
  const uint64_t init_blocks = std::min<uint64_t>((L.cap + bs - 1) / bs, 8192);
  k_table_init<<<static_cast<unsigned>(init_blocks), bs, 0, s>>>(slots, L.cap, counters);
  const unsigned ins_blocks = static_cast<unsigned>(std::min<int64_t>((n + bs - 1) / bs, 65536));
  k_insert<<<ins_blocks, bs, 0, s>>>(coords, n, batch, grid[0], grid[1], grid[2], slots,
                                     L.cap - 1, counters);
  const int64_t q = n * kTaps;
  const unsigned q_blocks = static_cast<unsigned>(std::min<int64_t>((q + bs - 1) / bs, 262144));
  k_query<<<q_blocks, bs, 0, s>>>(coords, n, batch, grid[0], grid[1], grid[2], slots,
                                  L.cap - 1, nbr);
  return launch_status();
}

ssc_status build_index_dense(const int4* coords, int64_t n, int32_t batch, const int32_t* grid,
                             uint64_t voxels, int32_t* nbr, char* ws, hipStream_t s) {
  const DenseIndexLayout D = dense_index_layout(n, voxels);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws);
  auto* bits = reinterpret_cast<uint64_t*>(ws + D.b.off_bits);
  auto* local = reinterpret_cast<uint16_t*>(ws + D.b.off_local);
  auto* sup = reinterpret_cast<uint32_t*>(ws + D.b.off_super);
  auto* rows = reinterpret_cast<int32_t*>(ws + D.off_rows);
  dense_build(coords, n, batch, grid, 0, D.b, ws, counters, 1, nullptr, s);
  const int bs = 256;
  const unsigned site_blocks = static_cast<unsigned>(std::min<int64_t>((n + bs - 1) / bs, 65536));
  k_dense_rows<<<site_blocks, bs, 0, s>>>(coords, n, batch, grid[0], grid[1], grid[2], bits,
                                          local, sup, rows, counters + 2);
  k_dense_query<<<static_cast<unsigned>((n + kQuerySites - 1) / kQuerySites), kQuerySites, 0,
                  s>>>(coords, n, batch, grid[0], grid[1], grid[2], bits, local, sup, rows,
                       counters + 2, nbr);
  return launch_status();
}
}  // namespace

extern "C" ssc_status ssc_build_index_ex(const int32_t* coords, int64_t n, int32_t batch,
                                         const int32_t* grid, int32_t* nbr, void* workspace,
                                         size_t workspace_bytes, int32_t check, int32_t method,
                                         void* stream) {
  if (n < 0 || grid == nullptr) return SSC_ERR_ARG;
  if (method < SSC_INDEX_AUTO || method > SSC_INDEX_DENSE) return SSC_ERR_ARG;
  if (n > 0 && (coords == nullptr || nbr == nullptr || workspace == nullptr)) return SSC_ERR_ARG;
  if (batch < 1 || batch > kMaxCoord) return SSC_ERR_UNSUPPORTED;
  for (int a = 0; a < 3; ++a)
    if (grid[a] < 1 || grid[a] > kMaxCoord) return SSC_ERR_UNSUPPORTED;
  if (n * kTaps > (int64_t(1) << 40) || n >= (int64_t(1) << 31)) return SSC_ERR_UNSUPPORTED;
  if (n == 0) return SSC_OK;
  if (!aligned(coords, 16) || !aligned(workspace, kAlign) || !aligned(nbr, 4)) return SSC_ERR_ARG;
  const uint64_t voxels = dense_voxels(batch, grid);
  bool dense = method == SSC_INDEX_DENSE || (method == SSC_INDEX_AUTO && dense_fits(n, voxels));
  if (dense) {
    if (voxels == 0) return SSC_ERR_UNSUPPORTED;
    if (workspace_bytes < dense_index_layout(n, voxels).total) return SSC_ERR_WORKSPACE;
  } else if (workspace_bytes < index_layout(n).total) {
    return SSC_ERR_WORKSPACE;
  }
  hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  const int4* c4 = reinterpret_cast<const int4*>(coords);
  const ssc_status st = dense ? build_index_dense(c4, n, batch, grid, voxels, nbr, ws, s)
                              : build_index_hash(c4, n, batch, grid, nbr, ws, s);
  if (st != SSC_OK) return SSC_ERR_HIP;
  if (check) {
    uint32_t host[2] = {0, 0};
    if (hipMemcpyAsync(host, ws, sizeof(host), hipMemcpyDeviceToHost, s) != hipSuccess)
      return SSC_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SSC_ERR_HIP;
    if (host[0]) return SSC_ERR_COORD_RANGE;
    if (host[1]) return SSC_ERR_DUPLICATE;
  }
  return SSC_OK;
}

extern "C" ssc_status ssc_build_index(const int32_t* coords, int64_t n, int32_t batch,
                                      const int32_t* grid, int32_t* nbr, void* workspace,
                                      size_t workspace_bytes, int32_t check, void* stream) {
  return ssc_build_index_ex(coords, n, batch, grid, nbr, workspace, workspace_bytes, check,
                            SSC_INDEX_AUTO, stream);
}

extern "C" size_t ssc_index_workspace_bytes_ex(int64_t n, int32_t batch, const int32_t* grid,
                                               int32_t method) {
  if (n < 0 || method < SSC_INDEX_AUTO || method > SSC_INDEX_DENSE) return 0;
  if (method != SSC_INDEX_DENSE) return index_layout(n).total;
  if (grid == nullptr || batch < 1) return 0;
  const uint64_t voxels = dense_voxels(batch, grid);
  return voxels == 0 ? 0 : dense_index_layout(n, voxels).total;
}

extern "C" int32_t ssc_index_method(int64_t n, int32_t batch, const int32_t* grid) {
  if (n < 0 || grid == nullptr || batch < 1) return SSC_INDEX_HASH;
  return dense_fits(n, dense_voxels(batch, grid)) ? SSC_INDEX_DENSE : SSC_INDEX_HASH;
}

extern "C" size_t ssc_plan_bytes(int64_t n) { return n < 0 ? 0 : plan_layout(n).total; }

extern "C" size_t ssc_plan_workspace_bytes(int64_t n) {
  return n < 0 ? 0 : plan_work_layout(n).total;
}

extern "C" ssc_status ssc_plan_layout(int64_t n, int64_t* layout) {
  if (n < 0 || layout == nullptr) return SSC_ERR_ARG;
  const PlanLayout L = plan_layout(n);
  layout[0] = L.npad;
  layout[1] = static_cast<int64_t>(L.off_perm);
  layout[2] = static_cast<int64_t>(L.off_bmask);
  layout[3] = static_cast<int64_t>(L.off_gidx);
  layout[4] = static_cast<int64_t>(L.off_zero);
  return SSC_OK;
}

// Bits that hold values 0 .. count-1.
inline int bits_for(int64_t count) {
  int b = 0;
  while ((int64_t(1) << b) < count) ++b;
  return b;
}

extern "C" ssc_status ssc_build_plan(const int32_t* nbr, const int32_t* coords, int64_t n,
                                     int32_t batch, const int32_t* grid, void* plan,
                                     size_t plan_bytes, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (n < 0 || plan == nullptr || workspace == nullptr) return SSC_ERR_ARG;
  if (n > 0 && nbr == nullptr) return SSC_ERR_ARG;
  if (n >= (int64_t(1) << 31)) return SSC_ERR_UNSUPPORTED;
  if (!aligned(plan, kAlign) || !aligned(workspace, kAlign)) return SSC_ERR_ARG;
  // The spatial candidate: bricks per axis and the brick count of the whole grid.
  int axis_bits = 0;
  int64_t bricks = 1;
  if (coords != nullptr) {
    if (grid == nullptr || !aligned(coords, 16)) return SSC_ERR_ARG;
    if (batch < 1 || batch > kMaxCoord) return SSC_ERR_UNSUPPORTED;
    bricks = batch;
    for (int a = 0; a < 3; ++a) {
      if (grid[a] < 1 || grid[a] > kMaxCoord) return SSC_ERR_UNSUPPORTED;
      const int64_t per_axis = ((int64_t(grid[a]) - 1) >> kBrickShift) + 1;
      bricks *= per_axis;
      axis_bits = std::max(axis_bits, bits_for(per_axis));
    }
  }
  const bool try_bricks = coords != nullptr && n > 0 && bricks >= kMinBricks;
  const PlanLayout P = plan_layout(n);
  const PlanWork W = plan_work_layout(n);
  if (plan_bytes < P.total || workspace_bytes < W.total) return SSC_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  char* pb = static_cast<char*>(plan);
  char* ws = static_cast<char*>(workspace);
  auto* masks = reinterpret_cast<uint32_t*>(ws + W.off_mask);
  auto* counts = reinterpret_cast<unsigned long long*>(ws + W.off_count);
  if (n == 0)
    k_plan_header<<<1, 64, 0, s>>>(reinterpret_cast<int64_t*>(pb), n, P.npad, P.nblocks,
                                   reinterpret_cast<uint4*>(pb + P.off_zero));
  uint32_t* mask_rows = reinterpret_cast<uint32_t*>(ws + W.g.off_vals_a);
  uint32_t* brick_rows = nullptr;
  const uint32_t* sorted_keys = nullptr;
  int32_t* tile_order = nullptr;
  if (n > 0) {
    const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
    k_mask_keys<<<blocks, 256, 0, s>>>(nbr, n, reinterpret_cast<uint32_t*>(ws + W.g.off_keys_a),
                                       mask_rows, reinterpret_cast<uint32_t*>(ws + W.g.off_totals),
                                       try_bricks ? masks : nullptr, counts,
                                       reinterpret_cast<int64_t*>(pb), P.npad, P.nblocks,
                                       reinterpret_cast<uint4*>(pb + P.off_zero));
    const bool keys_b = radix_sort_pairs<uint32_t, 9>(ws, W.g, n, kKeyBits, s) == 1;
    if (keys_b) mask_rows = reinterpret_cast<uint32_t*>(ws + W.g.off_vals_b);
    sorted_keys = reinterpret_cast<const uint32_t*>(ws + (keys_b ? W.g.off_keys_b : W.g.off_keys_a));
    if (try_bricks) {
      // Stable sort of the mask order by brick: within a brick the mask order remains.
      brick_rows = reinterpret_cast<uint32_t*>(ws + W.b.off_vals_a);
      k_brick_keys<<<blocks, 256, 0, s>>>(
          reinterpret_cast<const int4*>(coords), mask_rows, n, axis_bits,
          reinterpret_cast<unsigned long long*>(ws + W.b.off_keys_a), brick_rows,
          reinterpret_cast<uint32_t*>(ws + W.b.off_totals));
      if (radix_sort_pairs<uint64_t>(ws, W.b, n, bits_for(batch) + 3 * axis_bits, s) == 1)
        brick_rows = reinterpret_cast<uint32_t*>(ws + W.b.off_vals_b);
      k_block_taps<<<blocks, 256, 0, s>>>(mask_rows, brick_rows, masks, n, counts);
    }
    // Full tiles of the mask order by cost (both kernels return at once if the brick order
    // wins).
    if (W.full_tiles > 1 && W.full_tiles <= kOrderTiles) {
      auto* cost = reinterpret_cast<uint32_t*>(ws + W.off_cost);
      tile_order = reinterpret_cast<int32_t*>(ws + W.off_tiles);
      k_tile_cost<<<static_cast<unsigned>((W.full_tiles + 1) / 2), 256, 0, s>>>(
          sorted_keys, W.full_tiles, try_bricks ? counts : nullptr, cost);
      k_tile_order<<<1, 1024, 0, s>>>(cost, W.full_tiles, try_bricks ? counts : nullptr,
                                      tile_order);
    }
  }
  k_plan_fill<<<static_cast<unsigned>(P.npad / 256), 256, 0, s>>>(
      nbr, n, mask_rows, brick_rows, try_bricks ? counts : nullptr, tile_order, W.full_tiles,
      P.npad,
      reinterpret_cast<int64_t*>(pb), reinterpret_cast<int32_t*>(pb + P.off_perm),
      reinterpret_cast<uint32_t*>(pb + P.off_bmask), reinterpret_cast<int32_t*>(pb + P.off_gidx));
  return launch_status();
}
