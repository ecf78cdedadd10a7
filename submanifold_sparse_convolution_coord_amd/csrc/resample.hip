// Coordinate-changing neighbours of the convolution: the factor-2 sparse downsample (max
// pool), its cache-paired upsample, the spatial-to-channel shuffle, and the x8 subdivide.
//
// The LATO.2 page ("Status") lists SparseDownsample as a max pool (upstream passes
// reduce="amax") and, in its module table, replaces strided sparse convolution by
// SparseSubdivide (a coordinate expansion by 8); the Pixal3D README's module table pairs
// SparseUpsample(2) with a downsample through the cached mapping.  Each produces a new
// coordinate set, which the convolution then indexes cold.
//
//   downsample: parent(b,x,y,z) = (b, x>>1, y>>1, z>>1).  Parents are numbered in ascending
//               order of their dense row-major index in [batch, ceil(gx/2), ceil(gy/2),
//               ceil(gz/2)]: when that grid's bitmap fits the workspace, by the dense rank
//               structure of dense.h (every site marks its parent cell; a parent's number is
//               the rank of its bit: five launches); otherwise by a stable LSD radix sort of
//               (key, site), the first site of each run starting a parent and an exclusive
//               scan numbering them.  Either way each parent's 8 child slots (child k =
//               4(x&1) + 2(y&1) + (z&1)) record its sites, and its feature is the channel-wise
//               maximum over them.  `parent[i]` maps every input site to its parent.
//   upsample:   out[i] = parent_feats[parent[i]] for the parent map of a downsample.
//   spatial2channel: the same parents; parent p's features are its 8 children's, channel c of
//               child k = 4(x&1) + 2(y&1) + (z&1) at column c*8 + k, zeros for absent
//               children (Pixal3D README, module table: SparseSpatial2Channel(2)).
//   subdivide:  site i becomes 8 sites 8i + 4dx + 2dy + dz at (b, 2x+dx, 2y+dy, 2z+dz), each
//               with site i's features.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "dense.h"
#include "sort.h"

namespace ssc {
namespace {

constexpr int kScanTile = 2048;  // items per workgroup in the parent numbering scan

// Workspace of the downsample: the numbering's scratch (the sort path's buffers, or the dense
// path's bitmap in the same bytes), the parents' child slots (8 int32 per site: m <= n
// parents) and a counter.
struct DownLayout {
  SortLayout<uint64_t> sort;
  int64_t scan_tiles;
  size_t off_tile_sums, off_children, off_counter, total;
};

// Small device-side initialisations (no memset nodes in a stream a caller may capture).
__global__ void k_fill_u32(uint32_t* __restrict__ p, int count, uint32_t v) {
  if (static_cast<int>(threadIdx.x) < count) p[threadIdx.x] = v;
}
__global__ void k_zero_result(int64_t* __restrict__ result) {
  if (threadIdx.x < 2) result[threadIdx.x] = 0;
}

inline DownLayout down_layout(int64_t n) {
  DownLayout L;
  const int64_t m = n > 0 ? n : 1;
  L.sort = sort_layout<uint64_t>(m, 0);
  L.scan_tiles = (m + kScanTile - 1) / kScanTile;
  L.off_tile_sums = align_up(L.sort.total);
  L.off_children = align_up(L.off_tile_sums + sizeof(uint32_t) * L.scan_tiles);
  L.off_counter = align_up(L.off_children + sizeof(int32_t) * 8 * m);
  L.total = align_up(L.off_counter + sizeof(uint32_t) * 4);
  return L;
}

// The dense numbering's bitmap of the parent grid, in the numbering's scratch bytes.
inline DenseBits down_dense(uint64_t parent_cells) { return dense_bits_layout(parent_cells, 0); }
inline bool down_dense_fits(int64_t n, uint64_t parent_cells) {
  return parent_cells > 0 && down_dense(parent_cells).end <= down_layout(n).off_children;
}

__device__ __forceinline__ int child_slot(int4 c) {
  return ((c.y & 1) << 2) | ((c.z & 1) << 1) | (c.w & 1);
}

// Parent key of every site (invalid rows are counted and keyed 0); clears the sort totals and
// the invalid-row counter's neighbours.
__global__ void k_parent_keys(const int4* __restrict__ coords, int64_t n, int batch, int gx, int gy,
                              int gz, uint64_t hx, uint64_t hy, uint64_t hz,
                              uint64_t* __restrict__ keys, uint32_t* __restrict__ vals,
                              uint32_t* __restrict__ totals, uint32_t* __restrict__ bad,
                              int32_t* __restrict__ children) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0)
    for (int d = threadIdx.x; d < kDigits; d += blockDim.x) totals[d] = 0;
  if (i >= n) return;
#pragma unroll
  for (int k = 0; k < 8; ++k) children[i * 8 + k] = -1;  // slots of parent i, if it exists
  const int4 c = coords[i];
  uint64_t key = 0;
  if (c.x < 0 || c.x >= batch || c.y < 0 || c.y >= gx || c.z < 0 || c.z >= gy || c.w < 0 ||
      c.w >= gz) {
    atomicAdd(bad, 1u);
  } else {
    key = ((static_cast<uint64_t>(c.x) * hx + static_cast<uint64_t>(c.y >> 1)) * hy +
           static_cast<uint64_t>(c.z >> 1)) * hz + static_cast<uint64_t>(c.w >> 1);
  }
  keys[i] = key;
  vals[i] = static_cast<uint32_t>(i);
}

__device__ __forceinline__ uint32_t is_head(const uint64_t* __restrict__ keys, int64_t r, int64_t n) {
  return (r < n && (r == 0 || keys[r] != keys[r - 1])) ? 1u : 0u;
}

// Parents starting in each scan tile.
__global__ __launch_bounds__(256) void k_head_counts(const uint64_t* __restrict__ keys, int64_t n,
                                                     uint32_t* __restrict__ tile_sums) {
  __shared__ uint32_t sh[256];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanTile;
  uint32_t c = 0;
  for (int k = 0; k < kScanTile / 256; ++k) c += is_head(keys, base + k * 256 + threadIdx.x, n);
  const uint32_t tot = block_inclusive_scan(c, sh);
  if (threadIdx.x == 255) tile_sums[blockIdx.x] = tot;
}

// Exclusive scan of the tile counts in place (one workgroup); the parent count goes to
// result[0].
__global__ __launch_bounds__(256) void k_scan_tile_sums(uint32_t* __restrict__ tile_sums,
                                                        int64_t tiles, int64_t* __restrict__ result,
                                                        const uint32_t* __restrict__ bad) {
  __shared__ uint32_t sh[256];
  uint32_t carry = 0;
  for (int64_t base = 0; base < tiles; base += 256) {
    const int64_t e = base + threadIdx.x;
    const uint32_t v = e < tiles ? tile_sums[e] : 0u;
    const uint32_t inc = block_inclusive_scan(v, sh);
    if (e < tiles) tile_sums[e] = carry + inc - v;
    if (threadIdx.x == 255) sh[0] = inc;
    __syncthreads();
    carry += sh[0];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    result[0] = carry;
    result[1] = *bad;
  }
}

// Numbers the parents in sorted order: parent id of sorted position r = (heads in [0, r]) - 1.
// Writes each site's parent, each parent's coordinates and the position its run starts at.
__global__ __launch_bounds__(256) void k_assign_parents(
    const uint64_t* __restrict__ keys, const uint32_t* __restrict__ vals, int64_t n,
    const uint32_t* __restrict__ tile_offsets, uint64_t hx, uint64_t hy, uint64_t hz,
    const int4* __restrict__ coords, int32_t* __restrict__ parent, int4* __restrict__ out_coords,
    int32_t* __restrict__ children) {
  __shared__ uint32_t sh[256];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanTile;
  constexpr int kPer = kScanTile / 256;
  // Thread t owns the kPer consecutive positions base + t*kPer .. +kPer-1.
  uint32_t h[kPer];
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    h[k] = is_head(keys, base + threadIdx.x * kPer + k, n);
    c += h[k];
  }
  const uint32_t inc = block_inclusive_scan(c, sh);
  uint32_t run = tile_offsets[blockIdx.x] + inc - c;  // heads before this thread's first item
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int64_t r = base + threadIdx.x * kPer + k;
    if (r >= n) break;
    run += h[k];
    const int32_t p = static_cast<int32_t>(run) - 1;
    const uint32_t site = vals[r];
    parent[site] = p;
    children[static_cast<int64_t>(p) * 8 + child_slot(coords[site])] = static_cast<int32_t>(site);
    if (h[k]) {
      const uint64_t key = keys[r];
      const uint64_t z = key % hz, rest = key / hz;
      const uint64_t y = rest % hy, rest2 = rest / hy;
      const uint64_t x = rest2 % hx, b = rest2 / hx;
      out_coords[p] = make_int4(static_cast<int>(b), static_cast<int>(x), static_cast<int>(y),
                                static_cast<int>(z));
    }
  }
}

// Dense numbering, after dense.h's build over the parent cells: site i's parent is the rank
// of its cell's bit; it records the site in the parent's child slot and the parent's
// coordinates (every child writes the same four values).
__global__ void k_ds_assign(const int4* __restrict__ coords, int64_t n, int batch, int gx, int gy,
                            int gz, int hx, int hy, int hz, const uint64_t* __restrict__ bits,
                            const uint16_t* __restrict__ local,
                            const uint32_t* __restrict__ super_count,
                            int32_t* __restrict__ parent, int4* __restrict__ out_coords,
                            int32_t* __restrict__ children) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride) {
    const int4 c = coords[i];
    if (!in_range(c, batch, gx, gy, gz)) {
      parent[i] = -1;
      continue;
    }
    const uint64_t v = dense_id(c.x, c.y >> 1, c.z >> 1, c.w >> 1, hx, hy, hz);
    const uint32_t p = dense_rank(local, super_count, v, bits[v >> 6]);
    parent[i] = static_cast<int32_t>(p);
    children[static_cast<int64_t>(p) * 8 + child_slot(c)] = static_cast<int32_t>(i);
    out_coords[p] = make_int4(c.x, c.y >> 1, c.z >> 1, c.w >> 1);
  }
}

// Channel-wise maximum, 8 bf16 channels (one 16-byte word) per thread; channels % 8 == 0.
// The parent's sites are its child slots, taken in slot order; a larger value replaces the
// running maximum, so the result is one of the inputs, bit for bit.
__global__ void k_maxpool_bf16x8(const uint4* __restrict__ feats, int32_t words,
                                 const int32_t* __restrict__ children,
                                 const int64_t* __restrict__ result, uint4* __restrict__ out) {
  const int64_t m = result[0];
  const int64_t total = m * words;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += stride) {
    const int64_t p = g / words;
    const int w = static_cast<int>(g - p * words);
    // The parent's 8 child slots (32-byte aligned: the slot array starts on a 256-byte boundary
    // of the workspace) in two 16-byte loads, then every present child's word loaded before any
    // is compared, so that a thread has all its loads in flight at once (a loop of index load,
    // branch and feature load kept one in flight).  The maximum is taken in child order, keeping
    // the first of equal values, as before.
    const int4 c0 = *reinterpret_cast<const int4*>(children + p * 8);
    const int4 c1 = *reinterpret_cast<const int4*>(children + p * 8 + 4);
    const int32_t idx[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = idx[k] >= 0 ? feats[static_cast<int64_t>(idx[k]) * words + w]
                         : make_uint4(0u, 0u, 0u, 0u);
    uint4 best = make_uint4(0u, 0u, 0u, 0u);  // every parent has a site; zeros if none
    bool have = false;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (idx[k] < 0) continue;
      if (!have) {
        best = v[k];
        have = true;
        continue;
      }
      uint32_t* bb = reinterpret_cast<uint32_t*>(&best);
      const uint32_t* vv = reinterpret_cast<const uint32_t*>(&v[k]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // two bf16 per word: keep the larger of each half, bits and all
        const uint32_t lo_b = bb[q] & 0xffffu, hi_b = bb[q] >> 16;
        const uint32_t lo_v = vv[q] & 0xffffu, hi_v = vv[q] >> 16;
        const uint32_t lo = bf16_to_f32(static_cast<uint16_t>(lo_v)) > bf16_to_f32(static_cast<uint16_t>(lo_b)) ? lo_v : lo_b;
        const uint32_t hi = bf16_to_f32(static_cast<uint16_t>(hi_v)) > bf16_to_f32(static_cast<uint16_t>(hi_b)) ? hi_v : hi_b;
        bb[q] = lo | (hi << 16);
      }
    }
    out[g] = best;
  }
}

__device__ __forceinline__ float ld_f(const float* p) { return *p; }
__device__ __forceinline__ float ld_f(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float ld_f(const _Float16* p) { return static_cast<float>(*p); }

// Channel-wise maximum over each parent's sites (its child slots, in slot order).  Thread per
// (parent, channel); parents past the count (read on the device) do nothing.
template <typename T>
__global__ void k_maxpool(const T* __restrict__ feats, int32_t channels,
                          const int32_t* __restrict__ children,
                          const int64_t* __restrict__ result, T* __restrict__ out) {
  const int64_t m = result[0];
  const int64_t total = m * channels;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += stride) {
    const int64_t p = g / channels;
    const int c = static_cast<int>(g - p * channels);
    const int32_t* ch = children + p * 8;
    int k0 = 0;
    while (k0 < 7 && ch[k0] < 0) ++k0;  // every parent has at least one site
    if (ch[k0] < 0) {
      out[g] = T{};
      continue;
    }
    int64_t best_row = ch[k0];
    float best = ld_f(feats + best_row * channels + c);
    for (int k = k0 + 1; k < 8; ++k) {
      if (ch[k] < 0) continue;
      const float v = ld_f(feats + static_cast<int64_t>(ch[k]) * channels + c);
      if (v > best) {
        best = v;
        best_row = ch[k];
      }
    }
    out[g] = feats[best_row * channels + c];  // the maximum's own bits
  }
}

// Spatial-to-channel (a sparse 3D pixel unshuffle): parent p's row holds, for every channel c,
// its 8 children's values at c*8 + k, k = 4(x&1) + 2(y&1) + (z&1); absent children give 0.
// Thread per (parent, channel); the element type only moves bits.
template <typename T>
__global__ void k_space2channel(const T* __restrict__ feats, int32_t channels,
                                const int32_t* __restrict__ children,
                                const int64_t* __restrict__ result, T* __restrict__ out) {
  const int64_t m = result[0];
  const int64_t total = m * channels;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += stride) {
    const int64_t p = g / channels;
    const int c = static_cast<int>(g - p * channels);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int32_t i = children[p * 8 + k];
      out[g * 8 + k] = i >= 0 ? feats[static_cast<int64_t>(i) * channels + c] : T{};
    }
  }
}

// Output rows of the row-copy kernels (upsample, subdivide, spatial-to-channel) are stored
// non-temporally: they are written once and not read again by the kernel, and streaming them
// past the caches doubled the rate of the write-heavy ops (128^3, 10%, 128 bf16 channels:
// subdivide 108.9 -> 68.2 us for 513 MB, spatial-to-channel 123.5 -> 79.3 us with its parent
// numbering; 512^3 shell, 32 channels: 183.5 -> 117.7 us and 78.9 -> 68.5 us).
typedef uint32_t st_u32x4_t __attribute__((ext_vector_type(4)));
template <typename W>
__device__ __forceinline__ void st_out(W* p, const W& v) {
  if constexpr (sizeof(W) == 16)
    __builtin_nontemporal_store(__builtin_bit_cast(st_u32x4_t, v), reinterpret_cast<st_u32x4_t*>(p));
  else
    __builtin_nontemporal_store(v, p);
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Spatial-to-channel in words of 16 bytes (rows a multiple of 16 bytes): thread per (parent,
// word of E = 16 / ESZ channels).  The children's words land in 8 slot registers (zero for an
// absent child) and are transposed in registers into the 8 output words of the thread's E
// channels (columns c0*8 .. (c0+E)*8 - 1).  A block's 256 items own 256 * 8 consecutive
// output words, so the words go through LDS (slot e of thread t at t*8 + (e ^ (t & 7)), which
// spreads 8 neighbouring threads over distinct banks) and leave as consecutive 16-byte
// stores.  Every thread of a block runs the same number of rounds (the barriers need it).
template <int ESZ>
__global__ __launch_bounds__(256) void k_space2channel_w(const uint4* __restrict__ feats,
                                                         int32_t words,
                                                         const int32_t* __restrict__ children,
                                                         const int64_t* __restrict__ result,
                                                         uint4* __restrict__ out) {
  __shared__ uint4 stage[256 * 8];
  const int t = threadIdx.x;
  const int64_t m = result[0];
  const int64_t total = m * words;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256; base < total;
       base += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t g = base + t;
    uint4 o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = make_uint4(0u, 0u, 0u, 0u);
    if (g < total) {
      const int64_t p = g / words;
      const int w = static_cast<int>(g - p * words);
      uint4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int32_t i = children[p * 8 + k];
        v[k] = i >= 0 ? feats[static_cast<int64_t>(i) * words + w] : make_uint4(0u, 0u, 0u, 0u);
      }
      if constexpr (ESZ == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {  // channel c0 + e: its 8 slots make one word
          const int sh = (e & 1) * 16;
          uint32_t d[4];
#pragma unroll
          for (int h = 0; h < 4; ++h)
            d[h] = ((dword_of(v[2 * h], e >> 1) >> sh) & 0xffffu) |
                   (((dword_of(v[2 * h + 1], e >> 1) >> sh) & 0xffffu) << 16);
          o[e] = make_uint4(d[0], d[1], d[2], d[3]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // channel c0 + e: slots 0-3, then 4-7
          o[2 * e] = make_uint4(dword_of(v[0], e), dword_of(v[1], e), dword_of(v[2], e),
                                dword_of(v[3], e));
          o[2 * e + 1] = make_uint4(dword_of(v[4], e), dword_of(v[5], e), dword_of(v[6], e),
                                    dword_of(v[7], e));
        }
      }
    }
    __syncthreads();  // the previous round's words have left the stage
#pragma unroll
    for (int e = 0; e < 8; ++e) stage[t * 8 + (e ^ (t & 7))] = o[e];
    __syncthreads();
    const int64_t words_here = (total - base < 256 ? total - base : 256) * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = k * 256 + t;  // output word j of the block's run
      if (j < words_here) {
        const int src = j >> 3, e = j & 7;
        st_out(&out[base * 8 + j], stage[src * 8 + (e ^ (src & 7))]);
      }
    }
  }
}

// out[i] = src[parent[i]] row by row, in words of 16 bytes (rows a multiple of 16 bytes) or 4
// bytes; rows whose parent is outside [0, m) are written as zeros.
template <typename Word>
__global__ void k_gather_rows(const Word* __restrict__ src, const int32_t* __restrict__ parent,
                              int64_t n, int64_t m, int64_t row_words, Word* __restrict__ out) {
  const int64_t total = n * row_words;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += stride) {
    const int64_t i = g / row_words;
    const int64_t w = g - i * row_words;
    const int32_t p = parent[i];
    st_out(&out[g], (p >= 0 && p < m) ? src[static_cast<int64_t>(p) * row_words + w] : Word{});
  }
}

template <typename Word>
__global__ void k_subdivide(const int4* __restrict__ coords, int64_t n,
                            const Word* __restrict__ feats, int64_t row_words,
                            int4* __restrict__ out_coords, Word* __restrict__ out_feats) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < 8 * n;
       c += stride) {
    const int64_t i = c >> 3;
    const int k = static_cast<int>(c & 7);
    const int4 v = coords[i];
    out_coords[c] = make_int4(v.x, 2 * v.y + (k >> 2), 2 * v.z + ((k >> 1) & 1), 2 * v.w + (k & 1));
  }
  if (feats == nullptr) return;
  const int64_t total = 8 * n * row_words;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += stride) {
    const int64_t child = g / row_words;
    const int64_t w = g - child * row_words;
    st_out(&out_feats[g], feats[(child >> 3) * row_words + w]);
  }
}

unsigned grid_for(int64_t items, int64_t cap = 262144) {
  return static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>((items + 255) / 256, cap)));
}

int bits_for(uint64_t count) {  // bits needed for keys in [0, count)
  int b = 0;
  while (b < 64 && (count - 1) >> b) ++b;
  return b;
}

}  // namespace
}  // namespace ssc

using namespace ssc;

extern "C" size_t ssc_downsample_workspace_bytes(int64_t n) {
  return n < 0 ? 0 : down_layout(n).total;
}

namespace ssc {
namespace {

// Shared front of the downsample and the spatial-to-channel: checks, then numbers the
// parents (dense rank structure when the parent grid's bitmap fits the numbering's scratch,
// else the radix sort); both fill parent, out_coords, result and the child slots.  On success
// *children points at the slots.  Returns SSC_OK with *done = true when there is nothing left
// to launch.
ssc_status number_parents(const int32_t* coords, int64_t n, int32_t batch, const int32_t* grid,
                          const void* feats, int32_t dtype, int32_t channels, int32_t* out_coords,
                          void* out_feats, int32_t* parent, int64_t* result, void* workspace,
                          size_t workspace_bytes, hipStream_t s, const int32_t** children_out,
                          bool* done) {
  *done = true;
  if (n < 0 || grid == nullptr || result == nullptr || channels < 0) return SSC_ERR_ARG;
  if (dtype != SSC_F32 && dtype != SSC_BF16 && dtype != SSC_F16) return SSC_ERR_ARG;
  if (batch < 1 || batch > kMaxCoord) return SSC_ERR_UNSUPPORTED;
  for (int a = 0; a < 3; ++a)
    if (grid[a] < 1 || grid[a] > kMaxCoord) return SSC_ERR_UNSUPPORTED;
  if (n >= (int64_t(1) << 31)) return SSC_ERR_UNSUPPORTED;
  if (n > 0 && (coords == nullptr || out_coords == nullptr || parent == nullptr ||
                workspace == nullptr))
    return SSC_ERR_ARG;
  if (n > 0 && channels > 0 && (feats == nullptr || out_feats == nullptr)) return SSC_ERR_ARG;
  if (!aligned(coords, 16) || !aligned(out_coords, 16) || !aligned(workspace, kAlign) ||
      !aligned(result, 8))
    return SSC_ERR_ARG;
  const DownLayout L = down_layout(n);
  if (n > 0 && workspace_bytes < L.total) return SSC_ERR_WORKSPACE;
  if (n == 0) {
    k_zero_result<<<1, 64, 0, s>>>(result);
    return launch_status();
  }
  const uint64_t hx = (grid[0] + 1) / 2, hy = (grid[1] + 1) / 2, hz = (grid[2] + 1) / 2;
  char* ws = static_cast<char*>(workspace);
  auto* children = reinterpret_cast<int32_t*>(ws + L.off_children);
  auto* bad = reinterpret_cast<uint32_t*>(ws + L.off_counter);
  const int4* c4 = reinterpret_cast<const int4*>(coords);
  int4* oc = reinterpret_cast<int4*>(out_coords);
  const uint64_t cells = dense_voxels(batch, grid, 1);
  if (down_dense_fits(n, cells)) {
    const DenseBits D = down_dense(cells);
    dense_build(c4, n, batch, grid, 1, D, ws, bad, 0, result, s, children, 8 * n);
    k_ds_assign<<<grid_for(n), 256, 0, s>>>(
        c4, n, batch, grid[0], grid[1], grid[2], static_cast<int>(hx), static_cast<int>(hy),
        static_cast<int>(hz), reinterpret_cast<const uint64_t*>(ws + D.off_bits),
        reinterpret_cast<const uint16_t*>(ws + D.off_local),
        reinterpret_cast<const uint32_t*>(ws + D.off_super), parent, oc, children);
  } else {
    auto* keys = reinterpret_cast<uint64_t*>(ws + L.sort.off_keys_a);
    auto* vals = reinterpret_cast<uint32_t*>(ws + L.sort.off_vals_a);
    auto* totals = reinterpret_cast<uint32_t*>(ws + L.sort.off_totals);
    auto* tile_sums = reinterpret_cast<uint32_t*>(ws + L.off_tile_sums);
    k_fill_u32<<<1, 64, 0, s>>>(bad, 1, 0u);
    k_parent_keys<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
        c4, n, batch, grid[0], grid[1], grid[2], hx, hy, hz, keys, vals, totals, bad, children);
    const int bits = bits_for(static_cast<uint64_t>(batch) * hx * hy * hz);
    if (radix_sort_pairs<uint64_t, 9>(ws, L.sort, n, bits, s) == 1) {
      keys = reinterpret_cast<uint64_t*>(ws + L.sort.off_keys_b);
      vals = reinterpret_cast<uint32_t*>(ws + L.sort.off_vals_b);
    }
    k_head_counts<<<static_cast<unsigned>(L.scan_tiles), 256, 0, s>>>(keys, n, tile_sums);
    k_scan_tile_sums<<<1, 256, 0, s>>>(tile_sums, L.scan_tiles, result, bad);
    k_assign_parents<<<static_cast<unsigned>(L.scan_tiles), 256, 0, s>>>(
        keys, vals, n, tile_sums, hx, hy, hz, c4, parent, oc, children);
  }
  *children_out = children;
  *done = channels == 0;
  return launch_status();
}

}  // namespace
}  // namespace ssc

extern "C" ssc_status ssc_downsample2(const int32_t* coords, int64_t n, int32_t batch,
                                      const int32_t* grid, const void* feats, int32_t dtype,
                                      int32_t channels, int32_t* out_coords, void* out_feats,
                                      int32_t* parent, int64_t* result, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  hipStream_t s = as_stream(stream);
  const int32_t* ch = nullptr;
  bool done = true;
  const ssc_status st = number_parents(coords, n, batch, grid, feats, dtype, channels, out_coords,
                                       out_feats, parent, result, workspace, workspace_bytes, s,
                                       &ch, &done);
  if (st != SSC_OK || done) return st;
  const unsigned g = grid_for(n * channels);
  if (dtype == SSC_BF16 && channels % 8 == 0 && aligned(feats, 16) && aligned(out_feats, 16))
    k_maxpool_bf16x8<<<grid_for(n * (channels / 8)), 256, 0, s>>>(
        static_cast<const uint4*>(feats), channels / 8, ch, result,
        static_cast<uint4*>(out_feats));
  else if (dtype == SSC_BF16)
    k_maxpool<uint16_t><<<g, 256, 0, s>>>(static_cast<const uint16_t*>(feats), channels, ch,
                                          result, static_cast<uint16_t*>(out_feats));
  else if (dtype == SSC_F16)
    k_maxpool<_Float16><<<g, 256, 0, s>>>(static_cast<const _Float16*>(feats), channels, ch,
                                          result, static_cast<_Float16*>(out_feats));
  else
    k_maxpool<float><<<g, 256, 0, s>>>(static_cast<const float*>(feats), channels, ch, result,
                                       static_cast<float*>(out_feats));
  return launch_status();
}

extern "C" ssc_status ssc_spatial2channel2(const int32_t* coords, int64_t n, int32_t batch,
                                           const int32_t* grid, const void* feats, int32_t dtype,
                                           int32_t channels, int32_t* out_coords,
                                           void* out_feats, int32_t* parent, int64_t* result,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream) {
  if (channels < 1) return SSC_ERR_ARG;
  hipStream_t s = as_stream(stream);
  const int32_t* ch = nullptr;
  bool done = true;
  const ssc_status st = number_parents(coords, n, batch, grid, feats, dtype, channels, out_coords,
                                       out_feats, parent, result, workspace, workspace_bytes, s,
                                       &ch, &done);
  if (st != SSC_OK || done) return st;
  const int64_t row_bytes = static_cast<int64_t>(channels) * (dtype == SSC_F32 ? 4 : 2);
  if (row_bytes % 16 == 0 && aligned(feats, 16) && aligned(out_feats, 16)) {
    const int32_t words = static_cast<int32_t>(row_bytes / 16);
    const unsigned gw = grid_for(n * words);
    const auto* f4 = static_cast<const uint4*>(feats);
    auto* o4 = static_cast<uint4*>(out_feats);
    if (dtype == SSC_F32)
      k_space2channel_w<4><<<gw, 256, 0, s>>>(f4, words, ch, result, o4);
    else
      k_space2channel_w<2><<<gw, 256, 0, s>>>(f4, words, ch, result, o4);
    return launch_status();
  }
  const unsigned g = grid_for(n * channels);
  if (dtype == SSC_F32)
    k_space2channel<float><<<g, 256, 0, s>>>(static_cast<const float*>(feats), channels, ch,
                                             result, static_cast<float*>(out_feats));
  else
    k_space2channel<uint16_t><<<g, 256, 0, s>>>(static_cast<const uint16_t*>(feats), channels,
                                                ch, result, static_cast<uint16_t*>(out_feats));
  return launch_status();
}

extern "C" ssc_status ssc_upsample2(const void* parent_feats, int32_t dtype, int32_t channels,
                                    const int32_t* parent, int64_t n, int64_t m, void* out,
                                    void* stream) {
  if (n < 0 || m < 0 || channels < 1) return SSC_ERR_ARG;
  if (dtype != SSC_F32 && dtype != SSC_BF16 && dtype != SSC_F16) return SSC_ERR_ARG;
  if (n == 0) return SSC_OK;
  if (parent_feats == nullptr || parent == nullptr || out == nullptr) return SSC_ERR_ARG;
  const int64_t row_bytes = static_cast<int64_t>(channels) * (dtype == SSC_F32 ? 4 : 2);
  if (row_bytes % 4 != 0 || !aligned(parent_feats, 4) || !aligned(out, 4)) return SSC_ERR_ARG;
  hipStream_t s = as_stream(stream);
  if (row_bytes % 16 == 0 && aligned(parent_feats, 16) && aligned(out, 16))
    k_gather_rows<uint4><<<grid_for(n * (row_bytes / 16)), 256, 0, s>>>(
        static_cast<const uint4*>(parent_feats), parent, n, m, row_bytes / 16,
        static_cast<uint4*>(out));
  else
    k_gather_rows<uint32_t><<<grid_for(n * (row_bytes / 4)), 256, 0, s>>>(
        static_cast<const uint32_t*>(parent_feats), parent, n, m, row_bytes / 4,
        static_cast<uint32_t*>(out));
  return launch_status();
}

extern "C" ssc_status ssc_subdivide2(const int32_t* coords, int64_t n, const int32_t* grid,
                                     const void* feats, int32_t dtype, int32_t channels,
                                     int32_t* out_coords, void* out_feats, void* stream) {
  if (n < 0 || grid == nullptr || channels < 0) return SSC_ERR_ARG;
  if (dtype != SSC_F32 && dtype != SSC_BF16 && dtype != SSC_F16) return SSC_ERR_ARG;
  for (int a = 0; a < 3; ++a)
    if (grid[a] < 1 || 2 * static_cast<int64_t>(grid[a]) > kMaxCoord) return SSC_ERR_UNSUPPORTED;
  if (n >= (int64_t(1) << 28)) return SSC_ERR_UNSUPPORTED;
  if (n == 0) return SSC_OK;
  if (coords == nullptr || out_coords == nullptr) return SSC_ERR_ARG;
  if (channels > 0 && (feats == nullptr || out_feats == nullptr)) return SSC_ERR_ARG;
  const int64_t row_bytes = static_cast<int64_t>(channels) * (dtype == SSC_F32 ? 4 : 2);
  if (row_bytes % 4 != 0 || !aligned(coords, 16) || !aligned(out_coords, 16) ||
      (channels > 0 && (!aligned(feats, 4) || !aligned(out_feats, 4))))
    return SSC_ERR_ARG;
  hipStream_t s = as_stream(stream);
  const int4* c4 = reinterpret_cast<const int4*>(coords);
  int4* o4 = reinterpret_cast<int4*>(out_coords);
  if (channels > 0 && row_bytes % 16 == 0 && aligned(feats, 16) && aligned(out_feats, 16))
    k_subdivide<uint4><<<grid_for(8 * n * (row_bytes / 16)), 256, 0, s>>>(
        c4, n, static_cast<const uint4*>(feats), row_bytes / 16, o4,
        static_cast<uint4*>(out_feats));
  else
    k_subdivide<uint32_t><<<grid_for(8 * n * std::max<int64_t>(1, row_bytes / 4)), 256, 0, s>>>(
        c4, n, channels > 0 ? static_cast<const uint32_t*>(feats) : nullptr, row_bytes / 4, o4,
        channels > 0 ? static_cast<uint32_t*>(out_feats) : nullptr);
  return launch_status();
}
