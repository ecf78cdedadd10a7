// Dense rank structure over a voxel grid: an occupancy bitmap of the dense voxel id
// v = ((b * Gx + x) * Gy + y) * Gz + z with running counts, so that the rank of a set bit (the
// number of set bits before it) is the voxel's position in ascending (b, x, y, z) order.  This
// is the sorted-key index map (LATO.2 MLX port page, module table: gather / scatter over a
// sorted-key indice map) with the search replaced by a rank: a lookup is the voxel's bitmap
// word, the running count of its 1024-word superblock (32-bit) and of the word inside it
// (16-bit), and a popcount.  The arrays take about 3/16 byte per voxel.
//
// Used by the neighbour map (voxels = sites) and by the factor-2 downsample (voxels = parent
// cells, each site marking the cell x >> 1, y >> 1, z >> 1).  Device code only.
//   k_dense_clear  zero the bitmap (whole superblocks) and two error counters
//   k_dense_mark   one thread per site: validate, set the bit of its voxel (at level `shift`);
//                  lanes of a wave that set bits of one word (runs of equal words, as sites in
//                  key order give) OR them together first, so one 64-bit atomic serves the
//                  run; optionally a bit set twice counts as a duplicate
//   k_dense_count  one workgroup per superblock: each word's running count inside it and the
//                  superblock's total
//   k_dense_scan   one workgroup: exclusive scan of the superblock totals; the grand total
//                  lands past the last superblock
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "common.h"

namespace ssc {
namespace {

constexpr int kSuperWords = 1024;  // bitmap words per superblock (65536 voxels)

// The bitmap, its running counts and the superblock counts, from `base` in a workspace.
struct DenseBits {
  uint64_t voxels, words, supers;
  size_t off_bits, off_local, off_super, end;
};

inline DenseBits dense_bits_layout(uint64_t voxels, size_t base) {
  DenseBits L;
  L.voxels = voxels;
  L.words = (voxels + 63) / 64;
  L.supers = (L.words + kSuperWords - 1) / kSuperWords;
  L.off_bits = align_up(base);
  L.off_local = align_up(L.off_bits + sizeof(uint64_t) * L.supers * kSuperWords);
  L.off_super = align_up(L.off_local + sizeof(uint16_t) * L.supers * kSuperWords);
  L.end = align_up(L.off_super + sizeof(uint32_t) * (L.supers + 1));
  return L;
}

// Voxels of batch x (grid cells of 2^shift voxels per axis, rounded up), or 0 when the count
// does not fit 62 bits.
inline uint64_t dense_voxels(int32_t batch, const int32_t* grid, int shift = 0) {
  unsigned __int128 v = static_cast<unsigned __int128>(batch);
  for (int a = 0; a < 3; ++a) v *= (static_cast<uint64_t>(grid[a]) + (1u << shift) - 1) >> shift;
  return v >> 62 ? 0 : static_cast<uint64_t>(v);
}

__device__ __forceinline__ uint64_t dense_id(int b, int x, int y, int z, int gx, int gy, int gz) {
  return ((static_cast<uint64_t>(b) * gx + x) * gy + y) * static_cast<uint64_t>(gz) + z;
}

__device__ __forceinline__ bool in_range(int4 c, int batch, int gx, int gy, int gz) {
  return c.x >= 0 && c.x < batch && c.y >= 0 && c.y < gx && c.z >= 0 && c.z < gy && c.w >= 0 &&
         c.w < gz;
}

// Also sets fill[0, fill_count) to -1 when fill is given (a table the caller fills next).
// counters[0, 3) are cleared: out-of-range sites, duplicates, and a flag the index's row pass
// sets when the sites are not in key order.
__global__ void k_dense_clear(uint64_t* __restrict__ bits, uint64_t words,
                              uint32_t* __restrict__ counters, int32_t* __restrict__ fill,
                              int64_t fill_count) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < words;
       i += stride)
    bits[i] = 0ull;
  if (fill != nullptr)
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
         i < static_cast<uint64_t>(fill_count); i += stride)
      fill[i] = -1;
  if (blockIdx.x == 0 && threadIdx.x < 3) counters[threadIdx.x] = 0;
}

// Sites outside [0, batch) x (gx, gy, gz) count in counters[0] and mark nothing; the bit of a
// site is that of its cell (b, x >> shift, y >> shift, z >> shift) in the grid (px, py, pz).
// With count_dups a bit set twice counts in counters[1].  Grid-stride over whole waves (every
// lane of a wave runs the same iterations, so the lane shuffles see all 64 lanes).
__global__ __launch_bounds__(256) void k_dense_mark(const int4* __restrict__ coords, int64_t n,
                                                    int batch, int gx, int gy, int gz, int shift,
                                                    int px, int py, int pz,
                                                    unsigned long long* __restrict__ bits,
                                                    uint32_t* __restrict__ counters,
                                                    int count_dups) {
  const int lane = threadIdx.x & 63;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * blockDim.x + (threadIdx.x & ~63);
       base < n; base += stride) {
    const int64_t i = base + lane;
    bool bad = false;
    uint64_t w = ~0ull;  // no word: lanes past n and sites outside the grid
    unsigned long long m = 0ull;
    if (i < n) {
      const int4 c = coords[i];  // (b, x, y, z)
      if (in_range(c, batch, gx, gy, gz)) {
        const uint64_t v = dense_id(c.x, c.y >> shift, c.z >> shift, c.w >> shift, px, py, pz);
        w = v >> 6;
        m = 1ull << (v & 63);
      } else {
        bad = true;
      }
    }
    // Runs of equal words among consecutive lanes: segment id = heads up to this lane.
    const uint64_t wprev = __shfl_up(w, 1, 64);
    const bool head = lane == 0 || wprev != w;
    const unsigned long long heads = __ballot(head);
    const int seg = __popcll(heads & ((2ull << lane) - 1ull));
    bool dup = false;
    unsigned long long acc = m;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned long long o = __shfl_up(acc, off, 64);
      const int oseg = __shfl_up(seg, off, 64);
      if (lane >= off && oseg == seg) {
        dup |= (acc & o) != 0ull;  // the two ORs cover disjoint lanes of the run
        acc |= o;
      }
    }
    const int nseg = __shfl_down(seg, 1, 64);
    const bool tail = lane == 63 || nseg != seg;
    if (tail && w != ~0ull) {
      if (atomicOr(&bits[w], acc) & acc) dup = true;
    }
    if (bad) atomicAdd(&counters[0], 1u);
    if (dup && count_dups) atomicAdd(&counters[1], 1u);
  }
}

// One workgroup (1024 threads, one word each) per superblock: block-wide exclusive scan of
// the words' popcounts (< 65536: 16 bits) and the superblock total.
__global__ __launch_bounds__(1024) void k_dense_count(const uint64_t* __restrict__ bits,
                                                      uint16_t* __restrict__ local,
                                                      uint32_t* __restrict__ super_count) {
  __shared__ uint32_t wsum[16];
  const uint64_t wd = static_cast<uint64_t>(blockIdx.x) * kSuperWords + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t c = static_cast<uint32_t>(__popcll(bits[wd]));
  uint32_t incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  for (int k = 0; k < wave; ++k) before += wsum[k];
  local[wd] = static_cast<uint16_t>(before + incl - c);
  if (threadIdx.x == kSuperWords - 1) super_count[blockIdx.x] = before + incl;
}

// One workgroup of 1024 threads: in-place exclusive scan of the superblock totals, in chunks
// of 1024 with a running carry; super_count[supers] receives the grand total.  With result,
// result[0] = the grand total and result[1] = *bad.
__global__ __launch_bounds__(1024) void k_dense_scan(uint32_t* __restrict__ super_count,
                                                     uint64_t supers,
                                                     int64_t* __restrict__ result,
                                                     const uint32_t* __restrict__ bad) {
  __shared__ uint32_t wsum[16];
  __shared__ uint32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (uint64_t base = 0; base < supers; base += 1024) {
    const uint64_t i = base + threadIdx.x;
    const uint32_t c = i < supers ? super_count[i] : 0u;
    uint32_t incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = carry;
    for (int k = 0; k < wave; ++k) before += wsum[k];
    if (i < supers) super_count[i] = before + incl - c;
    __syncthreads();
    if (threadIdx.x == 1023) carry = before + incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    super_count[supers] = carry;
    if (result != nullptr) {
      result[0] = carry;
      result[1] = *bad;
    }
  }
}

// Rank of set bit v (its word given) among all set bits.
__device__ __forceinline__ uint32_t dense_rank(const uint16_t* __restrict__ local,
                                               const uint32_t* __restrict__ super_count,
                                               uint64_t v, uint64_t word) {
  const uint64_t w = v >> 6;
  const uint64_t below = word & ((1ull << (v & 63)) - 1ull);
  return super_count[w / kSuperWords] + local[w] + static_cast<uint32_t>(__popcll(below));
}

// Enqueues clear, mark, count and scan for n sites at level `shift`; bits etc. per D.
inline void dense_build(const int4* coords, int64_t n, int32_t batch, const int32_t* grid,
                        int shift, const DenseBits& D, char* ws, uint32_t* counters,
                        int count_dups, int64_t* result, hipStream_t s,
                        int32_t* fill = nullptr, int64_t fill_count = 0) {
  auto* bits = reinterpret_cast<uint64_t*>(ws + D.off_bits);
  auto* local = reinterpret_cast<uint16_t*>(ws + D.off_local);
  auto* sup = reinterpret_cast<uint32_t*>(ws + D.off_super);
  const int bs = 256;
  const uint64_t words = D.supers * kSuperWords;  // whole superblocks, tail words zero
  const uint64_t items = std::max<uint64_t>(words, static_cast<uint64_t>(fill_count));
  k_dense_clear<<<static_cast<unsigned>(std::min<uint64_t>((items + bs - 1) / bs, 8192)), bs, 0,
                  s>>>(bits, words, counters, fill, fill_count);
  const unsigned site_blocks = static_cast<unsigned>(std::min<int64_t>((n + bs - 1) / bs, 65536));
  const int p[3] = {static_cast<int>((grid[0] + (1 << shift) - 1) >> shift),
                    static_cast<int>((grid[1] + (1 << shift) - 1) >> shift),
                    static_cast<int>((grid[2] + (1 << shift) - 1) >> shift)};
  k_dense_mark<<<site_blocks, bs, 0, s>>>(coords, n, batch, grid[0], grid[1], grid[2], shift,
                                          p[0], p[1], p[2],
                                          reinterpret_cast<unsigned long long*>(bits), counters,
                                          count_dups);
  k_dense_count<<<static_cast<unsigned>(D.supers), kSuperWords, 0, s>>>(bits, local, sup);
  k_dense_scan<<<1, 1024, 0, s>>>(sup, D.supers, result, counters);
}

}  // namespace
}  // namespace ssc
