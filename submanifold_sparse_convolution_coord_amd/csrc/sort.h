// Stable LSD radix sort of (key, uint32 value) pairs on the GPU, 8 or 9 bits per pass: per-tile
// digit histograms (with per-digit totals), a digit-major exclusive scan with one workgroup
// per digit, then a scatter that ranks equal digits within a wave by intersecting ballots, so
// equal keys keep their input order.  Used by the plan (32-bit keys) and by the coordinate
// downsample (64-bit keys).  Device code only; no host state.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"

namespace ssc {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortItems = 8;
constexpr int kSortTile = kSortThreads * kSortItems;
constexpr int kMaxDigitBits = 9;
constexpr int kMaxDigits = 1 << kMaxDigitBits;  // scratch is sized for the widest digit
constexpr int kDigits = kMaxDigits;             // totals to clear before a first pass


// Scratch of one sort of n pairs with K-byte keys: two key and two value buffers (ping-pong),
// the per-tile histograms and the per-digit totals.
template <typename K>
struct SortLayout {
  int64_t ntiles;
  size_t off_keys_a, off_keys_b, off_vals_a, off_vals_b, off_hist, off_totals, total;
};

template <typename K>
inline SortLayout<K> sort_layout(int64_t n, size_t base) {
  SortLayout<K> L;
  const int64_t m = n > 0 ? n : 1;
  L.ntiles = (m + kSortTile - 1) / kSortTile;
  L.off_keys_a = align_up(base);
  L.off_keys_b = align_up(L.off_keys_a + sizeof(K) * m);
  L.off_vals_a = align_up(L.off_keys_b + sizeof(K) * m);
  L.off_vals_b = align_up(L.off_vals_a + sizeof(uint32_t) * m);
  L.off_hist = align_up(L.off_vals_b + sizeof(uint32_t) * m);
  L.off_totals = align_up(L.off_hist + sizeof(uint32_t) * kMaxDigits * L.ntiles);
  L.total = align_up(L.off_totals + sizeof(uint32_t) * kMaxDigits);
  return L;
}

// Per-tile digit counts -> hist[digit][tile]; per-digit totals accumulate in totals[digit]
// (zeroed by the previous scatter, or by the kernel that wrote the keys before the first
// pass).  DB bits per digit; each thread owns (1 << DB) / kSortThreads digits.
template <typename K, int DB>
__global__ __launch_bounds__(kSortThreads) void k_sort_hist(const K* __restrict__ keys,
                                                            int64_t n, int shift,
                                                            uint32_t* __restrict__ hist,
                                                            int64_t ntiles,
                                                            uint32_t* __restrict__ totals) {
  constexpr int D = 1 << DB, DPT = D / kSortThreads;
  static_assert(DPT >= 1 && D <= kMaxDigits, "digit width");
  __shared__ uint32_t h[D];
#pragma unroll
  for (int k = 0; k < DPT; ++k) h[threadIdx.x * DPT + k] = 0;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortTile;
#pragma unroll
  for (int k = 0; k < kSortItems; ++k) {
    const int64_t e = base + k * kSortThreads + threadIdx.x;
    if (e < n) atomicAdd(&h[static_cast<uint32_t>(keys[e] >> shift) & (D - 1)], 1u);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < DPT; ++k) {
    const int d = threadIdx.x * DPT + k;
    hist[static_cast<int64_t>(d) * ntiles + blockIdx.x] = h[d];
    if (h[d]) atomicAdd(&totals[d], h[d]);
  }
}

// Block-wide inclusive scan of one value per thread (kSortThreads threads), Hillis-Steele.
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int off = 1; off < kSortThreads; off <<= 1) {
    const uint32_t add = threadIdx.x >= off ? sh[threadIdx.x - off] : 0u;
    __syncthreads();
    sh[threadIdx.x] += add;
    __syncthreads();
  }
  const uint32_t r = sh[threadIdx.x];
  __syncthreads();
  return r;
}

// Exclusive scan of hist in digit-major order, one workgroup per digit: the digit's base is
// the sum of the totals of all smaller digits, then its row of per-tile counts is scanned.
template <int DB>
__global__ __launch_bounds__(kSortThreads) void k_sort_scan_rows(uint32_t* __restrict__ hist,
                                                                 int64_t ntiles,
                                                                 const uint32_t* __restrict__ totals) {
  constexpr int DPT = (1 << DB) / kSortThreads;
  __shared__ uint32_t sh[kSortThreads];
  const int d = blockIdx.x;
  uint32_t part = 0;
#pragma unroll
  for (int k = 0; k < DPT; ++k) {
    const int j = threadIdx.x * DPT + k;
    part += j < d ? totals[j] : 0u;
  }
  const uint32_t below = block_inclusive_scan(part, sh);
  // The last thread's inclusive value is the sum over all smaller digits.
  if (threadIdx.x == kSortThreads - 1) sh[0] = below;
  __syncthreads();
  uint32_t carry = sh[0];
  __syncthreads();
  uint32_t* row = hist + static_cast<int64_t>(d) * ntiles;
  for (int64_t base = 0; base < ntiles; base += kSortThreads) {
    const int64_t e = base + threadIdx.x;
    const uint32_t v = e < ntiles ? row[e] : 0u;
    const uint32_t inc = block_inclusive_scan(v, sh);
    if (e < ntiles) row[e] = carry + inc - v;
    if (threadIdx.x == kSortThreads - 1) sh[0] = inc;
    __syncthreads();
    carry += sh[0];
    __syncthreads();
  }
}

template <typename K, int DB>
__global__ __launch_bounds__(kSortThreads) void k_sort_scatter(
    const K* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, int64_t n, int shift,
    const uint32_t* __restrict__ hist, int64_t ntiles, K* __restrict__ keys_out,
    uint32_t* __restrict__ vals_out, uint32_t* __restrict__ totals) {
  constexpr int D = 1 << DB, DPT = D / kSortThreads;
  constexpr int kWaves = kSortThreads / 64;
  // The totals were consumed by k_sort_scan_rows; clear them for the next pass.
  if (blockIdx.x == 0)
#pragma unroll
    for (int k = 0; k < kMaxDigits / kSortThreads; ++k)
      totals[threadIdx.x * (kMaxDigits / kSortThreads) + k] = 0;
  __shared__ uint32_t running[D];
  __shared__ uint32_t wcnt[kWaves][D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int k = 0; k < DPT; ++k)
    running[tid * DPT + k] = hist[static_cast<int64_t>(tid * DPT + k) * ntiles + blockIdx.x];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortTile;
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  for (int k = 0; k < kSortItems; ++k) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int j = 0; j < DPT; ++j) wcnt[w][tid * DPT + j] = 0;
    __syncthreads();
    const int64_t e = base + k * kSortThreads + tid;
    const bool valid = e < n;
    const K key = valid ? keys_in[e] : K(0);
    const uint32_t d = static_cast<uint32_t>(key >> shift) & (D - 1);
    // Lanes of this wave holding the same digit: intersect the ballots of every digit bit.
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const bool bit = (d >> b) & 1u;
      const unsigned long long bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
    const uint32_t rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wcnt[wave][d] = __popcll(peers);
    __syncthreads();
    if (valid) {
      uint32_t pos = running[d] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][d];
      keys_out[pos] = key;
      vals_out[pos] = vals_in[e];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
      uint32_t add = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) add += wcnt[w][tid * DPT + j];
      running[tid * DPT + j] += add;
    }
    __syncthreads();
  }
}


// Runs the passes over bits [0, bits) of the keys in buffer a, DB bits at a time (totals must
// be zero on entry; every pass leaves them zero).  Returns which buffer (0: a, 1: b) holds the
// sorted pairs.
template <typename K, int DB = 8>
inline int radix_sort_pairs(char* ws, const SortLayout<K>& L, int64_t n, int bits, hipStream_t s) {
  K* keys[2] = {reinterpret_cast<K*>(ws + L.off_keys_a), reinterpret_cast<K*>(ws + L.off_keys_b)};
  uint32_t* vals[2] = {reinterpret_cast<uint32_t*>(ws + L.off_vals_a),
                       reinterpret_cast<uint32_t*>(ws + L.off_vals_b)};
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + L.off_hist);
  uint32_t* totals = reinterpret_cast<uint32_t*>(ws + L.off_totals);
  int cur = 0;
  for (int shift = 0; shift < bits; shift += DB) {
    k_sort_hist<K, DB><<<static_cast<unsigned>(L.ntiles), kSortThreads, 0, s>>>(
        keys[cur], n, shift, hist, L.ntiles, totals);
    k_sort_scan_rows<DB><<<1 << DB, kSortThreads, 0, s>>>(hist, L.ntiles, totals);
    k_sort_scatter<K, DB><<<static_cast<unsigned>(L.ntiles), kSortThreads, 0, s>>>(
        keys[cur], vals[cur], n, shift, hist, L.ntiles, keys[cur ^ 1], vals[cur ^ 1], totals);
    cur ^= 1;
  }
  return cur;
}

}  // namespace
}  // namespace ssc
