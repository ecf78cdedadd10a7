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
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
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

__global__ void k_plan_header(int64_t* __restrict__ header, int64_t n, int64_t npad,
                              int64_t nblocks, uint4* __restrict__ zero) {
  if (threadIdx.x == 0) {
    header[0] = kPlanMagic;
    header[1] = n;
    header[2] = npad;
    header[3] = nblocks;
  }
  for (int i = threadIdx.x; i < static_cast<int>(kZeroBytes / sizeof(uint4)); i += blockDim.x)
    zero[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ------------------------------------------------------------------------------------------
// Plan: stable LSD radix sort of (mask, row) pairs, then the tap-major neighbour rows.
// ------------------------------------------------------------------------------------------
constexpr int kKeyBits = 26;                     // the plan's sort key (Gray rank of the mask)
// The plan's sort scratch is one 32-bit-key sort of n pairs.
inline SortLayout<uint32_t> plan_work_layout(int64_t n) { return sort_layout<uint32_t>(n, 0); }

// Sort key of a site: bit (t < 13 ? t : t - 1) set when non-centre tap t has a neighbour.
__global__ void k_mask_keys(const int32_t* __restrict__ nbr, int64_t n, uint32_t* __restrict__ keys,
                            uint32_t* __restrict__ vals, uint32_t* __restrict__ totals) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0 && threadIdx.x < kDigits) totals[threadIdx.x] = 0;
  if (i >= n) return;
  const int32_t* row = nbr + i * kTaps;
  uint32_t m = 0;
#pragma unroll
  for (int t = 0; t < kTaps; ++t) {
    if (t == kCentreTap) continue;
    if (row[t] >= 0) m |= 1u << (t < kCentreTap ? t : t - 1);
  }
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

// perm, per-block tap masks and tap-major neighbour rows in sorted order.  A workgroup owns
// 256 sorted positions: it reads their 256 map rows cooperatively (consecutive lanes read
// consecutive entries of a row, so a wave touches a few 108-byte rows instead of 64 scattered
// words), stages them in LDS, then writes each tap's 256 entries as one coalesced run.  Each
// 16-lane group of a wave is one block for the tap masks.
__global__ __launch_bounds__(256) void k_plan_fill(const int32_t* __restrict__ nbr, int64_t n,
                                                   const uint32_t* __restrict__ sorted_rows,
                                                   int64_t npad, int32_t* __restrict__ perm,
                                                   uint32_t* __restrict__ bmask,
                                                   int32_t* __restrict__ gidx) {
  __shared__ int32_t rows[256 * kTaps];  // row-major [position][tap]; stride 27 is odd, so a
                                         // wave's column reads hit distinct banks
  __shared__ int32_t src[256];
  const int tid = threadIdx.x;
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 256;
  const int64_t r = r0 + tid;  // < npad
  const int32_t i = r < n ? static_cast<int32_t>(sorted_rows[r]) : -1;
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

extern "C" ssc_status ssc_build_index(const int32_t* coords, int64_t n, int32_t batch,
                                      const int32_t* grid, int32_t* nbr, void* workspace,
                                      size_t workspace_bytes, int32_t check, void* stream) {
  if (n < 0 || grid == nullptr) return SSC_ERR_ARG;
  if (n > 0 && (coords == nullptr || nbr == nullptr || workspace == nullptr)) return SSC_ERR_ARG;
  if (batch < 1 || batch > kMaxCoord) return SSC_ERR_UNSUPPORTED;
  for (int a = 0; a < 3; ++a)
    if (grid[a] < 1 || grid[a] > kMaxCoord) return SSC_ERR_UNSUPPORTED;
  if (n * kTaps > (int64_t(1) << 40) || n >= (int64_t(1) << 31)) return SSC_ERR_UNSUPPORTED;
  if (n == 0) return SSC_OK;
  if (!aligned(coords, 16) || !aligned(workspace, kAlign) || !aligned(nbr, 4)) return SSC_ERR_ARG;
  const IndexLayout L = index_layout(n);
  if (workspace_bytes < L.total) return SSC_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws);
  auto* slots = reinterpret_cast<Slot*>(ws + L.off_slots);
  const int bs = 256;
  const uint64_t init_blocks = std::min<uint64_t>((L.cap + bs - 1) / bs, 8192);
  k_table_init<<<static_cast<unsigned>(init_blocks), bs, 0, s>>>(slots, L.cap, counters);
  const unsigned ins_blocks = static_cast<unsigned>(std::min<int64_t>((n + bs - 1) / bs, 65536));
  k_insert<<<ins_blocks, bs, 0, s>>>(
      reinterpret_cast<const int4*>(coords), n, batch, grid[0], grid[1], grid[2], slots,
      L.cap - 1, counters);
  const int64_t q = n * kTaps;
  const unsigned q_blocks = static_cast<unsigned>(std::min<int64_t>((q + bs - 1) / bs, 262144));
  k_query<<<q_blocks, bs, 0, s>>>(
      reinterpret_cast<const int4*>(coords), n, batch, grid[0], grid[1], grid[2], slots,
      L.cap - 1, nbr);
  if (launch_status() != SSC_OK) return SSC_ERR_HIP;
  if (check) {
    uint32_t host[2] = {0, 0};
    if (hipMemcpyAsync(host, counters, sizeof(host), hipMemcpyDeviceToHost, s) != hipSuccess)
      return SSC_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SSC_ERR_HIP;
    if (host[0]) return SSC_ERR_COORD_RANGE;
    if (host[1]) return SSC_ERR_DUPLICATE;
  }
  return SSC_OK;
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

extern "C" ssc_status ssc_build_plan(const int32_t* nbr, int64_t n, void* plan, size_t plan_bytes,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (n < 0 || plan == nullptr || workspace == nullptr) return SSC_ERR_ARG;
  if (n > 0 && nbr == nullptr) return SSC_ERR_ARG;
  if (n >= (int64_t(1) << 31)) return SSC_ERR_UNSUPPORTED;
  if (!aligned(plan, kAlign) || !aligned(workspace, kAlign)) return SSC_ERR_ARG;
  const PlanLayout P = plan_layout(n);
  const SortLayout<uint32_t> W = plan_work_layout(n);
  if (plan_bytes < P.total || workspace_bytes < W.total) return SSC_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  char* pb = static_cast<char*>(plan);
  char* ws = static_cast<char*>(workspace);
  k_plan_header<<<1, 64, 0, s>>>(reinterpret_cast<int64_t*>(pb), n, P.npad, P.nblocks,
                                 reinterpret_cast<uint4*>(pb + P.off_zero));
  uint32_t* sorted_rows = reinterpret_cast<uint32_t*>(ws + W.off_vals_a);
  if (n > 0) {
    k_mask_keys<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
        nbr, n, reinterpret_cast<uint32_t*>(ws + W.off_keys_a), sorted_rows,
        reinterpret_cast<uint32_t*>(ws + W.off_totals));
    if (radix_sort_pairs<uint32_t>(ws, W, n, kKeyBits, s) == 1)
      sorted_rows = reinterpret_cast<uint32_t*>(ws + W.off_vals_b);
  }
  k_plan_fill<<<static_cast<unsigned>(P.npad / 256), 256, 0, s>>>(
      nbr, n, sorted_rows, P.npad, reinterpret_cast<int32_t*>(pb + P.off_perm),
      reinterpret_cast<uint32_t*>(pb + P.off_bmask), reinterpret_cast<int32_t*>(pb + P.off_gidx));
  return launch_status();
}
