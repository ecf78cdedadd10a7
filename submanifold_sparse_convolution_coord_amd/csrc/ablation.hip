// Building blocks of the pages' own convolution designs, kept to measure the compacted
// kernel against them on this GPU (the matrix products in between are plain library GEMMs):
//
//   dense 27-tap GEMM   every site's 27 neighbour rows side by side, zeros where a
//                       neighbour is missing, times the [27 * Cin, Cout] weights (LATO.2 MLX
//                       port page, "Fleet benchmark" version history: one dense matmul).
//   per-offset          for each tap: gather the rows that have that neighbour, multiply by
//                       W[t], scatter-add into the outputs (trellis-mac article, gather-scatter
//                       flowchart; LATO.2 page: the per-offset loop).
//
// ssc_gather_taps builds the dense operand; ssc_scatter_add_rows is the per-offset scatter
// (the per-offset gather is ssc_upsample2: out[p] = src[idx[p]]).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"

namespace ssc {
namespace {

// out[i][t][w] = X[nbr[i][t]][w] (16-byte words), zero where nbr[i][t] < 0.  Thread per
// output word; a row's 27 * words words are contiguous, so stores are whole lines.
__global__ __launch_bounds__(256) void k_gather_taps(const uint4* __restrict__ x,
                                                     const int32_t* __restrict__ nbr, int64_t n,
                                                     int words, uint4* __restrict__ out) {
  const int64_t per_row = static_cast<int64_t>(kTaps) * words;
  const int64_t total = n * per_row;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += stride) {
    const int64_t i = g / per_row;
    const int rem = static_cast<int>(g - i * per_row);
    const int t = rem / words, w = rem - t * words;
    const int32_t j = nbr[i * kTaps + t];
    out[g] = j >= 0 && j < n ? x[static_cast<int64_t>(j) * words + w] : make_uint4(0u, 0u, 0u, 0u);
  }
}

__device__ __forceinline__ float4 quad_f32(const float4* p, int64_t g) { return p[g]; }
__device__ __forceinline__ float4 quad_f32(const uint2* p, int64_t g) {
  const uint2 h = p[g];
  return make_float4(__uint_as_float(h.x << 16), __uint_as_float(h.x & 0xffff0000u),
                     __uint_as_float(h.y << 16), __uint_as_float(h.y & 0xffff0000u));
}

// y[idx[p]][c] += part[p][c] for 4 columns per thread (part fp32 or bf16, y fp32).  Within
// one call every idx is distinct (one tap's output rows), so no two threads touch the same
// element.
template <typename Q>
__global__ __launch_bounds__(256) void k_scatter_add(const Q* __restrict__ part,
                                                     const int32_t* __restrict__ idx, int64_t p,
                                                     int64_t n, int quads,
                                                     float4* __restrict__ y) {
  const int64_t total = p * quads;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += stride) {
    const int64_t r = g / quads;
    const int q = static_cast<int>(g - r * quads);
    const int32_t i = idx[r];
    if (i < 0 || i >= n) continue;
    const float4 a = quad_f32(part, g);
    float4* d = y + static_cast<int64_t>(i) * quads + q;
    float4 v = *d;
    v.x += a.x;
    v.y += a.y;
    v.z += a.z;
    v.w += a.w;
    *d = v;
  }
}

unsigned grid_for(int64_t items) {
  return static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>((items + 255) / 256, 262144)));
}

}  // namespace
}  // namespace ssc

using namespace ssc;

extern "C" ssc_status ssc_gather_taps(const void* feats, int32_t dtype, int64_t n,
                                      int32_t channels, const int32_t* nbr, void* out,
                                      void* stream) {
  if (n < 0 || channels < 1 || (dtype != SSC_F32 && dtype != SSC_BF16 && dtype != SSC_F16))
    return SSC_ERR_ARG;
  const int64_t row_bytes = static_cast<int64_t>(channels) * (dtype == SSC_F32 ? 4 : 2);
  if (row_bytes % 16 != 0) return SSC_ERR_UNSUPPORTED;
  if (n == 0) return SSC_OK;
  if (feats == nullptr || nbr == nullptr || out == nullptr || !aligned(feats, 16) ||
      !aligned(out, 16))
    return SSC_ERR_ARG;
  const int words = static_cast<int>(row_bytes / 16);
  k_gather_taps<<<grid_for(n * kTaps * words), 256, 0, as_stream(stream)>>>(
      static_cast<const uint4*>(feats), nbr, n, words, static_cast<uint4*>(out));
  return launch_status();
}

extern "C" ssc_status ssc_scatter_add_rows(const void* part, int32_t part_dtype,
                                           const int32_t* idx, int64_t p, int32_t channels,
                                           float* out, int64_t n, void* stream) {
  if (p < 0 || n < 0 || channels < 1 || channels % 4 != 0) return SSC_ERR_ARG;
  if (part_dtype != SSC_F32 && part_dtype != SSC_BF16) return SSC_ERR_ARG;
  if (p == 0) return SSC_OK;
  if (part == nullptr || idx == nullptr || out == nullptr || !aligned(part, 16) ||
      !aligned(out, 16))
    return SSC_ERR_ARG;
  const unsigned g = grid_for(p * (channels / 4));
  auto* y = reinterpret_cast<float4*>(out);
  if (part_dtype == SSC_F32)
    k_scatter_add<float4><<<g, 256, 0, as_stream(stream)>>>(
        static_cast<const float4*>(part), idx, p, n, channels / 4, y);
  else
    k_scatter_add<uint2><<<g, 256, 0, as_stream(stream)>>>(
        static_cast<const uint2*>(part), idx, p, n, channels / 4, y);
  return launch_status();
}
