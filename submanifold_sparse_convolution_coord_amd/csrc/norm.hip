// Sparse group norm (SparseGroupNorm32) for the blocks around the convolution: statistics per
// batch entry and channel group over the active sites, in three steps that are each one
// launch and bit-reproducible (fixed summation orders, no atomics):
//
//   partials  per slot of 128 rows: count, sum and sum of squares (fp32) of every
//             (batch entry, group); the k=3 convolution can write the same slots itself
//             from its epilogue (sums over its own 128- or 256-row tiles) for batch 1.
//   finalize  per (entry, group): the slots summed in fp64 in slot order, then mean and
//             1 / sqrt(var + eps) with the population variance.
//   apply     y = act((x - mean) * rstd * gamma + beta), one pass, in place allowed.
//
// The pages name the module (LATO.2 MLX port page, "Status": SparseGroupNorm32 among the
// remaining sparse ops) and say what the "32" of their norms means (fp32 accumulation, the
// same page's repository layout for LayerNorm32); the rest is the textbook group norm
// restricted to the active sites.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "common.h"

namespace ssc {
namespace {

constexpr int kSlotRows = 128;       // rows per partial-sum slot
constexpr int kPassBatch = 4;        // batch entries one partials pass accumulates

__device__ __forceinline__ float ld_val(const float* p) { return *p; }
__device__ __forceinline__ float ld_val(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float ld_val(const _Float16* p) { return static_cast<float>(*p); }

__device__ __forceinline__ void st_val(float* p, float v) { *p = v; }
__device__ __forceinline__ void st_val(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }
__device__ __forceinline__ void st_val(_Float16* p, float v) { *p = static_cast<_Float16>(v); }

// Partial sums of one slot (blockIdx.x) for batch entries [4 * blockIdx.y, + 4).  Thread
// (g, rl) = (t % groups, t / groups) walks rows rl, rl + RL, ... of the slot and the gs
// channels of group g; then one thread per (group, entry) adds the RL row lanes in order.
template <typename T>
__global__ __launch_bounds__(256) void k_gn_partials(const T* __restrict__ x, int64_t n,
                                                     int channels, int groups,
                                                     const int4* __restrict__ coords,
                                                     int batch, float4* __restrict__ partials) {
  __shared__ float red[256 * 3 * kPassBatch];
  const int t = threadIdx.x;
  const int64_t slot = blockIdx.x;
  const int base = blockIdx.y * kPassBatch;
  const int gs = channels / groups;
  const int lanes = 256 / groups;                 // row lanes (groups <= 256)
  const int g = t % groups, rl = t / groups;
  float s[kPassBatch], q[kPassBatch], c[kPassBatch];
#pragma unroll
  for (int k = 0; k < kPassBatch; ++k) s[k] = q[k] = c[k] = 0.f;
  if (rl < lanes) {
    for (int r = rl; r < kSlotRows; r += lanes) {
      const int64_t row = slot * kSlotRows + r;
      if (row >= n) break;
      const int k = (coords ? coords[row].x : 0) - base;
      if (k < 0 || k >= kPassBatch) continue;
      const T* p = x + row * channels + static_cast<int64_t>(g) * gs;
      float rs = 0.f, rq = 0.f;
      for (int j = 0; j < gs; ++j) {
        const float v = ld_val(p + j);
        rs += v;
        rq = fmaf(v, v, rq);
      }
#pragma unroll
      for (int kk = 0; kk < kPassBatch; ++kk)
        if (kk == k) {
          s[kk] += rs;
          q[kk] += rq;
          c[kk] += 1.f;
        }
    }
  }
#pragma unroll
  for (int k = 0; k < kPassBatch; ++k) {
    red[(k * 3 + 0) * 256 + t] = s[k];
    red[(k * 3 + 1) * 256 + t] = q[k];
    red[(k * 3 + 2) * 256 + t] = c[k];
  }
  __syncthreads();
  for (int pair = t; pair < groups * kPassBatch; pair += 256) {
    const int gg = pair % groups, k = pair / groups;
    if (base + k >= batch) continue;
    float S = 0.f, Q = 0.f, C = 0.f;
    for (int l = 0; l < lanes; ++l) {
      const int src = l * groups + gg;
      S += red[(k * 3 + 0) * 256 + src];
      Q += red[(k * 3 + 1) * 256 + src];
      C += red[(k * 3 + 2) * 256 + src];
    }
    partials[(slot * batch + base + k) * groups + gg] = make_float4(C * gs, S, Q, 0.f);
  }
}

// Block per (entry, group): thread t adds slots t, t + 256, ... in fp64, then a fixed tree.
__global__ __launch_bounds__(256) void k_gn_finalize(const float4* __restrict__ partials,
                                                     int64_t slots, int batch_groups, float eps,
                                                     float2* __restrict__ stats) {
  __shared__ double red[3][256];
  const int t = threadIdx.x;
  const int bg = blockIdx.x;
  double c = 0.0, s = 0.0, q = 0.0;
  for (int64_t i = t; i < slots; i += 256) {
    const float4 p = partials[i * batch_groups + bg];
    c += p.x;
    s += p.y;
    q += p.z;
  }
  red[0][t] = c;
  red[1][t] = s;
  red[2][t] = q;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
      red[0][t] += red[0][t + w];
      red[1][t] += red[1][t + w];
      red[2][t] += red[2][t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    const double cnt = red[0][0];
    const double mean = cnt > 0.0 ? red[1][0] / cnt : 0.0;
    const double var = cnt > 0.0 ? std::max(red[2][0] / cnt - mean * mean, 0.0) : 0.0;
    stats[bg] = make_float2(static_cast<float>(mean),
                            static_cast<float>(1.0 / std::sqrt(var + static_cast<double>(eps))));
  }
}

// Thread per (row, E consecutive channels); E = 16 bytes of elements when rows allow, else 1.
template <typename T, int E>
__global__ __launch_bounds__(256) void k_gn_apply(const T* __restrict__ x, int64_t n,
                                                  int channels, int groups,
                                                  const int4* __restrict__ coords, int batch,
                                                  const float2* __restrict__ stats,
                                                  const float* __restrict__ gamma,
                                                  const float* __restrict__ beta, int act,
                                                  T* __restrict__ out) {
  const int words = channels / E;
  const int gs = channels / groups;
  const int64_t total = n * words;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += stride) {
    const int64_t row = i / words;
    const int c0 = static_cast<int>(i - row * words) * E;
    // batch ids outside [0, batch) are invalid input; clamped so the read stays in bounds
    const int b = coords ? min(max(coords[row].x, 0), batch - 1) : 0;
    const float2* st = stats + static_cast<int64_t>(b) * groups;
    alignas(16) T v[E];
    if constexpr (E * sizeof(T) == 16)
      *reinterpret_cast<uint4*>(v) = *reinterpret_cast<const uint4*>(x + row * channels + c0);
    else
#pragma unroll
      for (int e = 0; e < E; ++e) v[e] = x[row * channels + c0 + e];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int c = c0 + e;
      const float2 m = st[c / gs];
      float y = (ld_val(&v[e]) - m.x) * m.y;
      if (gamma) y *= gamma[c];
      if (beta) y += beta[c];
      st_val(&v[e], apply_act(y, act));
    }
    if constexpr (E * sizeof(T) == 16)
      *reinterpret_cast<uint4*>(out + row * channels + c0) = *reinterpret_cast<const uint4*>(v);
    else
#pragma unroll
      for (int e = 0; e < E; ++e) out[row * channels + c0 + e] = v[e];
  }
}

int64_t gn_slots(int64_t n) {
  const int64_t rows = std::max<int64_t>(n, 1);
  return (rows + kPlanRowAlign - 1) / kPlanRowAlign * (kPlanRowAlign / kSlotRows);
}

bool gn_shape_ok(int64_t n, int32_t dtype, int32_t channels, int32_t batch, int32_t groups) {
  return n >= 0 && n < (int64_t(1) << 31) &&
         (dtype == SSC_F32 || dtype == SSC_BF16 || dtype == SSC_F16) && groups >= 1 &&
         groups <= 256 && channels >= 1 && channels % groups == 0 && batch >= 1 &&
         batch <= SSC_GN_MAX_BATCH;
}

}  // namespace

// Shared with the convolution's entry points: the standalone partial sums of an [n, C]
// tensor in the slots layout (used when the convolution cannot sum in its own epilogue).
ssc_status gn_partials_launch(const void* x, int32_t dtype, int64_t n, int32_t channels,
                              const int32_t* coords, int32_t batch, int32_t groups,
                              float* partials, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(gn_slots(n)),
                  static_cast<unsigned>((batch + kPassBatch - 1) / kPassBatch));
  const int4* c4 = batch > 1 ? reinterpret_cast<const int4*>(coords) : nullptr;
  auto* p4 = reinterpret_cast<float4*>(partials);
  if (dtype == SSC_F32)
    k_gn_partials<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), n, channels, groups,
                                              c4, batch, p4);
  else if (dtype == SSC_BF16)
    k_gn_partials<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), n, channels,
                                                 groups, c4, batch, p4);
  else
    k_gn_partials<_Float16><<<grid, 256, 0, s>>>(static_cast<const _Float16*>(x), n, channels,
                                                 groups, c4, batch, p4);
  return launch_status();
}

}  // namespace ssc

using namespace ssc;

extern "C" size_t ssc_gn_partials_bytes(int64_t n, int32_t batch, int32_t groups) {
  if (n < 0 || batch < 1 || batch > SSC_GN_MAX_BATCH || groups < 1 || groups > 256) return 0;
  return align_up(static_cast<size_t>(gn_slots(n)) * batch * groups * sizeof(float4));
}

extern "C" ssc_status ssc_gn_partials(const void* x, int32_t dtype, int64_t n, int32_t channels,
                                      const int32_t* coords, int32_t batch, int32_t groups,
                                      float* partials, size_t partials_bytes, void* stream) {
  if (!gn_shape_ok(n, dtype, channels, batch, groups) || partials == nullptr) return SSC_ERR_ARG;
  if (n > 0 && (x == nullptr || (batch > 1 && coords == nullptr))) return SSC_ERR_ARG;
  if (!aligned(partials, 16) || (coords && !aligned(coords, 16))) return SSC_ERR_ARG;
  if (partials_bytes < ssc_gn_partials_bytes(n, batch, groups)) return SSC_ERR_WORKSPACE;
  return gn_partials_launch(x, dtype, n, channels, coords, batch, groups, partials,
                            as_stream(stream));
}

extern "C" ssc_status ssc_gn_finalize(const float* partials, int64_t n, int32_t batch,
                                      int32_t groups, float eps, float* stats, void* stream) {
  if (n < 0 || batch < 1 || batch > SSC_GN_MAX_BATCH || groups < 1 || groups > 256 ||
      partials == nullptr || stats == nullptr || !(eps >= 0.f))
    return SSC_ERR_ARG;
  if (!aligned(partials, 16) || !aligned(stats, 8)) return SSC_ERR_ARG;
  k_gn_finalize<<<static_cast<unsigned>(batch * groups), 256, 0, as_stream(stream)>>>(
      reinterpret_cast<const float4*>(partials), gn_slots(n), batch * groups, eps,
      reinterpret_cast<float2*>(stats));
  return launch_status();
}

extern "C" ssc_status ssc_gn_apply(const void* x, int32_t dtype, int64_t n, int32_t channels,
                                   const int32_t* coords, int32_t batch, int32_t groups,
                                   const float* stats, const float* gamma, const float* beta,
                                   int32_t act, void* out, void* stream) {
  if (!gn_shape_ok(n, dtype, channels, batch, groups) || stats == nullptr) return SSC_ERR_ARG;
  if (act < SSC_ACT_NONE || act > SSC_ACT_SILU) return SSC_ERR_ARG;
  if (n == 0) return SSC_OK;
  if (x == nullptr || out == nullptr || (batch > 1 && coords == nullptr)) return SSC_ERR_ARG;
  if (!aligned(stats, 8) || (coords && !aligned(coords, 16)) || (gamma && !aligned(gamma, 4)) ||
      (beta && !aligned(beta, 4)))
    return SSC_ERR_ARG;
  const int esz = dtype == SSC_F32 ? 4 : 2;
  const bool vec = (static_cast<int64_t>(channels) * esz) % 16 == 0 && aligned(x, 16) &&
                   aligned(out, 16);
  const int E = vec ? 16 / esz : 1;
  const int64_t items = n * (channels / E);
  const unsigned grid =
      static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>((items + 255) / 256, 262144)));
  hipStream_t s = as_stream(stream);
  const int4* c4 = batch > 1 ? reinterpret_cast<const int4*>(coords) : nullptr;
  const auto* st = reinterpret_cast<const float2*>(stats);
  if (dtype == SSC_F32) {
    auto* xi = static_cast<const float*>(x);
    auto* xo = static_cast<float*>(out);
    if (vec)
      k_gn_apply<float, 4><<<grid, 256, 0, s>>>(xi, n, channels, groups, c4, batch, st, gamma, beta, act, xo);
    else
      k_gn_apply<float, 1><<<grid, 256, 0, s>>>(xi, n, channels, groups, c4, batch, st, gamma, beta, act, xo);
  } else if (dtype == SSC_BF16) {
    auto* xi = static_cast<const uint16_t*>(x);
    auto* xo = static_cast<uint16_t*>(out);
    if (vec)
      k_gn_apply<uint16_t, 8><<<grid, 256, 0, s>>>(xi, n, channels, groups, c4, batch, st, gamma, beta, act, xo);
    else
      k_gn_apply<uint16_t, 1><<<grid, 256, 0, s>>>(xi, n, channels, groups, c4, batch, st, gamma, beta, act, xo);
  } else {
    auto* xi = static_cast<const _Float16*>(x);
    auto* xo = static_cast<_Float16*>(out);
    if (vec)
      k_gn_apply<_Float16, 8><<<grid, 256, 0, s>>>(xi, n, channels, groups, c4, batch, st, gamma, beta, act, xo);
    else
      k_gn_apply<_Float16, 1><<<grid, 256, 0, s>>>(xi, n, channels, groups, c4, batch, st, gamma, beta, act, xo);
  }
  return launch_status();
}
