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
// Rows each apply thread handles per step of its stride.  Two: with 8 the 128-channel apply of
// 209K bf16 rows took 26.4 us, with 2 24.2 us (64 channels, 268K rows: 20.0 -> 15.9 us; 32
// channels, 1.2M rows: 32.7 -> 27.7 us); 16 rows, or a grid without the 1024-workgroup cap,
// were slower still.
constexpr int kApplyRows = 2;

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

// Values of one 16-byte word as floats.
template <typename T>
__device__ __forceinline__ void word_to_f32(const uint4& w, float* f) {
  if constexpr (sizeof(T) == 4) {
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
  } else {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t h = static_cast<uint16_t>(d[i >> 1] >> (16 * (i & 1)));
      f[i] = ld_val(reinterpret_cast<const T*>(&h));
    }
  }
}

// Partial sums with rows of whole 16-byte words (E values each).  Thread (w, rl) = (t %
// words, t / words) owns word w (channels E*w ...) and rows rl, rl + lanes, ... of the slot,
// all loaded before any is summed; per-channel sums for 4 batch entries per pass, then, one
// entry at a time, a fixed-order sum over the row lanes and over each group's channels.
// A block covers spb slots, spb = max(4, 16 / words), so that every thread has at least 8 rows
// and a block's reduction is paid once per 512 rows or more (max(1, 16 / words) took 21.3
// against 20.1 us at 128 bf16 channels and 209K rows, 16.3 against 13.6 us at 64 channels and
// 268K rows).  It writes their sum into the first of them and zeros into the rest: finalize
// adds all.
template <typename T>
__global__ __launch_bounds__(256) void k_gn_partials_w(const uint4* __restrict__ x, int64_t n,
                                                       int channels, int groups,
                                                       const int4* __restrict__ coords,
                                                       int batch, int64_t slots,
                                                       float4* __restrict__ partials) {
  constexpr int E = 16 / sizeof(T);
  __shared__ float red[256 * (2 * E + 1)];
  __shared__ float tot[2 * 1024 + 1];
  const int t = threadIdx.x;
  const int base = blockIdx.y * kPassBatch;
  const int words = channels / E;
  const int lanes = 256 / words;
  const int spb = 16 / words > 4 ? 16 / words : 4;
  const int64_t slot = static_cast<int64_t>(blockIdx.x) * spb;
  const int MAXR = spb * kSlotRows;            // rows of this block
  const int w = t % words, rl = t / words;
  const bool active = rl < lanes;
  float s[kPassBatch][E], q[kPassBatch][E], cnt[kPassBatch];
#pragma unroll
  for (int k = 0; k < kPassBatch; ++k) {
    cnt[k] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) s[k][e] = q[k][e] = 0.f;
  }
  if (active) {
    for (int r0 = rl; r0 < MAXR; r0 += 4 * lanes) {
      uint4 v[4];
      int kk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // issue up to 4 rows' loads, then sum them
        const int r = r0 + u * lanes;
        const int64_t row = slot * kSlotRows + r;
        const bool ok = r < MAXR && row < n;
        kk[u] = ok ? (coords ? coords[row].x : 0) - base : -1;
        v[u] = ok ? x[row * words + w] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float f[E];
        word_to_f32<T>(v[u], f);
#pragma unroll
        for (int k = 0; k < kPassBatch; ++k)
          if (kk[u] == k) {
            cnt[k] += 1.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
              s[k][e] += f[e];
              q[k][e] = fmaf(f[e], f[e], q[k][e]);
            }
          }
      }
    }
  }
  const int gs = channels / groups;
  // Rows of a power-of-two number of words (at most 64) put every word's lanes of a wave at a
  // fixed stride: a butterfly over them sums the wave's rows in registers, and only the 4 waves'
  // sums go through LDS (one thread per channel adding up 64 row lanes from LDS took 37.9 us
  // for 1.2M rows of 32 bf16 channels).
  const bool butterfly = (words & (words - 1)) == 0 && words <= 64;
  const int wave = t >> 6, lane = t & 63;
  for (int k = 0; k < kPassBatch && base + k < batch; ++k) {
    __syncthreads();  // red / tot of the previous entry are consumed
    if (butterfly) {
      float sk[E], qk[E], ck = cnt[k];
#pragma unroll
      for (int e = 0; e < E; ++e) sk[e] = s[k][e], qk[e] = q[k][e];
      for (int off = words; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          sk[e] += __shfl_xor(sk[e], off, 64);
          qk[e] += __shfl_xor(qk[e], off, 64);
        }
        ck += __shfl_xor(ck, off, 64);
      }
      if (lane < words) {  // lane = w: the wave's sums of word w
#pragma unroll
        for (int e = 0; e < E; ++e) {
          red[((2 * e) * 4 + wave) * words + lane] = sk[e];
          red[((2 * e + 1) * 4 + wave) * words + lane] = qk[e];
        }
        if (lane == 0) red[(2 * E) * 4 * words + wave] = ck;
      }
      __syncthreads();
      for (int c = t; c < channels; c += 256) {  // channel c = word c / E, element c % E
        const int ww = c / E, e = c % E;
        float S = 0.f, Q = 0.f;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) {
          S += red[((2 * e) * 4 + wv) * words + ww];
          Q += red[((2 * e + 1) * 4 + wv) * words + ww];
        }
        tot[2 * c] = S;
        tot[2 * c + 1] = Q;
      }
      if (t == 0) {
        float C = 0.f;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) C += red[(2 * E) * 4 * words + wv];
        tot[2 * channels] = C;
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        red[(2 * e) * 256 + t] = s[k][e];
        red[(2 * e + 1) * 256 + t] = q[k][e];
      }
      red[(2 * E) * 256 + t] = cnt[k];
      __syncthreads();
      for (int c = t; c < channels; c += 256) {  // channel c = word c / E, element c % E
        const int ww = c / E, e = c % E;
        float S = 0.f, Q = 0.f;
        for (int l = 0; l < lanes; ++l) {
          S += red[(2 * e) * 256 + l * words + ww];
          Q += red[(2 * e + 1) * 256 + l * words + ww];
        }
        tot[2 * c] = S;
        tot[2 * c + 1] = Q;
      }
      if (t == 0) {
        float C = 0.f;
        for (int l = 0; l < lanes; ++l) C += red[(2 * E) * 256 + l * words];
        tot[2 * channels] = C;
      }
    }
    __syncthreads();
    for (int g = t; g < groups; g += 256) {
      float S = 0.f, Q = 0.f;
      for (int j = 0; j < gs; ++j) {
        S += tot[2 * (g * gs + j)];
        Q += tot[2 * (g * gs + j) + 1];
      }
      partials[(slot * batch + base + k) * groups + g] =
          make_float4(tot[2 * channels] * gs, S, Q, 0.f);
      for (int j = 1; j < spb && slot + j < slots; ++j)
        partials[((slot + j) * batch + base + k) * groups + g] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
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
__global__ __launch_bounds__(256) void k_gn_apply(const T* x, int64_t n,
                                                  int channels, int groups,
                                                  const int4* __restrict__ coords, int batch,
                                                  const float2* __restrict__ stats,
                                                  const float* __restrict__ gamma,
                                                  const float* __restrict__ beta, int act,
                                                  T* out) {
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

// Apply with rows of whole 16-byte words: thread (w, rl) owns word w and 8 rows (rl + u *
// lanes of its block's 8 * lanes); per channel y = x * a + sh with a = rstd * gamma and
// sh = beta - mean * a, computed once per thread for batch 1 and per row otherwise.
template <typename T>
// x and out may be the same buffer (no __restrict__ on either).
__global__ __launch_bounds__(256) void k_gn_apply_w(const uint4* x, int64_t n,
                                                    int channels, int groups,
                                                    const int4* __restrict__ coords, int batch,
                                                    const float2* __restrict__ stats,
                                                    const float* __restrict__ gamma,
                                                    const float* __restrict__ beta, int act,
                                                    uint4* out) {
  constexpr int E = 16 / sizeof(T);
  const int words = channels / E;
  const int lanes = 256 / words;
  const int w = threadIdx.x % words, rl = threadIdx.x / words;
  if (rl >= lanes) return;
  const int gs = channels / groups;
  float gm[E], bt[E], a[E], sh[E];
  int grp[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = w * E + e;
    gm[e] = gamma ? gamma[c] : 1.f;
    bt[e] = beta ? beta[c] : 0.f;
    grp[e] = c / gs;
  }
  auto coeffs = [&](int b) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float2 m = stats[static_cast<int64_t>(b) * groups + grp[e]];
      a[e] = m.y * gm[e];
      sh[e] = fmaf(-m.x, a[e], bt[e]);
    }
  };
  if (!coords) coeffs(0);
  const int64_t step = static_cast<int64_t>(gridDim.x) * kApplyRows * lanes;
  for (int64_t r0 = static_cast<int64_t>(blockIdx.x) * kApplyRows * lanes + rl; r0 < n;
       r0 += step) {
    uint4 v[kApplyRows];
#pragma unroll
    for (int u = 0; u < kApplyRows; ++u) {
      const int64_t row = r0 + u * lanes;
      if (row < n) v[u] = x[row * words + w];
    }
#pragma unroll
    for (int u = 0; u < kApplyRows; ++u) {
      const int64_t row = r0 + u * lanes;
      if (row >= n) break;
      // batch ids outside [0, batch) are invalid input; clamped so the read stays in bounds
      if (coords) coeffs(min(max(coords[row].x, 0), batch - 1));
      float f[E];
      word_to_f32<T>(v[u], f);
      alignas(16) T o[E];
#pragma unroll
      for (int e = 0; e < E; ++e) st_val(&o[e], apply_act(fmaf(f[e], a[e], sh[e]), act));
      out[row * words + w] = *reinterpret_cast<const uint4*>(o);
    }
  }
}

// Layer norm (LayerNorm32: fp32 statistics) over each row's channels, rows of WORDS 16-byte
// words (a power of two <= 64): a row is WORDS neighbouring lanes, a wave holds 64 / WORDS
// rows per group and works on 4 groups at once (their loads in flight together); two
// butterfly sums give the mean and then the mean squared deviation (every lane of a row ends
// with the same sums); y = act((x - mean) * rstd * gamma + beta).  x and out may be the same
// buffer.
template <typename T, int WORDS>
__global__ __launch_bounds__(256) void k_layer_norm_w(const uint4* x, int64_t n, int channels,
                                                      const float* __restrict__ gamma,
                                                      const float* __restrict__ beta, float eps,
                                                      int act, uint4* out) {
  constexpr int E = 16 / sizeof(T);
  constexpr int RPW = 64 / WORDS;  // rows per group
  constexpr int G = 4;             // groups a wave keeps in flight
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int w = lane % WORDS, rsub = lane / WORDS;
  float gm[E], bt[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    gm[e] = 1.f;
    bt[e] = 0.f;
  }
  if (gamma) {
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(gamma + w * E + e);
      gm[e] = v.x, gm[e + 1] = v.y, gm[e + 2] = v.z, gm[e + 3] = v.w;
    }
  }
  if (beta) {
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(beta + w * E + e);
      bt[e] = v.x, bt[e + 1] = v.y, bt[e + 2] = v.z, bt[e + 3] = v.w;
    }
  }
  const float inv_c = 1.f / static_cast<float>(channels);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4 * G * RPW;
  for (int64_t base = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * G * RPW; base < n;
       base += stride) {  // uniform across the wave: every lane joins the shuffles
    uint4 v[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int64_t row = base + k * RPW + rsub;
      v[k] = row < n ? x[row * WORDS + w] : make_uint4(0u, 0u, 0u, 0u);
    }
    float f[G][E], sum[G], sq[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      word_to_f32<T>(v[k], f[k]);
      sum[k] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) sum[k] += f[k][e];
    }
#pragma unroll
    for (int m = 1; m < WORDS; m <<= 1)
#pragma unroll
      for (int k = 0; k < G; ++k) sum[k] += __shfl_xor(sum[k], m, 64);
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const float mean = sum[k] * inv_c;
      sq[k] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        f[k][e] -= mean;
        sq[k] = fmaf(f[k][e], f[k][e], sq[k]);
      }
    }
#pragma unroll
    for (int m = 1; m < WORDS; m <<= 1)
#pragma unroll
      for (int k = 0; k < G; ++k) sq[k] += __shfl_xor(sq[k], m, 64);
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int64_t row = base + k * RPW + rsub;
      if (row >= n) continue;
      const float rstd = 1.f / sqrtf(sq[k] * inv_c + eps);
      alignas(16) T o[E];
#pragma unroll
      for (int e = 0; e < E; ++e)
        st_val(&o[e], apply_act(fmaf(f[k][e] * rstd, gm[e], bt[e]), act));
      st16(&out[row * WORDS + w], *reinterpret_cast<const uint4*>(o));
    }
  }
}

// Layer norm for any row width: a thread per row, two passes over it.
template <typename T>
__global__ __launch_bounds__(256) void k_layer_norm_rows(const T* x, int64_t n, int channels,
                                                         const float* __restrict__ gamma,
                                                         const float* __restrict__ beta,
                                                         float eps, int act, T* out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; row < n;
       row += stride) {
    const T* p = x + row * channels;
    float sum = 0.f;
    for (int c = 0; c < channels; ++c) sum += ld_val(p + c);
    const float mean = sum / static_cast<float>(channels);
    float sq = 0.f;
    for (int c = 0; c < channels; ++c) {
      const float d = ld_val(p + c) - mean;
      sq = fmaf(d, d, sq);
    }
    const float rstd = 1.f / sqrtf(sq / static_cast<float>(channels) + eps);
    for (int c = 0; c < channels; ++c) {
      float y = (ld_val(p + c) - mean) * rstd;
      y = fmaf(y, gamma ? gamma[c] : 1.f, beta ? beta[c] : 0.f);
      st_val(out + row * channels + c, apply_act(y, act));
    }
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
  const int esz = dtype == SSC_F32 ? 4 : 2;
  const int64_t row_bytes = static_cast<int64_t>(channels) * esz;
  if (row_bytes % 16 == 0 && row_bytes / 16 <= 256 && channels <= 1024 && aligned(x, 16)) {
    const auto* x4 = static_cast<const uint4*>(x);
    const int64_t words = row_bytes / 16, slots = gn_slots(n);
    const int64_t spb = 16 / words > 4 ? 16 / words : 4;
    const dim3 gw(static_cast<unsigned>((slots + spb - 1) / spb), grid.y);
    if (dtype == SSC_F32)
      k_gn_partials_w<float><<<gw, 256, 0, s>>>(x4, n, channels, groups, c4, batch, slots, p4);
    else if (dtype == SSC_BF16)
      k_gn_partials_w<uint16_t><<<gw, 256, 0, s>>>(x4, n, channels, groups, c4, batch, slots, p4);
    else
      k_gn_partials_w<_Float16><<<gw, 256, 0, s>>>(x4, n, channels, groups, c4, batch, slots, p4);
    return launch_status();
  }
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
  hipStream_t s = as_stream(stream);
  const int4* c4 = batch > 1 ? reinterpret_cast<const int4*>(coords) : nullptr;
  const auto* st = reinterpret_cast<const float2*>(stats);
  if (vec && channels * esz / 16 <= 256) {
    const int lanes = 256 / (channels * esz / 16);
    const int64_t blocks = (n + kApplyRows * lanes - 1) / (kApplyRows * lanes);
    // At most 1024 workgroups (4 per CU), each striding over the rows, so that one
    // workgroup's stores overlap another's loads (128 channels, 209K rows: 30.6 -> 26.5 us).
    const unsigned g = static_cast<unsigned>(std::min<int64_t>(blocks, 1024));
    const auto* x4 = static_cast<const uint4*>(x);
    auto* o4 = static_cast<uint4*>(out);
    if (dtype == SSC_F32)
      k_gn_apply_w<float><<<g, 256, 0, s>>>(x4, n, channels, groups, c4, batch, st, gamma, beta, act, o4);
    else if (dtype == SSC_BF16)
      k_gn_apply_w<uint16_t><<<g, 256, 0, s>>>(x4, n, channels, groups, c4, batch, st, gamma, beta, act, o4);
    else
      k_gn_apply_w<_Float16><<<g, 256, 0, s>>>(x4, n, channels, groups, c4, batch, st, gamma, beta, act, o4);
    return launch_status();
  }
  const int E = vec ? 16 / esz : 1;
  const int64_t items = n * (channels / E);
  const unsigned grid =
      static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>((items + 255) / 256, 262144)));
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

extern "C" ssc_status ssc_layer_norm(const void* x, int32_t dtype, int64_t n, int32_t channels,
                                     const float* gamma, const float* beta, float eps,
                                     int32_t act, void* out, void* stream) {
  if (n < 0 || channels < 1 || channels > 65536 || !(eps >= 0.f)) return SSC_ERR_ARG;
  if (dtype != SSC_F32 && dtype != SSC_BF16 && dtype != SSC_F16) return SSC_ERR_ARG;
  if (act < SSC_ACT_NONE || act > SSC_ACT_SILU) return SSC_ERR_ARG;
  if (n == 0) return SSC_OK;
  if (x == nullptr || out == nullptr || (gamma && !aligned(gamma, 4)) ||
      (beta && !aligned(beta, 4)))
    return SSC_ERR_ARG;
  hipStream_t s = as_stream(stream);
  const int esz = dtype == SSC_F32 ? 4 : 2;
  const int64_t row_bytes = static_cast<int64_t>(channels) * esz;
  const int64_t words = row_bytes / 16;
  if (row_bytes % 16 == 0 && words <= 64 && (words & (words - 1)) == 0 && aligned(x, 16) &&
      aligned(out, 16) && (!gamma || aligned(gamma, 16)) && (!beta || aligned(beta, 16))) {
    const int64_t rpb = 4 * 4 * (64 / words);  // rows per block step: 4 waves x 4 groups
    const unsigned g =
        static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>((n + rpb - 1) / rpb, 65536)));
    const auto* x4 = static_cast<const uint4*>(x);
    auto* o4 = static_cast<uint4*>(out);
    auto launch = [&](auto tag) {
      using T = decltype(tag);
      switch (words) {
#define SSC_LN(W) case W: k_layer_norm_w<T, W><<<g, 256, 0, s>>>(x4, n, channels, gamma, beta, eps, act, o4); break;
        SSC_LN(1) SSC_LN(2) SSC_LN(4) SSC_LN(8) SSC_LN(16) SSC_LN(32) default: SSC_LN(64)
#undef SSC_LN
      }
    };
    if (dtype == SSC_F32)
      launch(float{});
    else if (dtype == SSC_BF16)
      launch(uint16_t{});
    else
      launch(_Float16{});
    return launch_status();
  }
  const unsigned g =
      static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 65536)));
  if (dtype == SSC_F32)
    k_layer_norm_rows<float><<<g, 256, 0, s>>>(static_cast<const float*>(x), n, channels, gamma,
                                               beta, eps, act, static_cast<float*>(out));
  else if (dtype == SSC_BF16)
    k_layer_norm_rows<uint16_t><<<g, 256, 0, s>>>(static_cast<const uint16_t*>(x), n, channels,
                                                  gamma, beta, eps, act,
                                                  static_cast<uint16_t*>(out));
  else
    k_layer_norm_rows<_Float16><<<g, 256, 0, s>>>(static_cast<const _Float16*>(x), n, channels,
                                                  gamma, beta, eps, act,
                                                  static_cast<_Float16*>(out));
  return launch_status();
}
