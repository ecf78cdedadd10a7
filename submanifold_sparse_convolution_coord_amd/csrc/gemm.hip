// k=1 layers wider than the streaming kernel's 128 channels (the C -> 4C -> C MLP of the
// ConvNeXt-style block; LATO.2 MLX port page, "Status": SparseLinear): out = act(X @ W +
// bias) + residual for 16-bit X [n, cin] and W, fp32 accumulation on the matrix cores.
//
// A workgroup owns 128 rows x 64 columns (128-column tiles need 238 VGPRs, 2 waves per SIMD,
// and ran 10-20% slower).  For Cin of 192 and more the K loop runs in stages of 64: the rows'
// next stage is loaded into registers while the matrix cores consume this one from LDS
// (16-byte chunks XOR-swizzled by row), then written to the other LDS buffer; the weight
// fragments (packed per 16-column tile, 1 KB per fragment) go straight from global memory
// (L2-resident) into VGPRs, one stage ahead.  Each of the 4 waves owns one 16-column tile for
// all 128 rows, so every weight fragment is loaded once per workgroup; with 32 rows x 64
// columns per wave the 4 waves loaded the same fragments, twice the rows' bytes per stage
// (512 -> 128 + skip at 209K rows: 84.7 -> 73.7 us, bit-identical).  Cin of 64 and 128 takes a
// one-pass kernel (k_gemm_rows_narrow), whose waves keep 32 rows x 64 columns: with all of K
// at once, reading every row fragment four times from LDS cost more than the shared weight
// loads saved (128 -> 512 + silu: 86.4 against 81.9 us).  Rows past n are read as row n-1 and
// never stored.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"

namespace ssc {
namespace {

typedef __bf16 g_bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 g_f16x8_t __attribute__((ext_vector_type(8)));
typedef float g_f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t g_u32x4_t __attribute__((ext_vector_type(4)));  // a 16-byte word in registers

template <int EK>
__device__ __forceinline__ g_f32x4_t gemm_mfma(g_u32x4_t a, g_u32x4_t b, g_f32x4_t c) {
  if constexpr (EK == 0)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(g_bf16x8_t, a),
                                                   __builtin_bit_cast(g_bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(g_f16x8_t, a),
                                                  __builtin_bit_cast(g_f16x8_t, b), c, 0, 0, 0);
}

template <int EK>
__device__ __forceinline__ float from16(uint16_t h) {
  if constexpr (EK == 0) return bf16_to_f32(h);
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

template <int EK>
__device__ __forceinline__ uint16_t round16(float v) {
  if constexpr (EK == 0) return f32_to_bf16_rne(v);
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

constexpr int kGRows = 128;  // rows per tile
constexpr int kGK = 64;      // K per stage

template <int CT, bool OUT16, int EK>
__global__ __launch_bounds__(256, 2) void k_gemm_rows(const uint16_t* __restrict__ X,
                                                      const uint16_t* __restrict__ Wp,
                                                      const float* __restrict__ bias, int64_t n,
                                                      int cin, int cout, void* Y, int act,
                                                      const void* res, int64_t row_tiles) {
  constexpr int NCT = CT / 16;  // 16-column tiles, one per wave
  static_assert(NCT == 4, "one 16-column tile per wave");
  constexpr int ESZ = OUT16 ? 2 : 4;
  constexpr int ROWB = CT * ESZ;          // bytes of an output row of the tile
  constexpr int CHUNKS = ROWB / 16;
  constexpr int SWM = (CHUNKS < 16 ? CHUNKS : 16) - 1;
  constexpr int OUT_BYTES = kGRows * ROWB;  // the staged output tile
  constexpr int A_BYTES = 2 * kGRows * kGK * 2;
  __shared__ __attribute__((aligned(16))) char smem[OUT_BYTES > A_BYTES ? OUT_BYTES : A_BYTES];
  // two 16 KB stages of 128 rows x 8 chunks of 16 bytes
  auto* sA = reinterpret_cast<g_u32x4_t (*)[kGRows * kGK / 8]>(smem);
  // Workgroup -> (row tile, column tile).  The hardware deals consecutive workgroups to the
  // 8 XCDs in turn; XCD x takes row tiles x, x + 8, ... and each with all its column tiles
  // back to back, so the workgroups that read the same 128 input rows run together on one
  // XCD and share its L2 (spread over the XCDs, every XCD fetched the rows again; C -> 4C at
  // 128 channels and 209K rows: 111 -> 108 us).
  const int col_tiles = cout / CT;
  const int64_t xcd = blockIdx.x % 8, j = blockIdx.x / 8;
  const int64_t rt = (j / col_tiles) * 8 + xcd;
  if (rt >= row_tiles) return;  // the grid is rounded up to whole groups of 8 row tiles
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row0 = rt * kGRows;
  const int ct0 = static_cast<int>(j % col_tiles) * NCT;  // first 16-column tile
  const int ksteps = cin / 32;       // fragment index stride of a column tile
  const int stages = cin / kGK;

  auto load_a = [&](int st, g_u32x4_t (&r)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = threadIdx.x + k * 256;
      const int row = idx >> 3, ch = idx & 7;
      const int64_t g = std::min<int64_t>(row0 + row, n - 1);
      r[k] = *reinterpret_cast<const g_u32x4_t*>(X + g * cin + st * kGK + ch * 8);
    }
  };
  auto store_a = [&](int buf, const g_u32x4_t (&r)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = threadIdx.x + k * 256;
      const int row = idx >> 3, ch = idx & 7;
      sA[buf][row * 8 + (ch ^ (row & 7))] = r[k];
    }
  };
  // The wave's 32 residual rows of the tile (whole 16-byte pieces, in the order the epilogue
  // stages them), loaded before the K loop so that their latency is hidden behind it.
  constexpr int RPT = 32 * CHUNKS / 64;  // residual pieces per lane
  const int64_t wrow0 = row0 + wave * 32;
  const int64_t col0b = static_cast<int64_t>(ct0) * 16 * ESZ;  // byte offset of the tile
  g_u32x4_t rres[RPT];
  if (res) {
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int idx = lane + k * 64;
      const int r = idx / CHUNKS, ch = idx % CHUNKS;
      const int64_t g = std::min<int64_t>(wrow0 + r, n - 1);
      rres[k] = *reinterpret_cast<const g_u32x4_t*>(static_cast<const char*>(res) +
                                                    g * cout * ESZ + col0b + ch * 16);
    }
  }
  // Wave w owns the 16-column tile ct0 + w for all 128 rows: each weight fragment is loaded
  // by one wave only, and the rows' fragments are read from LDS by all four.
  const int ctw = ct0 + wave;
  auto load_b = [&](int st, g_u32x4_t (&b)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      b[ks] = *reinterpret_cast<const g_u32x4_t*>(
          Wp + (static_cast<int64_t>(ctw) * ksteps + st * 2 + ks) * 512 + lane * 8);
  };
  g_f32x4_t acc[8];
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) acc[rb] = g_f32x4_t{0.f, 0.f, 0.f, 0.f};
  g_u32x4_t ra[4], bw[2], bn[2];
  load_a(0, ra);
  store_a(0, ra);
  load_b(0, bw);
  __syncthreads();
  for (int st = 0; st < stages; ++st) {
    const int cur = st & 1;
    const bool more = st + 1 < stages;
    if (more) {
      load_a(st + 1, ra);
      load_b(st + 1, bn);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int rb = 0; rb < 8; ++rb) {
        const int row = rb * 16 + (lane & 15);
        const int ch = ks * 4 + (lane >> 4);
        const g_u32x4_t a = sA[cur][row * 8 + (ch ^ (row & 7))];
        acc[rb] = gemm_mfma<EK>(a, bw[ks], acc[rb]);
      }
    if (more) {
      store_a(cur ^ 1, ra);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bw[ks] = bn[ks];
    }
    __syncthreads();
  }
  // Epilogue: one staging tile of 128 rows for the workgroup (16-byte chunks XOR-swizzled by
  // row); residual pieces first (each wave its 32 rows), then every wave its 16 columns.
  char* sO = smem;
  if (res) {
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int idx = lane + k * 64;
      const int r = wave * 32 + idx / CHUNKS, ch = idx % CHUNKS;
      *reinterpret_cast<g_u32x4_t*>(sO + r * ROWB + ((ch ^ (r & SWM)) << 4)) = rres[k];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __syncthreads();
  }
  {
    const int col = wave * 16 + (lane & 15);
    const float bc = bias ? bias[ctw * 16 + (lane & 15)] : 0.f;
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb * 16 + (lane >> 4) * 4 + i;
        const int byte = col * ESZ;
        char* dst = sO + r * ROWB + (((byte >> 4) ^ (r & SWM)) << 4) + (byte & 15);
        float v = apply_act(acc[rb][i] + bc, act);
        if (res) {
          if constexpr (OUT16)
            v += from16<EK>(*reinterpret_cast<const uint16_t*>(dst));
          else
            v += *reinterpret_cast<const float*>(dst);
        }
        if constexpr (OUT16)
          *reinterpret_cast<uint16_t*>(dst) = round16<EK>(v);
        else
          *reinterpret_cast<float*>(dst) = v;
      }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 32 * CHUNKS / 64; ++k) {
    const int idx = lane + k * 64;
    const int r = idx / CHUNKS, ch = idx % CHUNKS;
    const int tr = wave * 32 + r;
    if (wrow0 + r < n)
      st16(reinterpret_cast<g_u32x4_t*>(static_cast<char*>(Y) + (wrow0 + r) * cout * ESZ + col0b +
                                        ch * 16),
           *reinterpret_cast<const g_u32x4_t*>(sO + tr * ROWB + ((ch ^ (tr & SWM)) << 4)));
  }
}

// Cin 64 or 128: the tile's 128 rows, all of K, go to LDS in one batch of direct
// global->LDS copies (no registers held, one wait), with the weight fragments and the
// residual pieces loading alongside; then one pass of matrix work and the same epilogue.
// With only 2 or 4 k-steps there is nothing to pipeline, and the two-stage register path
// above spends its time in the latency of its stages (128 -> 512 at 209K rows: 109 -> 87
// us; 64 -> 256 at 268K rows: 57 -> 42 us, bit-identical results).  Copy k of a wave fills
// LDS bytes [k*1024, (k+1)*1024): lane l writes slot (row, p) = divmod(64 k + l, CPR), which
// holds the row's chunk p ^ (row & 7), the swizzle the fragment reads expect.
template <int KS, bool OUT16, int EK>
__global__ __launch_bounds__(256, (OUT16 || KS < 4) ? 4 : 3) void k_gemm_rows_narrow(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wp,
    const float* __restrict__ bias, int64_t n, int cout, void* Y, int act, const void* res,
    int64_t row_tiles) {
  constexpr int CIN = KS * 32;
  constexpr int CPR = CIN / 8;
  constexpr int NCT = 4;
  constexpr int ESZ = OUT16 ? 2 : 4;
  constexpr int ROWB = 64 * ESZ;
  constexpr int CHUNKS = ROWB / 16;
  constexpr int SWM = CHUNKS - 1;
  constexpr int RPT = 32 * CHUNKS / 64;
  constexpr int A_BYTES = kGRows * CIN * 2;
  constexpr int OUT_BYTES = 4 * 32 * ROWB;
  __shared__ __attribute__((aligned(1024))) char smem[A_BYTES > OUT_BYTES ? A_BYTES : OUT_BYTES];
  // (row tile, column tile) as in k_gemm_rows: a row tile's column tiles together on one XCD
  const int col_tiles = cout / 64;
  const int64_t xcd = blockIdx.x % 8, j = blockIdx.x / 8;
  const int64_t rt = (j / col_tiles) * 8 + xcd;
  if (rt >= row_tiles) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row0 = rt * kGRows;
  const int ct0 = static_cast<int>(j % col_tiles) * NCT;
  constexpr int COPIES = A_BYTES / 1024 / 4;  // per wave
#pragma unroll
  for (int i = 0; i < COPIES; ++i) {
    const int k = i * 4 + wave;
    const int slot = k * 64 + lane;
    const int r = slot / CPR, p = slot % CPR;
    const int64_t g = std::min<int64_t>(row0 + r, n - 1);
    dma16(X + g * CIN + (p ^ (r & 7)) * 8, lds_addr(smem + k * 1024));
  }
  g_u32x4_t bw[KS][NCT];
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int c = 0; c < NCT; ++c)
      bw[k][c] = *reinterpret_cast<const g_u32x4_t*>(
          Wp + (static_cast<int64_t>(ct0 + c) * KS + k) * 512 + lane * 8);
  float bcol[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) bcol[c] = bias ? bias[(ct0 + c) * 16 + (lane & 15)] : 0.f;
  const int64_t wrow0 = row0 + wave * 32;
  const int64_t col0b = static_cast<int64_t>(ct0) * 16 * ESZ;
  g_u32x4_t rres[RPT];
  if (res) {
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int idx = lane + k * 64;
      const int r = idx / CHUNKS, ch = idx % CHUNKS;
      const int64_t g = std::min<int64_t>(wrow0 + r, n - 1);
      rres[k] = *reinterpret_cast<const g_u32x4_t*>(static_cast<const char*>(res) +
                                                    g * cout * ESZ + col0b + ch * 16);
    }
  }
  wait_vm_lgkm0();  // the copies (and the loads) have landed
  __syncthreads();
  g_f32x4_t acc[2][NCT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int c = 0; c < NCT; ++c) acc[t][c] = g_f32x4_t{0.f, 0.f, 0.f, 0.f};
  const auto* sA = reinterpret_cast<const g_u32x4_t*>(smem);
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = wave * 32 + t * 16 + (lane & 15);
      const int ch = k * 4 + (lane >> 4);
      const g_u32x4_t a = sA[row * CPR + (ch ^ (row & 7))];
#pragma unroll
      for (int c = 0; c < NCT; ++c) acc[t][c] = gemm_mfma<EK>(a, bw[k][c], acc[t][c]);
    }
  __syncthreads();  // every wave is past its A reads: the area becomes the output staging
  char* sO = smem + wave * 32 * ROWB;
  if (res) {
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int idx = lane + k * 64;
      const int r = idx / CHUNKS, ch = idx % CHUNKS;
      *reinterpret_cast<g_u32x4_t*>(sO + r * ROWB + ((ch ^ (r & SWM)) << 4)) = rres[k];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int col = c * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = t * 16 + (lane >> 4) * 4 + i;
        const int byte = col * ESZ;
        char* dst = sO + r * ROWB + (((byte >> 4) ^ (r & SWM)) << 4) + (byte & 15);
        float v = apply_act(acc[t][c][i] + bcol[c], act);
        if (res) {
          if constexpr (OUT16)
            v += from16<EK>(*reinterpret_cast<const uint16_t*>(dst));
          else
            v += *reinterpret_cast<const float*>(dst);
        }
        if constexpr (OUT16)
          *reinterpret_cast<uint16_t*>(dst) = round16<EK>(v);
        else
          *reinterpret_cast<float*>(dst) = v;
      }
    }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's staging writes are done
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int idx = lane + k * 64;
    const int r = idx / CHUNKS, ch = idx % CHUNKS;
    if (wrow0 + r < n)
      st16(reinterpret_cast<g_u32x4_t*>(static_cast<char*>(Y) + (wrow0 + r) * cout * ESZ + col0b +
                                        ch * 16),
           *reinterpret_cast<const g_u32x4_t*>(sO + r * ROWB + ((ch ^ (r & SWM)) << 4)));
  }
}

}  // namespace

// Shapes the GEMM takes: 16-bit inputs, cin a multiple of 64, cout a multiple of 64, both
// at most 1024.
bool gemm_rows_supported(int cin, int cout) {
  return cin >= 64 && cout >= 64 && cin % 64 == 0 && cout % 64 == 0 && cin <= 1024 &&
         cout <= 1024;
}

// Weights in wp are packed per 16-column tile (the conv's fragment order with one tap and
// cout / 16 column groups).
ssc_status gemm_rows_launch(const void* feats, const uint16_t* wp, const float* bias, int64_t n,
                            int cin, int cout, void* out, bool out16, int ek, int act,
                            const void* res, hipStream_t s) {
  const int64_t row_tiles = (n + kGRows - 1) / kGRows;
  const auto* x = static_cast<const uint16_t*>(feats);
  const int64_t grid = (row_tiles + 7) / 8 * 8 * (cout / 64);
  if (cin == 64 || cin == 128) {
    using Fn = void (*)(const uint16_t*, const uint16_t*, const float*, int64_t, int, void*, int,
                        const void*, int64_t);
    Fn f;
    if (cin == 64)
      f = out16 ? (ek == 1 ? k_gemm_rows_narrow<2, true, 1> : k_gemm_rows_narrow<2, true, 0>)
                : (ek == 1 ? k_gemm_rows_narrow<2, false, 1> : k_gemm_rows_narrow<2, false, 0>);
    else
      f = out16 ? (ek == 1 ? k_gemm_rows_narrow<4, true, 1> : k_gemm_rows_narrow<4, true, 0>)
                : (ek == 1 ? k_gemm_rows_narrow<4, false, 1> : k_gemm_rows_narrow<4, false, 0>);
    hipLaunchKernelGGL(f, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, x, wp, bias, n,
                       cout, out, act, res, row_tiles);
    return launch_status();
  }
  auto fn = out16 ? (ek == 1 ? k_gemm_rows<64, true, 1> : k_gemm_rows<64, true, 0>)
                  : (ek == 1 ? k_gemm_rows<64, false, 1> : k_gemm_rows<64, false, 0>);
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, x, wp, bias, n, cin,
                     cout, out, act, res, row_tiles);
  return launch_status();
}

}  // namespace ssc
