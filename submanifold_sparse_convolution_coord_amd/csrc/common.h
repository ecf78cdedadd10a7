// Internal helpers shared by the libssc.so translation units (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssc.h"

namespace ssc {

constexpr int kTaps = 27;
constexpr int kCentreTap = 13;
constexpr int64_t kMaxCoord = 65535;   // grid extents and batch must fit 16-bit key fields
constexpr size_t kAlign = 256;         // every sub-buffer starts on this boundary

inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }
inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline ssc_status launch_status() {
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}

// Plan buffer layout (all offsets 256-byte aligned):
//   header  int64[8]: magic, n, npad, nblocks, tile schedule, reserved...
//           (tile schedule: kSchedInterleaved or kSchedPerXcd, chosen with the site order)
//   zero    2048 zero bytes   the source of missing neighbour rows (Cin <= 1024 bf16)
//   perm    int32[npad]       sorted position -> original row, -1 for padding
//   bmask   uint32[nblocks]   OR of the tap-validity masks of the 16 rows of each block
//   gidx    int32[27][npad]   neighbour row of sorted position r for tap t, -1 if none
constexpr int64_t kPlanMagic = 0x5353435031LL;  // "SSCP1"
constexpr int kPlanRowAlign = 256;              // npad is a multiple of this
constexpr int kBlockRows = 16;                  // rows per MFMA block
constexpr int kTileRows = 128;                  // rows per tile of the k=3 matrix-core kernel
constexpr int kPlanSchedWord = 4;               // header word holding the tile schedule
// Tile schedules of the k=3 matrix-core kernel (which workgroup takes which tile):
//   interleaved  workgroup b takes tile T-1-b: the hardware deals consecutive workgroups to
//                the 8 XCDs in turn, so every XCD sweeps the whole order, heaviest tiles first.
//   per XCD      XCD x (workgroups b with b % 8 == x) takes the x-th contiguous eighth of the
//                tiles, in order: with a spatially ordered plan each XCD's L2 then holds the
//                rows of one region and its halo.
constexpr int64_t kSchedInterleaved = 0;
constexpr int64_t kSchedPerXcd = 1;
constexpr int kXcds = 8;

struct PlanLayout {
  int64_t n, npad, nblocks;
  size_t off_zero, off_perm, off_bmask, off_gidx, total;
};
constexpr size_t kZeroBytes = 2048;

inline PlanLayout plan_layout(int64_t n) {
  PlanLayout L;
  L.n = n;
  L.npad = ((n > 0 ? n : 1) + kPlanRowAlign - 1) / kPlanRowAlign * kPlanRowAlign;
  L.nblocks = L.npad / kBlockRows;
  L.off_zero = kAlign;
  L.off_perm = align_up(L.off_zero + kZeroBytes);
  L.off_bmask = align_up(L.off_perm + sizeof(int32_t) * L.npad);
  L.off_gidx = align_up(L.off_bmask + sizeof(uint32_t) * L.nblocks);
  L.total = align_up(L.off_gidx + sizeof(int32_t) * kTaps * L.npad);
  return L;
}

// Round-to-nearest-even fp32 -> bf16 (ties to even; overflow to infinity; NaN stays a quiet
// NaN): the conversion instruction gfx950 has for it (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Epilogue activations: relu = max(v, 0), silu = v * sigmoid(v) = v * 1 / (1 + e^-v) (e^-v
// and the reciprocal from the hardware's approximate exp and rcp, each within about an ulp;
// at very negative v, e^-v overflows to inf and the product is -0).
// Contraction is off here: the silu product must round on its own, so that a caller adding to
// it (a residual) gets the same fp32 value in every kernel variant, whatever it then stores.
__device__ __forceinline__ float apply_act(float v, int act) {
#pragma clang fp contract(off)
  if (act == SSC_ACT_RELU) return v > 0.f ? v : 0.f;
  if (act == SSC_ACT_SILU) return v * __builtin_amdgcn_rcpf(1.f + __expf(-v));
  return v;
}

// LDS byte address of a __shared__ location (wave-uniform in every use).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<size_t>((__attribute__((address_space(3))) const char*)p));
}

// One direct global->LDS copy (global_load_lds_dwordx4): every active lane fetches 16 bytes
// from its own global address and the hardware writes them to LDS at lds_base + 16*lane.
// Written as inline asm, not the builtin, on purpose: the compiler then does not treat the
// copy as a pending write to every LDS location, which would otherwise make it drain all
// copies (vmcnt 0) before each LDS read and serialize the pipeline.  The instruction has no
// destination register (the data goes to LDS; the address VGPRs are read at issue), and
// every wait for these copies is explicit in the kernel (wait_vm_lgkm0 before each barrier).
// m0 (which holds the LDS base) is saved and restored inside the statement, so the compiler's
// view of every register is unchanged by it.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

// A non-temporal 16-byte store, for outputs that a kernel writes once and that the next op
// streams rather than gathers (the k=1 layers and the layer norm): streaming them past the
// caches measured 237.6 against 251.7 us for the 128-channel ConvNeXt-style block at 209K
// sites (4C -> C + skip 73.1 -> 66.2 us) and 24.2 against 26.1 us for a 128 -> 128 k=1 layer
// with an fp32 store.  The group-norm apply keeps plain stores: its output is gathered by the
// next convolution, which then read it from the caches (residual block 202 against 206 us).
typedef uint32_t st16_u32x4_t __attribute__((ext_vector_type(4)));
template <typename W>
__device__ __forceinline__ void st16(W* p, const W& v) {
  static_assert(sizeof(W) == 16, "16-byte word");
  __builtin_nontemporal_store(__builtin_bit_cast(st16_u32x4_t, v), reinterpret_cast<st16_u32x4_t*>(p));
}

// s_waitcnt vmcnt(0) lgkmcnt(0): every global load / direct copy and every LDS access issued
// by this wave has completed.
__device__ __forceinline__ void wait_vm_lgkm0() { __builtin_amdgcn_s_waitcnt(0x0070); }

}  // namespace ssc
