// SubMConv3d (k=3) and its k=1 case on the gfx950 matrix cores.
//
//   out[i] = bias + sum_t sum_c feats[nbr[i][t]][c] * W[t][c][:]      (cross-correlation,
//   LATO.2 MLX port page, "Correctness"; weights [K^3, Cin, Cout], Pixal3D README, "Status")
//
// The pages' own designs are a per-offset gather / matmul / scatter-add loop (trellis-mac
// article, flowchart; LATO.2 page, "Fleet benchmark": 2*K^3 = 54 dispatches, launch bound)
// and one fused [N, K^3*Cin] x [K^3*Cin, Cout] matmul over a cached device index (LATO.2
// page, version history).  Here the whole layer is ONE kernel, output-stationary:
//
//   * a workgroup owns a tile of NB 16-row blocks of the plan's site order (sites sorted by
//     their tap-validity mask, so a block's rows mostly share which taps exist; on surfaces
//     first by 128^3 brick, with the tiles dealt to the XCDs in contiguous shares);
//   * for every tap present in the tile, each wave loads its slice of W[t] into registers as
//     matrix-core B fragments, then, for each block whose mask has tap t, gathers the 16
//     neighbour rows straight from HBM/L2 into A fragments (a missing neighbour is a zero row,
//     never loaded) and issues bf16 16x16x32 MFMAs into fp32 accumulators held in VGPRs;
//   * (block, tap) pairs with no neighbour at all are skipped by a wave-uniform branch;
//   * the epilogue adds the bias and stores each row at its original index, fp32 or bf16
//     (round-to-nearest-even of the same fp32 value).
// Every output element is owned by exactly one lane, so there are no atomics and results
// are bit-identical run to run, and independent of the site order.
//
// The matrix cores want both operands k-contiguous per lane, so W is re-laid out per call
// (27*Cin*Cout*2 bytes in the caller's workspace): fragment by fragment for the k=3 kernel
// (k_pack_frag), as Wt[o][c] for the k=1 kernel (k_transpose_w).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"

namespace ssc {
// Standalone group-norm partial sums (norm.hip), for epilogues whose kernel cannot sum them.
ssc_status gn_partials_launch(const void* x, int32_t dtype, int64_t n, int32_t channels,
                              const int32_t* coords, int32_t batch, int32_t groups,
                              float* partials, hipStream_t s);
// Matrix-core GEMM for k=1 layers wider than the streaming kernel's (gemm.hip).
bool gemm_rows_supported(int cin, int cout);
ssc_status gemm_rows_launch(const void* feats, const uint16_t* wp, const float* bias, int64_t n,
                            int cin, int cout, void* out, bool out16, int ek, int act,
                            const void* res, hipStream_t s);
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ bf16x8_t zero_bf16x8() {
  return __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u});
}

// Matrix-core fragment layout of v_mfma_f32_16x16x32_bf16 (wave64), as used below:
//   A (16 x 32): lane l holds row (l & 15), k = 8*(l >> 4) .. +7
//   B (32 x 16): lane l holds column (l & 15), k = 8*(l >> 4) .. +7
//   D (16 x 16): lane l holds column (l & 15), rows 4*(l >> 4) .. +3
// Both operands use the same (lane, element) -> k assignment, so the product is the full
// k-sum whatever order the hardware walks k in.  A weight fragment (lane l: output channel
// l & 15, 8 input channels) is therefore also a valid A operand and a gathered-row fragment
// (lane l: site l & 15, 8 input channels) a valid B operand: the k=3 kernel multiplies them
// in that order, so its D holds output channels as rows and sites as columns.


// ------------------------------------------------------------------------------------------
// k=3 convolution kernel: gathers staged in LDS, software-pipelined over the taps of a tile.
//
// A workgroup of 4 waves owns one tile of NB 16-row blocks of the plan's site order.  The
// taps present in the tile (the OR of its block masks) are walked in ascending order.  For
// each tap one stage is prepared ahead of its use:
//   * the 16 neighbour feature rows of every block that has tap t are copied into LDS by the
//     gfx950 direct global->LDS loads (global_load_lds_dwordx4: no VGPRs held while in
//     flight); a missing neighbour copies a zero row;
//   * each wave loads its column slice of W[t] into VGPRs as matrix-core B fragments, into
//     the register set of the stage's parity.  The packed weights are stored fragment by
//     fragment, so each of these loads reads 1 KB of contiguous memory.
// While the matrix cores consume stage q, stage q+1 is in flight.  Per tap there is one wait
// (vmcnt 0, lgkmcnt 0: at that point only stage q is outstanding) and one bare workgroup
// barrier, which makes the copies of all waves visible and proves that every wave finished
// reading the buffer the next stage overwrites.
// 16-byte chunks of each LDS row are XOR-swizzled so that the 16 rows a fragment read touches
// fall in distinct banks.  Waves are WR x WC: column group wc owns COUT/WC output columns,
// row group wr owns blocks wr, wr+WR, ...; fp32 accumulators stay in VGPRs.
// The epilogue adds the bias, stages the tile's output rows in LDS (over the dead gather
// buffers; each lane writes its four consecutive channels of a site as one piece) and writes
// every row with 16-byte stores at its original index.
// ------------------------------------------------------------------------------------------
template <int CIN, int COUT, int NB, int WR, int WC>
struct LdsCfg {
  static constexpr int WAVES = WR * WC;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int CPR = CIN / 8;             // 16-byte chunks per feature row
  static constexpr int RPW = 16 / WAVES;          // rows of each block a wave copies
  static constexpr int A_LANES = RPW * CPR;       // lanes active in a block copy
  static constexpr int A_BLOCK = 16 * CIN;        // bf16 elements per block slot
  static constexpr int CS = COUT / WC;            // output columns per wave
  static constexpr int NCT = CS / 16;             // 16-column MFMA tiles per wave
  static constexpr int KS = CIN / 32;             // k-steps
  static constexpr int BPW = NB / WR;             // blocks accumulated per wave
  static constexpr int G_TAPS_PER_COPY = 64 / (NB * 4);  // taps of indices per 1 KB copy
  // LDS arena: [gather buffer 0][gather buffer 1][indices 27 x NB*16][row ids NB*16]
  static constexpr int ABUF_BYTES = NB * A_BLOCK * 2;
  static constexpr int OFF_A1 = ABUF_BYTES;
  static constexpr int OFF_G = 2 * ABUF_BYTES;
  static constexpr int OFF_P = OFF_G + kTaps * NB * 16 * 4;
  static constexpr int SMEM_BYTES = OFF_P + NB * 16 * 4;
  static constexpr int STAGE_BYTES = OFF_P;       // reusable for the output rows at the end
  static_assert(16 % WAVES == 0 && A_LANES <= 64 && A_LANES > 0, "block copy shape");
  static_assert(CIN % 32 == 0 && COUT % (16 * WC) == 0 && NB % WR == 0, "tile shape");
  static_assert(NB * 4 <= 64 && 64 % (NB * 4) == 0, "index copy shape");
  // Every LDS access stays inside its region (the kernel's index arithmetic, bound by bound):
  //   gather copies: block b < NB, piece offset + 64 lanes x 16 B within one block slot;
  static_assert(CIN < 128 ? (64 / CPR) * CIN * 2 * (16 / (64 / CPR)) == A_BLOCK * 2
                          : RPW * CIN * 2 * WAVES == A_BLOCK * 2 && RPW * CPR == 64,
                "copies tile a block slot exactly");
  //   A fragments: row (l & 15) and chunk (l >> 4) + 4 s < CPR stay in the block slot;
  static_assert(16 * CPR * 16 == A_BLOCK * 2 && 3 + 4 * (KS - 1) < CPR,
                "fragment reads inside a block slot");
  //   neighbour indices: at most 27 taps x NB * 16 rows, then NB * 16 row ids.
  static_assert(OFF_G + kTaps * NB * 16 * 4 == OFF_P && OFF_P + NB * 16 * 4 == SMEM_BYTES &&
                OFF_G == 2 * ABUF_BYTES, "index and row-id regions");
  static_assert(SMEM_BYTES <= 160 * 1024, "LDS of one workgroup");
};

// Fragment-major packed weights for WC column groups: element
//   Wp[(((v*WC + wc)*NCT + c)*KS + s)*512 + lane*8 + e]
//     = W[t][kc*CK + 32s + 8(lane>>4) + e][ct*COT + wc*CS + 16c + (lane&15)]
// i.e. the B fragment of (virtual tap v, wave column group wc, column tile c, k-step s) for
// `lane`.  A layer wider than one kernel tile is cut into input chunks of CK channels (kc of
// cin / CK) and output tiles of COT columns (ct of cout / COT); virtual tap v = (ct * taps +
// t) * (cin / CK) + kc, so every (t, kc) block of one output tile has the layout of a CK x COT
// layer's tap.  CK = cin and COT = cout give v = t.
// flip = 1 packs W[taps-1-t] into tap t: the tap at offset d then reads site c - d, the other
// orientation the LATO.2 page leaves open (its "--flip-kernel").
__global__ __launch_bounds__(256) void k_pack_frag(const uint16_t* __restrict__ W, int taps,
                                                   int cin, int cout, int ck, int cot,
                                                   int wc_groups, int flip,
                                                   uint16_t* __restrict__ Wp) {
  const int cs = cot / wc_groups, nct = cs / 16, ks = ck / 32;
  const int kch = cin / ck, ctn = cout / cot;
  const int64_t total = static_cast<int64_t>(taps) * kch * ctn * wc_groups * nct * ks * 64;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += stride) {
    const int lane = static_cast<int>(idx % 64);
    int64_t rest = idx / 64;
    const int s = static_cast<int>(rest % ks);
    rest /= ks;
    const int c = static_cast<int>(rest % nct);
    rest /= nct;
    const int wc = static_cast<int>(rest % wc_groups);
    const int64_t v = rest / wc_groups;
    const int kc = static_cast<int>(v % kch);
    const int64_t t = (v / kch) % taps;
    const int ct = static_cast<int>(v / (static_cast<int64_t>(kch) * taps));
    const int o = ct * cot + wc * cs + c * 16 + (lane & 15);
    const int k0 = kc * ck + s * 32 + (lane >> 4) * 8;
    const int64_t ts = flip ? taps - 1 - t : t;
    const uint16_t* src = W + (ts * cin + k0) * cout + o;
    uint16_t* dst = Wp + idx * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = src[static_cast<int64_t>(e) * cout];
  }
}

// Chunk swizzle: row r's logical 16-byte chunk c lives in slot c ^ swz(r).  For 16
// consecutive rows and a fixed chunk the slots then differ in their bank group.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  return ((r * CPR) >> 4) & (CPR - 1);
}


__device__ __forceinline__ bf16x8_t lds_read16(const void* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

// 16-bit element kinds of the matrix-core paths: EK = 0 bf16, EK = 1 fp16.  Fragments are
// carried as 16-byte words; the kind only picks the instruction and the output rounding.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
template <int EK>
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  if constexpr (EK == 0)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
// fp32 -> 16-bit output of kind EK, round to nearest even.
template <int EK>
__device__ __forceinline__ uint16_t to16(float v) {
  if constexpr (EK == 0)
    return f32_to_bf16_rne(v);
  else
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

// Copies of stage (union index q, tap t) for every block that has tap t.  Each copy
// instruction moves 64 lanes x 16 bytes = RPI whole rows of one block into LDS (the lane's
// 16-byte chunk of the row goes to its swizzled slot, missing neighbours read the zero row).
// A block is PIECES such copies; piece i of the tile (block i / PIECES, part i % PIECES) is
// always issued by wave i % WAVES, so a wave reads all its row indices before its first copy.
// With CIN = 128 that is one 4-row part of every block per wave; narrower rows give each
// wave whole blocks (CIN = 32) or half blocks (CIN = 64), and no lane of a copy idles.
// Blocks of the tile that have tap t, as a bit set (lane b of bmv holds block b's tap mask,
// lanes past the tile hold 0).
__device__ __forceinline__ uint32_t block_taps(uint32_t bmv, int t) {
  return static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(((bmv >> t) & 1u) != 0u));
}

// X points at the stage's input chunk (channel kc * CIN of row 0); xs is the row stride in
// elements (CIN times the number of chunks).
template <int CIN, int COUT, int NB, int WR, int WC>
__device__ __forceinline__ void issue_gather(int q, uint32_t act, const uint16_t* __restrict__ X,
                                             int64_t xs, const uint16_t* __restrict__ zrow,
                                             const int32_t* sG, uint32_t sA, int wave, int lane) {
  using C = LdsCfg<CIN, COUT, NB, WR, WC>;
  const int32_t* g = sG + q * (NB * 16);
  if constexpr (CIN < 128) {
    constexpr int RPI = 64 / C::CPR;
    constexpr int PIECES = 16 / RPI;
    constexpr int PPW = NB * PIECES / C::WAVES;
    static_assert(NB * PIECES % C::WAVES == 0 && (C::WAVES & (C::WAVES - 1)) == 0,
                  "pieces per wave");
    const int rsub = lane / C::CPR;
    int32_t j[PPW];
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int piece = i * C::WAVES + wave;
      j[i] = g[(piece / PIECES) * 16 + (piece % PIECES) * RPI + rsub];
    }
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int piece = i * C::WAVES + wave;
      const int b = piece / PIECES, part = piece % PIECES;
      if (!((act >> b) & 1u)) continue;
      const int chunk = (lane % C::CPR) ^ swz<C::CPR>(part * RPI + rsub);
      const uint16_t* src =
          j[i] >= 0 ? X + static_cast<int64_t>(j[i]) * xs + chunk * 8 : zrow + chunk * 8;
      dma16(src, sA + b * C::A_BLOCK * 2 + part * 1024);
    }
  } else {
    // CIN = 128: wave w copies rows 4w..4w+3 of every block (the same pieces as above, with
    // the block's test hoisted out of the index arithmetic).
    const int rr = (wave * C::RPW + lane / C::CPR) & 15;
    const int chunk = (lane % C::CPR) ^ swz<C::CPR>(rr);
    int32_t j[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) j[b] = g[b * 16 + rr];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (!((act >> b) & 1u)) continue;
      const uint16_t* src =
          j[b] >= 0 ? X + static_cast<int64_t>(j[b]) * xs + chunk * 8 : zrow + chunk * 8;
      dma16(src, sA + b * C::A_BLOCK * 2 + wave * C::RPW * CIN * 2);
    }
  }
}

template <int CIN, int COUT, int NB, int WR, int WC>
__device__ __forceinline__ void load_weights(int t, const uint16_t* __restrict__ Wp, int wc,
                                             int lane,
                                             bf16x8_t (&bw)[COUT / WC / 16][CIN / 32]) {
  using C = LdsCfg<CIN, COUT, NB, WR, WC>;
  const uint16_t* w =
      Wp + ((static_cast<int64_t>(t) * WC + wc) * (C::NCT * C::KS)) * 512 + lane * 8;
#pragma unroll
  for (int c = 0; c < C::NCT; ++c)
#pragma unroll
    for (int s = 0; s < C::KS; ++s) bw[c][s] = load_bf16x8(w + (c * C::KS + s) * 512);
}

// Byte offsets, within a block slot, of this lane's A fragments (row lane&15, logical chunk
// (lane>>4) + 4s, swizzled).  Block b's fragments are at b * A_BLOCK * 2 bytes more, which
// the compiler folds into the LDS instruction's immediate offset.
template <int CIN>
__device__ __forceinline__ void a_frag_offsets(int lane, uint32_t (&off)[CIN / 32]) {
  constexpr int CPR = CIN / 8;
  const int r = lane & 15;
#pragma unroll
  for (int s = 0; s < CIN / 32; ++s) {
    const int chunk = (lane >> 4) + 4 * s;
    off[s] = static_cast<uint32_t>((r * CPR + (chunk ^ swz<CPR>(r))) * 16);
  }
}

// This wave's first block's A fragments of a stage (block wr of the gather buffer at sA).
// The stage loop reads them right after the barrier that publishes the stage, before it issues
// the next stage's loads, so they are in registers when the matrix work starts.  (Read inside
// the stage's first block, the compiler waited for each of them in turn.)
template <int CIN, int COUT, int NB, int WR, int WC>
__device__ __forceinline__ void read_first(const char* sA, const uint32_t (&aoff)[CIN / 32],
                                           int wr, bf16x8_t (&a0)[CIN / 32]) {
  using C = LdsCfg<CIN, COUT, NB, WR, WC>;
#pragma unroll
  for (int s = 0; s < C::KS; ++s) a0[s] = lds_read16(sA + wr * (C::A_BLOCK * 2) + aoff[s]);
}

// Matrix work of one stage.  The product is computed transposed, D = W^T X^T (the weight
// fragment as the A operand, the gathered rows as the B operand: the same registers, the
// roles swapped), so that each lane's four accumulators are four consecutive output channels
// of one site (lane l: site row l & 15, channels 4 (l >> 4) .. +3 of the 16-column tile), which
// the epilogue stores as one 16-byte (fp32) or 8-byte (16-bit) piece.  The A fragments of this
// wave's blocks are read from LDS one block ahead of the MFMAs that use them (register set
// bl & 1), so the LDS latency of a block hides behind the previous block's matrix work; the
// first block's (a0) were read by read_first.
template <int CIN, int COUT, int NB, int WR, int WC, int EK>
__device__ __forceinline__ void compute_stage(uint32_t act, const char* sA,
                                              const bf16x8_t (&bw)[COUT / WC / 16][CIN / 32],
                                              const uint32_t (&aoff)[CIN / 32], int wr,
                                              const bf16x8_t (&a0)[CIN / 32],
                                              f32x4_t (&acc)[NB / WR][COUT / WC / 16]) {
  using C = LdsCfg<CIN, COUT, NB, WR, WC>;
  bf16x8_t a[2][C::KS];
#pragma unroll
  for (int s = 0; s < C::KS; ++s) a[0][s] = a0[s];
#pragma unroll
  for (int bl = 0; bl < C::BPW; ++bl) {
    if (bl + 1 < C::BPW) {
      const char* nblk = sA + ((bl + 1) * WR + wr) * (C::A_BLOCK * 2);
#pragma unroll
      for (int s = 0; s < C::KS; ++s) a[(bl + 1) & 1][s] = lds_read16(nblk + aoff[s]);
    }
    const int b = bl * WR + wr;
    if (!((act >> b) & 1u)) continue;
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
#pragma unroll
      for (int c = 0; c < C::NCT; ++c)
        acc[bl][c] = mfma16x16x32<EK>(bw[c][s], a[bl & 1][s], acc[bl][c]);
  }
}

// Epilogue arguments of the kernels: a residual added after the activation, and (k=3
// matrix-core kernel, batch 1) the group-norm partial slots it sums from its own stores.
struct Epi {
  const void* res;   // [n, cout] in the output type, rows in coords order, or null
  float* gn;         // float4 slots [npad / 128][groups] (count, sum, sum of squares, 0)
  int64_t rows;      // n: plan rows at or past it are padding (they sort last)
  int act;           // SSC_ACT_*
  int gn_groups;     // with gn: groups of cout / gn_groups channels, a power of two <= 16
  // The k=1 layer a pair kernel (C2 > 0) applies to its 16-bit k=3 output: packed weights
  // (the conv's column groups, one tap), fp32 bias or null, output [n, C2], and whether that
  // output is fp32 (else the input's 16-bit type).
  const uint16_t* w2;
  const float* b2;
  void* y2;
  int y2_f32;
};

// One value of the output's own type (a residual element, here read where it is staged).
template <bool OUT16, int EK>
__device__ __forceinline__ float load_out(const void* p, int64_t i) {
  if constexpr (!OUT16) return static_cast<const float*>(p)[i];
  const uint16_t h = static_cast<const uint16_t*>(p)[i];
  if constexpr (EK == 0) return bf16_to_f32(h);
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// EPI = false is the plain convolution (bias only); EPI = true adds the activation, the
// residual and the group-norm statistics as the Epi arguments ask.  WIDE = true runs a layer
// wider than the tile (kch input chunks, gridDim.y output tiles); WIDE = false compiles the
// single chunk and tile in.  C2 > 0 makes a pair kernel: the plain convolution's output,
// rounded to the 16-bit type as a store would round it, stays in LDS and a k=1 layer of C2
// outputs (Epi w2, b2, y2) is applied to it; only that layer's output is written.
template <int CIN, int COUT, int NB, int WR, int WC, bool OUT16, int EK, bool EPI, bool WIDE,
          int C2 = 0>
__global__ __launch_bounds__(WR * WC * 64, 2) void k_subm_lds(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wp,
    const float* __restrict__ bias, const int32_t* __restrict__ perm,
    const uint32_t* __restrict__ bmask, const int32_t* __restrict__ gidx,
    const uint16_t* __restrict__ zrow, const int64_t* __restrict__ sched, int64_t npad,
    int kch, void* __restrict__ Y, Epi ep) {
  using C = LdsCfg<CIN, COUT, NB, WR, WC>;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM_BYTES];
  const char* sA0 = smem;
  const char* sA1 = smem + C::OFF_A1;
  int32_t* sG = reinterpret_cast<int32_t*>(smem + C::OFF_G);
  int32_t* sP = reinterpret_cast<int32_t*>(smem + C::OFF_P);

  // Wave index as a scalar: every per-block decision below is uniform across the wave and
  // compiles to scalar branches, and LDS destinations are scalar byte addresses.
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wr = wave / WC, wc = wave % WC;
  const uint32_t lds0 = lds_addr(smem);
  // A layer wider than the tile: this workgroup computes output columns [ct * COUT, (ct + 1)
  // * COUT) (ct = blockIdx.y of gridDim.y tiles), and each tap is summed over kch input
  // chunks of CIN channels, whose packed weights follow the tile's (k_pack_frag).
  if constexpr (!WIDE) kch = 1;
  const int ct = WIDE ? static_cast<int>(blockIdx.y) : 0;
  const int64_t xs = WIDE ? static_cast<int64_t>(CIN) * kch : CIN;
  if constexpr (WIDE) Wp += static_cast<int64_t>(ct) * kTaps * kch * (CIN * COUT);
  // Which tile this workgroup takes follows the plan's schedule.  Interleaved: the plan puts
  // the mask order's tiles in ascending cost (a tile of near-empty masks walks a tap or two,
  // the costliest all 27), so taking them from the last, the heavy tiles go first and the
  // workgroups dispatched last are the short ones.  Per XCD: consecutive workgroups go to the 8 XCDs in turn, and
  // XCD x takes the x-th contiguous eighth of a spatially ordered plan, in order.  Both
  // candidates' block masks are fetched while the schedule word is read, so choosing costs no
  // extra round trip.
  const int64_t tiles = gridDim.x;
  const int64_t t_il = tiles - 1 - blockIdx.x;
  const int64_t xcd = blockIdx.x % kXcds, per = tiles / kXcds, extra = tiles % kXcds;
  const int64_t t_px = xcd * per + (xcd < extra ? xcd : extra) + blockIdx.x / kXcds;
  const uint32_t bm_il = lane < NB ? bmask[t_il * NB + lane] : 0u;
  const uint32_t bm_px = lane < NB ? bmask[t_px * NB + lane] : 0u;
  const bool per_xcd = sched[0] == kSchedPerXcd;
  const int64_t tile = per_xcd ? t_px : t_il;
  const int64_t row0 = tile * (NB * 16);

  // Block tap masks: lane b holds block b's (for the per-tap block sets, one ballot each), and
  // their union U is the set of taps the tile walks.
  const uint32_t bmv = per_xcd ? bm_px : bm_il;
  uint32_t U = bmv;
#pragma unroll
  for (int off = 1; off < NB; off <<= 1) U |= __shfl_xor(U, off, 64);
  U = __builtin_amdgcn_readfirstlane(U);

  // Neighbour rows of the tile for every tap present -> sG[q][NB*16].  One 1 KB copy holds
  // G_TAPS_PER_COPY taps; copies are dealt to the waves round robin.
  {
    constexpr int TPC = C::G_TAPS_PER_COPY;
    const int sub = lane / (NB * 4);            // which tap of the copy this lane serves
    const int off = (lane % (NB * 4)) * 4;      // first of its 4 indices
    uint32_t rem = U;
    int q = 0, k = 0;
    while (rem) {
      int tt[TPC];
#pragma unroll
      for (int i = 0; i < TPC; ++i) {
        tt[i] = rem ? __builtin_ctz(rem) : -1;
        rem &= rem ? rem - 1 : 0u;
      }
      if ((k % C::WAVES) == wave) {
        int mine = -1;
#pragma unroll
        for (int i = 0; i < TPC; ++i)
          if (i == sub) mine = tt[i];
        if (mine >= 0)
          dma16(gidx + static_cast<int64_t>(mine) * npad + row0 + off,
                lds0 + C::OFF_G + q * (NB * 16 * 4));
      }
      q += TPC;
      ++k;
    }
  }
  // The tile's original row indices -> sP (read by the epilogue), by the last wave.
  if (wave == C::WAVES - 1 && lane < NB * 4) dma16(perm + row0 + lane * 4, lds0 + C::OFF_P);
  // Bias of this lane's columns, loaded now so the epilogue issues no global loads.
  f32x4_t bv[C::NCT];
#pragma unroll
  for (int c = 0; c < C::NCT; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i)  // bias needs only 4-byte alignment: scalar loads
      bv[c][i] = bias ? bias[ct * COUT + wc * C::CS + c * 16 + 4 * (lane >> 4) + i] : 0.f;
  // Pair kernels: the k=1 layer's weight fragments (its COUT inputs in KS2 k-steps, this
  // wave's NCT2 16-column tiles of its C2 outputs) and bias, loaded with the prologue.
  constexpr int NCT2 = C2 > 0 ? C2 / WC / 16 : 1;
  constexpr int KS2 = COUT / 32;
  bf16x8_t bw2[NCT2][KS2];
  f32x4_t bv2[NCT2];
  if constexpr (C2 > 0) {
    static_assert(OUT16 && !EPI && !WIDE && C2 % (16 * WC) == 0, "pair kernel shape");
    const uint16_t* w2 = ep.w2 + wc * (NCT2 * KS2 * 512) + lane * 8;
#pragma unroll
    for (int c = 0; c < NCT2; ++c)
#pragma unroll
      for (int s2 = 0; s2 < KS2; ++s2)
        bw2[c][s2] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const u32x4_t*>(w2 + (c * KS2 + s2) * 512));
#pragma unroll
    for (int c = 0; c < NCT2; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bv2[c][i] = ep.b2 ? ep.b2[wc * (C2 / WC) + c * 16 + 4 * (lane >> 4) + i] : 0.f;
  }
  wait_vm_lgkm0();
  __builtin_amdgcn_s_barrier();

  // Output staging geometry (used by the epilogue below).
  constexpr int ESZ = OUT16 ? 2 : 4;
  constexpr int ROWB = COUT * ESZ;  // a row of the tile (staged)
  constexpr int CHUNKS = ROWB / 16;
  // Output and residual rows in memory: all gridDim.y tiles wide; this tile's part.
  const int64_t yrowb = WIDE ? static_cast<int64_t>(ROWB) * gridDim.y : ROWB;
  char* const ycol = static_cast<char*>(Y) + static_cast<int64_t>(ct) * ROWB;
  const char* const rcol =
      ep.res ? static_cast<const char*>(ep.res) + static_cast<int64_t>(ct) * ROWB : nullptr;
  constexpr int SWM = (CHUNKS < 16 ? CHUNKS : 16) - 1;
  constexpr int BPP_RAW = C::STAGE_BYTES / (16 * ROWB);
  // Blocks per pass: the largest power of two that fits (NB is a power of two, so every pass
  // is full and covers rows [p0*16, (p0+BPP)*16) of the tile exactly).
  constexpr int BPP = BPP_RAW >= NB ? NB : BPP_RAW >= 8 ? 8 : BPP_RAW >= 4 ? 4 : BPP_RAW >= 2 ? 2 : 1;
  static_assert(BPP_RAW >= 1 && NB % BPP == 0, "output staging space");
  // A pass stages rows [p0 * 16, (p0 + BPP) * 16) of the tile: the staging tile and the row
  // ids it reads (sP[p0 * 16 + row], row < BPP * 16) stay in range for every pass.
  static_assert(BPP * 16 * ROWB <= C::STAGE_BYTES && (NB / BPP) * BPP * 16 == NB * 16,
                "staging passes inside the arena and the tile");
  // Residual rows: when the tile leaves in one pass and each thread's share is at most 8
  // pieces, they are loaded now, in flight with the first gather, and held in registers.
  constexpr int RPT = BPP * 16 * CHUNKS / C::THREADS;
  constexpr bool RPRE = EPI && BPP == NB && RPT >= 1 && RPT <= 8 &&
                        BPP * 16 * CHUNKS % C::THREADS == 0;
  u32x4_t rpre[RPRE ? RPT : 1];
  if constexpr (RPRE) {
    if (ep.res) {
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const int idx = threadIdx.x + k * C::THREADS;
        const int row = idx / CHUNKS, ch = idx % CHUNKS;
        const int32_t o = sP[row];
        rpre[k] = o >= 0 ? *reinterpret_cast<const u32x4_t*>(rcol + static_cast<int64_t>(o) * yrowb +
                                                              ch * 16)
                         : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }

  f32x4_t acc[C::BPW][C::NCT];
#pragma unroll
  for (int bl = 0; bl < C::BPW; ++bl)
#pragma unroll
    for (int c = 0; c < C::NCT; ++c) acc[bl][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (U) {
    // Even stages live in (sA0, bw0), odd ones in (sA1, bw1).  Per stage: wait until
    // this wave's copies and loads of the stage have landed (nothing newer is outstanding at
    // that point), barrier, issue the next stage, then run the matrix cores on this one.
    bf16x8_t bw0[C::NCT][C::KS], bw1[C::NCT][C::KS];
    uint32_t aoff[C::KS];
    a_frag_offsets<CIN>(lane, aoff);
    // Stages walk (tap, input chunk) pairs: taps in ascending order, each tap's chunks in
    // order.  q counts the taps (their slot of neighbour rows), kc the chunk.
    uint32_t rem = U;
    int t_cur = __builtin_ctz(rem);
    rem &= rem - 1;
    int q = 0, kc = 0;
    uint32_t act = block_taps(bmv, t_cur);
    load_weights<CIN, COUT, NB, WR, WC>(t_cur * kch, Wp, wc, lane, bw0);
    issue_gather<CIN, COUT, NB, WR, WC>(0, act, X, xs, zrow, sG, lds0, wave, lane);
    // The stage after the current one: the tap's next chunk, else the next tap's first
    // (t_next = -1 when none is left).  Uniform across the workgroup.
    auto next = [&](int& t_next, int& kc_next, int& q_next, uint32_t& act_next)
        __attribute__((always_inline)) {
      if (WIDE && kc + 1 < kch) {
        t_next = t_cur, kc_next = kc + 1, q_next = q, act_next = act;
      } else if (rem) {
        t_next = __builtin_ctz(rem), kc_next = 0, q_next = q + 1;
        act_next = block_taps(bmv, t_next);
      } else {
        t_next = -1, kc_next = 0, q_next = q, act_next = 0;
      }
    };
    while (true) {
      wait_vm_lgkm0();
      __builtin_amdgcn_s_barrier();
      // The barrier builtin does not order memory for the compiler: keep the LDS reads below
      // after it.
      asm volatile("" ::: "memory");
      int t_next, kc_next, q_next;
      uint32_t act_next;
      next(t_next, kc_next, q_next, act_next);
      bf16x8_t a0[C::KS];
      read_first<CIN, COUT, NB, WR, WC>(sA0, aoff, wr, a0);
      if (t_next >= 0) {
        load_weights<CIN, COUT, NB, WR, WC>(t_next * kch + kc_next, Wp, wc, lane, bw1);
        issue_gather<CIN, COUT, NB, WR, WC>(q_next, act_next, X + (WIDE ? kc_next * CIN : 0), xs, zrow, sG,
                                            lds0 + C::OFF_A1, wave, lane);
      }
      compute_stage<CIN, COUT, NB, WR, WC, EK>(act, sA0, bw0, aoff, wr, a0, acc);
      if (t_next < 0) break;
      if (kc_next == 0) rem &= rem - 1;
      t_cur = t_next, kc = kc_next, q = q_next, act = act_next;
      wait_vm_lgkm0();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      next(t_next, kc_next, q_next, act_next);
      read_first<CIN, COUT, NB, WR, WC>(sA1, aoff, wr, a0);
      if (t_next >= 0) {
        load_weights<CIN, COUT, NB, WR, WC>(t_next * kch + kc_next, Wp, wc, lane, bw0);
        issue_gather<CIN, COUT, NB, WR, WC>(q_next, act_next, X + (WIDE ? kc_next * CIN : 0), xs, zrow, sG,
                                            lds0, wave, lane);
      }
      compute_stage<CIN, COUT, NB, WR, WC, EK>(act, sA1, bw1, aoff, wr, a0, acc);
      if (t_next < 0) break;
      if (kc_next == 0) rem &= rem - 1;
      t_cur = t_next, kc = kc_next, q = q_next, act = act_next;
    }
  }

  // Epilogue.  Every wave is past its last LDS read of the gather buffers after this barrier,
  // and nothing is outstanding (which also lets the compiler drop waits for weight loads it
  // cannot prove were skipped on the last tap).
  wait_vm_lgkm0();
  __builtin_amdgcn_s_barrier();
  // Output rows are staged in LDS over the gather buffers and indices, BPP blocks at a time,
  // 16-byte chunks XOR-swizzled by row; then every thread writes 16-byte pieces of whole
  // rows to their original index.
  char* sOut = smem;
  // Group-norm statistics of the stored values: each lane sums its own columns (NCT of
  // them) over the rows it stages that hold a site.
  f32x4_t csum[C::NCT], csq[C::NCT];
#pragma unroll
  for (int c = 0; c < C::NCT; ++c) csum[c] = csq[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t site_rows = EPI ? ep.rows - row0 : 0;  // rows of this tile holding a site
  // The epilogue, one copy per combination of its options (activation, residual, group-norm
  // statistics), chosen once per tile, so that no element pays a branch for them.
  auto epilogue = [&](auto act_c, auto res_c, auto gn_c) __attribute__((always_inline)) {
    constexpr int ACT = decltype(act_c)::value;
    constexpr bool RES = decltype(res_c)::value;
    constexpr bool GN = decltype(gn_c)::value;
#pragma unroll
    for (int p0 = 0; p0 < NB; p0 += BPP) {
      if constexpr (RES) {
        // Residual rows of this pass as whole 16-byte pieces in the staging tile (the layout
        // the output takes there); each value is then added by the lane that stages the output
        // value at the same place.
        if constexpr (RPRE) {
#pragma unroll
          for (int k = 0; k < RPT; ++k) {
            const int idx = threadIdx.x + k * C::THREADS;
            const int row = idx / CHUNKS, ch = idx % CHUNKS;
            *reinterpret_cast<u32x4_t*>(sOut + row * ROWB + ((ch ^ (row & SWM)) << 4)) = rpre[k];
          }
        } else {
          constexpr int RPIECES = BPP * 16 * CHUNKS;
#pragma unroll 4
          for (int idx = threadIdx.x; idx < RPIECES; idx += C::THREADS) {
            const int row = idx / CHUNKS, ch = idx % CHUNKS;
            const int32_t o = sP[p0 * 16 + row];
            if (o < 0) continue;
            *reinterpret_cast<u32x4_t*>(sOut + row * ROWB + ((ch ^ (row & SWM)) << 4)) =
                *reinterpret_cast<const u32x4_t*>(rcol + static_cast<int64_t>(o) * yrowb + ch * 16);
          }
        }
        wait_vm_lgkm0();
        __builtin_amdgcn_s_barrier();
      }
      // Stage this pass's outputs (the epilogue's options are compile-time here).
#pragma unroll
      for (int bl = 0; bl < C::BPW; ++bl) {
        const int b = bl * WR + wr;
        if (b < p0 || b >= p0 + BPP) continue;
#pragma unroll
        for (int c = 0; c < C::NCT; ++c) {
          // This lane's piece: channels col .. col + 3 of one site row.
          const int col = wc * C::CS + c * 16 + 4 * (lane >> 4);
          const int row = (b - p0) * 16 + (lane & 15);
          const int byte = col * ESZ;
          char* dst = sOut + row * ROWB + (((byte >> 4) ^ (row & SWM)) << 4) + (byte & 15);
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = apply_act(acc[bl][c][i] + bv[c][i], ACT);
          if constexpr (RES) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if constexpr (!OUT16)
                v[i] += reinterpret_cast<const float*>(dst)[i];
              else if constexpr (EK == 0)
                v[i] += bf16_to_f32(reinterpret_cast<const uint16_t*>(dst)[i]);
              else
                v[i] += static_cast<float>(reinterpret_cast<const _Float16*>(dst)[i]);
            }
          }
          float stored[4] = {v[0], v[1], v[2], v[3]};
          if constexpr (OUT16) {
            uint16_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              h[i] = to16<EK>(v[i]);
              if constexpr (GN)
                stored[i] = EK == 0 ? bf16_to_f32(h[i])
                                    : static_cast<float>(__builtin_bit_cast(_Float16, h[i]));
            }
            *reinterpret_cast<uint2*>(dst) =
                make_uint2(h[0] | (static_cast<uint32_t>(h[1]) << 16),
                           h[2] | (static_cast<uint32_t>(h[3]) << 16));
          } else {
            *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{v[0], v[1], v[2], v[3]};
          }
          if constexpr (GN) {
            if (b * 16 + (lane & 15) < site_rows) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                csum[c][i] += stored[i];
                csq[c][i] = fmaf(stored[i], stored[i], csq[c][i]);
              }
            }
          }
        }
      }
      wait_vm_lgkm0();
      __builtin_amdgcn_s_barrier();
      constexpr int PIECES = BPP * 16 * CHUNKS;
#pragma unroll 4
      for (int idx = threadIdx.x; idx < PIECES; idx += C::THREADS) {
        const int row = idx / CHUNKS, ch = idx % CHUNKS;
        const int32_t o = sP[p0 * 16 + row];
        if (o < 0) continue;
        const u32x4_t v =
            *reinterpret_cast<const u32x4_t*>(sOut + row * ROWB + ((ch ^ (row & SWM)) << 4));
        // Non-temporal: the output is not read again here, and streaming it past the caches
        // keeps them for the feature rows other tiles gather (about 2% at 128^3, 10%).
        __builtin_nontemporal_store(
            v, reinterpret_cast<u32x4_t*>(ycol + static_cast<int64_t>(o) * yrowb + ch * 16));
      }
      if (p0 + BPP < NB) {
        wait_vm_lgkm0();
        __builtin_amdgcn_s_barrier();
      }
    }
  };
  using A0 = std::integral_constant<int, SSC_ACT_NONE>;
  using A1 = std::integral_constant<int, SSC_ACT_RELU>;
  using A2 = std::integral_constant<int, SSC_ACT_SILU>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  if constexpr (C2 > 0) {
    static_assert(BPP == NB, "the pair's intermediate tile stays in LDS whole");
    // 1. The convolution's tile plus bias, rounded to the 16-bit type (the value its 16-bit
    //    store would hold), into the staging tile: rows of COUT channels, 16-byte chunks
    //    swizzled by row.
#pragma unroll
    for (int bl = 0; bl < C::BPW; ++bl) {
      const int b = bl * WR + wr;
#pragma unroll
      for (int c = 0; c < C::NCT; ++c) {
        const int col = wc * C::CS + c * 16 + 4 * (lane >> 4);
        const int row = b * 16 + (lane & 15);
        const int byte = col * 2;
        uint16_t h[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = to16<EK>(acc[bl][c][i] + bv[c][i]);
        *reinterpret_cast<uint2*>(sOut + row * ROWB + (((byte >> 4) ^ (row & SWM)) << 4) +
                                  (byte & 15)) =
            make_uint2(h[0] | (static_cast<uint32_t>(h[1]) << 16),
                       h[2] | (static_cast<uint32_t>(h[3]) << 16));
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
    __builtin_amdgcn_s_barrier();
    // 2. The k=1 layer on the staged rows, the same transposed product as the convolution's
    //    (lane l: row l & 15, its k-values at chunk (l >> 4) + 4 s).
    f32x4_t acc2[C::BPW][NCT2];
#pragma unroll
    for (int bl = 0; bl < C::BPW; ++bl) {
      const int row = (bl * WR + wr) * 16 + (lane & 15);
      bf16x8_t a2[KS2];
#pragma unroll
      for (int s2 = 0; s2 < KS2; ++s2)
        a2[s2] = lds_read16(sOut + row * ROWB + ((((lane >> 4) + 4 * s2) ^ (row & SWM)) << 4));
#pragma unroll
      for (int c = 0; c < NCT2; ++c) {
        acc2[bl][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < KS2; ++s2)
          acc2[bl][c] = mfma16x16x32<EK>(bw2[c][s2], a2[s2], acc2[bl][c]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();  // every wave is done reading the intermediate tile
    // 3. The k=1 output (plus its bias), staged and written as whole rows like the
    //    convolution's, BPP2 blocks per pass.
    auto store2 = [&](auto f32_c) __attribute__((always_inline)) {
      constexpr bool F32 = decltype(f32_c)::value;
      constexpr int ROWB2 = C2 * (F32 ? 4 : 2);
      constexpr int CHUNKS2 = ROWB2 / 16;
      constexpr int SWM2 = (CHUNKS2 < 16 ? CHUNKS2 : 16) - 1;
      constexpr int RAW2 = C::STAGE_BYTES / (16 * ROWB2);
      constexpr int BPP2 = RAW2 >= NB ? NB : RAW2 >= 8 ? 8 : RAW2 >= 4 ? 4 : RAW2 >= 2 ? 2 : 1;
      static_assert(RAW2 >= 1 && NB % BPP2 == 0 && BPP2 * 16 * ROWB2 <= C::STAGE_BYTES,
                    "pair output staging");
      char* y2 = static_cast<char*>(ep.y2);
#pragma unroll
      for (int p0 = 0; p0 < NB; p0 += BPP2) {
#pragma unroll
        for (int bl = 0; bl < C::BPW; ++bl) {
          const int b = bl * WR + wr;
          if (b < p0 || b >= p0 + BPP2) continue;
#pragma unroll
          for (int c = 0; c < NCT2; ++c) {
            const int col = wc * (C2 / WC) + c * 16 + 4 * (lane >> 4);
            const int row = (b - p0) * 16 + (lane & 15);
            const int byte = col * (F32 ? 4 : 2);
            char* dst = sOut + row * ROWB2 + (((byte >> 4) ^ (row & SWM2)) << 4) + (byte & 15);
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc2[bl][c][i] + bv2[c][i];
            if constexpr (F32) {
              *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{v[0], v[1], v[2], v[3]};
            } else {
              *reinterpret_cast<uint2*>(dst) =
                  make_uint2(to16<EK>(v[0]) | (static_cast<uint32_t>(to16<EK>(v[1])) << 16),
                             to16<EK>(v[2]) | (static_cast<uint32_t>(to16<EK>(v[3])) << 16));
            }
          }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        constexpr int PIECES2 = BPP2 * 16 * CHUNKS2;
#pragma unroll 4
        for (int idx = threadIdx.x; idx < PIECES2; idx += C::THREADS) {
          const int row = idx / CHUNKS2, ch = idx % CHUNKS2;
          const int32_t o = sP[p0 * 16 + row];
          if (o < 0) continue;
          const u32x4_t v =
              *reinterpret_cast<const u32x4_t*>(sOut + row * ROWB2 + ((ch ^ (row & SWM2)) << 4));
          __builtin_nontemporal_store(
              v, reinterpret_cast<u32x4_t*>(y2 + static_cast<int64_t>(o) * ROWB2 + ch * 16));
        }
        if (p0 + BPP2 < NB) {
          wait_vm_lgkm0();
          __builtin_amdgcn_s_barrier();
        }
      }
    };
    if (ep.y2_f32)
      store2(T_{});
    else
      store2(F_{});
  } else if constexpr (!EPI) {
    epilogue(A0{}, F_{}, F_{});
  } else {
    switch (ep.act * 4 + (ep.res ? 2 : 0) + (ep.gn ? 1 : 0)) {
      case 0: epilogue(A0{}, F_{}, F_{}); break;
      case 1: epilogue(A0{}, F_{}, T_{}); break;
      case 2: epilogue(A0{}, T_{}, F_{}); break;
      case 3: epilogue(A0{}, T_{}, T_{}); break;
      case 4: epilogue(A1{}, F_{}, F_{}); break;
      case 5: epilogue(A1{}, F_{}, T_{}); break;
      case 6: epilogue(A1{}, T_{}, F_{}); break;
      case 7: epilogue(A1{}, T_{}, T_{}); break;
      case 8: epilogue(A2{}, F_{}, F_{}); break;
      case 9: epilogue(A2{}, F_{}, T_{}); break;
      case 10: epilogue(A2{}, T_{}, F_{}); break;
      default: epilogue(A2{}, T_{}, T_{}); break;
    }
  }
  if (EPI && ep.gn) {
    // Fixed-order reduction, every step a butterfly (all lanes end with the same sums): each
    // lane holds four consecutive channels of one site row; first over the 16 site rows of a
    // tile (lane bits 0-3), then over the gs channels of a group: within the lane's four (gs <= 4)
    // and over lane bits 4, 5 (gs = 8, 16; a group never leaves a 16-column tile).  The tile's
    // count is its rows that hold a site.  One or two 128-row slots per tile.
    const int groups = ep.gn_groups, gs = COUT / groups;
    const int per_lane = gs >= 4 ? 1 : 4 / gs;  // groups among a lane's four channels
    float S[C::NCT][4], Q[C::NCT][4];
#pragma unroll
    for (int c = 0; c < C::NCT; ++c) {
#pragma unroll
      for (int m = 1; m < 16; m <<= 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          csum[c][i] += __shfl_xor(csum[c][i], m, 64);
          csq[c][i] += __shfl_xor(csq[c][i], m, 64);
        }
      if (gs == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[c][i] = csum[c][i], Q[c][i] = csq[c][i];
      } else if (gs == 2) {
        S[c][0] = csum[c][0] + csum[c][1];
        Q[c][0] = csq[c][0] + csq[c][1];
        S[c][1] = csum[c][2] + csum[c][3];
        Q[c][1] = csq[c][2] + csq[c][3];
      } else {
        S[c][0] = (csum[c][0] + csum[c][1]) + (csum[c][2] + csum[c][3]);
        Q[c][0] = (csq[c][0] + csq[c][1]) + (csq[c][2] + csq[c][3]);
        for (int m = 16; m < 16 * (gs / 4); m <<= 1) {
          S[c][0] += __shfl_xor(S[c][0], m, 64);
          Q[c][0] += __shfl_xor(Q[c][0], m, 64);
        }
      }
    }
    const float cnt = static_cast<float>(
        site_rows < 0 ? 0 : site_rows > NB * 16 ? NB * 16 : site_rows) * static_cast<float>(gs);
    constexpr int SLOTS = NB * 16 / 128;
    float4* part = reinterpret_cast<float4*>(ep.gn) + tile * SLOTS * groups;
    const int quad = lane >> 4;  // channels 4 quad .. +3 of each 16-column tile
    const bool leader = (lane & 15) == 0 && (gs < 8 || (quad & (gs / 4 - 1)) == 0);
    if constexpr (WR == 1) {
      if (leader) {
#pragma unroll
        for (int c = 0; c < C::NCT; ++c) {
          const int g0 = (wc * C::CS + c * 16 + 4 * quad) / gs;
          for (int k = 0; k < per_lane; ++k) {
            part[g0 + k] = make_float4(cnt, S[c][k], Q[c][k], 0.f);
#pragma unroll
            for (int sl = 1; sl < SLOTS; ++sl)
              part[sl * groups + g0 + k] = make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
      }
    } else {
      // Waves that share columns (WR of them) add their sums in wave-row order.
      constexpr int GN_OFF = BPP * 16 * ROWB;
      static_assert(GN_OFF + WR * COUT * 2 * 4 <= C::OFF_P, "group-norm reduction space");
      float* red = reinterpret_cast<float*>(smem + GN_OFF);
      if (leader) {
#pragma unroll
        for (int c = 0; c < C::NCT; ++c) {
          const int g0 = (wc * C::CS + c * 16 + 4 * quad) / gs;
          for (int k = 0; k < per_lane; ++k) {
            red[(wr * groups + g0 + k) * 2] = S[c][k];
            red[(wr * groups + g0 + k) * 2 + 1] = Q[c][k];
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); the row stores may still be in flight
      __builtin_amdgcn_s_barrier();
      for (int g = threadIdx.x; g < groups; g += C::THREADS) {
        float Ssum = 0.f, Qsum = 0.f;
        for (int r = 0; r < WR; ++r) {
          Ssum += red[(r * groups + g) * 2];
          Qsum += red[(r * groups + g) * 2 + 1];
        }
        part[g] = make_float4(cnt, Ssum, Qsum, 0.f);
#pragma unroll
        for (int sl = 1; sl < SLOTS; ++sl) part[sl * groups + g] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
}

template <typename T>
__device__ __forceinline__ float load_feat(const T* p);
template <>
__device__ __forceinline__ float load_feat<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_feat<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <>
__device__ __forceinline__ float load_feat<_Float16>(const _Float16* p) {
  return static_cast<float>(*p);
}

// Vector-ALU path for any shape and for fp32 inputs: one thread per (sorted row, column),
// fp32 fused multiply-add over taps in ascending order, then channels in ascending order.
// taps = 27 with a plan; taps = 1 (DENSE) for the k=1 linear map.
template <typename T, bool DENSE>
__global__ __launch_bounds__(256) void k_conv_valu(const T* __restrict__ X, const T* __restrict__ W,
                                                   const float* __restrict__ bias,
                                                   const int32_t* __restrict__ perm,
                                                   const int32_t* __restrict__ gidx, int64_t npad,
                                                   int64_t n, int cin, int cout,
                                                   void* __restrict__ Y, int out_kind, int act,
                                                   const void* res) {
  const int64_t rows = DENSE ? n : npad;
  const int64_t total = rows * cout;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += stride) {
    const int64_t r = g / cout;
    const int o = static_cast<int>(g - r * cout);
    const int64_t orow = DENSE ? r : perm[r];
    if (orow < 0) continue;
    float acc = 0.f;
    constexpr int taps = DENSE ? 1 : kTaps;
    // All taps' neighbour rows first (independent loads in flight together), then the taps in
    // ascending order; the channel loop is unrolled so its loads overlap too (the sum keeps
    // its order: taps, then channels, ascending).
    int32_t js[taps];
#pragma unroll
    for (int t = 0; t < taps; ++t)
      js[t] = DENSE ? static_cast<int32_t>(r) : gidx[static_cast<int64_t>(t) * npad + r];
#pragma unroll
    for (int t = 0; t < taps; ++t) {
      const int64_t j = js[t];
      if (j < 0) continue;
      const T* xr = X + j * cin;
      const T* wt = W + static_cast<int64_t>(t) * cin * cout + o;
#pragma unroll 8
      for (int c = 0; c < cin; ++c)
        acc = fmaf(load_feat<T>(xr + c), load_feat<T>(wt + static_cast<int64_t>(c) * cout), acc);
    }
    float v = apply_act(acc + (bias ? bias[o] : 0.f), act);
    if (res) {
      const int64_t k = orow * cout + o;
      v += out_kind == SSC_BF16  ? bf16_to_f32(static_cast<const uint16_t*>(res)[k])
           : out_kind == SSC_F16 ? static_cast<float>(static_cast<const _Float16*>(res)[k])
                                 : static_cast<const float*>(res)[k];
    }
    if (out_kind == SSC_BF16)
      static_cast<uint16_t*>(Y)[orow * cout + o] = f32_to_bf16_rne(v);
    else if (out_kind == SSC_F16)
      static_cast<uint16_t*>(Y)[orow * cout + o] = to16<1>(v);
    else
      static_cast<float*>(Y)[orow * cout + o] = v;
  }
}

// ------------------------------------------------------------------------------------------
// k=1 layer (per-site linear map) on bf16 features: a persistent streaming kernel.
//
// The map reads each feature row once and writes each output row once, so it is bound by
// HBM, not by the matrix cores.  Each workgroup keeps its column slice of W as B fragments in
// VGPRs for its whole life and walks tiles of TR contiguous rows (tile, tile + gridDim.x, ...).
// Per tile: the next tile's rows are copied into the other LDS buffer (direct global->LDS
// loads, whole 1 KB copies) while the matrix cores work on this one; the outputs plus bias
// are staged in LDS and leave as contiguous 16-byte stores of whole rows.
// The only vector-memory operations in the loop are those copies, the residual's copies and
// the output stores, and they retire in issue order, so "this tile's copies have landed" is
// "at most STORES (the previous tile's stores, issued after them) are outstanding": the loop
// waits for exactly that, not for the stores.  A residual is copied the same way, straight
// into the output staging tile (before the next tile's rows, so waiting for it leaves those
// in flight), and added where each output is staged; a per-element global load there would
// make the compiler drain every copy in flight before it.  Only the last tile of the layer
// can be partial, and it is the last tile its workgroup handles; rows past n are copied from
// row n-1 and never stored.
// ------------------------------------------------------------------------------------------
template <int CIN, int COUT, bool OUT16>
struct LinCfg {
  static constexpr int ESZ = OUT16 ? 2 : 4;
  static constexpr int ROWB = COUT * ESZ;                  // output bytes per row
  static constexpr int TR = ROWB >= 64 ? 64 : 128;         // rows per tile
  static constexpr int NB = TR / 16;
  static constexpr int WC = COUT >= 64 ? 4 : COUT / 16;
  static constexpr int WR = 4 / WC;
  using C = LdsCfg<CIN, COUT, NB, WR, WC>;
  static constexpr int XBUF = TR * CIN * 2;                // one tile of bf16 rows
  static constexpr int OBUF = TR * ROWB;                   // one tile of output rows
  static constexpr int SMEM = 2 * XBUF + OBUF;
  static constexpr int COPIES = XBUF / 1024;               // 1 KB copies per tile
  static constexpr int CPW = COPIES / C::WAVES;
  static constexpr int RPI = 512 / CIN;                    // rows per copy
  static constexpr int CHUNKS = ROWB / 16;
  static constexpr int SWM = (CHUNKS < 16 ? CHUNKS : 16) - 1;
  static constexpr int STORES = OBUF / 16 / C::THREADS;    // 16-byte stores per thread
  static_assert(COPIES % C::WAVES == 0 && OBUF % (16 * C::THREADS) == 0, "tile shape");
  static_assert(STORES >= 1 && STORES <= 63, "vmcnt range");
};

// s_waitcnt vmcnt(N) lgkmcnt(0), N < 64 (gfx9 encoding: vmcnt[3:0] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vm_n_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}

template <int CIN, int COUT, bool OUT16>
__device__ __forceinline__ void linear_copies(int64_t tile, int64_t n,
                                              const uint16_t* __restrict__ X, char* buf,
                                              int wave, int lane) {
  using L = LinCfg<CIN, COUT, OUT16>;
  constexpr int CPR = CIN / 8;
  const int rsub = lane / CPR, phys = lane % CPR;
#pragma unroll
  for (int i = 0; i < L::CPW; ++i) {
    const int k = i * L::C::WAVES + wave;
    const int r = k * L::RPI + rsub;                       // row of the tile
    int64_t g = tile * L::TR + r;
    g = g < n ? g : n - 1;
    const int chunk = phys ^ swz<CPR>(r & 15);
    dma16(X + g * CIN + chunk * 8, lds_addr(buf + k * 1024));
  }
}

// The residual rows of a tile into the output staging tile, in its swizzled layout: lane l of
// copy j fills 16 bytes at j * 1024 + 16 l, i.e. physical chunk p of some row, so it reads
// that row's logical chunk p ^ (row & SWM).
template <int CIN, int COUT, bool OUT16>
__device__ __forceinline__ void residual_copies(int64_t row0, int64_t n, const void* res,
                                                char* sOut, int wave, int lane) {
  using L = LinCfg<CIN, COUT, OUT16>;
  constexpr int RCPW = L::OBUF / 1024 / L::C::WAVES;
  static_assert(L::OBUF % (1024 * L::C::WAVES) == 0, "residual copy shape");
#pragma unroll
  for (int i = 0; i < RCPW; ++i) {
    const int j = i * L::C::WAVES + wave;
    const int o = j * 1024 + lane * 16;
    const int row = o / L::ROWB, p = (o % L::ROWB) >> 4;
    const int ch = p ^ (row & L::SWM);
    int64_t g = row0 + row;
    g = g < n ? g : n - 1;
    dma16(static_cast<const char*>(res) + g * L::ROWB + ch * 16, lds_addr(sOut + j * 1024));
  }
}

template <int CIN, int COUT, bool OUT16, int EK, bool EPI>
__global__ __launch_bounds__(256, 2) void k_linear_stream(const uint16_t* __restrict__ X,
                                                          const uint16_t* __restrict__ Wp,
                                                          const float* __restrict__ bias,
                                                          int64_t n, void* __restrict__ Y,
                                                          int act, const void* res) {
  using L = LinCfg<CIN, COUT, OUT16>;
  using C = typename L::C;
  __shared__ __attribute__((aligned(1024))) char smem[L::SMEM];
  char* sX0 = smem;
  char* sX1 = smem + L::XBUF;
  char* sOut = smem + 2 * L::XBUF;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave / L::WC, wc = wave % L::WC;
  const int64_t tiles = (n + L::TR - 1) / L::TR;
  int64_t tile = blockIdx.x;
  if (tile >= tiles) return;

  bf16x8_t bw[C::NCT][C::KS];
  load_weights<CIN, COUT, L::NB, L::WR, L::WC>(0, Wp, wc, lane, bw);
  float bv[C::NCT];
#pragma unroll
  for (int c = 0; c < C::NCT; ++c) bv[c] = bias ? bias[wc * C::CS + c * 16 + (lane & 15)] : 0.f;
  uint32_t aoff[C::KS];
  a_frag_offsets<CIN>(lane, aoff);
  // Weights and bias are in registers before the loop: inside it nothing waits for them, so
  // the compiler has no reason to drain the copies in flight.
  wait_vm_lgkm0();

  linear_copies<CIN, COUT, OUT16>(tile, n, X, sX0, wave, lane);
  for (int k = 0; tile < tiles; tile += gridDim.x, ++k) {
    if (k == 0)
      wait_vm_lgkm0();
    else
      wait_vm_n_lgkm0<L::STORES>();
    __builtin_amdgcn_s_barrier();
    char* cur = (k & 1) ? sX1 : sX0;
    const int64_t row0 = tile * L::TR;
    // The staging tile is free: the previous tile's reads of it finished before the barrier.
    if constexpr (EPI)
      if (res) residual_copies<CIN, COUT, OUT16>(row0, n, res, sOut, wave, lane);
    const int64_t next = tile + gridDim.x;
    if (next < tiles) linear_copies<CIN, COUT, OUT16>(next, n, X, (k & 1) ? sX0 : sX1, wave, lane);

    f32x4_t acc[C::BPW][C::NCT];
#pragma unroll
    for (int bl = 0; bl < C::BPW; ++bl) {
      const char* blk = cur + (bl * L::WR + wr) * (C::A_BLOCK * 2);
      bf16x8_t a[C::KS];
#pragma unroll
      for (int s = 0; s < C::KS; ++s) a[s] = lds_read16(blk + aoff[s]);
#pragma unroll
      for (int c = 0; c < C::NCT; ++c) {
        acc[bl][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < C::KS; ++s)
          acc[bl][c] = mfma16x16x32<EK>(a[s], bw[c][s], acc[bl][c]);
      }
    }
    // Stage the outputs: act(acc + bias) + residual (16-byte chunks XOR-swizzled by row).  The
    // residual copies were issued before the next tile's, so these are waited for alone.
    if constexpr (EPI) {
      if (res) {
        if (next < tiles)
          wait_vm_n_lgkm0<L::CPW>();
        else
          wait_vm_lgkm0();
        __builtin_amdgcn_s_barrier();
      }
    }
#pragma unroll
    for (int bl = 0; bl < C::BPW; ++bl) {
      const int b = bl * L::WR + wr;
#pragma unroll
      for (int c = 0; c < C::NCT; ++c) {
        const int col = wc * C::CS + c * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = b * 16 + (lane >> 4) * 4 + i;
          const int byte = col * L::ESZ;
          char* dst = sOut + row * L::ROWB + (((byte >> 4) ^ (row & L::SWM)) << 4) + (byte & 15);
          float v = acc[bl][c][i] + bv[c];
          if constexpr (EPI) {
            v = apply_act(v, act);
            if (res) v += load_out<OUT16, EK>(dst, 0);  // the staged residual value
          }
          if (OUT16)
            *reinterpret_cast<uint16_t*>(dst) = to16<EK>(v);
          else
            *reinterpret_cast<float*>(dst) = v;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int it = 0; it < L::STORES; ++it) {
      const int idx = threadIdx.x + it * C::THREADS;
      const int row = idx / L::CHUNKS, ch = idx % L::CHUNKS;
      const u32x4_t v =
          *reinterpret_cast<const u32x4_t*>(sOut + row * L::ROWB + ((ch ^ (row & L::SWM)) << 4));
      if (row0 + row < n)
        st16(reinterpret_cast<u32x4_t*>(static_cast<char*>(Y) + (row0 + row) * L::ROWB + ch * 16), v);
    }
  }
}

using LinFn = void (*)(const uint16_t*, const uint16_t*, const float*, int64_t, void*, int,
                      const void*);
using LdsFn = void (*)(const uint16_t*, const uint16_t*, const float*, const int32_t*,
                       const uint32_t*, const int32_t*, const uint16_t*, const int64_t*,
                       int64_t, int, void*, Epi);

// k=1 streaming kernel for the channel counts the matrix-core path is built for.
template <int CI, int CO, bool O16, int EK>
LinFn linear_fn(bool epi) {
  return epi ? k_linear_stream<CI, CO, O16, EK, true> : k_linear_stream<CI, CO, O16, EK, false>;
}

LinFn pick_linear(int cin, int cout, bool out16, int ek, int* wc_groups, int* rows_per_tile,
                  bool epi) {
#define SSC_CASE(CI, CO)                                                                      \
  if (cin == CI && cout == CO) {                                                              \
    *wc_groups = LinCfg<CI, CO, false>::WC;                                                   \
    *rows_per_tile = out16 ? LinCfg<CI, CO, true>::TR : LinCfg<CI, CO, false>::TR;            \
    if (ek == 1) return out16 ? linear_fn<CI, CO, true, 1>(epi) : linear_fn<CI, CO, false, 1>(epi); \
    return out16 ? linear_fn<CI, CO, true, 0>(epi) : linear_fn<CI, CO, false, 0>(epi);        \
  }
  SSC_CASE(32, 16) SSC_CASE(32, 32) SSC_CASE(32, 64) SSC_CASE(32, 128)
  SSC_CASE(64, 16) SSC_CASE(64, 32) SSC_CASE(64, 64) SSC_CASE(64, 128)
  SSC_CASE(128, 16) SSC_CASE(128, 32) SSC_CASE(128, 64) SSC_CASE(128, 128)
#undef SSC_CASE
  return nullptr;
}

// k=3 pipelined kernel: 4 waves as WR x WC, tile of NB = 8 blocks.  At Cin = 128 that keeps
// two gather stages plus the indices under 80 KB of LDS, so two workgroups share a CU;
// narrower rows leave room for more, and at Cin = 32 the extra workgroups keep more gathers
// in flight than 16-block tiles did (512^3 surface, C 32: 159 -> 130 us).
template <int CI, int CO>
struct LdsPick {
  static constexpr int WC = CO >= 64 ? 4 : CO / 16;
  static constexpr int WR = 4 / WC;
  static constexpr int NB = 8;
  // The plan orders whole tiles of this many rows by cost.
  static_assert(NB * 16 == kTileRows, "tile rows of the plan's tile order");
};

template <int CI, int CO, bool O16, int EK>
LdsFn lds_fn(bool epi, bool wide) {
  using P = LdsPick<CI, CO>;
  // Wide variants exist only for the chunk / tile widths a wider layer is cut into.
  if constexpr (CI == 128 || CO == 128) {
    if (wide)
      return epi ? k_subm_lds<CI, CO, P::NB, P::WR, P::WC, O16, EK, true, true>
                 : k_subm_lds<CI, CO, P::NB, P::WR, P::WC, O16, EK, false, true>;
  }
  return epi ? k_subm_lds<CI, CO, P::NB, P::WR, P::WC, O16, EK, true, false>
             : k_subm_lds<CI, CO, P::NB, P::WR, P::WC, O16, EK, false, false>;
}

// Layers wider than 128 channels run the 128-wide kernels: cin in chunks of 128 (kch of
// them, summed over in the stage loop), cout in tiles of 128 (ctn workgroups per row tile).
// *ck / *cot receive the kernel's chunk and tile widths.
LdsFn pick_lds(int cin, int cout, bool out16, int ek, int* threads, int* rows_per_tile,
               int* wc_groups, bool epi, int* ck_out = nullptr, int* cot_out = nullptr) {
  if ((cin > 128 && cin % 128 != 0) || (cout > 128 && cout % 128 != 0)) return nullptr;
  const int ck = cin > 128 ? 128 : cin, cot = cout > 128 ? 128 : cout;
  const bool wide = cin > 128 || cout > 128;
  if (ck_out) *ck_out = ck;
  if (cot_out) *cot_out = cot;
#define SSC_CASE(CI, CO)                                                             \
  if (ck == CI && cot == CO) {                                                       \
    using P = LdsPick<CI, CO>;                                                       \
    *threads = P::WR * P::WC * 64;                                                   \
    *rows_per_tile = P::NB * 16;                                                     \
    *wc_groups = P::WC;                                                              \
    if (ek == 1)                                                                     \
      return out16 ? lds_fn<CI, CO, true, 1>(epi, wide) : lds_fn<CI, CO, false, 1>(epi, wide); \
    return out16 ? lds_fn<CI, CO, true, 0>(epi, wide) : lds_fn<CI, CO, false, 0>(epi, wide); \
  }
  SSC_CASE(32, 16) SSC_CASE(32, 32) SSC_CASE(32, 64) SSC_CASE(32, 128)
  SSC_CASE(64, 16) SSC_CASE(64, 32) SSC_CASE(64, 64) SSC_CASE(64, 128)
  SSC_CASE(128, 16) SSC_CASE(128, 32) SSC_CASE(128, 64) SSC_CASE(128, 128)
#undef SSC_CASE
  return nullptr;
}

// Pair kernels (k=3 cin -> cmid, then k=1 cmid -> c2, bf16): the shapes whose 16-bit
// intermediate tile fits the conv kernel's staging space and whose k=1 outputs divide into
// the conv's column groups.
template <int CI, int CM, int CO>
LdsFn pair_fn() {
  using P = LdsPick<CI, CM>;
  return k_subm_lds<CI, CM, P::NB, P::WR, P::WC, true, 0, false, false, CO>;
}

LdsFn pick_pair(int cin, int cmid, int c2, int* threads, int* rows_per_tile, int* wc_groups) {
#define SSC_PAIR(CI, CM, CO)                                                         \
  if (cin == CI && cmid == CM && c2 == CO) {                                         \
    using P = LdsPick<CI, CM>;                                                       \
    *threads = P::WR * P::WC * 64;                                                   \
    *rows_per_tile = P::NB * 16;                                                     \
    *wc_groups = P::WC;                                                              \
    return pair_fn<CI, CM, CO>();                                                    \
  }
  SSC_PAIR(32, 64, 64) SSC_PAIR(64, 64, 64) SSC_PAIR(128, 64, 64)
  SSC_PAIR(64, 128, 64) SSC_PAIR(64, 128, 128) SSC_PAIR(128, 128, 64) SSC_PAIR(128, 128, 128)
#undef SSC_PAIR
  return nullptr;
}

bool valid_dtype(int d) { return d == SSC_F32 || d == SSC_BF16 || d == SSC_F16; }

// Element kind of a 16-bit feature type for the matrix-core kernels (-1: none).
int elem_kind(int d) { return d == SSC_BF16 ? 0 : d == SSC_F16 ? 1 : -1; }

// Compute units of the current device, cached per device id.  The cache is a table of
// atomics: concurrent first calls on one device may both query the attribute, and each
// stores the same value, so every reader sees 0 (not cached yet) or the device's count.
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

ssc_status launch_linear(LinFn fn, int rows_per_tile, const void* feats, const uint16_t* wp,
                         const float* bias, int64_t n, void* out, const Epi& ep, hipStream_t s) {
  // Persistent: four resident workgroups per compute unit, each walking tiles with a stride.
  // Two keep HBM as busy for the plain map; a silu epilogue (an exp and a reciprocal per
  // output) needs the other two to overlap with the copies (1.2M rows, 32 -> 128 + silu:
  // 119 -> 84 us).
  const int64_t tiles = (n + rows_per_tile - 1) / rows_per_tile;
  const int64_t grid = std::min<int64_t>(tiles, 4 * static_cast<int64_t>(device_cu_count()));
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(feats), wp, bias, n, out, ep.act, ep.res);
  return launch_status();
}

// kch input chunks and ctn output tiles of the kernel's widths (1 and 1 for a layer of them).
ssc_status launch_lds(LdsFn fn, int threads, int rows_per_tile, const void* feats,
                      const uint16_t* wt, const float* bias, const void* plan, int64_t n,
                      void* out, const Epi& ep, hipStream_t s, int kch = 1, int ctn = 1) {
  const PlanLayout P = plan_layout(n);
  const char* pb = static_cast<const char*>(plan);
  const int64_t tiles = P.npad / rows_per_tile;
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(ctn)),
                     dim3(threads), 0, s,
                     static_cast<const uint16_t*>(feats), wt, bias,
                     reinterpret_cast<const int32_t*>(pb + P.off_perm),
                     reinterpret_cast<const uint32_t*>(pb + P.off_bmask),
                     reinterpret_cast<const int32_t*>(pb + P.off_gidx),
                     reinterpret_cast<const uint16_t*>(pb + P.off_zero),
                     reinterpret_cast<const int64_t*>(pb) + kPlanSchedWord, P.npad, kch, out,
                     ep);
  return launch_status();
}

// Host checks of an epilogue; fills the kernel-side arguments (gn left null: the caller
// decides whether the kernel sums the statistics itself).
ssc_status check_epilogue(const ssc_epilogue* e, int64_t n, int cout, Epi* ep) {
  *ep = Epi{nullptr, nullptr, n, SSC_ACT_NONE, 0, nullptr, nullptr, nullptr, 0};
  if (e == nullptr) return SSC_OK;
  if (e->act < SSC_ACT_NONE || e->act > SSC_ACT_SILU || e->reserved != 0) return SSC_ERR_ARG;
  if (e->residual && !aligned(e->residual, 16)) return SSC_ERR_ARG;
  if (e->gn_partials) {
    if (e->gn_groups < 1 || e->gn_groups > 256 || cout % e->gn_groups != 0) return SSC_ERR_ARG;
    if (e->batch < 1 || e->batch > SSC_GN_MAX_BATCH) return SSC_ERR_ARG;
    if (e->batch > 1 && n > 0 && e->coords == nullptr) return SSC_ERR_ARG;
    if (!aligned(e->gn_partials, 16) || (e->coords && !aligned(e->coords, 16)))
      return SSC_ERR_ARG;
    if (e->gn_partials_bytes < ssc_gn_partials_bytes(n, e->batch, e->gn_groups))
      return SSC_ERR_WORKSPACE;
  }
  ep->act = e->act;
  ep->res = e->residual;
  ep->gn_groups = e->gn_groups;
  return SSC_OK;
}

// Whether the k=3 kernel sums the group-norm statistics in its epilogue: one batch entry and
// groups of a power-of-two number of channels up to 16 (a group inside one 16-column tile).
bool gn_fusable(const ssc_epilogue* e, int cout) {
  // One output tile only (the kernel's statistics cover the columns of its own tile).
  if (e == nullptr || e->gn_partials == nullptr || e->batch != 1 || cout > 128) return false;
  const int gs = cout / e->gn_groups;
  return gs <= 16 && (gs & (gs - 1)) == 0;
}

// The group-norm partial sums of out, when the kernel did not sum them in its epilogue.
ssc_status gn_after(const ssc_epilogue* e, bool fused, const void* out, int out_dtype, int64_t n,
                    int cout, hipStream_t s) {
  if (e == nullptr || e->gn_partials == nullptr || fused) return SSC_OK;
  return gn_partials_launch(out, out_dtype, n, cout, e->coords, e->batch, e->gn_groups,
                            e->gn_partials, s);
}

// ck / cot: the input chunk and output tile of the kernel the weights are for (0: the layer's
// own cin / cout).
void launch_pack_frag(const void* weight, int taps, int cin, int cout, int wc_groups, int flip,
                      uint16_t* wp, hipStream_t s, int ck = 0, int cot = 0) {
  const int64_t total = static_cast<int64_t>(taps) * (cout / 16) * (cin / 32) * 64;
  const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((total + 255) / 256, 65536));
  k_pack_frag<<<blocks, 256, 0, s>>>(static_cast<const uint16_t*>(weight), taps, cin, cout,
                                     ck ? ck : cin, cot ? cot : cout, wc_groups, flip, wp);
}


ssc_status run_conv(bool dense, const void* feats, int in_dtype, const void* weight,
                    const float* bias, const void* plan, int64_t n, int cin, int cout, void* out,
                    int out_dtype, const ssc_epilogue* epi, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (n < 0 || !valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return SSC_ERR_ARG;
  if (cin < 1 || cout < 1 || cin > 1024 || cout > 1024) return SSC_ERR_UNSUPPORTED;
  if (n >= (int64_t(1) << 31)) return SSC_ERR_UNSUPPORTED;
  if (weight == nullptr || (!dense && plan == nullptr)) return SSC_ERR_ARG;
  if (n > 0 && (feats == nullptr || out == nullptr)) return SSC_ERR_ARG;
  if (!aligned(weight, 16) || (n > 0 && (!aligned(feats, 16) || !aligned(out, 16))))
    return SSC_ERR_ARG;
  if (!dense && !aligned(plan, kAlign)) return SSC_ERR_ARG;
  if (bias && !aligned(bias, 4)) return SSC_ERR_ARG;
  const size_t need = ssc_conv_workspace_bytes(cin, cout, in_dtype);
  if (workspace_bytes < need || (need > 0 && (workspace == nullptr || !aligned(workspace, kAlign))))
    return SSC_ERR_WORKSPACE;
  Epi ep;
  if (const ssc_status st = check_epilogue(epi, n, cout, &ep); st != SSC_OK) return st;
  hipStream_t s = as_stream(stream);
  if (n == 0) return gn_after(epi, false, out, out_dtype, n, cout, s);
  const PlanLayout P = plan_layout(n);
  const char* pb = static_cast<const char*>(plan);
  const int32_t* perm = dense ? nullptr : reinterpret_cast<const int32_t*>(pb + P.off_perm);
  const uint32_t* bmask = dense ? nullptr : reinterpret_cast<const uint32_t*>(pb + P.off_bmask);
  const int32_t* gidx = dense ? nullptr : reinterpret_cast<const int32_t*>(pb + P.off_gidx);
  const int ek = elem_kind(in_dtype);
  // Matrix-core kernels store fp32 or the input's own 16-bit type.
  if (ek >= 0 && (out_dtype == SSC_F32 || out_dtype == in_dtype)) {
    const bool out16 = out_dtype != SSC_F32;
    uint16_t* wt = static_cast<uint16_t*>(workspace);
    if (dense) {
      int wcg = 0, rows = 0;
      const bool use_epi = ep.act != SSC_ACT_NONE || ep.res != nullptr;
      if (LinFn fn = pick_linear(cin, cout, out16, ek, &wcg, &rows, use_epi)) {
        launch_pack_frag(weight, 1, cin, cout, wcg, 0, wt, s);
        if (const ssc_status st = launch_linear(fn, rows, feats, wt, bias, n, out, ep, s);
            st != SSC_OK)
          return st;
        return gn_after(epi, false, out, out_dtype, n, cout, s);
      }
      if (gemm_rows_supported(cin, cout)) {
        launch_pack_frag(weight, 1, cin, cout, cout / 16, 0, wt, s);  // 16-column tiles
        if (const ssc_status st = gemm_rows_launch(feats, wt, bias, n, cin, cout, out, out16,
                                                   ek, ep.act, ep.res, s);
            st != SSC_OK)
          return st;
        return gn_after(epi, false, out, out_dtype, n, cout, s);
      }
    } else {
      int threads = 0, rows = 0, wcg = 0;
      const bool fused = gn_fusable(epi, cout);
      if (fused) ep.gn = epi->gn_partials;
      const bool use_epi = fused || ep.act != SSC_ACT_NONE || ep.res != nullptr;
      int ck = 0, cot = 0;
      if (LdsFn fn = pick_lds(cin, cout, out16, ek, &threads, &rows, &wcg, use_epi, &ck, &cot)) {
        launch_pack_frag(weight, kTaps, cin, cout, wcg, 0, wt, s, ck, cot);
        if (const ssc_status st = launch_lds(fn, threads, rows, feats, wt, bias, plan, n, out, ep,
                                             s, cin / ck, cout / cot);
            st != SSC_OK)
          return st;
        return gn_after(epi, fused, out, out_dtype, n, cout, s);
      }
    }
  }
  const int64_t rows = dense ? n : P.npad;
  const int64_t total = rows * cout;
  const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((total + 255) / 256, 262144));
  if (in_dtype == SSC_BF16) {
    auto fn = dense ? k_conv_valu<uint16_t, true> : k_conv_valu<uint16_t, false>;
    hipLaunchKernelGGL(fn, dim3(blocks), dim3(256), 0, s, static_cast<const uint16_t*>(feats),
                       static_cast<const uint16_t*>(weight), bias, perm, gidx, P.npad, n, cin,
                       cout, out, out_dtype, ep.act, ep.res);
  } else if (in_dtype == SSC_F16) {
    auto fn = dense ? k_conv_valu<_Float16, true> : k_conv_valu<_Float16, false>;
    hipLaunchKernelGGL(fn, dim3(blocks), dim3(256), 0, s, static_cast<const _Float16*>(feats),
                       static_cast<const _Float16*>(weight), bias, perm, gidx, P.npad, n, cin,
                       cout, out, out_dtype, ep.act, ep.res);
  } else {
    auto fn = dense ? k_conv_valu<float, true> : k_conv_valu<float, false>;
    hipLaunchKernelGGL(fn, dim3(blocks), dim3(256), 0, s, static_cast<const float*>(feats),
                       static_cast<const float*>(weight), bias, perm, gidx, P.npad, n, cin, cout,
                       out, out_dtype, ep.act, ep.res);
  }
  if (const ssc_status st = launch_status(); st != SSC_OK) return st;
  return gn_after(epi, false, out, out_dtype, n, cout, s);
}

}  // namespace
}  // namespace ssc

using namespace ssc;

extern "C" size_t ssc_conv_workspace_bytes(int32_t cin, int32_t cout, int32_t in_dtype) {
  if ((in_dtype != SSC_BF16 && in_dtype != SSC_F16) || cin < 1 || cout < 1) return 0;
  return align_up(static_cast<size_t>(kTaps) * cin * cout * sizeof(uint16_t));
}

extern "C" ssc_status ssc_subm_conv3d_plan(const void* feats, int32_t in_dtype,
                                           const void* weight, const float* bias,
                                           const void* plan, int64_t n, int32_t cin,
                                           int32_t cout, void* out, int32_t out_dtype,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream) {
  return run_conv(false, feats, in_dtype, weight, bias, plan, n, cin, cout, out, out_dtype,
                  nullptr, workspace, workspace_bytes, stream);
}

extern "C" ssc_status ssc_subm_conv3d_plan_ex(const void* feats, int32_t in_dtype,
                                              const void* weight, const float* bias,
                                              const void* plan, int64_t n, int32_t cin,
                                              int32_t cout, void* out, int32_t out_dtype,
                                              const ssc_epilogue* epilogue, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  return run_conv(false, feats, in_dtype, weight, bias, plan, n, cin, cout, out, out_dtype,
                  epilogue, workspace, workspace_bytes, stream);
}

// The map-taking call: the workspace holds [plan][plan scratch][re-laid-out weights], each
// part 256-byte aligned.
namespace {
struct MapWork {
  size_t off_plan, off_scratch, off_weights, total;
};
MapWork map_work(int64_t n, int32_t cin, int32_t cout, int32_t in_dtype) {
  MapWork M;
  M.off_plan = 0;
  M.off_scratch = align_up(ssc_plan_bytes(n));
  M.off_weights = M.off_scratch + align_up(ssc_plan_workspace_bytes(n));
  M.total = M.off_weights + ssc_conv_workspace_bytes(cin, cout, in_dtype);
  return M;
}
}  // namespace

extern "C" size_t ssc_subm_conv3d_workspace_bytes(int64_t n, int32_t cin, int32_t cout,
                                                  int32_t in_dtype) {
  if (n < 0 || cin < 1 || cout < 1) return 0;
  return map_work(n, cin, cout, in_dtype).total;
}

extern "C" ssc_status ssc_subm_conv3d(const void* feats, int32_t in_dtype, const void* weight,
                                      const float* bias, const int32_t* nbr, int64_t n,
                                      int32_t cin, int32_t cout, void* out, int32_t out_dtype,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (n < 0 || !valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return SSC_ERR_ARG;
  if (cin < 1 || cout < 1 || cin > 1024 || cout > 1024) return SSC_ERR_UNSUPPORTED;
  if (n >= (int64_t(1) << 31)) return SSC_ERR_UNSUPPORTED;
  if (weight == nullptr || (n > 0 && nbr == nullptr)) return SSC_ERR_ARG;
  if (n == 0) return SSC_OK;
  // Every host-detectable error is reported before the plan kernels are enqueued.
  if (feats == nullptr || out == nullptr || workspace == nullptr) return SSC_ERR_ARG;
  if (!aligned(weight, 16) || !aligned(feats, 16) || !aligned(out, 16) || !aligned(nbr, 4) ||
      !aligned(workspace, kAlign) || (bias && !aligned(bias, 4)))
    return SSC_ERR_ARG;
  const MapWork M = map_work(n, cin, cout, in_dtype);
  if (workspace_bytes < M.total) return SSC_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  if (const ssc_status st =
          ssc_build_plan(nbr, nullptr, n, 1, nullptr, ws + M.off_plan, M.off_scratch,
                         ws + M.off_scratch, M.off_weights - M.off_scratch, stream);
      st != SSC_OK)
    return st;
  return run_conv(false, feats, in_dtype, weight, bias, ws + M.off_plan, n, cin, cout, out,
                  out_dtype, nullptr, ws + M.off_weights, M.total - M.off_weights, stream);
}

// ------------------------------------------------------------------------------------------
// Allocation-free variant of ssc_subm_conv3d_plan: the re-laid-out weights go to a static
// device array instead of a caller workspace.  Its device address is looked up once per
// device (the runtime's address of this device's copy of the array) and kept; host code uses
// that address, never the array's name.
// ------------------------------------------------------------------------------------------
namespace ssc {
namespace {
static __device__ __align__(256) unsigned char scratch[SSC_STATIC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_ptr[64];

// This device's copy of the static scratch, or null if the runtime cannot give its address.
void* static_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
      return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);  // same value on every race
    p = q;
  }
  return p;
}
}  // namespace
}  // namespace ssc

extern "C" ssc_status ssc_subm_conv3d_plan_static(const void* feats, int32_t in_dtype,
                                                  const void* weight, const float* bias,
                                                  const void* plan, int64_t n, int32_t cin,
                                                  int32_t cout, void* out, int32_t out_dtype,
                                                  void* stream) {
  if (!valid_dtype(in_dtype)) return SSC_ERR_ARG;
  const size_t need = ssc_conv_workspace_bytes(cin, cout, in_dtype);
  if (need > SSC_STATIC_SCRATCH_BYTES) return SSC_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && (ws = static_scratch()) == nullptr) return SSC_ERR_HIP;
  return run_conv(false, feats, in_dtype, weight, bias, plan, n, cin, cout, out, out_dtype,
                  nullptr, ws, ws ? need : 0, stream);
}

extern "C" ssc_status ssc_linear(const void* feats, int32_t in_dtype, const void* weight,
                                 const float* bias, int64_t n, int32_t cin, int32_t cout, void* out,
                                 int32_t out_dtype, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return run_conv(true, feats, in_dtype, weight, bias, nullptr, n, cin, cout, out, out_dtype,
                  nullptr, workspace, workspace_bytes, stream);
}

extern "C" ssc_status ssc_linear_ex(const void* feats, int32_t in_dtype, const void* weight,
                                    const float* bias, int64_t n, int32_t cin, int32_t cout,
                                    void* out, int32_t out_dtype, const ssc_epilogue* epilogue,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return run_conv(true, feats, in_dtype, weight, bias, nullptr, n, cin, cout, out, out_dtype,
                  epilogue, workspace, workspace_bytes, stream);
}

extern "C" size_t ssc_packed_weight_bytes(int32_t taps, int32_t cin, int32_t cout) {
  if (taps < 1 || cin < 1 || cout < 1) return 0;
  return align_up(static_cast<size_t>(taps) * cin * cout * sizeof(uint16_t));
}

extern "C" ssc_status ssc_pack_weights(const void* weight, int32_t taps, int32_t cin, int32_t cout,
                                       void* packed, size_t packed_bytes, void* stream) {
  return ssc_pack_weights_ex(weight, taps, cin, cout, 0, packed, packed_bytes, stream);
}

extern "C" ssc_status ssc_pack_weights_ex(const void* weight, int32_t taps, int32_t cin,
                                          int32_t cout, int32_t flags, void* packed,
                                          size_t packed_bytes, void* stream) {
  if (weight == nullptr || packed == nullptr) return SSC_ERR_ARG;
  if ((flags & ~(SSC_PACK_FLIP | SSC_PACK_PAIR)) ||
      ((flags & SSC_PACK_PAIR) && (taps != 1 || (flags & SSC_PACK_FLIP))))
    return SSC_ERR_ARG;
  int threads = 0, rows = 0, wcg = 0;
  int ck = 0, cot = 0;
  if (flags & SSC_PACK_PAIR) {
    // The k=1 layer (cin -> cout) of a pair kernel, in the column groups of the k=3 layer
    // before it (whose output width is this layer's cin).
    bool any = false;
    for (const int ci : {32, 64, 128})
      any = any || pick_pair(ci, cin, cout, &threads, &rows, &wcg) != nullptr;
    if (!any) return SSC_ERR_UNSUPPORTED;
  } else if (taps == kTaps) {
    if (pick_lds(cin, cout, false, 0, &threads, &rows, &wcg, false, &ck, &cot) == nullptr)
      return SSC_ERR_UNSUPPORTED;
  } else if (taps == 1) {
    // The k=1 kernels' layouts: the streaming kernel's column groups, else 16-column tiles.
    if (pick_linear(cin, cout, false, 0, &wcg, &rows, false) == nullptr) {
      if (!gemm_rows_supported(cin, cout)) return SSC_ERR_UNSUPPORTED;
      wcg = cout / 16;
    }
  } else {
    return SSC_ERR_UNSUPPORTED;
  }
  if (!aligned(weight, 16) || !aligned(packed, kAlign)) return SSC_ERR_ARG;
  if (packed_bytes < ssc_packed_weight_bytes(taps, cin, cout)) return SSC_ERR_WORKSPACE;
  // A single tap is its own mirror image: the flag changes nothing there.
  launch_pack_frag(weight, taps, cin, cout, wcg, (taps == kTaps && (flags & SSC_PACK_FLIP)) ? 1 : 0,
                   static_cast<uint16_t*>(packed), as_stream(stream), ck, cot);
  return launch_status();
}

extern "C" ssc_status ssc_linear_packed(const void* feats, const void* packed_weight,
                                        const float* bias, int64_t n, int32_t cin, int32_t cout,
                                        void* out, int32_t out_dtype, void* stream) {
  return ssc_linear_packed_ex(feats, packed_weight, bias, n, cin, cout, out, out_dtype, nullptr,
                              stream);
}

extern "C" ssc_status ssc_linear_packed_ex(const void* feats, const void* packed_weight,
                                           const float* bias, int64_t n, int32_t cin,
                                           int32_t cout, void* out, int32_t out_dtype,
                                           const ssc_epilogue* epilogue, void* stream) {
  if (n < 0 || !valid_dtype(out_dtype) || packed_weight == nullptr) return SSC_ERR_ARG;
  if (n >= (int64_t(1) << 31) || out_dtype == SSC_F16) return SSC_ERR_UNSUPPORTED;
  const bool out16 = out_dtype == SSC_BF16;
  Epi ep;
  if (const ssc_status st = check_epilogue(epilogue, n, cout, &ep); st != SSC_OK) return st;
  const bool use_epi = ep.act != SSC_ACT_NONE || ep.res != nullptr;
  int wcg = 0, rows = 0;
  LinFn fn = pick_linear(cin, cout, out16, 0, &wcg, &rows, use_epi);
  if (fn == nullptr && !gemm_rows_supported(cin, cout)) return SSC_ERR_UNSUPPORTED;
  if (n > 0 && (feats == nullptr || out == nullptr)) return SSC_ERR_ARG;
  if (!aligned(packed_weight, 16) || (n > 0 && (!aligned(feats, 16) || !aligned(out, 16))) ||
      (bias && !aligned(bias, 4)))
    return SSC_ERR_ARG;
  hipStream_t s = as_stream(stream);
  if (n == 0) return gn_after(epilogue, false, out, out_dtype, n, cout, s);
  const auto* wp = static_cast<const uint16_t*>(packed_weight);
  if (const ssc_status st =
          fn ? launch_linear(fn, rows, feats, wp, bias, n, out, ep, s)
             : gemm_rows_launch(feats, wp, bias, n, cin, cout, out, out16, 0, ep.act, ep.res, s);
      st != SSC_OK)
    return st;
  return gn_after(epilogue, false, out, out_dtype, n, cout, s);
}

extern "C" ssc_status ssc_subm_conv3d_pair_packed(const void* feats, const void* packed1,
                                                  const float* bias1, const void* plan,
                                                  int64_t n, int32_t cin, int32_t cmid,
                                                  const void* packed2, const float* bias2,
                                                  int32_t cout, void* out, int32_t out_dtype,
                                                  void* stream) {
  if (n < 0 || !valid_dtype(out_dtype) || packed1 == nullptr || packed2 == nullptr ||
      plan == nullptr)
    return SSC_ERR_ARG;
  if (n >= (int64_t(1) << 31) || out_dtype == SSC_F16) return SSC_ERR_UNSUPPORTED;
  int threads = 0, rows = 0, wcg = 0;
  LdsFn fn = pick_pair(cin, cmid, cout, &threads, &rows, &wcg);
  if (fn == nullptr) return SSC_ERR_UNSUPPORTED;
  if (n > 0 && (feats == nullptr || out == nullptr)) return SSC_ERR_ARG;
  if (!aligned(packed1, 16) || !aligned(packed2, 16) || !aligned(plan, kAlign) ||
      (n > 0 && (!aligned(feats, 16) || !aligned(out, 16))) || (bias1 && !aligned(bias1, 4)) ||
      (bias2 && !aligned(bias2, 4)))
    return SSC_ERR_ARG;
  if (n == 0) return SSC_OK;
  const Epi ep{nullptr, nullptr, n, SSC_ACT_NONE, 0, static_cast<const uint16_t*>(packed2),
               bias2, out, out_dtype == SSC_F32 ? 1 : 0};
  return launch_lds(fn, threads, rows, feats, static_cast<const uint16_t*>(packed1), bias1, plan,
                    n, nullptr, ep, as_stream(stream));
}

extern "C" ssc_status ssc_subm_conv3d_packed(const void* feats, const void* packed_weight,
                                             const float* bias, const void* plan, int64_t n,
                                             int32_t cin, int32_t cout, void* out,
                                             int32_t out_dtype, void* stream) {
  return ssc_subm_conv3d_packed_ex(feats, packed_weight, bias, plan, n, cin, cout, out,
                                   out_dtype, nullptr, stream);
}

extern "C" ssc_status ssc_subm_conv3d_packed_ex(const void* feats, const void* packed_weight,
                                                const float* bias, const void* plan, int64_t n,
                                                int32_t cin, int32_t cout, void* out,
                                                int32_t out_dtype, const ssc_epilogue* epilogue,
                                                void* stream) {
  if (n < 0 || !valid_dtype(out_dtype) || packed_weight == nullptr || plan == nullptr)
    return SSC_ERR_ARG;
  if (n >= (int64_t(1) << 31) || out_dtype == SSC_F16) return SSC_ERR_UNSUPPORTED;
  int threads = 0, rows = 0, wcg = 0;
  if (pick_lds(cin, cout, out_dtype == SSC_BF16, 0, &threads, &rows, &wcg, false) == nullptr)
    return SSC_ERR_UNSUPPORTED;
  if (n > 0 && (feats == nullptr || out == nullptr)) return SSC_ERR_ARG;
  if (!aligned(packed_weight, 16) || !aligned(plan, kAlign) ||
      (n > 0 && (!aligned(feats, 16) || !aligned(out, 16))) || (bias && !aligned(bias, 4)))
    return SSC_ERR_ARG;
  Epi ep;
  if (const ssc_status st = check_epilogue(epilogue, n, cout, &ep); st != SSC_OK) return st;
  hipStream_t s = as_stream(stream);
  if (n == 0) return gn_after(epilogue, false, out, out_dtype, n, cout, s);
  const bool fused = gn_fusable(epilogue, cout);
  if (fused) ep.gn = epilogue->gn_partials;
  const bool use_epi = fused || ep.act != SSC_ACT_NONE || ep.res != nullptr;
  int ck = 0, cot = 0;
  LdsFn fn = pick_lds(cin, cout, out_dtype == SSC_BF16, 0, &threads, &rows, &wcg, use_epi, &ck,
                      &cot);
  if (const ssc_status st = launch_lds(fn, threads, rows, feats,
                                       static_cast<const uint16_t*>(packed_weight), bias, plan, n,
                                       out, ep, s, cin / ck, cout / cot);
      st != SSC_OK)
    return st;
  return gn_after(epilogue, fused, out, out_dtype, n, cout, s);
}
