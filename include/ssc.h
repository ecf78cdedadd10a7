/*
 * ssc.h - C ABI of libssc.so: submanifold sparse 3x3x3 convolution (SubMConv3d, stride 1,
 * output sites = input sites) over active voxel coordinates, for AMD MI355X (gfx950).
 *
 * The operation (as the pages define it):
 *   - Every SparseConv3d of the TRELLIS.2-lineage sparse VAEs is built with stride 1 and no
 *     padding and so runs as a submanifold convolution: outputs live exactly on the input
 *     sites (LATO.2 MLX port page, "The scope, once measured").  k=3 and k=1 both occur
 *     (same page, "Status").
 *   - Cross-correlation: the tap at offset d reads the features of site c + d (same page,
 *     "Correctness").
 *   - Weights are [K^3, Cin, Cout] (Pixal3D MLX port README, "Status", the KRSC remap).
 *   - The coordinate -> row map is built once per coordinate set and reused by every layer
 *     on that set (LATO.2 page, "Fleet benchmark" version history: "cached device index";
 *     trellis-mac article, gather-scatter flowchart, last step: cache the neighbour map per
 *     tensor; Pixal3D README: the spatial cache).
 *
 * Conventions shared by every entry point:
 *   - All array pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors) unless
 *     marked "host".  Arrays are contiguous and row-major.  The caller owns every buffer,
 *     including outputs and workspaces; the library never allocates device memory.  Its only
 *     host-side state is a per-device cache of the compute-unit count (an array of atomics,
 *     written once per device with the value the runtime reports), so calls on different
 *     streams with different buffers are independent.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is enqueued on it and
 *     the call returns without waiting, except ssc_build_index with check != 0, which waits
 *     for its own work to read two error counters back.
 *   - Host-detectable argument errors return before anything is launched.  A failed launch
 *     returns SSC_ERR_HIP.  On any error the contents of output buffers are unspecified.
 *   - bf16 means IEEE-754 binary32 truncated to its upper 16 bits (bfloat16), passed as
 *     uint16_t storage; feature, weight and output pointers must be 16-byte aligned.
 *   - Taps are numbered t = 9*(dx+1) + 3*(dy+1) + (dz+1) for offsets dx,dy,dz in {-1,0,1};
 *     the centre tap is t = 13.  (The pages do not fix an order; this is row-major over the
 *     3x3x3 kernel, which is also how a [Cout,Cin,3,3,3] dense kernel flattens.)
 */
#ifndef SSC_H
#define SSC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSC_OK = 0,
  SSC_ERR_ARG = -1,          /* null pointer, negative size, bad enum, misaligned pointer    */
  SSC_ERR_COORD_RANGE = -2,  /* a coordinate outside [0,batch) x [0,Gx) x [0,Gy) x [0,Gz)    */
  SSC_ERR_DUPLICATE = -3,    /* two rows with the same (b, x, y, z)                            */
  SSC_ERR_UNSUPPORTED = -4,  /* shape outside what the kernels handle (see each call)          */
  SSC_ERR_WORKSPACE = -5,    /* workspace or plan buffer smaller than the *_bytes() figure     */
  SSC_ERR_HIP = -6           /* a HIP runtime call failed                                      */
} ssc_status;

typedef enum { SSC_F32 = 0, SSC_BF16 = 1, SSC_F16 = 2 } ssc_dtype;

/* Library version (major*10000 + minor*100 + patch). */
int ssc_version(void);

/* Human-readable text for a status code (static storage; never NULL). */
const char* ssc_status_string(int status);

/* Digest (16 hex digits, static storage) of the sources the library was built from; the
 * Python binding refuses a library whose digest differs from the sources beside it. */
const char* ssc_source_digest(void);

/* ---------------------------------------------------------------------------------------
 * Coordinate index (cold path, once per coordinate set)
 * ------------------------------------------------------------------------------------- */

/* Bytes of device workspace ssc_build_index needs for n sites (an open-addressing hash table
 * of 2^ceil(log2(2n)) slots, at least 64, plus two counters). */
size_t ssc_index_workspace_bytes(int64_t n);

/* Neighbour map of n active sites (trellis-mac article, gather-scatter flowchart: "build a
 * hash map of the active voxel coordinates", then gather per kernel offset).
 *   coords     [n, 4] int32 rows (b, x, y, z), any order, no duplicates.
 *   batch      number of batch entries; 1 <= batch <= 65535.
 *   grid       host int32[3] = (Gx, Gy, Gz), each in [1, 65535].
 *   nbr        [n, 27] int32 output: nbr[i][t] = row index (into coords) of the site at
 *              (b, x+dx, y+dy, z+dz), or -1 when that voxel is inactive or outside the grid.
 *              Sites in different batch entries are never neighbours.
 *   workspace  >= ssc_index_workspace_bytes(n) bytes, 256-byte aligned, scratch only.
 *   check      nonzero: wait for the kernels and return SSC_ERR_COORD_RANGE or
 *              SSC_ERR_DUPLICATE if any row is out of range or repeated.  Zero: no wait; such
 *              input then leaves nbr unspecified (never out-of-bounds memory access).
 * n = 0 is valid and launches nothing. */
ssc_status ssc_build_index(const int32_t* coords, int64_t n, int32_t batch, const int32_t* grid,
                           int32_t* nbr, void* workspace, size_t workspace_bytes, int32_t check,
                           void* stream);

/* ssc_build_index with the choice of index structure (the map is the same, bit for bit):
 *   SSC_INDEX_HASH   the open-addressing hash of the packed 64-bit keys (trellis-mac article,
 *                    flowchart: a hash map of the active coordinates);
 *   SSC_INDEX_DENSE  the sorted-key index (LATO.2 MLX port page, module table: a sorted-key
 *                    indice map) kept as an occupancy bitmap over the dense voxel id
 *                    v = ((b*Gx + x)*Gy + y)*Gz + z with running counts, so that the rank of
 *                    a site's bit is its position in key order and a lookup is four loads
 *                    without a search; its arrays take 3/16 byte per voxel + 4 bytes per site;
 *   SSC_INDEX_AUTO   (what ssc_build_index uses) the dense index when its arrays fit in
 *                    ssc_index_workspace_bytes(n), i.e. when batch*Gx*Gy*Gz is at most about
 *                    85 voxels per hash slot; the hash otherwise.
 * SSC_INDEX_DENSE with a larger grid than the workspace holds returns SSC_ERR_WORKSPACE (or
 * SSC_ERR_UNSUPPORTED when batch*Gx*Gy*Gz >= 2^62); an unknown method SSC_ERR_ARG. */
#define SSC_INDEX_AUTO 0
#define SSC_INDEX_HASH 1
#define SSC_INDEX_DENSE 2
ssc_status ssc_build_index_ex(const int32_t* coords, int64_t n, int32_t batch,
                              const int32_t* grid, int32_t* nbr, void* workspace,
                              size_t workspace_bytes, int32_t check, int32_t method,
                              void* stream);

/* Workspace bytes of ssc_build_index_ex with that method (host only): the hash's size for
 * SSC_INDEX_AUTO and SSC_INDEX_HASH (= ssc_index_workspace_bytes(n)), the dense index's own
 * for SSC_INDEX_DENSE (0 when batch*Gx*Gy*Gz >= 2^62 or on bad arguments). */
size_t ssc_index_workspace_bytes_ex(int64_t n, int32_t batch, const int32_t* grid,
                                    int32_t method);

/* The structure SSC_INDEX_AUTO picks for n sites in batch x grid (host only, no GPU). */
int32_t ssc_index_method(int64_t n, int32_t batch, const int32_t* grid);

/* ---------------------------------------------------------------------------------------
 * Warm plan (derived from the neighbour map once per coordinate set, reused by every layer)
 * ------------------------------------------------------------------------------------- */

/* Bytes of the plan buffer for n sites, and of the scratch workspace ssc_build_plan needs. */
size_t ssc_plan_bytes(int64_t n);
size_t ssc_plan_workspace_bytes(int64_t n);

/* Reorders the sites for the convolution kernels and stores the neighbour rows in that order
 * (the "prepared device index" the LATO.2 page caches per coordinate set).  The plan holds:
 * the site order, each 16-row block's tap mask, the neighbour rows tap-major in that order,
 * and the tile schedule the k=3 matrix-core kernel follows.  It is valid for any features and
 * weights and for every k=3 layer on the same coordinate set.
 * Site order.  Mask order: rows stably sorted by the rank of their 26-bit mask of valid
 * non-centre taps read as a reflected Gray code, so that 16-row blocks share which taps are
 * present.  With coords, when the grid holds at least 8 bricks of 128^3 voxels (batch entries
 * count separately), the spatial order is tried as well: the mask order stably re-sorted by
 * brick (batch entry, then Morton code of the brick).  It is kept when its count of (16-row
 * block, tap present) pairs is at most 21/20 of the mask order's; the kernel then gives each
 * XCD a contiguous share of the tiles, so that each XCD's L2 holds one region's rows.
 *   nbr    [n, 27] int32 from ssc_build_index (or any map with the same meaning).
 *   coords [n, 4] int32 rows (b, x, y, z) that nbr was built from, 16-byte aligned, or NULL
 *          for the mask order only (batch and grid are then ignored).
 *   batch, grid  as for ssc_build_index (host int32[3]); used with coords only.
 *   plan   >= ssc_plan_bytes(n) bytes, 256-byte aligned; written completely.
 *   workspace >= ssc_plan_workspace_bytes(n) bytes, 256-byte aligned, scratch only.
 * Errors: SSC_ERR_ARG for null or misaligned buffers (or coords without grid),
 * SSC_ERR_UNSUPPORTED for batch or grid outside [1, 65535] (with coords) or n >= 2^31,
 * SSC_ERR_WORKSPACE for short buffers.
 * Bit-reproducible: the same arguments always yield the same plan. */
ssc_status ssc_build_plan(const int32_t* nbr, const int32_t* coords, int64_t n, int32_t batch,
                          const int32_t* grid, void* plan, size_t plan_bytes, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Where the parts of a plan for n sites live (for inspection and tests; host only, no GPU).
 * Writes layout[0] = npad (rows, n rounded up to a multiple of 256, at least 256), then byte
 * offsets within the plan buffer: layout[1] perm (int32 [npad]: original site of each sorted
 * row, -1 on padding rows), layout[2] block masks (uint32 [npad / 16]: OR over the block's
 * rows of (1 << t) for every tap t with a neighbour), layout[3] neighbour rows (int32
 * [27][npad]: row r of tap t holds nbr[perm[r]][t], -1 on padding), layout[4] the zero row
 * (2048 bytes of zeros).  Returns SSC_ERR_ARG for n < 0 or a null layout. */
ssc_status ssc_plan_layout(int64_t n, int64_t* layout);

/* ---------------------------------------------------------------------------------------
 * Convolution (warm path)
 * ------------------------------------------------------------------------------------- */

/* SubMConv3d, k=3, stride 1, on the neighbour map of a coordinate set:
 *   out[i][o] = bias[o] + sum_{t : nbr[i][t] != -1} sum_c feats[nbr[i][t]][c] * weight[t][c][o]
 * (cross-correlation; LATO.2 MLX port page, "Correctness"; the gather per kernel offset from
 * the neighbour map, trellis-mac article, gather-scatter flowchart).
 *   feats    [n, cin], in_dtype (SSC_F32, SSC_BF16 or SSC_F16); rows in coords order.
 *   weight   [27, cin, cout], same dtype as feats (Pixal3D MLX port README, "Status").
 *   bias     [cout] fp32, or NULL for none.
 *   nbr      [n, 27] int32 neighbour map from ssc_build_index (or any map with its meaning).
 *   out      [n, cout], out_dtype; rows in coords order; must not alias feats.
 *   workspace >= ssc_subm_conv3d_workspace_bytes(n, cin, cout, in_dtype) bytes, 256-byte
 *            aligned, scratch only: every call builds the warm plan of the map into it
 *            (ssc_build_plan, mask order) and re-lays the weights out, then runs the same
 *            kernels as ssc_subm_conv3d_plan.  Callers that run several layers on one
 *            coordinate set build the plan once (ssc_build_plan) and call
 *            ssc_subm_conv3d_plan or ssc_subm_conv3d_packed instead: that is the warm path.
 * Accumulation is fp32 (bf16 and fp16 products are exact in fp32).  out_dtype is SSC_F32 or
 * a 16-bit type: each 16-bit output is the round-to-nearest-even value of the fp32 result
 * the SSC_F32 output holds.  Results are bit-identical from run to run (no atomics in the
 * accumulation) and equal, bit for bit, to ssc_subm_conv3d_plan on a plan of the same map.
 * Shapes and errors as for ssc_subm_conv3d_plan; every host-detectable error returns before
 * anything is launched; n = 0 launches nothing. */
size_t ssc_subm_conv3d_workspace_bytes(int64_t n, int32_t cin, int32_t cout, int32_t in_dtype);
ssc_status ssc_subm_conv3d(const void* feats, int32_t in_dtype, const void* weight,
                           const float* bias, const int32_t* nbr, int64_t n, int32_t cin,
                           int32_t cout, void* out, int32_t out_dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Bytes of scratch workspace ssc_subm_conv3d_plan and ssc_linear need (the weights re-laid out
 * for the matrix cores; 0 for the fp32 path). */
size_t ssc_conv_workspace_bytes(int32_t cin, int32_t cout, int32_t in_dtype);

/* SubMConv3d, k=3, stride 1, over the warm plan of a coordinate set (the same sum as
 * ssc_subm_conv3d):
 *   feats    [n, cin], in_dtype (SSC_F32, SSC_BF16 or SSC_F16); rows in coords order.
 *   weight   [27, cin, cout], same dtype as feats.
 *   bias     [cout] fp32, or NULL for none.
 *   plan     from ssc_build_plan for the same n.
 *   out      [n, cout], out_dtype; rows in coords order; must not alias feats.
 *   workspace >= ssc_conv_workspace_bytes(cin, cout, in_dtype) bytes, 256-byte aligned.
 * fp16 is the checkpoints' source precision (trellis2-mlx-8bit page); the matrix-core kernels
 * store fp32 or the input's own 16-bit type.
 * Shapes: 1 <= cin, cout <= 1024.  bf16 or fp16 with cin in {32, 64, 128} or a multiple of
 * 128, and cout in {16, 32, 64, 128} or a multiple of 128 (and out_dtype fp32 or the input's
 * type) runs on the matrix cores: wider layers as 128-channel input chunks summed in one
 * kernel and 128-column output tiles.  The rest runs a vector-ALU kernel with the same
 * numerics contract.
 * Errors: SSC_ERR_ARG (null or misaligned buffers, bad dtype, n < 0), SSC_ERR_UNSUPPORTED
 * (channels outside [1, 1024], n >= 2^31), SSC_ERR_WORKSPACE (short workspace). */
ssc_status ssc_subm_conv3d_plan(const void* feats, int32_t in_dtype, const void* weight,
                                const float* bias, const void* plan, int64_t n, int32_t cin,
                                int32_t cout, void* out, int32_t out_dtype, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ssc_subm_conv3d_plan for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): no workspace argument; the
 * weights are re-laid out into a static device array of SSC_STATIC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.  The call allocates nothing
 * (no hipMalloc, no library allocation); its first call on a device looks the array's address
 * up once.  Limit: ssc_conv_workspace_bytes(cin, cout, in_dtype) <= SSC_STATIC_SCRATCH_BYTES
 * (27 * cin * cout * 2 bytes: every matrix-core shape with cin and cout <= 128 fits, and
 * wider ones as far as that bound, e.g. 256 -> 64; larger 16-bit layers return
 * SSC_ERR_WORKSPACE before anything is launched).  All calls on one GPU share that GPU's
 * array: calls that overlap on one GPU (concurrent streams, threads) race; calls in order on
 * one stream do not.  Other arguments, results (bit for bit) and errors as for
 * ssc_subm_conv3d_plan; SSC_ERR_HIP if the runtime cannot give the array's address. */
#define SSC_STATIC_SCRATCH_BYTES (1u << 20)
ssc_status ssc_subm_conv3d_plan_static(const void* feats, int32_t in_dtype, const void* weight,
                                       const float* bias, const void* plan, int64_t n,
                                       int32_t cin, int32_t cout, void* out, int32_t out_dtype,
                                       void* stream);

/* Weights re-laid out once for the matrix cores, for callers that keep a layer's weights
 * (the same re-layout ssc_subm_conv3d_plan and ssc_linear perform into their workspace on
 * every call).
 *   weight  [taps, cin, cout] bf16: taps = 27 (k=3) or 1 (k=1).
 *   packed  >= ssc_packed_weight_bytes(taps, cin, cout) bytes, 256-byte aligned; receives
 *           the weights in the kernel's fragment order (an opaque layout of the same byte
 *           count, valid only for ssc_subm_conv3d_packed (taps = 27) or ssc_linear_packed
 *           (taps = 1) with the same cin and cout).
 * taps = 27: the shapes ssc_subm_conv3d_plan runs on the matrix cores (cin in {32, 64, 128}
 * or a multiple of 128, cout in {16, 32, 64, 128} or a multiple of 128).  taps = 1: the shapes ssc_linear runs on the matrix
 * cores (cin, cout in {32, 64, 128}, or multiples of 64 up to 1024).  Otherwise
 * SSC_ERR_UNSUPPORTED. */
size_t ssc_packed_weight_bytes(int32_t taps, int32_t cin, int32_t cout);
ssc_status ssc_pack_weights(const void* weight, int32_t taps, int32_t cin, int32_t cout,
                            void* packed, size_t packed_bytes, void* stream);

/* ssc_pack_weights with options.  flags = 0 or SSC_PACK_FLIP:
 *   SSC_PACK_FLIP  the other kernel orientation, which the LATO.2 page leaves open and builds
 *                  with "--flip-kernel" ("Correctness"): the tap at offset d reads the site
 *                  c - d, i.e. out[i] = bias + sum_t feats[nbr[i][26-t]] @ weight[t]. */
#define SSC_PACK_FLIP 1
/*   SSC_PACK_PAIR  taps = 1 only: the k=1 layer of ssc_subm_conv3d_pair_packed (cin = the k=3
 *                  layer's cout); not combined with SSC_PACK_FLIP. */
#define SSC_PACK_PAIR 2
ssc_status ssc_pack_weights_ex(const void* weight, int32_t taps, int32_t cin, int32_t cout,
                               int32_t flags, void* packed, size_t packed_bytes, void* stream);

/* A k=3 layer followed by a k=1 layer in one kernel (the two-layer stack of the benchmark's
 * batched workload; LATO.2 page, "Status": SubMConv3d k=3 and k=1):
 *   out = (bf16(conv(feats) + bias1)) @ W2 + bias2
 * where bf16() is the round to nearest even that ssc_subm_conv3d_packed applies when it
 * stores bf16, so the result is that of the two calls (conv with out_dtype SSC_BF16, then
 * ssc_linear on its output) without the intermediate ever reaching memory.
 *   feats [n, cin] bf16; packed1 from ssc_pack_weights (taps = 27, cin -> cmid); packed2 from
 *   ssc_pack_weights_ex (taps = 1, cmid -> cout, SSC_PACK_PAIR); bias1 [cmid], bias2 [cout]
 *   fp32 or NULL; plan from ssc_build_plan; out [n, cout] in out_dtype (SSC_F32 or SSC_BF16).
 * Shapes (cin, cmid, cout): (32 | 64 | 128, 64, 64), (64 | 128, 128, 64 | 128); otherwise
 * SSC_ERR_UNSUPPORTED.  Other errors as for ssc_subm_conv3d_packed. */
ssc_status ssc_subm_conv3d_pair_packed(const void* feats, const void* packed1,
                                       const float* bias1, const void* plan, int64_t n,
                                       int32_t cin, int32_t cmid, const void* packed2,
                                       const float* bias2, int32_t cout, void* out,
                                       int32_t out_dtype, void* stream);

/* ssc_subm_conv3d_plan with weights from ssc_pack_weights (taps = 27): one kernel launch, no
 * workspace.  Same results, bit for bit, as ssc_subm_conv3d_plan on the unpacked weights.
 * bf16 inputs and the shapes ssc_pack_weights accepts only. */
ssc_status ssc_subm_conv3d_packed(const void* feats, const void* packed_weight,
                                  const float* bias, const void* plan, int64_t n, int32_t cin,
                                  int32_t cout, void* out, int32_t out_dtype, void* stream);

/* k=1 SubMConv3d, i.e. the per-voxel linear map out = feats @ weight + bias (LATO.2 page,
 * "Status": SubMConv3d k=1; SparseLinear).  No map is needed.  16-bit inputs run on the
 * matrix cores: a streaming kernel for cin, cout in {32, 64, 128}, a tiled GEMM for other
 * multiples of 64 up to 1024 (the ConvNeXt-style MLP's 4C), the vector-ALU kernel otherwise.
 *   feats [n, cin], weight [cin, cout] (the single-tap [1, cin, cout] has the same bytes),
 *   bias [cout] fp32 or NULL, out [n, cout] out_dtype; workspace as for ssc_subm_conv3d_plan. */
ssc_status ssc_linear(const void* feats, int32_t in_dtype, const void* weight, const float* bias,
                      int64_t n, int32_t cin, int32_t cout, void* out, int32_t out_dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ssc_linear with weights from ssc_pack_weights (taps = 1): one kernel launch, no
 * workspace.  Same results, bit for bit, as ssc_linear on the unpacked weights.  bf16 feats,
 * out_dtype SSC_F32 or SSC_BF16; shapes as ssc_pack_weights accepts for taps = 1 (else
 * SSC_ERR_UNSUPPORTED). */
ssc_status ssc_linear_packed(const void* feats, const void* packed_weight, const float* bias,
                             int64_t n, int32_t cin, int32_t cout, void* out, int32_t out_dtype,
                             void* stream);

/* ---------------------------------------------------------------------------------------
 * Epilogues and the sparse group norm of the blocks around the convolution.
 *
 * The LATO.2 MLX port page ("Status") lists what surrounds SubMConv3d in the sparse blocks:
 * SparseLinear, LayerNorm32, SparseGroupNorm32, activations, SparseResBlock; its repository
 * layout says the "32" norms accumulate in fp32.  The pages give no formulas; the readings
 * here are the textbook ones:
 *   activation   relu(v) = max(v, 0); silu(v) = v * sigmoid(v).
 *   group norm   per batch entry b and group g of C / groups consecutive channels: mean and
 *                population variance over the ACTIVE sites of b (inactive voxels are not
 *                zeros) and the channels of g; y = act((x - mean) / sqrt(var + eps) * gamma
 *                + beta).  Statistics in fp32 per slot, fp64 across slots.
 * ------------------------------------------------------------------------------------- */

#define SSC_ACT_NONE 0
#define SSC_ACT_RELU 1
#define SSC_ACT_SILU 2
#define SSC_GN_MAX_BATCH 64

/* What the _ex convolution entry points do after the sum, in this order:
 *   v = act(conv + bias);  v += residual (if any);  store v in out_dtype;
 *   and, if gn_partials != NULL, the group-norm partial sums of the STORED values (as
 *   ssc_gn_partials computes them from out) into gn_partials, ready for ssc_gn_finalize.
 * A zeroed struct (or a NULL pointer) is the plain convolution.
 *   act        SSC_ACT_NONE, SSC_ACT_RELU or SSC_ACT_SILU.
 *   gn_groups  groups of the statistics (1..256, dividing cout); read with gn_partials.
 *   batch      batch entries of the sites (1..SSC_GN_MAX_BATCH); read with gn_partials.
 *   reserved   0.
 *   residual   [n, cout] in out_dtype, 16-byte aligned, rows in coords order, or NULL; may
 *              be the same buffer as out (each row is read before it is written).
 *   coords     [n, 4] int32 sites (their batch ids), 16-byte aligned; needed with
 *              gn_partials when batch > 1.
 *   gn_partials, gn_partials_bytes  >= ssc_gn_partials_bytes(n, batch, gn_groups) bytes,
 *              16-byte aligned; written completely.
 * The k=3 matrix-core kernels sum the statistics in their own epilogue when batch = 1;
 * otherwise one extra pass over out runs after the convolution, on the same stream. */
typedef struct ssc_epilogue {
  int32_t act;
  int32_t gn_groups;
  int32_t batch;
  int32_t reserved;
  const void* residual;
  const int32_t* coords;
  float* gn_partials;
  size_t gn_partials_bytes;
} ssc_epilogue;

/* ssc_subm_conv3d_plan, ssc_subm_conv3d_packed, ssc_linear and ssc_linear_packed with an
 * epilogue (NULL = none); other arguments, shapes and errors as there.  Bad epilogue fields return SSC_ERR_ARG, a
 * short gn_partials buffer SSC_ERR_WORKSPACE. */
ssc_status ssc_subm_conv3d_plan_ex(const void* feats, int32_t in_dtype, const void* weight,
                                   const float* bias, const void* plan, int64_t n,
                                   int32_t cin, int32_t cout, void* out, int32_t out_dtype,
                                   const ssc_epilogue* epilogue, void* workspace,
                                   size_t workspace_bytes, void* stream);
ssc_status ssc_subm_conv3d_packed_ex(const void* feats, const void* packed_weight,
                                     const float* bias, const void* plan, int64_t n,
                                     int32_t cin, int32_t cout, void* out, int32_t out_dtype,
                                     const ssc_epilogue* epilogue, void* stream);
ssc_status ssc_linear_ex(const void* feats, int32_t in_dtype, const void* weight,
                         const float* bias, int64_t n, int32_t cin, int32_t cout, void* out,
                         int32_t out_dtype, const ssc_epilogue* epilogue, void* workspace,
                         size_t workspace_bytes, void* stream);
ssc_status ssc_linear_packed_ex(const void* feats, const void* packed_weight, const float* bias,
                                int64_t n, int32_t cin, int32_t cout, void* out,
                                int32_t out_dtype, const ssc_epilogue* epilogue, void* stream);

/* Bytes of the group-norm partial sums for n sites: one slot per 128 rows of n rounded up
 * to a multiple of 256, each slot holding float4 (count, sum, sum of squares, 0) per
 * (batch entry, group).  0 for bad arguments. */
size_t ssc_gn_partials_bytes(int64_t n, int32_t batch, int32_t groups);

/* Partial sums of x [n, channels] (dtype SSC_F32, SSC_BF16 or SSC_F16) per slot of 128
 * rows, batch entry and group.  coords [n, 4] int32 (batch ids) is needed when batch > 1;
 * sites whose batch id is outside [0, batch) are left out.  The work grows with
 * ceil(batch / 4) passes over x.  partials as for ssc_gn_partials_bytes; written completely. */
ssc_status ssc_gn_partials(const void* x, int32_t dtype, int64_t n, int32_t channels,
                           const int32_t* coords, int32_t batch, int32_t groups,
                           float* partials, size_t partials_bytes, void* stream);

/* stats [batch][groups] float2 = (mean, 1 / sqrt(var + eps)) from partials written for the
 * same n, batch and groups (by ssc_gn_partials or a convolution epilogue); slots are added
 * in fp64 in slot order, the variance is the population variance; an entry without sites
 * gets mean 0 and 1 / sqrt(eps).  Bit-reproducible. */
ssc_status ssc_gn_finalize(const float* partials, int64_t n, int32_t batch, int32_t groups,
                           float eps, float* stats, void* stream);

/* out[i][c] = act((x[i][c] - mean) * rstd * gamma[c] + beta[c]) with (mean, rstd) =
 * stats[b][c / (channels / groups)] for the batch id b of site i (0 when batch = 1, else from
 * coords).  gamma / beta fp32 [channels] or NULL (1 / 0); out in x's dtype, may be x. */
ssc_status ssc_gn_apply(const void* x, int32_t dtype, int64_t n, int32_t channels,
                        const int32_t* coords, int32_t batch, int32_t groups,
                        const float* stats, const float* gamma, const float* beta, int32_t act,
                        void* out, void* stream);

/* LayerNorm32 over each site's channels (LATO.2 MLX port page, "Status" and repository
 * layout: a layer norm with fp32 accumulation), the norm of the ConvNeXt-style block:
 *   out[i][c] = act((x[i][c] - mean_i) / sqrt(var_i + eps) * gamma[c] + beta[c]),
 * mean and population variance of row i over its channels, computed in fp32 (the mean first,
 * then the mean squared deviation).  x [n, channels] SSC_F32 / SSC_BF16 / SSC_F16; out the
 * same dtype, may be x; gamma / beta fp32 [channels] or NULL (1 / 0). */
ssc_status ssc_layer_norm(const void* x, int32_t dtype, int64_t n, int32_t channels,
                          const float* gamma, const float* beta, float eps, int32_t act,
                          void* out, void* stream);

/* ---------------------------------------------------------------------------------------
 * Coordinate-changing neighbours: factor-2 downsample (max pool), its paired upsample, and
 * the x8 subdivide.  Each yields a new coordinate set, indexed cold by ssc_build_index.
 * ------------------------------------------------------------------------------------- */

/* Bytes of scratch workspace ssc_downsample2 needs for n sites. */
size_t ssc_downsample_workspace_bytes(int64_t n);

/* SparseDownsample(2) with the max reduction (LATO.2 page, "Status": a max pool, not an
 * average, as upstream passes reduce="amax").  The parent of site (b,x,y,z) is
 * (b, x>>1, y>>1, z>>1) in the grid (ceil(gx/2), ceil(gy/2), ceil(gz/2)); every distinct
 * parent is one output site, in ascending (b,x,y,z) order; its feature is the channel-wise
 * maximum over its sites (only the sites present; the value returned is one of theirs,
 * bit for bit).
 *   coords     [n, 4] int32 (b,x,y,z), 16-byte aligned, inside batch / grid (as for
 *              ssc_build_index; rows outside are counted in result[1], outputs then undefined).
 *   feats      [n, channels] dtype (SSC_F32, SSC_BF16 or SSC_F16); may be NULL when
 *              channels = 0.
 *   out_coords [n, 4] int32 capacity, 16-byte aligned: rows [0, m) receive the parents.
 *   out_feats  [n, channels] capacity: rows [0, m) receive the maxima.
 *   parent     [n] int32: parent[i] = output row of site i's parent (the cache that
 *              ssc_upsample2 consumes).
 *   result     device int64[2], 8-byte aligned: result[0] = m, result[1] = rows outside the
 *              grid.  Written on the stream (read it after synchronising).
 *   workspace  >= ssc_downsample_workspace_bytes(n) bytes, 256-byte aligned, scratch only.
 * Deterministic: a stable sort by parent. */
ssc_status ssc_downsample2(const int32_t* coords, int64_t n, int32_t batch, const int32_t* grid,
                           const void* feats, int32_t dtype, int32_t channels,
                           int32_t* out_coords, void* out_feats, int32_t* parent, int64_t* result,
                           void* workspace, size_t workspace_bytes, void* stream);

/* SparseSpatial2Channel(2), the sparse pixel unshuffle (Pixal3D README, module table): the
 * parents and parent map of ssc_downsample2, and each parent's row of 8 * channels values
 * holds channel c of its child k = 4(x&1) + 2(y&1) + (z&1) at column c * 8 + k (zero where the
 * child is absent).  Arguments as for ssc_downsample2, with out_feats [n, 8 * channels] of
 * capacity and channels >= 1; the values are moved, never converted. */
ssc_status ssc_spatial2channel2(const int32_t* coords, int64_t n, int32_t batch,
                                const int32_t* grid, const void* feats, int32_t dtype,
                                int32_t channels, int32_t* out_coords, void* out_feats,
                                int32_t* parent, int64_t* result, void* workspace,
                                size_t workspace_bytes, void* stream);

/* SparseUpsample(2), the cache-paired inverse of a downsample (Pixal3D README, module table):
 * out[i] = parent_feats[parent[i]] for the n sites of the finer set.
 *   parent_feats [m, channels] dtype; parent [n] int32 from ssc_downsample2 (entries outside
 *   [0, m) produce zero rows); out [n, channels] dtype.  Rows must be a multiple of 4 bytes. */
ssc_status ssc_upsample2(const void* parent_feats, int32_t dtype, int32_t channels,
                         const int32_t* parent, int64_t n, int64_t m, void* out, void* stream);

/* SparseSubdivide: the x8 coordinate expansion the LATO.2 page uses for upsampling (module
 * table: "upsampling is SparseSubdivide").  Site i becomes the 8 sites 8i + 4dx + 2dy + dz,
 * dx,dy,dz in {0,1}, at (b, 2x+dx, 2y+dy, 2z+dz) in the grid (2gx, 2gy, 2gz), each carrying
 * site i's features.
 *   coords [n, 4] int32 inside the grid (not checked); grid extents <= 32767 (so the
 *   subdivided grid fits the 16-bit key fields), else SSC_ERR_UNSUPPORTED.
 *   feats [n, channels] dtype or NULL with channels = 0; out_coords [8n, 4];
 *   out_feats [8n, channels].  Rows must be a multiple of 4 bytes. */
ssc_status ssc_subdivide2(const int32_t* coords, int64_t n, const int32_t* grid,
                          const void* feats, int32_t dtype, int32_t channels,
                          int32_t* out_coords, void* out_feats, void* stream);

/* ---------------------------------------------------------------------------------------
 * Building blocks of the pages' own convolution designs, for measuring the kernels above
 * against them (the matrix products in between are plain library GEMMs, not part of this
 * library).
 * ------------------------------------------------------------------------------------- */

/* The dense operand of the one-matmul design (LATO.2 MLX port page, "Fleet benchmark"
 * version history: the 27 neighbour rows of every site side by side, one dense matmul):
 *   out[i][t][c] = feats[nbr[i][t]][c], or 0 where nbr[i][t] = -1.
 *   feats [n, channels] dtype (rows a multiple of 16 bytes, else SSC_ERR_UNSUPPORTED),
 *   nbr [n, 27] int32 from ssc_build_index, out [n, 27 * channels] dtype, 16-byte aligned. */
ssc_status ssc_gather_taps(const void* feats, int32_t dtype, int64_t n, int32_t channels,
                           const int32_t* nbr, void* out, void* stream);

/* The scatter of the per-offset design (trellis-mac article, gather-scatter flowchart: per
 * offset, gather the rows that have the neighbour, multiply by W[t], scatter-add):
 *   out[idx[k]][c] += part[k][c] for k < p, c < channels (channels a multiple of 4).
 *   part [p, channels] SSC_F32 or SSC_BF16, idx [p] int32 rows of out (distinct within a
 *   call; rows outside [0, n) are skipped), out [n, channels] fp32, 16-byte aligned. */
ssc_status ssc_scatter_add_rows(const void* part, int32_t part_dtype, const int32_t* idx,
                                int64_t p, int32_t channels, float* out, int64_t n,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSC_H */
