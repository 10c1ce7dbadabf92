/*
 * ssc.h - C ABI of libssc, a 3x3x3 submanifold sparse convolution for AMD
 * Instinct MI355X (gfx950).
 *
 * The operator is FlexGEMM's submanifold convolution,
 * sparse_submanifold_conv3d(feats, coords, shape, weight, bias), whose output
 * sites are its input sites (FlexGEMM contributor report: section one
 * "project positioning"; section two tables of modules and key functions).
 * Its neighbour cache is built once per coordinate set and reused across
 * calls (same report, section two, "how one call flows through the
 * modules").  The forward and backward passes are a masked implicit GEMM
 * over K = 27 * Ci (the Triton compile-cache post, section six: signature
 * of the masked implicit GEMM kernel and its autotune key), with the rows
 * reordered by a sorted_idx permutation.
 *
 * Definitions used by every call (offset index k = (dx+1)*9 + (dy+1)*3 +
 * (dz+1), dx on coordinate column 1; sentinel S = 0xFFFFFFFF):
 *   nmap[i][k] = row of the voxel at coords[i] + offset_k in the same batch,
 *                or S when that voxel is absent or off the grid;
 *   out[i]     = bias + sum_{k: nmap[i][k] != S} X[nmap[i][k]] @ W[k];
 *   dX[j]      = sum over (i, k) with nmap[i][k] = j of W[k] @ dY[i];
 *   dW[k]      = sum_{i: nmap[i][k] != S} outer(X[nmap[i][k]], dY[i]);
 *   dbias      = sum_i dY[i].
 *
 * Conventions for every call:
 *  - Pointers are device pointers unless the argument says "host".
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *    null stream) and returns; ssc_plan_status, ssc_plan_pair_counts and
 *    ssc_plan_row_orders
 *    also synchronise that stream.
 *  - The caller owns and allocates every buffer (coords, nmap, perm, plan,
 *    workspace, outputs).  The library never allocates device memory, keeps
 *    no global state and may be called from several threads on different
 *    buffers.
 *  - Inputs are read-only.  Outputs are overwritten, never accumulated.
 *  - Arrays are row-major and contiguous; device pointers must be 16-byte
 *    aligned.
 *  - Errors a host can see (NULL required pointer, negative or too large
 *    sizes, unsupported dtype or channel count, a buffer that is too small,
 *    misalignment) return at once with nothing enqueued.  Errors only the
 *    device can see (coordinate out of range, duplicate coordinate, hash
 *    table full) are recorded in the plan and reported by ssc_plan_status;
 *    a plan with such an error gives undefined (but memory-safe) results.
 *  - No C++ exception crosses this interface.
 */
#ifndef SSC_H
#define SSC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of feats, weight, bias, dout and all gradients */
enum ssc_dtype {
  SSC_F32 = 0,   /* fp32 in, fp32 MFMA products, fp32 accumulation */
  SSC_F16 = 1,   /* fp16 in, fp32 accumulation, outputs rounded to nearest even */
  SSC_BF16 = 2   /* bf16 in, fp32 accumulation, outputs rounded to nearest even */
};

enum ssc_status {
  SSC_OK = 0,
  SSC_ERR_INVALID_ARG = 1,   /* NULL pointer, bad size, misaligned pointer */
  SSC_ERR_UNSUPPORTED = 2,   /* dtype, channel count or grid outside what the kernels handle */
  SSC_ERR_WORKSPACE = 3,     /* plan or workspace buffer smaller than required */
  SSC_ERR_HIP = 4,           /* a HIP runtime call failed */
  SSC_ERR_COORD_RANGE = 5,   /* device: some coordinate outside [0,B) x [0,X) x [0,Y) x [0,Z) */
  SSC_ERR_DUPLICATE = 6,     /* device: two rows share one coordinate */
  SSC_ERR_HASH_FULL = 7,     /* device: the coordinate hash table overflowed */
  SSC_ERR_SCRATCH = 8        /* the call needs more than the built-in scratch of the no-allocation entry point */
};

/* Largest number of active voxels one plan may hold (27 * n stays below 2^31). */
#define SSC_MAX_VOXELS (1LL << 26)

/*
 * Bytes of device memory a plan for n voxels needs.  key_bits selects the
 * width of the packed coordinate keys of the voxel hash table: 0 picks 32
 * bits when B*X*Y*Z <= 2^32 - 1 and 64 bits otherwise (the report's
 * init_hashmap picks uint32 or uint64 by grid volume, section two module
 * table); 32 or 64 force a width (32 fails when the volume does not fit).
 * The table is keyed by bricks of 4 x 4 x 4 cells, key
 * ((b*X4 + x/4)*Y4 + y/4)*Z4 + z/4 with X4 = ceil(X/4) and so on, each slot
 * holding the brick's 64-bit occupancy mask; the brick grid is never larger
 * than the voxel grid, so the same width holds.  Returns 0 for invalid
 * arguments.  Needs no GPU.
 */
size_t ssc_plan_bytes(int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z, int32_t key_bits);

/*
 * Build the neighbour map, the sorted permutation and the neighbour cache.
 *   coords [n][4] int32 (b, x, y, z), any row order, read-only.
 *   nmap   [n][27] uint32, out: nmap[i][k] as defined above.
 *   perm   [n] int32, out: perm[r] = original row at sorted position r, rows
 *          ascending by (mask, z-order key), where mask = sum_k 2^k over the
 *          offsets whose neighbour exists and the z-order key is
 *          (b << 3m) | interleave(x, y, z) with m = ceil(log2(max(X, Y, Z)))
 *          bits per axis and x the highest bit of each triplet (the
 *          report's z_order_encode in the serialize module; the pages'
 *          sorted_idx).  Coordinates are unique, so perm is unique.
 *   plan   ssc_plan_bytes(...) bytes, out: the neighbour cache that
 *          ssc_subm_conv3d_fwd/bwd read; valid while coords are unchanged.
 * Kernels: coordinate check + insert of each voxel's brick (atomicCAS on
 * 32/64-bit keys, the cell's bit ORed into the slot's occupancy mask), the
 * voxel rows grouped by brick, one lookup per (brick, neighbouring brick)
 * and then every (voxel, offset) entry from the neighbour cell's bit, with
 * per-axis bounds checked before any key is packed; mask and sort key,
 * stable LSD radix sort, per-offset pair lists.  n == 0 is valid.
 * Device-side problems are reported by ssc_plan_status; after such a
 * problem every map entry is still a row index or the sentinel.
 */
int ssc_build_neighbor_map(const int32_t* coords, int64_t n, int32_t B, int32_t X, int32_t Y,
                           int32_t Z, int32_t key_bits, uint32_t* nmap, int32_t* perm,
                           void* plan, size_t plan_bytes, void* stream);

/*
 * Synchronise `stream` and copy the plan's device-detected status into
 * *status_host (host pointer): SSC_OK, SSC_ERR_COORD_RANGE, SSC_ERR_DUPLICATE
 * or SSC_ERR_HASH_FULL (the first that applies, in that order).  Returns
 * SSC_OK when the status could be read.
 */
int ssc_plan_status(const void* plan, void* stream, int32_t* status_host);

/*
 * Synchronise `stream` and copy the number of valid (voxel, offset) pairs of
 * each offset into counts_host[27] (host pointer).  Their sum P is the
 * number of valid-neighbour multiply-accumulate rows: each pass does
 * 2 * P * Ci * Co useful flops.
 */
int ssc_plan_pair_counts(const void* plan, void* stream, int64_t* counts_host);

/*
 * Synchronise `stream` and describe how the built plan orders rows for the
 * masked GEMMs (the pages' sorted_idx and per-block valid offsets: the Triton
 * compile-cache post, section six, kernel signature).  orders_host[0] (host)
 * receives 1 when every offset runs in the one (mask, z-order) row order, or
 * 3 when the build also sorted the rows by the masks of the offsets 0..8 and
 * of 9..17 alone, and the wide-channel fwd / input-gradient GEMMs run those
 * offsets in those orders (and the offsets 18..26 in the first).
 * orders_host[1] and orders_host[2] receive the two sums the build decided it
 * from: 32 times the offsets present in each 32-row group of the first order,
 * summed over the groups, and the valid pairs P (both 0 when the build did not
 * consider it).  The results never depend on it.
 */
int ssc_plan_row_orders(const void* plan, void* stream, int64_t* orders_host);

/*
 * Bytes of workspace ssc_subm_conv3d_fwd and ssc_subm_conv3d_bwd need for
 * n voxels and these channel counts (the larger of the two).  Returns 0 for
 * invalid or unsupported arguments.  Needs no GPU.
 */
size_t ssc_conv_workspace_bytes(int64_t n, int32_t Ci, int32_t Co, int32_t dtype);

/*
 * Forward pass: out[n][Co] = the definition of out above.
 *   plan, nmap, perm  as filled by ssc_build_neighbor_map for these n rows
 *                     (unchanged since).  The kernels read all three: the
 *                     plan's sorted masks, pair lists and row orders, perm,
 *                     and the rows of nmap each tile of sorted rows needs.
 *   feats  [n][Ci], weight [27][Ci][Co], bias [Co] or NULL (zero), all `dtype`.
 *   out    [n][Co] `dtype`, out.
 * Ci and Co must be multiples of 8 (fp16, bf16) or 4 (fp32), so that every
 * row is whole 16-byte vectors, and at most 4096; otherwise
 * SSC_ERR_UNSUPPORTED and nothing is enqueued.  The kernel walks
 * tiles of rows in perm order and, per tile, only the offsets some row of
 * the tile has; rows are gathered through the map, products run on MFMA with
 * fp32 accumulation, and out is rounded to `dtype` once.
 */
int ssc_subm_conv3d_fwd(const void* plan, const uint32_t* nmap, const int32_t* perm, int64_t n,
                        int32_t Ci, int32_t Co, int32_t dtype, const void* feats,
                        const void* weight, const void* bias, void* out, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * ssc_subm_conv3d_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and result without the workspace.  Its
 * workspace is a scratch array of SSC_NOALLOC_SCRATCH_BYTES compiled into the
 * library, one per GPU, held until the process ends; the first call on a GPU
 * looks its address up (no allocation).  Layers whose workspace
 * (ssc_conv_workspace_bytes) exceeds that size return SSC_ERR_SCRATCH and
 * enqueue nothing.  Every call on one GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (on different streams) race; calls ordered
 * on one stream do not.  The array keeps the last call's contents; nothing the
 * forward pass reads from it starts from a previous call's values.
 */
#define SSC_NOALLOC_SCRATCH_BYTES (64LL << 20)
int ssc_subm_conv3d_fwd_noalloc(const void* plan, const uint32_t* nmap, const int32_t* perm, int64_t n,
                                int32_t Ci, int32_t Co, int32_t dtype, const void* feats,
                                const void* weight, const void* bias, void* out, void* stream);

/*
 * Backward pass.  dout [n][Co] is dY.  Each output may be NULL to skip it:
 *   dfeats [n][Ci]       = dX, computed as the forward kernel on dY with the
 *                          offsets flipped (k -> 26 - k) and W[k] transposed;
 *   dweight [27][Ci][Co] = dW, per-offset gather GEMMs over the offset's
 *                          pair list, Split-K over the voxels with partial
 *                          sums reduced in a fixed order (deterministic);
 *   dbias [Co]           = dbias.
 * All `dtype`, accumulated in fp32 and rounded once.
 */
int ssc_subm_conv3d_bwd(const void* plan, const uint32_t* nmap, const int32_t* perm, int64_t n,
                        int32_t Ci, int32_t Co, int32_t dtype, const void* feats,
                        const void* weight, const void* dout, void* dfeats, void* dweight,
                        void* dbias, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Voxel serialisation: encode_seq / decode_seq of the report's serialize
 * module (section two: the ops.serialize and kernels.cuda.serialize rows and
 * the z_order / hilbert encode and decode functions; section three: the
 * serialize snippet, which round-trips coordinates).  Layout of a code, for
 * a grid (B, X, Y, Z) with n = ceil(log2(max(X, Y, Z))) bits per axis:
 *   code = (b << 3n) | index(x, y, z),
 * where index is the z-order index (bits interleaved from the top, x most
 * significant in each triplet -- the key the plan's row sort uses) or the
 * Hilbert index of J. Skilling's transform (AIP Conf. Proc. 707, 2004) with
 * axes (x, y, z), its transposed bits interleaved the same way.  A code is
 * int32 when it needs at most 31 bits, else int64.
 */
enum ssc_seq_mode {
  SSC_SEQ_ZORDER = 0,
  SSC_SEQ_HILBERT = 1
};

/* Bits of a code for this grid, or -1 for invalid dimensions (each in
 * [1, 2^20]).  Needs no GPU. */
int32_t ssc_seq_code_bits(int32_t B, int32_t X, int32_t Y, int32_t Z);

/* 32 or 64: the code width for this grid (32 when the code fits 31 bits);
 * -1 for invalid dimensions or codes wider than 63 bits.  Needs no GPU. */
int32_t ssc_seq_code_width(int32_t B, int32_t X, int32_t Y, int32_t Z);

/*
 * codes[i] = the code of coords[i], or -1 for a row outside the grid.
 *   coords  [n][4] int32 rows (b, x, y, z), 16-byte aligned.
 *   mode    an ssc_seq_mode.
 *   codes   [n] int32 (code_width 32) or int64 (code_width 64), out.
 * code_width may exceed ssc_seq_code_width (64 is always allowed when the
 * grid fits); a narrower width, a bad mode or bad dimensions return
 * SSC_ERR_UNSUPPORTED / SSC_ERR_INVALID_ARG with nothing enqueued.
 */
int ssc_encode_seq(const int32_t* coords, int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z,
                   int32_t mode, void* codes, int32_t code_width, void* stream);

/*
 * coords[i] = the row (b, x, y, z) whose code is codes[i]; (-1, -1, -1, -1)
 * for a negative code or one that names no cell of the grid (the curve
 * covers the cube of side 2^n, which may exceed X, Y or Z).  Same argument
 * rules as ssc_encode_seq; coords [n][4] int32, 16-byte aligned, out.
 */
int ssc_decode_seq(const void* codes, int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z,
                   int32_t mode, int32_t code_width, int32_t* coords, void* stream);

/* ------------------------------------------------------------------------
 * Sparse grid sampling: trilinear interpolation of the features of a voxel
 * set at continuous points (the report's sparse grid_sample operator, whose
 * forward and backward kernels are index-weighted sums; section two, the
 * ops.grid_sample and kernels.triton.grid_sample module rows and the
 * indice_weighed_sum_fwd / bwd key-function row; trilinear is the mode the
 * extension section names).
 *
 * A point is a float row [b, x, y, z] in voxel-index units: voxel
 * [b, x, y, z] sits at the integer point (x, y, z) of sample b.  With
 * x0 = floor(x) and t = x - x0 (likewise y, z), corner j = 4 dx + 2 dy + dz
 * (dx, dy, dz in {0, 1}) is the cell (x0 + dx, y0 + dy, z0 + dz) with weight
 * w_j = wx * wy * wz, wx = t if dx else 1 - t, and
 *   out[m]    = sum_j w_j * feats[row of corner j]      (fwd)
 *   dfeats[i] = sum over (m, j) whose corner is voxel i of w_j * dout[m]  (bwd)
 * A corner off the grid or not among the voxels adds nothing (no
 * renormalisation); a point whose b is not an integer in [0, B) or whose
 * coordinates are not finite samples zero.  Gradients with respect to the
 * points are not computed.
 *
 * plan      a plan from ssc_build_neighbor_map over the same n voxels with
 *           the same B, X, Y, Z and key_bits: its voxel hash table is read.
 * C         channels; C * element bytes must be a multiple of 16, C <= 4096.
 * points    [m][4] float32, 16-byte aligned; m <= SSC_MAX_POINTS.
 * Accumulation is fp32 and outputs are rounded to nearest even.  The
 * forward pass adds the corners in corner order.  The backward pass buckets
 * the (point, corner) pairs by voxel with integer atomics and sums each
 * voxel's bucket in the order the atomics placed it, so the last bits of
 * dfeats can vary from run to run.
 * ------------------------------------------------------------------------ */
#define SSC_MAX_POINTS (1LL << 28)

/* Workspace bytes ssc_grid_sample_bwd needs for n voxels and m points
 * (about 8 n + 64 m); 0 for sizes out of range. */
size_t ssc_grid_sample_workspace_bytes(int64_t n, int64_t m);

/* out [m][C] (dtype), overwritten; feats [n][C].  n == 0 writes zeros. */
int ssc_grid_sample_fwd(const void* plan, int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z,
                        int32_t key_bits, int32_t C, int32_t dtype, const void* feats, const float* points,
                        int64_t m, void* out, void* stream);

/* dfeats [n][C] (dtype), overwritten; dout [m][C]; workspace of
 * ssc_grid_sample_workspace_bytes(n, m) bytes (unused when m == 0, which
 * writes zeros). */
int ssc_grid_sample_bwd(const void* plan, int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z,
                        int32_t key_bits, int32_t C, int32_t dtype, const float* points, int64_t m,
                        const void* dout, void* dfeats, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ------------------------------------------------------------------------
 * Strided (generalised) sparse convolution: the regular sparse_conv3d of
 * the report, whose output sites differ from its input sites and whose map
 * comes from its own sparse_neighbor_map primitive (section two: the
 * ops.spconv and kernels.cuda.spconv module rows; the sparse_conv3d,
 * sparse_conv_[masked_]implicit_gemm[_splitk] and subm / sparse
 * neighbor_map key-function rows).  The same masked implicit GEMM runs it.
 *
 * Geometry, the same on every axis: kernel side ks in {1, 2, 3} (V = ks^3
 * offsets), stride s in [1, 64], padding p in [0, ks).  Offset
 * k = (a*ks + b)*ks + c for window position (a, b, c) in [0, ks)^3 on
 * (x, y, z).  The output grid is (B, Xo, Yo, Zo), Xo = (X + 2p - ks)/s + 1
 * (integer division; every side must be >= 1).  Output site o meets the
 * input site o*s - p + (a, b, c) of the same sample:
 *   nmap[o][k] = row of that input voxel, or S (absent, or off the input
 *                grid); columns k >= V are always S;
 *   out[o]     = bias + sum_{k: nmap[o][k] != S} X[nmap[o][k]] @ W[k];
 *   dX[j]      = sum over (o, k) with nmap[o][k] = j of W[k] @ dY[o];
 *   dW[k]      = sum_o outer(X[nmap[o][k]], dY[o]);  dbias = sum_o dY[o];
 * with W [V][Ci][Co].  With ks = 3, s = 1, p = 1 and the input sites given
 * as the output sites this is the submanifold convolution above.
 * ------------------------------------------------------------------------ */

/* Output-grid sides for this geometry into dims_host[4] (host pointer:
 * B, Xo, Yo, Zo).  Returns SSC_ERR_INVALID_ARG for a bad grid or geometry.
 * Needs no GPU. */
int ssc_sparse_out_shape(int32_t B, int32_t X, int32_t Y, int32_t Z, int32_t ks, int32_t stride, int32_t pad,
                         int32_t* dims_host);

/* Workspace bytes of ssc_sparse_out_count / ssc_sparse_out_coords: one bit
 * per output-grid site plus a count per 32 sites (about B*Xo*Yo*Zo / 4
 * bytes); 0 for invalid arguments or an output grid above 2^38 sites. */
size_t ssc_sparse_out_workspace_bytes(int32_t B, int32_t X, int32_t Y, int32_t Z, int32_t ks, int32_t stride,
                                      int32_t pad);

/*
 * Active output sites, step 1: mark every output site whose window holds
 * an active input (one bit per site), count them and write the count to
 * *count (one int64 in device memory).  coords [n_in][4] int32 rows
 * (b, x, y, z), read-only.  A coordinate outside the input grid makes the
 * count -1.  The caller reads the count, allocates [count][4], then calls
 * ssc_sparse_out_coords with the same workspace, grid and geometry.
 */
int ssc_sparse_out_count(const int32_t* coords, int64_t n_in, int32_t B, int32_t X, int32_t Y, int32_t Z,
                         int32_t ks, int32_t stride, int32_t pad, void* workspace, size_t workspace_bytes,
                         int64_t* count, void* stream);

/* Active output sites, step 2: out_coords [n_out][4] int32, out, in
 * ascending lexicographic (b, x, y, z) order; n_out must be the count of
 * step 1. */
int ssc_sparse_out_coords(const void* workspace, size_t workspace_bytes, int32_t B, int32_t X, int32_t Y,
                          int32_t Z, int32_t ks, int32_t stride, int32_t pad, int32_t* out_coords, int64_t n_out,
                          void* stream);

/* Bytes of a strided-conv plan for n_in input and n_out output rows (the
 * key width rule of ssc_plan_bytes applied to each grid); 0 for invalid
 * arguments.  Needs no GPU. */
size_t ssc_sparse_plan_bytes(int64_t n_in, int64_t n_out, int32_t B, int32_t X, int32_t Y, int32_t Z,
                             int32_t ks, int32_t stride, int32_t pad, int32_t key_bits);

/*
 * Build the strided-conv map and its neighbour cache (sparse_neighbor_map).
 *   coords_in  [n_in][4] int32 input sites in grid (B, X, Y, Z), any order.
 *   coords_out [n_out][4] int32 output sites in the output grid, any order
 *              (from ssc_sparse_out_coords, or the caller's own set).
 *   nmap       [n_out][27] uint32, out, as defined above.
 *   perm_out   [n_out] int32, out: the output rows ascending by (mask,
 *              z-order key over the output grid), as perm of the
 *              submanifold build.
 *   plan       ssc_sparse_plan_bytes(...) bytes, out.  It also holds the
 *              transposed map (per input row, the outputs it feeds, column
 *              26 - k for offset k) in its own GEMM order, which the input
 *              gradient walks.
 * Both coordinate sets must be unique and inside their grids;
 * ssc_sparse_plan_status reports device-detected problems.
 */
int ssc_build_sparse_map(const int32_t* coords_in, int64_t n_in, int32_t B, int32_t X, int32_t Y, int32_t Z,
                         const int32_t* coords_out, int64_t n_out, int32_t ks, int32_t stride, int32_t pad,
                         int32_t key_bits, uint32_t* nmap, int32_t* perm_out, void* plan, size_t plan_bytes,
                         void* stream);

/* As ssc_plan_status, for a strided-conv plan of n_out output rows: the
 * first problem of the output sites, else of the input sites. */
int ssc_sparse_plan_status(const void* plan, int64_t n_out, void* stream, int32_t* status_host);

/* Workspace bytes of ssc_sparse_conv3d_fwd / _bwd; 0 for invalid or
 * unsupported arguments.  Needs no GPU. */
size_t ssc_sparse_conv_workspace_bytes(int64_t n_in, int64_t n_out, int32_t Ci, int32_t Co, int32_t dtype);

/*
 * Forward pass: out [n_out][Co] = the definition above.  plan and perm_out
 * from ssc_build_sparse_map with these n_in, n_out and ks; feats
 * [n_in][Ci], weight [V][Ci][Co], bias [Co] or NULL, all `dtype`.  Channel
 * rules, rounding and kernels as ssc_subm_conv3d_fwd.
 */
int ssc_sparse_conv3d_fwd(const void* plan, int64_t n_in, int64_t n_out, int32_t ks, const int32_t* perm_out,
                          int32_t Ci, int32_t Co, int32_t dtype, const void* feats, const void* weight,
                          const void* bias, void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass; each output may be NULL to skip it: dfeats [n_in][Ci] = dX
 * (the masked implicit GEMM over the input rows through the transposed
 * map), dweight [V][Ci][Co] = dW (pair-list Split-K, deterministic), dbias
 * [Co].  dout [n_out][Co].  All `dtype`, fp32 accumulation.
 */
int ssc_sparse_conv3d_bwd(const void* plan, int64_t n_in, int64_t n_out, int32_t ks, const int32_t* perm_out,
                          int32_t Ci, int32_t Co, int32_t dtype, const void* feats, const void* weight,
                          const void* dout, void* dfeats, void* dweight, void* dbias, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code (host only). */
const char* ssc_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SSC_H */
