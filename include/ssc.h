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
 *    null stream) and returns; ssc_plan_status and ssc_plan_pair_counts
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
  SSC_ERR_HASH_FULL = 7      /* device: the coordinate hash table overflowed */
};

/* Largest number of active voxels one plan may hold (27 * n stays below 2^31). */
#define SSC_MAX_VOXELS (1LL << 26)

/*
 * Bytes of device memory a plan for n voxels needs.  key_bits selects the
 * width of the packed coordinate key ((b*X + x)*Y + y)*Z + z in the hash
 * table: 0 picks 32 bits when B*X*Y*Z <= 2^32 - 1 and 64 bits otherwise (the
 * report's init_hashmap picks uint32 or uint64 by grid volume, section two
 * module table); 32 or 64 force a width (32 fails when the volume does not
 * fit).  Returns 0 for invalid arguments.  Needs no GPU.
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
 * Kernels: coordinate check + hash insert (atomicCAS on 32/64-bit keys),
 * one probe per (voxel, offset) with per-axis bounds checked before any key
 * is packed, mask and sort key, stable LSD radix sort, per-offset pair lists.
 * n == 0 is valid.  Device-side problems are reported by ssc_plan_status.
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
 * Bytes of workspace ssc_subm_conv3d_fwd and ssc_subm_conv3d_bwd need for
 * n voxels and these channel counts (the larger of the two).  Returns 0 for
 * invalid or unsupported arguments.  Needs no GPU.
 */
size_t ssc_conv_workspace_bytes(int64_t n, int32_t Ci, int32_t Co, int32_t dtype);

/*
 * Forward pass: out[n][Co] = the definition of out above.
 *   plan, nmap, perm  as filled by ssc_build_neighbor_map for these n rows.
 *                     The kernels read the plan (its sorted-order copy of
 *                     nmap, the sorted masks, the pair lists) and perm;
 *                     nmap itself is only checked (non-NULL, aligned).
 *   feats  [n][Ci], weight [27][Ci][Co], bias [Co] or NULL (zero), all `dtype`.
 *   out    [n][Co] `dtype`, out.
 * Ci and Co must be multiples of 16 and at most 4096.  The kernel walks
 * tiles of rows in perm order and, per tile, only the offsets some row of
 * the tile has; rows are gathered through the map, products run on MFMA with
 * fp32 accumulation, and out is rounded to `dtype` once.
 */
int ssc_subm_conv3d_fwd(const void* plan, const uint32_t* nmap, const int32_t* perm, int64_t n,
                        int32_t Ci, int32_t Co, int32_t dtype, const void* feats,
                        const void* weight, const void* bias, void* out, void* workspace,
                        size_t workspace_bytes, void* stream);

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

/* Static, human-readable name of a status code (host only). */
const char* ssc_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SSC_H */
