// Sparse grid sampling on gfx950: trilinear weighted sums of voxel feature
// rows at continuous points, and the transposed sums for the feature gradient.
//
// The FlexGEMM pages list a sparse grid_sample operator whose forward and
// backward kernels are index-weighted sums (contributor report, section two:
// the ops.grid_sample and kernels.triton.grid_sample module rows and the
// indice_weighed_sum_fwd / bwd key-function row), with trilinear
// interpolation as the existing mode (the extension section).  Readings used
// here: a point is a float row [b, x, y, z] in voxel-index units (voxel
// [b, x, y, z] sits at the integer point); with x0 = floor(x), t = x - x0,
// corner j = 4 dx + 2 dy + dz is (x0 + dx, y0 + dy, z0 + dz) with weight
// wx * wy * wz, wx = t if dx else 1 - t; a corner that is off the grid or not
// an active voxel adds nothing and the other weights are not renormalised; a
// point whose batch value is not an integer in [0, B) or whose coordinates
// are not finite samples zero.
//
// Design.  A group of L lanes (8..64, a power of two) owns one point: its
// first 8 lanes look up the 8 corners in the plan's voxel hash table at the
// same time and the group shares rows and weights through lane shuffles;
// then each lane streams 16-byte vectors of the 8 corner rows (an absent
// corner reads the plan's zero row, so the loads carry no branch) and
// accumulates in fp32 in corner order.
//
// The backward pass is the same sum transposed.  Scattering weight * dout
// into dfeats with float atomics costs one atomic per (point, corner,
// channel) and is atomic-bound, so it gathers instead: the (point, corner)
// pairs are bucketed by voxel with a counting sort (one integer atomic to
// count and one to place each pair, a device-wide scan between them), then a
// group of lanes per voxel walks its bucket, recomputes each pair's weight
// from the point, gathers the dout rows and writes the voxel's gradient row
// once.  The order of pairs inside a bucket follows the placing atomics, so
// the fp32 summation order (and the last bits) may vary from run to run.

#include <hip/hip_runtime.h>

#include "hash.h"
#include "ssc_internal.h"

namespace ssc {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte vectors of one element type: VEC elements, unpacked to fp32 and
// packed back with round-to-nearest-even
template <int DT>
struct GsVec;

template <>
struct GsVec<SSC_F32> {
  static constexpr int kVec = 4;
  __device__ static void unpack(const u32x4& v, float (&f)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v[e]);
  }
  __device__ static u32x4 pack(const float (&f)[4]) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(f[e]);
    return v;
  }
};

template <>
struct GsVec<SSC_F16> {
  static constexpr int kVec = 8;
  __device__ static float lo(uint32_t u, int h) {
    return float(__builtin_bit_cast(_Float16, uint16_t(h ? (u >> 16) : (u & 0xffffu))));
  }
  __device__ static void unpack(const u32x4& v, float (&f)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = lo(v[e / 2], e & 1);
  }
  __device__ static u32x4 pack(const float (&f)[8]) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = uint32_t(__builtin_bit_cast(uint16_t, _Float16(f[2 * e]))) |
             (uint32_t(__builtin_bit_cast(uint16_t, _Float16(f[2 * e + 1]))) << 16);
    return v;
  }
};

template <>
struct GsVec<SSC_BF16> {
  static constexpr int kVec = 8;
  __device__ static void unpack(const u32x4& v, float (&f)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = bf16_to_f32(uint16_t((e & 1) ? (v[e / 2] >> 16) : (v[e / 2] & 0xffffu)));
  }
  __device__ static u32x4 pack(const float (&f)[8]) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = uint32_t(f32_to_bf16_rne(f[2 * e])) | (uint32_t(f32_to_bf16_rne(f[2 * e + 1])) << 16);
    return v;
  }
};

struct GsGrid {
  int B, X, Y, Z;
};

// The weight of corner j of point p (any point whose corner j was found in
// the table passed the range checks of corner_lookup).
__device__ __forceinline__ float corner_weight(const float4 p, int j) {
  const int dx = (j >> 2) & 1, dy = (j >> 1) & 1, dz = j & 1;
  const float tx = p.y - floorf(p.y), ty = p.z - floorf(p.z), tz = p.w - floorf(p.w);
  const float wx = dx ? tx : 1.f - tx, wy = dy ? ty : 1.f - ty, wz = dz ? tz : 1.f - tz;
  return (wx * wy) * wz;
}

// Corner j of point p: its voxel row, or the sentinel when the point names
// no sample, the corner is off the grid or no voxel sits there.
template <typename KeyT>
__device__ __forceinline__ uint32_t corner_row(const float4 p, int j, const GsGrid g,
                                               const VoxelTable<KeyT>& table) {
  // NaN fails every comparison below, so it lands here too
  if (!(p.x >= 0.f && p.x < float(g.B) && p.x == floorf(p.x))) return kSentinel;
  if (!(p.y > -1.f && p.y < float(g.X) && p.z > -1.f && p.z < float(g.Y) && p.w > -1.f && p.w < float(g.Z)))
    return kSentinel;
  const int cx = int(floorf(p.y)) + ((j >> 2) & 1);
  const int cy = int(floorf(p.z)) + ((j >> 1) & 1);
  const int cz = int(floorf(p.w)) + (j & 1);
  if (cx < 0 || cx >= g.X || cy < 0 || cy >= g.Y || cz < 0 || cz >= g.Z) return kSentinel;
  return voxel_lookup<KeyT>(table, int(p.x), cx, cy, cz);
}

// corner row and weight (0 when absent)
template <typename KeyT>
__device__ __forceinline__ void corner_lookup(const float4 p, int j, const GsGrid g,
                                              const VoxelTable<KeyT>& table,
                                              uint32_t* row, float* w) {
  *row = corner_row<KeyT>(p, j, g, table);
  *w = *row == kSentinel ? 0.f : corner_weight(p, j);
}

// The 8 corners of the group's point, shared from the group's first 8 lanes.
template <typename KeyT, int L>
__device__ __forceinline__ void group_corners(const float4* __restrict__ pts, int64_t p, const GsGrid g,
                                              const VoxelTable<KeyT>& table,
                                              uint32_t (&rows)[8], float (&ws)[8]) {
  static_assert(L >= 8 && L <= 64 && (L & (L - 1)) == 0, "a group is 8..64 lanes, a power of two");
  const int q = threadIdx.x % L;
  uint32_t row = kSentinel;
  float w = 0.f;
  if (q < 8) corner_lookup<KeyT>(pts[p], q, g, table, &row, &w);
  const int first = int(threadIdx.x % 64) - q;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = uint32_t(__shfl(int(row), first + j, 64));
    ws[j] = __shfl(w, first + j, 64);
  }
}

template <int DT, typename KeyT, int L>
__global__ void __launch_bounds__(256) gs_fwd(const u32x4* __restrict__ feats, const float4* __restrict__ pts,
                                              int64_t m, int nvec, const GsGrid g,
                                              const VoxelTable<KeyT> table,
                                              const u32x4* __restrict__ zrow, u32x4* __restrict__ out) {
  using V = GsVec<DT>;
  constexpr int kG = 256 / L;
  const int64_t p = int64_t(blockIdx.x) * kG + threadIdx.x / L;
  if (p >= m) return;  // uniform over the group
  uint32_t rows[8];
  float ws[8];
  group_corners<KeyT, L>(pts, p, g, table, rows, ws);
  for (int v = int(threadIdx.x % L); v < nvec; v += L) {
    u32x4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      x[j] = *(rows[j] != kSentinel ? feats + int64_t(rows[j]) * nvec + v : zrow + v);
    float acc[V::kVec];
#pragma unroll
    for (int e = 0; e < V::kVec; ++e) acc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float f[V::kVec];
      V::unpack(x[j], f);
#pragma unroll
      for (int e = 0; e < V::kVec; ++e) acc[e] = fmaf(ws[j], f[e], acc[e]);
    }
    out[p * nvec + v] = V::pack(acc);
  }
}

// Backward, step 1: one thread per (point, corner) pair t = 8 p + j: the
// corner's row into idx[t] and one count for that voxel.
template <typename KeyT>
__global__ void __launch_bounds__(256) gs_pairs(const float4* __restrict__ pts, int64_t m, const GsGrid g,
                                                const VoxelTable<KeyT> table,
                                                uint32_t* __restrict__ idx, uint32_t* __restrict__ cnt) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= m * 8) return;
  const uint32_t r = corner_row<KeyT>(pts[t >> 3], int(t & 7), g, table);
  idx[t] = r;
  if (r != kSentinel) atomicAdd(&cnt[r], 1u);
}

// Backward, step 2 (after the scan turned the counts into bucket starts):
// place each pair in its voxel's bucket.
__global__ void __launch_bounds__(256) gs_place(const uint32_t* __restrict__ idx, int64_t pairs,
                                                const uint32_t* __restrict__ start, uint32_t* __restrict__ fill,
                                                uint32_t* __restrict__ list) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= pairs) return;
  const uint32_t r = idx[t];
  if (r == kSentinel) return;
  list[start[r] + atomicAdd(&fill[r], 1u)] = uint32_t(t);
}

// Backward, step 3: a group of L lanes per voxel sums weight * dout over its
// bucket, four pairs at a time, and writes the voxel's gradient row.
template <int DT, int L>
__global__ void __launch_bounds__(256) gs_gather(const uint32_t* __restrict__ list,
                                                 const uint32_t* __restrict__ start, int64_t n,
                                                 const float4* __restrict__ pts, const u32x4* __restrict__ dout,
                                                 int nvec, u32x4* __restrict__ dfeats) {
  using V = GsVec<DT>;
  constexpr int kG = 256 / L, kU = 4;
  const int64_t i = int64_t(blockIdx.x) * kG + threadIdx.x / L;
  if (i >= n) return;  // uniform over the group
  const uint32_t b0 = start[i], b1 = start[i + 1];
  for (int v = int(threadIdx.x % L); v < nvec; v += L) {
    float acc[V::kVec];
#pragma unroll
    for (int e = 0; e < V::kVec; ++e) acc[e] = 0.f;
    for (uint32_t k = b0; k < b1; k += kU) {
      uint32_t t[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) t[u] = list[k + u < b1 ? k + u : b1 - 1];
      float4 p[kU];
      u32x4 d[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        p[u] = pts[t[u] >> 3];
        d[u] = dout[int64_t(t[u] >> 3) * nvec + v];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float w = k + u < b1 ? corner_weight(p[u], int(t[u] & 7)) : 0.f;
        float f[V::kVec];
        V::unpack(d[u], f);
#pragma unroll
        for (int e = 0; e < V::kVec; ++e) acc[e] = fmaf(w, f[e], acc[e]);
      }
    }
    dfeats[i * nvec + v] = V::pack(acc);
  }
}

// zero `count` 16-byte vectors (a kernel, not a memset, so the call can be
// captured into a graph)
__global__ void __launch_bounds__(256) gs_zero(u32x4* __restrict__ p, int64_t count) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < count; i += int64_t(gridDim.x) * 256) p[i] = z;
}

unsigned stream_grid(int64_t count) {
  const int64_t b = (count + 255) / 256;
  return unsigned(b < 1 ? 1 : (b > 4096 ? 4096 : b));
}

int group_lanes(int nvec) { return nvec <= 8 ? 8 : nvec <= 16 ? 16 : nvec <= 32 ? 32 : 64; }

template <int DT, typename KeyT>
void launch_fwd(const void* feats, const float* pts, int64_t m, int nvec, GsGrid g, const VoxelTable<KeyT> table,
                const void* zrow, void* out, hipStream_t s) {
  const int L = group_lanes(nvec);
  const unsigned grid = unsigned((m + (256 / L) - 1) / (256 / L));
  const u32x4* f = static_cast<const u32x4*>(feats);
  const float4* p = reinterpret_cast<const float4*>(pts);
  const u32x4* z = static_cast<const u32x4*>(zrow);
  u32x4* o = static_cast<u32x4*>(out);
  if (L == 8) gs_fwd<DT, KeyT, 8><<<grid, 256, 0, s>>>(f, p, m, nvec, g, table, z, o);
  else if (L == 16) gs_fwd<DT, KeyT, 16><<<grid, 256, 0, s>>>(f, p, m, nvec, g, table, z, o);
  else if (L == 32) gs_fwd<DT, KeyT, 32><<<grid, 256, 0, s>>>(f, p, m, nvec, g, table, z, o);
  else gs_fwd<DT, KeyT, 64><<<grid, 256, 0, s>>>(f, p, m, nvec, g, table, z, o);
}

template <int DT>
void launch_gather(const uint32_t* list, const uint32_t* start, int64_t n, const float* pts, const void* dout,
                   int nvec, void* dfeats, hipStream_t s) {
  const int L = group_lanes(nvec);
  const unsigned grid = unsigned((n + (256 / L) - 1) / (256 / L));
  const float4* p = reinterpret_cast<const float4*>(pts);
  const u32x4* d = static_cast<const u32x4*>(dout);
  u32x4* o = static_cast<u32x4*>(dfeats);
  if (L == 8) gs_gather<DT, 8><<<grid, 256, 0, s>>>(list, start, n, p, d, nvec, o);
  else if (L == 16) gs_gather<DT, 16><<<grid, 256, 0, s>>>(list, start, n, p, d, nvec, o);
  else if (L == 32) gs_gather<DT, 32><<<grid, 256, 0, s>>>(list, start, n, p, d, nvec, o);
  else gs_gather<DT, 64><<<grid, 256, 0, s>>>(list, start, n, p, d, nvec, o);
}

template <int DT>
void dispatch_fwd(int kb, const char* plan, const PlanLayout& L, const void* feats, const float* pts, int64_t m,
                  int nvec, GsGrid g, void* out, hipStream_t s) {
  const void* zrow = plan + L.zrow;
  if (kb == 64)
    launch_fwd<DT, uint64_t>(feats, pts, m, nvec, g, voxel_table<uint64_t>(plan, L, g.X, g.Y, g.Z), zrow, out, s);
  else
    launch_fwd<DT, uint32_t>(feats, pts, m, nvec, g, voxel_table<uint32_t>(plan, L, g.X, g.Y, g.Z), zrow, out, s);
}

// workspace of the backward pass: bucket starts (n + 1), fill counters (n),
// the corner row of every pair (8 m), the buckets (8 m), the scan's scratch
struct GsWs {
  size_t start, fill, idx, list, tmp, total;
};

GsWs gs_ws_layout(int64_t n, int64_t m) {
  GsWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  w.start = take(size_t(n + 1) * 4);
  w.fill = take(size_t(n) * 4);
  w.idx = take(size_t(m) * 32);
  w.list = take(size_t(m) * 32);
  w.tmp = take(size_t(scan_tmp_words(n + 1)) * 4);
  w.total = off;
  return w;
}

int esize(int32_t dtype) { return dtype == SSC_F32 ? 4 : 2; }

// checks shared by both passes; on success *kb is the plan's key width
int gs_check(const void* plan, int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z, int32_t key_bits, int32_t C,
             int32_t dtype, int64_t m, int* kb) {
  if (!plan || !aligned16(plan)) return SSC_ERR_INVALID_ARG;
  if (n < 0 || n > SSC_MAX_VOXELS || m < 0 || m > SSC_MAX_POINTS) return SSC_ERR_INVALID_ARG;
  if (!grid_ok(B, X, Y, Z)) return SSC_ERR_INVALID_ARG;
  if (key_bits != 0 && key_bits != 32 && key_bits != 64) return SSC_ERR_INVALID_ARG;
  if (dtype != SSC_F32 && dtype != SSC_F16 && dtype != SSC_BF16) return SSC_ERR_UNSUPPORTED;
  if (C <= 0 || C > 4096 || (int64_t(C) * esize(dtype)) % 16 != 0) return SSC_ERR_UNSUPPORTED;
  *kb = effective_key_bits(B, X, Y, Z, key_bits);
  return *kb < 0 ? SSC_ERR_UNSUPPORTED : SSC_OK;
}

}  // namespace

}  // namespace ssc

using namespace ssc;

extern "C" size_t ssc_grid_sample_workspace_bytes(int64_t n, int64_t m) {
  if (n < 0 || n > SSC_MAX_VOXELS || m < 0 || m > SSC_MAX_POINTS) return 0;
  return gs_ws_layout(n, m).total;
}

extern "C" int ssc_grid_sample_fwd(const void* plan, int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z,
                                   int32_t key_bits, int32_t C, int32_t dtype, const void* feats,
                                   const float* points, int64_t m, void* out, void* stream) {
  int kb = 0;
  const int st = gs_check(plan, n, B, X, Y, Z, key_bits, C, dtype, m, &kb);
  if (st != SSC_OK) return st;
  if (m == 0) return SSC_OK;
  if (!points || !out || !aligned16(points) || !aligned16(out)) return SSC_ERR_INVALID_ARG;
  if (n > 0 && (!feats || !aligned16(feats))) return SSC_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int nvec = int(int64_t(C) * esize(dtype) / 16);
  (void)hipGetLastError();
  if (n == 0) {
    // no voxels: every sample is zero
    gs_zero<<<stream_grid(m * nvec), 256, 0, s>>>(static_cast<u32x4*>(out), m * nvec);
    return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
  }
  const PlanLayout L = plan_layout(n, kb);
  const char* pl = static_cast<const char*>(plan);
  const GsGrid g{B, X, Y, Z};
  if (dtype == SSC_F32) dispatch_fwd<SSC_F32>(kb, pl, L, feats, points, m, nvec, g, out, s);
  else if (dtype == SSC_F16) dispatch_fwd<SSC_F16>(kb, pl, L, feats, points, m, nvec, g, out, s);
  else dispatch_fwd<SSC_BF16>(kb, pl, L, feats, points, m, nvec, g, out, s);
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}

extern "C" int ssc_grid_sample_bwd(const void* plan, int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z,
                                   int32_t key_bits, int32_t C, int32_t dtype, const float* points, int64_t m,
                                   const void* dout, void* dfeats, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  int kb = 0;
  const int st = gs_check(plan, n, B, X, Y, Z, key_bits, C, dtype, m, &kb);
  if (st != SSC_OK) return st;
  if (n == 0) return SSC_OK;
  if (!dfeats || !aligned16(dfeats)) return SSC_ERR_INVALID_ARG;
  if (m > 0 && (!points || !dout || !aligned16(points) || !aligned16(dout))) return SSC_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int nvec = int(int64_t(C) * esize(dtype) / 16);
  (void)hipGetLastError();
  if (m == 0) {
    // no points: the gradient is zero
    gs_zero<<<stream_grid(n * nvec), 256, 0, s>>>(static_cast<u32x4*>(dfeats), n * nvec);
    return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
  }
  if (!workspace || !aligned16(workspace)) return SSC_ERR_INVALID_ARG;
  const GsWs W = gs_ws_layout(n, m);
  if (workspace_bytes < W.total) return SSC_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  uint32_t* start = reinterpret_cast<uint32_t*>(ws + W.start);
  uint32_t* fill = reinterpret_cast<uint32_t*>(ws + W.fill);
  uint32_t* idx = reinterpret_cast<uint32_t*>(ws + W.idx);
  uint32_t* list = reinterpret_cast<uint32_t*>(ws + W.list);
  uint32_t* tmp = reinterpret_cast<uint32_t*>(ws + W.tmp);
  // start and fill are adjacent regions: one zero launch covers both
  const int64_t zvecs = int64_t((W.idx - W.start) / 16);
  gs_zero<<<stream_grid(zvecs), 256, 0, s>>>(reinterpret_cast<u32x4*>(start), zvecs);
  const PlanLayout L = plan_layout(n, kb);
  const char* pl = static_cast<const char*>(plan);
  const GsGrid g{B, X, Y, Z};
  const float4* p4 = reinterpret_cast<const float4*>(points);
  const unsigned pgrid = unsigned((m * 8 + 255) / 256);
  if (kb == 64)
    gs_pairs<uint64_t><<<pgrid, 256, 0, s>>>(p4, m, g, voxel_table<uint64_t>(pl, L, g.X, g.Y, g.Z), idx, start);
  else
    gs_pairs<uint32_t><<<pgrid, 256, 0, s>>>(p4, m, g, voxel_table<uint32_t>(pl, L, g.X, g.Y, g.Z), idx, start);
  launch_scan(start, n + 1, tmp, s);
  gs_place<<<pgrid, 256, 0, s>>>(idx, m * 8, start, fill, list);
  if (dtype == SSC_F32) launch_gather<SSC_F32>(list, start, n, points, dout, nvec, dfeats, s);
  else if (dtype == SSC_F16) launch_gather<SSC_F16>(list, start, n, points, dout, nvec, dfeats, s);
  else launch_gather<SSC_BF16>(list, start, n, points, dout, nvec, dfeats, s);
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}
