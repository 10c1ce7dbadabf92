// Strided (generalised) sparse convolution on gfx950: active output sites and
// the rectangular neighbour map with its neighbour cache.
//
// What the FlexGEMM pages name for this operator (contributor report,
// section two: the ops.spconv and kernels.cuda.spconv module rows and the
// key-function rows sparse_conv3d, sparse_conv_[masked_]implicit_gemm and
// sparse_neighbor_map): a regular sparse convolution whose output sites are
// not its input sites, run by the same masked implicit GEMM through a map
// built by its own primitive.  Geometry, output rule and offset order are the
// readings stated in ssc.h.
//
// Output sites (two calls, the count read by the host in between):
//   os_mark    one thread per (input voxel, window position): the output site
//              whose window holds the voxel at that position, if any, sets its
//              bit in a bitmap over the output grid (read before the atomic, so
//              a set bit costs no atomic)
//   os_count   popcount per 32-site word; a device-wide exclusive scan turns the
//              counts into row starts (and the total)
//   os_emit    one thread per word: its set bits, in increasing linear index
//              (= lexicographic (b, x, y, z) order), become rows
//
// Map and cache (one call):
//   the submanifold builder's region steps, once over the output rows (hash of
//   the output sites for the uniqueness check, sentinel fill of nmap) and once
//   over the input rows (hash of the input sites, sentinel fill of the
//   transposed map), then
//   sparse_probe  one thread per (output row, offset k < V): the input site at
//                 o*s - p + window(k) is looked up once; a hit j fills nmap[o][k]
//                 and the transposed entry tmap[j][26 - k] = o (for one k the map
//                 is injective, so no two threads write one entry)
//   order_rows    masks, radix sort, sorted map and pair lists of each direction

#include <hip/hip_runtime.h>

#include "hash.h"
#include "ssc_internal.h"

namespace ssc {

namespace {

constexpr int kMaxStride = 64;
constexpr uint64_t kMaxOutSites = uint64_t(1) << 36;

inline unsigned blocks_for(int64_t work, int threads) {
  const int64_t b = (work + threads - 1) / threads;
  return unsigned(b < 1 ? 1 : b);
}

bool geometry_ok(int32_t B, int32_t X, int32_t Y, int32_t Z, int ks, int stride, int pad, int32_t* od) {
  if (!grid_ok(B, X, Y, Z)) return false;
  if (ks < 1 || ks > 3 || stride < 1 || stride > kMaxStride || pad < 0 || pad >= ks) return false;
  const int32_t dims[3] = {X, Y, Z};
  od[0] = B;
  for (int a = 0; a < 3; ++a) {
    const int64_t span = int64_t(dims[a]) + 2 * pad - ks;
    if (span < 0) return false;
    od[a + 1] = int32_t(span / stride + 1);
  }
  return true;
}

uint64_t out_sites(const int32_t* od) {
  return uint64_t(od[0]) * uint64_t(od[1]) * uint64_t(od[2]) * uint64_t(od[3]);
}

// workspace of the output-site calls: flag word, bitmap, per-word counts (+1), scan scratch
struct OutLayout {
  size_t flag = 0, bits = 0, cnt = 0, tmp = 0, total = 0;
  int64_t words = 0;
};
OutLayout out_layout(uint64_t sites) {
  OutLayout o;
  o.words = int64_t((sites + 31) / 32);
  size_t off = 256;
  o.bits = off;
  off = align_up(off + size_t(o.words) * 4, 256);
  o.cnt = off;
  off = align_up(off + size_t(o.words + 1) * 4, 256);
  o.tmp = off;
  off = align_up(off + size_t(scan_tmp_words(o.words + 1)) * 4, 256);
  o.total = off;
  return o;
}

}  // namespace

__global__ void __launch_bounds__(256) os_clear(uint32_t* __restrict__ bits, int64_t words,
                                                uint32_t* __restrict__ flag) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t t0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t0 == 0) *flag = 0;
  for (int64_t i = t0; i < words; i += stride) bits[i] = 0;
}

__global__ void __launch_bounds__(256) os_mark(const int4* __restrict__ coords, int64_t n, int B, int X, int Y,
                                               int Z, int ks, int stride, int pad, int Xo, int Yo, int Zo,
                                               uint32_t* __restrict__ bits, uint32_t* __restrict__ flag) {
  const int V = ks * ks * ks;
  const int64_t g = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= n * V) return;
  const int64_t i = g / V;
  const int k = int(g - i * V);
  const int4 c = coords[i];
  if (!coord_ok(c.x, c.y, c.z, c.w, B, X, Y, Z)) {
    if (k == 0) atomicOr(flag, 1u);
    return;
  }
  // window position (a, b, e) of offset k; the voxel is at o*stride - pad + position
  const int a = k / (ks * ks), b = (k / ks) % ks, e = k % ks;
  const int qx = c.y + pad - a, qy = c.z + pad - b, qz = c.w + pad - e;
  if (qx < 0 || qy < 0 || qz < 0) return;
  if (qx % stride || qy % stride || qz % stride) return;
  const int ox = qx / stride, oy = qy / stride, oz = qz / stride;
  if (ox >= Xo || oy >= Yo || oz >= Zo) return;
  const uint64_t L = pack_key(c.x, ox, oy, oz, Xo, Yo, Zo);
  const uint32_t m = 1u << (L & 31u);
  uint32_t* w = bits + (L >> 5);
  // a relaxed atomic read first: a bit that is already set costs no atomic update
  if (!(__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & m)) atomicOr(w, m);
}

__global__ void __launch_bounds__(256) os_count(const uint32_t* __restrict__ bits, int64_t words,
                                                uint32_t* __restrict__ cnt) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < words) cnt[i] = uint32_t(__popc(bits[i]));
  if (i == words) cnt[i] = 0;
}

__global__ void os_total(const uint32_t* __restrict__ cnt, int64_t words, const uint32_t* __restrict__ flag,
                         int64_t* __restrict__ count) {
  if (threadIdx.x == 0) *count = *flag ? int64_t(-1) : int64_t(cnt[words]);
}

__global__ void __launch_bounds__(256) os_emit(const uint32_t* __restrict__ bits, const uint32_t* __restrict__ cnt,
                                               int64_t words, int Xo, int Yo, int Zo, int4* __restrict__ out,
                                               int64_t n_out) {
  const int64_t wi = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (wi >= words) return;
  uint32_t w = bits[wi];
  int64_t row = cnt[wi];
  while (w) {
    const int bit = __ffs(w) - 1;
    w &= w - 1;
    const uint64_t L = uint64_t(wi) * 32 + uint64_t(bit);
    const uint64_t z = L % uint64_t(Zo), r1 = L / uint64_t(Zo);
    const uint64_t y = r1 % uint64_t(Yo), r2 = r1 / uint64_t(Yo);
    const uint64_t x = r2 % uint64_t(Xo), b = r2 / uint64_t(Xo);
    if (row < n_out) out[row] = make_int4(int(b), int(x), int(y), int(z));
    ++row;
  }
}

// One thread per (output row o, offset k < V).  Entries no thread writes keep
// the sentinel of the fill; an output row outside the output grid is left
// empty (the output hash insert has flagged it).
template <typename KeyT>
__global__ void __launch_bounds__(256) sparse_probe(const int4* __restrict__ coords_out, int64_t n_out, int B,
                                                    int Xo, int Yo, int Zo, int X, int Y, int Z, int ks,
                                                    int stride, int pad, const VoxelTable<KeyT> table,
                                                    uint32_t* __restrict__ nmap,
                                                    uint32_t* __restrict__ tmap) {
  const int V = ks * ks * ks;
  const int64_t g = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= n_out * V) return;
  const int64_t o = g / V;
  const int k = int(g - o * V);
  const int4 c = coords_out[o];
  if (!coord_ok(c.x, c.y, c.z, c.w, B, Xo, Yo, Zo)) return;
  const int px = c.y * stride - pad + k / (ks * ks);
  const int py = c.z * stride - pad + (k / ks) % ks;
  const int pz = c.w * stride - pad + k % ks;
  if (px < 0 || px >= X || py < 0 || py >= Y || pz < 0 || pz >= Z) return;
  const uint32_t j = voxel_lookup<KeyT>(table, c.x, px, py, pz);
  if (j == kSentinel) return;
  nmap[o * kV + k] = j;
  tmap[int64_t(j) * kV + (kV - 1 - k)] = uint32_t(o);
}

// The compact copy of a sorted map for a 2x2x2 kernel: out[r][c] =
// snmap[r][col0 + c] for c < 8; with smask given, row r's sorted mask moves
// down by col0 to the same columns (one thread per row touches it).
__global__ void __launch_bounds__(256) compact_map(const uint32_t* __restrict__ snmap, int64_t n, int col0,
                                                   uint32_t* __restrict__ out, uint32_t* __restrict__ smask) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= n * kCompactCols) return;
  const int64_t r = e / kCompactCols;
  const int c = int(e - r * kCompactCols);
  out[e] = snmap[r * kV + col0 + c];
  if (smask && c == 0) smask[r] >>= col0;
}

}  // namespace ssc

using namespace ssc;

extern "C" int ssc_sparse_out_shape(int32_t B, int32_t X, int32_t Y, int32_t Z, int32_t ks, int32_t stride,
                                    int32_t pad, int32_t* dims_host) {
  if (!dims_host) return SSC_ERR_INVALID_ARG;
  int32_t od[4];
  if (!geometry_ok(B, X, Y, Z, ks, stride, pad, od)) return SSC_ERR_INVALID_ARG;
  for (int a = 0; a < 4; ++a) dims_host[a] = od[a];
  return SSC_OK;
}

extern "C" size_t ssc_sparse_out_workspace_bytes(int32_t B, int32_t X, int32_t Y, int32_t Z, int32_t ks,
                                                 int32_t stride, int32_t pad) {
  int32_t od[4];
  if (!geometry_ok(B, X, Y, Z, ks, stride, pad, od)) return 0;
  const uint64_t sites = out_sites(od);
  if (sites > kMaxOutSites) return 0;
  return out_layout(sites).total;
}

extern "C" int ssc_sparse_out_count(const int32_t* coords, int64_t n_in, int32_t B, int32_t X, int32_t Y,
                                    int32_t Z, int32_t ks, int32_t stride, int32_t pad, void* workspace,
                                    size_t workspace_bytes, int64_t* count, void* stream) {
  if (n_in < 0 || n_in > SSC_MAX_VOXELS || !workspace || !count) return SSC_ERR_INVALID_ARG;
  if (n_in > 0 && !coords) return SSC_ERR_INVALID_ARG;
  if (!aligned16(workspace) || (n_in > 0 && !aligned16(coords)) || (reinterpret_cast<uintptr_t>(count) & 7u))
    return SSC_ERR_INVALID_ARG;
  int32_t od[4];
  if (!geometry_ok(B, X, Y, Z, ks, stride, pad, od)) return SSC_ERR_INVALID_ARG;
  const uint64_t sites = out_sites(od);
  if (sites > kMaxOutSites) return SSC_ERR_UNSUPPORTED;
  const OutLayout O = out_layout(sites);
  if (workspace_bytes < O.total) return SSC_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  uint32_t* flag = reinterpret_cast<uint32_t*>(ws + O.flag);
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + O.bits);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws + O.cnt);
  (void)hipGetLastError();
  const unsigned cb = blocks_for(O.words, 256);
  os_clear<<<cb < 4096 ? cb : 4096, 256, 0, s>>>(bits, O.words, flag);
  const int V = ks * ks * ks;
  if (n_in > 0)
    os_mark<<<blocks_for(n_in * V, 256), 256, 0, s>>>(reinterpret_cast<const int4*>(coords), n_in, B, X, Y, Z,
                                                       ks, stride, pad, od[1], od[2], od[3], bits, flag);
  os_count<<<blocks_for(O.words + 1, 256), 256, 0, s>>>(bits, O.words, cnt);
  launch_scan(cnt, O.words + 1, reinterpret_cast<uint32_t*>(ws + O.tmp), s);
  os_total<<<1, 64, 0, s>>>(cnt, O.words, flag, count);
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}

extern "C" int ssc_sparse_out_coords(const void* workspace, size_t workspace_bytes, int32_t B, int32_t X,
                                     int32_t Y, int32_t Z, int32_t ks, int32_t stride, int32_t pad,
                                     int32_t* out_coords, int64_t n_out, void* stream) {
  if (!workspace || n_out < 0 || n_out > SSC_MAX_VOXELS) return SSC_ERR_INVALID_ARG;
  if (n_out > 0 && (!out_coords || !aligned16(out_coords))) return SSC_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return SSC_ERR_INVALID_ARG;
  int32_t od[4];
  if (!geometry_ok(B, X, Y, Z, ks, stride, pad, od)) return SSC_ERR_INVALID_ARG;
  const uint64_t sites = out_sites(od);
  if (sites > kMaxOutSites) return SSC_ERR_UNSUPPORTED;
  const OutLayout O = out_layout(sites);
  if (workspace_bytes < O.total) return SSC_ERR_WORKSPACE;
  if (n_out == 0) return SSC_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const char* ws = static_cast<const char*>(workspace);
  (void)hipGetLastError();
  os_emit<<<blocks_for(O.words, 256), 256, 0, s>>>(reinterpret_cast<const uint32_t*>(ws + O.bits),
                                                    reinterpret_cast<const uint32_t*>(ws + O.cnt), O.words, od[1],
                                                    od[2], od[3], reinterpret_cast<int4*>(out_coords), n_out);
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}

namespace {

// key widths and z-order bits of both grids; false when unsupported
bool sparse_keys(int32_t B, int32_t X, int32_t Y, int32_t Z, const int32_t* od, int32_t key_bits, int* kb_in,
                 int* kb_out) {
  *kb_in = effective_key_bits(B, X, Y, Z, key_bits);
  *kb_out = effective_key_bits(od[0], od[1], od[2], od[3], key_bits);
  if (*kb_in < 0 || *kb_out < 0) return false;
  int ab, zb;
  sort_key_bits(B, X, Y, Z, &ab, &zb);
  if (kV + zb > 64) return false;
  sort_key_bits(od[0], od[1], od[2], od[3], &ab, &zb);
  return kV + zb <= 64;
}

}  // namespace

extern "C" size_t ssc_sparse_plan_bytes(int64_t n_in, int64_t n_out, int32_t B, int32_t X, int32_t Y, int32_t Z,
                                        int32_t ks, int32_t stride, int32_t pad, int32_t key_bits) {
  if (n_in < 0 || n_in > SSC_MAX_VOXELS || n_out < 0 || n_out > SSC_MAX_VOXELS) return 0;
  if (key_bits != 0 && key_bits != 32 && key_bits != 64) return 0;
  int32_t od[4];
  if (!geometry_ok(B, X, Y, Z, ks, stride, pad, od)) return 0;
  int kb_in, kb_out;
  if (!sparse_keys(B, X, Y, Z, od, key_bits, &kb_in, &kb_out)) return 0;
  return sparse_layout(n_in, n_out, kb_in, kb_out, ks).total;
}

extern "C" int ssc_build_sparse_map(const int32_t* coords_in, int64_t n_in, int32_t B, int32_t X, int32_t Y,
                                    int32_t Z, const int32_t* coords_out, int64_t n_out, int32_t ks,
                                    int32_t stride, int32_t pad, int32_t key_bits, uint32_t* nmap,
                                    int32_t* perm_out, void* plan, size_t plan_bytes, void* stream) {
  if (n_in < 0 || n_in > SSC_MAX_VOXELS || n_out < 0 || n_out > SSC_MAX_VOXELS || !plan)
    return SSC_ERR_INVALID_ARG;
  if ((n_in > 0 && !coords_in) || (n_out > 0 && (!coords_out || !nmap || !perm_out))) return SSC_ERR_INVALID_ARG;
  const void* ptrs[] = {coords_in, coords_out, nmap, perm_out, plan};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSC_ERR_INVALID_ARG;
  if (key_bits != 0 && key_bits != 32 && key_bits != 64) return SSC_ERR_INVALID_ARG;
  int32_t od[4];
  if (!geometry_ok(B, X, Y, Z, ks, stride, pad, od)) return SSC_ERR_INVALID_ARG;
  int kb_in, kb_out;
  if (!sparse_keys(B, X, Y, Z, od, key_bits, &kb_in, &kb_out)) return SSC_ERR_UNSUPPORTED;
  const SparseLayout S = sparse_layout(n_in, n_out, kb_in, kb_out, ks);
  if (plan_bytes < S.total) return SSC_ERR_WORKSPACE;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(plan);
  char* fb = base + S.o.fwd;
  char* bb = base + S.o.bwd;
  uint32_t* tmap = reinterpret_cast<uint32_t*>(base + S.o.tmap);
  int32_t* perm_in = reinterpret_cast<int32_t*>(base + S.o.perm_in);
  int ab, zb_out, zb_in;
  sort_key_bits(od[0], od[1], od[2], od[3], &ab, &zb_out);
  sort_key_bits(B, X, Y, Z, &ab, &zb_in);
  const int4* ci = reinterpret_cast<const int4*>(coords_in);
  const int4* co = reinterpret_cast<const int4*>(coords_out);
  (void)hipGetLastError();
  // both regions: header, zero row, first histogram, sentinel fill of the map, empty table
  prepare_region(fb, S.f, n_out, od[0], od[1], od[2], od[3], kb_out, zb_out, n_out > 0 ? nmap : nullptr, s);
  prepare_region(bb, S.b, n_in, B, X, Y, Z, kb_in, zb_in, n_in > 0 ? tmap : nullptr, s);
  // output sites: range and uniqueness checks (their table is not probed); input sites: the probed table
  insert_coords(co, n_out, od[0], od[1], od[2], od[3], kb_out, fb, S.f, false, s);
  insert_coords(ci, n_in, B, X, Y, Z, kb_in, bb, S.b, true, s);
  if (n_out > 0 && n_in > 0) {
    const int V = ks * ks * ks;
    if (kb_in == 64)
      sparse_probe<uint64_t><<<blocks_for(n_out * V, 256), 256, 0, s>>>(
          co, n_out, od[0], od[1], od[2], od[3], X, Y, Z, ks, stride, pad,
          voxel_table<uint64_t>(bb, S.b, X, Y, Z), nmap, tmap);
    else
      sparse_probe<uint32_t><<<blocks_for(n_out * V, 256), 256, 0, s>>>(
          co, n_out, od[0], od[1], od[2], od[3], X, Y, Z, ks, stride, pad,
          voxel_table<uint32_t>(bb, S.b, X, Y, Z), nmap, tmap);
  }
  // GEMM order, sorted maps and (forward direction) the pair lists the weight gradient walks
  order_rows(co, nmap, n_out, od[0], od[1], od[2], od[3], perm_out, fb, S.f, true, false, s);
  order_rows(ci, tmap, n_in, B, X, Y, Z, perm_in, bb, S.b, false, false, s);
  if (S.o.compact) {
    // 8-column copies for the GEMMs: the forward map's columns 0..7, the transposed map's 19..26
    if (n_out > 0)
      compact_map<<<blocks_for(n_out * kCompactCols, 256), 256, 0, s>>>(
          reinterpret_cast<const uint32_t*>(fb + S.f.snmap), n_out, 0,
          reinterpret_cast<uint32_t*>(base + S.o.cmap_f), nullptr);
    if (n_in > 0)
      compact_map<<<blocks_for(n_in * kCompactCols, 256), 256, 0, s>>>(
          reinterpret_cast<const uint32_t*>(bb + S.b.snmap), n_in, kV - kCompactCols,
          reinterpret_cast<uint32_t*>(base + S.o.cmap_b), reinterpret_cast<uint32_t*>(bb + S.b.smask));
  }
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}

extern "C" int ssc_sparse_plan_status(const void* plan, int64_t n_out, void* stream, int32_t* status_host) {
  if (!plan || !status_host || n_out < 0 || n_out > SSC_MAX_VOXELS) return SSC_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return SSC_ERR_HIP;
  const SparseOffsets o = sparse_offsets(0, n_out, 1);  // both headers' places depend on n_out only
  PlanHeader hf, hb;
  const char* base = static_cast<const char*>(plan);
  if (hipMemcpy(&hf, base + o.fwd, sizeof(hf), hipMemcpyDeviceToHost) != hipSuccess) return SSC_ERR_HIP;
  if (hipMemcpy(&hb, base + o.bwd, sizeof(hb), hipMemcpyDeviceToHost) != hipSuccess) return SSC_ERR_HIP;
  if (hf.magic != kPlanMagic || hb.magic != kPlanMagic || hf.n != n_out) return SSC_ERR_INVALID_ARG;
  int32_t st = SSC_OK;
  for (const PlanHeader* h : {&hf, &hb}) {
    if (st != SSC_OK) break;
    if (h->status_bits & kBitCoordRange)
      st = SSC_ERR_COORD_RANGE;
    else if (h->status_bits & kBitDuplicate)
      st = SSC_ERR_DUPLICATE;
    else if (h->status_bits & kBitHashFull)
      st = SSC_ERR_HASH_FULL;
  }
  *status_host = st;
  return SSC_OK;
}
