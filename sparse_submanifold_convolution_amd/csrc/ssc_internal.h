// Internal declarations shared by the libssc translation units: plan layout,
// constants and small device helpers.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ssc.h"

namespace ssc {

constexpr uint32_t kSentinel = 0xFFFFFFFFu;
constexpr int kV = 27;
constexpr int kCentre = 13;
constexpr uint32_t kPlanMagic = 0x50435353u;  // "SSCP"

// status bits the device sets in the plan header
constexpr uint32_t kBitCoordRange = 1u;
constexpr uint32_t kBitDuplicate = 2u;
constexpr uint32_t kBitHashFull = 4u;

// radix sort: keys per workgroup of the histogram / scatter kernels
constexpr int kSortThreads = 256;
constexpr int kSortItems = 8;       // keys per thread of a large sort
constexpr int kSortItemsSmall = 4;  // of a small one: more, shorter blocks (fewer sequential rounds)
// up to this many sort blocks, radix_scatter reads the histograms directly
constexpr int kSortDirectBlocks = 64;
// sorts of at most kSortSmallKeys keys use kSortItemsSmall (and so the direct path)
constexpr int64_t kSortSmallKeys = int64_t(kSortDirectBlocks) * kSortThreads * kSortItemsSmall;
inline int sort_items_for(int64_t n) { return n <= kSortSmallKeys ? kSortItemsSmall : kSortItems; }
// pair-list build: rows per workgroup
constexpr int kPairRows = 256;
// voxel-table build: voxels per workgroup of the allocation passes
constexpr int kTableBlock = 256;
static_assert((kSortThreads * kSortItemsSmall) % kPairRows == 0, "a row_scan block must lie in one sort block");
// up to this many pair-list blocks, pair_scatter sums the block counts itself
constexpr int kPairDirectBlocks = 256;
// bytes of the plan's all-zero row: the GEMM loads it in place of a missing
// neighbour or an out-of-range weight column, so that no load is conditional
constexpr size_t kZeroRowBytes = 16384;
// device-wide scan: elements per workgroup
constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanBlock = kScanThreads * kScanItems;

// In-place exclusive scan of len uint32 on stream s (three launches); tmp
// holds ceil(len / kScanBlock) + 1 words.  Defined with the plan builder.
// A non-null gate word that reads zero on the device makes the launches no-ops.
void launch_scan(uint32_t* data, int64_t len, uint32_t* tmp, hipStream_t s, const uint32_t* gate = nullptr);
inline int64_t scan_tmp_words(int64_t len) { return (len + kScanBlock - 1) / kScanBlock + 1; }

struct PlanHeader {
  uint32_t magic;
  uint32_t status_bits;
  int64_t n;
  int32_t dims[4];
  int32_t key_bits;
  int32_t zbits;  // bits of the z-order key (batch + interleaved coordinates)
  uint64_t capacity;
  uint32_t pair_count[32];  // [27] used: valid pairs per offset
  uint32_t pair_off[32];    // [28] used: start of each offset's pair list
  // Three-part offset split (see kParts): non-zero when the build sorted the
  // rows again by the masks of parts 0 and 1, so the GEMMs run each part in its
  // own row order.  Decided on the device from the two sums below.
  uint32_t part_split;
  uint32_t reserved;
  unsigned long long union_rows;  // sum over 32-row groups of the main order: 32 * |OR of their masks|
  unsigned long long mask_bits;   // sum over rows of popcount(mask): the valid pairs
};
static_assert(sizeof(PlanHeader) <= 4096, "plan header too large");

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Three-part offset split of the fwd / input-gradient GEMMs.  The 27 offsets
// fall into three runs of nine, part q holding offsets 9q..9q+8.  Part 2 (the
// offsets 18..26) is the top of the 27-bit mask, so the main (mask, z-order)
// row order already groups the rows by their part-2 masks; parts 0 and 1 get
// orders of their own, sorted by (that part's 9-bit mask, z-order).  Each part
// runs the masked GEMM in its order over its offsets only: part 2 into fp32
// sums, part 1 adding to them, part 0 adding them, the bias and the one
// rounding.  With random (volumetric) occupancy the rows of a 256-row tile of
// the main order share few of their low mask bits, and the tile multiplies
// about twice the valid pairs; inside a part a tile spans one or two 9-bit
// masks.  Shells and solids share their masks already and keep one order.
constexpr int kParts = 3;
constexpr int kPartCols = 9;                  // offsets (map columns) per part
constexpr int kOwnOrderParts = kParts - 1;    // parts 0 and 1 have their own row orders
constexpr uint32_t kPartColMask = 0x1FFu;     // a part's mask in its own column space
constexpr uint32_t kTopPartMask = 0x7FC0000u; // part 2 in the main order's 27-bit mask
// the build considers the split from this many rows, with the voxels filling at
// least 1/kPartMaxSparsity of the grid's cells
constexpr int64_t kPartMinRows = 131072;
constexpr int64_t kPartMaxSparsity = 32;
// the split is taken when the main order's 32-row groups multiply at least
// kPartWasteNum / kPartWasteDen times the valid pairs
constexpr unsigned long long kPartWasteNum = 5, kPartWasteDen = 4;
// the GEMMs use it from this many channels on both sides (the MFMA-bound regime)
constexpr int kPartMinChannels = 256;

inline bool part_build_wanted(int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z) {
  const double cells = double(B) * double(X) * double(Y) * double(Z);
  return n >= kPartMinRows && double(n) * double(kPartMaxSparsity) >= cells;
}

inline int ceil_log2_u64(uint64_t v) {
  int e = 0;
  while ((uint64_t(1) << e) < v) ++e;
  return e;
}

// Offsets (bytes from the plan base) of every plan region.  The regions the
// convolution calls read depend on n only and come first.
struct PlanLayout {
  size_t header = 0;
  size_t zrow = 0;    // kZeroRowBytes of zeros (a row of up to 4096 fp32 channels)
  size_t smask = 0;   // [n] u32: neighbour mask of the row at each sorted position
  size_t snmap = 0;   // [n][27] u32: nmap rows in sorted order, snmap[r] = nmap[perm[r]] (strided plans)
  size_t pair_i = 0;  // [27n] u32: pair lists, output row i
  size_t pair_j = 0;  // [27n] u32: pair lists, input row j = nmap[i][k]
  size_t pseg = 0;    // [27][pblk + 1] u32: where each kPairRows block of rows starts in each list
  // row orders of parts 0 and 1 (valid while the header's part_split is set),
  // part q at row offset q * n of each region
  size_t pperm = 0;   // [2][n] i32: original row at each sorted position of the part
  size_t psmask = 0;  // [2][n] u32: the part's 9-bit mask there (bit 9 holds q)
  size_t psnmap = 0;  // [2][n][9] u32: nmap columns 9q..9q+8 in the part's order
  // the voxel table (read by the build's probe and by grid sampling) and build-only scratch
  size_t table = 0;  // [capacity] brick slots: {key, 64-bit occupancy mask}, 16 bytes
  size_t bbase = 0;  // [capacity] u32: first entry of each occupied brick in brows
  size_t brows = 0;  // [n] u32: voxel rows grouped by brick, cells in mask-bit order
  size_t vslot = 0;  // [n] u32: each voxel's brick slot (kCreator set on the voxel that inserted it)
  size_t bcnt = 0;   // [2 (n / 256 + 1) + 1] u32: entries and bricks of each block of 256 voxels, then their scan
  size_t blist = 0;  // [n] u32: slot of each occupied brick, in the order of the voxels that inserted them
  size_t bcoord = 0; // [n] int4: (batch, x / 4, y / 4, z / 4) of each listed brick
  size_t key0 = 0, key1 = 0, val0 = 0, val1 = 0, hist = 0, pcnt = 0, scan_tmp = 0;
  size_t total = 0;
  uint64_t capacity = 0;
  int key_bytes = 4;
  int64_t sort_blocks = 0;
  int sort_items = kSortItems;  // keys per thread of the radix sort
  int64_t pair_blocks = 0;
};

inline PlanLayout conv_layout(int64_t n) {
  PlanLayout L;
  size_t off = 4096;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.header = 0;
  L.zrow = take(kZeroRowBytes);
  L.smask = take(size_t(n) * 4);
  L.snmap = take(size_t(n) * kV * 4);
  L.pair_i = take(size_t(n) * kV * 4);
  L.pair_j = take(size_t(n) * kV * 4);
  L.pseg = take(size_t(kV) * size_t((n + kPairRows - 1) / kPairRows + 1) * 4);
  L.pperm = take(size_t(kOwnOrderParts) * size_t(n) * 4);
  L.psmask = take(size_t(kOwnOrderParts) * size_t(n) * 4);
  L.psnmap = take(size_t(kOwnOrderParts) * size_t(n) * kPartCols * 4);
  L.total = off;
  return L;
}

// parts: the build also sorts the rows of parts 0 and 1 (2n keys at once)
inline PlanLayout plan_layout(int64_t n, int key_bits, bool parts = false) {
  PlanLayout L = conv_layout(n);
  size_t off = L.total;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  // a brick slot per voxel at most: load factor at most 1/2 when every voxel has
  // a brick of its own, far less when bricks hold many voxels
  uint64_t want = uint64_t(n) * 2 < 1024 ? 1024 : uint64_t(n) * 2;
  L.capacity = uint64_t(1) << ceil_log2_u64(want);
  L.key_bytes = key_bits == 64 ? 8 : 4;
  L.sort_items = sort_items_for(n);
  L.sort_blocks = (n + kSortThreads * L.sort_items - 1) / (kSortThreads * L.sort_items);
  L.pair_blocks = (n + kPairRows - 1) / kPairRows;
  L.table = take(L.capacity * 16);
  L.bbase = take(L.capacity * 4);
  L.brows = take(size_t(n) * 4);
  L.vslot = take(size_t(n) * 4);
  L.bcnt = take((2 * (size_t(n) / kTableBlock + 2)) * 4);
  L.blist = take(size_t(n) * 4);
  L.bcoord = take(size_t(n) * 16);
  const size_t nkeys = size_t(n) * (parts ? kOwnOrderParts : 1);
  L.key0 = take(nkeys * 8);
  L.key1 = take(nkeys * 8);
  L.val0 = take(nkeys * 4);
  L.val1 = take(nkeys * 4);
  {
    // multi-block sort: one [256][blocks] histogram (+1 for the scan total);
    // direct sort (few blocks): three rotating ones, see the plan builder
    const size_t one = size_t(L.sort_blocks) * 256;
    size_t need = L.sort_blocks <= kSortDirectBlocks ? 3 * one : one + 1;
    if (need < one + 1) need = one + 1;
    if (parts) {
      // the part sort: multi-block over 2n keys
      const size_t pb = (nkeys + kSortThreads * kSortItems - 1) / (kSortThreads * kSortItems);
      if (need < pb * 256 + 1) need = pb * 256 + 1;
    }
    L.hist = take(need * 4);
  }
  L.pcnt = take((size_t(L.pair_blocks) * kV + 1) * 4);
  size_t scan_len = size_t(L.sort_blocks) * 256 + 1;
  if (parts) {
    // the part sort's histogram: one [256][blocks] table over 2n keys
    const size_t pb = (nkeys + kSortThreads * kSortItems - 1) / (kSortThreads * kSortItems);
    if (pb * 256 + 1 > scan_len) scan_len = pb * 256 + 1;
  }
  if (size_t(L.pair_blocks) * kV + 1 > scan_len) scan_len = size_t(L.pair_blocks) * kV + 1;
  if (2 * (size_t(n) / kTableBlock + 2) > scan_len) scan_len = 2 * (size_t(n) / kTableBlock + 2);
  L.scan_tmp = take(((scan_len + kScanBlock - 1) / kScanBlock + 1) * 4);
  L.total = off;
  return L;
}

// Bits per axis and total bits of the z-order part of the sort key of grid (B, X, Y, Z).
inline void sort_key_bits(int32_t B, int32_t X, int32_t Y, int32_t Z, int* axis_bits, int* zbits) {
  int m = X;
  if (Y > m) m = Y;
  if (Z > m) m = Z;
  *axis_bits = ceil_log2_u64(uint64_t(m));
  *zbits = 3 * *axis_bits + ceil_log2_u64(uint64_t(B));
}

// Moves a plan layout's build-only scratch by delta bytes (its conv regions stay).
inline PlanLayout relocate_scratch(PlanLayout L, size_t delta) {
  L.table += delta;
  L.bbase += delta;
  L.brows += delta;
  L.vslot += delta;
  L.bcnt += delta;
  L.blist += delta;
  L.bcoord += delta;

  L.key0 += delta;
  L.key1 += delta;
  L.val0 += delta;
  L.val1 += delta;
  L.hist += delta;
  L.pcnt += delta;
  L.scan_tmp += delta;
  L.total += delta;
  return L;
}

// A strided (generalised) convolution plan.  Its conv-time regions depend on
// the row counts only and come first: the forward region over the n_out
// output rows (sorted map into the input rows, masks, pair lists), the
// backward region over the n_in input rows (sorted transposed map), the input
// rows' GEMM order and the transposed map itself.  The build scratch of both
// directions (hash tables, sort buffers) follows.
// A 2x2x2 kernel (ks = 2) has 8 offsets: its GEMMs read compact 8-column
// copies of the two sorted maps (the forward map's columns 0..7, the
// transposed map's columns 19..26, whose masks are shifted down to match).
constexpr int kCompactCols = 8;
struct SparseOffsets {
  size_t fwd = 0, bwd = 0, perm_in = 0, tmap = 0, cmap_f = 0, cmap_b = 0, conv_total = 0;
  bool compact = false;
};
inline SparseOffsets sparse_offsets(int64_t n_in, int64_t n_out, int ks) {
  SparseOffsets o;
  o.compact = ks == 2;
  o.fwd = 0;
  o.bwd = align_up(conv_layout(n_out).total, 256);
  o.perm_in = align_up(o.bwd + conv_layout(n_in).total, 256);
  o.tmap = align_up(o.perm_in + size_t(n_in) * 4, 256);
  o.cmap_f = align_up(o.tmap + size_t(n_in) * kV * 4, 256);
  o.cmap_b = align_up(o.cmap_f + (o.compact ? size_t(n_out) * kCompactCols * 4 : 0), 256);
  o.conv_total = align_up(o.cmap_b + (o.compact ? size_t(n_in) * kCompactCols * 4 : 0), 256);
  return o;
}
struct SparseLayout {
  SparseOffsets o;
  PlanLayout f, b;  // relative to base + o.fwd and base + o.bwd, scratch relocated past conv_total
  size_t total = 0;
};
inline SparseLayout sparse_layout(int64_t n_in, int64_t n_out, int kb_in, int kb_out, int ks) {
  SparseLayout S;
  S.o = sparse_offsets(n_in, n_out, ks);
  const PlanLayout f = plan_layout(n_out, kb_out), b = plan_layout(n_in, kb_in);
  const size_t cf = conv_layout(n_out).total, cb = conv_layout(n_in).total;
  size_t off = S.o.conv_total;
  S.f = relocate_scratch(f, off - S.o.fwd - cf);
  off = align_up(S.o.fwd + S.f.total, 256);
  S.b = relocate_scratch(b, off - S.o.bwd - cb);
  S.total = align_up(S.o.bwd + S.b.total, 256);
  return S;
}

// Plan-build steps shared by the submanifold and strided builders (plan builder):
// header, zero row, first sort histogram, sentinel fill of map[n][27], empty
// hash keys of one region
void prepare_region(char* base, const PlanLayout& L, int64_t n, int B, int X, int Y, int Z, int kb, int zbits,
                    uint32_t* map, hipStream_t s);
// coordinate checks and the voxel table of n rows in the region (lookups: also
// group the rows by brick, which the lookups need; without it only the range
// and duplicate checks are made)
void insert_coords(const int4* c4, int64_t n, int B, int X, int Y, int Z, int kb, char* base,
                   const PlanLayout& L, bool lookups, hipStream_t s);
// masks, (mask, z-order) sort -> perm and sorted masks, and (want_pairs) the
// per-offset pair lists, of a [n][27] map whose rows sit at coords in grid
// (B, X, Y, Z); centre: every row has its centre offset (a submanifold map),
// otherwise the sorted-order copy of the map is written too
void order_rows(const int4* c4, const uint32_t* nmap, int64_t n, int B, int X, int Y, int Z, int32_t* perm,
                char* base, const PlanLayout& L, bool want_pairs, bool centre, hipStream_t s);

// round-to-nearest-even float -> bfloat16 bits
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Every third bit: bit i of v (v < 2^21) moves to bit 3i.  The masks are the
// usual public-domain "interleave by magic numbers" steps (halving the shift
// each round); spread3 / gather3 are exact inverses on 21-bit values.
__device__ __forceinline__ uint64_t spread3(uint32_t v) {
  uint64_t x = v & 0x1fffffu;
  x = (x | (x << 32)) & 0x1f00000000ffffull;
  x = (x | (x << 16)) & 0x1f0000ff0000ffull;
  x = (x | (x << 8)) & 0x100f00f00f00f00full;
  x = (x | (x << 4)) & 0x10c30c30c30c30c3ull;
  x = (x | (x << 2)) & 0x1249249249249249ull;
  return x;
}
__device__ __forceinline__ uint32_t gather3(uint64_t x) {
  x &= 0x1249249249249249ull;
  x = (x ^ (x >> 2)) & 0x10c30c30c30c30c3ull;
  x = (x ^ (x >> 4)) & 0x100f00f00f00f00full;
  x = (x ^ (x >> 8)) & 0x1f0000ff0000ffull;
  x = (x ^ (x >> 16)) & 0x1f00000000ffffull;
  x = (x ^ (x >> 32)) & 0x1fffffull;
  return uint32_t(x);
}

// z-order index of (x, y, z) (each below 2^21): bits interleaved from the top,
// each triplet (x, y, z) with x most significant.
__device__ __forceinline__ uint64_t zorder(uint32_t x, uint32_t y, uint32_t z, int /*bits*/) {
  return (spread3(x) << 2) | (spread3(y) << 1) | spread3(z);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace ssc
