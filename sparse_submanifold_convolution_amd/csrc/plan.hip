// Neighbour-cache build for the 3x3x3 submanifold convolution on gfx950.
//
// What the FlexGEMM pages name for this stage (contributor report, section
// two: the kernels.cuda.hash, kernels.cuda.serialize and kernels.cuda.spconv
// rows of the module table, and "how one call flows through the modules"):
// a coordinate hashmap (insert, then lookup), the submanifold neighbour map,
// z-order codes, and the masked-implicit-GEMM preprocessing that orders rows
// (sorted_idx) so that tiles of rows share their valid offsets.
//
// Kernels, in launch order:
//   plan_prepare    header fields, status word, pair counters; the zero row;
//                   empty slots (all-ones key, zero mask); the sentinel fill of
//                   a strided map (the submanifold probe writes every entry)
//   brick_insert    coordinate check, key packing of the voxel's 4x4x4 brick;
//                   the workgroup merges its bricks in LDS, then inserts each
//                   once (open addressing, atomicCAS on 32- or 64-bit keys) and
//                   ORs the cells' bits into the slot's occupancy mask (a bit
//                   already set is a duplicate voxel)
//   brick_count /   the bricks' row ranges and list: one scan over the voxels
//   brick_base /    that inserted a brick (each allocating popcount(mask)
//   brick_rows      entries), in voxel order, so deterministic; every voxel
//                   then writes its row at its brick's base + its cell's rank
//   probe_bricks    brick by brick: the 3x3x3 bricks around it looked up once,
//                   then every (voxel, offset k) entry from the neighbour cell's
//                   place in those bricks; whole map rows are written at once
//   fill_orphans    rows no brick wrote become all sentinel (only after an error)
//   row_scan        per row: neighbour mask and 64-bit sort key
//                   (mask << zbits) | zorder; per block: pair-list histogram
//   radix_hist /    stable LSD radix sort, 8 bits a pass, wave64 ballots rank
//   radix_scatter   equal digits; the last pass writes perm and sorted masks;
//                   with few blocks the scatter sums the block histograms itself
//                   instead of a device-wide scan
//   permute_rows    the map in sorted row order (strided plans)
//   pair_scatter    per-offset lists of (i, nmap[i][k]) in increasing i, from the
//                   row_scan histogram, a device-wide scan and a stable scatter
//   scan_*          device-wide exclusive scan of uint32 (three kernels)

#include <hip/hip_runtime.h>

#include "ssc_internal.h"
#include "hash.h"

namespace ssc {

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint64_t lanemask_lt() {
  const unsigned lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// interleave the low `bits` bits of x, y, z: triplet (x, y, z) per bit, x highest

// ---------------------------------------------------------------------------
// device-wide exclusive scan of uint32
// ---------------------------------------------------------------------------

// exclusive scan of one value per thread across the workgroup; returns the total
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds_waves,
                                                         uint32_t* out_excl) {
  const int lane = __lane_id();
  const int wave = threadIdx.x / 64;
  const int nwaves = blockDim.x / 64;
  uint32_t incl = v;
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t t = __shfl_up(incl, d, 64);
    if (lane >= d) incl += t;
  }
  if (lane == 63) lds_waves[wave] = incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
  for (int w = 0; w < nwaves; ++w) {
    uint32_t c = lds_waves[w];
    if (w < wave) before += c;
    total += c;
  }
  *out_excl = before + incl - v;
  __syncthreads();
  return total;
}

// A non-null `gate` word that reads zero turns a launch into a no-op (steps of
// the build that the device decides to skip).
__device__ __forceinline__ bool gated_off(const uint32_t* gate) { return gate && *gate == 0u; }

__global__ void __launch_bounds__(kScanThreads) scan_reduce(const uint32_t* __restrict__ data,
                                                            int64_t len, uint32_t* __restrict__ tmp,
                                                            const uint32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  __shared__ uint32_t waves[kScanThreads / 64];
  const int64_t base = int64_t(blockIdx.x) * kScanBlock;
  // all loads issued before the first use (clamped in range, masked after):
  // a load under a branch would wait for each one in turn
  uint32_t v[kScanItems];
#pragma unroll
  for (int e = 0; e < kScanItems; ++e) {
    const int64_t idx = base + int64_t(e) * kScanThreads + threadIdx.x;
    v[e] = data[idx < len ? idx : len - 1];
  }
  uint32_t s = 0;
#pragma unroll
  for (int e = 0; e < kScanItems; ++e)
    s += (base + int64_t(e) * kScanThreads + threadIdx.x < len) ? v[e] : 0u;
  uint32_t excl;
  uint32_t total = block_exclusive_scan(s, waves, &excl);
  if (threadIdx.x == 0) tmp[blockIdx.x] = total;
}

// one workgroup: exclusive scan of the block sums, in chunks with a carry
__global__ void __launch_bounds__(kScanThreads) scan_top(uint32_t* __restrict__ tmp, int64_t nb,
                                                         const uint32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  __shared__ uint32_t waves[kScanThreads / 64];
  uint32_t carry = 0;
  for (int64_t c0 = 0; c0 < nb; c0 += kScanThreads) {
    int64_t idx = c0 + threadIdx.x;
    uint32_t v = idx < nb ? tmp[idx] : 0u;
    uint32_t excl;
    uint32_t total = block_exclusive_scan(v, waves, &excl);
    if (idx < nb) tmp[idx] = carry + excl;
    carry += total;
  }
}

__global__ void __launch_bounds__(kScanThreads) scan_apply(uint32_t* __restrict__ data, int64_t len,
                                                           const uint32_t* __restrict__ tmp,
                                                           const uint32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  __shared__ uint32_t waves[kScanThreads / 64];
  const int64_t base = int64_t(blockIdx.x) * kScanBlock + int64_t(threadIdx.x) * kScanItems;
  uint32_t v[kScanItems];
  uint32_t s = 0;
#pragma unroll
  for (int e = 0; e < kScanItems; ++e) {
    const int64_t idx = base + e;
    v[e] = data[idx < len ? idx : len - 1];
  }
#pragma unroll
  for (int e = 0; e < kScanItems; ++e) {
    v[e] = base + e < len ? v[e] : 0u;
    s += v[e];
  }
  uint32_t excl;
  block_exclusive_scan(s, waves, &excl);
  uint32_t run = (tmp ? tmp[blockIdx.x] : 0u) + excl;
#pragma unroll
  for (int e = 0; e < kScanItems; ++e) {
    int64_t idx = base + e;
    if (idx < len) data[idx] = run;
    run += v[e];
  }
}

void launch_scan(uint32_t* data, int64_t len, uint32_t* tmp, hipStream_t s, const uint32_t* gate) {
  if (len <= 0) return;
  const int64_t nb = (len + kScanBlock - 1) / kScanBlock;
  if (nb == 1) {
    // one workgroup's worth: a single launch with no block offsets
    scan_apply<<<dim3(1), dim3(kScanThreads), 0, s>>>(data, len, nullptr, gate);
    return;
  }
  scan_reduce<<<dim3(unsigned(nb)), dim3(kScanThreads), 0, s>>>(data, len, tmp, gate);
  scan_top<<<dim3(1), dim3(kScanThreads), 0, s>>>(tmp, nb, gate);
  scan_apply<<<dim3(unsigned(nb)), dim3(kScanThreads), 0, s>>>(data, len, tmp, gate);
}

// ---------------------------------------------------------------------------
// header, fills, hash insert, probe
// ---------------------------------------------------------------------------

// Header fields, status word and pair counters (block 0), the sentinel fill of
// nmap and the empty fill of the hash keys, in one grid-stride kernel.
template <typename KeyT>
__global__ void __launch_bounds__(256) plan_prepare(PlanHeader* h, int64_t n, int B, int X, int Y, int Z,
                                                   int key_bits, int zbits, uint64_t capacity,
                                                   uint32_t* __restrict__ nmap, BrickSlot<KeyT>* __restrict__ table,
                                                   uint4* __restrict__ zrow, uint32_t* __restrict__ hzero,
                                                   int64_t hzero_len) {
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0) {
      h->magic = kPlanMagic;
      h->status_bits = 0;
      h->n = n;
      h->dims[0] = B;
      h->dims[1] = X;
      h->dims[2] = Y;
      h->dims[3] = Z;
      h->key_bits = key_bits;
      h->zbits = zbits;
      h->capacity = capacity;
      h->part_split = 0;
      h->union_rows = 0;
      h->mask_bits = 0;
    }
    if (threadIdx.x < 32) {
      h->pair_count[threadIdx.x] = 0;
      h->pair_off[threadIdx.x] = 0;
    }
  }
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t t0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (int64_t i = t0; i < int64_t(kZeroRowBytes / 16); i += stride) zrow[i] = make_uint4(0, 0, 0, 0);
  for (int64_t i = t0; i < hzero_len; i += stride) hzero[i] = 0;
  if (nmap)
    for (int64_t i = t0; i < n * kV; i += stride) nmap[i] = kSentinel;
  // whole slots (one aligned 16-byte store each): empty key, empty mask
  BrickSlot<KeyT> empty{};
  empty.key = empty_key<KeyT>();
  for (int64_t i = t0; i < int64_t(capacity); i += stride) table[i] = empty;
}

__device__ __forceinline__ unsigned long long cas_key(uint32_t* p, unsigned long long expect,
                                                     unsigned long long want) {
  return atomicCAS(p, uint32_t(expect), uint32_t(want));
}
__device__ __forceinline__ unsigned long long cas_key(unsigned long long* p, unsigned long long expect,
                                                     unsigned long long want) {
  return atomicCAS(p, expect, want);
}

// One thread per voxel.  The workgroup first merges its voxels' bricks in a
// small LDS table (keys, OR of the cell bits), then inserts each distinct
// brick of the group once into the global table: one CAS and one atomicOr per
// (group, brick) instead of per voxel.  A cell bit met twice, in the group or
// already in the global mask, is a duplicate voxel.  The voxel that put a key
// into the LDS table of the group that created the brick is its creator.
constexpr int kInsertSlots = 512;  // LDS slots: at most 256 keys, load factor at most 1/2
template <typename KeyT>
__global__ void __launch_bounds__(256) brick_insert(const int4* __restrict__ coords, int64_t n,
                                                    int B, int X, int Y, int Z,
                                                    BrickSlot<KeyT>* __restrict__ table, uint64_t capacity,
                                                    uint32_t* __restrict__ vslot, uint32_t* __restrict__ status) {
  constexpr unsigned long long kNone = ~0ull;  // no brick key is all ones
  __shared__ unsigned long long lkey[kInsertSlots];
  __shared__ unsigned long long lmask[kInsertSlots];
  __shared__ uint32_t lslot[kInsertSlots];
  for (int e = threadIdx.x; e < kInsertSlots; e += 256) {
    lkey[e] = kNone;
    lmask[e] = 0ull;
  }
  __syncthreads();
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const bool in = i < n;
  const int4 c = in ? coords[i] : make_int4(0, 0, 0, 0);
  const bool ok = in && coord_ok(c.x, c.y, c.z, c.w, B, X, Y, Z);
  if (in && !ok) atomicOr(status, kBitCoordRange);
  int mine = 0;
  bool first = false, dup = false;
  if (ok) {
    const unsigned long long key = brick_key(c.x, c.y, c.z, c.w, X, Y, Z);
    uint32_t h = mix_hash(KeyT(key)) & uint32_t(kInsertSlots - 1);
    // at most 256 distinct keys in kInsertSlots slots: the walk ends
    for (;;) {
      const unsigned long long was = atomicCAS(&lkey[h], kNone, key);
      if (was == kNone) {
        first = true;
        break;
      }
      if (was == key) break;
      h = (h + 1) & uint32_t(kInsertSlots - 1);
    }
    mine = int(h);
    const unsigned long long bit = 1ull << brick_bit(c.y, c.z, c.w);
    if (atomicOr(&lmask[h], bit) & bit) dup = true;
  }
  __syncthreads();
  const uint64_t cm = capacity - 1;
  for (int e = threadIdx.x; e < kInsertSlots; e += 256) {
    const unsigned long long key = lkey[e];
    if (key == kNone) continue;
    uint64_t slot = mix_hash(KeyT(key)) & cm;
    uint32_t created = 0;
    uint64_t probe = 0;
    for (; probe < capacity; ++probe) {
      const unsigned long long was = cas_key(&table[slot].key, (unsigned long long)empty_key<KeyT>(), key);
      if (was == (unsigned long long)empty_key<KeyT>()) {
        created = kCreator;
        break;
      }
      if (was == key) break;
      slot = (slot + 1) & cm;
    }
    if (probe == capacity) {
      atomicOr(status, kBitHashFull);
      lslot[e] = kSentinel;
      continue;
    }
    const unsigned long long m = lmask[e];
    if (atomicOr(&table[slot].mask, m) & m) dup = true;
    lslot[e] = uint32_t(slot) | created;
  }
  __syncthreads();
  if (dup) atomicOr(status, kBitDuplicate);
  if (in) {
    uint32_t v = kSentinel;
    if (ok) {
      const uint32_t g = lslot[mine];
      if (g != kSentinel) v = first ? g : (g & ~kCreator);
    }
    vslot[i] = v;
  }
}

// Entries a voxel allocates in brows: its brick's voxel count if it inserted
// the brick, else none.
template <typename KeyT>
__device__ __forceinline__ uint32_t brick_alloc(const uint32_t* __restrict__ vslot,
                                                const BrickSlot<KeyT>* __restrict__ table, int64_t i, int64_t n,
                                                uint32_t* slot) {
  const uint32_t v = i < n ? vslot[i] : kSentinel;
  *slot = v & ~kCreator;
  if (v == kSentinel || !(v & kCreator)) return 0u;
  return uint32_t(__popcll(table[v & ~kCreator].mask));
}

// Per block of kTableBlock voxels: the entries it allocates in brows
// (bcnt[b]) and the bricks it inserted (bcnt[nb + b]); bcnt[2 nb] = 0, so one
// exclusive scan over the 2 nb + 1 words gives both prefix sums (the second
// offset by the total of the first).  Inside a block the two counts share one
// word (entries in the low 16 bits: at most 256 x 64).
template <typename KeyT>
__global__ void __launch_bounds__(kTableBlock) brick_count(const uint32_t* __restrict__ vslot, int64_t n,
                                                           const BrickSlot<KeyT>* __restrict__ table,
                                                           uint32_t* __restrict__ bcnt, int64_t nb) {
  __shared__ uint32_t waves[kTableBlock / 64];
  uint32_t slot, excl;
  const uint32_t c = brick_alloc<KeyT>(vslot, table, int64_t(blockIdx.x) * kTableBlock + threadIdx.x, n, &slot);
  const uint32_t total = block_exclusive_scan(c ? (1u << 16) | c : 0u, waves, &excl);
  if (threadIdx.x == 0) {
    bcnt[blockIdx.x] = total & 0xFFFFu;
    bcnt[nb + blockIdx.x] = total >> 16;
    if (blockIdx.x == 0) bcnt[2 * nb] = 0;
  }
}

// Each inserting voxel: its brick's first entry in brows, and the brick's
// place in the list of bricks (slot and brick coordinates), both in voxel
// order.
template <typename KeyT>
__global__ void __launch_bounds__(kTableBlock) brick_base(const int4* __restrict__ coords,
                                                          const uint32_t* __restrict__ vslot, int64_t n,
                                                          const BrickSlot<KeyT>* __restrict__ table,
                                                          const uint32_t* __restrict__ bcnt, int64_t nb,
                                                          uint32_t* __restrict__ bbase, uint32_t* __restrict__ blist,
                                                          int4* __restrict__ bcoord) {
  __shared__ uint32_t waves[kTableBlock / 64];
  uint32_t slot, excl;
  const int64_t i = int64_t(blockIdx.x) * kTableBlock + threadIdx.x;
  const uint32_t c = brick_alloc<KeyT>(vslot, table, i, n, &slot);
  block_exclusive_scan(c ? (1u << 16) | c : 0u, waves, &excl);
  if (c) {
    bbase[slot] = bcnt[blockIdx.x] + (excl & 0xFFFFu);
    const uint32_t id = bcnt[nb + blockIdx.x] - bcnt[nb] + (excl >> 16);
    blist[id] = slot;
    const int4 v = coords[i];
    bcoord[id] = make_int4(v.x, v.y >> kBrickShift, v.z >> kBrickShift, v.w >> kBrickShift);
  }
}

// every voxel: its row at its brick's base + the rank of its cell bit
template <typename KeyT>
__global__ void __launch_bounds__(256) brick_rows(const int4* __restrict__ coords, const uint32_t* __restrict__ vslot,
                                                  int64_t n, const BrickSlot<KeyT>* __restrict__ table,
                                                  const uint32_t* __restrict__ bbase, uint32_t* __restrict__ brows) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t v = vslot[i];
  if (v == kSentinel) return;
  const uint32_t slot = v & ~kCreator;
  const int4 c = coords[i];
  const unsigned long long m = table[slot].mask;
  const int bit = brick_bit(c.y, c.z, c.w);
  brows[bbase[slot] + uint32_t(__popcll(m & ((1ull << bit) - 1ull)))] = uint32_t(i);
}

// Position of the q-th set bit (q < popcount(m)) of m.
__device__ __forceinline__ int nth_set_bit(unsigned long long m, int q) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const int c = __popcll(m & ((1ull << w) - 1ull));
    if (q >= c) {
      q -= c;
      m >>= w;
      pos += w;
    }
  }
  return pos;
}

// The neighbour map brick by brick.  A wave takes two listed bricks at a time:
// in each half, lanes 0..26 look up the 3x3x3 bricks around its brick (lane 13
// is the brick itself) and keep their masks and row bases in registers.  Then
// the wave walks each brick's items (occupied cell q, offset k), 64 per round
// and kUnroll rounds at once: the neighbour cell's brick and bit follow from
// the cell's place in the brick, that brick's mask and base come from the lane
// holding it, and the row from the grouped rows.  A voxel's 27 entries are
// written by consecutive lanes, so whole map rows are stored at once and the
// map needs no fill beforehand.
constexpr int kProbeUnroll = 4;
template <typename KeyT>
__global__ void __launch_bounds__(256) probe_bricks(int X, int Y, int Z, const VoxelTable<KeyT> t,
                                                    const uint32_t* __restrict__ blist,
                                                    const int4* __restrict__ bcoord,
                                                    const uint32_t* __restrict__ bcnt, int64_t nb,
                                                    uint32_t* __restrict__ nmap) {
  const int lane = int(__lane_id());
  const int half = lane >> 5, hl = lane & 31;
  const int64_t nw = int64_t(gridDim.x) * (blockDim.x / 64);
  const int64_t nbricks = int64_t(bcnt[2 * nb]) - int64_t(bcnt[nb]);
  const int BX = (X + 3) >> kBrickShift, BY = (Y + 3) >> kBrickShift, BZ = (Z + 3) >> kBrickShift;
  const int ox = hl / 9 - 1, oy = (hl / 3) % 3 - 1, oz = hl % 3 - 1;
  for (int64_t b = 2 * (int64_t(blockIdx.x) * (blockDim.x / 64) + threadIdx.x / 64); b < nbricks; b += 2 * nw) {
    // set-up of this half's brick
    const int64_t hb = b + half;
    unsigned long long nm = 0ull;
    uint32_t nbase = 0u;
    if (hb < nbricks && hl < kV) {
      if (hl == 13) {
        const uint32_t slot = blist[hb];
        nm = t.slots[slot].mask;
        nbase = t.base[slot];
      } else {
        const int4 bc = bcoord[hb];
        const int nx = bc.y + ox, ny = bc.z + oy, nz = bc.w + oz;
        if (nx >= 0 && nx < BX && ny >= 0 && ny < BY && nz >= 0 && nz < BZ) {
          unsigned long long m;
          const uint32_t s =
              find_brick<KeyT>(t.slots, t.capacity, KeyT(pack_key(bc.x, nx, ny, nz, BX, BY, BZ)), &m);
          if (s != kSentinel) {
            nm = m;
            nbase = t.base[s];
          }
        }
      }
    }
    const uint32_t nm_lo = uint32_t(nm), nm_hi = uint32_t(nm >> 32);
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      if (b + h >= nbricks) break;
      const int src = 32 * h;
      const unsigned long long m0 = (unsigned long long)__shfl(nm_lo, src + 13, 64) |
                                    ((unsigned long long)__shfl(nm_hi, src + 13, 64) << 32);
      const uint32_t base0 = __shfl(nbase, src + 13, 64);
      const int total = __popcll(m0) * kV;
#pragma unroll 1
      for (int t0 = 0; t0 < total; t0 += 64 * kProbeUnroll) {
        uint32_t ri[kProbeUnroll], rj[kProbeUnroll], jok[kProbeUnroll];
        int kk[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
          const int it = t0 + 64 * u + lane;
          const int item = it < total ? it : 0;
          const int q = item / kV, k = item - q * kV;
          const int cell = nth_set_bit(m0, q);
          const int nx = (cell >> 4) + k / 9 - 1, ny = ((cell >> 2) & 3) + (k / 3) % 3 - 1, nz = (cell & 3) + k % 3 - 1;
          // each of nx, ny, nz lies in -1..4: the brick among the 27, then the cell in it
          const int d = src + ((nx >> 2) + 1) * 9 + ((ny >> 2) + 1) * 3 + ((nz >> 2) + 1);
          const unsigned long long m = (unsigned long long)__shfl(nm_lo, d, 64) |
                                       ((unsigned long long)__shfl(nm_hi, d, 64) << 32);
          const uint32_t nbs = __shfl(nbase, d, 64);
          const int bit = brick_bit(nx & 3, ny & 3, nz & 3);
          jok[u] = uint32_t((m >> bit) & 1ull);
          // both loads unconditional (a present row, or this brick's first one)
          ri[u] = base0 + uint32_t(q);
          rj[u] = jok[u] ? nbs + uint32_t(__popcll(m & ((1ull << bit) - 1ull))) : base0;
          kk[u] = it < total ? k : -1;
        }
        uint32_t vi[kProbeUnroll], vj[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
          vi[u] = t.rows[ri[u]];
          vj[u] = t.rows[rj[u]];
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
          if (kk[u] >= 0) nmap[int64_t(vi[u]) * kV + kk[u]] = jok[u] ? vj[u] : kSentinel;
      }
    }
  }
}

// Rows no brick wrote (coordinates out of range, a full table, the second of
// two voxels on one cell) become all sentinel.  Runs only when the build
// flagged such a voxel.
template <typename KeyT>
__global__ void __launch_bounds__(256) fill_orphans(const int4* __restrict__ coords, const uint32_t* __restrict__ vslot,
                                                    int64_t n, const VoxelTable<KeyT> t,
                                                    const uint32_t* __restrict__ status, uint32_t* __restrict__ nmap) {
  if ((*status & (kBitCoordRange | kBitDuplicate | kBitHashFull)) == 0u) return;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t v = vslot[i];
  bool orphan = v == kSentinel;
  if (!orphan) {
    const uint32_t slot = v & ~kCreator;
    const int4 c = coords[i];
    orphan = brick_row(t.base, t.rows, slot, t.slots[slot].mask, brick_bit(c.y, c.z, c.w)) != uint32_t(i);
  }
  if (orphan)
    for (int k = 0; k < kV; ++k) nmap[i * kV + k] = kSentinel;
}

// Rows of nmap in blocks of kPairRows, read cooperatively through LDS so the
// loads coalesce.  Per row: the neighbour mask and the 64-bit sort key
// (mask << zbits) | (b << 3*axis_bits) | zorder(x, y, z).  Per block: the
// number of valid entries of each offset (the pair-list histogram).
// The block's rows of nmap (up to 256 x kV entries) into LDS.  The loads of
// all kV rounds are issued before the first store, so the copy costs one
// memory round trip instead of kV.
__device__ __forceinline__ void fetch_rows(const uint32_t* __restrict__ nmap, int64_t row0, int64_t here,
                                           uint32_t (&v)[kV]) {
  const int64_t lim = here * kV;
#pragma unroll
  for (int t = 0; t < kV; ++t) {
    const int64_t e = int64_t(t) * 256 + threadIdx.x;
    v[t] = e < lim ? nmap[row0 * kV + e] : kSentinel;
  }
}
__device__ __forceinline__ void store_rows(uint32_t* rows, const uint32_t (&v)[kV]) {
#pragma unroll
  for (int t = 0; t < kV; ++t) rows[t * 256 + threadIdx.x] = v[t];
}

// Without bit 13 of the mask in the key (squeeze): where every row has its
// centre offset that bit is constant and the order is the same with one key
// bit, and often one radix pass, fewer.
__device__ __forceinline__ uint32_t squeeze_centre(uint32_t m) {
  return (m & ((1u << kCentre) - 1u)) | ((m >> 1) & ~((1u << kCentre) - 1u));
}
__device__ __forceinline__ uint32_t expand_centre(uint32_t v) {
  return (v & ((1u << kCentre) - 1u)) | ((v & ~((1u << kCentre) - 1u)) << 1) | (1u << kCentre);
}

__global__ void __launch_bounds__(256) row_scan(const int4* __restrict__ coords, const uint32_t* __restrict__ nmap,
                                                int64_t n, int B, int X, int Y, int Z, int axis_bits, int zbits,
                                                uint64_t* __restrict__ sort_key, uint32_t* __restrict__ pcnt,
                                                int64_t pblk, uint32_t* __restrict__ h0, uint32_t* __restrict__ h1,
                                                int64_t nsb, int sort_block_keys, int squeeze) {
  __shared__ uint32_t rows[256 * kV];
  __shared__ uint32_t cnt[32];
  __shared__ uint32_t dcnt[256];
  if (threadIdx.x < 32) cnt[threadIdx.x] = 0;
  dcnt[threadIdx.x] = 0;
  if (h1) {
    // the direct sort's next histogram starts at zero
    for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < nsb * 256; e += int64_t(gridDim.x) * 256)
      h1[e] = 0;
  }
  uint32_t local[kV];
#pragma unroll
  for (int k = 0; k < kV; ++k) local[k] = 0;
  static_assert(kPairRows == 256, "one row per thread");
  {
    const int64_t row0 = int64_t(blockIdx.x) * kPairRows;
    const int64_t here = (n - row0) < 256 ? (n - row0) : 256;
    const int4 c = threadIdx.x < here ? coords[row0 + threadIdx.x] : make_int4(0, 0, 0, 0);
    uint32_t v[kV];
    fetch_rows(nmap, row0, here, v);
    store_rows(rows, v);
    __syncthreads();
    if (threadIdx.x < here) {
      const int64_t i = row0 + threadIdx.x;
      uint32_t mask = 0;
#pragma unroll
      for (int k = 0; k < kV; ++k) {
        const bool v = rows[threadIdx.x * kV + k] != kSentinel;
        mask |= uint32_t(v) << k;
        local[k] += v ? 1u : 0u;
      }
      uint64_t key = 0;
      if (coord_ok(c.x, c.y, c.z, c.w, B, X, Y, Z)) {
        const uint64_t z = (uint64_t(uint32_t(c.x)) << (3 * axis_bits)) |
                           zorder(uint32_t(c.y), uint32_t(c.z), uint32_t(c.w), axis_bits);
        key = (uint64_t(squeeze ? squeeze_centre(mask) : mask) << zbits) | z;
      }
      sort_key[i] = key;
      if (h0) atomicAdd(&dcnt[uint32_t(key) & 255u], 1u);
    }
  }
#pragma unroll
  for (int k = 0; k < kV; ++k) {
    uint32_t v = local[k];
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    if (__lane_id() == 0) atomicAdd(&cnt[k], v);
  }
  __syncthreads();
  if (threadIdx.x < kV) pcnt[int64_t(threadIdx.x) * pblk + blockIdx.x] = cnt[threadIdx.x];
  if (blockIdx.x == 0 && threadIdx.x == 0) pcnt[kV * pblk] = 0;
  if (h0) {
    // the direct sort's first-pass digit counts; these 256 rows lie in one sort block
    const int64_t sb = int64_t(blockIdx.x) * kPairRows / sort_block_keys;
    const uint32_t c = dcnt[threadIdx.x];
    if (c) atomicAdd(&h0[int64_t(threadIdx.x) * nsb + sb], c);
  }
}

// ---------------------------------------------------------------------------
// stable LSD radix sort of 64-bit keys with a 32-bit payload
// ---------------------------------------------------------------------------

template <int ITEMS>
__global__ void __launch_bounds__(kSortThreads) radix_hist(const uint64_t* __restrict__ keys, int64_t n,
                                                           int shift, uint32_t* __restrict__ hist,
                                                           int64_t nblk, const uint32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  __shared__ uint32_t cnt[256];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = int64_t(blockIdx.x) * kSortThreads * ITEMS;
  uint64_t k[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {  // every load before the first use, as in the scan
    const int64_t idx = base + int64_t(q) * kSortThreads + threadIdx.x;
    k[q] = keys[idx < n ? idx : n - 1];
  }
#pragma unroll
  for (int q = 0; q < ITEMS; ++q)
    if (base + int64_t(q) * kSortThreads + threadIdx.x < n) atomicAdd(&cnt[(k[q] >> shift) & 255u], 1u);
  __syncthreads();
  hist[int64_t(threadIdx.x) * nblk + blockIdx.x] = cnt[threadIdx.x];
  if (blockIdx.x == 0 && threadIdx.x == 0) hist[256 * nblk] = 0;
}

__device__ __forceinline__ void pair_scatter_block(int64_t blk, const uint32_t* __restrict__ nmap, int64_t n,
                                                   const uint32_t* __restrict__ pcnt, int64_t pblk,
                                                   uint32_t* __restrict__ pair_i, uint32_t* __restrict__ pair_j,
                                                   int direct, PlanHeader* __restrict__ h,
                                                   uint32_t* __restrict__ pseg);

// The pair-list scatter (pair_scatter_block) of a small input rides along with
// the first sort pass: it reads only nmap and row_scan's counts, so the
// workgroups past the sort blocks do it and one launch is saved.
struct PairJob {
  const uint32_t* nmap;
  const uint32_t* pcnt;
  int64_t pblk;  // 0: no pair blocks in this launch
  uint32_t* pair_i;
  uint32_t* pair_j;
  PlanHeader* h;
  uint32_t* pseg;
};

// Keys of one workgroup are taken in rounds of 256 in index order; inside a
// round, lanes with equal digits are ranked by a 64-lane ballot match and waves
// are ranked by their counts, so equal digits keep their input order.
//
// FUSE (direct sorts only): instead of a separate histogram kernel before
// every pass, this pass counts the next pass's digits per destination block
// in an LDS table as it places its keys (one global atomic per non-zero entry
// at the end), and clears the histogram the pass after next will fill.  Three
// histograms rotate: a pass reads one, fills the next, clears the third.
template <bool FUSE, int ITEMS>
__global__ void __launch_bounds__(kSortThreads)
    radix_scatter(const uint64_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in,
                  uint64_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out, int64_t n, int shift,
                  const uint32_t* __restrict__ offsets, int64_t nblk, int first, int last,
                  int32_t* __restrict__ perm, uint32_t* __restrict__ smask, int zbits, int direct,
                  uint32_t* __restrict__ hnext, uint32_t* __restrict__ hclear, PairJob pj,
                  const uint32_t* __restrict__ gate, int squeezed) {
  if (gated_off(gate)) return;
  if constexpr (FUSE) {
    if (int64_t(blockIdx.x) >= nblk) {
      pair_scatter_block(int64_t(blockIdx.x) - nblk, pj.nmap, n, pj.pcnt, pj.pblk, pj.pair_i, pj.pair_j, 1, pj.h,
                         pj.pseg);
      return;
    }
  }
  __shared__ uint32_t base[256];
  __shared__ uint32_t wcnt[kSortThreads / 64][256];
  __shared__ uint32_t nxt[FUSE ? kSortDirectBlocks * 256 : 1];
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  if constexpr (FUSE) {
    for (int64_t e = tid; e < nblk * 256; e += kSortThreads) nxt[e] = 0;
    if (hclear)
      for (int64_t e = int64_t(blockIdx.x) * kSortThreads + tid; e < nblk * 256; e += int64_t(gridDim.x) * kSortThreads)
        hclear[e] = 0;
  }
  // every round's keys and values are loaded before anything else
  constexpr int kBlockKeys = kSortThreads * ITEMS;
  const int64_t blk0 = int64_t(blockIdx.x) * kBlockKeys;
  uint64_t kk[ITEMS];
  uint32_t vv[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    const int64_t idx = blk0 + int64_t(q) * kSortThreads + tid;
    const bool valid = idx < n;
    kk[q] = valid ? keys_in[idx] : 0ull;
    vv[q] = valid ? (first ? uint32_t(idx) : vals_in[idx]) : 0u;
  }
  if (direct) {
    // few blocks: this block's start for digit tid = (keys of smaller digits) +
    // (keys of digit tid in earlier blocks), read straight from the histograms
    __shared__ uint32_t waves_sum[kSortThreads / 64];
    uint32_t tot = 0, before = 0;
    int64_t b = 0;
    for (; b + 3 < nblk; b += 4) {
      uint32_t c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) c[u] = offsets[int64_t(tid) * nblk + b + u];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        tot += c[u];
        if (b + u < int64_t(blockIdx.x)) before += c[u];
      }
    }
    for (; b < nblk; ++b) {
      const uint32_t c = offsets[int64_t(tid) * nblk + b];
      tot += c;
      if (b < int64_t(blockIdx.x)) before += c;
    }
    uint32_t excl;
    block_exclusive_scan(tot, waves_sum, &excl);
    base[tid] = excl + before;
  } else {
    base[tid] = offsets[int64_t(tid) * nblk + blockIdx.x];
  }
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    const int64_t idx = blk0 + int64_t(q) * kSortThreads + tid;
    const bool valid = idx < n;
    const uint64_t key = kk[q];
    const uint32_t val = vv[q];
    const uint32_t d = uint32_t(key >> shift) & 255u;
#pragma unroll
    for (int w = 0; w < kSortThreads / 64; ++w) wcnt[w][tid] = 0;
    __syncthreads();
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t ones = __ballot(bit);
      peers &= bit ? ones : ~ones;
    }
    const uint32_t rank = __popcll(peers & lanemask_lt());
    if (valid && rank == 0) wcnt[wave][d] = __popcll(peers);
    __syncthreads();
    if (valid) {
      uint32_t pos = base[d] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][d];
      if (FUSE && !last)
        atomicAdd(&nxt[((key >> (shift + 8)) & 255u) * nblk + pos / kBlockKeys], 1u);
      if (last) {
        perm[pos] = int32_t(val);
        smask[pos] = squeezed ? expand_centre(uint32_t(key >> zbits)) : uint32_t(key >> zbits);
      } else {
        keys_out[pos] = key;
        vals_out[pos] = val;
      }
    }
    __syncthreads();
    uint32_t add = 0;
#pragma unroll
    for (int w = 0; w < kSortThreads / 64; ++w) add += wcnt[w][tid];
    base[tid] += add;
    __syncthreads();
  }
  if constexpr (FUSE) {
    if (!last) {
      __syncthreads();
      for (int64_t e = tid; e < nblk * 256; e += kSortThreads)
        if (nxt[e]) atomicAdd(&hnext[e], nxt[e]);
    }
  }
}

// snmap[r] = nmap[perm[r]]: the map in sorted row order, so that a tile of
// consecutive sorted rows reads its gather indices as one contiguous block.
__global__ void __launch_bounds__(256) permute_rows(const uint32_t* __restrict__ nmap,
                                                    const int32_t* __restrict__ perm, int64_t n,
                                                    uint32_t* __restrict__ snmap) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= n * kV) return;
  const int64_t r = e / kV;
  const int k = int(e - r * kV);
  snmap[e] = nmap[int64_t(perm[r]) * kV + k];
}

// ---------------------------------------------------------------------------
// per-offset pair lists
// ---------------------------------------------------------------------------

__global__ void pair_offsets(const uint32_t* __restrict__ pcnt, int64_t pblk, PlanHeader* h) {
  const int k = threadIdx.x;
  if (k <= kV) h->pair_off[k] = pcnt[int64_t(k) * pblk];
  if (k < kV) h->pair_count[k] = pcnt[int64_t(k + 1) * pblk] - pcnt[int64_t(k) * pblk];
}

// pcnt holds scanned offsets (direct = 0) or raw per-block counts (direct = 1:
// few blocks, each block sums the counts itself and block 0 fills the header).
__device__ __forceinline__ void pair_scatter_block(int64_t blk, const uint32_t* __restrict__ nmap, int64_t n,
                                                   const uint32_t* __restrict__ pcnt, int64_t pblk,
                                                   uint32_t* __restrict__ pair_i, uint32_t* __restrict__ pair_j,
                                                   int direct, PlanHeader* __restrict__ h,
                                                   uint32_t* __restrict__ pseg) {
  __shared__ uint32_t base[32];
  __shared__ uint32_t tot[32];
  __shared__ uint32_t wc[kV][4];
  __shared__ uint32_t rows[256 * kV];
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  static_assert(kPairRows == 256, "one row per thread");
  const int64_t rbase = blk * kPairRows;
  const int64_t here = (n - rbase) < 256 ? (n - rbase) : 256;
  {
    // the rows' loads go out first; the offsets below overlap them
    uint32_t v[kV];
    fetch_rows(nmap, rbase, here, v);
    store_rows(rows, v);
  }
  if (direct) {
    // offset k = tid / 8 summed over blocks b = tid % 8 (mod 8), then the 8 sums in order
    __shared__ uint32_t part_t[kV][8], part_b[kV][8];
    if (tid < kV * 8) {
      const int k = tid >> 3, ph = tid & 7;
      uint32_t t = 0, before = 0;
      int64_t b = ph;
      for (; b + 24 < pblk; b += 32) {
        uint32_t c[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) c[u] = pcnt[int64_t(k) * pblk + b + 8 * u];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          t += c[u];
          if (b + 8 * u < blk) before += c[u];
        }
      }
      for (; b < pblk; b += 8) {
        const uint32_t c = pcnt[int64_t(k) * pblk + b];
        t += c;
        if (b < blk) before += c;
      }
      part_t[k][ph] = t;
      part_b[k][ph] = before;
    }
    __syncthreads();
    if (tid < kV) {
      uint32_t t = 0, before = 0;
      for (int ph = 0; ph < 8; ++ph) {
        t += part_t[tid][ph];
        before += part_b[tid][ph];
      }
      tot[tid] = t;
      base[tid] = before;
    }
    __syncthreads();
    if (tid < kV) {
      uint32_t off = 0;
      for (int k = 0; k < tid; ++k) off += tot[k];
      base[tid] += off;
      if (blk == 0) {
        h->pair_off[tid] = off;
        h->pair_count[tid] = tot[tid];
        if (tid == kV - 1) h->pair_off[kV] = off + tot[tid];
      }
    }
  } else if (tid < kV) {
    base[tid] = pcnt[int64_t(tid) * pblk + blk];
  }
  __syncthreads();
  // where this block's rows start in each list (the weight gradient chunks by rows)
  if (tid < kV) pseg[int64_t(tid) * (pblk + 1) + blk] = base[tid];
  {
    const int64_t row = rbase + tid;
    const bool in = row < n;
    uint32_t j[kV];
    uint32_t rank[kV];
#pragma unroll
    for (int k = 0; k < kV; ++k) {
      j[k] = in ? rows[tid * kV + k] : kSentinel;
      const uint64_t b = __ballot(j[k] != kSentinel);
      rank[k] = __popcll(b & lanemask_lt());
      if (__lane_id() == 0) wc[k][wave] = __popcll(b);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kV; ++k) {
      if (j[k] != kSentinel) {
        uint32_t pos = base[k] + rank[k];
        for (int w = 0; w < wave; ++w) pos += wc[k][w];
        pair_i[pos] = uint32_t(row);
        pair_j[pos] = j[k];
      }
    }
    __syncthreads();
    if (tid < kV) base[tid] += wc[tid][0] + wc[tid][1] + wc[tid][2] + wc[tid][3];
    __syncthreads();
  }
  if (blk == pblk - 1 && tid < kV) pseg[int64_t(tid) * (pblk + 1) + pblk] = base[tid];
}

__global__ void __launch_bounds__(256) pair_scatter(const uint32_t* __restrict__ nmap, int64_t n,
                                                    const uint32_t* __restrict__ pcnt, int64_t pblk,
                                                    uint32_t* __restrict__ pair_i,
                                                    uint32_t* __restrict__ pair_j, int direct,
                                                    PlanHeader* __restrict__ h, uint32_t* __restrict__ pseg) {
  pair_scatter_block(blockIdx.x, nmap, n, pcnt, pblk, pair_i, pair_j, direct, h, pseg);
}

// ---------------------------------------------------------------------------
// the row orders of offset parts 0 and 1 (see kParts)
// ---------------------------------------------------------------------------

// Sums over the main order: 32 * popcount(OR of each 32-row group's masks) and
// the masks' popcounts.  Grid-stride over the rows, a workgroup reduction, one
// pair of atomics per workgroup into the header.
__global__ void __launch_bounds__(256) union_stats(const uint32_t* __restrict__ smask, int64_t n,
                                                   PlanHeader* __restrict__ h) {
  __shared__ unsigned long long red[2][4];
  unsigned long long rows = 0, bits = 0;
  for (int64_t r0 = int64_t(blockIdx.x) * 256; r0 < n; r0 += int64_t(gridDim.x) * 256) {
    const int64_t r = r0 + threadIdx.x;
    const uint32_t m = r < n ? smask[r] : 0u;
    uint32_t u = m;
    for (int d = 1; d < 32; d <<= 1) u |= __shfl_xor(u, d, 64);  // OR over each 32-lane half
    bits += __popc(m);
    if ((__lane_id() & 31) == 0) rows += 32u * __popc(u);
  }
  for (int d = 32; d >= 1; d >>= 1) {
    bits += __shfl_xor(bits, d, 64);
    rows += __shfl_xor(rows, d, 64);
  }
  const int wave = threadIdx.x / 64;
  if (__lane_id() == 0) {
    red[0][wave] = rows;
    red[1][wave] = bits;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(&h->union_rows, red[0][0] + red[0][1] + red[0][2] + red[0][3]);
    atomicAdd(&h->mask_bits, red[1][0] + red[1][1] + red[1][2] + red[1][3]);
  }
}

// Takes the split when the main order's groups multiply enough zero rows, and
// then writes the sort keys of parts 0 and 1: for part q,
// (q << (9 + zbits)) | (the part's 9-bit mask << zbits) | z-order code, with
// the original row as payload, at position q * n + r for main sorted position
// r.  Keys are unique, so the input order cannot change the result, and one
// sort of the 2n keys orders both parts, part 0 first.
__global__ void __launch_bounds__(256) part_keys(const int4* __restrict__ coords, const int32_t* __restrict__ perm,
                                                 const uint32_t* __restrict__ smask, int64_t n, int axis_bits,
                                                 int zbits, PlanHeader* __restrict__ h,
                                                 uint64_t* __restrict__ key, uint32_t* __restrict__ val) {
  const unsigned long long rows = h->union_rows, bits = h->mask_bits;
  if (rows * kPartWasteDen < bits * kPartWasteNum) return;
  if (blockIdx.x == 0 && threadIdx.x == 0) h->part_split = 1u;
  const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (r >= n) return;
  const int32_t i = perm[r];
  const int4 c = coords[i];
  const uint64_t z = (uint64_t(uint32_t(c.x)) << (3 * axis_bits)) |
                     zorder(uint32_t(c.y), uint32_t(c.z), uint32_t(c.w), axis_bits);
  const uint32_t m = smask[r];
#pragma unroll
  for (int q = 0; q < kOwnOrderParts; ++q) {
    key[q * n + r] = (uint64_t(q) << (kPartCols + zbits)) |
                     (uint64_t((m >> (q * kPartCols)) & kPartColMask) << zbits) | z;
    val[q * n + r] = uint32_t(i);
  }
}

// Part q's map rows in its own order: dst[q][r][c] = nmap[pperm[q][r]][9q + c].
__global__ void __launch_bounds__(256) permute_parts(const uint32_t* __restrict__ nmap,
                                                     const int32_t* __restrict__ pperm, int64_t n,
                                                     uint32_t* __restrict__ dst, const uint32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= kOwnOrderParts * n * kPartCols) return;
  const int64_t R = e / kPartCols;  // row of the 2n part rows
  const int c = int(e - R * kPartCols);
  const int q = int(R / n);
  dst[e] = nmap[int64_t(pperm[R]) * kV + q * kPartCols + c];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static inline unsigned grid1d(int64_t work, int threads) {
  int64_t b = (work + threads - 1) / threads;
  return unsigned(b < 1 ? 1 : b);
}

// One LSD pass of 8 bits at `shift` over keys of the multi-block path
// (histogram, device-wide scan, stable scatter).  first: the payload is the
// key's index; last: write perm and the sorted masks (key >> zbits) instead of
// keys and payloads.
static void sort_pass(const uint64_t* kin, const uint32_t* vin, uint64_t* kout, uint32_t* vout, int64_t n,
                      int shift, bool first, bool last, int32_t* perm, uint32_t* smask, int zbits, uint32_t* hist,
                      uint32_t* scan_tmp, const uint32_t* gate, int squeezed, hipStream_t s) {
  const int64_t nblk = (n + kSortThreads * kSortItems - 1) / (kSortThreads * kSortItems);
  const PairJob no_pairs{nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr};
  radix_hist<kSortItems><<<unsigned(nblk), kSortThreads, 0, s>>>(kin, n, shift, hist, nblk, gate);
  launch_scan(hist, nblk * 256 + 1, scan_tmp, s, gate);
  radix_scatter<false, kSortItems><<<unsigned(nblk), kSortThreads, 0, s>>>(
      kin, vin, kout, vout, n, shift, hist, nblk, first ? 1 : 0, last ? 1 : 0, perm, smask, zbits, 0, nullptr,
      nullptr, no_pairs, gate, squeezed);
}

}  // namespace ssc

using namespace ssc;

extern "C" size_t ssc_plan_bytes(int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z,
                                 int32_t key_bits) {
  if (n < 0 || n > SSC_MAX_VOXELS || !grid_ok(B, X, Y, Z)) return 0;
  const int kb = effective_key_bits(B, X, Y, Z, key_bits);
  if (kb < 0) return 0;
  int axis_bits, zbits;
  sort_key_bits(B, X, Y, Z, &axis_bits, &zbits);
  if (kV + zbits > 64) return 0;
  return plan_layout(n, kb, part_build_wanted(n, B, X, Y, Z)).total;
}

namespace ssc {

void prepare_region(char* base, const PlanLayout& L, int64_t n, int B, int X, int Y, int Z, int kb, int zbits,
                    uint32_t* map, hipStream_t s) {
  PlanHeader* h = reinterpret_cast<PlanHeader*>(base + L.header);
  uint4* zrow = reinterpret_cast<uint4*>(base + L.zrow);
  // few sort blocks: row_scan adds the first pass's digit counts to a histogram that starts at zero
  const bool direct = L.sort_blocks <= kSortDirectBlocks;
  uint32_t* h0 = (n > 0 && direct) ? reinterpret_cast<uint32_t*>(base + L.hist) : nullptr;
  const int64_t h0_len = h0 ? L.sort_blocks * 256 : 0;
  const unsigned prep_blocks = grid1d((n * kV > int64_t(L.capacity) ? n * kV : int64_t(L.capacity)) / 4, 256);
  const unsigned prep = prep_blocks < 2048 ? prep_blocks : 2048;
  if (kb == 64)
    plan_prepare<uint64_t><<<prep, 256, 0, s>>>(h, n, B, X, Y, Z, kb, zbits, L.capacity, map,
                                                reinterpret_cast<BrickSlot<uint64_t>*>(base + L.table), zrow,
                                                h0, h0_len);
  else
    plan_prepare<uint32_t><<<prep, 256, 0, s>>>(h, n, B, X, Y, Z, kb, zbits, L.capacity, map,
                                                reinterpret_cast<BrickSlot<uint32_t>*>(base + L.table), zrow,
                                                h0, h0_len);
}

template <typename KeyT>
static void build_table(const int4* c4, int64_t n, int B, int X, int Y, int Z, char* base, const PlanLayout& L,
                        bool lookups, hipStream_t s) {
  PlanHeader* h = reinterpret_cast<PlanHeader*>(base + L.header);
  BrickSlot<KeyT>* table = reinterpret_cast<BrickSlot<KeyT>*>(base + L.table);
  uint32_t* vslot = reinterpret_cast<uint32_t*>(base + L.vslot);
  brick_insert<KeyT><<<grid1d(n, 256), 256, 0, s>>>(c4, n, B, X, Y, Z, table, L.capacity, vslot, &h->status_bits);
  if (!lookups) return;
  uint32_t* bcnt = reinterpret_cast<uint32_t*>(base + L.bcnt);
  uint32_t* bbase = reinterpret_cast<uint32_t*>(base + L.bbase);
  const int64_t nb = (n + kTableBlock - 1) / kTableBlock;
  brick_count<KeyT><<<unsigned(nb), kTableBlock, 0, s>>>(vslot, n, table, bcnt, nb);
  launch_scan(bcnt, 2 * nb + 1, reinterpret_cast<uint32_t*>(base + L.scan_tmp), s);
  brick_base<KeyT><<<unsigned(nb), kTableBlock, 0, s>>>(c4, vslot, n, table, bcnt, nb, bbase,
                                                        reinterpret_cast<uint32_t*>(base + L.blist),
                                                        reinterpret_cast<int4*>(base + L.bcoord));
  brick_rows<KeyT><<<grid1d(n, 256), 256, 0, s>>>(c4, vslot, n, table, bbase,
                                                  reinterpret_cast<uint32_t*>(base + L.brows));
}

void insert_coords(const int4* c4, int64_t n, int B, int X, int Y, int Z, int kb, char* base,
                   const PlanLayout& L, bool lookups, hipStream_t s) {
  if (n == 0) return;
  if (kb == 64)
    build_table<uint64_t>(c4, n, B, X, Y, Z, base, L, lookups, s);
  else
    build_table<uint32_t>(c4, n, B, X, Y, Z, base, L, lookups, s);
}

void order_rows(const int4* c4, const uint32_t* nmap, int64_t n, int B, int X, int Y, int Z, int32_t* perm,
                char* base, const PlanLayout& L, bool want_pairs, bool centre, hipStream_t s) {
  if (n == 0) return;
  int axis_bits, zbits;
  sort_key_bits(B, X, Y, Z, &axis_bits, &zbits);
  PlanHeader* h = reinterpret_cast<PlanHeader*>(base + L.header);
  uint32_t* smask = reinterpret_cast<uint32_t*>(base + L.smask);
  uint32_t* pair_i = reinterpret_cast<uint32_t*>(base + L.pair_i);
  uint32_t* pair_j = reinterpret_cast<uint32_t*>(base + L.pair_j);
  uint64_t* key0 = reinterpret_cast<uint64_t*>(base + L.key0);
  uint64_t* key1 = reinterpret_cast<uint64_t*>(base + L.key1);
  uint32_t* val0 = reinterpret_cast<uint32_t*>(base + L.val0);
  uint32_t* val1 = reinterpret_cast<uint32_t*>(base + L.val1);
  uint32_t* hist = reinterpret_cast<uint32_t*>(base + L.hist);
  uint32_t* pcnt = reinterpret_cast<uint32_t*>(base + L.pcnt);
  uint32_t* scan_tmp = reinterpret_cast<uint32_t*>(base + L.scan_tmp);

  const int64_t pblk = L.pair_blocks;
  const int64_t nblk = L.sort_blocks;
  // few sort blocks: the scatter passes build each other's histograms (radix_scatter<true>);
  // the first one was cleared by prepare_region
  const int direct = nblk <= kSortDirectBlocks ? 1 : 0;
  uint32_t* h0 = direct ? hist : nullptr;
  // centre: every row has its centre offset (submanifold), so the key leaves that mask bit out
  const int sq = centre ? 1 : 0;
  row_scan<<<unsigned(pblk), 256, 0, s>>>(c4, nmap, n, B, X, Y, Z, axis_bits, zbits, key0, pcnt, pblk, h0,
                                          direct ? hist + nblk * 256 : nullptr, nblk, kSortThreads * L.sort_items, sq);

  // radix sort over the key's kV (- 1) + zbits low bits
  const int bits = kV - sq + zbits;
  const int passes = (bits + 7) / 8;
  const uint64_t* kin = key0;
  const uint32_t* vin = val0;
  uint64_t* kout = key1;
  uint32_t* vout = val1;
  const int pdirect = pblk <= kPairDirectBlocks ? 1 : 0;
  // small inputs: the pair lists are built by extra workgroups of the first pass
  const bool pairs_ride = want_pairs && direct && pdirect;
  const PairJob no_pairs{nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr};
  const PairJob pair_job{nmap, pcnt, pblk, pair_i, pair_j, h, reinterpret_cast<uint32_t*>(base + L.pseg)};
  for (int p = 0; p < passes; ++p) {
    const int shift = 8 * p;
    const int last = p == passes - 1 ? 1 : 0;
    const PairJob pj = (pairs_ride && p == 0) ? pair_job : no_pairs;
    const unsigned grid = unsigned(nblk + pj.pblk);
    if (direct) {
      // histograms rotate: row_scan filled hist[0] for pass 0; pass p reads
      // hist[p % 3], fills hist[(p + 1) % 3] and clears hist[(p + 2) % 3]
      uint32_t* hcur = hist + (p % 3) * nblk * 256;
      uint32_t* hnext = hist + ((p + 1) % 3) * nblk * 256;
      uint32_t* hclr = hist + ((p + 2) % 3) * nblk * 256;
      if (L.sort_items == kSortItemsSmall)
        radix_scatter<true, kSortItemsSmall><<<grid, kSortThreads, 0, s>>>(
            kin, vin, kout, vout, n, shift, hcur, nblk, p == 0 ? 1 : 0, last, perm, smask, zbits, 1, hnext,
            last ? nullptr : hclr, pj, nullptr, sq);
      else
        radix_scatter<true, kSortItems><<<grid, kSortThreads, 0, s>>>(
            kin, vin, kout, vout, n, shift, hcur, nblk, p == 0 ? 1 : 0, last, perm, smask, zbits, 1, hnext,
            last ? nullptr : hclr, pj, nullptr, sq);
    } else {
      sort_pass(kin, vin, kout, vout, n, shift, p == 0, last, perm, smask, zbits, hist, scan_tmp, nullptr, sq, s);
    }
    const uint64_t* tk = kout;
    const uint32_t* tv = vout;
    kout = const_cast<uint64_t*>(kin);
    vout = const_cast<uint32_t*>(vin);
    kin = tk;
    vin = tv;
  }

  // The strided convolution's GEMMs read the map in sorted order; the
  // submanifold GEMMs gather the rows of nmap itself through perm.
  if (!centre)
    permute_rows<<<grid1d(n * kV, 256), 256, 0, s>>>(nmap, perm, n, reinterpret_cast<uint32_t*>(base + L.snmap));

  // per-offset pair lists (already built by the first pass for small inputs)
  if (!want_pairs) return;
  if (!pdirect) {
    launch_scan(pcnt, pblk * kV + 1, scan_tmp, s);
    pair_offsets<<<1, 64, 0, s>>>(pcnt, pblk, h);
  }
  if (!pairs_ride)
    pair_scatter<<<unsigned(pblk), 256, 0, s>>>(nmap, n, pcnt, pblk, pair_i, pair_j, pdirect, h,
                                              reinterpret_cast<uint32_t*>(base + L.pseg));
}

void order_parts(const int4* c4, const uint32_t* nmap, const int32_t* perm, int64_t n, int B, int X, int Y, int Z,
                 char* base, const PlanLayout& L, hipStream_t s) {
  if (n == 0) return;
  int axis_bits, zbits;
  sort_key_bits(B, X, Y, Z, &axis_bits, &zbits);
  PlanHeader* h = reinterpret_cast<PlanHeader*>(base + L.header);
  const uint32_t* smask = reinterpret_cast<const uint32_t*>(base + L.smask);
  uint64_t* key0 = reinterpret_cast<uint64_t*>(base + L.key0);
  uint64_t* key1 = reinterpret_cast<uint64_t*>(base + L.key1);
  uint32_t* val0 = reinterpret_cast<uint32_t*>(base + L.val0);
  uint32_t* val1 = reinterpret_cast<uint32_t*>(base + L.val1);
  uint32_t* hist = reinterpret_cast<uint32_t*>(base + L.hist);
  uint32_t* scan_tmp = reinterpret_cast<uint32_t*>(base + L.scan_tmp);
  const uint32_t* gate = &h->part_split;
  const int64_t nblk_stats = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  union_stats<<<unsigned(nblk_stats), 256, 0, s>>>(smask, n, h);
  part_keys<<<grid1d(n, 256), 256, 0, s>>>(c4, perm, smask, n, axis_bits, zbits, h, key0, val0);
  // (part, part mask, z-order) keys over both parts, the payload already the original row
  const int64_t nk = kOwnOrderParts * n;
  const int bits = 1 + kPartCols + zbits;
  const int passes = (bits + 7) / 8;
  const uint64_t* kin = key0;
  const uint32_t* vin = val0;
  uint64_t* kout = key1;
  uint32_t* vout = val1;
  for (int p = 0; p < passes; ++p) {
    sort_pass(kin, vin, kout, vout, nk, 8 * p, false, p == passes - 1, reinterpret_cast<int32_t*>(base + L.pperm),
              reinterpret_cast<uint32_t*>(base + L.psmask), zbits, hist, scan_tmp, gate, 0, s);
    const uint64_t* tk = kout;
    const uint32_t* tv = vout;
    kout = const_cast<uint64_t*>(kin);
    vout = const_cast<uint32_t*>(vin);
    kin = tk;
    vin = tv;
  }
  permute_parts<<<grid1d(nk * kPartCols, 256), 256, 0, s>>>(nmap, reinterpret_cast<const int32_t*>(base + L.pperm),
                                                           n, reinterpret_cast<uint32_t*>(base + L.psnmap), gate);
}

}  // namespace ssc

extern "C" int ssc_build_neighbor_map(const int32_t* coords, int64_t n, int32_t B, int32_t X, int32_t Y,
                                      int32_t Z, int32_t key_bits, uint32_t* nmap, int32_t* perm,
                                      void* plan, size_t plan_bytes, void* stream) {
  if (n < 0 || n > SSC_MAX_VOXELS || !plan) return SSC_ERR_INVALID_ARG;
  if (n > 0 && (!coords || !nmap || !perm)) return SSC_ERR_INVALID_ARG;
  if (!aligned16(plan) || (n > 0 && (!aligned16(coords) || !aligned16(nmap) || !aligned16(perm))))
    return SSC_ERR_INVALID_ARG;
  if (!grid_ok(B, X, Y, Z)) return SSC_ERR_INVALID_ARG;
  if (key_bits != 0 && key_bits != 32 && key_bits != 64) return SSC_ERR_INVALID_ARG;
  const int kb = effective_key_bits(B, X, Y, Z, key_bits);
  if (kb < 0) return SSC_ERR_UNSUPPORTED;
  int axis_bits, zbits;
  sort_key_bits(B, X, Y, Z, &axis_bits, &zbits);
  if (kV + zbits > 64) return SSC_ERR_UNSUPPORTED;
  const bool parts = part_build_wanted(n, B, X, Y, Z);
  const PlanLayout L = plan_layout(n, kb, parts);
  if (plan_bytes < L.total) return SSC_ERR_WORKSPACE;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(plan);
  (void)hipGetLastError();
  // header, zero row, first histogram, empty table (the probe writes every map entry)
  prepare_region(base, L, n, B, X, Y, Z, kb, zbits, nullptr, s);
  if (n == 0) return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;

  const int4* c4 = reinterpret_cast<const int4*>(coords);
  insert_coords(c4, n, B, X, Y, Z, kb, base, L, true, s);
  {
    PlanHeader* h = reinterpret_cast<PlanHeader*>(base + L.header);
    const uint32_t* blist = reinterpret_cast<const uint32_t*>(base + L.blist);
    const int4* bcoord = reinterpret_cast<const int4*>(base + L.bcoord);
    const uint32_t* bcnt = reinterpret_cast<const uint32_t*>(base + L.bcnt);
    const uint32_t* vslot = reinterpret_cast<const uint32_t*>(base + L.vslot);
    const int64_t nb = (n + kTableBlock - 1) / kTableBlock;
    // two bricks per wave and round: at most one wave per 32 voxels, at most 8192 workgroups of 4 waves
    const int64_t want = (n + 127) / 128;
    const unsigned bgrid = unsigned(want < 8192 ? want : 8192);
    if (kb == 64) {
      const VoxelTable<uint64_t> t = voxel_table<uint64_t>(base, L, X, Y, Z);
      probe_bricks<uint64_t><<<bgrid, 256, 0, s>>>(X, Y, Z, t, blist, bcoord, bcnt, nb, nmap);
      fill_orphans<uint64_t><<<grid1d(n, 256), 256, 0, s>>>(c4, vslot, n, t, &h->status_bits, nmap);
    } else {
      const VoxelTable<uint32_t> t = voxel_table<uint32_t>(base, L, X, Y, Z);
      probe_bricks<uint32_t><<<bgrid, 256, 0, s>>>(X, Y, Z, t, blist, bcoord, bcnt, nb, nmap);
      fill_orphans<uint32_t><<<grid1d(n, 256), 256, 0, s>>>(c4, vslot, n, t, &h->status_bits, nmap);
    }
  }
  order_rows(c4, nmap, n, B, X, Y, Z, perm, base, L, true, true, s);
  if (parts) order_parts(c4, nmap, perm, n, B, X, Y, Z, base, L, s);
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}

extern "C" int ssc_plan_status(const void* plan, void* stream, int32_t* status_host) {
  if (!plan || !status_host) return SSC_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PlanHeader h;
  if (hipStreamSynchronize(s) != hipSuccess) return SSC_ERR_HIP;
  if (hipMemcpy(&h, plan, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return SSC_ERR_HIP;
  if (h.magic != kPlanMagic) return SSC_ERR_INVALID_ARG;
  int32_t st = SSC_OK;
  if (h.status_bits & kBitCoordRange)
    st = SSC_ERR_COORD_RANGE;
  else if (h.status_bits & kBitDuplicate)
    st = SSC_ERR_DUPLICATE;
  else if (h.status_bits & kBitHashFull)
    st = SSC_ERR_HASH_FULL;
  *status_host = st;
  return SSC_OK;
}

extern "C" int ssc_plan_pair_counts(const void* plan, void* stream, int64_t* counts_host) {
  if (!plan || !counts_host) return SSC_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PlanHeader h;
  if (hipStreamSynchronize(s) != hipSuccess) return SSC_ERR_HIP;
  if (hipMemcpy(&h, plan, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return SSC_ERR_HIP;
  if (h.magic != kPlanMagic) return SSC_ERR_INVALID_ARG;
  for (int k = 0; k < kV; ++k) counts_host[k] = h.pair_count[k];
  return SSC_OK;
}

extern "C" int ssc_plan_row_orders(const void* plan, void* stream, int64_t* orders_host) {
  if (!plan || !orders_host) return SSC_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PlanHeader h;
  if (hipStreamSynchronize(s) != hipSuccess) return SSC_ERR_HIP;
  if (hipMemcpy(&h, plan, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return SSC_ERR_HIP;
  if (h.magic != kPlanMagic) return SSC_ERR_INVALID_ARG;
  orders_host[0] = h.part_split ? 1 + kOwnOrderParts : 1;
  orders_host[1] = int64_t(h.union_rows);
  orders_host[2] = int64_t(h.mask_bits);
  return SSC_OK;
}

extern "C" const char* ssc_status_string(int status) {
  switch (status) {
    case SSC_OK: return "ok";
    case SSC_ERR_INVALID_ARG: return "invalid argument";
    case SSC_ERR_UNSUPPORTED: return "unsupported dtype, channel count or grid";
    case SSC_ERR_WORKSPACE: return "plan or workspace buffer too small";
    case SSC_ERR_HIP: return "HIP runtime error";
    case SSC_ERR_COORD_RANGE: return "coordinate out of range";
    case SSC_ERR_DUPLICATE: return "duplicate coordinate";
    case SSC_ERR_HASH_FULL: return "hash table full";
    case SSC_ERR_SCRATCH: return "larger than the built-in scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}
