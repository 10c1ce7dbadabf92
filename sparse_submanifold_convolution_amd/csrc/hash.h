// Voxel hash table shared by the plan builder, the strided-map builder and the
// grid sampler: keys, slots, the mixing function and the lookup.
#pragma once

#include <hip/hip_runtime.h>

#include "ssc_internal.h"

namespace ssc {

// MurmurHash3 finalisers (Austin Appleby, public domain): full avalanche of the
// packed coordinate key before it is masked to a table slot.
__device__ __forceinline__ uint32_t mix_hash(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}
__device__ __forceinline__ uint32_t mix_hash(uint64_t k) {
  k ^= k >> 33;
  k *= 0xff51afd7ed558ccdull;
  k ^= k >> 33;
  k *= 0xc4ceb9fe1a85ec53ull;
  k ^= k >> 33;
  return uint32_t(k);
}

// The voxel table is an open-addressing hash keyed by bricks of 4 x 4 x 4
// cells: the key packs the brick's coordinates (batch, x/4, y/4, z/4) in 32 or
// 64 bits, and the slot holds the brick's 64-bit occupancy mask beside it.  A
// brick's voxel rows sit side by side in `rows` from `base[slot]` on, in the
// order of their cells' mask bits, so a voxel's row is found by one slot read,
// a mask test (which answers a miss at once) and a popcount.  The neighbours of
// a voxel mostly share its brick or an adjacent one, so the lookups of
// neighbouring voxels hit the same few slots in cache instead of one random
// line each.
constexpr int kBrickShift = 2;                 // 4 cells per brick side
constexpr uint32_t kCreator = 0x80000000u;     // vslot flag: this voxel inserted its brick's key

template <typename KeyT>
struct BrickSlot;
template <>
struct __align__(16) BrickSlot<uint32_t> {
  uint32_t key, pad;
  unsigned long long mask;
};
template <>
struct __align__(16) BrickSlot<uint64_t> {
  unsigned long long key;
  unsigned long long mask;
};
static_assert(sizeof(BrickSlot<uint32_t>) == 16 && sizeof(BrickSlot<uint64_t>) == 16, "one 16-byte slot");

template <typename KeyT>
__device__ __forceinline__ KeyT empty_key() {
  return KeyT(~KeyT(0));
}

__device__ __forceinline__ bool coord_ok(int b, int x, int y, int z, int B, int X, int Y, int Z) {
  return b >= 0 && b < B && x >= 0 && x < X && y >= 0 && y < Y && z >= 0 && z < Z;
}

__device__ __forceinline__ uint64_t pack_key(int b, int x, int y, int z, int X, int Y, int Z) {
  return ((uint64_t(b) * uint64_t(X) + uint64_t(x)) * uint64_t(Y) + uint64_t(y)) * uint64_t(Z) +
         uint64_t(z);
}

// The key of the brick holding cell (b, x, y, z) of grid (X, Y, Z).  The
// brick grid has no more cells than the voxel grid, so the key fits the
// same width and never equals the empty key.
__device__ __forceinline__ uint64_t brick_key(int b, int x, int y, int z, int X, int Y, int Z) {
  return pack_key(b, x >> kBrickShift, y >> kBrickShift, z >> kBrickShift, (X + 3) >> kBrickShift,
                  (Y + 3) >> kBrickShift, (Z + 3) >> kBrickShift);
}
// the cell's bit in its brick's occupancy mask
__device__ __forceinline__ int brick_bit(int x, int y, int z) { return ((x & 3) << 4) | ((y & 3) << 2) | (z & 3); }
__device__ __forceinline__ bool same_brick(int x0, int y0, int z0, int x1, int y1, int z1) {
  return ((x0 ^ x1) | (y0 ^ y1) | (z0 ^ z1)) >> kBrickShift == 0;
}

// The slot of a brick key (and its mask), or the sentinel when absent.
template <typename KeyT>
__device__ __forceinline__ uint32_t find_brick(const BrickSlot<KeyT>* __restrict__ slots, uint64_t capacity,
                                               KeyT key, unsigned long long* mask) {
  const uint64_t cm = capacity - 1;
  uint64_t slot = mix_hash(key) & cm;
  for (uint64_t probe = 0; probe < capacity; ++probe) {
    const BrickSlot<KeyT> e = slots[slot];
    if (e.key == key) {
      *mask = e.mask;
      return uint32_t(slot);
    }
    if (e.key == empty_key<KeyT>()) return kSentinel;
    slot = (slot + 1) & cm;
  }
  return kSentinel;
}

// The row of cell `bit` of the brick in `slot` with mask m, or the sentinel.
__device__ __forceinline__ uint32_t brick_row(const uint32_t* __restrict__ base, const uint32_t* __restrict__ rows,
                                              uint32_t slot, unsigned long long m, int bit) {
  if (!((m >> bit) & 1ull)) return kSentinel;
  return rows[base[slot] + uint32_t(__popcll(m & ((1ull << bit) - 1ull)))];
}

// A built voxel table, as the lookups see it.
template <typename KeyT>
struct VoxelTable {
  const BrickSlot<KeyT>* slots;
  const uint32_t* base;  // [capacity]: first entry of each occupied brick's rows
  const uint32_t* rows;  // [n]: voxel rows grouped by brick
  uint64_t capacity;
  int X, Y, Z;           // the voxel grid (the brick grid follows from it)
};

// The table of a plan region whose voxels sit in grid (X, Y, Z).
template <typename KeyT>
inline VoxelTable<KeyT> voxel_table(const char* base, const PlanLayout& L, int X, int Y, int Z) {
  return VoxelTable<KeyT>{reinterpret_cast<const BrickSlot<KeyT>*>(base + L.table),
                          reinterpret_cast<const uint32_t*>(base + L.bbase),
                          reinterpret_cast<const uint32_t*>(base + L.brows), L.capacity, X, Y, Z};
}

// The row of voxel (b, x, y, z) (inside the grid), or the sentinel.
template <typename KeyT>
__device__ __forceinline__ uint32_t voxel_lookup(const VoxelTable<KeyT>& t, int b, int x, int y, int z) {
  unsigned long long m;
  const uint32_t slot = find_brick<KeyT>(t.slots, t.capacity, KeyT(brick_key(b, x, y, z, t.X, t.Y, t.Z)), &m);
  if (slot == kSentinel) return kSentinel;
  return brick_row(t.base, t.rows, slot, m, brick_bit(x, y, z));
}

// host side: grid limits and the key width a plan uses
inline bool grid_ok(int32_t B, int32_t X, int32_t Y, int32_t Z) {
  return B >= 1 && X >= 1 && Y >= 1 && Z >= 1 && X <= (1 << 20) && Y <= (1 << 20) &&
         Z <= (1 << 20) && B <= (1 << 20);
}

inline int effective_key_bits(int32_t B, int32_t X, int32_t Y, int32_t Z, int32_t key_bits) {
  const unsigned __int128 vol = (unsigned __int128)(uint64_t)B * (uint64_t)X * (uint64_t)Y * (uint64_t)Z;
  const bool fits32 = vol <= (unsigned __int128)0xFFFFFFFFu;
  if (key_bits == 0) return fits32 ? 32 : 64;
  if (key_bits == 32) return fits32 ? 32 : -1;
  if (key_bits == 64) return vol < ((unsigned __int128)1 << 64) ? 64 : -1;
  return -1;
}

}  // namespace ssc
