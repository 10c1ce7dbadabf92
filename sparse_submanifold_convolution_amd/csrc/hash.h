// Voxel hash table shared by the plan builder and the grid sampler: keys,
// slots, the mixing function and the lookup.
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

// One hash-table slot: the key and its row index side by side, so a lookup
// that hits reads one aligned 8- or 16-byte entry.
template <typename KeyT>
struct Slot;
template <>
struct __align__(8) Slot<uint32_t> {
  uint32_t key, val;
};
template <>
struct __align__(16) Slot<uint64_t> {
  uint64_t key;
  uint32_t val, pad;
};

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

template <typename KeyT>
__device__ __forceinline__ uint32_t hash_lookup(const Slot<KeyT>* __restrict__ table, uint64_t capacity,
                                                KeyT key) {
  const uint64_t mask = capacity - 1;
  uint64_t slot = mix_hash(key) & mask;
  for (uint64_t probe = 0; probe < capacity; ++probe) {
    const Slot<KeyT> e = table[slot];
    if (e.key == key) return e.val;
    if (e.key == empty_key<KeyT>()) return kSentinel;
    slot = (slot + 1) & mask;
  }
  return kSentinel;
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
