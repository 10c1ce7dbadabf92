// Forward, input-gradient and weight-gradient kernels of the 3x3x3 submanifold
// convolution on gfx950.
//
// The FlexGEMM pages compute all three as implicit GEMMs over K = 27 * Ci
// whose row tiles skip the offsets no row of the tile has (masked implicit
// GEMM; the compile-cache post, section six, kernel signature with its
// neighbor, sorted_idx and valid_kernel arguments), with Split-K for the
// backward pass (contributor report, section two: the ..._bwd_masked_implicit
// _gemm_splitk kernel that fills weight.grad and feats.grad).
//
// Kernels here:
//   igemm          masked implicit GEMM.  One workgroup owns BM consecutive
//                  rows of the sorted order and BN output channels.  It ORs
//                  the rows' neighbour masks into the tile's offset set, reads
//                  the tile's gather indices into LDS, then walks (offset,
//                  K-slice) stages: each wave gathers its own rows straight into
//                  registers, the offset's weight slice goes through
//                  double-buffered LDS, and 32x32 MFMAs accumulate in fp32.
//                  The epilogue adds bias, rounds once and writes each row at
//                  its original index perm[r].
//                  Forward: A = X, B[k] = W[k]^T.  Input gradient: A = dY and
//                  B[k] = W[26-k] as stored, because nmap[i][k] = j exactly
//                  when nmap[j][26-k] = i.
//   transpose_w    W[k] -> W[k]^T for the forward B operand.
//   wgrad          dW[k] partial over one chunk of offset k's pair list:
//                  X rows (gathered by j) and dY rows (gathered by i) are
//                  transposed into LDS so that the pair index is the MFMA
//                  reduction dimension; fp32 partials per chunk.
//   wgrad_reduce   fixed-order sum of the chunk partials -> dW (deterministic).
//   colsum_*       dbias = column sums of dY, two fixed-order stages.

#include <hip/hip_runtime.h>

#include <mutex>

#include "ssc_internal.h"

namespace ssc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct bf16s {
  uint16_t bits;
};


template <typename T>
struct Elt;

template <>
struct Elt<float> {
  using frag_t = float;
  static constexpr int kStep = 2;  // reduction length of one MFMA
  static constexpr int kFrag = 1;  // elements each lane supplies
  __device__ static f32x16 mfma(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static float store(float v) { return v; }
  __device__ static float load(float v) { return v; }
};

template <>
struct Elt<_Float16> {
  using frag_t = f16x8;
  static constexpr int kStep = 16;
  static constexpr int kFrag = 8;
  __device__ static f32x16 mfma(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static _Float16 store(float v) { return _Float16(v); }
  __device__ static float load(_Float16 v) { return float(v); }
};

template <>
struct Elt<bf16s> {
  using frag_t = bf16x8;
  static constexpr int kStep = 16;
  static constexpr int kFrag = 8;
  __device__ static f32x16 mfma(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static bf16s store(float v) { return bf16s{f32_to_bf16_rne(v)}; }
  __device__ static float load(bf16s v) { return bf16_to_f32(v.bits); }
};

// Workgroup ids reach the 8 XCDs round-robin.  Work that shares data comes in
// groups of `members` items (the column blocks of one row tile, the channel
// tiles of one pair chunk); a group's items go to consecutive slots of one XCD
// so they share its L2, and whole groups are dealt to the XCDs in turn so
// neighbouring groups (similar cost) spread over all of them.  Launch
// 8 * ceil(groups / 8) * members workgroups; returns false for the padding.
__device__ __forceinline__ bool xcd_group_work(int groups, int members, int* group, int* member) {
  const int x = int(blockIdx.x % 8u), slot = int(blockIdx.x / 8u);
  *group = x + 8 * (slot / members);
  *member = slot % members;
  return *group < groups;
}

// consecutive row tiles grouped per XCD when a tile is a single work item
constexpr int kTileGroup = 4;

static inline unsigned xcd_group_grid(int groups, int members) {
  return unsigned((groups + 7) / 8) * 8u * unsigned(members);
}

// Row index inside a 32x32 MFMA accumulator block held by `lane`, register i.
__device__ __forceinline__ int acc_row(int lane, int i) { return (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3); }

// ---------------------------------------------------------------------------
// masked implicit GEMM (forward and input gradient)
// ---------------------------------------------------------------------------
//
// A workgroup of NWM x NWN waves owns a tile of BM = NWM * FM * 32 consecutive
// rows in sorted order and BN = NWN * FN * 32 output channels.  Wave (wm, wn)
// owns rows [wm*FM*32, (wm+1)*FM*32) and channels [wn*FN*32, (wn+1)*FN*32) of
// the tile; each lane loads its rows' K-slices straight from global memory
// into registers in MFMA operand order, DEPTH stages ahead, and no A data
// passes through LDS (waves of one wm gather the same rows, mostly from L1).
// The weight slice of the stage (dense, shared by all waves) is fetched DEPTH
// stages ahead too and staged through a double-buffered LDS tile.  Every
// weight fragment read from LDS feeds FM MFMAs and every gathered fragment FN,
// so NWN > 1 trades gather traffic for LDS read bandwidth, which alone would
// match the MFMA rate when FM = 1 and 8 waves share a CU.
//
// Inside a stage of BK reduction elements, lane half h (lanes 32h..32h+31)
// covers the contiguous run [h*BK/2, (h+1)*BK/2): MFMA step s takes its
// elements s*kFrag..s*kFrag+kFrag-1 of that run, for both operands.  Any
// one-to-one assignment of reduction indices to (step, half, element) slots
// gives the same sum, and this one makes every lane's gather one contiguous
// run of its row.

template <typename T, int FM, int FN, int BK, int NWM, int NWN>
struct IgemmCfg {
  static constexpr int kThreads = 64 * NWM * NWN;
  static constexpr int kBM = NWM * FM * 32;
  static constexpr int kBN = NWN * FN * 32;
  static constexpr int kVec = 16 / int(sizeof(T));                 // elements per 16-byte load
  static constexpr int kLd = BK + kVec;                            // LDS row stride of B (elements)
  static constexpr int kNV = (BK / 2) * int(sizeof(T)) / 16;       // 16-byte loads per lane per row block
  static constexpr int kSteps = BK / Elt<T>::kStep;                // MFMAs per stage per block
  static constexpr int kBV = (kBN * BK / kVec + kThreads - 1) / kThreads;  // B vectors per thread
  static constexpr size_t kLdsB = size_t(kBN) * kLd * sizeof(T);
  static_assert(kNV >= 1, "BK too small for 16-byte gathers");
  static_assert(BK % Elt<T>::kStep == 0, "bad BK");
};

template <typename T, int NV>
__device__ __forceinline__ typename Elt<T>::frag_t a_frag(const u32x4 (&v)[NV], int s) {
  if constexpr (sizeof(T) == 4) {
    return __uint_as_float(v[s / 4][s % 4]);
  } else {
    return __builtin_bit_cast(typename Elt<T>::frag_t, v[s]);
  }
}

// Split-K (nsplit > 1): work item (tile, column block, part) takes the part-th
// contiguous share of the tile's offset set and writes fp32 partial sums, in
// sorted row order, to partial[part][row][N]; split_reduce finishes them.
// One launch may cover only some offsets and hand its sums to another (the
// three-part split of the plan header's part_split): `kmask` keeps the offsets
// of this launch (map columns), `gate` makes the launch a no-op unless the
// plan took the split (1) or did not (2), and `emode` picks the epilogue:
// 0 bias + rounding + scatter to perm, 1 fp32 sums to pbuf[perm[r]], 3 those
// sums plus this launch's back to pbuf, 2 those sums + this launch's + bias,
// rounded, to out.  Map column c meets weight W[kbase + c], or W[kflip - c]
// with flip.  With `gmap` set (a 27-column map in original row order), the
// tile's map rows are gathered from it through perm instead of read from the
// sorted-order copy.
struct GemmPart {
  const PlanHeader* hdr;
  int gate;
  uint32_t kmask;
  int kbase;
  int kflip;
  int emode;
  float* pbuf;
  const uint32_t* gmap = nullptr;
};

// Epilogue of a GEMM tile (see GemmPart): each wave holds FM x FN 32x32
// accumulator blocks for tile rows r0.. and channels n0 + c0..; prow maps tile
// rows to original rows (-1 past the end).
// Whole-GEMM epilogue of 16-bit layers through LDS: a wave rounds one 32 x 32
// block of its outputs (with the bias) into its own 2 KB of LDS, then writes
// the block's rows as 16-byte vectors, four lanes a row: two store
// instructions per block instead of sixteen two-byte ones.  `stage` is the
// wave's 2 KB, free to overwrite (the caller has passed a workgroup barrier).
// The wave's LDS writes and reads complete in program order.
template <typename T, int FN>
__device__ __forceinline__ void gemm_store_rows(const f32x16 (&acc)[1][FN], const int32_t* prow, int r0, int lane,
                                                int n0, int N, const T* __restrict__ bias, T* __restrict__ out,
                                                T* stage) {
  using E = Elt<T>;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int cb = n0 + j * 32;  // the block's first column
    if (cb >= N) break;
    const int c = cb + (lane & 31);
    const float bv = (bias && c < N) ? E::load(bias[c]) : 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) stage[acc_row(lane, e) * 32 + (lane & 31)] = E::store(acc[0][j][e] + bv);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = q * 64 + lane, row = idx >> 2, cv = idx & 3;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * 32 + cv * 8);
      const int32_t p = prow[r0 + row];
      const int col = cb + cv * 8;
      if (p >= 0 && col < N) *reinterpret_cast<u32x4*>(out + int64_t(p) * N + col) = v;
    }
  }
}

// The same for the offset parts of a split GEMM: a wave stages one 32 x 32
// block of fp32 sums in its own 4 KB of LDS, then moves the block's rows as
// 16-byte vectors of four sums, eight lanes a row: the first part writes its
// sums, the middle part adds them to the handed-over sums, the last adds
// them, the bias (in that order, as the direct epilogue does) and rounds.
template <typename T, int FN>
__device__ __forceinline__ void gemm_store_parts(const f32x16 (&acc)[1][FN], const int32_t* prow, int r0, int lane,
                                                 int n0, int N, const T* __restrict__ bias, T* __restrict__ out,
                                                 const GemmPart& gp, float* stage) {
  using E = Elt<T>;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  // a lane always moves the same four columns of a block (lane % 8)
  const int cv = lane & 7;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int cb = n0 + j * 32;
    if (cb >= N) break;
    const int col = cb + cv * 4;
    float bv[4] = {0.f, 0.f, 0.f, 0.f};
    if (gp.emode == 2 && bias && col < N) {
      const uint2 braw = *reinterpret_cast<const uint2*>(bias + col);
      const T* bt = reinterpret_cast<const T*>(&braw);
#pragma unroll
      for (int u = 0; u < 4; ++u) bv[u] = E::load(bt[u]);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) stage[acc_row(lane, e) * 32 + (lane & 31)] = acc[0][j][e];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = (q * 64 + lane) >> 3;
      const f32x4 v = *reinterpret_cast<const f32x4*>(stage + row * 32 + cv * 4);
      const int32_t p = prow[r0 + row];
      if (p < 0 || col >= N) continue;
      f32x4* pb = reinterpret_cast<f32x4*>(gp.pbuf + int64_t(p) * N + col);
      if (gp.emode == 1) {
        *pb = v;
      } else if (gp.emode == 3) {
        const f32x4 o = *pb;
        *pb = o + v;
      } else {
        const f32x4 o = *pb;
        T r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u] = E::store(v[u] + o[u] + bv[u]);
        *reinterpret_cast<uint2*>(out + int64_t(p) * N + col) = *reinterpret_cast<const uint2*>(r);
      }
    }
  }
}

template <typename T, int FM, int FN>
__device__ __forceinline__ void gemm_store(const f32x16 (&acc)[FM][FN], const int32_t* prow, int r0, int c0, int lane,
                                           int n0, int N, const T* __restrict__ bias, T* __restrict__ out,
                                           const GemmPart& gp) {
  using E = Elt<T>;
  if (gp.emode == 0) {
    // a whole GEMM: bias, round once, scatter rows to perm
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int c = n0 + c0 + j * 32 + (lane & 31);
      if (c >= N) continue;
      const float bv = bias ? E::load(bias[c]) : 0.f;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int32_t p = prow[r0 + i * 32 + acc_row(lane, e)];
          if (p >= 0) out[int64_t(p) * N + c] = E::store(acc[i][j][e] + bv);
        }
    }
    return;
  }
  if (gp.emode == 1 || gp.emode == 3) {
    // first or middle part of a split: fp32 sums by original row, no bias
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int c = n0 + c0 + j * 32 + (lane & 31);
      if (c >= N) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        float prev[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int32_t p = prow[r0 + i * 32 + acc_row(lane, e)];
          prev[e] = (gp.emode == 3 && p >= 0) ? gp.pbuf[int64_t(p) * N + c] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int32_t p = prow[r0 + i * 32 + acc_row(lane, e)];
          if (p >= 0) gp.pbuf[int64_t(p) * N + c] = prev[e] + acc[i][j][e];
        }
      }
    }
    return;
  }
  // last part: the earlier parts' sums, the bias, round once, scatter rows to perm
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int c = n0 + c0 + j * 32 + (lane & 31);
    if (c >= N) continue;
    const float bv = bias ? E::load(bias[c]) : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float prev[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int32_t p = prow[r0 + i * 32 + acc_row(lane, e)];
        prev[e] = p >= 0 ? gp.pbuf[int64_t(p) * N + c] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int32_t p = prow[r0 + i * 32 + acc_row(lane, e)];
        if (p >= 0) out[int64_t(p) * N + c] = E::store(acc[i][j][e] + prev[e] + bv);
      }
    }
  }
}

// GM: the map rows come from a map in original row order (gp.gmap) through
// perm, instead of from a sorted-order map; a compile-time choice, so that
// the sorted-map prologue issues all of its loads in one round trip.
template <typename T, int FM, int FN, int BK, int NWM, int NWN, int DEPTH, int KMAP, int MW, bool GM>
__global__ void __launch_bounds__(64 * NWM * NWN)
    igemm(const T* __restrict__ A, const T* __restrict__ Bt, const T* __restrict__ bias, T* __restrict__ out,
          const uint32_t* __restrict__ snmap, const int32_t* __restrict__ perm,
          const uint32_t* __restrict__ smask, const T* __restrict__ zrow, int64_t n, int K, int N, int flip,
          int ntiles, int nblk_n, int nsplit, float* __restrict__ partial, int tgroup, GemmPart gp) {
  if (gp.gate != 0 && (gp.hdr->part_split != 0u) != (gp.gate == 1)) return;
  using C = IgemmCfg<T, FM, FN, BK, NWM, NWN>;
  using E = Elt<T>;
  using frag_t = typename E::frag_t;
  constexpr int NT = C::kThreads;
  constexpr int BM = C::kBM, BN = C::kBN, NV = C::kNV;
  static_assert(KMAP == 0 || sizeof(T) == 2, "the natural order needs one 16-byte load per MFMA fragment");
  static_assert(KMAP != 2 || NWN == 1, "row-coalesced gathers keep each wave's rows private");
  // KMAP 2: lanes per gathered row segment and rows per load instruction
  constexpr int LPR = BK / C::kVec, RPI = 64 / LPR;
  // The host picks BK = 64 or 32 only when it divides the reduction length K;
  // the 16-wide slices also serve every other K (a multiple of 8 for 16-bit
  // types, 4 for fp32), whose last slice is ragged.
  constexpr bool RAG = BK == 16;

  // tgroup consecutive row tiles with all their column blocks (and Split-K
  // parts) run on one XCD: they gather overlapping neighbour rows
  int grp, member;
  if (!xcd_group_work((ntiles + tgroup - 1) / tgroup, tgroup * nblk_n * nsplit, &grp, &member)) return;
  const int tile = grp * tgroup + member / (nblk_n * nsplit);
  if (tile >= ntiles) return;
  member %= nblk_n * nsplit;
  const int part = member % nsplit;
  const int n0 = (member / nsplit) * BN;

  __shared__ __align__(16) char lds_b[2 * C::kLdsB];
  // KMAP 2: each wave's gathered rows of the current stage, 16-byte slots
  // XOR-swizzled so that both the row-major writes and the MFMA-order reads
  // of 8 lanes hit 8 distinct bank groups
  __shared__ __align__(16) T lds_a[KMAP == 2 ? NWM * FM * 32 * BK : 8];
  __shared__ uint32_t jtab[BM * MW];  // [row][column]: this tile's rows of the sorted-order map
  __shared__ int32_t prow[BM];
  __shared__ uint32_t tile_union;
  __shared__ uint32_t wave_union[NWM];  // offsets present among each wave row's rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int wm = wave / NWN, wn = wave % NWN;
  const int64_t row0 = int64_t(tile) * BM;

  // ---- prologue: rows, the tile's offset set, gather indices ----
  // The tile's rows of a sorted-order map are one contiguous block; all of
  // its loads are issued before any is stored, so the prologue costs one
  // memory round trip, independent of perm.  A map in original row order
  // (gp.gmap) costs a second one: perm first, then the rows it names.
  constexpr int JV = (BM * MW + NT - 1) / NT;
  uint32_t jv[JV];
  int32_t pr = -1;
  uint32_t msk = 0;
  if (tid < BM) {
    const int64_t g = row0 + tid;
    if (g < n) {
      pr = perm[g];
      msk = smask[g] & gp.kmask;
    }
  }
  if constexpr (GM) {
    static_assert(MW <= kV, "map rows");
    if (tid < BM) prow[tid] = pr;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < JV; ++q) {
      const int el = q * NT + tid;
      const int rr = el / MW, cc = el - rr * MW;
      const int32_t p = el < BM * MW ? prow[rr] : -1;
      jv[q] = p >= 0 ? gp.gmap[int64_t(p) * kV + cc] : kSentinel;
    }
  } else {
    const int64_t jbase = row0 * MW, jend = n * MW;
#pragma unroll
    for (int q = 0; q < JV; ++q) {
      const int64_t e = jbase + q * NT + tid;
      jv[q] = (q * NT + tid < BM * MW && e < jend) ? snmap[e] : kSentinel;
    }
  }
  if (tid == 0) tile_union = 0;
  if (tid < NWM) wave_union[tid] = 0;
#pragma unroll
  for (int q = 0; q < JV; ++q)
    if (q * NT + tid < BM * MW) jtab[q * NT + tid] = jv[q];
  __syncthreads();
  if (tid < BM) {
    prow[tid] = pr;
    if (msk) {
      atomicOr(&tile_union, msk);
      atomicOr(&wave_union[tid / (FM * 32)], msk);
    }
  }
  __syncthreads();
  uint32_t uni = tile_union;
  if (nsplit > 1) {
    // keep this part's contiguous share of the offsets (in increasing k)
    const int cnt = __popc(uni);
    const int lo = part * cnt / nsplit, hi = (part + 1) * cnt / nsplit;
    uint32_t keep = 0, rest = uni;
    for (int r = 0; rest; ++r) {
      const uint32_t bit = rest & (0u - rest);
      if (r >= lo && r < hi) keep |= bit;
      rest ^= bit;
    }
    uni = keep;
  }

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int kslices = (K + BK - 1) / BK;
  const int nstages = __popc(uni) * kslices;
  // A wave skips the MFMAs of a stage whose offset none of its rows has (its
  // loads still run and read the zero row), so only the tile's weight slices
  // are shared and the work follows each wave's own rows.
  const uint32_t wuni = wave_union[wm] & uni;

  // stage cursors: A and B both run DEPTH stages ahead of the compute cursor c
  uint32_t a_rem = uni, b_rem = uni, c_rem = uni;
  int a_k = a_rem ? __ffs(a_rem) - 1 : 0, a_ks = 0;
  int b_k = a_k, b_ks = 0, c_k = a_k, c_ks = 0;
  auto advance = [&](uint32_t& rem, int& k, int& ks) {
    if (++ks == kslices) {
      ks = 0;
      rem &= rem - 1;
      k = rem ? __ffs(rem) - 1 : 0;
    }
  };

  constexpr int AR = FM * NV;  // per-lane MFMA fragments of the wave's rows
  // native vectors, so every ring copy is a plain register load or store
  u32x4 abuf[DEPTH][AR];
  u32x4 bbuf[DEPTH][C::kBV];

  // Every load is unconditional (a branch around a load, even a uniform one,
  // makes the compiler drain the whole prefetch ring at the next wait): a
  // missing neighbour, an out-of-range weight column and any stage past the
  // last one (the ring runs DEPTH stages ahead) read the plan's zero row.
  //
  // KMAP 0: lane half h reads the run [h*BK/2, (h+1)*BK/2) of the stage, one
  // contiguous piece per lane.  KMAP 1 (16-bit only): the natural MFMA order,
  // load v of half h reads 16 bytes at element (2v + h) * 8, so each load
  // instruction covers 32 contiguous bytes of 32 rows.  KMAP 2 (16-bit only):
  // LPR lanes read one row's whole stage segment, so each load instruction
  // covers RPI rows completely (fewer, fuller cache lines per instruction);
  // compute() moves the rows into MFMA order through the wave's LDS slots.
  auto load_a = [&](u32x4 (&dst)[AR]) {
    // a byte offset from A selects the zero row: selects, never branches
    const int64_t zoff = reinterpret_cast<const char*>(zrow) - reinterpret_cast<const char*>(A);
    const uint32_t live = a_rem != 0 ? ~0u : 0u;
    if constexpr (KMAP == 2) {
      const int c0 = a_ks * BK + (lane % LPR) * C::kVec;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int rr = i * 32 + v * RPI + lane / LPR;
          const uint32_t j = jtab[(wm * FM * 32 + rr) * MW + a_k] | ~live;
          const int64_t off = j != kSentinel ? (int64_t(j) * K + c0) * int64_t(sizeof(T)) : zoff;
          dst[i * NV + v] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(A) + off);
        }
    } else {
      const int c0 = a_ks * BK + (KMAP == 0 ? half * (BK / 2) : half * C::kVec);
      constexpr int vstride = KMAP == 0 ? 1 : 2;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint32_t j = jtab[(wm * FM * 32 + i * 32 + (lane & 31)) * MW + a_k] | ~live;
        if constexpr (RAG) {
          // a reduction length that is not a multiple of BK leaves the last
          // slice ragged: its columns at or past K read zeros
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            const int col = c0 + v * vstride * C::kVec;
            const int64_t off = (j != kSentinel && col < K) ? (int64_t(j) * K + col) * int64_t(sizeof(T)) : zoff;
            dst[i * NV + v] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(A) + off);
          }
        } else {
          const int64_t off = j != kSentinel ? (int64_t(j) * K + c0) * int64_t(sizeof(T)) : zoff;
          const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(A) + off);
#pragma unroll
          for (int v = 0; v < NV; ++v) dst[i * NV + v] = src[v * vstride];
        }
      }
    }
    advance(a_rem, a_k, a_ks);
  };
  // KMAP 2 slot of (wave row rr, 16-byte chunk c) in the wave's LDS rows
  auto a_slot = [&](int rr, int c) {
    const int q = rr * LPR + c;
    return q ^ ((q >> 3) & 7);
  };
  auto load_b = [&](u32x4 (&rb)[C::kBV]) {
    const int kb = flip ? (gp.kflip - b_k) : (gp.kbase + b_k);
    const int64_t base = (int64_t(kb) * N * K + b_ks * BK) * int64_t(sizeof(T));
    const int64_t zoff = reinterpret_cast<const char*>(zrow) - reinterpret_cast<const char*>(Bt);
    const int rlim = b_rem != 0 ? N - n0 : 0;  // rows at or past rlim read the zero row
    constexpr int VPR = BK / C::kVec;
#pragma unroll
    for (int v = 0; v < C::kBV; ++v) {
      const int idx = tid + v * NT;
      const int id = idx < BN * VPR ? idx : 0;  // surplus threads reload element 0 and store nothing
      const int r = id / VPR, cv = id % VPR;
      const bool in = r < rlim && (!RAG || b_ks * BK + cv * C::kVec < K);  // ragged last slice: zeros past K
      const int64_t off = in ? base + int64_t(n0 + r) * K * int64_t(sizeof(T)) + cv * 16 : zoff;
      rb[v] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(Bt) + off);
    }
    advance(b_rem, b_k, b_ks);
  };
  auto store_b = [&](int buf, const u32x4 (&rb)[C::kBV]) {
    T* sb = reinterpret_cast<T*>(lds_b + buf * C::kLdsB);
    constexpr int VPR = BK / C::kVec;
#pragma unroll
    for (int v = 0; v < C::kBV; ++v) {
      const int idx = tid + v * NT;
      if (C::kBV * NT == BN * VPR || idx < BN * VPR) {
        const int r = idx / VPR, cv = idx % VPR;
        *reinterpret_cast<u32x4*>(sb + r * C::kLd + cv * C::kVec) = rb[v];
      }
    }
  };
  auto compute = [&](const u32x4 (&a)[AR], int buf) {
    const T* sb = reinterpret_cast<const T*>(lds_b + buf * C::kLdsB);
    T* sa = lds_a + (KMAP == 2 ? wave * FM * 32 * BK : 0);
    if constexpr (KMAP == 2) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int v = 0; v < NV; ++v)
          *reinterpret_cast<u32x4*>(sa + a_slot(i * 32 + v * RPI + lane / LPR, lane % LPR) * C::kVec) =
              a[i * NV + v];
      // the wave's own rows: in-order LDS needs no barrier, only no reordering
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      frag_t bfr[FN];
      const int kofs = KMAP == 0 ? half * (BK / 2) + s * E::kFrag : (2 * s + half) * E::kFrag;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int c = (wn * FN + j) * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const frag_t*>(sb + c * C::kLd + kofs);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        frag_t af;
        if constexpr (KMAP == 2) {
          af = *reinterpret_cast<const frag_t*>(sa + a_slot(i * 32 + (lane & 31), 2 * s + half) * C::kVec);
        } else {
          u32x4 ai[NV];
#pragma unroll
          for (int v = 0; v < NV; ++v) ai[v] = a[i * NV + v];
          af = a_frag<T, NV>(ai, s);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = E::mfma(af, bfr[j], acc[i][j]);
      }
    }
    // the next stage's slot writes stay behind this stage's reads
    if constexpr (KMAP == 2) __builtin_amdgcn_wave_barrier();
  };

  // One stage of prefetch in the natural order: the gathered piece of MFMA
  // step q is reloaded for the next stage right after that step's MFMAs, so
  // each gather has most of a stage to arrive (with a whole-stage refill it
  // would be issued after the last MFMA and awaited right after the next
  // barrier) and the ring costs no more registers.
  constexpr bool kRoll = DEPTH == 1 && KMAP == 1 && FM == 1 && sizeof(T) == 2 && !RAG && C::kSteps == NV;

  // the row pieces of the gather cursor's stage (the zero row past the last
  // stage); advances the cursor
  auto a_src = [&]() {
    const int64_t zoff = reinterpret_cast<const char*>(zrow) - reinterpret_cast<const char*>(A);
    const uint32_t live = a_rem != 0 ? ~0u : 0u;
    const uint32_t j = jtab[(wm * 32 + (lane & 31)) * MW + a_k] | ~live;
    const int64_t off = j != kSentinel ? (int64_t(j) * K + a_ks * BK + half * C::kVec) * int64_t(sizeof(T)) : zoff;
    advance(a_rem, a_k, a_ks);
    return reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(A) + off);
  };

  // prologue loads: both operands DEPTH stages deep
#pragma unroll
  for (int d = 0; !kRoll && d < DEPTH; ++d) {
    load_a(abuf[d]);
    load_b(bbuf[d]);
  }

  if constexpr (kRoll) {
    // Stage s: barrier (B(s) is in LDS and every wave is past stage s - 1),
    // B(s + 1) loads, the MFMAs of stage s with A(s + 1) loads between
    // their steps, then B(s + 1) to the other LDS buffer.  The weight slice
    // gets a whole stage to arrive, and each wait sees the same loads in
    // flight on every path into it.
    load_b(bbuf[0]);
    {
      const u32x4* src = a_src();
#pragma unroll
      for (int q = 0; q < C::kSteps; ++q) {
        abuf[0][q] = src[2 * q];
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    store_b(0, bbuf[0]);
    for (int s = 0; s < nstages; ++s) {
      const int buf = s & 1;
      __syncthreads();
      load_b(bbuf[0]);
      const u32x4* src = a_src();  // the next stage's pieces
      // A wave whose rows all lack the stage's offset skips its MFMAs.  The
      // skip tests sit around each step's LDS reads and MFMAs only; the
      // gathers between them are issued on every path, so the compiler sees
      // one sequence of loads and waits only for the pieces each step needs.
      const bool run = (wuni >> c_k) & 1u;
      const T* sb = reinterpret_cast<const T*>(lds_b + buf * C::kLdsB);
      auto read_b = [&](frag_t (&bfr)[FN], int q) {
#pragma unroll
        for (int jn = 0; jn < FN; ++jn)
          bfr[jn] = *reinterpret_cast<const frag_t*>(sb + ((wn * FN + jn) * 32 + (lane & 31)) * C::kLd +
                                                     (2 * q + half) * E::kFrag);
      };
      frag_t bfr[2][FN];  // this step's weight fragments and the next step's
      if (run) read_b(bfr[0], 0);
#pragma unroll
      for (int q = 0; q < C::kSteps; ++q) {
        if (run) {
          if (q + 1 < C::kSteps) read_b(bfr[(q + 1) & 1], q + 1);
          const frag_t af = __builtin_bit_cast(frag_t, abuf[0][q]);
#pragma unroll
          for (int jn = 0; jn < FN; ++jn) acc[0][jn] = E::mfma(af, bfr[q & 1][jn], acc[0][jn]);
        }
        abuf[0][q] = src[2 * q];
        // keep the refill here: the scheduler would otherwise move it after
        // the last MFMA
        __builtin_amdgcn_sched_barrier(0);
      }
      advance(c_rem, c_k, c_ks);
      store_b(buf ^ 1, bbuf[0]);
    }
  }

  // Each stage refills its ring slot DEPTH stages ahead.  Only the LDS store,
  // the barrier and the MFMAs depend on the (uniform) stage bound; the loads
  // are issued on every path.
  for (int s0 = 0; !kRoll && s0 < nstages; s0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int s = s0 + d;
      const int buf = s & 1;
      const bool run = s < nstages;
      if (run) {
        store_b(buf, bbuf[d]);
        __syncthreads();
      }
      load_b(bbuf[d]);
      if (run && ((wuni >> c_k) & 1u)) compute(abuf[d], buf);
      advance(c_rem, c_k, c_ks);
      load_a(abuf[d]);
    }
  }

  if (nsplit > 1) {
    // fp32 partials in sorted row order; bias, rounding and perm come later
    float* dst = partial + int64_t(part) * n * N;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int c = n0 + (wn * FN + j) * 32 + (lane & 31);
      if (c >= N) continue;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t g = row0 + wm * FM * 32 + i * 32 + acc_row(lane, e);
          if (g < n) dst[g * N + c] = acc[i][j][e];
        }
    }
    return;
  }

  if constexpr (sizeof(T) == 2 && FM == 1 && NWN == 1) {
    // every wave is past its last stage (barrier below): the weight buffers are free
    if constexpr (2 * C::kLdsB >= size_t(NWM) * 2048) {
      if (gp.emode == 0) {
        __syncthreads();
        gemm_store_rows<T, FN>(acc, prow, wm * 32, lane, n0, N, bias, out, reinterpret_cast<T*>(lds_b) + wave * 1024);
        return;
      }
    }
    if constexpr (2 * C::kLdsB >= size_t(NWM) * 4096) {
      if (gp.emode != 0) {
        __syncthreads();
        gemm_store_parts<T, FN>(acc, prow, wm * 32, lane, n0, N, bias, out, gp,
                                reinterpret_cast<float*>(lds_b) + wave * 1024);
        return;
      }
    }
  }
  gemm_store<T, FM, FN>(acc, prow, wm * FM * 32, wn * FN * 32, lane, n0, N, bias, out, gp);
}

// W[k] ([K][N]) -> Wt[k] ([N][K]) for every offset, through a 32x32 LDS tile.
template <typename T>
__global__ void __launch_bounds__(256) transpose_w(const T* __restrict__ W, T* __restrict__ Wt, int K, int N) {
  __shared__ T tile[32][33];
  const int k = blockIdx.z;
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const T* src = W + int64_t(k) * K * N;
  T* dst = Wt + int64_t(k) * K * N;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8)
    if (r0 + r < K && c0 + tx < N) tile[r][tx] = src[int64_t(r0 + r) * N + c0 + tx];
  __syncthreads();
  for (int r = ty; r < 32; r += 8)
    if (c0 + r < N && r0 + tx < K) dst[int64_t(c0 + r) * K + r0 + tx] = tile[tx][r];
}

// out[perm[r]][c] = bias[c] + sum over parts, in part order, of partial[part][r][c]
template <typename T>
__global__ void __launch_bounds__(256) split_reduce(const float* __restrict__ partial, int nsplit, int64_t n, int N,
                                                    const T* __restrict__ bias, const int32_t* __restrict__ perm,
                                                    T* __restrict__ out) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= n * N) return;
  const int64_t r = e / N;
  const int c = int(e - r * N);
  float s = 0.f;
  for (int p = 0; p < nsplit; ++p) s += partial[int64_t(p) * n * N + e];
  if (bias) s += Elt<T>::load(bias[c]);
  out[int64_t(perm[r]) * N + c] = Elt<T>::store(s);
}

// ---------------------------------------------------------------------------
// weight gradient: per-offset gather GEMM over pair-list chunks (Split-K)
// ---------------------------------------------------------------------------

template <typename T, int BM, int BN, int BKP, int WM, int WN>
struct WgradCfg {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kVec = 16 / int(sizeof(T));
  static constexpr int kLd = BKP + (sizeof(T) == 4 ? 4 : 8);  // LDS row stride in elements (row = channel)
  static constexpr int kTM = BM / WM, kTN = BN / WN;
  static constexpr int kFM = kTM / 32, kFN = kTN / 32;
  static constexpr size_t kLdsA = size_t(BM) * kLd * sizeof(T);
  static constexpr size_t kLdsB = size_t(BN) * kLd * sizeof(T);
  // one staging item = a group of G pairs x one 16-byte column vector
  static constexpr int kG = sizeof(T) == 4 ? 1 : 2;
  static constexpr int kItemsA = (BKP / kG) * (BM / kVec);
  static constexpr int kItemsB = (BKP / kG) * (BN / kVec);
  static constexpr int kIA = (kItemsA + kThreads - 1) / kThreads;
  static constexpr int kIB = (kItemsB + kThreads - 1) / kThreads;
  static_assert(kTM % 32 == 0 && kTN % 32 == 0, "wave tile must be whole 32x32 MFMA blocks");
};

template <typename T, int BM, int BN, int BKP, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
    wgrad(const T* __restrict__ X, const T* __restrict__ dY, const uint32_t* __restrict__ pair_i,
          const uint32_t* __restrict__ pair_j, const PlanHeader* __restrict__ hdr, float* __restrict__ partial,
          int Ci, int Co, int64_t chunk_len, int max_chunks, int ntiles_n) {
  using C = WgradCfg<T, BM, BN, BKP, WM, WN>;
  using E = Elt<T>;
  using frag_t = typename E::frag_t;
  constexpr int NT = C::kThreads;
  constexpr int G = C::kG;
  constexpr int V8 = C::kVec;

  const int chunk = blockIdx.x;
  const int k = blockIdx.y;
  const int64_t pk = hdr->pair_count[k];
  const int64_t start = int64_t(chunk) * chunk_len;
  if (start >= pk) return;
  const int64_t end = (start + chunk_len < pk) ? start + chunk_len : pk;
  const int64_t off = hdr->pair_off[k];
  const int m0 = (blockIdx.z / ntiles_n) * BM;
  const int c0 = (blockIdx.z % ntiles_n) * BN;

  __shared__ __align__(16) char lds_a[2 * C::kLdsA];
  __shared__ __align__(16) char lds_b[2 * C::kLdsB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  f32x16 acc[C::kFM][C::kFN];
#pragma unroll
  for (int i = 0; i < C::kFM; ++i)
#pragma unroll
    for (int j = 0; j < C::kFN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nstages = int((end - start + BKP - 1) / BKP);
  uint4 ra[C::kIA][G], rb[C::kIB][G];

  auto load_stage = [&](int s) {
    const int64_t p0 = off + start + int64_t(s) * BKP;
    const int64_t pend = off + end;
#pragma unroll
    for (int v = 0; v < C::kIA; ++v) {
      const int idx = tid + v * NT;
      const int grp = idx / (BM / V8), cv = idx % (BM / V8);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        uint4 val = make_uint4(0, 0, 0, 0);
        const int64_t p = p0 + grp * G + g;
        if (idx < C::kItemsA && p < pend && m0 + cv * V8 < Ci)
          val = *reinterpret_cast<const uint4*>(X + int64_t(pair_j[p]) * Ci + m0 + cv * V8);
        ra[v][g] = val;
      }
    }
#pragma unroll
    for (int v = 0; v < C::kIB; ++v) {
      const int idx = tid + v * NT;
      const int grp = idx / (BN / V8), cv = idx % (BN / V8);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        uint4 val = make_uint4(0, 0, 0, 0);
        const int64_t p = p0 + grp * G + g;
        if (idx < C::kItemsB && p < pend && c0 + cv * V8 < Co)
          val = *reinterpret_cast<const uint4*>(dY + int64_t(pair_i[p]) * Co + c0 + cv * V8);
        rb[v][g] = val;
      }
    }
  };
  // transposed store: LDS row = channel, column = pair
  auto store_one = [&](char* lds, const uint4 (&r)[G], int grp, int cv) {
    if constexpr (G == 1) {
      float* s = reinterpret_cast<float*>(lds);
      const float* f = reinterpret_cast<const float*>(&r[0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[(cv * 4 + e) * C::kLd + grp] = f[e];
    } else {
      // pack pairs (2 grp, 2 grp + 1) of each channel into one 32-bit word
      uint32_t* s = reinterpret_cast<uint32_t*>(lds);
      const uint16_t* lo = reinterpret_cast<const uint16_t*>(&r[0]);
      const uint16_t* hi = reinterpret_cast<const uint16_t*>(&r[1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[(cv * 8 + e) * (C::kLd / 2) + grp] = uint32_t(lo[e]) | (uint32_t(hi[e]) << 16);
    }
  };
  auto store_stage = [&](int buf) {
    char* sa = lds_a + buf * C::kLdsA;
    char* sb = lds_b + buf * C::kLdsB;
#pragma unroll
    for (int v = 0; v < C::kIA; ++v) {
      const int idx = tid + v * NT;
      if (idx < C::kItemsA) store_one(sa, ra[v], idx / (BM / V8), idx % (BM / V8));
    }
#pragma unroll
    for (int v = 0; v < C::kIB; ++v) {
      const int idx = tid + v * NT;
      if (idx < C::kItemsB) store_one(sb, rb[v], idx / (BN / V8), idx % (BN / V8));
    }
  };

  load_stage(0);
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    store_stage(buf);
    __syncthreads();
    if (s + 1 < nstages) load_stage(s + 1);
    const T* sa = reinterpret_cast<const T*>(lds_a + buf * C::kLdsA);
    const T* sb = reinterpret_cast<const T*>(lds_b + buf * C::kLdsB);
    const int koff = (lane >> 5) * E::kFrag;
#pragma unroll
    for (int kk = 0; kk < BKP; kk += E::kStep) {
      frag_t af[C::kFM], bfr[C::kFN];
#pragma unroll
      for (int i = 0; i < C::kFM; ++i) {
        const int r = wm * C::kTM + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const frag_t*>(sa + r * C::kLd + kk + koff);
      }
#pragma unroll
      for (int j = 0; j < C::kFN; ++j) {
        const int c = wn * C::kTN + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const frag_t*>(sb + c * C::kLd + kk + koff);
      }
#pragma unroll
      for (int i = 0; i < C::kFM; ++i)
#pragma unroll
        for (int j = 0; j < C::kFN; ++j) acc[i][j] = E::mfma(af[i], bfr[j], acc[i][j]);
    }
  }

  float* dst = partial + (int64_t(k) * max_chunks + chunk) * int64_t(Ci) * Co;
#pragma unroll
  for (int j = 0; j < C::kFN; ++j) {
    const int c = c0 + wn * C::kTN + j * 32 + (lane & 31);
    if (c >= Co) continue;
#pragma unroll
    for (int i = 0; i < C::kFM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * C::kTM + i * 32 + acc_row(lane, e);
        if (m < Ci) dst[int64_t(m) * Co + c] = acc[i][j][e];
      }
  }
}

// Weight gradient for 16-bit types, built on the gfx950 LDS transpose read.
// Gathered X rows (by j) and dY rows (by i) are stored in LDS as they sit in
// memory: row = pair, columns = channels, plain 16-byte writes.  The MFMA
// operands need 8 consecutive pairs of one channel per lane; the transpose
// read delivers them: within each 16-lane group, lane i receives element
// (i mod 4) of the 64-bit pieces addressed by lanes i/4, i/4+4, i/4+8 and
// i/4+12, so pointing lane j at pair row j/4, channels 4*(j mod 4)..+3 hands
// lane i channel i of four consecutive pairs.  Two such reads make one
// fragment.  Row strides are 64 bytes past a multiple of 256 so the four
// rows of a read fall in different bank groups.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

template <int C>
struct TrPad {
  // smallest padding (elements) giving a row of 2*(C+pad) bytes = 64 mod 256
  static constexpr int v = ((2 * C) % 256 == 64) ? 0 : ((64 - (2 * C) % 256 + 256) % 256) / 2;
};

template <typename T, int FM, int FN, int NWM, int NWN, int BKP>
struct WgradTrCfg {
  static constexpr int kThreads = 64 * NWM * NWN;
  static constexpr int kBM = NWM * FM * 32, kBN = NWN * FN * 32;
  static constexpr int kLdA = kBM + TrPad<kBM>::v, kLdB = kBN + TrPad<kBN>::v;
  static constexpr size_t kLdsA = size_t(BKP) * kLdA * 2, kLdsB = size_t(BKP) * kLdB * 2;
  static constexpr int kItemsA = BKP * kBM / 8, kItemsB = BKP * kBN / 8;
  static constexpr int kIA = (kItemsA + kThreads - 1) / kThreads, kIB = (kItemsB + kThreads - 1) / kThreads;
  // pair indices are staged through LDS in groups of kGP pairs, one group ahead
  static constexpr int kGP = 512;
  static constexpr int kSG = kGP / BKP;                 // stages per group
  static constexpr int kPI = kGP / kThreads;            // index pairs each thread fetches per group
  static_assert((2 * kLdA) % 256 == 64 && (2 * kLdB) % 256 == 64, "row stride must be 64 mod 256 bytes");
  static_assert(BKP % 16 == 0 && kGP % BKP == 0 && kGP % kThreads == 0, "bad staging sizes");
};

__device__ __forceinline__ s16x4 lds_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<void*>(p)));
}

// dbias stage 1: work item (x, y) sums rows [x*rows, (x+1)*rows) of the column
// vectors [y*cvb, (y+1)*cvb) (16 bytes each) with NT threads.  Thread t takes
// vector t % cvb and every (NT/cvb)-th row from phase t / cvb, four loads in
// flight, adding in increasing row order; the phases are then added in order.
// `red` is NT * (16 / sizeof(T)) floats of LDS.
template <typename T, int NT>
__device__ __forceinline__ void colsum_partial_block(int bx, int by, const T* __restrict__ dY, int64_t n, int Co,
                                                     int64_t rows, int cvb, float* __restrict__ part, float* red) {
  constexpr int VEC = 16 / int(sizeof(T));
  const int cv = threadIdx.x % cvb, ph = threadIdx.x / cvb, nph = NT / cvb;
  const int col = (by * cvb + cv) * VEC;
  const int64_t r0 = int64_t(bx) * rows;
  const int64_t r1 = (r0 + rows < n) ? r0 + rows : n;
  float acc[VEC];
#pragma unroll
  for (int q = 0; q < VEC; ++q) acc[q] = 0.f;
  auto add = [&](const u32x4& v) {
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int q = 0; q < VEC; ++q) acc[q] += Elt<T>::load(e[q]);
  };
  if (col < Co && ph < nph) {
    const T* base = dY + col;
    int64_t r = r0 + ph;
    for (; r + 3 * nph < r1; r += 4 * nph) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const u32x4*>(base + (r + u * nph) * Co);
#pragma unroll
      for (int u = 0; u < 4; ++u) add(v[u]);
    }
    for (; r < r1; r += nph) add(*reinterpret_cast<const u32x4*>(base + r * Co));
  }
  if (ph < nph) {
#pragma unroll
    for (int q = 0; q < VEC; ++q) red[(ph * cvb + cv) * VEC + q] = acc[q];
  }
  __syncthreads();
  for (int t = threadIdx.x; t < cvb * VEC; t += NT) {
    const int c = by * cvb * VEC + t;
    if (c >= Co) break;
    float sum = 0.f;
    for (int q = 0; q < nph; ++q) sum += red[q * cvb * VEC + t];
    part[int64_t(bx) * Co + c] = sum;
  }
}

template <typename T>
__global__ void __launch_bounds__(256) colsum_partial(const T* __restrict__ dY, int64_t n, int Co,
                                                      int64_t rows, int cvb, float* __restrict__ part) {
  __shared__ float red[256 * (16 / int(sizeof(T)))];
  colsum_partial_block<T, 256>(blockIdx.x, blockIdx.y, dY, n, Co, rows, cvb, part, red);
}

// dbias stage 2: 16 columns per work item, 16 phases each adding every 16th
// partial (four loads in flight), then the phases in a fixed order.  256 threads.
template <typename T>
__device__ __forceinline__ void colsum_final_block(int bx, const float* __restrict__ part, int nb, int Co,
                                                   T* __restrict__ dbias) {
  __shared__ float red[16][16];
  const int cl = threadIdx.x & 15, ph = threadIdx.x >> 4;
  const int c = bx * 16 + cl;
  float s = 0.f;
  if (c < Co) {
    int b = ph;
    for (; b + 48 < nb; b += 64) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = part[int64_t(b + 16 * u) * Co + c];
#pragma unroll
      for (int u = 0; u < 4; ++u) s += v[u];
    }
    for (; b < nb; b += 16) s += part[int64_t(b) * Co + c];
  }
  red[ph][cl] = s;
  __syncthreads();
  if (ph == 0 && c < Co) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) t += red[q][cl];
    dbias[c] = Elt<T>::store(t);
  }
}

template <typename T>
__global__ void __launch_bounds__(256) colsum_final(const float* __restrict__ part, int nb, int Co,
                                                    T* __restrict__ dbias) {
  colsum_final_block<T>(blockIdx.x, part, nb, Co, dbias);
}

// dbias stage 1 riding on a weight-gradient launch: workgroups past the
// weight-gradient grid each sum one (row block, column group) of dY.
template <typename T>
struct BiasJob {
  const T* dY;
  int64_t n, rows;
  int Co, cvb, nbx;  // nbx row blocks per column group
  unsigned first;    // first workgroup index of the job; no job when past the grid
  float* part;
};

// Pipeline: pair indices for group g+1 are written to LDS at the first stage
// of group g (fetched one group earlier into registers); row gathers for stage
// s+DEPTH are issued during stage s from indices already in LDS; the stage's
// rows go through double-buffered LDS into transpose reads and MFMAs.  As in
// the GEMM, no load sits under a branch (the compiler would drain the ring at
// the next wait): a pair past the chunk or a channel past the layer reads the
// plan's zero row, and the stage loop runs whole index groups, unrolled, with
// only the LDS store, the barrier and the MFMAs guarded by the stage bound.
template <typename T, int FM, int FN, int NWM, int NWN, int BKP, int DEPTH>
__global__ void __launch_bounds__(64 * NWM * NWN)
    wgrad_tr(const T* __restrict__ X, const T* __restrict__ dY, const uint32_t* __restrict__ pair_i,
             const uint32_t* __restrict__ pair_j, const PlanHeader* __restrict__ hdr, float* __restrict__ partial,
             int Ci, int Co, int64_t chunk_len, int max_chunks, int ntiles_m, int ntiles_n,
             const uint32_t* __restrict__ pseg, int pblk, int rows_bpc, const T* __restrict__ zrow,
             BiasJob<T> bj, int nk) {
  using C = WgradTrCfg<T, FM, FN, NWM, NWN, BKP>;
  using E = Elt<T>;
  using frag_t = typename E::frag_t;
  constexpr int NT = C::kThreads, BM = C::kBM, BN = C::kBN, SG = C::kSG, GP = C::kGP;
  static_assert(DEPTH >= 1 && DEPTH < C::kSG && C::kSG % DEPTH == 0,
                "prefetch depth must stay inside one index group and divide it");

  __shared__ __align__(16) char lds_a[2 * C::kLdsA];
  __shared__ __align__(16) char lds_b[2 * C::kLdsB];
  __shared__ uint32_t pidx[2][GP][2];  // (i, j) per pair; sentinel past the chunk

  if (blockIdx.x >= bj.first) {
    static_assert(NT * (16 / sizeof(T)) * sizeof(float) <= sizeof(lds_a), "column-sum scratch too small");
    const int j = int(blockIdx.x - bj.first);
    colsum_partial_block<T, NT>(j % bj.nbx, j / bj.nbx, bj.dY, bj.n, bj.Co, bj.rows, bj.cvb, bj.part,
                                reinterpret_cast<float*>(lds_a));
    return;
  }

  int k, chunk, mn;
  int64_t pbeg, pend;
  if (rows_bpc > 0) {
    // Row-range chunks (narrow layers): chunk c holds the pairs of every offset
    // whose output row lies in blocks [c*bpc, (c+1)*bpc) of kPairRows rows.  The
    // nk offsets of one chunk run together on one XCD and share its dY rows and
    // their neighbours' X rows in L2.  Empty segments still write zeros.
    const int nmn = ntiles_m * ntiles_n;
    int m;
    if (!xcd_group_work(max_chunks, nk * nmn, &chunk, &m)) return;
    k = m / nmn;
    mn = m % nmn;
    const int b0 = chunk * rows_bpc, b1 = (b0 + rows_bpc < pblk) ? b0 + rows_bpc : pblk;
    pbeg = pseg[int64_t(k) * (pblk + 1) + b0];
    pend = pseg[int64_t(k) * (pblk + 1) + b1];
  } else {
    // Pair-index chunks: the channel tiles of one (offset, chunk) run together
    // on one XCD, so the pair rows they all gather are shared in its L2; groups
    // cycle through the offsets first so every XCD gets dense and sparse ones.
    int g;
    if (!xcd_group_work(nk * max_chunks, ntiles_m * ntiles_n, &g, &mn)) return;
    k = g % nk;
    chunk = g / nk;
    const int64_t pk = hdr->pair_count[k];
    const int64_t start = int64_t(chunk) * chunk_len;
    if (start >= pk) return;
    const int64_t end = (start + chunk_len < pk) ? start + chunk_len : pk;
    const int64_t off = hdr->pair_off[k];
    pbeg = off + start;
    pend = off + end;
  }
  const int m0 = (mn / ntiles_n) * BM;
  const int c0 = (mn % ntiles_n) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int grp = lane >> 4, src = lane & 15;
  const int tr_row = (grp >> 1) * 8 + (src >> 2);
  const int tr_col = (grp & 1) * 16 + (src & 3) * 4;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nstages = int((pend - pbeg + BKP - 1) / BKP);

  uint32_t ri[C::kPI], rj[C::kPI];
  auto fetch_idx = [&](int g) {
#pragma unroll
    for (int q = 0; q < C::kPI; ++q) {
      const int64_t p = pbeg + int64_t(g) * GP + q * NT + tid;
      ri[q] = p < pend ? pair_i[p] : kSentinel;
      rj[q] = p < pend ? pair_j[p] : kSentinel;
    }
  };
  auto put_idx = [&](int g) {
#pragma unroll
    for (int q = 0; q < C::kPI; ++q) {
      pidx[g & 1][q * NT + tid][0] = ri[q];
      pidx[g & 1][q * NT + tid][1] = rj[q];
    }
  };

  u32x4 ra[DEPTH][C::kIA], rb[DEPTH][C::kIB];
  const int64_t zoff_x = reinterpret_cast<const char*>(zrow) - reinterpret_cast<const char*>(X);
  const int64_t zoff_y = reinterpret_cast<const char*>(zrow) - reinterpret_cast<const char*>(dY);
  auto load_stage = [&](int s, u32x4 (&da)[C::kIA], u32x4 (&db)[C::kIB]) {
    const uint32_t(*pi)[2] = pidx[(s / SG) & 1];
    const int r0 = (s % SG) * BKP;
#pragma unroll
    for (int v = 0; v < C::kIA; ++v) {
      const int idx0 = tid + v * NT;
      const int idx = idx0 < C::kItemsA ? idx0 : 0;  // surplus threads reload item 0 and store nothing
      const int r = idx / (BM / 8), cv = idx % (BM / 8);
      const uint32_t j = pi[r0 + r][1];
      const int64_t off = (j != kSentinel && m0 + cv * 8 < Ci) ? (int64_t(j) * Ci + m0 + cv * 8) * 2 : zoff_x;
      da[v] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(X) + off);
    }
#pragma unroll
    for (int v = 0; v < C::kIB; ++v) {
      const int idx0 = tid + v * NT;
      const int idx = idx0 < C::kItemsB ? idx0 : 0;
      const int r = idx / (BN / 8), cv = idx % (BN / 8);
      const uint32_t i = pi[r0 + r][0];
      const int64_t off = (i != kSentinel && c0 + cv * 8 < Co) ? (int64_t(i) * Co + c0 + cv * 8) * 2 : zoff_y;
      db[v] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(dY) + off);
    }
  };
  auto store_stage = [&](int buf, const u32x4 (&da)[C::kIA], const u32x4 (&db)[C::kIB]) {
    char* sa = lds_a + buf * C::kLdsA;
    char* sb = lds_b + buf * C::kLdsB;
#pragma unroll
    for (int v = 0; v < C::kIA; ++v) {
      const int idx = tid + v * NT;
      if (C::kIA * NT == C::kItemsA || idx < C::kItemsA) {
        const int r = idx / (BM / 8), cv = idx % (BM / 8);
        *reinterpret_cast<u32x4*>(sa + (size_t(r) * C::kLdA + cv * 8) * 2) = da[v];
      }
    }
#pragma unroll
    for (int v = 0; v < C::kIB; ++v) {
      const int idx = tid + v * NT;
      if (C::kIB * NT == C::kItemsB || idx < C::kItemsB) {
        const int r = idx / (BN / 8), cv = idx % (BN / 8);
        *reinterpret_cast<u32x4*>(sb + (size_t(r) * C::kLdB + cv * 8) * 2) = db[v];
      }
    }
  };
  auto frag = [&](const char* base, int ld, int row0, int col0) {
    const char* p = base + (size_t(row0 + tr_row) * ld + col0 + tr_col) * 2;
    const s16x4 lo = lds_tr16(p);
    const s16x4 hi = lds_tr16(p + size_t(4) * ld * 2);
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(frag_t, v);
  };
  auto compute = [&](int buf) {
    const char* sa = lds_a + buf * C::kLdsA;
    const char* sb = lds_b + buf * C::kLdsB;
#pragma unroll
    for (int kk = 0; kk < BKP; kk += 16) {
      frag_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = frag(sa, C::kLdA, kk, wm * FM * 32 + i * 32);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = frag(sb, C::kLdB, kk, wn * FN * 32 + j * 32);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = E::mfma(af[i], bfr[j], acc[i][j]);
    }
  };

  // prologue: indices of groups 0 (to LDS) and 1 (registers), first DEPTH stages of rows
  fetch_idx(0);
  put_idx(0);
  fetch_idx(1);
  __syncthreads();
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load_stage(d, ra[d], rb[d]);

  // whole index groups; a group's first stage always runs (the group count
  // rounds nstages up), so the index fetch and every row load are unconditional
  const int ngroups = (nstages + SG - 1) / SG;
  for (int g = 0; g < ngroups; ++g) {
#pragma unroll
    for (int t = 0; t < SG; ++t) {
      const int s = g * SG + t;
      const bool run = s < nstages;
      if (t == 0) {
        put_idx(g + 1);
        fetch_idx(g + 2);
      }
      if (run) {
        store_stage(s & 1, ra[t % DEPTH], rb[t % DEPTH]);
        __syncthreads();
      }
      load_stage(s + DEPTH, ra[t % DEPTH], rb[t % DEPTH]);
      if (run) compute(s & 1);
    }
  }

  float* dst = partial + (int64_t(k) * max_chunks + chunk) * int64_t(Ci) * Co;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int c = c0 + wn * FN * 32 + j * 32 + (lane & 31);
    if (c >= Co) continue;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + wm * FM * 32 + i * 32 + acc_row(lane, e);
        if (m < Ci) dst[int64_t(m) * Co + c] = acc[i][j][e];
      }
  }
}

// dW[k] = sum of offset k's chunk partials in chunk order.  Row-range chunking
// (rowmode) writes every chunk of every offset; pair-index chunking writes the
// first ceil(P_k / chunk_len).
template <typename T>
__global__ void __launch_bounds__(256) wgrad_reduce(const float* __restrict__ partial,
                                                    const PlanHeader* __restrict__ hdr, T* __restrict__ dW,
                                                    int64_t cico, int64_t chunk_len, int max_chunks, int rowmode,
                                                    const float* __restrict__ bias_part, int bias_nb, int Co,
                                                    T* __restrict__ dbias, int nk) {
  const int k = blockIdx.y;
  if (k == nk) {  // row nk of the grid: dbias stage 2, when the stage-1 partials ride along
    if (int(blockIdx.x) * 16 < Co) colsum_final_block<T>(blockIdx.x, bias_part, bias_nb, Co, dbias);
    return;
  }
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= cico) return;
  const int64_t pk = hdr->pair_count[k];
  const int nch = rowmode ? max_chunks : int((pk + chunk_len - 1) / chunk_len);
  const float* src = partial + int64_t(k) * max_chunks * cico + e;
  // chunks added in increasing order, eight loads in flight
  float s = 0.f;
  int c = 0;
  for (; c + 8 <= nch; c += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[int64_t(c + u) * cico];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; c < nch; ++c) s += src[int64_t(c) * cico];
  dW[int64_t(k) * cico + e] = Elt<T>::store(s);
}

template <typename T>
__global__ void zero_kernel(T* __restrict__ p, int64_t count) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (; i < count; i += stride) p[i] = Elt<T>::store(0.f);
}

// ---------------------------------------------------------------------------
// host-side configuration
// ---------------------------------------------------------------------------

// Offset-set parts per tile: only tiny problems (fewer than 128 of the
// smallest tiles) split each tile's offsets over up to 4 workgroups; measured
// on MI355X, a 2k-voxel layer runs 1.9x faster split four ways while a
// 24k-voxel layer (381 tiles) runs faster unsplit.
static int split_parts(int64_t n, int N) {
  const int64_t nblk = N > 128 ? (N + 255) / 256 : (N > 64 ? (N + 127) / 128 : (N > 32 ? (N + 63) / 64 : 1));
  const int64_t wg = (n + 63) / 64 * nblk;  // the smallest-tile count igemm_pick_rows may launch
  if (n == 0 || wg >= 128) return 1;
  int64_t sp = (512 + wg - 1) / wg;
  return int(sp > 4 ? 4 : sp);
}

// Weight-gradient tile edge for a channel count: fp32 uses the LDS-transposing
// kernel (up to 128), 16-bit types the transpose-read kernel (up to 256).
static int wgrad_tile(int c, int esize) {
  if (esize == 2 && c >= 256) return 256;
  return c >= 128 ? 128 : (c > 32 ? 64 : 32);
}

struct BwdShape {
  int bm = 0, bn = 0, mt = 0, nt = 0;
  int64_t chunk_len = 0;
  int max_chunks = 0;
  int rows_bpc = 0;  // > 0: row-range chunks of rows_bpc pair-list blocks
  int pblk = 0;
  int64_t bias_rows = 0;
  int bias_blocks = 0;
};

static BwdShape bwd_shape(int64_t n, int Ci, int Co, int esize) {
  BwdShape s;
  if (esize == 2) {
    // square tiles of the narrower side
    const int t = wgrad_tile(Ci < Co ? Ci : Co, 2);
    s.bm = s.bn = t;
  } else {
    s.bm = wgrad_tile(Ci, 4);
    s.bn = wgrad_tile(Co, 4);
  }
  s.mt = (Ci + s.bm - 1) / s.bm;
  s.nt = (Co + s.bn - 1) / s.bn;
  // aim for about 2048 workgroups at P ~ 14 n valid pairs; small layers stop
  // at a floor that keeps enough chunks in flight (measured on MI355X: the fp32
  // kernel on 1.9k voxels 72 -> 29 us at 256 instead of 1024 pairs; the 16-bit
  // kernel on 24k voxels 22.9 -> 21.3 us at 512, slower at 256)
  int64_t len = (14 * n * int64_t(s.mt) * s.nt + 2047) / 2048;
  len = (len + 255) / 256 * 256;
  const int64_t floor_len = esize == 2 ? 512 : 256;
  if (len < floor_len) len = floor_len;
  if (len > (int64_t(1) << 20)) len = int64_t(1) << 20;
  s.chunk_len = len;
  s.max_chunks = int(n > 0 ? (n + len - 1) / len : 1);
  s.pblk = int((n + kPairRows - 1) / kPairRows);
  if (esize == 2 && s.mt * s.nt == 1 && int64_t(Ci) * Co <= 64 * 64 && s.pblk >= 1024) {
    // one narrow channel tile and many rows: chunk by row ranges, about 512
    // chunks (measured best on a 6.4M-voxel, 64-channel layer; small or wide
    // layers keep pair-index chunks, which run faster there)
    s.rows_bpc = (s.pblk + 511) / 512;
    s.max_chunks = (s.pblk + s.rows_bpc - 1) / s.rows_bpc;
  }
  s.bias_rows = n > 0 ? (n + 511) / 512 : 1;
  if (s.bias_rows < 256) s.bias_rows = 256;
  s.bias_blocks = int(n > 0 ? (n + s.bias_rows - 1) / s.bias_rows : 1);
  return s;
}

struct WsLayout {
  size_t wt = 0, partial = 0, bias = 0, split = 0, part = 0, total = 0;
};

// Whether a submanifold layer of n rows may run its fwd / input-gradient GEMMs
// in two parts (the plan decides on the device whether it does): 16-bit types,
// many rows, wide channels on both sides.
static bool parts_possible(int64_t n, int Ci, int Co, int esize) {
  return esize == 2 && n >= kPartMinRows && Ci >= kPartMinChannels && Co >= kPartMinChannels;
}

// n_f: rows of the forward GEMM and of the weight gradient's pair lists (the
// output rows); n_b: rows of the input-gradient GEMM (the input rows).  Every
// region is disjoint, so the input gradient and the weight gradient may run
// concurrently on one workspace.
static WsLayout ws_layout(int64_t n_f, int64_t n_b, int Ci, int Co, int esize, bool parts) {
  WsLayout w;
  const BwdShape b = bwd_shape(n_f, Ci, Co, esize);
  size_t off = 0;
  w.wt = off;
  off = align_up(off + size_t(kV) * Ci * Co * esize, 256);
  w.partial = off;
  off = align_up(off + size_t(kV) * b.max_chunks * size_t(Ci) * Co * 4, 256);
  w.bias = off;
  off = align_up(off + size_t(b.bias_blocks) * Co * 4, 256);
  // Split-K partials of the forward (N = Co) or input-gradient (N = Ci) GEMM
  const int sf = split_parts(n_f, Co), sd = split_parts(n_b, Ci);
  const size_t sbytes_f = sf > 1 ? size_t(sf) * size_t(n_f) * Co * 4 : 0;
  const size_t sbytes_d = sd > 1 ? size_t(sd) * size_t(n_b) * Ci * 4 : 0;
  w.split = off;
  off = align_up(off + (sbytes_f > sbytes_d ? sbytes_f : sbytes_d), 256);
  // fp32 sums handed from the first GEMM part to the second ([n][Co] fwd, [n][Ci] dX)
  w.part = off;
  if (parts && parts_possible(n_f, Ci, Co, esize))
    off = align_up(off + size_t(n_f) * size_t(Ci > Co ? Ci : Co) * 4, 256);
  w.total = off;
  return w;
}

static int esize_of(int dtype) { return dtype == SSC_F32 ? 4 : 2; }

// Every row of X, dY, W and dW starts 16-byte aligned, so that each gather is
// whole 16-byte vectors: channel counts are multiples of 8 (16-bit) or 4 (fp32).
static bool channels_ok(int Ci, int Co, int dtype) {
  const int vec = dtype == SSC_F32 ? 4 : 8;
  return Ci > 0 && Co > 0 && Ci % vec == 0 && Co % vec == 0 && Ci <= 4096 && Co <= 4096;
}

template <typename T, int MW, int FM, int FN, int BK, int NWM, int NWN, int DEPTH, int KMAP, bool GM>
static void igemm_go(const T* A, const T* Bt, const T* bias, T* out, const uint32_t* nmap, const int32_t* perm,
                     const uint32_t* smask, const T* zrow, int64_t n, int K, int N, int flip, float* partial,
                     hipStream_t s, const GemmPart& gp) {
  constexpr int BM = NWM * FM * 32, BN = NWN * FN * 32;
  const int ntiles = int((n + BM - 1) / BM);
  const int nblk = (N + BN - 1) / BN;
  const int nsplit = split_parts(n, N);
  const int tgroup = nblk * nsplit == 1 ? kTileGroup : 1;
  const unsigned grid = xcd_group_grid((ntiles + tgroup - 1) / tgroup, tgroup * nblk * nsplit);
  igemm<T, FM, FN, BK, NWM, NWN, DEPTH, KMAP, MW, GM><<<grid, 64 * NWM * NWN, 0, s>>>(
      A, Bt, bias, out, nmap, perm, smask, zrow, n, K, N, flip, ntiles, nblk, nsplit, partial, tgroup, gp);
  if (nsplit > 1)
    split_reduce<T><<<unsigned((n * N + 255) / 256), 256, 0, s>>>(partial, nsplit, n, N, bias, perm, out);
}

// Tile choice (measured on MI355X): every wave owns 32 rows; the workgroup
// spans as many output channels as the layer has, up to 256, so the gathered
// rows are fetched once per channel block; 8 waves share one weight tile when
// there are enough rows to fill the chip, fewer waves (more, smaller
// workgroups) otherwise.  With 8 waves and a reduction of at most 128 (at most
// two stages per offset, so the gathers dominate) the rows are gathered whole
// (KMAP 2); wider reductions keep the register-only natural order.
template <typename T, int MW, int FN, bool GM>
static void igemm_pick_rows(const T* A, const T* Bt, const T* bias, T* out, const uint32_t* nmap,
                            const int32_t* perm, const uint32_t* smask, const T* zrow, int64_t n, int K, int N,
                            int flip, float* partial, hipStream_t s, const GemmPart& gp) {
  const int64_t nblk = (N + FN * 32 - 1) / (FN * 32);
  const int64_t wg256 = (n + 255) / 256 * nblk, wg128 = (n + 127) / 128 * nblk;
#define SSC_GO(NW, BK, DEPTH, KMAP) \
  igemm_go<T, MW, 1, FN, BK, NW, 1, DEPTH, KMAP, GM>(A, Bt, bias, out, nmap, perm, smask, zrow, n, K, N, flip, partial, \
                                                     s, \
                                                 gp)
#define SSC_BK(NW, DEPTH)                                                 \
  do {                                                                    \
    if constexpr (sizeof(T) == 4) {                                       \
      SSC_GO(NW, 16, 2, 0);                                               \
    } else {                                                              \
      if (K % 64 == 0) SSC_GO(NW, 64, DEPTH, 1);                          \
      else if (K % 32 == 0) SSC_GO(NW, 32, DEPTH, 1);                     \
      else SSC_GO(NW, 16, DEPTH, 1);                                      \
    }                                                                     \
  } while (0)
  // prefetch depth: as deep as the registers allow without spilling
  constexpr int D8 = FN >= 8 ? 2 : 3, D4 = FN >= 8 ? 3 : 4;
  if (FN >= 2 && wg256 >= 512) {
    if constexpr (sizeof(T) == 2) {
      if (K % 64 == 0 && K <= 128) {
        SSC_GO(8, 64, 2, 2);
        return;
      }
    }
    SSC_BK(8, D8);
  } else if (wg128 >= 128) {
    SSC_BK(4, D4);
  } else {
    SSC_BK(2, D4);
  }
#undef SSC_BK
#undef SSC_GO
}

// MW: columns of the sorted-order map rows (27, or 8 for the compact map of a
// 2x2x2 strided kernel); with flip the weight of column c is W[MW - 1 - c].
template <typename T, int MW, bool GM>
static void launch_igemm(const T* A, const T* Bt, const T* bias, T* out, const uint32_t* nmap,
                         const int32_t* perm, const uint32_t* smask, const T* zrow, int64_t n, int K, int N,
                         int flip, float* partial, hipStream_t s, const uint32_t* gmap) {
  // every offset, one row order; with flip, column c meets W[MW - 1 - c]
  const GemmPart gp{nullptr, 0, ~0u, 0, MW - 1, 0, nullptr, gmap};
  if (N > 128)
    igemm_pick_rows<T, MW, 8, GM>(A, Bt, bias, out, nmap, perm, smask, zrow, n, K, N, flip, partial, s, gp);
  else if (N > 64)
    igemm_pick_rows<T, MW, 4, GM>(A, Bt, bias, out, nmap, perm, smask, zrow, n, K, N, flip, partial, s, gp);
  else if (N > 32)
    igemm_pick_rows<T, MW, 2, GM>(A, Bt, bias, out, nmap, perm, smask, zrow, n, K, N, flip, partial, s, gp);
  else
    igemm_pick_rows<T, MW, 1, GM>(A, Bt, bias, out, nmap, perm, smask, zrow, n, K, N, flip, partial, s, gp);
}

// One gated part of a possibly split GEMM: wide layers only (parts_possible),
// so always 8 waves of 32 rows and 256 channels.
template <typename T, int MW, bool GM>
static void igemm_part_go(const T* A, const T* Bt, const T* bias, T* out, const uint32_t* nmap, const int32_t* perm,
                          const uint32_t* smask, const T* zrow, int64_t n, int K, int N, int flip, hipStream_t s,
                          const GemmPart& gp) {
  // Prefetch one stage ahead: at two stages the gather and weight rings take
  // the registers the weight fragments need, and the compiler then reads each
  // fragment just before its MFMA (measured on MI355X, C = 1024 layer of
  // random occupancy: 16.9 ms against 17.4 ms per input-gradient pass).
  if constexpr (sizeof(T) == 2) {
    if (K % 64 == 0)
      igemm_go<T, MW, 1, 8, 64, 8, 1, 1, 1, GM>(A, Bt, bias, out, nmap, perm, smask, zrow, n, K, N, flip, nullptr, s,
                                                gp);
    else if (K % 32 == 0)
      igemm_go<T, MW, 1, 8, 32, 8, 1, 1, 1, GM>(A, Bt, bias, out, nmap, perm, smask, zrow, n, K, N, flip, nullptr, s,
                                                gp);
    else
      igemm_go<T, MW, 1, 8, 16, 8, 1, 1, 1, GM>(A, Bt, bias, out, nmap, perm, smask, zrow, n, K, N, flip, nullptr, s,
                                                gp);
  }
}

// The fwd (flip = 0) or input-gradient (flip = 1) GEMM of a submanifold plan
// region whose build may have taken the three-part split: four gated launches,
// of which either the first (single order, every offset) or the other three
// do the work: part 2 (offsets 18..26) in the main order into pbuf, part 1
// (9..17) in its own order adding to pbuf, part 0 (0..8) in its own order
// adding pbuf, the bias and the rounding.
template <typename T>
static void launch_igemm_split(const T* A, const T* Bt, const T* bias, T* out, const char* region,
                               const int32_t* perm, int64_t n, int K, int N, int flip, float* pbuf, hipStream_t s,
                               const uint32_t* gmap) {
  const PlanLayout L = conv_layout(n);
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(region + L.header);
  const uint32_t* snmap = reinterpret_cast<const uint32_t*>(region + L.snmap);
  const uint32_t* smask = reinterpret_cast<const uint32_t*>(region + L.smask);
  const T* zrow = reinterpret_cast<const T*>(region + L.zrow);
  igemm_part_go<T, kV, true>(A, Bt, bias, out, snmap, perm, smask, zrow, n, K, N, flip, s,
                             GemmPart{h, 2, ~0u, 0, kV - 1, 0, nullptr, gmap});
  igemm_part_go<T, kV, true>(A, Bt, bias, out, snmap, perm, smask, zrow, n, K, N, flip, s,
                             GemmPart{h, 1, kTopPartMask, 0, kV - 1, 1, pbuf, gmap});
  for (int q = kOwnOrderParts - 1; q >= 0; --q) {
    const int lo = q * kPartCols;
    igemm_part_go<T, kPartCols, false>(A, Bt, bias, out,
                                reinterpret_cast<const uint32_t*>(region + L.psnmap) + int64_t(q) * n * kPartCols,
                                reinterpret_cast<const int32_t*>(region + L.pperm) + int64_t(q) * n,
                                reinterpret_cast<const uint32_t*>(region + L.psmask) + int64_t(q) * n, zrow, n, K, N,
                                flip, s, GemmPart{h, 1, kPartColMask, lo, kV - 1 - lo, q == 0 ? 2 : 3, pbuf});
  }
}

template <typename T>
static void launch_igemm_w(int mw, const T* A, const T* Bt, const T* bias, T* out, const uint32_t* nmap,
                           const int32_t* perm, const uint32_t* smask, const T* zrow, int64_t n, int K, int N,
                           int flip, float* partial, hipStream_t s, const uint32_t* gmap) {
  if (mw == kCompactCols)
    launch_igemm<T, kCompactCols, false>(A, Bt, bias, out, nmap, perm, smask, zrow, n, K, N, flip, partial, s,
                                         nullptr);
  else if (gmap)
    launch_igemm<T, kV, true>(A, Bt, bias, out, nmap, perm, smask, zrow, n, K, N, flip, partial, s, gmap);
  else
    launch_igemm<T, kV, false>(A, Bt, bias, out, nmap, perm, smask, zrow, n, K, N, flip, partial, s, nullptr);
}

// dbias stage 1 geometry: column vectors (16 bytes) per work item, all of them
// up to 32, as a power of two
static inline int colsum_cvb(int Co, int esize) {
  const int nvec = Co / (16 / esize);
  int cvb = 1;
  while (cvb < nvec && cvb < 32) cvb *= 2;
  return cvb;
}
static inline int colsum_groups(int Co, int esize) {
  const int nvec = Co / (16 / esize), cvb = colsum_cvb(Co, esize);
  return (nvec + cvb - 1) / cvb;
}

// Launches the weight-gradient partials.  With `bias_part` set (16-bit types),
// dbias stage 1 runs in the same launch, as extra workgroups after the grid;
// returns whether it did.
template <typename T>
static bool launch_wgrad(const T* X, const T* dY, const uint32_t* pi, const uint32_t* pj, const PlanHeader* h,
                         const uint32_t* pseg, const T* zrow, float* partial, int64_t n, int Ci, int Co,
                         const BwdShape& b, float* bias_part, int nk, hipStream_t s) {
  dim3 grid(unsigned(b.max_chunks), unsigned(nk), unsigned(b.mt * b.nt));
  if constexpr (sizeof(T) == 2) {
    const unsigned nwg = b.rows_bpc > 0 ? xcd_group_grid(b.max_chunks, nk * b.mt * b.nt)
                                        : xcd_group_grid(nk * b.max_chunks, b.mt * b.nt);
    BiasJob<T> bj{dY, n, b.bias_rows, Co, colsum_cvb(Co, 2), b.bias_blocks, nwg, bias_part};
    const unsigned nbias = bias_part ? unsigned(b.bias_blocks) * unsigned(colsum_groups(Co, 2)) : 0u;
    const dim3 grid1(nwg + nbias);
#define SSC_WTR(FM, FN, NWM, NWN)                                                                        \
  wgrad_tr<T, FM, FN, NWM, NWN, 32, 2><<<grid1, 64 * NWM * NWN, 0, s>>>(X, dY, pi, pj, h, partial, Ci, Co, \
                                                                       b.chunk_len, b.max_chunks, b.mt, b.nt, \
                                                                       pseg, b.pblk, b.rows_bpc, zrow, bj, nk)
    if (b.bm == 256) SSC_WTR(2, 4, 4, 2);
    else if (b.bm == 128) SSC_WTR(2, 2, 2, 2);
    else if (b.bm == 64) SSC_WTR(1, 1, 2, 2);
    else SSC_WTR(1, 1, 1, 1);
#undef SSC_WTR
    return bias_part != nullptr;
  } else {
  if (b.bm == 128 && b.bn == 128)
    wgrad<T, 128, 128, 32, 2, 2><<<grid, 256, 0, s>>>(X, dY, pi, pj, h, partial, Ci, Co, b.chunk_len,
                                                       b.max_chunks, b.nt);
  else if (b.bm == 128 && b.bn == 64)
    wgrad<T, 128, 64, 32, 2, 2><<<grid, 256, 0, s>>>(X, dY, pi, pj, h, partial, Ci, Co, b.chunk_len,
                                                      b.max_chunks, b.nt);
  else if (b.bm == 64 && b.bn == 128)
    wgrad<T, 64, 128, 32, 2, 2><<<grid, 256, 0, s>>>(X, dY, pi, pj, h, partial, Ci, Co, b.chunk_len,
                                                      b.max_chunks, b.nt);
  else if (b.bm == 64 && b.bn == 64)
    wgrad<T, 64, 64, 32, 2, 2><<<grid, 256, 0, s>>>(X, dY, pi, pj, h, partial, Ci, Co, b.chunk_len,
                                                     b.max_chunks, b.nt);
  else if (b.bm == 32 && b.bn == 32)
    wgrad<T, 32, 32, 32, 1, 1><<<grid, 64, 0, s>>>(X, dY, pi, pj, h, partial, Ci, Co, b.chunk_len,
                                                    b.max_chunks, b.nt);
  else if (b.bm == 32 && b.bn == 64)
    wgrad<T, 32, 64, 32, 1, 2><<<grid, 128, 0, s>>>(X, dY, pi, pj, h, partial, Ci, Co, b.chunk_len,
                                                     b.max_chunks, b.nt);
  else if (b.bm == 64 && b.bn == 32)
    wgrad<T, 64, 32, 32, 2, 1><<<grid, 128, 0, s>>>(X, dY, pi, pj, h, partial, Ci, Co, b.chunk_len,
                                                     b.max_chunks, b.nt);
  else if (b.bm == 32 && b.bn == 128)
    wgrad<T, 32, 128, 32, 1, 2><<<grid, 128, 0, s>>>(X, dY, pi, pj, h, partial, Ci, Co, b.chunk_len,
                                                      b.max_chunks, b.nt);
  else
    wgrad<T, 128, 32, 32, 2, 1><<<grid, 128, 0, s>>>(X, dY, pi, pj, h, partial, Ci, Co, b.chunk_len,
                                                      b.max_chunks, b.nt);
  }
  return false;
}

// What one convolution call reads from its plan.  The forward GEMM runs over
// the output rows (fwd region: sorted map into the input rows, masks, pair
// lists); the input-gradient GEMM runs over the input rows (bwd region: the
// transposed map with its columns flipped, k -> 26 - k).  A submanifold plan
// is one region serving both, with nk = 27 offsets.
struct ConvView {
  const char* fwd = nullptr;
  const int32_t* perm_f = nullptr;
  int64_t n_f = 0;  // output rows
  const char* bwd = nullptr;
  const int32_t* perm_b = nullptr;
  int64_t n_b = 0;  // input rows
  int nk = kV;      // weight offsets
  // sorted-order maps the GEMMs read and their row widths (NULL: the region's 27-wide snmap)
  const uint32_t* map_f = nullptr;
  const uint32_t* map_b = nullptr;
  int mw = kV;
  bool parts = false;  // a submanifold plan: its build may have taken the three-part split
  // a submanifold plan's map in original row order (the caller's nmap): the
  // GEMMs gather their tiles' rows of it through perm (the plan keeps no
  // sorted-order copy)
  const uint32_t* gmap = nullptr;
};

static size_t view_ws_bytes(const ConvView& v, int Ci, int Co, int esize) {
  return ws_layout(v.n_f, v.n_b, Ci, Co, esize, v.parts).total;
}

template <typename T>
static void zero_out(T* p, int64_t count, hipStream_t s) {
  if (!p || count <= 0) return;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  zero_kernel<T><<<unsigned(blocks), 256, 0, s>>>(p, count);
}

template <typename T>
static int run_fwd(const ConvView& v, int Ci, int Co, const void* feats, const void* weight, const void* bias,
                   void* out, char* ws, hipStream_t s) {
  if (v.n_f == 0) return SSC_OK;
  const PlanLayout L = conv_layout(v.n_f);
  const WsLayout W = ws_layout(v.n_f, v.n_b, Ci, Co, sizeof(T), v.parts);
  T* wt = reinterpret_cast<T*>(ws + W.wt);
  dim3 tg(unsigned((Co + 31) / 32), unsigned((Ci + 31) / 32), unsigned(v.nk));
  transpose_w<T><<<tg, 256, 0, s>>>(static_cast<const T*>(weight), wt, Ci, Co);
  if (v.parts && parts_possible(v.n_f, Ci, Co, sizeof(T))) {
    launch_igemm_split<T>(static_cast<const T*>(feats), wt, static_cast<const T*>(bias), static_cast<T*>(out), v.fwd,
                          v.perm_f, v.n_f, Ci, Co, 0, reinterpret_cast<float*>(ws + W.part), s, v.gmap);
    return SSC_OK;
  }
  launch_igemm_w<T>(v.mw, static_cast<const T*>(feats), wt, static_cast<const T*>(bias), static_cast<T*>(out),
                  v.map_f ? v.map_f : reinterpret_cast<const uint32_t*>(v.fwd + L.snmap), v.perm_f,
                  reinterpret_cast<const uint32_t*>(v.fwd + L.smask), reinterpret_cast<const T*>(v.fwd + L.zrow),
                  v.n_f, Ci, Co, 0, reinterpret_cast<float*>(ws + W.split), s, v.gmap);
  return SSC_OK;
}

template <typename T>
static int run_bwd(const ConvView& v, int Ci, int Co, const void* feats, const void* weight, const void* dout,
                   void* dfeats, void* dweight, void* dbias, char* ws, hipStream_t s) {
  const T* dY = static_cast<const T*>(dout);
  if (dfeats && v.n_b > 0) {
    // dX = masked implicit GEMM over the input rows of dY with B[k] = W[26-k]
    // read as [Ci][Co] (K = Co, N = Ci); the bwd map's column 26-k holds offset k
    const PlanLayout Lb = conv_layout(v.n_b);
    const WsLayout Wb = ws_layout(v.n_f, v.n_b, Ci, Co, sizeof(T), v.parts);
    if (v.n_f == 0) {
      zero_out<T>(static_cast<T*>(dfeats), v.n_b * Ci, s);  // no outputs: nothing reaches the inputs
    } else if (v.parts && parts_possible(v.n_b, Ci, Co, sizeof(T))) {
      launch_igemm_split<T>(dY, static_cast<const T*>(weight), nullptr, static_cast<T*>(dfeats), v.bwd, v.perm_b,
                            v.n_b, Co, Ci, 1, reinterpret_cast<float*>(ws + Wb.part), s, v.gmap);
    } else {
      launch_igemm_w<T>(v.mw, dY, static_cast<const T*>(weight), nullptr, static_cast<T*>(dfeats),
                      v.map_b ? v.map_b : reinterpret_cast<const uint32_t*>(v.bwd + Lb.snmap), v.perm_b,
                      reinterpret_cast<const uint32_t*>(v.bwd + Lb.smask),
                      reinterpret_cast<const T*>(v.bwd + Lb.zrow), v.n_b, Co, Ci, 1,
                      reinterpret_cast<float*>(ws + Wb.split), s, v.gmap);
    }
  }
  if (v.n_f == 0) {
    // no outputs: dW and dbias are zero
    if (dweight) zero_out<T>(static_cast<T*>(dweight), int64_t(v.nk) * Ci * Co, s);
    if (dbias) zero_out<T>(static_cast<T*>(dbias), Co, s);
    return SSC_OK;
  }
  const int64_t n = v.n_f;
  const PlanLayout L = conv_layout(n);
  const WsLayout W = ws_layout(n, v.n_b, Ci, Co, sizeof(T), v.parts);
  const BwdShape b = bwd_shape(n, Ci, Co, int(sizeof(T)));
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(v.fwd + L.header);
  float* bpart = reinterpret_cast<float*>(ws + W.bias);
  bool bias_done = false;
  if (dweight) {
    float* part = reinterpret_cast<float*>(ws + W.partial);
    const bool ride = launch_wgrad<T>(static_cast<const T*>(feats), dY,
                                      reinterpret_cast<const uint32_t*>(v.fwd + L.pair_i),
                                      reinterpret_cast<const uint32_t*>(v.fwd + L.pair_j), h,
                                      reinterpret_cast<const uint32_t*>(v.fwd + L.pseg),
                                      reinterpret_cast<const T*>(v.fwd + L.zrow), part, n, Ci, Co, b,
                                      dbias ? bpart : nullptr, v.nk, s);
    // with the stage-1 partials written by that launch, stage 2 is one more grid row here
    const int64_t cico = int64_t(Ci) * Co;
    int64_t rx = (cico + 255) / 256;
    if (ride && (Co + 15) / 16 > rx) rx = (Co + 15) / 16;
    dim3 rg(unsigned(rx), unsigned(v.nk + (ride ? 1 : 0)));
    wgrad_reduce<T><<<rg, 256, 0, s>>>(part, h, static_cast<T*>(dweight), cico, b.chunk_len, b.max_chunks,
                                       b.rows_bpc > 0 ? 1 : 0, bpart, b.bias_blocks, Co,
                                       static_cast<T*>(dbias), v.nk);
    bias_done = ride;
  }
  if (dbias && !bias_done) {
    const int cvb = colsum_cvb(Co, int(sizeof(T)));
    colsum_partial<T><<<dim3(unsigned(b.bias_blocks), unsigned(colsum_groups(Co, int(sizeof(T))))), 256, 0, s>>>(
        dY, n, Co, b.bias_rows, cvb, bpart);
    colsum_final<T><<<unsigned((Co + 15) / 16), 256, 0, s>>>(bpart, b.bias_blocks, Co, static_cast<T*>(dbias));
  }
  return SSC_OK;
}

template <typename F>
static void by_dtype(int dtype, F&& f) {
  if (dtype == SSC_F32)
    f(float{});
  else if (dtype == SSC_F16)
    f(_Float16{});
  else
    f(bf16s{});
}

}  // namespace ssc

using namespace ssc;

extern "C" size_t ssc_conv_workspace_bytes(int64_t n, int32_t Ci, int32_t Co, int32_t dtype) {
  if (dtype != SSC_F32 && dtype != SSC_F16 && dtype != SSC_BF16) return 0;
  if (n < 0 || n > SSC_MAX_VOXELS || !channels_ok(Ci, Co, dtype)) return 0;
  return ws_layout(n, n, Ci, Co, esize_of(dtype), true).total;
}

extern "C" int ssc_subm_conv3d_fwd(const void* plan, const uint32_t* nmap, const int32_t* perm, int64_t n,
                                   int32_t Ci, int32_t Co, int32_t dtype, const void* feats, const void* weight,
                                   const void* bias, void* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (n < 0 || n > SSC_MAX_VOXELS || !plan || !weight) return SSC_ERR_INVALID_ARG;
  if (dtype != SSC_F32 && dtype != SSC_F16 && dtype != SSC_BF16) return SSC_ERR_UNSUPPORTED;
  if (!channels_ok(Ci, Co, dtype)) return SSC_ERR_UNSUPPORTED;
  if (n > 0 && (!nmap || !perm || !feats || !out || !workspace)) return SSC_ERR_INVALID_ARG;
  const void* ptrs[] = {plan, nmap, perm, feats, weight, bias, out, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSC_ERR_INVALID_ARG;
  if (n == 0) return SSC_OK;
  if (workspace_bytes < ws_layout(n, n, Ci, Co, esize_of(dtype), true).total) return SSC_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const char* pl = static_cast<const char*>(plan);
  ConvView v{pl, perm, n, pl, perm, n, kV};
  v.parts = true;
  v.gmap = nmap;
  char* ws = static_cast<char*>(workspace);
  (void)hipGetLastError();
  by_dtype(dtype, [&](auto t) { run_fwd<decltype(t)>(v, Ci, Co, feats, weight, bias, out, ws, s); });
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}

// ---------------------------------------------------------------------------
// forward pass without a caller workspace
// ---------------------------------------------------------------------------

// The workspace of ssc_subm_conv3d_fwd_noalloc.  Each GPU the library runs on
// holds its own copy from module load until the process ends.  Host code must
// not use this name as a device address: the address of each GPU's copy comes
// from hipGetSymbolAddress, looked up once per GPU with that GPU current.
static __device__ __align__(256) char scratch[SSC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mutex;
void* scratch_address[kMaxScratchDevices] = {};

// Device address of the scratch array on the GPU that runs `stream`.
int scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return SSC_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return SSC_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return SSC_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_address[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return SSC_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return SSC_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return SSC_ERR_HIP;
    if (e != hipSuccess || !p) return SSC_ERR_HIP;
    scratch_address[dev] = p;
  }
  *out = scratch_address[dev];
  return SSC_OK;
}

}  // namespace

extern "C" int ssc_subm_conv3d_fwd_noalloc(const void* plan, const uint32_t* nmap, const int32_t* perm, int64_t n,
                                           int32_t Ci, int32_t Co, int32_t dtype, const void* feats,
                                           const void* weight, const void* bias, void* out, void* stream) {
  if (n < 0 || n > SSC_MAX_VOXELS || !plan || !weight) return SSC_ERR_INVALID_ARG;
  if (dtype != SSC_F32 && dtype != SSC_F16 && dtype != SSC_BF16) return SSC_ERR_UNSUPPORTED;
  if (!channels_ok(Ci, Co, dtype)) return SSC_ERR_UNSUPPORTED;
  if (n > 0 && (!nmap || !perm || !feats || !out)) return SSC_ERR_INVALID_ARG;
  const void* ptrs[] = {plan, nmap, perm, feats, weight, bias, out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSC_ERR_INVALID_ARG;
  if (n == 0) return SSC_OK;
  // the same workspace layout as ssc_subm_conv3d_fwd, checked before any HIP call
  if (ws_layout(n, n, Ci, Co, esize_of(dtype), true).total > size_t(SSC_NOALLOC_SCRATCH_BYTES))
    return SSC_ERR_SCRATCH;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const int st = scratch_for_stream(s, &ws);
  if (st != SSC_OK) return st;
  const char* pl = static_cast<const char*>(plan);
  ConvView v{pl, perm, n, pl, perm, n, kV};
  v.parts = true;
  v.gmap = nmap;
  (void)hipGetLastError();
  // every region of the workspace the forward kernels read is written first in
  // this call (W transposed, Split-K and part sums), so nothing is cleared
  by_dtype(dtype, [&](auto t) {
    run_fwd<decltype(t)>(v, Ci, Co, feats, weight, bias, out, static_cast<char*>(ws), s);
  });
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}

extern "C" int ssc_subm_conv3d_bwd(const void* plan, const uint32_t* nmap, const int32_t* perm, int64_t n,
                                   int32_t Ci, int32_t Co, int32_t dtype, const void* feats, const void* weight,
                                   const void* dout, void* dfeats, void* dweight, void* dbias, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (n < 0 || n > SSC_MAX_VOXELS || !plan) return SSC_ERR_INVALID_ARG;
  if (dtype != SSC_F32 && dtype != SSC_F16 && dtype != SSC_BF16) return SSC_ERR_UNSUPPORTED;
  if (!channels_ok(Ci, Co, dtype)) return SSC_ERR_UNSUPPORTED;
  if (dfeats && !weight) return SSC_ERR_INVALID_ARG;
  if (n > 0 && (!nmap || !perm || !dout || (dweight && !feats))) return SSC_ERR_INVALID_ARG;
  if ((dfeats || dweight || dbias) && !workspace) return SSC_ERR_INVALID_ARG;
  const void* ptrs[] = {plan, nmap, perm, feats, weight, dout, dfeats, dweight, dbias, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSC_ERR_INVALID_ARG;
  const int es = esize_of(dtype);
  if ((dfeats || dweight || dbias) && workspace_bytes < ws_layout(n, n, Ci, Co, es, true).total)
    return SSC_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const char* pl = static_cast<const char*>(plan);
  ConvView v{pl, perm, n, pl, perm, n, kV};
  v.parts = true;
  v.gmap = nmap;
  char* ws = static_cast<char*>(workspace);
  (void)hipGetLastError();
  by_dtype(dtype, [&](auto t) {
    run_bwd<decltype(t)>(v, Ci, Co, feats, weight, dout, dfeats, dweight, dbias, ws, s);
  });
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}

namespace {

// The strided-conv plan's two GEMM regions (their starts depend on n_in and n_out only).
ConvView sparse_view(const void* plan, int64_t n_in, int64_t n_out, int ks, const int32_t* perm_out) {
  const SparseOffsets o = sparse_offsets(n_in, n_out, ks);
  const char* base = static_cast<const char*>(plan);
  ConvView v{base + o.fwd, perm_out, n_out, base + o.bwd,
             reinterpret_cast<const int32_t*>(base + o.perm_in), n_in, ks * ks * ks};
  if (o.compact) {
    v.map_f = reinterpret_cast<const uint32_t*>(base + o.cmap_f);
    v.map_b = reinterpret_cast<const uint32_t*>(base + o.cmap_b);
    v.mw = kCompactCols;
  }
  return v;
}

bool sparse_sizes_ok(int64_t n_in, int64_t n_out, int32_t ks) {
  return n_in >= 0 && n_in <= SSC_MAX_VOXELS && n_out >= 0 && n_out <= SSC_MAX_VOXELS && ks >= 1 && ks <= 3;
}

}  // namespace

extern "C" size_t ssc_sparse_conv_workspace_bytes(int64_t n_in, int64_t n_out, int32_t Ci, int32_t Co,
                                                  int32_t dtype) {
  if (dtype != SSC_F32 && dtype != SSC_F16 && dtype != SSC_BF16) return 0;
  if (!sparse_sizes_ok(n_in, n_out, 1) || !channels_ok(Ci, Co, dtype)) return 0;
  ConvView v;
  v.n_f = n_out;
  v.n_b = n_in;
  return view_ws_bytes(v, Ci, Co, esize_of(dtype));
}

extern "C" int ssc_sparse_conv3d_fwd(const void* plan, int64_t n_in, int64_t n_out, int32_t ks,
                                     const int32_t* perm_out, int32_t Ci, int32_t Co, int32_t dtype,
                                     const void* feats, const void* weight, const void* bias, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!sparse_sizes_ok(n_in, n_out, ks) || !plan || !weight) return SSC_ERR_INVALID_ARG;
  if (dtype != SSC_F32 && dtype != SSC_F16 && dtype != SSC_BF16) return SSC_ERR_UNSUPPORTED;
  if (!channels_ok(Ci, Co, dtype)) return SSC_ERR_UNSUPPORTED;
  if (n_out > 0 && (!perm_out || !out || !workspace || (n_in > 0 && !feats))) return SSC_ERR_INVALID_ARG;
  const void* ptrs[] = {plan, perm_out, feats, weight, bias, out, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSC_ERR_INVALID_ARG;
  if (n_out == 0) return SSC_OK;
  const ConvView v = sparse_view(plan, n_in, n_out, ks, perm_out);
  if (workspace_bytes < view_ws_bytes(v, Ci, Co, esize_of(dtype))) return SSC_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  (void)hipGetLastError();
  by_dtype(dtype, [&](auto t) { run_fwd<decltype(t)>(v, Ci, Co, feats, weight, bias, out, ws, s); });
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}

extern "C" int ssc_sparse_conv3d_bwd(const void* plan, int64_t n_in, int64_t n_out, int32_t ks,
                                     const int32_t* perm_out, int32_t Ci, int32_t Co, int32_t dtype,
                                     const void* feats, const void* weight, const void* dout, void* dfeats,
                                     void* dweight, void* dbias, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (!sparse_sizes_ok(n_in, n_out, ks) || !plan) return SSC_ERR_INVALID_ARG;
  if (dtype != SSC_F32 && dtype != SSC_F16 && dtype != SSC_BF16) return SSC_ERR_UNSUPPORTED;
  if (!channels_ok(Ci, Co, dtype)) return SSC_ERR_UNSUPPORTED;
  if (dfeats && !weight) return SSC_ERR_INVALID_ARG;
  if (n_out > 0 && (!perm_out || !dout || (dweight && n_in > 0 && !feats))) return SSC_ERR_INVALID_ARG;
  if ((dfeats || dweight || dbias) && !workspace) return SSC_ERR_INVALID_ARG;
  const void* ptrs[] = {plan, perm_out, feats, weight, dout, dfeats, dweight, dbias, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSC_ERR_INVALID_ARG;
  const ConvView v = sparse_view(plan, n_in, n_out, ks, perm_out);
  if ((dfeats || dweight || dbias) && workspace_bytes < view_ws_bytes(v, Ci, Co, esize_of(dtype)))
    return SSC_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  (void)hipGetLastError();
  by_dtype(dtype, [&](auto t) {
    run_bwd<decltype(t)>(v, Ci, Co, feats, weight, dout, dfeats, dweight, dbias, ws, s);
  });
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}
