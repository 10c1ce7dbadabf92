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
//                  K-slice) stages: gathered A rows and the offset's weight
//                  slice go through double-buffered LDS into 32x32 MFMA tiles
//                  with fp32 accumulators.  The epilogue adds bias, rounds once
//                  and writes each row at its original index perm[r].
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

#include "ssc_internal.h"

namespace ssc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct bf16s {
  uint16_t bits;
};

// round-to-nearest-even float -> bfloat16 bits
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

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

// Row index inside a 32x32 MFMA accumulator block held by `lane`, register i.
__device__ __forceinline__ int acc_row(int lane, int i) { return (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3); }

// ---------------------------------------------------------------------------
// masked implicit GEMM (forward and input gradient)
// ---------------------------------------------------------------------------

template <typename T, int BM, int BN, int BK, int WM, int WN>
struct IgemmCfg {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kVec = 16 / int(sizeof(T));          // elements per 16-byte load
  static constexpr int kPad = kVec;                         // LDS row padding (elements)
  static constexpr int kLd = BK + kPad;                     // LDS row stride (elements)
  static constexpr int kTM = BM / WM, kTN = BN / WN;        // per-wave tile
  static constexpr int kFM = kTM / 32, kFN = kTN / 32;      // MFMA blocks per wave
  static constexpr int kVpr = BK / kVec;                    // 16-byte vectors per tile row
  static constexpr int kAV = (BM * kVpr + kThreads - 1) / kThreads;
  static constexpr int kBV = (BN * kVpr + kThreads - 1) / kThreads;
  static constexpr size_t kLdsA = size_t(BM) * kLd * sizeof(T);
  static constexpr size_t kLdsB = size_t(BN) * kLd * sizeof(T);
  static_assert(kTM % 32 == 0 && kTN % 32 == 0, "wave tile must be whole 32x32 MFMA blocks");
  static_assert(BK % Elt<T>::kStep == 0 && BK % kVec == 0, "bad BK");
};

template <typename T, int BM, int BN, int BK, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
    igemm(const T* __restrict__ A, const T* __restrict__ Bt, const T* __restrict__ bias, T* __restrict__ out,
          const uint32_t* __restrict__ nmap, const int32_t* __restrict__ perm,
          const uint32_t* __restrict__ smask, int64_t n, int K, int N, int flip) {
  using C = IgemmCfg<T, BM, BN, BK, WM, WN>;
  using E = Elt<T>;
  using frag_t = typename E::frag_t;
  constexpr int NT = C::kThreads;

  __shared__ __align__(16) char lds_a[2 * C::kLdsA];
  __shared__ __align__(16) char lds_b[2 * C::kLdsB];
  __shared__ uint32_t jtab[kV][BM];
  __shared__ int32_t prow[BM];
  __shared__ uint32_t tile_union;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t row0 = int64_t(blockIdx.x) * BM;
  const int n0 = blockIdx.y * BN;

  // ---- prologue: rows, tile offset set, gather indices ----
  if (tid == 0) tile_union = 0;
  __syncthreads();
  for (int r = tid; r < BM; r += NT) {
    const int64_t g = row0 + r;
    int32_t p = -1;
    uint32_t m = 0;
    if (g < n) {
      p = perm[g];
      m = smask[g];
    }
    prow[r] = p;
    if (m) atomicOr(&tile_union, m);
  }
  __syncthreads();
  const uint32_t uni = tile_union;
  for (int e = tid; e < kV * BM; e += NT) {
    const int k = e / BM, r = e - k * BM;
    if ((uni >> k) & 1u) {
      const int32_t p = prow[r];
      jtab[k][r] = p >= 0 ? nmap[int64_t(p) * kV + k] : kSentinel;
    }
  }

  f32x16 acc[C::kFM][C::kFN];
#pragma unroll
  for (int i = 0; i < C::kFM; ++i)
#pragma unroll
    for (int j = 0; j < C::kFN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int kslices = K / BK;
  const int nstages = __popc(uni) * kslices;
  uint4 ra[C::kAV], rb[C::kBV];
  __syncthreads();  // jtab ready

  uint32_t rem = uni;
  int kcur = rem ? __ffs(rem) - 1 : 0;
  int kslice = 0;

  auto load_stage = [&](int k, int ks) {
    const int kb = flip ? (kV - 1 - k) : k;
    const int c0 = ks * BK;
#pragma unroll
    for (int v = 0; v < C::kAV; ++v) {
      const int idx = tid + v * NT;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (idx < BM * C::kVpr) {
        const int r = idx / C::kVpr, cv = idx % C::kVpr;
        const uint32_t j = jtab[k][r];
        if (j != kSentinel)
          val = *reinterpret_cast<const uint4*>(A + int64_t(j) * K + c0 + cv * C::kVec);
      }
      ra[v] = val;
    }
    const T* bbase = Bt + int64_t(kb) * N * K;
#pragma unroll
    for (int v = 0; v < C::kBV; ++v) {
      const int idx = tid + v * NT;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (idx < BN * C::kVpr) {
        const int r = idx / C::kVpr, cv = idx % C::kVpr;
        if (n0 + r < N) val = *reinterpret_cast<const uint4*>(bbase + int64_t(n0 + r) * K + c0 + cv * C::kVec);
      }
      rb[v] = val;
    }
  };
  auto store_stage = [&](int buf) {
    T* sa = reinterpret_cast<T*>(lds_a + buf * C::kLdsA);
    T* sb = reinterpret_cast<T*>(lds_b + buf * C::kLdsB);
#pragma unroll
    for (int v = 0; v < C::kAV; ++v) {
      const int idx = tid + v * NT;
      if (idx < BM * C::kVpr) {
        const int r = idx / C::kVpr, cv = idx % C::kVpr;
        *reinterpret_cast<uint4*>(sa + r * C::kLd + cv * C::kVec) = ra[v];
      }
    }
#pragma unroll
    for (int v = 0; v < C::kBV; ++v) {
      const int idx = tid + v * NT;
      if (idx < BN * C::kVpr) {
        const int r = idx / C::kVpr, cv = idx % C::kVpr;
        *reinterpret_cast<uint4*>(sb + r * C::kLd + cv * C::kVec) = rb[v];
      }
    }
  };

  if (nstages > 0) load_stage(kcur, 0);
  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    store_stage(buf);
    __syncthreads();
    if (s + 1 < nstages) {
      if (++kslice == kslices) {
        kslice = 0;
        rem &= rem - 1;
        kcur = __ffs(rem) - 1;
      }
      load_stage(kcur, kslice);
    }
    const T* sa = reinterpret_cast<const T*>(lds_a + buf * C::kLdsA);
    const T* sb = reinterpret_cast<const T*>(lds_b + buf * C::kLdsB);
    const int koff = (lane >> 5) * E::kFrag;
#pragma unroll
    for (int kk = 0; kk < BK; kk += E::kStep) {
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

  // ---- epilogue: bias, round once, scatter rows to perm ----
#pragma unroll
  for (int j = 0; j < C::kFN; ++j) {
    const int c = n0 + wn * C::kTN + j * 32 + (lane & 31);
    if (c >= N) continue;
    const float bv = bias ? E::load(bias[c]) : 0.f;
#pragma unroll
    for (int i = 0; i < C::kFM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = wm * C::kTM + i * 32 + acc_row(lane, e);
        const int32_t p = prow[r];
        if (p >= 0) out[int64_t(p) * N + c] = E::store(acc[i][j][e] + bv);
      }
    }
  }
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

template <typename T>
__global__ void __launch_bounds__(256) wgrad_reduce(const float* __restrict__ partial,
                                                    const PlanHeader* __restrict__ hdr, T* __restrict__ dW,
                                                    int64_t cico, int64_t chunk_len, int max_chunks) {
  const int k = blockIdx.y;
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= cico) return;
  const int64_t pk = hdr->pair_count[k];
  const int nch = int((pk + chunk_len - 1) / chunk_len);
  const float* src = partial + int64_t(k) * max_chunks * cico + e;
  float s = 0.f;
  for (int c = 0; c < nch; ++c) s += src[int64_t(c) * cico];
  dW[int64_t(k) * cico + e] = Elt<T>::store(s);
}

// dbias stage 1: block b sums rows [b*rows, (b+1)*rows) of every column
template <typename T>
__global__ void __launch_bounds__(256) colsum_partial(const T* __restrict__ dY, int64_t n, int Co,
                                                      int64_t rows, float* __restrict__ part) {
  const int64_t r0 = int64_t(blockIdx.x) * rows;
  const int64_t r1 = (r0 + rows < n) ? r0 + rows : n;
  for (int c = threadIdx.x; c < Co; c += 256) {
    float s = 0.f;
    for (int64_t r = r0; r < r1; ++r) s += Elt<T>::load(dY[r * Co + c]);
    part[int64_t(blockIdx.x) * Co + c] = s;
  }
}

template <typename T>
__global__ void __launch_bounds__(256) colsum_final(const float* __restrict__ part, int nb, int Co,
                                                    T* __restrict__ dbias) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= Co) return;
  float s = 0.f;
  for (int b = 0; b < nb; ++b) s += part[int64_t(b) * Co + c];
  dbias[c] = Elt<T>::store(s);
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

// Weight-gradient tile edge for a channel count.
static int wgrad_tile(int c) { return c >= 128 ? 128 : (c > 32 ? 64 : 32); }

struct BwdShape {
  int bm = 0, bn = 0, mt = 0, nt = 0;
  int64_t chunk_len = 0;
  int max_chunks = 0;
  int64_t bias_rows = 0;
  int bias_blocks = 0;
};

static BwdShape bwd_shape(int64_t n, int Ci, int Co) {
  BwdShape s;
  s.bm = wgrad_tile(Ci);
  s.bn = wgrad_tile(Co);
  s.mt = (Ci + s.bm - 1) / s.bm;
  s.nt = (Co + s.bn - 1) / s.bn;
  // aim for about 4096 workgroups at P ~ 14 n valid pairs
  int64_t len = (14 * n * int64_t(s.mt) * s.nt + 4095) / 4096;
  len = (len + 255) / 256 * 256;
  if (len < 1024) len = 1024;
  if (len > (int64_t(1) << 20)) len = int64_t(1) << 20;
  s.chunk_len = len;
  s.max_chunks = int(n > 0 ? (n + len - 1) / len : 1);
  s.bias_rows = n > 0 ? (n + 511) / 512 : 1;
  if (s.bias_rows < 256) s.bias_rows = 256;
  s.bias_blocks = int(n > 0 ? (n + s.bias_rows - 1) / s.bias_rows : 1);
  return s;
}

struct WsLayout {
  size_t wt = 0, partial = 0, bias = 0, total = 0;
};

static WsLayout ws_layout(int64_t n, int Ci, int Co, int esize) {
  WsLayout w;
  const BwdShape b = bwd_shape(n, Ci, Co);
  size_t off = 0;
  w.wt = off;
  off = align_up(off + size_t(kV) * Ci * Co * esize, 256);
  w.partial = off;
  off = align_up(off + size_t(kV) * b.max_chunks * size_t(Ci) * Co * 4, 256);
  w.bias = off;
  off = align_up(off + size_t(b.bias_blocks) * Co * 4, 256);
  w.total = off;
  return w;
}

static int esize_of(int dtype) { return dtype == SSC_F32 ? 4 : 2; }

static bool channels_ok(int Ci, int Co) {
  return Ci > 0 && Co > 0 && Ci % 16 == 0 && Co % 16 == 0 && Ci <= 4096 && Co <= 4096;
}

template <typename T>
static void launch_igemm(const T* A, const T* Bt, const T* bias, T* out, const uint32_t* nmap,
                         const int32_t* perm, const uint32_t* smask, int64_t n, int K, int N, int flip,
                         hipStream_t s) {
  const unsigned tiles = unsigned((n + 127) / 128);
  constexpr bool f32 = sizeof(T) == 4;
  // BK: the largest of 32/16 that divides K (16-bit MFMA reduces 16 at a time; fp32 takes 2)
  const bool bk32 = K % 32 == 0;
  if (N >= 128) {
    dim3 grid(tiles, unsigned((N + 127) / 128));
    if (bk32)
      igemm<T, 128, 128, 32, 2, 2><<<grid, 256, 0, s>>>(A, Bt, bias, out, nmap, perm, smask, n, K, N, flip);
    else
      igemm<T, 128, 128, 16, 2, 2><<<grid, 256, 0, s>>>(A, Bt, bias, out, nmap, perm, smask, n, K, N, flip);
  } else if (N > 32) {
    dim3 grid(tiles, unsigned((N + 63) / 64));
    if (bk32)
      igemm<T, 128, 64, 32, 4, 1><<<grid, 256, 0, s>>>(A, Bt, bias, out, nmap, perm, smask, n, K, N, flip);
    else
      igemm<T, 128, 64, 16, 4, 1><<<grid, 256, 0, s>>>(A, Bt, bias, out, nmap, perm, smask, n, K, N, flip);
  } else {
    dim3 grid(tiles, 1);
    if (bk32)
      igemm<T, 128, 32, 32, 4, 1><<<grid, 256, 0, s>>>(A, Bt, bias, out, nmap, perm, smask, n, K, N, flip);
    else
      igemm<T, 128, 32, 16, 4, 1><<<grid, 256, 0, s>>>(A, Bt, bias, out, nmap, perm, smask, n, K, N, flip);
  }
  (void)f32;
}

template <typename T>
static void launch_wgrad(const T* X, const T* dY, const uint32_t* pi, const uint32_t* pj, const PlanHeader* h,
                         float* partial, int Ci, int Co, const BwdShape& b, hipStream_t s) {
  dim3 grid(unsigned(b.max_chunks), kV, unsigned(b.mt * b.nt));
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

template <typename T>
static int run_fwd(const char* plan, const uint32_t* nmap, const int32_t* perm, int64_t n, int Ci, int Co,
                   const void* feats, const void* weight, const void* bias, void* out, char* ws,
                   hipStream_t s) {
  const PlanLayout L = conv_layout(n);
  const WsLayout W = ws_layout(n, Ci, Co, sizeof(T));
  T* wt = reinterpret_cast<T*>(ws + W.wt);
  dim3 tg(unsigned((Co + 31) / 32), unsigned((Ci + 31) / 32), kV);
  transpose_w<T><<<tg, 256, 0, s>>>(static_cast<const T*>(weight), wt, Ci, Co);
  launch_igemm<T>(static_cast<const T*>(feats), wt, static_cast<const T*>(bias), static_cast<T*>(out), nmap,
                  perm, reinterpret_cast<const uint32_t*>(plan + L.smask), n, Ci, Co, 0, s);
  return SSC_OK;
}

template <typename T>
static int run_bwd(const char* plan, const uint32_t* nmap, const int32_t* perm, int64_t n, int Ci, int Co,
                   const void* feats, const void* weight, const void* dout, void* dfeats, void* dweight,
                   void* dbias, char* ws, hipStream_t s) {
  const PlanLayout L = conv_layout(n);
  const WsLayout W = ws_layout(n, Ci, Co, sizeof(T));
  const BwdShape b = bwd_shape(n, Ci, Co);
  const PlanHeader* h = reinterpret_cast<const PlanHeader*>(plan + L.header);
  const T* dY = static_cast<const T*>(dout);
  if (dfeats) {
    // dX = masked implicit GEMM of dY with B[k] = W[26-k] read as [Ci][Co] (K = Co, N = Ci)
    launch_igemm<T>(dY, static_cast<const T*>(weight), nullptr, static_cast<T*>(dfeats), nmap, perm,
                    reinterpret_cast<const uint32_t*>(plan + L.smask), n, Co, Ci, 1, s);
  }
  if (dweight) {
    float* part = reinterpret_cast<float*>(ws + W.partial);
    launch_wgrad<T>(static_cast<const T*>(feats), dY, reinterpret_cast<const uint32_t*>(plan + L.pair_i),
                    reinterpret_cast<const uint32_t*>(plan + L.pair_j), h, part, Ci, Co, b, s);
    const int64_t cico = int64_t(Ci) * Co;
    dim3 rg(unsigned((cico + 255) / 256), kV);
    wgrad_reduce<T><<<rg, 256, 0, s>>>(part, h, static_cast<T*>(dweight), cico, b.chunk_len, b.max_chunks);
  }
  if (dbias) {
    float* part = reinterpret_cast<float*>(ws + W.bias);
    colsum_partial<T><<<unsigned(b.bias_blocks), 256, 0, s>>>(dY, n, Co, b.bias_rows, part);
    colsum_final<T><<<unsigned((Co + 255) / 256), 256, 0, s>>>(part, b.bias_blocks, Co, static_cast<T*>(dbias));
  }
  return SSC_OK;
}

}  // namespace ssc

using namespace ssc;

extern "C" size_t ssc_conv_workspace_bytes(int64_t n, int32_t Ci, int32_t Co, int32_t dtype) {
  if (n < 0 || n > SSC_MAX_VOXELS || !channels_ok(Ci, Co)) return 0;
  if (dtype != SSC_F32 && dtype != SSC_F16 && dtype != SSC_BF16) return 0;
  return ws_layout(n, Ci, Co, esize_of(dtype)).total;
}

extern "C" int ssc_subm_conv3d_fwd(const void* plan, const uint32_t* nmap, const int32_t* perm, int64_t n,
                                   int32_t Ci, int32_t Co, int32_t dtype, const void* feats, const void* weight,
                                   const void* bias, void* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (n < 0 || n > SSC_MAX_VOXELS || !plan || !weight) return SSC_ERR_INVALID_ARG;
  if (dtype != SSC_F32 && dtype != SSC_F16 && dtype != SSC_BF16) return SSC_ERR_UNSUPPORTED;
  if (!channels_ok(Ci, Co)) return SSC_ERR_UNSUPPORTED;
  if (n > 0 && (!nmap || !perm || !feats || !out || !workspace)) return SSC_ERR_INVALID_ARG;
  const void* ptrs[] = {plan, nmap, perm, feats, weight, bias, out, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSC_ERR_INVALID_ARG;
  if (n == 0) return SSC_OK;
  if (workspace_bytes < ws_layout(n, Ci, Co, esize_of(dtype)).total) return SSC_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const char* pl = static_cast<const char*>(plan);
  char* ws = static_cast<char*>(workspace);
  (void)hipGetLastError();
  if (dtype == SSC_F32)
    run_fwd<float>(pl, nmap, perm, n, Ci, Co, feats, weight, bias, out, ws, s);
  else if (dtype == SSC_F16)
    run_fwd<_Float16>(pl, nmap, perm, n, Ci, Co, feats, weight, bias, out, ws, s);
  else
    run_fwd<bf16s>(pl, nmap, perm, n, Ci, Co, feats, weight, bias, out, ws, s);
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}

extern "C" int ssc_subm_conv3d_bwd(const void* plan, const uint32_t* nmap, const int32_t* perm, int64_t n,
                                   int32_t Ci, int32_t Co, int32_t dtype, const void* feats, const void* weight,
                                   const void* dout, void* dfeats, void* dweight, void* dbias, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (n < 0 || n > SSC_MAX_VOXELS || !plan) return SSC_ERR_INVALID_ARG;
  if (dtype != SSC_F32 && dtype != SSC_F16 && dtype != SSC_BF16) return SSC_ERR_UNSUPPORTED;
  if (!channels_ok(Ci, Co)) return SSC_ERR_UNSUPPORTED;
  if (dfeats && !weight) return SSC_ERR_INVALID_ARG;
  if (n > 0 && (!nmap || !perm || !dout || (dweight && !feats))) return SSC_ERR_INVALID_ARG;
  if ((dfeats || dweight || dbias) && !workspace) return SSC_ERR_INVALID_ARG;
  const void* ptrs[] = {plan, nmap, perm, feats, weight, dout, dfeats, dweight, dbias, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSC_ERR_INVALID_ARG;
  const int es = esize_of(dtype);
  if ((dfeats || dweight || dbias) && workspace_bytes < ws_layout(n, Ci, Co, es).total) return SSC_ERR_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (n == 0) {
    // no voxels: dW and dbias are zero, dX is empty
    const int64_t wcount = int64_t(kV) * Ci * Co;
    if (dtype == SSC_F32) {
      if (dweight) zero_kernel<float><<<256, 256, 0, s>>>(static_cast<float*>(dweight), wcount);
      if (dbias) zero_kernel<float><<<1, 256, 0, s>>>(static_cast<float*>(dbias), Co);
    } else if (dtype == SSC_F16) {
      if (dweight) zero_kernel<_Float16><<<256, 256, 0, s>>>(static_cast<_Float16*>(dweight), wcount);
      if (dbias) zero_kernel<_Float16><<<1, 256, 0, s>>>(static_cast<_Float16*>(dbias), Co);
    } else {
      if (dweight) zero_kernel<bf16s><<<256, 256, 0, s>>>(static_cast<bf16s*>(dweight), wcount);
      if (dbias) zero_kernel<bf16s><<<1, 256, 0, s>>>(static_cast<bf16s*>(dbias), Co);
    }
    return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
  }
  const char* pl = static_cast<const char*>(plan);
  char* ws = static_cast<char*>(workspace);
  if (dtype == SSC_F32)
    run_bwd<float>(pl, nmap, perm, n, Ci, Co, feats, weight, dout, dfeats, dweight, dbias, ws, s);
  else if (dtype == SSC_F16)
    run_bwd<_Float16>(pl, nmap, perm, n, Ci, Co, feats, weight, dout, dfeats, dweight, dbias, ws, s);
  else
    run_bwd<bf16s>(pl, nmap, perm, n, Ci, Co, feats, weight, dout, dfeats, dweight, dbias, ws, s);
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}
