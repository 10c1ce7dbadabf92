// Voxel serialisation on gfx950: z-order and Hilbert codes of [b, x, y, z]
// rows and their inverses.
//
// The FlexGEMM pages name encode_seq / decode_seq over z_order_encode /
// decode and hilbert_encode / decode, with the code width (int32 or int64)
// chosen from the spatial size (contributor report, section two: the
// ops.serialize and kernels.cuda.serialize rows of the module table and the
// key-function table).  They give no bit layout; the one used here:
//   n     = ceil(log2(max(X, Y, Z))) bits per axis (the cube of side 2^n
//           that holds the grid);
//   code  = (b << 3n) | index(x, y, z);
//   index = z-order (bits interleaved from the top, x most significant in
//           each triplet; the row sort's key) or Hilbert;
//   width = int32 when the code fits 31 bits, else int64.
// The Hilbert index follows J. Skilling's transform between axes and the
// "transposed" index (Programming the Hilbert curve, AIP Conf. Proc. 707,
// 381, 2004), axes in the order (x, y, z); the transposed bits are then
// interleaved like the z-order index.
//
// One thread per row; both kernels are plain streams (16 bytes of
// coordinates and 4 or 8 bytes of code per row), bound by HBM.

#include <hip/hip_runtime.h>

#include "ssc_internal.h"

namespace ssc {

namespace {

// Grids have at most 2^20 cells per axis, so a curve has at most 20 levels;
// the level loops below run a fixed count (fully unrolled) with a uniform
// guard, and each per-axis step is a select, not a branch.
constexpr int kMaxLevel = 20;

// Axes -> transposed Hilbert index, in place.
__device__ __forceinline__ void hilbert_from_axes(uint32_t (&t)[3], int bits) {
#pragma unroll
  for (int lvl = kMaxLevel - 1; lvl >= 1; --lvl) {  // q = 2^lvl from the top bit down to 2
    if (lvl < bits) {
      const uint32_t q = 1u << lvl, low = q - 1;
      t[0] ^= (t[0] & q) ? low : 0u;  // axis 0: invert, or a swap with itself
#pragma unroll
      for (int i = 1; i < 3; ++i) {
        const uint32_t sw = (t[0] ^ t[i]) & low;
        const bool set = (t[i] & q) != 0;
        t[0] ^= set ? low : sw;
        t[i] ^= set ? 0u : sw;
      }
    }
  }
  t[1] ^= t[0];
  t[2] ^= t[1];
  uint32_t flip = 0;
#pragma unroll
  for (int lvl = kMaxLevel - 1; lvl >= 1; --lvl)
    if (lvl < bits && (t[2] & (1u << lvl))) flip ^= (1u << lvl) - 1;
  t[0] ^= flip;
  t[1] ^= flip;
  t[2] ^= flip;
}

// Transposed Hilbert index -> axes, in place.
__device__ __forceinline__ void hilbert_to_axes(uint32_t (&a)[3], int bits) {
  if (bits == 0) return;
  const uint32_t g = a[2] >> 1;
  a[2] ^= a[1];
  a[1] ^= a[0];
  a[0] ^= g;
#pragma unroll
  for (int lvl = 1; lvl < kMaxLevel; ++lvl) {  // q = 2^lvl from 2 up to the top bit
    if (lvl < bits) {
      const uint32_t q = 1u << lvl, low = q - 1;
#pragma unroll
      for (int i = 2; i >= 1; --i) {
        const uint32_t sw = (a[0] ^ a[i]) & low;
        const bool set = (a[i] & q) != 0;
        a[0] ^= set ? low : sw;
        a[i] ^= set ? 0u : sw;
      }
      a[0] ^= (a[0] & q) ? low : 0u;
    }
  }
}

// inverse of zorder(): the three axes of a z-order index
__device__ __forceinline__ void zorder_split(uint64_t code, int /*bits*/, uint32_t (&a)[3]) {
  a[0] = gather3(code >> 2);
  a[1] = gather3(code >> 1);
  a[2] = gather3(code);
}

template <typename CodeT>
__global__ void __launch_bounds__(256) seq_encode(const int4* __restrict__ coords, int64_t n, int B, int X,
                                                  int Y, int Z, int bits, int hilbert,
                                                  CodeT* __restrict__ codes) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int4 c = coords[i];
  if (c.x < 0 || c.x >= B || c.y < 0 || c.y >= X || c.z < 0 || c.z >= Y || c.w < 0 || c.w >= Z) {
    codes[i] = CodeT(-1);
    return;
  }
  uint32_t t[3] = {uint32_t(c.y), uint32_t(c.z), uint32_t(c.w)};
  if (hilbert) hilbert_from_axes(t, bits);
  codes[i] = CodeT((uint64_t(uint32_t(c.x)) << (3 * bits)) | zorder(t[0], t[1], t[2], bits));
}

template <typename CodeT>
__global__ void __launch_bounds__(256) seq_decode(const CodeT* __restrict__ codes, int64_t n, int B, int X,
                                                  int Y, int Z, int bits, int hilbert,
                                                  int4* __restrict__ coords) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t c = int64_t(codes[i]);
  int4 r = make_int4(-1, -1, -1, -1);
  if (c >= 0) {
    const uint64_t b = uint64_t(c) >> (3 * bits);
    const uint64_t idx = uint64_t(c) & ((uint64_t(1) << (3 * bits)) - 1);
    uint32_t a[3];
    zorder_split(idx, bits, a);
    if (hilbert) hilbert_to_axes(a, bits);
    if (b < uint64_t(B) && a[0] < uint32_t(X) && a[1] < uint32_t(Y) && a[2] < uint32_t(Z))
      r = make_int4(int(b), int(a[0]), int(a[1]), int(a[2]));
  }
  coords[i] = r;
}

bool dims_ok(int32_t B, int32_t X, int32_t Y, int32_t Z) {
  return B >= 1 && X >= 1 && Y >= 1 && Z >= 1 && B <= (1 << 20) && X <= (1 << 20) && Y <= (1 << 20) &&
         Z <= (1 << 20);
}

int axis_bits_of(int32_t X, int32_t Y, int32_t Z) {
  int32_t m = X > Y ? X : Y;
  if (Z > m) m = Z;
  return ceil_log2_u64(uint64_t(m));
}

int code_bits_of(int32_t B, int32_t X, int32_t Y, int32_t Z) {
  return 3 * axis_bits_of(X, Y, Z) + ceil_log2_u64(uint64_t(B));
}

unsigned blocks_for(int64_t n) { return unsigned((n + 255) / 256); }

}  // namespace

}  // namespace ssc

using namespace ssc;

extern "C" int32_t ssc_seq_code_bits(int32_t B, int32_t X, int32_t Y, int32_t Z) {
  if (!dims_ok(B, X, Y, Z)) return -1;
  return code_bits_of(B, X, Y, Z);
}

extern "C" int32_t ssc_seq_code_width(int32_t B, int32_t X, int32_t Y, int32_t Z) {
  if (!dims_ok(B, X, Y, Z)) return -1;
  const int bits = code_bits_of(B, X, Y, Z);
  if (bits > 63) return -1;
  return bits <= 31 ? 32 : 64;
}

static int seq_check(int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z, int32_t mode, int32_t code_width) {
  if (n < 0 || n > (int64_t(1) << 40)) return SSC_ERR_INVALID_ARG;
  if (!dims_ok(B, X, Y, Z)) return SSC_ERR_INVALID_ARG;
  if (mode != SSC_SEQ_ZORDER && mode != SSC_SEQ_HILBERT) return SSC_ERR_UNSUPPORTED;
  const int32_t need = ssc_seq_code_width(B, X, Y, Z);
  if (need < 0) return SSC_ERR_UNSUPPORTED;
  if (code_width != 32 && code_width != 64) return SSC_ERR_UNSUPPORTED;
  if (code_width < need) return SSC_ERR_UNSUPPORTED;
  return SSC_OK;
}

extern "C" int ssc_encode_seq(const int32_t* coords, int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z,
                              int32_t mode, void* codes, int32_t code_width, void* stream) {
  const int st = seq_check(n, B, X, Y, Z, mode, code_width);
  if (st != SSC_OK) return st;
  if (n == 0) return SSC_OK;
  if (!coords || !codes || !aligned16(coords)) return SSC_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(codes) & uintptr_t(code_width / 8 - 1)) != 0) return SSC_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int bits = axis_bits_of(X, Y, Z);
  const int4* c4 = reinterpret_cast<const int4*>(coords);
  (void)hipGetLastError();
  if (code_width == 32)
    seq_encode<int32_t><<<blocks_for(n), 256, 0, s>>>(c4, n, B, X, Y, Z, bits, mode, static_cast<int32_t*>(codes));
  else
    seq_encode<int64_t><<<blocks_for(n), 256, 0, s>>>(c4, n, B, X, Y, Z, bits, mode, static_cast<int64_t*>(codes));
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}

extern "C" int ssc_decode_seq(const void* codes, int64_t n, int32_t B, int32_t X, int32_t Y, int32_t Z,
                              int32_t mode, int32_t code_width, int32_t* coords, void* stream) {
  const int st = seq_check(n, B, X, Y, Z, mode, code_width);
  if (st != SSC_OK) return st;
  if (n == 0) return SSC_OK;
  if (!coords || !codes || !aligned16(coords)) return SSC_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(codes) & uintptr_t(code_width / 8 - 1)) != 0) return SSC_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int bits = axis_bits_of(X, Y, Z);
  int4* c4 = reinterpret_cast<int4*>(coords);
  (void)hipGetLastError();
  if (code_width == 32)
    seq_decode<int32_t><<<blocks_for(n), 256, 0, s>>>(static_cast<const int32_t*>(codes), n, B, X, Y, Z, bits,
                                                       mode, c4);
  else
    seq_decode<int64_t><<<blocks_for(n), 256, 0, s>>>(static_cast<const int64_t*>(codes), n, B, X, Y, Z, bits,
                                                       mode, c4);
  return hipGetLastError() == hipSuccess ? SSC_OK : SSC_ERR_HIP;
}
