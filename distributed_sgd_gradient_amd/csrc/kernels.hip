// kernels.hip - gfx950 kernels of the Adasum combine.
//
// The pairwise operator of "Scaling Distributed Training with Adaptive
// Summation" needs the dot product and both norms of its operands before it
// can combine them (Sec. 4: the operation cannot be streamed).  Every node of
// the tree is a linear combination of the operands below it, so all the
// statistics of a subtree are quadratic forms in the Gram matrix of its
// operands.  A block (a subtree of at most 16 operands, four levels; 32
// operands and five levels for 16-bit inputs that fit one block) is
// therefore combined in three passes:
//   gram  - one pass over the operands: per tile, the Gram matrix (packed
//           upper triangle) on the matrix cores: fp64 instructions on the
//           widened values (exact products, fp64 sums) for fp32 operands and
//           for the fp64 slots of later stages, 32-row sums of exact
//           products added in fp64 for 16-bit operands, whose loads are
//           transposed through LDS for blocks of 16 or more (tiles of at
//           most 256 rows: exact products summed in double-double); reduced
//           across the workgroup in a fixed order;
//   tree  - per segment: the tile partials summed in tile order, then the
//           block's merges evaluated level by level on the Gram matrix:
//           d = wL.G.wR, A = wL.G.wL, B = wR.G.wR, ca = 1 - d/(2A),
//           cb = 1 - d/(2B) (coefficient 1 for a zero norm), and the
//           weights of the merged operands scaled by ca and cb; the walk
//           keeps these forms as the current nodes' dot products, each
//           merge updating those of its result;
//   wsum  - one pass: y = sum_k w_k x_k in fp64, rounded once.
// Each block's Gram entries carry a known rounding bound; the walk flags the
// (block, segment) pairs whose coefficients that rounding could move beyond
// tolerance (a merge under deep cancellation, where the quadratic forms
// amplify it); gram_exact recomputes their partials as double-double sums of
// exact products, the walk is repeated for them alone on double-double tile
// sums, and their weighted sums (with those of any block whose result is far
// smaller than its parts) are summed in double-double.
// The merge walk keeps its dot products in double-double (products of fp64
// coefficients with double-double entries), and the weighted sum uses separately rounded products and sums
// (no fused multiply-add); either way mirrored terms cancel exactly: an
// operand pair (a, -a) gives an exactly zero node, as the plain definition
// does.
//
// Every kernel walks tiles of the plan's tile table.  A tile lies inside
// one segment; its body starts at a multiple of kGroup elements, so vector
// loads and stores are 16-byte aligned (base pointers are 16-byte aligned);
// the unaligned head and the ragged tail are handled element by element.
// No atomics anywhere: results are bitwise reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "kernels.h"

namespace adasum {
namespace {

struct bf16_t {
  uint16_t bits;
};

// ----------------------------------------------------------------- element traits

// fp64 -> fp32 with round-to-odd: rounding that value once more to a format
// with at least two fewer significand bits is the correctly rounded result.
__device__ __forceinline__ float round_odd_f32(double x) {
  float f = (float)x;
  const double back = (double)f;
  if (back != x && x == x) {
    uint32_t u = __float_as_uint(f);
    if (fabs(back) > fabs(x)) u -= 1;  // step the magnitude down: truncation toward zero
    f = __uint_as_float(u | 1u);
  }
  return f;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Loads through address space 1, so that pointers fetched from argument
// tables still compile to global (not flat) memory instructions.
template <typename T>
__device__ __forceinline__ T gload(const T* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef double v2d __attribute__((ext_vector_type(2)));

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  struct Raw8 {
    v4f a, b;
  };
  static __device__ __forceinline__ Raw8 load_raw8(const float* p) {
    return Raw8{gload(reinterpret_cast<const v4f*>(p)), gload(reinterpret_cast<const v4f*>(p + 4))};
  }
  static __device__ __forceinline__ void unpack8(const Raw8& r, float (&v)[kGroup]) {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
  static __device__ __forceinline__ float load1(const float* p) { return gload(p); }
  static __device__ __forceinline__ void load8(const float* p, float (&v)[kGroup]) {
    const v4f a = gload(reinterpret_cast<const v4f*>(p));
    const v4f b = gload(reinterpret_cast<const v4f*>(p + 4));
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  // round x once to the storage type; also return the stored value widened
  static __device__ __forceinline__ float round(double x, double* stored) {
    const float f = (float)x;
    *stored = (double)f;
    return f;
  }
  static __device__ __forceinline__ void store1(float* p, float v) { *p = v; }
  static __device__ __forceinline__ void store8(float* p, const float (&v)[kGroup]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

template <>
struct Elem<_Float16> {
  typedef v4u Raw8;
  static __device__ __forceinline__ Raw8 load_raw8(const _Float16* p) { return gload(reinterpret_cast<const v4u*>(p)); }
  static __device__ __forceinline__ void unpack8(const Raw8& raw, float (&v)[kGroup]) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
      v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    }
  }
  static __device__ __forceinline__ float load1(const _Float16* p) { return (float)gload(p); }
  static __device__ __forceinline__ void load8(const _Float16* p, float (&v)[kGroup]) {
    const v4u raw = gload(reinterpret_cast<const v4u*>(p));
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
      v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    }
  }
  static __device__ __forceinline__ _Float16 round(double x, double* stored) {
    const _Float16 h = (_Float16)round_odd_f32(x);
    *stored = (double)(float)h;
    return h;
  }
  static __device__ __forceinline__ void store1(_Float16* p, _Float16 v) { *p = v; }
  static __device__ __forceinline__ void store8(_Float16* p, const _Float16 (&v)[kGroup]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)__builtin_bit_cast(uint16_t, v[2 * i]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

template <>
struct Elem<bf16_t> {
  static __device__ __forceinline__ float widen(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
  typedef v4u Raw8;
  static __device__ __forceinline__ Raw8 load_raw8(const bf16_t* p) { return gload(reinterpret_cast<const v4u*>(p)); }
  static __device__ __forceinline__ void unpack8(const Raw8& raw, float (&v)[kGroup]) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ float load1(const bf16_t* p) {
    return widen(gload(reinterpret_cast<const uint16_t*>(p)));
  }
  static __device__ __forceinline__ void load8(const bf16_t* p, float (&v)[kGroup]) {
    const v4u raw = gload(reinterpret_cast<const v4u*>(p));
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = widen(w[i] & 0xffffu);
      v[2 * i + 1] = widen(w[i] >> 16);
    }
  }
  static __device__ __forceinline__ bf16_t round(double x, double* stored) {
    const bf16_t b{f32_to_bf16_rne(round_odd_f32(x))};
    *stored = (double)widen(b.bits);
    return b;
  }
  static __device__ __forceinline__ void store1(bf16_t* p, bf16_t v) { *p = v; }
  static __device__ __forceinline__ void store8(bf16_t* p, const bf16_t (&v)[kGroup]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)v[2 * i].bits | ((uint32_t)v[2 * i + 1].bits << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// An fp64 slot: the block result that feeds a later stage, kept unrounded.
template <>
struct Elem<double> {
  static __device__ __forceinline__ double round(double x, double* stored) {
    *stored = x;
    return x;
  }
  static __device__ __forceinline__ void store1(double* p, double v) { *p = v; }
  static __device__ __forceinline__ void store8(double* p, const double (&v)[kGroup]) {
#pragma unroll
    for (int i = 0; i < kGroup; i += 2) *reinterpret_cast<v2d*>(p + i) = v2d{v[i], v[i + 1]};
  }
};

// A 16-bit input gradient read by a launch over fp64 slots (an input carried
// into a later stage), widened exactly to fp32.
template <typename TN>
__device__ __forceinline__ float narrow_to_f32(uint32_t bits16);
template <>
__device__ __forceinline__ float narrow_to_f32<_Float16>(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
template <>
__device__ __forceinline__ float narrow_to_f32<bf16_t>(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// ----------------------------------------------------------------- tiles

// Bounds of a tile: [lo, body_lo) head, [body_lo, body_hi) aligned body,
// [body_hi, hi) tail.
struct TileSpan {
  int64_t lo, body_lo, body_hi, hi;
};

__device__ __forceinline__ TileSpan span_of(const Tile& t) {
  TileSpan s;
  s.lo = t.start;
  s.hi = t.start + t.len;
  const int64_t up = (s.lo + kGroup - 1) & ~int64_t(kGroup - 1);
  s.body_lo = up < s.hi ? up : s.hi;
  const int64_t down = s.hi & ~int64_t(kGroup - 1);
  s.body_hi = down > s.body_lo ? down : s.body_lo;
  return s;
}

// ----------------------------------------------------------------- Gram pass, fp32 operands on the matrix cores

// An fp32 value widened to fp64 multiplies exactly (24 x 24 significant bits
// fit fp64's 53), and v_mfma_f64_16x16x4_f64 accumulates in fp64, so the
// matrix cores give the Gram block the accuracy of fp64 fused multiply-adds
// on exact products, with a handful of accumulator registers and no LDS
// staging: every lane loads 16 bytes (4 rows of one operand) per 16-row
// chunk, so many loads stay in flight.  Lane l, output register r holds
// D[l % 16][4 r + l / 16] (measured on gfx950).  Blocks of NB < 16 operands
// pack 16 / NB row sets into the 16 operand lanes: lane l carries operand
// (l % 16) % NB of row set (l % 16) / NB, and the Gram matrix is the sum of
// the diagonal NB x NB blocks of D.
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kF64Unroll = 16; // 16-row chunks per wave per iteration
constexpr int kGramWaves = kBlock / 64;

// Four consecutive fp32 values at rows [row, row + 4) of x, zero outside [lo, hi).
__device__ __forceinline__ v4f load_f32x4(const float* __restrict__ x, int64_t row, int64_t lo, int64_t hi) {
  if (row >= lo && row + 4 <= hi) return gload(reinterpret_cast<const v4f*>(x + row));
  float w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = (row + e >= lo && row + e < hi) ? gload(x + row + e) : 0.f;
  return v4f{w[0], w[1], w[2], w[3]};
}

// Double-double values (hi + lo, |lo| <= ulp(hi) / 2) for the merge walk's
// sums and the Gram entries of short tiles.  A node far smaller than the
// operands under it (a near-cancellation) makes its quadratic form cancel: summed in fp64, the rounding of the terms
// would be amplified by the ratio of their size to the result's.  With exact
// products (a fused multiply-add gives the product's rounding error) and
// compensated sums, the form is accurate to about 2^-104 of the terms.
// Terms that mirror each other still cancel exactly.
struct DD {
  double hi, lo;
};

__device__ __forceinline__ DD dd_prod(double a, double b) {
  const double p = a * b;
  return DD{p, fma(a, b, -p)};
}

__device__ __forceinline__ DD dd_add(DD x, DD y) {
  const double s = x.hi + y.hi;
  const double bb = s - x.hi;
  double e = (x.hi - (s - bb)) + (y.hi - bb);
  e += x.lo + y.lo;
  const double hi = s + e;
  return DD{hi, e - (hi - s)};
}

// s + x*y.  Products of fp32 or 16-bit values (widened) are exact in fp64,
// at most 48 significant bits, so their low part is zero and the
// fused multiply-add that would find it is skipped; products of fp64 values
// carry their rounding error in the low part.  The two forms give the same
// bits where both apply.
template <bool kExactProducts>
__device__ __forceinline__ DD dd_add_prod(DD s, double x, double y) {
  if constexpr (kExactProducts) {
    return dd_add(s, DD{x * y, 0.0});
  } else {
    return dd_add(s, dd_prod(x, y));
  }
}

__device__ __forceinline__ DD dd_scale(DD x, double b) {
  DD p = dd_prod(x.hi, b);
  p.lo += x.lo * b;
  const double hi = p.hi + p.lo;
  return DD{hi, p.lo - (hi - p.hi)};
}

__device__ __forceinline__ DD dd_mul(DD x, DD y) {
  DD p = dd_prod(x.hi, y.hi);
  p.lo += x.hi * y.lo + x.lo * y.hi;
  const double hi = p.hi + p.lo;
  return DD{hi, p.lo - (hi - p.hi)};
}

// Sum the four waves' 16 x 16 blocks (and the row sets' diagonal NB x NB
// blocks) in a fixed order; write the packed triangle to out.  Lane l,
// register r of a wave holds D[l % 16][4 r + l / 16].
template <int NB>
__device__ __forceinline__ void f64_gram_reduce(double (*red)[64 * 4], const f64x4& acc, double* out) {
  constexpr int SETS = 16 / NB;
  constexpr int NE = gram_entries(NB);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][lane * 4 + r] = acc[r];
  __syncthreads();
  for (int e = threadIdx.x; e < NE; e += kBlock) {
    int i = 0, rem = e;
    while (rem >= NB - i) {
      rem -= NB - i;
      ++i;
    }
    const int k = i + rem;  // entry (i, k), i <= k
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < kGramWaves; ++w)
#pragma unroll
      for (int q = 0; q < SETS; ++q) {
        const int m = q * NB + i, n = q * NB + k;  // D[m][n]: lane m + 16 (n % 4), register n / 4
        sum += red[w][(m + 16 * (n & 3)) * 4 + (n >> 2)];
      }
    out[e] = sum;
  }
}

// U: 16-row chunks per wave per iteration.  Plans of short tiles (at most
// kMinTile rows) take fewer chunks for blocks of 2 or 4 operands, so that
// the four waves share a tile's rows instead of one wave taking them all.
template <int NB, int U = kF64Unroll, typename GA = GramArgs>
__global__ __launch_bounds__(kBlock) void gram_f64mfma_kernel(GA args) {
  constexpr int SETS = 16 / NB;          // row sets packed into the 16 operand lanes
  constexpr int RC = 16 * SETS;          // rows per chunk
  constexpr int R = RC * U;              // rows per wave per iteration
  constexpr int NE = gram_entries(NB);
  static_assert(NB * SETS == 16, "NB divides 16");
  __shared__ double red[kGramWaves][64 * 4];

  const int tile_id = blockIdx.x;
  const int j = blockIdx.y;
  const Tile tile = args.tiles[tile_id];
  const int64_t lo = tile.start, hi = tile.start + tile.len;
  const int64_t first = lo & ~int64_t(kGroup - 1);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int op = (lane & 15) % NB, set = (lane & 15) / NB, grp = lane >> 4;

  // a NULL operand (beyond the block's count) reads operand 0, masked to zero
  const void* mine = args.x[j * op_stride(NB) + op];
  const bool live = mine != nullptr;
  const float* xp = static_cast<const float*>(live ? mine : args.x[j * op_stride(NB)]);

  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  const int64_t niter = (hi - first + R - 1) / R;
  const int64_t lane_row = (int64_t)set * 16 + 4 * grp;  // first row of this lane in a chunk
  for (int64_t it = wave; it < niter; it += kGramWaves) {
    const int64_t r0 = first + it * R;
    v4f v[U];
    if (r0 >= lo && r0 + R <= hi) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = gload(reinterpret_cast<const v4f*>(xp + r0 + u * RC + lane_row));
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = load_f32x4(xp, r0 + u * RC + lane_row, lo, hi);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!live) v[u] = v4f{0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)v[u].x, (double)v[u].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)v[u].y, (double)v[u].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)v[u].z, (double)v[u].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)v[u].w, (double)v[u].w, acc, 0, 0, 0);
    }
  }
  f64_gram_reduce<NB>(red, acc, args.partials + args.poff[j] + (int64_t)tile_id * NE);
}

// ----------------------------------------------------------------- Gram pass, stages above the first

// Operands of a later stage are fp64 slots (results of lower blocks) and, in
// lanes that the job's narrow mask marks, input gradients of type TN carried
// up (widened exactly).  Products of fp64 values are rounded by the matrix
// cores (an entry then errs by a few units of 2^-53 of the sum of |x_i x_j|,
// the bound the tree walk's flags assume), and flagged pairs are recomputed
// exactly.  Lane l reads four consecutive rows of its operand per 16-row
// chunk, as in the fp32 pass.
constexpr int kStageUnroll = 8;  // 16-row chunks per wave per iteration

// Zeros that the branch-free loads below read in place of the type an
// operand does not have (cache hits).
__device__ __align__(16) const double kZeroRow[4] = {0.0, 0.0, 0.0, 0.0};

// Four consecutive rows [row, row + 4) (all inside the tile) of an fp64 slot
// or, where narrow, a TN input, widened to fp64.  Both loads are issued
// whatever the operand's type (one of them from kZeroRow) and the values
// selected after, so that no branch separates the loads of an iteration:
// with a branch per operand the compiler waits on each load before the
// branch joins.
template <typename TN>
__device__ __forceinline__ void load_whole4(const void* p, bool narrow, int64_t row, double (&v)[4]) {
  const double* pd = narrow ? kZeroRow : static_cast<const double*>(p) + row;
  const v2d a = gload(reinterpret_cast<const v2d*>(pd));
  const v2d b = gload(reinterpret_cast<const v2d*>(pd + 2));
  double n[4];
  if constexpr (std::is_same<TN, float>::value) {
    const float* pf = narrow ? static_cast<const float*>(p) + row : reinterpret_cast<const float*>(kZeroRow);
    const v4f f = gload(reinterpret_cast<const v4f*>(pf));
    n[0] = f.x; n[1] = f.y; n[2] = f.z; n[3] = f.w;
  } else {
    const uint16_t* ph = narrow ? static_cast<const uint16_t*>(p) + row : reinterpret_cast<const uint16_t*>(kZeroRow);
    const v2u w = gload(reinterpret_cast<const v2u*>(ph));
    n[0] = narrow_to_f32<TN>(w.x & 0xffffu); n[1] = narrow_to_f32<TN>(w.x >> 16);
    n[2] = narrow_to_f32<TN>(w.y & 0xffffu); n[3] = narrow_to_f32<TN>(w.y >> 16);
  }
  v[0] = narrow ? n[0] : a.x;
  v[1] = narrow ? n[1] : a.y;
  v[2] = narrow ? n[2] : b.x;
  v[3] = narrow ? n[3] : b.y;
}

// Four consecutive rows [row, row + 4) of an fp64 slot or a TN input,
// widened to fp64, zero outside [lo, hi).
template <typename TN>
__device__ __forceinline__ void load_stage4(const void* p, bool narrow, int64_t row, int64_t lo, int64_t hi,
                                            double (&v)[4]) {
  const bool whole = row >= lo && row + 4 <= hi;
  if (!narrow) {
    const double* x = static_cast<const double*>(p);
    if (whole) {
      const v2d a = gload(reinterpret_cast<const v2d*>(x + row));
      const v2d b = gload(reinterpret_cast<const v2d*>(x + row + 2));
      v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (row + e >= lo && row + e < hi) ? gload(x + row + e) : 0.0;
    }
  } else if constexpr (std::is_same<TN, float>::value) {
    const v4f f = load_f32x4(static_cast<const float*>(p), row, lo, hi);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
    const uint16_t* x = static_cast<const uint16_t*>(p);
    if (whole) {
      const v2u w = gload(reinterpret_cast<const v2u*>(x + row));
      v[0] = narrow_to_f32<TN>(w.x & 0xffffu); v[1] = narrow_to_f32<TN>(w.x >> 16);
      v[2] = narrow_to_f32<TN>(w.y & 0xffffu); v[3] = narrow_to_f32<TN>(w.y >> 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = (row + e >= lo && row + e < hi) ? (double)narrow_to_f32<TN>(gload(x + row + e)) : 0.0;
    }
  }
}

template <int NB, typename TN>
__global__ __launch_bounds__(kBlock) void gram_stage_kernel(GramArgs args) {
  constexpr int SETS = 16 / NB;
  constexpr int U = kStageUnroll;
  constexpr int RC = 16 * SETS;
  constexpr int R = RC * U;
  constexpr int NE = gram_entries(NB);
  static_assert(NB * SETS == 16, "NB divides 16");
  __shared__ double red[kGramWaves][64 * 4];

  const int tile_id = blockIdx.x;
  const int j = blockIdx.y;
  const Tile tile = args.tiles[tile_id];
  const int64_t lo = tile.start, hi = tile.start + tile.len;
  const int64_t first = lo & ~int64_t(kGroup - 1);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int op = (lane & 15) % NB, set = (lane & 15) / NB, grp = lane >> 4;
  const void* mine = args.x[j * op_stride(NB) + op];
  const bool live = mine != nullptr;
  const void* xp = live ? mine : args.x[j * op_stride(NB)];
  // a masked operand reads operand 0, in operand 0's type
  const bool narrow = (args.narrow[j] >> (live ? op : 0)) & 1u;

  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  const int64_t niter = (hi - first + R - 1) / R;
  const int64_t lane_row = (int64_t)set * 16 + 4 * grp;
  for (int64_t it = wave; it < niter; it += kGramWaves) {
    const int64_t r0 = first + it * R;
    double v[U][4];
    if (r0 >= lo && r0 + R <= hi) {  // wave-uniform: the iteration's rows are all in the tile
#pragma unroll
      for (int u = 0; u < U; ++u) load_whole4<TN>(xp, narrow, r0 + u * RC + lane_row, v[u]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) load_stage4<TN>(xp, narrow, r0 + u * RC + lane_row, lo, hi, v[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double x = live ? v[u][e] : 0.0;
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(x, x, acc, 0, 0, 0);
      }
    }
  }
  f64_gram_reduce<NB>(red, acc, args.partials + args.poff[j] + (int64_t)tile_id * NE);
}

// ----------------------------------------------------------------- Gram pass, 16-bit operands

// For 16-bit operands the Gram matrix of a block is a dense contraction
// G = X^T X (X: rows x operands), done on the matrix cores: one
// v_mfma_f32_16x16x32 with the same register as both A and B gives the
// 16 x 16 Gram matrix of 32 rows.  Lane l holds operand l % 16 at rows
// 8 * (l / 16) .. +7 (one 16-byte load); output register r of lane l is
// G[4 * (l / 16) + r][l % 16].  Every instruction starts from zero and its
// four results go straight into fp64 accumulators, so the fp32 part of the
// sum is one instruction's 32 products.
//
// Those products are exact, and gfx950's matrix cores keep fp16 subnormal
// inputs and fp32 subnormal results: fp16 values are multiples of 2^-24
// below 2^16, so products are multiples of 2^-48 below 2^32; bf16 values
// with magnitudes in [2^-56, 2^61) are multiples of 2^-63, so their products
// are multiples of 2^-126 below 2^122, and 32 of them stay below 2^127.
// The hardware rounds the sum of the 32 products once (measured: the sum
// 1 + 31 * 2^-24 comes out as the nearest fp32 value wherever the 1 sits),
// so each entry is off by at most 2^-24 of the sum of |a_i b_i| over each
// 32-row chunk.
constexpr int kMfmaUnroll = 16;   // 32-row chunks per wave per iteration

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Mfma;

template <>
struct Mfma<_Float16> {
  static constexpr bool kGuard = false;  // every fp16 product is exact
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x4 gram(v4u a, v4u b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b),
                                                  f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
};

template <>
struct Mfma<bf16_t> {
  static constexpr bool kGuard = true;
  // magnitude bits of 2^-56 and 2^61: biased exponents 71 and 188
  static constexpr unsigned kLoBits = 71u << 7, kHiBits = 188u << 7;
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x4 gram(v4u a, v4u b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b),
                                                   f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  }
};

// Running range of the magnitude bits of packed 16-bit pairs: the largest,
// and the smallest nonzero one less one (zero wraps to 0xffff).
struct RangeU16 {
  u16x2 mx = {0, 0};
  u16x2 mn1 = {0xffff, 0xffff};
  __device__ __forceinline__ void add(uint32_t w) {
    const u16x2 m = __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
    mx = __builtin_elementwise_max(mx, m);
    mn1 = __builtin_elementwise_min(mn1, m - (u16x2){1, 1});
  }
  __device__ __forceinline__ bool outside(unsigned lo_bits, unsigned hi_bits) const {
    const unsigned hi = mx.x > mx.y ? mx.x : mx.y;
    const unsigned lo1 = mn1.x < mn1.y ? mn1.x : mn1.y;
    return hi >= hi_bits || lo1 < lo_bits - 1;
  }
};

// Eight raw 16-bit values at rows [row, row + 8) of x, zero outside [lo, hi).
__device__ __forceinline__ v4u load_raw_group(const uint16_t* __restrict__ x, int64_t row, int64_t lo, int64_t hi) {
  if (row >= lo && row + kGroup <= hi) return gload(reinterpret_cast<const v4u*>(x + row));
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    uint32_t pair = 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t i = row + 2 * h + e;
      if (i >= lo && i < hi) pair |= (uint32_t)gload(x + i) << (16 * e);
    }
    w[h] = pair;
  }
  return v4u{w[0], w[1], w[2], w[3]};
}

// A bf16 iteration holding a value outside [2^-56, 2^61) takes the scaled
// path: every operand is multiplied, per iteration, by the power of two that
// brings its largest magnitude just below 2^61 (exact, a change of exponent),
// the matrix cores run on the scaled values, and each result is scaled back
// exactly in fp64 by 2^-(s_row + s_col).  A product lost to the fp32 range
// then lies at least 2^-190 below the largest value of its operands, and an
// operand whose values are all tiny keeps its own full precision (its norm
// decides its Adasum coefficient).  Inf and NaN stay what they are and spoil
// only the entries of their own operand.
constexpr int kScaleTop = 127 + 60;  // biased exponent of the scaled maximum

// x * 2^s for a 16-bit bf16 value, rounded back to bf16 (exact unless the
// result leaves the normal range)
__device__ __forceinline__ uint32_t bf16_scale(uint32_t bits, int s) {
  const float f = (float)__builtin_amdgcn_ldexp((double)__uint_as_float(bits << 16), s);
  return __float_as_uint(f) >> 16;
}

__device__ __forceinline__ uint32_t bf16x2_scale(uint32_t w, int s) {
  return bf16_scale(w & 0xffffu, s) | (bf16_scale(w >> 16, s) << 16);
}

// Tiles of at most kExactRows rows skip the matrix cores: the tile is staged
// in LDS and every Gram entry is summed in fp64, row by row.  A product of
// two fp16 or two bf16 values is exact in fp64, so such an entry is the
// row-order sum of exact products, like an entry of the fp32 pass.  Short
// segments are where operands can nearly cancel by chance (a segment of a
// few elements is a short random vector); there the fp32 rounding of a
// 32-row matrix-core sum, amplified by the cancellation, would reach the
// coefficients.  (kExactRows: the plan's short-tile limit.)

template <typename T>
__device__ __forceinline__ double widen16(uint16_t bits);
template <>
__device__ __forceinline__ double widen16<_Float16>(uint16_t bits) {
  return (double)__builtin_bit_cast(_Float16, bits);
}
template <>
__device__ __forceinline__ double widen16<bf16_t>(uint16_t bits) {
  return (double)__uint_as_float((uint32_t)bits << 16);
}

// The packed Gram triangle of rows [lo, lo + len) of the operands in
// `table` (NULL: zero) into out, every entry the row-order double-double sum
// of exact products, its low part into out_lo (NULL: dropped).  The rows
// pass through sh (NB * kExactRows 16-bit values) kExactRows at a time.
// Called by every thread of the workgroup.
template <typename T, int NB, int NT = kBlock>
__device__ void gram_exact_rows(const void* const* table, int64_t lo, int64_t len, double* __restrict__ out,
                                double* __restrict__ out_lo, uint16_t* sh) {
  constexpr int NE = gram_entries(NB);
  constexpr int EPT = (NE + NT - 1) / NT;  // entries per thread
  int ei[EPT], ek[EPT];
  DD acc[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    const int e = threadIdx.x + q * NT;
    int i = 0, rem = e < NE ? e : 0;
    while (rem >= NB - i) {
      rem -= NB - i;
      ++i;
    }
    ei[q] = i;
    ek[q] = i + rem;
    acc[q] = DD{0.0, 0.0};
  }
  for (int64_t c0 = 0; c0 < len; c0 += kExactRows) {
    const int n = (int)min<int64_t>(kExactRows, len - c0);
    if (c0 > 0) __syncthreads();  // the previous chunk is consumed
    for (int idx = threadIdx.x; idx < NB * n; idx += NT) {
      const int k = idx / n, r = idx - k * n;
      const uint16_t* x = static_cast<const uint16_t*>(table[k]);
      sh[k * kExactRows + r] = x != nullptr ? gload(x + lo + c0 + r) : (uint16_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      if (threadIdx.x + q * NT >= NE) continue;
      const uint16_t* x = sh + ei[q] * kExactRows;
      const uint16_t* y = sh + ek[q] * kExactRows;
      DD sum = acc[q];
      for (int r = 0; r < n; ++r) sum = dd_add(sum, DD{widen16<T>(x[r]) * widen16<T>(y[r]), 0.0});  // exact product
      acc[q] = sum;
    }
  }
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    if (threadIdx.x + q * NT >= NE) continue;
    out[threadIdx.x + q * NT] = acc[q].hi;
    if (out_lo != nullptr) out_lo[threadIdx.x + q * NT] = acc[q].lo;
  }
}

// Exact recomputation of the Gram partials of every tile of a (block,
// segment) pair that the tree walk flagged (see TreeArgs): a merge far
// smaller than the operands under it (a near-cancellation) amplifies the
// rounding of the Gram entries into its statistics.  Every entry of such a
// tile is recomputed as the row-order double-double sum of exact products (a
// fused multiply-add gives each product's rounding error, so even products of
// fp64 slot values are exact), its high part written to partials and its low
// part to partials_lo; the refining walk then sums tiles in double-double.
// The rows pass through LDS kExactChunk at a time, in fp64.  Operand k is of
// type TIn, or TN where the job's narrow mask marks it (launches over fp64
// slots).  Tiles of other pairs return at once.
constexpr int kExactChunk = 128;

template <typename T>
__device__ __forceinline__ double widen_any(const void* p, int64_t i) {
  if constexpr (std::is_same<T, double>::value) return gload(static_cast<const double*>(p) + i);
  else if constexpr (std::is_same<T, float>::value) return (double)gload(static_cast<const float*>(p) + i);
  else return (double)narrow_to_f32<T>(gload(static_cast<const uint16_t*>(p) + i));
}

template <typename TIn, typename TN, int NB>
__global__ __launch_bounds__(kBlock) void gram_exact_kernel(GramArgs args) {
  constexpr int NE = gram_entries(NB);
  constexpr int EPT = (NE + kBlock - 1) / kBlock;  // entries per thread
  // rows padded by one double, so that the threads of a wave reading row r of
  // different operands hit different LDS banks
  __shared__ double sh[NB][kExactChunk + 1];
  const int tile_id = blockIdx.x;
  const int j = blockIdx.y;
  const Tile tile = args.tiles[tile_id];
  if ((args.flags[(int64_t)args.wrow[j] * args.nseg + tile.seg] & 1u) == 0) return;  // workgroup-uniform
  int ei[EPT], ek[EPT];
  DD acc[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    const int e = threadIdx.x + q * kBlock;
    int i = 0, rem = e < NE ? e : 0;
    while (rem >= NB - i) {
      rem -= NB - i;
      ++i;
    }
    ei[q] = i;
    ek[q] = i + rem;
    acc[q] = DD{0.0, 0.0};
  }
  for (int64_t c0 = 0; c0 < tile.len; c0 += kExactChunk) {
    const int n = (int)min<int64_t>(kExactChunk, tile.len - c0);
    if (c0 > 0) __syncthreads();  // the previous chunk is consumed
    for (int idx = threadIdx.x; idx < NB * n; idx += kBlock) {
      const int k = idx / n, r = idx - k * n;
      const void* x = args.x[j * op_stride(NB) + k];
      const int64_t row = tile.start + c0 + r;
      double v = 0.0;
      if (x != nullptr) {
        if constexpr (std::is_same<TIn, TN>::value) {
          v = widen_any<TIn>(x, row);
        } else {
          v = ((args.narrow[j] >> k) & 1u) ? widen_any<TN>(x, row) : widen_any<TIn>(x, row);
        }
      }
      sh[k][r] = v;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      if (threadIdx.x + q * kBlock >= NE) continue;
      const double* x = sh[ei[q]];
      const double* y = sh[ek[q]];
      DD sum = acc[q];
      for (int r = 0; r < n; ++r) sum = dd_add_prod<!std::is_same<TIn, double>::value>(sum, x[r], y[r]);
      acc[q] = sum;
    }
  }
  double* out = args.partials + args.poff[j] + (int64_t)tile_id * NE;
  double* out_lo = args.partials_lo + args.poff[j] + (int64_t)tile_id * NE;
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    if (threadIdx.x + q * kBlock >= NE) continue;
    out[threadIdx.x + q * kBlock] = acc[q].hi;
    out_lo[threadIdx.x + q * kBlock] = acc[q].lo;
  }
}

// Loads in the matrix cores' fragment layout; the launches use this kernel
// for blocks of 2 to 8 operands, whose few live streams read as fast in that
// layout (blocks of 16, 32 and 64 take the transposed loads of
// gram_tr_kernel and gram_wide_kernel below).  Blocks of up to 16 operands
// use one 16-operand group; a 32-operand block uses two, with three
// instructions per 32-row chunk: the two diagonal 16 x 16 blocks and the
// cross block (A from the first group, B from the second).
// Lane l, output register r of sub-block q = (h1, h2) holds
// G[16 h1 + 4 (l / 16) + r][16 h2 + l % 16].
template <typename T, int NB, typename GA = GramArgs>
__global__ __launch_bounds__(kBlock) void gram_mfma_kernel(GA args) {
  static_assert(NB <= 32, "one or two 16-operand groups");
  constexpr int NH = NB > 16 ? 2 : 1;  // 16-operand groups
  constexpr int NP = NH * (NH + 1) / 2;  // sub-blocks (h1 <= h2)
  constexpr int U = kMfmaUnroll / NH;  // chunks per wave per iteration
  constexpr int R = 32 * U;            // rows per wave per iteration
  constexpr int NE = gram_entries(NB);
  __shared__ double red[kGramWaves][NP][64 * 4];  // the wave sums of every sub-block

  const int tile_id = blockIdx.x;
  const int j = blockIdx.y;
  const Tile tile = args.tiles[tile_id];
  const int64_t lo = tile.start, hi = tile.start + tile.len;
  if (tile.len <= kExactRows) {  // workgroup-uniform: a short tile, summed exactly
    static_assert(sizeof(red) >= sizeof(uint16_t) * NB * kExactRows, "staging fits the reduction buffer");
    const int64_t at = args.poff[j] + (int64_t)tile_id * NE;
    gram_exact_rows<T, NB>(args.x + j * op_stride(NB), lo, tile.len, args.partials + at,
                           args.partials_lo != nullptr ? args.partials_lo + at : nullptr,
                           reinterpret_cast<uint16_t*>(&red[0][0][0]));
    return;
  }
  const int64_t first = lo & ~int64_t(kGroup - 1);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int op = lane & 15, grp = lane >> 4;

  // Lanes of absent operands (index >= NB, or a NULL slot) read operand 0
  // and are masked to zero, so every load of an iteration is unconditional.
  const void* const* table = args.x + j * op_stride(NB);
  const uint16_t* xp[NH];
  bool live[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int k = 16 * h + op;
    const void* mine = k < NB ? table[k] : nullptr;
    live[h] = mine != nullptr;
    xp[h] = static_cast<const uint16_t*>(live[h] ? mine : table[0]);
  }

  double acc[NP][4];
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[q][r] = 0.0;

  const int64_t niter = (hi - first + R - 1) / R;
  for (int64_t it = wave; it < niter; it += kGramWaves) {
    const int64_t r0 = first + it * R;
    v4u v[NH][U];
    if (r0 >= lo && r0 + R <= hi) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int h = 0; h < NH; ++h) v[h][u] = gload(reinterpret_cast<const v4u*>(xp[h] + r0 + 32 * u + 8 * grp));
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int h = 0; h < NH; ++h) v[h][u] = load_raw_group(xp[h], r0 + 32 * u + 8 * grp, lo, hi);
    }
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (!live[h]) v[h][u] = v4u{0u, 0u, 0u, 0u};

    bool scaled = false;
    int sc[NH] = {};  // per-operand power of two of the scaled path
    if constexpr (Mfma<T>::kGuard) {
      RangeU16 range;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          range.add(v[h][u].x);
          range.add(v[h][u].y);
          range.add(v[h][u].z);
          range.add(v[h][u].w);
        }
      scaled = __ballot(range.outside(Mfma<T>::kLoBits, Mfma<T>::kHiBits)) != 0;
      if (scaled) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          uint32_t m = 0;  // largest biased exponent among the lane's values
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const uint32_t w[4] = {v[h][u].x, v[h][u].y, v[h][u].z, v[h][u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) m = max(m, max((w[e] >> 7) & 0xffu, (w[e] >> 23) & 0xffu));
          }
          // the four lanes holding this operand's rows
          m = max(m, (uint32_t)__shfl_xor((int)m, 16));
          m = max(m, (uint32_t)__shfl_xor((int)m, 32));
          sc[h] = kScaleTop - (int)(m == 0 ? 1 : m);  // all-zero or subnormal operand: exponent 1
        }
        // entry (row, col) of sub-block (h1, h2): row operand 4 grp + r of
        // half h1 (its scale from the lane that holds it), column operand op
        // of half h2 (this lane's own)
        int back[NP][4];
        {
          int q = 0;
#pragma unroll
          for (int h1 = 0; h1 < NH; ++h1)
#pragma unroll
            for (int h2 = h1; h2 < NH; ++h2, ++q)
#pragma unroll
              for (int r = 0; r < 4; ++r) back[q][r] = -(__shfl(sc[h1], 4 * grp + r) + sc[h2]);
        }
        // one chunk at a time, read again (it was just read, so from cache):
        // scale, multiply, accumulate scaled back.  The registers of the
        // first read are free by now, which keeps this rare path from
        // raising the kernel's register count.
#pragma unroll 1
        for (int u = 0; u < U; ++u) {
          v4u c[NH];
#pragma unroll
          for (int h = 0; h < NH; ++h) {
            const int64_t row = r0 + 32 * u + 8 * grp;
            c[h] = live[h] ? load_raw_group(xp[h], row, lo, hi) : v4u{0u, 0u, 0u, 0u};
            c[h] = v4u{bf16x2_scale(c[h].x, sc[h]), bf16x2_scale(c[h].y, sc[h]), bf16x2_scale(c[h].z, sc[h]),
                       bf16x2_scale(c[h].w, sc[h])};
          }
          int q = 0;
#pragma unroll
          for (int h1 = 0; h1 < NH; ++h1)
#pragma unroll
            for (int h2 = h1; h2 < NH; ++h2, ++q) {
              const f32x4 d = Mfma<T>::gram(c[h1], c[h2]);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[q][r] += __builtin_amdgcn_ldexp((double)d[r], back[q][r]);
            }
        }
      }
    }
    if (!scaled) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int q = 0;
#pragma unroll
        for (int h1 = 0; h1 < NH; ++h1)
#pragma unroll
          for (int h2 = h1; h2 < NH; ++h2, ++q) {
            const f32x4 d = Mfma<T>::gram(v[h1][u], v[h2][u]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[q][r] += (double)d[r];
          }
      }
    }
  }

  double* out = args.partials + args.poff[j] + (int64_t)tile_id * NE;
  // Sum the four waves' matrices in wave order; write the packed triangle.
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][q][lane * 4 + r] = acc[q][r];
  __syncthreads();
  for (int e = threadIdx.x; e < NE; e += kBlock) {
    int i = 0, rem = e;
    while (rem >= NB - i) {
      rem -= NB - i;
      ++i;
    }
    const int k = i + rem;  // entry (i, k), i <= k
    const int q = (i >> 4) == 0 ? (k >> 4) : 2;  // (0,0) -> 0, (0,1) -> 1, (1,1) -> 2
    const int src = ((k & 15) + 16 * ((i & 15) >> 2)) * 4 + (i & 3);
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < kGramWaves; ++w) sum += red[w][q][src];
    out[e] = sum;
  }
}

// The 64-operand block (33 to 64 16-bit inputs, one stage), loaded in runs
// of 256 bytes per operand and transposed through LDS.  In the
// matrix cores' fragment layout a load instruction covers 64 bytes of each
// of 16 operands, and with all 64 operands in flight per wave that pattern
// reads at less than half the rate of 256-byte runs (2.8 against 6.0 TB/s,
// measured at this kernel's occupancy).  So each wave loads its 128 rows of
// all 64 operands as sixteen instructions of four operands (lane l of load
// i: operand 4 i + l / 16, rows 8 (l % 16) of the 128; bf16: 64 rows in
// 128-byte runs, eight operands per instruction), writes them to its
// own LDS area (operand-major, rows contiguous, each operand padded by 16
// bytes so that the fragment reads below are free of bank conflicts), and
// reads each 32-row chunk back in fragment layout: lane l, group h, operand
// 16 h + l % 16, rows 8 (l / 16) of the chunk.  The LDS area is the wave's
// own, so no workgroup barrier is needed inside the loop, and the next
// iteration's loads are issued as soon as this one's are in LDS, so that they
// fly during its matrix work.  Per 32-row chunk the ten instructions and the
// fp64 sums are those of gram_mfma_kernel; waves 1-3 then pass their sums
// through LDS and wave 0 adds them in wave order.  A bf16 iteration holding
// a value outside the matrix cores' exact range (see gram_mfma_kernel) is
// summed instead by each lane over its own forty entries, in fp64 from the
// staged rows: a product of two bf16 values is exact in fp64, and each
// entry adds its 128 products in row order.  That rare path takes few
// registers, which keeps the kernel at two waves per SIMD (the scaled
// matrix-core path of gram_mfma_kernel does not fit).
constexpr int kWideRows = 128;                   // rows per wave per iteration
constexpr int kWideStride = 2 * kWideRows + 16;  // bytes per operand in a wave's LDS area

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
__global__ __launch_bounds__(kBlock) void gram_wide_kernel(GramArgs args) {
  constexpr int NB = 64, NH = 4, NP = 10;
  // rows per wave per iteration: 64 for bf16, whose range check and exact
  // path need the registers that half the loads in flight free
  constexpr int ROWS = Mfma<T>::kGuard ? 64 : kWideRows;
  constexpr int STRIDE = 2 * ROWS + 16;  // bytes per operand in a wave's LDS area
  constexpr int LPO = ROWS / 8;          // load lanes per operand
  constexpr int OPI = 64 / LPO;          // operands per load instruction
  constexpr int C = ROWS / 32;           // chunks per iteration
  constexpr int L = NB / OPI;            // load instructions per iteration
  // the waves' staging areas; after the loop, the wave sums of waves 1-3
  constexpr int kStage = kGramWaves * NB * STRIDE, kRed = (kGramWaves - 1) * NP * 4 * 64 * 8;
  __shared__ __attribute__((aligned(16))) unsigned char stage[kStage > kRed ? kStage : kRed];
  const int tile_id = blockIdx.x;
  const int j = blockIdx.y;
  const Tile tile = args.tiles[tile_id];
  const int64_t lo = tile.start, hi = tile.start + tile.len;
  const void* const* table = args.x + j * op_stride(NB);
  if (tile.len <= kExactRows) {  // workgroup-uniform: a short tile, summed exactly
    static_assert(sizeof(stage) >= sizeof(uint16_t) * NB * kExactRows, "staging fits the transpose buffer");
    const int64_t at = args.poff[j] + (int64_t)tile_id * gram_entries(NB);
    gram_exact_rows<T, NB>(table, lo, tile.len, args.partials + at,
                           args.partials_lo != nullptr ? args.partials_lo + at : nullptr,
                           reinterpret_cast<uint16_t*>(&stage[0]));
    return;
  }
  const int64_t first = lo & ~int64_t(kGroup - 1);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int op = lane & 15, grp = lane >> 4;  // fragment lane
  const int sub = lane / LPO, rq = lane % LPO;  // load lane: operand OPI i + sub, rows 8 rq
  // Absent operands (a NULL slot) read operand 0 and are masked to zero.
  const uint16_t* xp[L];
  uint32_t live = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const void* p = table[OPI * i + sub];
    if (p != nullptr) live |= 1u << i;
    xp[i] = static_cast<const uint16_t*>(p != nullptr ? p : table[0]);
  }
  unsigned char* const st = &stage[wave * NB * STRIDE];

  double acc[NP][4];
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[q][r] = 0.0;

  v4u v[L];
  auto load = [&](int64_t it) {
    const int64_t r0 = first + it * ROWS;
    if (r0 >= lo && r0 + ROWS <= hi) {
#pragma unroll
      for (int i = 0; i < L; ++i) v[i] = gload(reinterpret_cast<const v4u*>(xp[i] + r0 + 8 * rq));
    } else {
#pragma unroll
      for (int i = 0; i < L; ++i) v[i] = load_raw_group(xp[i], r0 + 8 * rq, lo, hi);
    }
#pragma unroll
    for (int i = 0; i < L; ++i)
      if (!((live >> i) & 1u)) v[i] = v4u{0u, 0u, 0u, 0u};
  };

  const int64_t niter = (hi - first + ROWS - 1) / ROWS;
  if (wave < niter) load(wave);
  for (int64_t it = wave; it < niter; it += kGramWaves) {
    bool outside = false;  // bf16: some value of the iteration is outside the exact range
    if constexpr (Mfma<T>::kGuard) {
      RangeU16 range;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        range.add(v[i].x);
        range.add(v[i].y);
        range.add(v[i].z);
        range.add(v[i].w);
      }
      outside = __ballot(range.outside(Mfma<T>::kLoBits, Mfma<T>::kHiBits)) != 0;  // wave-uniform
    }
#pragma unroll
    for (int i = 0; i < L; ++i) *reinterpret_cast<v4u*>(st + (OPI * i + sub) * STRIDE + 16 * rq) = v[i];
    if (it + kGramWaves < niter) load(it + kGramWaves);  // in flight during this iteration's matrix work
    wave_sync();  // the staged rows are visible to the whole wave
    if (outside) {
      if constexpr (Mfma<T>::kGuard) {
        // Entry (row, col) of sub-block (h1, h2): row operand 16 h1 + 4 grp + r,
        // column operand 16 h2 + op.  One entry at a time (a runtime loop,
        // so that this rare path holds few registers), added to its sum by
        // a select over the lane's forty sums.
#pragma unroll 1
        for (int e = 0; e < NP * 4; ++e) {
          const int q = e >> 2, r = e & 3;
          const int h1 = q < 4 ? 0 : q < 7 ? 1 : q < 9 ? 2 : 3;  // (h1, h2), h1 <= h2, in order
          const int h2 = h1 + q - (h1 == 0 ? 0 : h1 == 1 ? 4 : h1 == 2 ? 7 : 9);
          const unsigned char* xi = st + (16 * h1 + 4 * grp + r) * STRIDE;
          const unsigned char* xk = st + (16 * h2 + op) * STRIDE;
          double sum = 0.0;
#pragma unroll 1
          for (int g = 0; g < ROWS / 8; ++g) {
            const v4u a = *reinterpret_cast<const v4u*>(xi + 16 * g);
            const v4u b = *reinterpret_cast<const v4u*>(xk + 16 * g);
            const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              sum = fma(widen16<T>((uint16_t)(wa[x] & 0xffffu)), widen16<T>((uint16_t)(wb[x] & 0xffffu)), sum);
              sum = fma(widen16<T>((uint16_t)(wa[x] >> 16)), widen16<T>((uint16_t)(wb[x] >> 16)), sum);
            }
          }
#pragma unroll
          for (int q2 = 0; q2 < NP; ++q2)
#pragma unroll
            for (int r2 = 0; r2 < 4; ++r2) acc[q2][r2] = (4 * q2 + r2 == e) ? acc[q2][r2] + sum : acc[q2][r2];
        }
      }
      wave_sync();  // the staged rows are read before the next iteration stages its own
      continue;
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      v4u f[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h)
        f[h] = *reinterpret_cast<const v4u*>(st + (16 * h + op) * STRIDE + 2 * (32 * c + 8 * grp));
      int q = 0;
#pragma unroll
      for (int h1 = 0; h1 < NH; ++h1)
#pragma unroll
        for (int h2 = h1; h2 < NH; ++h2, ++q) {
          const f32x4 d = Mfma<T>::gram(f[h1], f[h2]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[q][r] += (double)d[r];
        }
    }
    wave_sync();  // the fragments are read before the next iteration stages its rows
  }

  // Waves 1-3 pass their matrices through LDS; wave 0 adds them to its own in
  // wave order and writes its lanes' entries of the packed triangle.
  __syncthreads();  // every wave is done with its staging area
  double(*red)[NP][4 * 64] = reinterpret_cast<double(*)[NP][4 * 64]>(&stage[0]);
  if (wave > 0) {
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave - 1][q][r * 64 + lane] = acc[q][r];
  }
  __syncthreads();
  if (wave == 0) {
    double* out = args.partials + args.poff[j] + (int64_t)tile_id * gram_entries(NB);
    int q = 0;
#pragma unroll
    for (int h1 = 0; h1 < NH; ++h1)
#pragma unroll
      for (int h2 = h1; h2 < NH; ++h2, ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * h1 + 4 * grp + r, k = 16 * h2 + op;
          if (i > k) continue;
          double sum = acc[q][r];
#pragma unroll
          for (int w = 0; w < kGramWaves - 1; ++w) sum += red[w][q][r * 64 + lane];
          out[gram_index(NB, i, k)] = sum;
        }
  }
}

// Blocks of 16 and 32 16-bit operands (one or two 16-operand groups) with the
// same loads: 256-byte runs per operand staged in each wave's LDS area and
// read back in fragment layout, the next iteration's loads in flight during
// the matrix work.  bf16 keeps the range check and scaled path of
// gram_mfma_kernel, on the staged rows: per wave and iteration, every operand
// scaled by the power of two that brings its largest value of the 128 rows
// just below 2^61.  The waves' matrices are summed in wave order, as there.
template <typename T, int NB, typename GA = GramArgs>
__global__ __launch_bounds__(kBlock) void gram_tr_kernel(GA args) {
  static_assert(NB == 16 || NB == 32, "one or two 16-operand groups");
  constexpr int NH = NB / 16, NP = NH * (NH + 1) / 2, NE = gram_entries(NB);
  constexpr int C = kWideRows / 32;  // chunks per iteration
  constexpr int L = NB / 4;          // load instructions per iteration
  constexpr int kStage = kGramWaves * NB * kWideStride, kRed = kGramWaves * NP * 64 * 4 * 8;
  constexpr int kBytes = kStage > kRed ? kStage : kRed;
  static_assert(kBytes >= (int)sizeof(uint16_t) * NB * kExactRows, "staging fits the short-tile rows");
  __shared__ __attribute__((aligned(16))) unsigned char stage[kBytes];
  __shared__ int scale[kGramWaves][NB];  // bf16 scaled path: per-operand power of two of the wave's iteration
  const int tile_id = blockIdx.x;
  const int j = blockIdx.y;
  const Tile tile = args.tiles[tile_id];
  const int64_t lo = tile.start, hi = tile.start + tile.len;
  const void* const* table = args.x + j * op_stride(NB);
  if (tile.len <= kExactRows) {  // workgroup-uniform: a short tile, summed exactly
    const int64_t at = args.poff[j] + (int64_t)tile_id * NE;
    gram_exact_rows<T, NB>(table, lo, tile.len, args.partials + at,
                           args.partials_lo != nullptr ? args.partials_lo + at : nullptr,
                           reinterpret_cast<uint16_t*>(&stage[0]));
    return;
  }
  const int64_t first = lo & ~int64_t(kGroup - 1);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int op = lane & 15, grp = lane >> 4;  // fragment lane
  const int sub = lane >> 4, rq = lane & 15;  // load lane: operand 4 i + sub, rows 8 rq
  // Absent operands (a NULL slot) read operand 0 and are masked to zero.
  const uint16_t* xp[L];
  uint32_t live = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const void* p = table[4 * i + sub];
    if (p != nullptr) live |= 1u << i;
    xp[i] = static_cast<const uint16_t*>(p != nullptr ? p : table[0]);
  }
  unsigned char* const st = &stage[wave * NB * kWideStride];

  double acc[NP][4];
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[q][r] = 0.0;

  v4u v[L];
  auto load = [&](int64_t it) {
    const int64_t r0 = first + it * kWideRows;
    if (r0 >= lo && r0 + kWideRows <= hi) {
#pragma unroll
      for (int i = 0; i < L; ++i) v[i] = gload(reinterpret_cast<const v4u*>(xp[i] + r0 + 8 * rq));
    } else {
#pragma unroll
      for (int i = 0; i < L; ++i) v[i] = load_raw_group(xp[i], r0 + 8 * rq, lo, hi);
    }
#pragma unroll
    for (int i = 0; i < L; ++i)
      if (!((live >> i) & 1u)) v[i] = v4u{0u, 0u, 0u, 0u};
  };
  auto fragment = [&](int h, int c) {
    return *reinterpret_cast<const v4u*>(st + (16 * h + op) * kWideStride + 2 * (32 * c + 8 * grp));
  };

  const int64_t niter = (hi - first + kWideRows - 1) / kWideRows;
  if (wave < niter) load(wave);
  for (int64_t it = wave; it < niter; it += kGramWaves) {
    bool scaled = false;
    if constexpr (Mfma<T>::kGuard) {
      RangeU16 range;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        range.add(v[i].x);
        range.add(v[i].y);
        range.add(v[i].z);
        range.add(v[i].w);
      }
      scaled = __ballot(range.outside(Mfma<T>::kLoBits, Mfma<T>::kHiBits)) != 0;  // wave-uniform
      if (scaled) {
#pragma unroll
        for (int i = 0; i < L; ++i) {
          const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
          uint32_t m = 0;  // largest biased exponent among the lane's values
#pragma unroll
          for (int e = 0; e < 4; ++e) m = max(m, max((w[e] >> 7) & 0xffu, (w[e] >> 23) & 0xffu));
          // over the sixteen lanes that hold this operand's 128 rows
          m = max(m, (uint32_t)__shfl_xor((int)m, 1));
          m = max(m, (uint32_t)__shfl_xor((int)m, 2));
          m = max(m, (uint32_t)__shfl_xor((int)m, 4));
          m = max(m, (uint32_t)__shfl_xor((int)m, 8));
          if (rq == 0) scale[wave][4 * i + sub] = kScaleTop - (int)(m == 0 ? 1 : m);  // all-zero: exponent 1
        }
      }
    }
#pragma unroll
    for (int i = 0; i < L; ++i) *reinterpret_cast<v4u*>(st + (4 * i + sub) * kWideStride + 16 * rq) = v[i];
    if (it + kGramWaves < niter) load(it + kGramWaves);  // in flight during this iteration's matrix work
    wave_sync();  // the staged rows (and scales) are visible to the whole wave
    if (!scaled) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        v4u f[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) f[h] = fragment(h, c);
        int q = 0;
#pragma unroll
        for (int h1 = 0; h1 < NH; ++h1)
#pragma unroll
          for (int h2 = h1; h2 < NH; ++h2, ++q) {
            const f32x4 d = Mfma<T>::gram(f[h1], f[h2]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[q][r] += (double)d[r];
          }
      }
    } else if constexpr (Mfma<T>::kGuard) {
      // entry (row, col) of sub-block (h1, h2): row operand 16 h1 + 4 grp + r,
      // column operand 16 h2 + op; every fragment scaled by its operand's
      // power of two (exact), the results scaled back exactly in fp64
      int sc[NH], back[NP][4];
#pragma unroll
      for (int h = 0; h < NH; ++h) sc[h] = scale[wave][16 * h + op];
      {
        int q = 0;
#pragma unroll
        for (int h1 = 0; h1 < NH; ++h1)
#pragma unroll
          for (int h2 = h1; h2 < NH; ++h2, ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) back[q][r] = -(scale[wave][16 * h1 + 4 * grp + r] + sc[h2]);
      }
#pragma unroll 1
      for (int c = 0; c < C; ++c) {
        v4u f[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const v4u x = fragment(h, c);
          f[h] = v4u{bf16x2_scale(x.x, sc[h]), bf16x2_scale(x.y, sc[h]), bf16x2_scale(x.z, sc[h]),
                     bf16x2_scale(x.w, sc[h])};
        }
        int q = 0;
#pragma unroll
        for (int h1 = 0; h1 < NH; ++h1)
#pragma unroll
          for (int h2 = h1; h2 < NH; ++h2, ++q) {
            const f32x4 d = Mfma<T>::gram(f[h1], f[h2]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[q][r] += __builtin_amdgcn_ldexp((double)d[r], back[q][r]);
          }
      }
    }
    wave_sync();  // the fragments and scales are read before the next iteration stages its own
  }

  // Sum the four waves' matrices in wave order; write the packed triangle.
  __syncthreads();  // every wave is done with its staging area
  double(*red)[NP][64 * 4] = reinterpret_cast<double(*)[NP][64 * 4]>(&stage[0]);
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][q][lane * 4 + r] = acc[q][r];
  __syncthreads();
  double* out = args.partials + args.poff[j] + (int64_t)tile_id * NE;
  for (int e = threadIdx.x; e < NE; e += kBlock) {
    int i = 0, rem = e;
    while (rem >= NB - i) {
      rem -= NB - i;
      ++i;
    }
    const int k = i + rem;  // entry (i, k), i <= k
    const int q = (i >> 4) == 0 ? (k >> 4) : 2;  // (0,0) -> 0, (0,1) -> 1, (1,1) -> 2
    const int src = ((k & 15) + 16 * ((i & 15) >> 2)) * 4 + (i & 3);
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < kGramWaves; ++w) sum += red[w][q][src];
    out[e] = sum;
  }
}

// ----------------------------------------------------------------- tree walk

// Products and sums rounded separately, never fused, so that terms that
// mirror each other cancel exactly.
__device__ __forceinline__ double mul_rn(double a, double b) { return __dmul_rn(a, b); }
__device__ __forceinline__ double add_rn(double a, double b) { return __dadd_rn(a, b); }

// Packed index of entry (i, k) of a symmetric n x n matrix, either order.
__device__ __forceinline__ int sym_index(int n, int i, int k) { return i <= k ? gram_index(n, i, k) : gram_index(n, k, i); }

constexpr int kTreeWaves = kBlock / 64;
// Per-wave tile sums of blocks of up to 32 operands (528 Gram entries); the
// 2080 entries of a 64-operand block fit the same space.
constexpr int kPartStride = gram_entries(kArgOps);
static_assert(kTreeWaves * kPartStride >= gram_entries(kMaxOps), "a 64-operand Gram matrix fits the wave sums");

// Groups of kTileGroup tiles of the segments of a stage: see
// launch_tile_groups.  One workgroup per window of kTileGroup consecutive
// tiles (and block) forms every group that starts in its window, one after
// another: a window holds one group start of a long segment, or several of
// short ones.  Each thread adds an entry's partials in tile order, all of
// its loads in flight at once.
__global__ __launch_bounds__(kBlock) void tile_group_kernel(TreeArgs a, int ntiles) {
  const BlockDesc d = a.descs[a.desc0 + blockIdx.y];
  const int ne = gram_entries(d.nbt);
  const int w0 = blockIdx.x * kTileGroup, w1 = min(w0 + kTileGroup, ntiles);
  for (int t = w0; t < w1; ++t) {
    const Tile tile = a.tiles[t];
    if (tile.seg_t1 - tile.seg_t0 < 2 || (t - tile.seg_t0) % kTileGroup != 0) continue;  // workgroup-uniform
    const int n = min(tile.seg_t1 - t, kTileGroup);
    // the partials live in the workspace; only the walk reads them as const
    double* p = const_cast<double*>(a.partials) + d.poff + (int64_t)t * ne;
    for (int e = threadIdx.x; e < ne; e += kBlock) {
      double v[kTileGroup];
#pragma unroll
      for (int u = 0; u < kTileGroup; ++u) v[u] = u < n ? p[(int64_t)u * ne + e] : 0.0;
      double sum = 0.0;
#pragma unroll
      for (int u = 0; u < kTileGroup; ++u) sum += v[u];
      p[e] = sum;
    }
  }
}

// The merge walk of block d over segment s.  On entry N holds the block's
// Gram matrix (packed upper triangle, nbt x nbt) and, where exact_g, Nlo its
// double-double low parts (otherwise the walk zeroes Nlo).  Every node of
// the block is a linear combination of its operands, and a merge P = ca L +
// cb R of two current nodes changes the dot products with P linearly:
// P.Y = ca L.Y + cb R.Y for every other current node Y, and
// |P|^2 = ca (ca A + cb d) + cb (ca d + cb B).  So the walk keeps the dot
// products of the current nodes, in double-double, in N itself (node X is
// stored at the index of its first operand): a merge reads A = |L|^2,
// B = |R|^2 and d = L.R directly, and a level's updates take a constant
// number of steps whatever the block size.  Products of the fp64
// coefficients with double-double entries are exact up to the double-double
// rounding, so a node that nearly cancels keeps about 2^-104 of its terms'
// size, and nodes that mirror each other cancel exactly, as the plain
// definition does (rounding is symmetric under negation).
// Returns the block's flags (see TreeArgs) to every thread, and leaves the
// operands' weights, products of the coefficients above them in
// double-double, in w (and rounded, in wf).  Where outputs is set, the
// coefficients, statistics, weights, input norms, orthogonality and flags
// are also written out.  Called by every thread of the workgroup; ms (the
// block's merges, loaded by the caller before a barrier), N, Nlo, w and wf
// are in LDS, and N and Nlo are overwritten.
template <bool kRefine, int MO>
__device__ uint32_t walk_block(const TreeArgs& a, const BlockDesc& d, int s, const Merge* ms, double* N, double* Nlo,
                               bool exact_g, DD* w, double* wf, bool outputs) {
  const int tid = threadIdx.x;
  const int n = d.nbt;
  const int nm = d.nmerges;
  // the updates of one level: at most MO / 2 merges times MO nodes
  constexpr int kPairs = (MO / 2 * MO + kBlock - 1) / kBlock;
  __shared__ double cab[MO][2];  // coefficients of each merge
  // per node (operand index of its first operand): sum_i w_i^2 G_ii over its
  // operands, the scale of its Gram entries' rounding
  __shared__ double S[MO];
  __shared__ double diag[MO];    // the Gram diagonal: the operands' squared norms
  __shared__ int own[MO];        // the last merge that took in operand i
  __shared__ int alive[MO];      // node i is current (not merged into another)
  __shared__ int unsure;         // some coefficient may be off by more than kRefineTol
  __shared__ uint32_t fl;
  // entries already exact (double-double) are not flagged again
  const double gram_err = exact_g ? 0.0 : d.gram_err;
  __syncthreads();  // N (and Nlo) are complete
  if (!exact_g)
    for (int e = tid; e < gram_entries(n); e += kBlock) Nlo[e] = 0.0;
  if (tid < MO) {
    const double g = tid < n ? N[gram_index(n, tid, tid)] : 0.0;
    diag[tid] = g;
    S[tid] = g;
    own[tid] = -1;
    alive[tid] = tid < d.nb;
  }
  if (tid == 0) unsure = 0;
  __syncthreads();
  // Merges are stored children before parents; a level (a batch) ends where
  // a merge overlaps the one before it.  Bit m: merge m starts a batch.
  const int lane = tid & 63;
  const uint64_t starts = __ballot(lane < nm && (lane == 0 || ms[lane].llo < ms[lane - 1].rhi));
  // |root|^2 in double-double: the last merge (the block's root, alone in
  // its level) forms it itself, since no other node is left to update
  __shared__ DD root2;
  DD wi{1.0, 0.0};  // weight of operand tid
  for (int m0 = 0; m0 < nm;) {
    const uint64_t later = starts & ~((uint64_t(2) << m0) - 1u);
    const int m1 = later != 0 ? (int)__builtin_ctzll(later) : nm;
    const bool last = m1 == nm;  // workgroup-uniform
    // the statistics and coefficients, one thread per merge
    if (tid < m1 - m0) {
      const int mi = m0 + tid;
      const Merge mg = ms[mi];
      const int L = mg.llo, R = mg.lhi;
      const int eLL = gram_index(n, L, L), eRR = gram_index(n, R, R), eLR = gram_index(n, L, R);
      const double A = N[eLL], B = N[eRR], dd = N[eLR];  // double-double: hi is the rounded value
      const double ca = (A == 0.0) ? 1.0 : 1.0 - dd / (2.0 * A);
      const double cb = (B == 0.0) ? 1.0 : 1.0 - dd / (2.0 * B);
      cab[mi][0] = ca;
      cab[mi][1] = cb;
      if (last) {
        const DD nA{A, Nlo[eLL]}, nB{B, Nlo[eRR]}, nd{dd, Nlo[eLR]};
        const DD pl = dd_add(dd_scale(nA, ca), dd_scale(nd, cb));  // P.L
        const DD pr = dd_add(dd_scale(nd, ca), dd_scale(nB, cb));  // P.R
        root2 = dd_add(dd_scale(pl, ca), dd_scale(pr, cb));
      }
      const double sl = S[L], sr = S[R];
      if (!kRefine && a.flags != nullptr && gram_err > 0.0) {
        // The rounding errors of separate chunk sums are independent, so a
        // quadratic form over a node errs by about gram_err S (S: the norm
        // the node would have if its operands were orthogonal): S <= A for
        // parallel parts, S ~ A for orthogonal ones, S >> A only under
        // cancellation.  (The worst case, with every error aligned, replaces
        // S by (sum |w_i| sqrt(G_ii))^2, which exceeds A for any orthogonal
        // parts and would flag ordinary data.)  c = 1 - d / (2A) then moves
        // by about (|d err| + |d| |A err| / A) / (2A).  A node whose norm the
        // estimate cannot tell from zero is flagged too.
        // (Compared multiplied out by A^2 and B^2, both positive there.)
        const double eA = gram_err * sl, eB = gram_err * sr, ed = gram_err * sqrt(fmax(sl * sr, 0.0));
        const double tol = gram_err < 1e-10 ? kRefineTol : kRefineTol16;
        bool bad = (sl > 0.0 && A <= eA) || (sr > 0.0 && B <= eB);
        if (A > eA) bad = bad || ed * A + fabs(dd) * eA > 2.0 * tol * fmax(1.0, fabs(ca)) * A * A;
        if (B > eB) bad = bad || ed * B + fabs(dd) * eB > 2.0 * tol * fmax(1.0, fabs(cb)) * B * B;
        if (bad) unsure = 1;
      }
      S[L] = ca * ca * sl + cb * cb * sr;
      alive[R] = 0;
      for (int i = L; i < mg.rhi; ++i) own[i] = mi;
      if (outputs) {
        const int64_t at = (int64_t)mg.node * a.nseg + s;
        a.coeffs[at * 2] = ca;
        a.coeffs[at * 2 + 1] = cb;
        a.stats[at * 3] = dd;
        a.stats[at * 3 + 1] = A;
        a.stats[at * 3 + 2] = B;
      }
    }
    __syncthreads();
    if (last) {
      if (tid < MO) {
        const int o = own[tid];
        if (o >= m0) wi = dd_scale(wi, tid < ms[o].lhi ? cab[o][0] : cab[o][1]);
      }
      break;
    }
    // The merged nodes' dot products, from the entries before this level:
    // pair (m, Y) gives P_m.Y for a current node Y that no merge of the level
    // takes in, and P_m.P_m' for Y = L_m' with m <= m' (P_m'.Y' expanded the
    // same way); a node R_m is gone.
    DD val[kPairs];
    int at[kPairs];
    const int npairs = (m1 - m0) * n;
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
      at[q] = -1;
      const int x = tid + q * kBlock;
      if (x >= npairs) continue;
      const int m = m0 + x / n, Y = x - (x / n) * n;
      // the reads this pair may need, issued together (o < 0: merge 0, unused)
      const int live = alive[Y], o = own[Y];
      const Merge mg = ms[m], mo = ms[max(o, 0)];
      const double ca = cab[m][0], cb = cab[m][1], ca2 = cab[max(o, 0)][0], cb2 = cab[max(o, 0)][1];
      const bool cross = o >= m0;  // Y is L_o of a merge of this level
      if (!live || (cross && o < m)) continue;
      const int L = mg.llo, R = mg.lhi;
      const int Y1 = cross ? mo.llo : Y, Y2 = cross ? mo.lhi : Y;
      const int e1 = sym_index(n, L, Y1), e2 = sym_index(n, R, Y1), e3 = sym_index(n, L, Y2), e4 = sym_index(n, R, Y2);
      const DD n1{N[e1], Nlo[e1]}, n2{N[e2], Nlo[e2]}, n3{N[e3], Nlo[e3]}, n4{N[e4], Nlo[e4]};
      const DD pl = dd_add(dd_scale(n1, ca), dd_scale(n2, cb));  // P_m.Y, or P_m.L_o
      if (cross) {
        const DD pr = dd_add(dd_scale(n3, ca), dd_scale(n4, cb));  // P_m.R_o
        val[q] = dd_add(dd_scale(pl, ca2), dd_scale(pr, cb2));
      } else {
        val[q] = pl;
      }
      at[q] = sym_index(n, L, Y);
    }
    // this thread's operand weight: scaled by the coefficient of its side
    if (tid < MO) {
      const int o = own[tid];
      if (o >= m0) wi = dd_scale(wi, tid < ms[o].lhi ? cab[o][0] : cab[o][1]);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPairs; ++q)
      if (at[q] >= 0) {
        N[at[q]] = val[q].hi;
        Nlo[at[q]] = val[q].lo;
      }
    __syncthreads();
    m0 = m1;
  }
  if (tid < MO) {
    w[tid] = wi;
    wf[tid] = wi.hi;  // normalised: hi is the rounded value
  }
  // The block's result is node 0: its squared norm and its scale S[0].
  if (tid == 0) {
    const double out2 = nm > 0 ? root2.hi : N[0], parts = S[0];
    if (outputs) {
      // sum of |g_k|^2 over the block's input operands, in operand order
      double leaf = 0.0;
      for (int k = 0; k < d.nb; ++k)
        if ((d.leafmask >> k) & 1u) leaf += diag[k];
      a.leafnorm[(int64_t)d.wrow * a.nseg + s] = leaf;
      if (d.root && a.ortho != nullptr) {
        // orthogonality of the segment's gradients: |result|^2 over the sum
        // of their squared norms (lower blocks finished in earlier launches)
        double total = 0.0;
        for (int r = 0; r < a.nblocks_total; ++r)
          total += (r == d.wrow) ? leaf : a.leafnorm[(int64_t)r * a.nseg + s];
        a.ortho[s] = (total == 0.0) ? __builtin_nan("") : out2 / total;
      }
    }
    if (!kRefine) {
      // Bit 1: the block's result is summed in double-double.  Where it is
      // far smaller than its weighted parts, sum_k w_k x_k in fp64 would lose
      // the ratio of the two to rounding, and a later stage could amplify
      // that loss again; every pair flagged for recomputation (bit 0) is
      // summed so too.
      uint32_t f = unsure ? 3u : 0u;
      if (parts > 0.0 && !(out2 > kSumCancel * parts)) f |= 2u;
      fl = f;
      if (outputs && a.flags != nullptr) a.flags[(int64_t)d.wrow * a.nseg + s] = f;
    }
  }
  if (outputs && tid < MO) {
    const int64_t wat = ((int64_t)d.wrow * a.nseg + s) * kMaxOps;
    a.weights[wat + tid] = wi.hi;
    a.weights_lo[wat + tid] = wi.lo;
  }
  __syncthreads();
  return kRefine ? 3u : fl;  // a refined pair is summed in double-double
}

// One workgroup per (block, segment).  The units summed are the segment's
// tiles, or, where the launch formed tile groups (TreeArgs::grouped: always
// for 64-operand blocks, else where some segment has many tiles), its tile
// groups, whose sums sit in each group's first tile.  Blocks of up to 32
// operands: wave q sums the q-th quarter of the units (lanes over Gram
// entries, units in order); the four quarter sums are then added in wave
// order.  64-operand blocks: one thread per entry adds the units in order.
// Either way the split depends only on the shape, so the result is
// reproducible.  The refining walk (kRefine) visits only flagged pairs,
// whose tiles hold double-double entries, and sums them in double-double,
// tile by tile.

// Sums over units u0 .. u1 - 1 (the tiles t0 + u * step) of a lane's Gram
// entries lane, lane + 64, ... (EPL of them; ne entries per tile), each
// entry's units added in order, UB units at a time.  Entries past the last
// are read at the last one (in bounds, no branch), so every load of a step
// is in flight together; they are not stored.
template <int EPL, int UB>
__device__ __forceinline__ void lane_unit_sums(const double* pb, int ne, int lane, int t0, int u0, int u1, int step,
                                               double* out) {
  int idx[EPL];
  double acc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    idx[i] = min(lane + 64 * i, ne - 1);
    acc[i] = 0.0;
  }
  int u = u0;
  for (; u + UB <= u1; u += UB) {
    double v[UB][EPL];
#pragma unroll
    for (int k = 0; k < UB; ++k)
#pragma unroll
      for (int i = 0; i < EPL; ++i) v[k][i] = pb[(int64_t)(t0 + (u + k) * step) * ne + idx[i]];
#pragma unroll
    for (int k = 0; k < UB; ++k)
#pragma unroll
      for (int i = 0; i < EPL; ++i) acc[i] += v[k][i];
  }
  for (; u < u1; ++u) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[i] += pb[(int64_t)(t0 + u * step) * ne + idx[i]];
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + 64 * i < ne) out[lane + 64 * i] = acc[i];
}

// kWide: the launch holds a 64-operand block (its Gram matrix takes 2080
// entries of LDS; the other variant, 528, keeps more workgroups per CU).
template <bool kRefine, bool kWide>
__global__ __launch_bounds__(kBlock) void tree_kernel(TreeArgs a) {
  __shared__ double part[kTreeWaves * kPartStride];
  __shared__ double part_lo[kRefine ? kTreeWaves * kPartStride : 1];
  constexpr int MO = kWide ? kMaxOps : kArgOps;  // operands of the launch's largest block
  __shared__ double G[gram_entries(MO)];
  // operand weights: products of the coefficients of the merges above each
  // operand, in double-double (a chain multiplies up to K - 1 of them, and a
  // node that nearly cancels would amplify their fp64 rounding)
  __shared__ DD w[MO];
  __shared__ double wf[MO];  // the weights rounded to fp64
  __shared__ Merge ms[MO];
  const int item = blockIdx.x;
  const int b = item / a.nseg;
  const int s = item % a.nseg;
  const BlockDesc d = a.descs[a.desc0 + b];
  if (kRefine && (a.flags[(int64_t)d.wrow * a.nseg + s] & 1u) == 0) return;  // workgroup-uniform
  const int n = d.nbt;
  const int ne = gram_entries(n);
  const int tid = threadIdx.x;
  if (tid < d.nmerges) ms[tid] = a.merges[d.merge0 + tid];  // read by the walk, after the barriers below
  const int t0 = a.seg_tile[s], t1 = a.seg_tile[s + 1];
  // The low parts of the Gram entries, where the walk has them: the refining
  // walk's tile sums, or below the exact entries of a single short tile.
  // Entry e of either is written only after every wave sum of entry e is
  // read, by the thread that read them, and above all wave sums' first
  // quarter-stride, so the space can be shared.
  double* const Glo = kRefine ? &part_lo[0] : &part[0];
  // where tile groups were formed (see launch_tile_groups), the first tile
  // of each group holds the group's sum; the refining walk reads the
  // recomputed partials of every tile
  const int step = (a.grouped && !kRefine && t1 - t0 > 1) ? kTileGroup : 1;
  if (kWide && n > kArgOps) {
    if constexpr (kRefine) {
      for (int e = tid; e < ne; e += kBlock) {
        const double* p = a.partials + d.poff + e;
        const double* pl = a.partials_lo + d.poff + e;
        DD sum{0.0, 0.0};
        for (int t = t0; t < t1; ++t) sum = dd_add(sum, DD{p[(int64_t)t * ne], pl[(int64_t)t * ne]});
        G[e] = sum.hi;
        Glo[e] = sum.lo;
      }
    } else {
      // All of this thread's entries (2080 over 256 threads) at once, four
      // units at a time, each entry's units added in order.  Entries past
      // the last are read at the last one (in bounds, no branch), so every
      // load of a step is in flight together; they are not stored.
      constexpr int EPT = (gram_entries(kMaxOps) + kBlock - 1) / kBlock;
      constexpr int UB = 4;
      const double* pb = a.partials + d.poff;
      int idx[EPT];
      double acc[EPT];
#pragma unroll
      for (int i = 0; i < EPT; ++i) {
        idx[i] = min(tid + i * kBlock, ne - 1);
        acc[i] = 0.0;
      }
      int t = t0;
      for (; t + (UB - 1) * step < t1; t += UB * step) {
        double v[UB][EPT];
#pragma unroll
        for (int k = 0; k < UB; ++k)
#pragma unroll
          for (int i = 0; i < EPT; ++i) v[k][i] = pb[(int64_t)(t + k * step) * ne + idx[i]];
#pragma unroll
        for (int k = 0; k < UB; ++k)
#pragma unroll
          for (int i = 0; i < EPT; ++i) acc[i] += v[k][i];
      }
      for (; t < t1; t += step) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) acc[i] += pb[(int64_t)t * ne + idx[i]];
      }
#pragma unroll
      for (int i = 0; i < EPT; ++i)
        if (tid + i * kBlock < ne) G[tid + i * kBlock] = acc[i];
    }
    __syncthreads();
  } else {
    // wave q sums a contiguous share of the segment's tiles (or groups)
    const int q = tid >> 6, lane = tid & 63;
    const int nu = (t1 - t0 + step - 1) / step;
    const int chunk = (nu + kTreeWaves - 1) / kTreeWaves;
    const int u0 = min(nu, q * chunk), u1 = min(nu, u0 + chunk);
    if constexpr (kRefine) {
      for (int e = lane; e < ne; e += 64) {
        const double* p = a.partials + d.poff + e;
        const double* pl = a.partials_lo + d.poff + e;
        DD sum{0.0, 0.0};
        for (int u = u0; u < u1; ++u) {
          const int64_t t = t0 + u;  // step is 1
          sum = dd_add(sum, DD{p[t * ne], pl[t * ne]});
        }
        part[q * kPartStride + e] = sum.hi;
        part_lo[q * kPartStride + e] = sum.lo;
      }
    } else {
      // a lane's entries (1, 3 or 9 of them) together, several units at a time
      const double* pb = a.partials + d.poff;
      double* out = &part[q * kPartStride];
      if (ne <= 64)
        lane_unit_sums<1, 8>(pb, ne, lane, t0, u0, u1, step, out);
      else if (ne <= 192)
        lane_unit_sums<3, 4>(pb, ne, lane, t0, u0, u1, step, out);
      else
        lane_unit_sums<9, 1>(pb, ne, lane, t0, u0, u1, step, out);
    }
    __syncthreads();
    for (int e = tid; e < ne; e += kBlock) {
      if constexpr (kRefine) {
        DD sum{part[e], part_lo[e]};
#pragma unroll
        for (int i = 1; i < kTreeWaves; ++i) sum = dd_add(sum, DD{part[i * kPartStride + e], part_lo[i * kPartStride + e]});
        G[e] = sum.hi;
        Glo[e] = sum.lo;
      } else {
        double sum = part[e];
#pragma unroll
        for (int i = 1; i < kTreeWaves; ++i) sum += part[i * kPartStride + e];
        G[e] = sum;
      }
    }
  }
  // A segment of one short tile of 16-bit inputs has its Gram entries in
  // double-double (hi: that tile's partial, taken exactly above) from the
  // exact short-tile sums; a refined pair has all of them so.  The walk then
  // starts its node dot products from both parts, so their rounding is not
  // amplified by a merge that cancels.  Workgroup-uniform.
  const uint64_t all_inputs = d.nb >= 64 ? ~uint64_t(0) : (uint64_t(1) << d.nb) - 1u;
  const bool exact_g = kRefine || (a.partials_lo != nullptr && t1 - t0 == 1 && a.tiles[t0].len <= kExactRows &&
                                   a.lo_inputs && d.leafmask == all_inputs);
  if (!kRefine && exact_g) {
    __syncthreads();  // every wave sum is consumed
    for (int e = tid; e < ne; e += kBlock) Glo[e] = a.partials_lo[d.poff + (int64_t)t0 * ne + e];
  }
  walk_block<kRefine, MO>(a, d, s, ms, G, Glo, exact_g, w, wf, true);
}

// ----------------------------------------------------------------- weighted sum

// A (block, segment) pair whose walk set bit 1 of its flag: every element's
// sum_k w_k x_k in double-double, with the walk's double-double weights and
// exact products, rounded once.  Operand k is of type TIn, or TN where the
// job's narrow mask marks it; a NULL operand adds nothing.  Up to 32
// operands, every operand's load of an element is issued before the sums (a
// NULL operand reads operand 0; an operand of the other type reads
// kZeroRow), so they are all in flight together; 64 operands (whose kernel
// keeps fewer registers) are read one at a time.  Either way the terms are
// added in operand order.
template <typename TIn, typename TN, int NB, typename TOut, typename WA = WsumArgs>
__device__ void wsum_exact_range(const WA& args, int j, int64_t lo, int64_t hi, const double* w_hi,
                                 const double* w_lo) {
  TOut* __restrict__ y = static_cast<TOut*>(args.y[j]);
  const void* x0 = args.x[j * op_stride(NB)];
  double unused;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kBlock) {
    DD acc{0.0, 0.0};
    if constexpr (NB > kArgOps) {
#pragma unroll 1
      for (int k = 0; k < NB; ++k) {
        const void* x = args.x[j * op_stride(NB) + k];
        if (x == nullptr) continue;
        double v;
        if constexpr (std::is_same<TIn, TN>::value) {
          v = widen_any<TIn>(x, i);
        } else {
          v = ((args.narrow[j] >> k) & 1u) ? widen_any<TN>(x, i) : widen_any<TIn>(x, i);
        }
        acc = dd_add(acc, dd_mul(DD{w_hi[k], w_lo[k]}, DD{v, 0.0}));
      }
    } else {
      double v[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const void* xk = args.x[j * op_stride(NB) + k];
        const void* x = xk != nullptr ? xk : x0;
        if constexpr (std::is_same<TIn, TN>::value) {
          v[k] = widen_any<TIn>(x, i);
        } else {
          const bool nk = (args.narrow[j] >> (xk != nullptr ? k : 0)) & 1u;
          const double a = widen_any<TIn>(nk ? static_cast<const void*>(kZeroRow) : x, nk ? 0 : i);
          const double n = widen_any<TN>(nk ? x : static_cast<const void*>(kZeroRow), nk ? i : 0);
          v[k] = nk ? n : a;
        }
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const DD t = dd_add(acc, dd_mul(DD{w_hi[k], w_lo[k]}, DD{v[k], 0.0}));
        if (args.x[j * op_stride(NB) + k] != nullptr) acc = t;
      }
    }
    Elem<TOut>::store1(y + i, Elem<TOut>::round(acc.hi, &unused));  // normalised: hi is the rounded sum
  }
}

// Operands at or beyond the block's count are NULL in the argument table;
// they alias operand 0 (cache hits, no extra HBM traffic) and their terms are
// masked to zero, so the loop has no branches and every load of a step is in
// flight at once.  First stage: every operand is an input of type TIn; the
// result is the output (TOut = TIn) or an fp64 slot (TOut = double).
// Part `part` of kSplit of a tile: the p-th share of the aligned body; the
// unaligned head goes with part 0 and the tail with the last part.
__device__ __forceinline__ TileSpan tile_part(const Tile& tile, int part, int kSplit) {
  TileSpan sp = span_of(tile);
  const int64_t groups = (sp.body_hi - sp.body_lo) / kGroup;
  const int64_t per = (groups + kSplit - 1) / kSplit * kGroup;
  const int64_t b0 = min(sp.body_lo + part * per, sp.body_hi);
  const int64_t b1 = min(b0 + per, sp.body_hi);
  if (part > 0) sp.lo = b0;
  if (part < kSplit - 1) sp.hi = b1;
  sp.body_lo = b0;
  sp.body_hi = b1;
  return sp;
}

// The weighted sum of job j over the range sp, with weights wrow (and their
// double-double low parts wlo, used where dd is set).  Called by every
// thread of the workgroup.  kPre: pre holds this thread's first group of
// every operand, already loaded.
template <typename TIn, int NB, typename TOut, typename WA = WsumArgs, bool kPre = false>
__device__ __forceinline__ void wsum_tile_range(const WA& args, int j, const TileSpan& sp, const double* wrow,
                                                const double* wlo, bool dd,
                                                const typename Elem<TIn>::Raw8* pre = nullptr) {
  if (dd) {  // workgroup-uniform
    wsum_exact_range<TIn, TIn, NB, TOut, WA>(args, j, sp.lo, sp.hi, wrow, wlo);
    return;
  }
  const TIn* x0 = static_cast<const TIn*>(args.x[j * op_stride(NB)]);
  const TIn* xs[NB];
  bool live[NB];
  double w[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    live[k] = args.x[j * op_stride(NB) + k] != nullptr;
    xs[k] = live[k] ? static_cast<const TIn*>(args.x[j * op_stride(NB) + k]) : x0;
    w[k] = wrow[k];
  }
  TOut* __restrict__ y = static_cast<TOut*>(args.y[j]);
  const int tid = threadIdx.x;
  double unused;

  auto one = [&](int64_t i) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const double t = mul_rn(w[k], (double)Elem<TIn>::load1(xs[k] + i));
      acc = add_rn(acc, live[k] ? t : 0.0);
    }
    Elem<TOut>::store1(y + i, Elem<TOut>::round(acc, &unused));
  };

  if (tid < sp.body_lo - sp.lo) one(sp.lo + tid);
  // Operand-outer: the raw loads of all operands are in flight together,
  // but only one operand is widened at a time; every element still sums
  // its terms in operand order, starting from zero.
  const int64_t g0 = sp.body_lo + (int64_t)tid * kGroup;
  for (int64_t g = g0; g < sp.body_hi; g += (int64_t)kBlock * kGroup) {
    typename Elem<TIn>::Raw8 raw[NB];
    if (kPre && g == g0) {
#pragma unroll
      for (int k = 0; k < NB; ++k) raw[k] = pre[k];
    } else {
#pragma unroll
      for (int k = 0; k < NB; ++k) raw[k] = Elem<TIn>::load_raw8(xs[k] + g);
    }
    double acc[kGroup];
#pragma unroll
    for (int e = 0; e < kGroup; ++e) acc[e] = 0.0;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      float v[kGroup];
      Elem<TIn>::unpack8(raw[k], v);
#pragma unroll
      for (int e = 0; e < kGroup; ++e) {
        const double t = mul_rn(w[k], (double)v[e]);
        acc[e] = add_rn(acc[e], live[k] ? t : 0.0);
      }
    }
    TOut r[kGroup];
#pragma unroll
    for (int e = 0; e < kGroup; ++e) r[e] = Elem<TOut>::round(acc[e], &unused);
    Elem<TOut>::store8(y + g, r);
  }
  if (tid < sp.hi - sp.body_hi) one(sp.body_hi + tid);
}

template <typename TIn, int NB, typename TOut>
__global__ __launch_bounds__(kBlock) void wsum_kernel(WsumArgs args) {
  constexpr int kSplit = wsum_split(sizeof(TIn));
  const int tile_id = blockIdx.x / kSplit;
  const int j = blockIdx.y;
  const Tile tile = args.tiles[tile_id];
  const TileSpan sp = tile_part(tile, blockIdx.x % kSplit, kSplit);
  const int64_t wat = ((int64_t)args.wrow[j] * args.nseg + tile.seg) * kMaxOps;
  wsum_tile_range<TIn, NB, TOut>(args, j, sp, args.weights + wat, args.weights_lo + wat,
                                 (args.flags[(int64_t)args.wrow[j] * args.nseg + tile.seg] & 2u) != 0);
}

// Weighted sum of a 64-operand block (16-bit inputs of type T, one stage, so
// the result is the output).  The four waves of a workgroup take the same
// 512 elements, wave w the operands 16 w .. 16 w + 15, as wsum_kernel takes
// a 16-operand block (eight elements per lane, all sixteen loads in flight,
// terms in operand order from zero); waves 1-3 pass their sums through LDS
// and wave 0 adds them to its own in wave order, rounds once and stores.
// So each element is (((s0 + s1) + s2) + s3), s_w the fp64 sum of wave w's
// sixteen terms.
template <typename T>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void wsum_wide_kernel(WsumArgs args) {
  constexpr int NB = 64;
  constexpr int NG = 16;  // operands per wave
  constexpr int kSplit = wsum_split(sizeof(T));
  constexpr int kStep = 64 * kGroup;  // elements per iteration
  __shared__ double sums[kGramWaves - 1][kStep];
  const int tile_id = blockIdx.x / kSplit;
  const int part = blockIdx.x % kSplit;
  const int j = blockIdx.y;
  const Tile tile = args.tiles[tile_id];
  TileSpan sp = span_of(tile);
  {
    const int64_t groups = (sp.body_hi - sp.body_lo) / kGroup;
    const int64_t per = (groups + kSplit - 1) / kSplit * kGroup;
    const int64_t b0 = min(sp.body_lo + part * per, sp.body_hi);
    const int64_t b1 = min(b0 + per, sp.body_hi);
    if (part > 0) sp.lo = b0;
    if (part < kSplit - 1) sp.hi = b1;
    sp.body_lo = b0;
    sp.body_hi = b1;
  }
  const int64_t wat = ((int64_t)args.wrow[j] * args.nseg + tile.seg) * kMaxOps;
  const double* wrow = args.weights + wat;
  if (args.flags[(int64_t)args.wrow[j] * args.nseg + tile.seg] & 2u) {  // workgroup-uniform
    wsum_exact_range<T, T, NB, T>(args, j, sp.lo, sp.hi, wrow, args.weights_lo + wat);
    return;
  }
  const void* const* table = args.x + j * op_stride(NB);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: pointers and weights in scalars
  const T* x0 = static_cast<const T*>(table[0]);
  const T* xs[NG];
  bool live[NG];
  double w[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int k = NG * wave + i;
    live[i] = table[k] != nullptr;
    xs[i] = live[i] ? static_cast<const T*>(table[k]) : x0;
    w[i] = wrow[k];
  }
  T* __restrict__ y = static_cast<T*>(args.y[j]);
  double unused;

  auto one = [&](int64_t i) {
    double acc = 0.0;
    for (int k = 0; k < NB; ++k) {
      const void* x = table[k];
      if (x != nullptr) acc = add_rn(acc, mul_rn(wrow[k], (double)Elem<T>::load1(static_cast<const T*>(x) + i)));
    }
    Elem<T>::store1(y + i, Elem<T>::round(acc, &unused));
  };

  if (tid < sp.body_lo - sp.lo) one(sp.lo + tid);
  for (int64_t g0 = sp.body_lo; g0 < sp.body_hi; g0 += kStep) {
    // the body is a whole number of groups; lanes past its end read its last
    // group again (so every load is unconditional) and store nothing
    const int64_t gl = g0 + (int64_t)lane * kGroup;
    const bool in = gl < sp.body_hi;
    const int64_t g = in ? gl : sp.body_hi - kGroup;
    typename Elem<T>::Raw8 raw[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) raw[i] = Elem<T>::load_raw8(xs[i] + g);
    double acc[kGroup];
#pragma unroll
    for (int e = 0; e < kGroup; ++e) acc[e] = 0.0;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      float v[kGroup];
      Elem<T>::unpack8(raw[i], v);
#pragma unroll
      for (int e = 0; e < kGroup; ++e) {
        const double t = mul_rn(w[i], (double)v[e]);
        acc[e] = add_rn(acc[e], live[i] ? t : 0.0);
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int e = 0; e < kGroup; ++e) sums[wave - 1][e * 64 + lane] = acc[e];
    }
    __syncthreads();
    if (wave == 0 && in) {
      T r[kGroup];
#pragma unroll
      for (int e = 0; e < kGroup; ++e) {
        double t = acc[e];
#pragma unroll
        for (int q = 0; q < kGramWaves - 1; ++q) t = add_rn(t, sums[q][e * 64 + lane]);
        r[e] = Elem<T>::round(t, &unused);
      }
      Elem<T>::store8(y + g, r);
    }
    __syncthreads();  // the sums are consumed before the next iteration writes its own
  }
  if (tid < sp.hi - sp.body_hi) one(sp.body_hi + tid);
}

// Weighted sum of a stage above the first: operands are fp64 slots or, where
// the job's narrow mask marks them, inputs of type TN carried up; the result
// is an fp64 slot (TOut = double) or the output (TOut = TN).  Each thread
// takes runs of four elements (the body starts at a multiple of kGroup, so
// every fp64 run is 32-byte aligned), loaded with load_whole4.
template <int NB, typename TN, typename TOut>
__global__ __launch_bounds__(kBlock) void wsum_stage_kernel(WsumArgs args) {
  constexpr int kSplit = kWsumSplitMax;
  constexpr int kRun = 4;
  const int tile_id = blockIdx.x / kSplit;
  const int part = blockIdx.x % kSplit;
  const int j = blockIdx.y;
  const Tile tile = args.tiles[tile_id];
  TileSpan sp = span_of(tile);
  {
    const int64_t groups = (sp.body_hi - sp.body_lo) / kGroup;
    const int64_t per = (groups + kSplit - 1) / kSplit * kGroup;
    const int64_t b0 = min(sp.body_lo + part * per, sp.body_hi);
    const int64_t b1 = min(b0 + per, sp.body_hi);
    if (part > 0) sp.lo = b0;
    if (part < kSplit - 1) sp.hi = b1;
    sp.body_lo = b0;
    sp.body_hi = b1;
  }
  const int64_t wat = ((int64_t)args.wrow[j] * args.nseg + tile.seg) * kMaxOps;
  const double* wrow = args.weights + wat;
  if (args.flags[(int64_t)args.wrow[j] * args.nseg + tile.seg] & 2u) {  // workgroup-uniform
    wsum_exact_range<double, TN, NB, TOut>(args, j, sp.lo, sp.hi, wrow, args.weights_lo + wat);
    return;
  }
  const void* xs[NB];
  bool live[NB], nk[NB];
  double w[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    live[k] = args.x[j * op_stride(NB) + k] != nullptr;
    xs[k] = live[k] ? args.x[j * op_stride(NB) + k] : args.x[j * op_stride(NB)];
    nk[k] = (args.narrow[j] >> (live[k] ? k : 0)) & 1u;  // a masked operand reads operand 0, in its type
    w[k] = wrow[k];
  }
  TOut* __restrict__ y = static_cast<TOut*>(args.y[j]);
  const int tid = threadIdx.x;
  double unused;

  auto one = [&](int64_t i) {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const double v = nk[k] ? widen_any<TN>(xs[k], i) : widen_any<double>(xs[k], i);
      acc = add_rn(acc, live[k] ? mul_rn(w[k], v) : 0.0);
    }
    Elem<TOut>::store1(y + i, Elem<TOut>::round(acc, &unused));
  };

  if (tid < sp.body_lo - sp.lo) one(sp.lo + tid);
  for (int64_t g = sp.body_lo + (int64_t)tid * kRun; g < sp.body_hi; g += (int64_t)kBlock * kRun) {
    double v[NB][kRun];
#pragma unroll
    for (int k = 0; k < NB; ++k) load_whole4<TN>(xs[k], nk[k], g, v[k]);
    double acc[kRun] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int k = 0; k < NB; ++k)
#pragma unroll
      for (int e = 0; e < kRun; ++e) acc[e] = add_rn(acc[e], live[k] ? mul_rn(w[k], v[k][e]) : 0.0);
#pragma unroll
    for (int e = 0; e < kRun; ++e) Elem<TOut>::store1(y + g + e, Elem<TOut>::round(acc[e], &unused));
  }
  if (tid < sp.hi - sp.body_hi) one(sp.body_hi + tid);
}

// ----------------------------------------------------------------- small combines: walk and weighted sum in one launch

// The double-double Gram matrix of rows [lo, hi) of the block's operands
// (table; NULL: zero), every entry the row-order sum of exact products, high
// parts into G and low parts into Glo; the rows pass through sh
// (NB rows of kFusedStride doubles: kFusedChunk values and one of padding,
// so that a wave's reads of one row index across operands hit different LDS
// banks).  Called by every thread of the workgroup.
constexpr int kFusedChunk = 64;
constexpr int kFusedStride = kFusedChunk + 1;
constexpr int kFusedRuns = 16;  // runs of tiles whose partials one workgroup sums in parallel

template <typename TIn, int NB>
__device__ void segment_exact_gram(const void* const* table, int64_t lo, int64_t hi, double* G, double* Glo,
                                   double* sh) {
  constexpr int NE = gram_entries(NB);
  constexpr int EPT = (NE + kBlock - 1) / kBlock;  // entries per thread
  int ei[EPT], ek[EPT];
  DD acc[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    const int e = threadIdx.x + q * kBlock;
    int i = 0, rem = e < NE ? e : 0;
    while (rem >= NB - i) {
      rem -= NB - i;
      ++i;
    }
    ei[q] = i;
    ek[q] = i + rem;
    acc[q] = DD{0.0, 0.0};
  }
  for (int64_t c0 = lo; c0 < hi; c0 += kFusedChunk) {
    const int n = (int)min<int64_t>(kFusedChunk, hi - c0);
    if (c0 > lo) __syncthreads();  // the previous chunk is consumed
    for (int idx = threadIdx.x; idx < NB * n; idx += kBlock) {
      const int k = idx / n, r = idx - k * n;
      const void* x = table[k];
      sh[k * kFusedStride + r] = x != nullptr ? widen_any<TIn>(x, c0 + r) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      if (threadIdx.x + q * kBlock >= NE) continue;
      const double* x = sh + ei[q] * kFusedStride;
      const double* y = sh + ek[q] * kFusedStride;
      DD sum = acc[q];
      for (int r = 0; r < n; ++r) sum = dd_add_prod<!std::is_same<TIn, double>::value>(sum, x[r], y[r]);
      acc[q] = sum;
    }
  }
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    if (threadIdx.x + q * kBlock >= NE) continue;
    G[threadIdx.x + q * kBlock] = acc[q].hi;
    Glo[threadIdx.x + q * kBlock] = acc[q].lo;
  }
}

// A one-stage combine whose segments have few tiles, after its Gram pass,
// in one launch instead of four (walk, exact recomputation, second walk,
// weighted sum), one workgroup per tile.  Each workgroup first walks its
// own segment's block on the segment's tile partials, summed in a fixed
// order, so every workgroup of a segment takes the same walk and the same
// weights; the segment's first workgroup writes the tables.  A pair the walk
// flags is recomputed exactly by each of its workgroups over the whole
// segment (rare, and bounded by the plan's limits on these combines) and
// walked again.
template <typename TIn, int NB>
__global__ __launch_bounds__(kBlock) void fused_kernel(TreeArgs ta, WsumArgs1 wa) {
  constexpr int kSplit = kFusedSplit;
  constexpr int MO = kArgOps;
  static_assert(NB <= MO, "blocks of at most 32 operands");
  static_assert(kTreeWaves * kPartStride >= NB * kFusedStride, "the exact rows fit the wave sums");
  __shared__ double part[kTreeWaves * kPartStride];
  __shared__ double G[gram_entries(MO)];
  __shared__ double glo[gram_entries(MO)];
  __shared__ DD w[MO];
  __shared__ double wf[MO];
  __shared__ double wlo[MO];
  __shared__ Merge ms[MO];
  const int tile_id = blockIdx.x / kSplit;
  const int part_id = blockIdx.x % kSplit;
  const Tile tile = wa.tiles[tile_id];
  const int s = tile.seg;
  const BlockDesc d = ta.descs[ta.desc0];
  const int ne = gram_entries(d.nbt);
  const int tid = threadIdx.x;
  const int t0 = tile.seg_t0, t1 = tile.seg_t1;
  if (tid < d.nmerges) ms[tid] = ta.merges[d.merge0 + tid];  // read by the walk, after the barrier below
  // This thread's first group of every operand, loaded now so that the loads
  // overlap the walk (where that takes few registers: up to 32 bytes per
  // element over the operands).  A NULL operand reads operand 0, unused.
  constexpr bool kPre = NB * sizeof(TIn) <= 32;
  typename Elem<TIn>::Raw8 pre[kPre ? NB : 1];
  const TileSpan sp = tile_part(tile, part_id, kSplit);
  if constexpr (kPre) {
    const int64_t g = sp.body_lo + (int64_t)tid * kGroup;
    if (g < sp.body_hi) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const void* x = wa.x[k] != nullptr ? wa.x[k] : wa.x[0];
        pre[k] = Elem<TIn>::load_raw8(static_cast<const TIn*>(x) + g);
      }
    }
  }
  {
    // the tile partials: the segment's tiles cut into Q runs of consecutive
    // tiles (Q = kBlock / ne, at most kFusedRuns, at least 1); thread (q, e)
    // adds run q of entry e in tile order, and the Q run sums of each entry
    // are added in q order
    const int Q = min(kFusedRuns, max(1, kBlock / ne));
    const int run = (t1 - t0 + Q - 1) / Q;
    for (int x = tid; x < Q * ne; x += kBlock) {
      const int q = x / ne, e = x - q * ne;
      const double* p = ta.partials + d.poff + e;
      const int r0 = t0 + q * run, r1 = min(t1, r0 + run);
      double sum = 0.0;
#pragma unroll 8
      for (int t = r0; t < r1; ++t) sum += p[(int64_t)t * ne];
      part[x] = sum;
    }
    __syncthreads();
    for (int e = tid; e < ne; e += kBlock) {
      double sum = part[e];
#pragma unroll 4
      for (int q = 1; q < Q; ++q) sum += part[q * ne + e];
      G[e] = sum;
    }
  }
  const uint64_t all_inputs = (uint64_t(1) << d.nb) - 1u;
  const bool exact_g = ta.partials_lo != nullptr && t1 - t0 == 1 && tile.len <= kExactRows && ta.lo_inputs &&
                       d.leafmask == all_inputs;
  if (exact_g)
    for (int e = tid; e < ne; e += kBlock) glo[e] = ta.partials_lo[d.poff + (int64_t)t0 * ne + e];
  const bool first = tile_id == t0 && part_id == 0;
  uint32_t f = walk_block<false, MO>(ta, d, s, ms, G, glo, exact_g, w, wf, first);
  if (f & 1u) {  // workgroup-uniform
    const Tile last = ta.tiles[t1 - 1];
    segment_exact_gram<TIn, NB>(wa.x, ta.tiles[t0].start, last.start + last.len, G, glo, part);
    __syncthreads();
    f = walk_block<true, MO>(ta, d, s, ms, G, glo, true, w, wf, first);
  }
  if (tid < MO) wlo[tid] = w[tid].lo;
  __syncthreads();
  wsum_tile_range<TIn, NB, TIn, WsumArgs1, kPre>(wa, 0, sp, wf, wlo, (f & 2u) != 0, pre);
}

// ----------------------------------------------------------------- plain sum

template <typename T>
__device__ __forceinline__ void sum_group(const SumArgs& a, int64_t g, int cnt) {
  double acc[kGroup];
  int k0 = 0;
  if (a.acc_in != nullptr) {
#pragma unroll
    for (int e = 0; e < kGroup; ++e) acc[e] = e < cnt ? a.acc_in[g + e] : 0.0;
  } else {  // the sum starts from the first operand itself
    const T* x = static_cast<const T*>(a.x[0]);
    float v[kGroup];
    if (cnt == kGroup) {
      Elem<T>::load8(x + g, v);
    } else {
#pragma unroll
      for (int e = 0; e < kGroup; ++e) v[e] = e < cnt ? Elem<T>::load1(x + g + e) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < kGroup; ++e) acc[e] = (double)v[e];
    k0 = 1;
  }
  for (int k = k0; k < a.nx; ++k) {
    const T* x = static_cast<const T*>(a.x[k]);
    float v[kGroup];
    if (cnt == kGroup) {
      Elem<T>::load8(x + g, v);
    } else {
#pragma unroll
      for (int e = 0; e < kGroup; ++e) v[e] = e < cnt ? Elem<T>::load1(x + g + e) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < kGroup; ++e) acc[e] = add_rn(acc[e], (double)v[e]);
  }
  if (a.acc_out != nullptr) {
#pragma unroll
    for (int e = 0; e < kGroup; ++e)
      if (e < cnt) a.acc_out[g + e] = acc[e];
  } else {
    T* y = static_cast<T*>(a.out);
    double unused;
    if (cnt == kGroup) {
      T r[kGroup];
#pragma unroll
      for (int e = 0; e < kGroup; ++e) r[e] = Elem<T>::round(acc[e], &unused);
      Elem<T>::store8(y + g, r);
    } else {
      for (int e = 0; e < cnt; ++e) Elem<T>::store1(y + g + e, Elem<T>::round(acc[e], &unused));
    }
  }
}

// A whole group of kGroup elements.  The operands go in batches of
// kSumBatch whose loads are all in flight together; an operand index past the
// count loads the batch's first operand again (a cache hit) and its term is
// dropped by a select, not added as zero, so the sum, its operand order and
// the sign of a zero result are those of the serial loop above.
constexpr int kSumBatch = 16;

template <typename T>
__device__ __forceinline__ void sum_full_group(const SumArgs& a, int64_t g) {
  const bool from_acc = a.acc_in != nullptr;
  double acc[kGroup];
#pragma unroll
  for (int e = 0; e < kGroup; ++e) acc[e] = from_acc ? a.acc_in[g + e] : 0.0;
  for (int kb = 0; kb < a.nx; kb += kSumBatch) {
    typename Elem<T>::Raw8 raw[kSumBatch];
#pragma unroll
    for (int i = 0; i < kSumBatch; ++i) {
      const int k = kb + i < a.nx ? kb + i : kb;
      raw[i] = Elem<T>::load_raw8(static_cast<const T*>(a.x[k]) + g);
    }
    // keep the whole batch's loads ahead of its first add (the operand
    // pointers come from runtime-indexed argument loads, and the scheduler
    // would otherwise interleave them with the adds, two operands deep)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kSumBatch; ++i) {
      float v[kGroup];
      Elem<T>::unpack8(raw[i], v);
      const bool live = kb + i < a.nx;
      const bool first = !from_acc && kb + i == 0;  // the sum starts from the first operand itself
#pragma unroll
      for (int e = 0; e < kGroup; ++e) {
        const double s = first ? (double)v[e] : add_rn(acc[e], (double)v[e]);
        acc[e] = live ? s : acc[e];
      }
    }
  }
  if (a.acc_out != nullptr) {
#pragma unroll
    for (int e = 0; e < kGroup; ++e) a.acc_out[g + e] = acc[e];
  } else {
    T r[kGroup];
    double unused;
#pragma unroll
    for (int e = 0; e < kGroup; ++e) r[e] = Elem<T>::round(acc[e], &unused);
    Elem<T>::store8(static_cast<T*>(a.out) + g, r);
  }
}

// Every workgroup takes a contiguous range of groups of kGroup elements that
// holds 16 KB of every operand (the weighted sum's rule; a grid-stride walk
// streamed 3-6 % slower); the last group may be short.
constexpr int64_t kSumSpanBytes = 16384;

template <typename T>
__global__ __launch_bounds__(kBlock) void sum_kernel(SumArgs a) {
  constexpr int64_t kSpan = kSumSpanBytes / (int64_t)sizeof(T) / kGroup;  // groups per workgroup
  const int64_t full = a.n / kGroup;
  const int64_t ngroups = (a.n + kGroup - 1) / kGroup;
  const int64_t q0 = (int64_t)blockIdx.x * kSpan, q1 = min(ngroups, q0 + kSpan);
  for (int64_t q = q0 + threadIdx.x; q < q1; q += kBlock) {
    const int64_t g = q * kGroup;
    if (q < full)
      sum_full_group<T>(a, g);
    else
      sum_group<T>(a, g, (int)(a.n - g));
  }
}

// ----------------------------------------------------------------- dispatch helpers

template <template <typename> class F, typename... Args>
hipError_t by_type(DType t, Args&&... args) {
  switch (t) {
    case DType::F32: return F<float>::run(args...);
    case DType::F16: return F<_Float16>::run(args...);
    case DType::BF16: return F<bf16_t>::run(args...);
    case DType::F64: break;  // not an input dtype
  }
  return hipErrorInvalidValue;
}


template <typename T>
struct RunSum {
  static hipError_t run(const SumArgs& a, hipStream_t st) {
    const int64_t groups = (a.n + kGroup - 1) / kGroup;
    const int64_t span = kSumSpanBytes / (int64_t)sizeof(T) / kGroup;
    const int64_t blocks = (groups + span - 1) / span;
    hipLaunchKernelGGL(sum_kernel<T>, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(kBlock), 0, st, a);
    return hipGetLastError();
  }
};

template <typename GA = GramArgs>
hipError_t run_gram_f64(int nbt, const GA& a, int ntiles, int njobs, hipStream_t st) {
  const dim3 grid(ntiles, njobs);
  // short tiles: at most kMinTile rows, 4 x 16 x (16 / nbt) x U rows per workgroup iteration
  static_assert(kMinTile <= 4 * 16 * 8 * 4 && kMinTile <= 4 * 16 * 4 * 8, "short tiles take one iteration per wave");
  switch (nbt) {
    case 2:
      if (a.short_tiles)
        hipLaunchKernelGGL((gram_f64mfma_kernel<2, 4, GA>), grid, dim3(kBlock), 0, st, a);
      else
        hipLaunchKernelGGL((gram_f64mfma_kernel<2, kF64Unroll, GA>), grid, dim3(kBlock), 0, st, a);
      break;
    case 4:
      if (a.short_tiles)
        hipLaunchKernelGGL((gram_f64mfma_kernel<4, 8, GA>), grid, dim3(kBlock), 0, st, a);
      else
        hipLaunchKernelGGL((gram_f64mfma_kernel<4, kF64Unroll, GA>), grid, dim3(kBlock), 0, st, a);
      break;
    case 8: hipLaunchKernelGGL((gram_f64mfma_kernel<8, kF64Unroll, GA>), grid, dim3(kBlock), 0, st, a); break;
    case 16: hipLaunchKernelGGL((gram_f64mfma_kernel<16, kF64Unroll, GA>), grid, dim3(kBlock), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TN>
struct RunGramStage {
  static hipError_t run(int nbt, const GramArgs& a, int ntiles, int njobs, hipStream_t st) {
    const dim3 grid(ntiles, njobs);
    switch (nbt) {
      case 2: hipLaunchKernelGGL((gram_stage_kernel<2, TN>), grid, dim3(kBlock), 0, st, a); break;
      case 4: hipLaunchKernelGGL((gram_stage_kernel<4, TN>), grid, dim3(kBlock), 0, st, a); break;
      case 8: hipLaunchKernelGGL((gram_stage_kernel<8, TN>), grid, dim3(kBlock), 0, st, a); break;
      case 16: hipLaunchKernelGGL((gram_stage_kernel<16, TN>), grid, dim3(kBlock), 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
};

template <typename T>
struct RunGramMfma {
  template <typename GA = GramArgs>
  static hipError_t run(int nbt, const GA& a, int ntiles, int njobs, hipStream_t st) {
    const dim3 grid(ntiles, njobs);
    switch (nbt) {
      case 2: hipLaunchKernelGGL((gram_mfma_kernel<T, 2, GA>), grid, dim3(kBlock), 0, st, a); break;
      case 4: hipLaunchKernelGGL((gram_mfma_kernel<T, 4, GA>), grid, dim3(kBlock), 0, st, a); break;
      case 8: hipLaunchKernelGGL((gram_mfma_kernel<T, 8, GA>), grid, dim3(kBlock), 0, st, a); break;
      case 16: hipLaunchKernelGGL((gram_tr_kernel<T, 16, GA>), grid, dim3(kBlock), 0, st, a); break;
      case 32: hipLaunchKernelGGL((gram_tr_kernel<T, 32, GA>), grid, dim3(kBlock), 0, st, a); break;
      case 64:
        if constexpr (std::is_same<GA, GramArgs>::value) {  // 64-operand blocks: never a one-job small launch
          hipLaunchKernelGGL((gram_wide_kernel<T>), grid, dim3(kBlock), 0, st, a);
          break;
        }
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
};

template <typename TIn, typename TN>
hipError_t run_gram_exact(int nbt, const GramArgs& a, int ntiles, int njobs, hipStream_t st) {
  const dim3 grid(ntiles, njobs);
  switch (nbt) {
    case 2: hipLaunchKernelGGL((gram_exact_kernel<TIn, TN, 2>), grid, dim3(kBlock), 0, st, a); break;
    case 4: hipLaunchKernelGGL((gram_exact_kernel<TIn, TN, 4>), grid, dim3(kBlock), 0, st, a); break;
    case 8: hipLaunchKernelGGL((gram_exact_kernel<TIn, TN, 8>), grid, dim3(kBlock), 0, st, a); break;
    case 16: hipLaunchKernelGGL((gram_exact_kernel<TIn, TN, 16>), grid, dim3(kBlock), 0, st, a); break;
    case 32:
      if constexpr (sizeof(TIn) == 2) {  // 32-operand blocks exist only over 16-bit inputs
        hipLaunchKernelGGL((gram_exact_kernel<TIn, TN, 32>), grid, dim3(kBlock), 0, st, a);
        break;
      }
      return hipErrorInvalidValue;
    case 64:
      if constexpr (sizeof(TIn) == 2 && std::is_same<TIn, TN>::value) {  // so are 64-operand blocks, one stage
        hipLaunchKernelGGL((gram_exact_kernel<TIn, TN, 64>), grid, dim3(kBlock), 0, st, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t run_wsum(int nbt, const WsumArgs& a, int ntiles, int njobs, hipStream_t st) {
  const dim3 grid((unsigned)ntiles * wsum_split(sizeof(TIn)), njobs);
  switch (nbt) {
    case 2: hipLaunchKernelGGL((wsum_kernel<TIn, 2, TOut>), grid, dim3(kBlock), 0, st, a); break;
    case 4: hipLaunchKernelGGL((wsum_kernel<TIn, 4, TOut>), grid, dim3(kBlock), 0, st, a); break;
    case 8: hipLaunchKernelGGL((wsum_kernel<TIn, 8, TOut>), grid, dim3(kBlock), 0, st, a); break;
    case 16: hipLaunchKernelGGL((wsum_kernel<TIn, 16, TOut>), grid, dim3(kBlock), 0, st, a); break;
    case 32:
      if constexpr (sizeof(TIn) == 2) {  // 32-operand blocks exist only over 16-bit inputs
        hipLaunchKernelGGL((wsum_kernel<TIn, 32, TOut>), grid, dim3(kBlock), 0, st, a);
        break;
      }
      return hipErrorInvalidValue;
    case 64:
      if constexpr (sizeof(TIn) == 2 && std::is_same<TIn, TOut>::value) {  // one stage: the result is the output
        hipLaunchKernelGGL((wsum_wide_kernel<TIn>), grid, dim3(kBlock), 0, st, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// First stage: inputs of type TIn; the result is an fp64 slot or the output.
template <typename TIn>
struct RunWsum {
  static hipError_t run(int nbt, DType out_t, const WsumArgs& a, int ntiles, int njobs, hipStream_t st) {
    if (out_t == DType::F64) return run_wsum<TIn, double>(nbt, a, ntiles, njobs, st);
    return run_wsum<TIn, TIn>(nbt, a, ntiles, njobs, st);
  }
};

template <typename TN, typename TOut>
hipError_t run_wsum_stage(int nbt, const WsumArgs& a, int ntiles, int njobs, hipStream_t st) {
  const dim3 grid((unsigned)ntiles * kWsumSplitMax, njobs);
  switch (nbt) {
    case 2: hipLaunchKernelGGL((wsum_stage_kernel<2, TN, TOut>), grid, dim3(kBlock), 0, st, a); break;
    case 4: hipLaunchKernelGGL((wsum_stage_kernel<4, TN, TOut>), grid, dim3(kBlock), 0, st, a); break;
    case 8: hipLaunchKernelGGL((wsum_stage_kernel<8, TN, TOut>), grid, dim3(kBlock), 0, st, a); break;
    case 16: hipLaunchKernelGGL((wsum_stage_kernel<16, TN, TOut>), grid, dim3(kBlock), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Later stages: fp64 slots and inputs of type TN; the result is an fp64 slot
// or the output.
template <typename TN>
struct RunWsumStage {
  static hipError_t run(int nbt, DType out_t, const WsumArgs& a, int ntiles, int njobs, hipStream_t st) {
    if (out_t == DType::F64) return run_wsum_stage<TN, double>(nbt, a, ntiles, njobs, st);
    return run_wsum_stage<TN, TN>(nbt, a, ntiles, njobs, st);
  }
};

template <typename TN>
struct RunExactStage {
  static hipError_t run(int nbt, const GramArgs& a, int ntiles, int njobs, hipStream_t st) {
    return run_gram_exact<double, TN>(nbt, a, ntiles, njobs, st);
  }
};

template <typename TIn>
struct RunExactFirst {
  static hipError_t run(int nbt, const GramArgs& a, int ntiles, int njobs, hipStream_t st) {
    return run_gram_exact<TIn, TIn>(nbt, a, ntiles, njobs, st);
  }
};

template <typename TIn>
struct RunFused {
  static hipError_t run(int nbt, const TreeArgs& t, const WsumArgs1& w, int ntiles, hipStream_t st) {
    const dim3 grid((unsigned)ntiles * kFusedSplit);
    switch (nbt) {
      case 2: hipLaunchKernelGGL((fused_kernel<TIn, 2>), grid, dim3(kBlock), 0, st, t, w); break;
      case 4: hipLaunchKernelGGL((fused_kernel<TIn, 4>), grid, dim3(kBlock), 0, st, t, w); break;
      case 8: hipLaunchKernelGGL((fused_kernel<TIn, 8>), grid, dim3(kBlock), 0, st, t, w); break;
      case 16: hipLaunchKernelGGL((fused_kernel<TIn, 16>), grid, dim3(kBlock), 0, st, t, w); break;
      case 32:
        if constexpr (sizeof(TIn) == 2) {  // 32-operand blocks exist only over 16-bit inputs
          hipLaunchKernelGGL((fused_kernel<TIn, 32>), grid, dim3(kBlock), 0, st, t, w);
          break;
        }
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
};

}  // namespace

hipError_t launch_gram(DType operand, DType narrow_t, int nbt, const GramArgs& a, int ntiles, int njobs,
                       hipStream_t st) {
  switch (operand) {
    case DType::F64: return by_type<RunGramStage>(narrow_t, nbt, a, ntiles, njobs, st);
    case DType::F32: return run_gram_f64(nbt, a, ntiles, njobs, st);
    case DType::F16: return RunGramMfma<_Float16>::run(nbt, a, ntiles, njobs, st);
    case DType::BF16: return RunGramMfma<bf16_t>::run(nbt, a, ntiles, njobs, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_tree(const TreeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)a.nblocks * a.nseg));
  if (a.refine) {
    if (a.wide)
      hipLaunchKernelGGL((tree_kernel<true, true>), grid, dim3(kBlock), 0, st, a);
    else
      hipLaunchKernelGGL((tree_kernel<true, false>), grid, dim3(kBlock), 0, st, a);
  } else {
    if (a.wide)
      hipLaunchKernelGGL((tree_kernel<false, true>), grid, dim3(kBlock), 0, st, a);
    else
      hipLaunchKernelGGL((tree_kernel<false, false>), grid, dim3(kBlock), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_fused(DType in_t, int nbt, const TreeArgs& t, const WsumArgs1& w, int ntiles, hipStream_t st) {
  return by_type<RunFused>(in_t, nbt, t, w, ntiles, st);
}

hipError_t launch_gram1(DType operand, int nbt, const GramArgs1& a, int ntiles, hipStream_t st) {
  switch (operand) {
    case DType::F32: return run_gram_f64<GramArgs1>(nbt, a, ntiles, 1, st);
    case DType::F16: return RunGramMfma<_Float16>::run<GramArgs1>(nbt, a, ntiles, 1, st);
    case DType::BF16: return RunGramMfma<bf16_t>::run<GramArgs1>(nbt, a, ntiles, 1, st);
    case DType::F64: break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_tile_groups(const TreeArgs& a, int ntiles, hipStream_t st) {
  const unsigned windows = (unsigned)((ntiles + kTileGroup - 1) / kTileGroup);
  hipLaunchKernelGGL(tile_group_kernel, dim3(windows, (unsigned)a.nblocks), dim3(kBlock), 0, st, a, ntiles);
  return hipGetLastError();
}

hipError_t launch_gram_exact(DType operand, DType narrow_t, int nbt, const GramArgs& a, int ntiles, int njobs,
                             hipStream_t st) {
  if (operand == DType::F64) return by_type<RunExactStage>(narrow_t, nbt, a, ntiles, njobs, st);
  return by_type<RunExactFirst>(operand, nbt, a, ntiles, njobs, st);
}

hipError_t launch_wsum(DType in_t, DType narrow_t, int nbt, DType out_t, const WsumArgs& a, int ntiles, int njobs,
                       hipStream_t st) {
  if (in_t == DType::F64) return by_type<RunWsumStage>(narrow_t, nbt, out_t, a, ntiles, njobs, st);
  return by_type<RunWsum>(in_t, nbt, out_t, a, ntiles, njobs, st);
}

hipError_t launch_sum(DType t, const SumArgs& a, hipStream_t st) { return by_type<RunSum>(t, a, st); }

}  // namespace adasum
