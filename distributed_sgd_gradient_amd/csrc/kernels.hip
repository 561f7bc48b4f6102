// kernels.hip - gfx950 kernels of the level-by-level Adasum combine.
//
// Every kernel walks tiles of the plan's tile table.  A tile lies inside one
// segment; its body starts at a multiple of kGroup elements, so each thread
// moves kGroup elements per step with 16-byte loads and stores (base pointers
// are 16-byte aligned), and the unaligned head of a segment's first tile and
// the ragged tail of its last tile are done one element per thread.
//
// Arithmetic (the pairwise operator of "Scaling Distributed Training with
// Adaptive Summation", whose dot product and norms must be complete before
// the pair is combined, Sec. 4):
//   * statistics a.b, |a|^2, |b|^2 accumulate in fp64 per thread, then a
//     fixed xor-butterfly over the wave64 and a fixed-order sum of the four
//     waves give one partial per tile; the finalize kernel sums the tiles of a
//     segment in a fixed order, so results are bitwise reproducible without
//     atomics;
//   * coefficients ca = 1 - d/(2A), cb = 1 - d/(2B) in fp64 with IEEE
//     division; a zero-norm operand (A == 0 exactly) gets coefficient 1;
//   * the combine evaluates fma(ca, a, cb*b) in fp64 and rounds once, to fp32
//     for an intermediate level or to the output dtype at the root; the
//     statistics it emits for the next level are taken from the rounded
//     values it stores.
#include <hip/hip_runtime.h>

#include <cstdint>

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

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ void load8(const float* p, float (&v)[kGroup]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
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
  static __device__ __forceinline__ float load1(const _Float16* p) { return (float)*p; }
  static __device__ __forceinline__ void load8(const _Float16* p, float (&v)[kGroup]) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
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
  static __device__ __forceinline__ float load1(const bf16_t* p) { return widen(p->bits); }
  static __device__ __forceinline__ void load8(const bf16_t* p, float (&v)[kGroup]) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
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

// ----------------------------------------------------------------- reductions

// xor butterfly: partners add the same two values, so every lane ends with
// the identical, order-fixed sum
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum three fp64 values over the block; the result is valid in thread 0.
__device__ __forceinline__ void block_sum3(double& a, double& b, double& c) {
  __shared__ double red[kBlock / 64][3];
  a = wave_sum(a);
  b = wave_sum(b);
  c = wave_sum(c);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    red[w][0] = a;
    red[w][1] = b;
    red[w][2] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a = red[0][0];
    b = red[0][1];
    c = red[0][2];
#pragma unroll
    for (int i = 1; i < kBlock / 64; ++i) {
      a += red[i][0];
      b += red[i][1];
      c += red[i][2];
    }
  }
}

__device__ __forceinline__ void add_stats(double x, double y, double& d, double& A, double& B) {
  d = fma(x, y, d);
  A = fma(x, x, A);
  B = fma(y, y, B);
}

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

// ----------------------------------------------------------------- triple dot

template <typename T>
__global__ __launch_bounds__(kBlock) void triple_dot_kernel(DotArgs args) {
  const int tile_id = blockIdx.x;
  const int j = blockIdx.y;
  const TileSpan sp = span_of(args.tiles[tile_id]);
  const T* __restrict__ a = static_cast<const T*>(args.a[j]);
  const T* __restrict__ b = static_cast<const T*>(args.b[j]);
  const int tid = threadIdx.x;
  double d = 0.0, A = 0.0, B = 0.0;
  if (tid < sp.body_lo - sp.lo) {
    const int64_t i = sp.lo + tid;
    add_stats(Elem<T>::load1(a + i), Elem<T>::load1(b + i), d, A, B);
  }
  for (int64_t g = sp.body_lo + (int64_t)tid * kGroup; g < sp.body_hi; g += (int64_t)kBlock * kGroup) {
    float x[kGroup], y[kGroup];
    Elem<T>::load8(a + g, x);
    Elem<T>::load8(b + g, y);
#pragma unroll
    for (int e = 0; e < kGroup; ++e) add_stats(x[e], y[e], d, A, B);
  }
  if (tid < sp.hi - sp.body_hi) {
    const int64_t i = sp.body_hi + tid;
    add_stats(Elem<T>::load1(a + i), Elem<T>::load1(b + i), d, A, B);
  }
  block_sum3(d, A, B);
  if (tid == 0) {
    double* out = args.partials + ((int64_t)args.row[j] * args.ntiles + tile_id) * 3;
    out[0] = d;
    out[1] = A;
    out[2] = B;
  }
}

// ----------------------------------------------------------------- finalize

constexpr int kFinalizeItemsPerBlock = kBlock / 64;  // one wave per (pair, segment)

__global__ __launch_bounds__(kBlock) void finalize_kernel(FinalizeArgs args) {
  const int64_t item = (int64_t)blockIdx.x * kFinalizeItemsPerBlock + (threadIdx.x >> 6);
  if (item >= (int64_t)args.npairs * args.nseg) return;  // uniform per wave; no block barrier below
  const int p = (int)(item / args.nseg);
  const int s = (int)(item % args.nseg);
  const int lane = threadIdx.x & 63;
  const double* row = args.partials + (int64_t)p * args.ntiles * 3;
  double d = 0.0, A = 0.0, B = 0.0;
  for (int t = args.seg_tile[s] + lane; t < args.seg_tile[s + 1]; t += 64) {
    d += row[(int64_t)t * 3];
    A += row[(int64_t)t * 3 + 1];
    B += row[(int64_t)t * 3 + 2];
  }
  d = wave_sum(d);
  A = wave_sum(A);
  B = wave_sum(B);
  if (lane == 0) {
    const double ca = (A == 0.0) ? 1.0 : 1.0 - d / (2.0 * A);
    const double cb = (B == 0.0) ? 1.0 : 1.0 - d / (2.0 * B);
    const int64_t at = (int64_t)(args.first_node + p) * args.nseg + s;
    args.coeffs[at * 2] = ca;
    args.coeffs[at * 2 + 1] = cb;
    args.stats[at * 3] = d;
    args.stats[at * 3 + 1] = A;
    args.stats[at * 3 + 2] = B;
  }
}

// ----------------------------------------------------------------- combine

template <typename TIn, typename TOut, bool SIB>
__global__ __launch_bounds__(kBlock) void combine_kernel(CombineArgs args) {
  const int tile_id = blockIdx.x;
  const int j = blockIdx.y;
  const Tile tile = args.tiles[tile_id];
  const TileSpan sp = span_of(tile);
  const int64_t c0 = ((int64_t)args.node[j][0] * args.nseg + tile.seg) * 2;
  const double ca0 = args.coeffs[c0], cb0 = args.coeffs[c0 + 1];
  double ca1 = 0.0, cb1 = 0.0;
  if (SIB) {
    const int64_t c1 = ((int64_t)args.node[j][1] * args.nseg + tile.seg) * 2;
    ca1 = args.coeffs[c1];
    cb1 = args.coeffs[c1 + 1];
  }
  const TIn* __restrict__ x0 = static_cast<const TIn*>(args.x[j][0]);
  const TIn* __restrict__ x1 = static_cast<const TIn*>(args.x[j][1]);
  const TIn* __restrict__ x2 = static_cast<const TIn*>(args.x[j][2]);
  const TIn* __restrict__ x3 = static_cast<const TIn*>(args.x[j][3]);
  TOut* __restrict__ y0 = static_cast<TOut*>(args.y[j][0]);
  TOut* __restrict__ y1 = static_cast<TOut*>(args.y[j][1]);
  const int tid = threadIdx.x;
  double d = 0.0, A = 0.0, B = 0.0;

  auto one = [&](int64_t i) {
    double p;
    Elem<TOut>::store1(y0 + i, Elem<TOut>::round(fma(ca0, (double)Elem<TIn>::load1(x0 + i),
                                                     cb0 * (double)Elem<TIn>::load1(x1 + i)), &p));
    if (SIB) {
      double q;
      Elem<TOut>::store1(y1 + i, Elem<TOut>::round(fma(ca1, (double)Elem<TIn>::load1(x2 + i),
                                                       cb1 * (double)Elem<TIn>::load1(x3 + i)), &q));
      add_stats(p, q, d, A, B);
    }
  };

  if (tid < sp.body_lo - sp.lo) one(sp.lo + tid);
  for (int64_t g = sp.body_lo + (int64_t)tid * kGroup; g < sp.body_hi; g += (int64_t)kBlock * kGroup) {
    float a0[kGroup], a1[kGroup];
    Elem<TIn>::load8(x0 + g, a0);
    Elem<TIn>::load8(x1 + g, a1);
    TOut r0[kGroup];
    double p[kGroup];
#pragma unroll
    for (int e = 0; e < kGroup; ++e) r0[e] = Elem<TOut>::round(fma(ca0, (double)a0[e], cb0 * (double)a1[e]), &p[e]);
    Elem<TOut>::store8(y0 + g, r0);
    if (SIB) {
      float a2[kGroup], a3[kGroup];
      Elem<TIn>::load8(x2 + g, a2);
      Elem<TIn>::load8(x3 + g, a3);
      TOut r1[kGroup];
#pragma unroll
      for (int e = 0; e < kGroup; ++e) {
        double q;
        r1[e] = Elem<TOut>::round(fma(ca1, (double)a2[e], cb1 * (double)a3[e]), &q);
        add_stats(p[e], q, d, A, B);
      }
      Elem<TOut>::store8(y1 + g, r1);
    }
  }
  if (tid < sp.hi - sp.body_hi) one(sp.body_hi + tid);

  if (SIB) {
    block_sum3(d, A, B);
    if (tid == 0) {
      double* out = args.partials + ((int64_t)args.emit[j] * args.ntiles + tile_id) * 3;
      out[0] = d;
      out[1] = A;
      out[2] = B;
    }
  }
}

// ----------------------------------------------------------------- widen

template <typename T>
__global__ __launch_bounds__(kBlock) void widen_kernel(WidenArgs args) {
  const TileSpan sp = span_of(args.tiles[blockIdx.x]);
  const T* __restrict__ src = static_cast<const T*>(args.src);
  float* __restrict__ dst = args.dst;
  const int tid = threadIdx.x;
  if (tid < sp.body_lo - sp.lo) dst[sp.lo + tid] = Elem<T>::load1(src + sp.lo + tid);
  for (int64_t g = sp.body_lo + (int64_t)tid * kGroup; g < sp.body_hi; g += (int64_t)kBlock * kGroup) {
    float v[kGroup];
    Elem<T>::load8(src + g, v);
    Elem<float>::store8(dst + g, v);
  }
  if (tid < sp.hi - sp.body_hi) dst[sp.body_hi + tid] = Elem<T>::load1(src + sp.body_hi + tid);
}

// ----------------------------------------------------------------- dispatch helpers

template <template <typename> class F, typename... Args>
hipError_t by_type(DType t, Args&&... args) {
  switch (t) {
    case DType::F32: return F<float>::run(args...);
    case DType::F16: return F<_Float16>::run(args...);
    case DType::BF16: return F<bf16_t>::run(args...);
  }
  return hipErrorInvalidValue;
}

template <typename T>
struct RunDot {
  static hipError_t run(const DotArgs& a, int npairs, hipStream_t st) {
    hipLaunchKernelGGL(triple_dot_kernel<T>, dim3(a.ntiles, npairs), dim3(kBlock), 0, st, a);
    return hipGetLastError();
  }
};

template <typename T>
struct RunWiden {
  static hipError_t run(const WidenArgs& a, int ntiles, hipStream_t st) {
    hipLaunchKernelGGL(widen_kernel<T>, dim3(ntiles), dim3(kBlock), 0, st, a);
    return hipGetLastError();
  }
};

template <typename TIn, typename TOut>
hipError_t run_combine(bool siblings, const CombineArgs& a, int njobs, hipStream_t st) {
  const dim3 grid(a.ntiles, njobs);
  if (siblings)
    hipLaunchKernelGGL((combine_kernel<TIn, TOut, true>), grid, dim3(kBlock), 0, st, a);
  else
    hipLaunchKernelGGL((combine_kernel<TIn, TOut, false>), grid, dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

template <typename TIn>
struct RunCombineIn {
  static hipError_t run(DType out_t, bool siblings, const CombineArgs& a, int njobs, hipStream_t st) {
    switch (out_t) {
      case DType::F32: return run_combine<TIn, float>(siblings, a, njobs, st);
      case DType::F16: return run_combine<TIn, _Float16>(siblings, a, njobs, st);
      case DType::BF16: return run_combine<TIn, bf16_t>(siblings, a, njobs, st);
    }
    return hipErrorInvalidValue;
  }
};

}  // namespace

hipError_t launch_triple_dot(DType operand, const DotArgs& a, int npairs, hipStream_t st) {
  return by_type<RunDot>(operand, a, npairs, st);
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t st) {
  const int64_t items = (int64_t)a.npairs * a.nseg;
  const int64_t blocks = (items + kFinalizeItemsPerBlock - 1) / kFinalizeItemsPerBlock;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_combine(DType in_t, DType out_t, bool siblings, const CombineArgs& a, int njobs,
                          hipStream_t st) {
  return by_type<RunCombineIn>(in_t, out_t, siblings, a, njobs, st);
}

hipError_t launch_widen(DType src_t, const WidenArgs& a, int ntiles, hipStream_t st) {
  return by_type<RunWiden>(src_t, a, ntiles, st);
}

}  // namespace adasum
