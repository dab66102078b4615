// Small device helpers: bfloat16 <-> float, vector element access, reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace matopt {

// Device memory is accessed through address-space-1 (global) pointers so that
// loads and stores compile to global_* instructions: generic (flat) accesses
// would also count against the LDS counter and make every LDS wait also wait
// for outstanding HBM traffic.
#define MATOPT_GAS __attribute__((address_space(1)))
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T gload(const void* p) {
  return *(const MATOPT_GAS T*)p;
}
template <typename T>
__device__ __forceinline__ void gstore(void* p, T v) {
  *(MATOPT_GAS T*)p = v;
}
// Streaming accesses (each byte touched once per kernel): non-temporal, so
// that they do not displace cached data; on this part they also raise the
// sustained bandwidth of the memory-bound kernels (prep 5.3 -> 6.1 TB/s).
template <typename T>
__device__ __forceinline__ T gload_nt(const void* p) {
  return __builtin_nontemporal_load((const MATOPT_GAS T*)p);
}
template <typename T>
__device__ __forceinline__ void gstore_nt(void* p, T v) {
  __builtin_nontemporal_store(v, (MATOPT_GAS T*)p);
}

// bfloat16 is handled as its 16-bit pattern.
__device__ __forceinline__ float bf2f(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// float -> bfloat16, round to nearest even (lowers to v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// float64 -> float32 with round-to-odd: when x is not a float32, take the
// neighbour of x whose last significand bit is 1.  A value rounded to odd with
// p >= q + 2 bits and then rounded to nearest-even with q bits equals the direct
// nearest-even rounding of x (float32 24 bits >= bfloat16 8 bits + 2).
__device__ __forceinline__ float f64_to_f32_odd(double x) {
  float f = (float)x;
  const double back = (double)f;
  if (back != x) {
    uint32_t u = __float_as_uint(f);
    if (!(u & 1u)) u += (fabs(x) > fabs(back)) ? 1u : 0xffffffffu;
    f = __uint_as_float(u);
  }
  return f;
}

// Nearest-even bfloat16 of a float64 value, rounded once.
__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
  return f2bf(f64_to_f32_odd(x));
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return f2bf(lo) | (f2bf(hi) << 16);
}

__device__ __forceinline__ float lo_bf(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float hi_bf(uint32_t d) { return __uint_as_float(d & 0xffff0000u); }

// The weight update W - lr*wd*W + upd*o in float64, before its one rounding to
// storage (decoupled weight decay; wdl = lr*wd).  With wdl == 0 it is exactly
// fma(upd, o, w), so a step without decay is unchanged bit for bit.
__device__ __forceinline__ double w_update(double w, float upd, float o, double wdl) {
  return fma((double)upd, (double)o, wdl != 0.0 ? fma(-wdl, w, w) : w);
}

// bfloat16 of the weight update of a bfloat16 weight w, rounded once: the same
// bits as f64_to_bf16(w_update(w, upd, o, wdl)).  Without decay the float32 fma
// fma(upd, o, w) is the exact value rounded once; rounding that float32 to
// bfloat16 can differ from rounding the exact value only when it lands on a
// bfloat16 midpoint (low 16 bits 0x8000) -- every midpoint is a float32, so
// an exact value strictly between two midpoints rounds to a float32 in the
// same interval -- and there the float64 value decides the side (the
// float32 is moved one unit toward it, as rounding to odd does).  With decay
// the float64 path is used throughout.
__device__ __forceinline__ uint32_t w_update_bf16(float w, float upd, float o, double wdl) {
  if (wdl != 0.0) return f64_to_bf16(w_update(w, upd, o, wdl));
  float s = fmaf(upd, o, w);
  uint32_t u = __float_as_uint(s);
  if ((u & 0xffffu) == 0x8000u) {
    const double x = fma((double)upd, (double)o, (double)w);
    const double sd = (double)s;
    if (x != sd) u += ((x > sd) == (s > 0.f)) ? 1u : 0xffffffffu;
    s = __uint_as_float(u);
  }
  return f2bf(s);
}

// a * b[e] + c[e] for N elements, as float32 values whose nearest-even
// bfloat16 is the exact value rounded once to bfloat16 -- the same bits as
// f64_to_bf16 of the float64 fma, element by element.  The float32 fma is the
// exact value rounded once; rounding that to bfloat16 can differ from rounding
// the exact value only when it lands on a bfloat16 midpoint (low 16 bits
// 0x8000), and there the float64 value decides the side (the float32 is moved
// one unit toward it, as rounding to odd does).  The midpoint test is taken
// for all N first, and one branch -- rarely taken: about once in 65536
// elements -- covers the float64 decision of the whole group, instead of one
// branch per element around it.
template <int N>
__device__ __forceinline__ void fma_bf16_f32_n(float a, const float (&b)[N], const float (&c)[N],
                                               float (&s)[N]) {
  uint32_t z = 0xffffffffu;   // zero iff some element sits on a midpoint
#pragma unroll
  for (int e = 0; e < N; ++e) {
    s[e] = fmaf(a, b[e], c[e]);
    z = min(z, (__float_as_uint(s[e]) ^ 0x8000u) & 0xffffu);
  }
  if (z == 0u) {
#pragma unroll
    for (int e = 0; e < N; ++e) {
      uint32_t u = __float_as_uint(s[e]);
      if ((u & 0xffffu) == 0x8000u) {
        const double x = fma((double)a, (double)b[e], (double)c[e]);
        const double sd = (double)s[e];
        if (x != sd) u += ((x > sd) == (s[e] > 0.f)) ? 1u : 0xffffffffu;
        s[e] = __uint_as_float(u);
      }
    }
  }
}

// The weight update of N bfloat16 weights at once, as float32 values whose
// nearest-even bfloat16 (pack_bf2) is the bits of w_update_bf16 element by
// element: fma_bf16_f32_n without decay; with decay each value is the float64
// update rounded to odd (whose nearest-even bfloat16 is the float64 value
// rounded once), behind one branch on the uniform wdl.
template <int N>
__device__ __forceinline__ void w_update_f32_n(const float (&w)[N], float upd,
                                               const float (&o)[N], double wdl,
                                               float (&s)[N]) {
  if (wdl != 0.0) {
#pragma unroll
    for (int e = 0; e < N; ++e) s[e] = f64_to_f32_odd(w_update(w[e], upd, o[e], wdl));
    return;
  }
  fma_bf16_f32_n<N>(upd, o, w, s);
}

// Element traits: 16-byte vectors hold E elements of T.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int E = 4;
  __device__ static void unpack(const u32x4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static u32x4 pack(const float* f) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]),
                 __float_as_uint(f[2]), __float_as_uint(f[3])};
  }
  // a*b + c rounded once to storage (float32 fma is exact-then-round)
  __device__ static float fma_store(float a, float b, float c) { return fmaf(a, b, c); }
  template <int N>
  __device__ static void fma_store_n(float a, const float (&b)[N], const float (&c)[N],
                                     float (&out)[N]) {
#pragma unroll
    for (int e = 0; e < N; ++e) out[e] = fmaf(a, b[e], c[e]);
  }
  // a float64 value rounded to storage
  __device__ static float round_store(double x) { return (float)x; }
  __device__ static float load1(const void* p, int64_t i) {
    return gload<float>((const float*)p + i);
  }
  __device__ static void store1(void* p, int64_t i, float f) { gstore<float>((float*)p + i, f); }
};
template <> struct Elem<uint16_t> {  // bfloat16
  static constexpr int E = 8;
  __device__ static void unpack(const u32x4& v, float* f) {
    f[0] = lo_bf(v.x); f[1] = hi_bf(v.x); f[2] = lo_bf(v.y); f[3] = hi_bf(v.y);
    f[4] = lo_bf(v.z); f[5] = hi_bf(v.z); f[6] = lo_bf(v.w); f[7] = hi_bf(v.w);
  }
  __device__ static u32x4 pack(const float* f) {
    return u32x4{pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]),
                 pack_bf2(f[4], f[5]), pack_bf2(f[6], f[7])};
  }
  // a*b + c rounded once to bfloat16.  The float64 fma is exact whenever the
  // result fits 53 bits -- always for float32 * bfloat16 + bfloat16 (the
  // momentum); otherwise its own rounding sits 45 bits below bfloat16 precision.
  __device__ static float fma_store(float a, float b, float c) {
    return bf2f(f64_to_bf16(fma((double)a, (double)b, (double)c)));
  }
  // fma_store of N elements (the same values), through fma_bf16_f32_n
  template <int N>
  __device__ static void fma_store_n(float a, const float (&b)[N], const float (&c)[N],
                                     float (&out)[N]) {
    float s[N];
    fma_bf16_f32_n<N>(a, b, c, s);
#pragma unroll
    for (int e = 0; e < N; ++e) out[e] = bf2f(f2bf(s[e]));
  }
  __device__ static float round_store(double x) { return bf2f(f64_to_bf16(x)); }
  __device__ static float load1(const void* p, int64_t i) {
    return bf2f(gload<uint16_t>((const uint16_t*)p + i));
  }
  __device__ static void store1(void* p, int64_t i, float f) {
    gstore<uint16_t>((uint16_t*)p + i, (uint16_t)f2bf(f));
  }
};

// Store n (<= 8) consecutive values of dtype dt at element index i of p.
__device__ __forceinline__ void store_any(void* p, int dt, int64_t i, float f) {
  if (dt == 1) gstore<uint16_t>((uint16_t*)p + i, (uint16_t)f2bf(f));
  else gstore<float>((float*)p + i, f);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace matopt
