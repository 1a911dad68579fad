// Device-side helpers shared by the gfx950 kernels of this library: bfloat16
// storage, per-lane fragments of MFMA operands, the MFMA chains over them, and
// sums over the four lane groups of a column.
//
// MFMA operand convention: for a 16x16 output tile D = A (16 x K) * B (K x
// 16), lane l = 16*lg + li (li = l % 16, lg = l / 16) supplies row li of A
// and column li of B for its share of the contraction; both operands use the
// same assignment of contraction indices to (lane group, slot), so any such
// assignment is a valid product. The result leaves D[4*lg + r][li] in
// accumulator r of lane l.
#pragma once

#include "ea_internal.h"

namespace ea {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t bf16_t;  // bfloat16 storage

__device__ __forceinline__ float bf_bits_to_f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
// Two floats to packed bfloat16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <typename T>
struct Num;
template <>
struct Num<float> {
  // ldraw / fromraw: a load whose conversion to float is left for later
  // (kept apart so that the conversion does not wait for the load early)
  static __device__ __forceinline__ uint32_t ldraw(const float* p) { return __float_as_uint(*p); }
  static __device__ __forceinline__ float fromraw(uint32_t r) { return __uint_as_float(r); }
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ float rnd(float v) { return v; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <>
struct Num<bf16_t> {
  static __device__ __forceinline__ uint32_t ldraw(const bf16_t* p) { return *p; }
  static __device__ __forceinline__ float fromraw(uint32_t r) { return bf_bits_to_f(r); }
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf_bits_to_f(*p); }
  static __device__ __forceinline__ float rnd(float v) { return bf_bits_to_f(pack_bf2(v, 0.f) & 0xffffu); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = (bf16_t)(pack_bf2(v, 0.f) & 0xffffu); }
};

// 256 zero bytes in device memory. Lanes whose element does not exist, and
// absent optional parameters, load from here instead of skipping the load: a
// load under a divergent condition makes the compiler wait for it, and for
// every load and store issued before it, right where the branches join,
// which would serialize the small loads of a kernel behind one another.
// Not declared const: it stays in the global address space like the
// parameter vectors, so a select between the two is still a global load.
// Nothing writes it.
__device__ __align__(16) uint32_t kZeros[64] = {};

// Cache-policy operand of the global-to-LDS transfers: the default, or the
// non-temporal (streaming) policy for data read once.
constexpr int kCpolDefault = 0;
constexpr int kCpolStream = 2;

template <typename T>
__device__ __forceinline__ const T* zeros() { return reinterpret_cast<const T*>(kZeros); }

// Address of element k of the optional vector p when ok holds, else of a zero.
template <typename T>
__device__ __forceinline__ const T* elem_or_zero(const void* p, size_t k, bool ok) {
  return (p != nullptr && ok) ? static_cast<const T*>(p) + k : zeros<T>();
}

template <typename T>
__device__ __forceinline__ float ld_or0(const void* p, size_t k) {
  return Num<T>::ld(elem_or_zero<T>(p, k, true));
}

// Q consecutive elements of type T held by one lane, packed in dwords.
template <typename T, int Q>
struct Frag {
  static constexpr int ND = Q * (int)sizeof(T) / 4;
  static_assert(ND == 1 || ND == 2 || ND % 4 == 0, "fragment size");
  uint32_t w[ND];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int k = 0; k < ND; ++k) w[k] = 0u;
  }
  __device__ __forceinline__ void load(const T* p) {
    if constexpr (ND % 4 == 0) {
      const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int s = 0; s < ND / 4; ++s) {
        const u32x4 v = q[s];
        w[4 * s] = v.x; w[4 * s + 1] = v.y; w[4 * s + 2] = v.z; w[4 * s + 3] = v.w;
      }
    } else if constexpr (ND == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p);
      w[0] = v.x; w[1] = v.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
  }
  // The same with the non-temporal (streaming) cache policy: data read once
  // that should not displace the caches' other contents (used for E, whose
  // lines would otherwise push the written E' lines out of the Infinity
  // Cache early).
  __device__ __forceinline__ void load_nt(const T* p) {
    if constexpr (ND % 4 == 0) {
      const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int s = 0; s < ND / 4; ++s) {
        const u32x4 v = __builtin_nontemporal_load(q + s);
        w[4 * s] = v.x; w[4 * s + 1] = v.y; w[4 * s + 2] = v.z; w[4 * s + 3] = v.w;
      }
    } else {
      load(p);
    }
  }
  __device__ __forceinline__ void store(T* p) const {
    if constexpr (ND % 4 == 0) {
      u32x4* q = reinterpret_cast<u32x4*>(p);
#pragma unroll
      for (int s = 0; s < ND / 4; ++s) q[s] = u32x4{w[4 * s], w[4 * s + 1], w[4 * s + 2], w[4 * s + 3]};
    } else if constexpr (ND == 2) {
      *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
    } else {
      *reinterpret_cast<uint32_t*>(p) = w[0];
    }
  }
  __device__ __forceinline__ float get(int k) const {
    if constexpr (sizeof(T) == 4) {
      return __uint_as_float(w[k]);
    } else {
      return (k & 1) ? __uint_as_float(w[k >> 1] & 0xffff0000u) : __uint_as_float(w[k >> 1] << 16);
    }
  }
  // From Q floats; bfloat16 fragments round to nearest even.
  __device__ __forceinline__ void set(const float* v) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int k = 0; k < Q; ++k) w[k] = __float_as_uint(v[k]);
    } else {
#pragma unroll
      for (int k = 0; k < ND; ++k) w[k] = pack_bf2(v[2 * k], v[2 * k + 1]);
    }
  }
};

// acc += A * B over one fragment pair (see the operand convention above).
template <int Q>
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<bf16_t, Q>& a, const Frag<bf16_t, Q>& b) {
  if constexpr (Q % 8 == 0) {
#pragma unroll
    for (int s = 0; s < Q / 8; ++s) {
      const u32x4 av = {a.w[4 * s], a.w[4 * s + 1], a.w[4 * s + 2], a.w[4 * s + 3]};
      const u32x4 bv = {b.w[4 * s], b.w[4 * s + 1], b.w[4 * s + 2], b.w[4 * s + 3]};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                    __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    }
  } else {
    static_assert(Q == 4, "bfloat16 fragments hold 4 or a multiple of 8 values");
    const u32x2 av = {a.w[0], a.w[1]};
    const u32x2 bv = {b.w[0], b.w[1]};
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, av),
                                                   __builtin_bit_cast(i16x4, bv), acc, 0, 0, 0);
  }
  return acc;
}
template <int Q>
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<float, Q>& a, const Frag<float, Q>& b) {
#pragma unroll
  for (int s = 0; s < Q; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w[s]), __uint_as_float(b.w[s]), acc, 0, 0, 0);
  return acc;
}

// Max / sum over the 4 lane groups of a column (lanes li, li+16, li+32,
// li+48); every lane receives the same bits. Swapping a register with itself
// through v_permlane32_swap / v_permlane16_swap yields both halves in each
// lane, so the combine order is identical in all four lanes.
__device__ __forceinline__ float lg_max(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float lg_sum(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Data-parallel-primitive moves within a row of 16 lanes (VALU, no LDS round
// trip): quad_perm [1,0,3,2] (0xB1) and [2,3,0,1] (0x4E), row_half_mirror
// (0x141), row_mirror (0x140).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a row (lanes 16 lg .. 16 lg + 15): pairs, quads,
// halves, then the whole row; every lane receives the same bits.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}
// Sum over all 64 lanes of the wave; every lane receives the same bits.
__device__ __forceinline__ float wave64_sum(float v) { return lg_sum(row16_sum(v)); }

}  // namespace
}  // namespace ea
