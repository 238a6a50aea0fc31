// Device-side building blocks shared by the gfx950 kernels: element types,
// bf16 rounding, MFMA fragments and the two feature maps.
//
// Feature maps ("Simple linear attention language models balance the
// recall-throughput tradeoff", Knowl 3):
//   ELU1    phi(x) = elu(x) + 1 = x + 1 (x > 0), exp(x) (x <= 0).
//   TAYLOR2 phi(x) = [1, x, vec(x (x) x)/sqrt 2], so phi(q).phi(k) =
//           1 + q.k + (q.k)^2 / 2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "shapes.hpp"

namespace linattn {

typedef uint16_t bf16_t;  // bf16 storage: raw bit pattern
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kInvSqrt2 = 0.70710678118654752440f;
constexpr float kSqrt2 = 1.41421356237309504880f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane 4i + j passes the
// address of 4 consecutive 16-bit elements (row i, columns 4j..4j+3 of a
// 4 x 16 block); lane c receives column c of the 4 rows.
__device__ __forceinline__ uint2 lds_read_tr4(const uint16_t* p) {
  typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
  const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Workgroup barrier that orders LDS traffic only.  __syncthreads() would
// also wait for every outstanding global load of the calling wave, which
// would drain the prefetch of the next tile before each barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw buffer resource over [base, base + bytes): loads outside the range
// return zero (hardware range check), so tails need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                           uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                          (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r,
                                               uint32_t byte_offset) {
  return __builtin_bit_cast(
      uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0));
}

__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r,
                                                 uint32_t byte_offset) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, byte_offset, 0, 0);
}

// Lane shift inside a wave through DPP (no LDS round trip): lanes whose
// source is outside the pattern or in a row excluded by ROWS keep `old`
// (or read 0 where the bound-control bit is set).
//   row_shl:n (0x100 + n)  lane i of a 16-lane row reads lane i + n of it
//   row_shr:n (0x110 + n)  lane i of a 16-lane row reads lane i - n of it
//   row_bcast:15 (0x142)   rows 1, 3 read lane 15 of the row before (ROWS 0xa)
//   row_bcast:31 (0x143)   rows 2, 3 read lane 31 (ROWS 0xc)
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_move(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xf, false);
}

template <int CTRL, int ROWS, bool BOUND>
__device__ __forceinline__ float dpp_move_f(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v),
                                                    CTRL, ROWS, 0xf, BOUND));
}

// Sum of lanes i .. i + G - 1 into lane i, for i a multiple of G (G = 1, 2,
// 4, 8 or 16: a group inside one 16-lane row); other lanes hold partial
// sums.  DPP row shifts with out-of-row sources reading 0.
template <int G>
__device__ __forceinline__ float group_sum_to_first(float v) {
  if constexpr (G >= 2) v += dpp_move_f<0x101, 0xf, true>(0.0f, v);
  if constexpr (G >= 4) v += dpp_move_f<0x102, 0xf, true>(0.0f, v);
  if constexpr (G >= 8) v += dpp_move_f<0x104, 0xf, true>(0.0f, v);
  if constexpr (G >= 16) v += dpp_move_f<0x108, 0xf, true>(0.0f, v);
  static_assert(G >= 1 && G <= 16, "a group inside one row");
  return v;
}

// Sum / maximum over the whole wave, returned to every lane: an inclusive
// scan within each row (row_shr 1, 2, 4, 8), the row totals carried through
// lanes 15 and 31 (row_bcast), then lane 63's value.  A lane without a
// source keeps its own value for the maximum and adds 0 for the sum.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move_f<0x111, 0xf, true>(0.0f, v);
  v += dpp_move_f<0x112, 0xf, true>(0.0f, v);
  v += dpp_move_f<0x114, 0xf, true>(0.0f, v);
  v += dpp_move_f<0x118, 0xf, true>(0.0f, v);
  v += dpp_move_f<0x142, 0xa, false>(0.0f, v);
  v += dpp_move_f<0x143, 0xc, false>(0.0f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_move_f<0x111, 0xf, false>(v, v));
  v = fmaxf(v, dpp_move_f<0x112, 0xf, false>(v, v));
  v = fmaxf(v, dpp_move_f<0x114, 0xf, false>(v, v));
  v = fmaxf(v, dpp_move_f<0x118, 0xf, false>(v, v));
  v = fmaxf(v, dpp_move_f<0x142, 0xa, false>(v, v));
  v = fmaxf(v, dpp_move_f<0x143, 0xc, false>(v, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// elu(x) + 1 without a compare: exp(x) >= 1 + x for every x (convexity),
// with equality only at 0, and exp(-|x|) <= 1 < 1 + x for x > 0, so
//   phi(x) = max(1 + x, exp(-|x|))
// picks 1 + x for x > 0 and exp(x) for x <= 0.  One multiply, one v_exp_f32
// (2^t, the |.| and minus are free operand modifiers), one add, one max.
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float phi_elu1(float x) {
  return fmaxf(x + 1.0f, __builtin_amdgcn_exp2f(-fabsf(x * kLog2e)));
}

// 1 / x in one v_rcp_f32 (1 ulp): normalisers only.
__device__ __forceinline__ float fast_rcp(float x) {
  return __builtin_amdgcn_rcpf(x);
}

// ---------------------------------------------------------------------------
// Element traits: T is the storage type of q, k, v, y (float or bf16_t).
// A "fragment" is one lane's 8-element share of an MFMA operand: for
// v_mfma_f32_16x16x32_bf16 the 64 lanes hold a 16 x 32 operand, lane l
// owning row (l % 16) and eight K slots of lane group (l / 16).  The float32
// path emulates the same 16x16x32 step with eight v_mfma_f32_16x16x4_f32.
// Which logical K index a (lane group, slot) pair stands for is up to the
// caller; the product is correct whenever A and B use the same assignment.
// ---------------------------------------------------------------------------
template <typename T> struct Elem;

template <> struct Elem<bf16_t> {
  typedef bf16x8_t frag;
  static constexpr int kPer16B = 8;  // elements per 16-byte vector
  __device__ static __forceinline__ float to_f32(bf16_t x) {
    return bf16_to_f32(x);
  }
  __device__ static __forceinline__ bf16_t from_f32(float x) {
    return f32_to_bf16(x);
  }
  __device__ static __forceinline__ frag make(const float (&v)[8]) {
    const uint4 u = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                               pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    return __builtin_bit_cast(frag, u);
  }
  __device__ static __forceinline__ frag zero() {
    return __builtin_bit_cast(frag, make_uint4(0u, 0u, 0u, 0u));
  }
  // 8 consecutive elements, 16-byte aligned (LDS or global).
  __device__ static __forceinline__ frag load8(const bf16_t* p) {
    return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(p));
  }
  __device__ static __forceinline__ void load8f(const bf16_t* p, float (&v)[8]) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static __forceinline__ void mma(f32x4_t& acc, const frag& a,
                                             const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
};

template <> struct Elem<float> {
  typedef f32x8_t frag;
  static constexpr int kPer16B = 4;
  __device__ static __forceinline__ float to_f32(float x) { return x; }
  __device__ static __forceinline__ float from_f32(float x) { return x; }
  __device__ static __forceinline__ frag make(const float (&v)[8]) {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = v[i];
    return f;
  }
  __device__ static __forceinline__ frag zero() {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = 0.0f;
    return f;
  }
  __device__ static __forceinline__ frag load8(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    frag f;
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    return f;
  }
  __device__ static __forceinline__ void load8f(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ static __forceinline__ void mma(f32x4_t& acc, const frag& a,
                                             const frag& b) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
  }
};

// Unpack one 16-byte vector of stored elements into floats.
template <typename T>
__device__ __forceinline__ void unpack16(const uint4& u,
                                         float (&v)[Elem<T>::kPer16B]);

template <>
__device__ __forceinline__ void unpack16<bf16_t>(const uint4& u,
                                                 float (&v)[8]) {
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void unpack16<float>(const uint4& u,
                                                float (&v)[4]) {
  v[0] = __uint_as_float(u.x);
  v[1] = __uint_as_float(u.y);
  v[2] = __uint_as_float(u.z);
  v[3] = __uint_as_float(u.w);
}

// Pack floats into one 16-byte vector of stored elements.
template <typename T>
__device__ __forceinline__ uint4 pack16(const float (&v)[Elem<T>::kPer16B]);

template <>
__device__ __forceinline__ uint4 pack16<bf16_t>(const float (&v)[8]) {
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                    pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

template <>
__device__ __forceinline__ uint4 pack16<float>(const float (&v)[4]) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]),
                    __float_as_uint(v[2]), __float_as_uint(v[3]));
}

// Two consecutive elements (a token pair of one transposed row) in one
// LDS store: 4 bytes for bf16, 8 bytes for float.
__device__ __forceinline__ void store_pair(bf16_t* p, float a, float b) {
  *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
}

__device__ __forceinline__ void store_pair(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}

}  // namespace linattn
