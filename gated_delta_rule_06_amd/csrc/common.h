// common.h -- small device helpers shared by the KDA kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Packed sequences up to this count are started longest first.
#define KDA_LPT_MAX 256
// The chunk-parallel prefill schedule is taken for at most this many
// (sequence, head) chains of at least KDA_PAR_MIN_T tokens each (bf16,
// d_k = d_v = 128), while its workspace stays within KDA_PAR_MAX_WS bytes.
#define KDA_PAR_MAX_CHAINS 64
#define KDA_PAR_MIN_T 512
#define KDA_PAR_MAX_WS ((size_t)8 << 30)
// The balanced prefill schedule uses at most this many resident workgroups,
// and a workgroup polls a state hand-over at most KDA_SPLIT_SPIN times (about
// 0.2 us apart; the environment variable KDA_SPLIT_SPIN_POLLS may set fewer)
// before it recomputes the first chunks itself.
#define KDA_SPLIT_MAX_WG 1024
#define KDA_SPLIT_SPIN (1 << 22)

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> one dword holding two bf16 (lo = a, hi = b), round to nearest
// even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Element access for the two I/O types.  IoBf16 stores raw bf16 bit patterns.
struct IoF32 {
  typedef float storage;
  static constexpr bool is_bf16 = false;
  __device__ static __forceinline__ float load(const void* p, size_t i) {
    return reinterpret_cast<const float*>(p)[i];
  }
  // four consecutive elements starting at i (i % 4 == 0)
  __device__ static __forceinline__ f32x4 load4(const void* p, size_t i) {
    return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + i);
  }
  __device__ static __forceinline__ void store(void* p, size_t i, float x) {
    reinterpret_cast<float*>(p)[i] = x;
  }
  __device__ static __forceinline__ void store4(void* p, size_t i, f32x4 x) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p) + i) = x;
  }
  // 16 bytes (four elements) starting at element i
  __device__ static __forceinline__ void store16(void* p, size_t i, u32x4 x) {
    *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(p) + i) = x;
  }
};

struct IoBf16 {
  typedef uint16_t storage;
  static constexpr bool is_bf16 = true;
  __device__ static __forceinline__ float load(const void* p, size_t i) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
  }
  __device__ static __forceinline__ f32x4 load4(const void* p, size_t i) {
    u32x2 w = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(p) + i);
    f32x4 r;
    r[0] = __uint_as_float(w[0] << 16);
    r[1] = __uint_as_float(w[0] & 0xffff0000u);
    r[2] = __uint_as_float(w[1] << 16);
    r[3] = __uint_as_float(w[1] & 0xffff0000u);
    return r;
  }
  __device__ static __forceinline__ void store(void* p, size_t i, float x) {
    reinterpret_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(x);
  }
  __device__ static __forceinline__ void store4(void* p, size_t i, f32x4 x) {
    u32x2 w;
    w[0] = pack_bf16x2(x[0], x[1]);
    w[1] = pack_bf16x2(x[2], x[3]);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p) + i) = w;
  }
  // 16 bytes (eight elements) starting at element i
  __device__ static __forceinline__ void store16(void* p, size_t i, u32x4 x) {
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p) + i) = x;
  }
};

// ---------------------------------------------------------------- lane reductions
// Sum over the 16 lanes of the lane's DPP row (row_ror 8, 4, 2, 1, each fused
// into the add); every lane gets the total.
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, true));
  return x;
}

// ---------------------------------------------------------------- input transforms
// Optional transforms of a token's raw inputs, applied in the kernels before
// the step ("Linear Attention, From Scratch to Kimi 3", sections 6 and 7):
//  PRO_L2NORM:       q, k <- x / sqrt(sum x^2 + PRO_NORM_EPS) per (token, head)
//  PRO_BETA_SIGMOID: beta <- sigmoid(beta)
//  PRO_GATE:         g <- -5 sigmoid(exp(A_log[h]) (g + bias)), bias per key
//                    channel [H, d_k] (per head [H] for Gated DeltaNet), or 0
enum : uint32_t { PRO_L2NORM = 1u, PRO_BETA_SIGMOID = 2u, PRO_GATE = 4u };
constexpr float PRO_NORM_EPS = 1e-6f;

struct Prologue {
  uint32_t flags;
  const float* A_log;
  const float* bias;
};

__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

// log alpha from the raw gate g, the head's exp(A_log) and the channel's bias
__device__ __forceinline__ float gate_logalpha(float g, float ea, float b) {
  return -5.f * sigmoid_f(ea * (g + b));
}

}  // namespace kda
