// Device-side helpers shared by the libgdn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t bf16;  // bfloat16 stored as its 16 raw bits

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(bf16 h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16>(u >> 16);
}

// ------------------------------------------------------------------ gates

// The gates of one (token, value head) from its raw inputs (pymllm
// `gdn_extend_chunkwise` parameters; formulas of the regolith `gdn.metal`
// header comment): xa = a + dt_bias[h], g = -exp(A_log[h]) softplus(xa)
// (log-space) and beta = sigmoid(b).  softplus(x) is evaluated as
// max(x, 0) + log1p(exp(-|x|)), the same function with no overflow and no
// threshold.  Every kernel that forms gates calls this, so they agree bit
// for bit.
__device__ __forceinline__ void gates_of(float xa, float A_log, float braw, float& g, float& beta) {
  g = -expf(A_log) * (fmaxf(xa, 0.0f) + log1pf(expf(-fabsf(xa))));
  beta = 1.0f / (1.0f + expf(-braw));
}

// sigmoid and SiLU on the hardware exponential and reciprocal (v_exp_f32,
// v_rcp_f32; a few ulp), for the elementwise layer kernels, which are
// otherwise bound by the instruction sequences of an exact exp and an IEEE
// division.  Saturates correctly: a large -x gives exp = inf and a
// reciprocal of 0.  The conv prologue of the prefill calls these wherever it
// runs, so its outputs agree bit for bit.
__device__ __forceinline__ float sigmoid_fast(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float silu_fast(float x) { return x * sigmoid_fast(x); }

// ---------------------------------------------------- activation loads/stores

template <typename T> struct Act;

template <> struct Act<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float x) { *p = x; }
  // four consecutive elements (16-byte aligned)
  static __device__ __forceinline__ f32x4 load4(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
  }
  static __device__ __forceinline__ void store4(float* p, f32x4 x) {
    *reinterpret_cast<f32x4*>(p) = x;
  }
};

template <> struct Act<bf16> {
  static __device__ __forceinline__ float load(const bf16* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16* p, float x) { *p = f32_to_bf16(x); }
  // four consecutive elements (8-byte aligned)
  static __device__ __forceinline__ f32x4 load4(const bf16* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    f32x4 r;
    r.x = __uint_as_float(w.x << 16);
    r.y = __uint_as_float(w.x & 0xffff0000u);
    r.z = __uint_as_float(w.y << 16);
    r.w = __uint_as_float(w.y & 0xffff0000u);
    return r;
  }
  static __device__ __forceinline__ void store4(bf16* p, f32x4 x) {
    uint2 w;
    w.x = static_cast<uint32_t>(f32_to_bf16(x.x)) | (static_cast<uint32_t>(f32_to_bf16(x.y)) << 16);
    w.y = static_cast<uint32_t>(f32_to_bf16(x.z)) | (static_cast<uint32_t>(f32_to_bf16(x.w)) << 16);
    *reinterpret_cast<uint2*>(p) = w;
  }
};

// One activation element as stored, converted to fp32 on use.
__device__ __forceinline__ float to_f32(bf16 h) { return bf16_to_f32(h); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// Four consecutive activations as stored (one 8- or 16-byte load), converted
// on use: keeping a load's result unconverted lets later loads issue before
// the compiler's wait for it.
template <typename T> struct Raw4;
template <> struct Raw4<bf16> {
  uint2 w;
  __device__ __forceinline__ void load(const bf16* p) { w = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ f32x4 f() const {
    return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
  }
};
template <> struct Raw4<float> {
  f32x4 w;
  __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ f32x4 f() const { return w; }
};

// Lanes given to one row of n float4 columns: n rounded up to a power of two
// (a lane group of group_sum).  Head sizes that are multiples of 32 but not
// powers of two (96, 160, 192, 224) leave the lanes past n idle.
constexpr int row_lanes(int n) { return n <= 8 ? 8 : n <= 16 ? 16 : n <= 32 ? 32 : 64; }

// ------------------------------------------------------- streaming state I/O

__device__ __forceinline__ f32x4 load_stream(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void store_stream(float* p, f32x4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) {
  return (a.x * b.x + a.y * b.y) + (a.z * b.z + a.w * b.w);
}

// ------------------------------------------------------ lane-group reductions
//
// group_sum<W>(x): sum of x over each aligned group of W consecutive lanes
// (W in {1, 2, 4, 8, 16, 32, 64}); every lane of the group receives the sum.
// Steps inside a 16-lane DPP row use DPP lane permutations (quad_perm,
// row_half_mirror, row_mirror); the steps across rows use ds_swizzle /
// ds_bpermute.  All groups of the wave reduce in the same order, so equal
// inputs give bitwise equal sums on every lane.

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "W");
  if constexpr (W >= 2) x += dpp<0xb1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (W >= 4) x += dpp<0x4e>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (W >= 8) x += dpp<0x141>(x);  // row_half_mirror: other quad of the 8
  if constexpr (W >= 16) x += dpp<0x140>(x); // row_mirror: other half of the row
  if constexpr (W >= 32) {
    // lane ^ 16 inside each 32-lane half: ds_swizzle bit mode, and 0x1f, xor 0x10
    x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401f));
  }
  if constexpr (W >= 64) x += __shfl_xor(x, 32);
  return x;
}

}  // namespace gdn
