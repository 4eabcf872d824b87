// Shared device-side definitions for the gfx950 kernels: element types, 16-byte fragments, the
// MFMA 32x32 tile product for fp32 and bf16, wave reductions and small vector helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

#define DEV __device__ __forceinline__

// ---------------------------------------------------------------------------------------------
// Element conversions. fp32 -> bf16 rounds to nearest even (the hardware conversion).
// ---------------------------------------------------------------------------------------------
DEV float to_f32(float x) { return x; }
DEV float to_f32(bf16 x) { return (float)x; }
template <typename T> DEV T from_f32(float x);
template <> DEV float from_f32<float>(float x) { return x; }
template <> DEV bf16 from_f32<bf16>(float x) { return (bf16)x; }

DEV uint32_t bf16_bits(bf16 x) { return (uint32_t)__builtin_bit_cast(uint16_t, x); }
DEV float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
DEV float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
// Two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32, lo in bits 0..15.
DEV uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// 2^x with the bare v_exp_f32 (about 1 ulp, as exp2f). exp2f adds a range check and rescaling
// around it so that results below 2^-126 stay exact denormals; softmax and cross-entropy do not
// need those (they add nothing to a sum dominated by the maximum term), so the hot loops skip it.
DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------------------------
// Elements per 16-byte vector, and unpack/pack of one 16-byte vector into floats.
// ---------------------------------------------------------------------------------------------
template <typename T> struct Vec;
template <> struct Vec<float> {
  static constexpr int N = 4;
  DEV static void unpack(const u32x4& v, float* f) {
    // whole-vector cast: a bit-cast of one ext-vector element is miscompiled (reads element 0)
    const f32x4 t = __builtin_bit_cast(f32x4, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = t[i];
  }
  DEV static u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(uint32_t, f[i]);
    return v;
  }
};
template <> struct Vec<bf16> {
  static constexpr int N = 8;
  DEV static void unpack(const u32x4& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16lo(v[i]);
      f[2 * i + 1] = bf16hi(v[i]);
    }
  }
  DEV static u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16(f[2 * i], f[2 * i + 1]);
    return v;
  }
};

// ---------------------------------------------------------------------------------------------
// 32x32 MFMA tile product over one 16-byte fragment per lane.
//   Operand A (32 x k): lane l supplies row l%32; operand B (k x 32): lane l supplies column l%32.
//   Lanes 0-31 and 32-63 hold two disjoint halves of the fragment's k-range.
//   bf16: one v_mfma_f32_32x32x16_bf16 (8 k-values per lane).
//   fp32: four v_mfma_f32_32x32x2f32; product e pairs element e of both lanes' fragments, so the
//         k-slots of A and B line up element by element (a permutation of k shared by both).
//   Result: lane l holds column l%32, rows (r/4)*8 + (l/32)*4 + r%4 for r = 0..15.
// ---------------------------------------------------------------------------------------------
template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  DEV static void mma(f32x16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  DEV static void mma(f32x16& acc, const u32x4& a, const u32x4& b) {
    // cast whole vectors: a per-lane bit-cast of an ext-vector element is folded to element 0
    const f32x4 af = __builtin_bit_cast(f32x4, a);
    const f32x4 bf = __builtin_bit_cast(f32x4, b);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[0], bf[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[1], bf[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[2], bf[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[3], bf[3], acc, 0, 0, 0);
  }
};

// Row of the 32x32 result held in register r by lane half h (= lane / 32).
DEV int mfma_row(int r, int h) { return (r >> 2) * 8 + h * 4 + (r & 3); }

// ---------------------------------------------------------------------------------------------
// Global memory helpers
// ---------------------------------------------------------------------------------------------
DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
DEV void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
DEV u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
DEV void st8(void* p, const u32x2& v) { *reinterpret_cast<u32x2*>(p) = v; }

// ---------------------------------------------------------------------------------------------
// Wave (64 lanes) reductions
// ---------------------------------------------------------------------------------------------
DEV float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
DEV float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Device error word bits
enum { ERR_TOKEN_RANGE = 1, ERR_TARGET_RANGE = 2 };
