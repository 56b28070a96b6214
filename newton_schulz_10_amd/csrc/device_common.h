// Device helpers shared by the HIP kernels of the batched Muon step.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace muon {

typedef unsigned short bf16_t;  // bf16 storage

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<unsigned>(h) << 16);
}

// Round to nearest, ties to even (gfx950's v_cvt_pk_bf16_f32); NaN stays
// NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two values rounded as one packed pair (lo in bits 0..15): a single
// v_cvt_pk_bf16_f32 instead of two conversions and a repack.
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ unsigned f32x2_to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// Deterministic sum over a 256-thread block (fixed shuffle tree, then the
// four wave totals in order). Every thread returns the total.
__device__ __forceinline__ float block_sum_256(float v, float* red /* >= 4 floats LDS */) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float t = ((red[0] + red[1]) + red[2]) + red[3];
  return t;
}

// Maps the hardware block id to a logical tile id so that each XCD (blocks
// are dealt round-robin over the 8 XCDs) works on a contiguous range of
// logical tiles, i.e. on whole matrices, keeping each matrix's operands in
// one XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int kXcd = 8;
  const int x = bid % kXcd, slot = bid / kXcd;
  const int base = total / kXcd, rem = total % kXcd;
  return x * base + (x < rem ? x : rem) + slot;
}

}  // namespace muon
