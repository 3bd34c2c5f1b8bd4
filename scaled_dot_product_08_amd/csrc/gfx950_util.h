// Device helpers shared by the gfx950 attention kernels: vector types, the
// 32x32x16 16-bit MFMA, 16-bit packing, the exchange between the two halves of
// a wave, raw buffer descriptors and the 16-byte-chunk swizzle of 16-bit LDS
// tile rows. One copy, so that a fix to any of them reaches every kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa08 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int NXCD = 8;                 // accelerator complex dies; workgroups go round-robin over them
constexpr int BUF_FLAGS = 0x00020000;   // raw buffer descriptor word 3 (32-bit dwords)

// 32x32x16 MFMA, fp32 accumulate; a and b carry eight 16-bit values each.
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Two floats -> two 16-bit values (round to nearest even), low half first.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  f32x2 v = {x, y};
  if constexpr (BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
}

// The two 16-bit values of a packed pair, widened to fp32 exactly.
template <bool BF16>
__device__ __forceinline__ f32x2 unpack2(uint32_t w) {
  if constexpr (BF16) {
    return f32x2{__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u)};
  } else {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
  }
}

// Swap bits 2 and 3 of a small index (orders head-dim outputs so that every
// lane ends with runs of eight consecutive columns).
__device__ __forceinline__ int swap23(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

// 16-byte chunk swizzle of a 16-bit LDS tile row of D elements. Chunk c of
// row r lives at chunk c ^ swz(r). Chosen so that (a) 16 consecutive rows read
// at one logical chunk hit 16 different bank groups (operand reads with
// ds_read_b128), (b) 4 consecutive rows read over 64 contiguous bytes hit 16
// different bank groups (transposing reads), and (c) the 1 KB direct loads
// write whole rows, on the 64-bank, 4-byte-wide LDS.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
}

// Combine the two halves of a wave: lane i gets op(x[i % 32], x[i % 32 + 32]).
// v_permlane32_swap_b32 a, b exchanges the upper half of a with the lower
// half of b; with a = b = x, afterwards {a, b} = {x[i % 32], x[i % 32 + 32]}
// at every lane (measured), in some order, and max and + are symmetric. It is
// written in assembly because the compiler's model of the builtin's second
// result folds it into the first; the s_nops on either side cover the
// VALU-to-permlane and permlane-to-VALU hazards.
__device__ __forceinline__ void swap_halves(float x, float& a, float& b) {
  a = x;
  b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float half_max(float x) {
  float a, b;
  swap_halves(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float half_sum(float x) {
  float a, b;
  swap_halves(x, a, b);
  return a + b;
}

// Raw buffer descriptor of nbytes from base: loads past the end return zero
// and stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, BUF_FLAGS);
}

// s_waitcnt vmcnt(0), the other counters untouched (gfx9 encoding).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Workgroup i of a grid of G runs on XCD i % 8. The logical index that gives
// each XCD one contiguous run of the logical order.
__device__ __forceinline__ int xcd_logical(int i, int G) {
  const int xcd = i % NXCD, local = i / NXCD;
  const int gq = G / NXCD, gr = G % NXCD;
  return (xcd < gr) ? xcd * (gq + 1) + local : gr * (gq + 1) + (xcd - gr) * gq + local;
}

}  // namespace sdpa08
