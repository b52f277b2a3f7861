// Device building blocks for the gfx950 FAVOR+ kernels.
//
// Matrix-core conventions (32x32 output blocks, wave64):
//   * v_mfma_f32_32x32x16_bf16: lane l supplies A[l%32][8*(l/32) + 0..7] and
//     B[8*(l/32) + 0..7][l%32]; accumulator value r of lane l is
//     C[crow(r, l/32)][l%32] with crow(r, h) = 8*(r/4) + 4*h + r%4.
//   * v_mfma_f32_32x32x2_f32: lane l supplies A[l%32][l/32] and B[l/32][l%32];
//     same accumulator layout.
// The contraction index of a product is a dummy index, so each kernel is free
// to permute it as long as both operands use the same permutation.  Two
// permutations are used throughout:
//   * "d-major": for a k-step s and lane half h, slot j covers
//     d = (D/2)*h + VPS*s + j, so a lane reads D/2 contiguous elements of a
//     row of Q, K or W;
//   * "c-row": an operand produced as an accumulator (a feature value, a
//     score) is consumed in the k-slot order of crow(), so no data moves
//     between lanes; the matching operand is gathered in the same order with
//     transposed LDS reads (ds_read_b64_tr_b16), which hand each lane of a
//     16-lane group one column of a 4 x 16 block of 16-bit values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace favor {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ constexpr int crow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Round two floats to bf16 (nearest even) and pack them into one dword.
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(unsigned, b);
}

// Round two floats to fp16 (nearest even) and pack them into one dword.
__device__ __forceinline__ unsigned pack_f16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
}

// Reinterpret a dword as float.  Vector elements are passed by value: a
// __builtin_bit_cast applied directly to a vector subscript has been seen to
// read element 0 whatever the subscript.
__device__ __forceinline__ float as_f32(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned as_u32(float x) { return __builtin_bit_cast(unsigned, x); }

__device__ __forceinline__ float bf16_lo(unsigned u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned u) { return __builtin_bit_cast(float, u & 0xffff0000u); }

// Two floats as fp16 (nearest even), saturated at +-65504 rather than
// rounded to infinity: an input row of the projection with entries past
// fp16's range keeps a finite projection, and its float32 row bias
// -|x|^2/2 (taken from the unsaturated values) sends FAVOR+ features to 0.
__device__ __forceinline__ unsigned pack_f16_sat(float lo, float hi) {
  return pack_f16(__builtin_amdgcn_fmed3f(lo, -65504.f, 65504.f), __builtin_amdgcn_fmed3f(hi, -65504.f, 65504.f));
}

// A dword of two bf16 values re-encoded as two fp16 values.  Exact for
// magnitudes in fp16's normal range [2^-14, 65504]; smaller values keep an
// absolute error below 2^-25; larger ones saturate at +-65504.
__device__ __forceinline__ unsigned bf16x2_to_f16x2(unsigned u) { return pack_f16_sat(bf16_lo(u), bf16_hi(u)); }

// Sum of the two bf16 halves of a dword plus acc (exact products with 1.0).
__device__ __forceinline__ float dot2_bf16(unsigned a, unsigned b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

// Transposed LDS read: 4 x 16-bit values; see the header comment.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, p));
  return __builtin_bit_cast(u32x2, v);
}

// Batches of the same transposed read issued from inline assembly.  The
// compiler cannot prove that the builtin does not read LDS that an
// outstanding global->LDS copy is filling, and waits for every copy
// (vmcnt(0)) before it.  Each batch below is a single statement that issues
// its reads and then waits for them (lgkmcnt(0)), so no result can be used,
// moved or copied before its data has arrived; the caller orders the reads
// after the copies it depends on.
__device__ __forceinline__ unsigned lds_addr(const void* p) { return (unsigned)(uintptr_t)LDS_PTR(const char, p); }

__device__ __forceinline__ void lds_read_tr16_x4(const void* p0, const void* p1, const void* p2, const void* p3,
                                                 u32x2& r0, u32x2& r1, u32x2& r2, u32x2& r3) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(lds_addr(p0)), "v"(lds_addr(p1)), "v"(lds_addr(p2)), "v"(lds_addr(p3))
      : "memory");
}

// Two groups of transposed reads at compile-time offsets from two addresses
// (four reads each): group g reads at a_g + O[g][0..3].
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void lds_read_tr16_2x4(unsigned a0, unsigned a1, u32x2 (&r)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%10\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%11\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %4, %9 offset:%10\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:%11\n\t"
      "ds_read_b64_tr_b16 %6, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a0), "v"(a1), "n"(O0), "n"(O1), "n"(O2), "n"(O3)
      : "memory");
}
template <int O0, int O1, int O2, int O3>
__device__ __forceinline__ void lds_read_tr16_1x4(unsigned a0, u32x2 (&r)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%5\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %3, %4 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a0), "n"(O0), "n"(O1), "n"(O2), "n"(O3)
      : "memory");
}

template <int O0, int O1>
__device__ __forceinline__ void lds_read_tr16_1x2(unsigned a0, u32x2 (&r)[2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2 offset:%3\n\t"
      "ds_read_b64_tr_b16 %1, %2 offset:%4\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1])
      : "v"(a0), "n"(O0), "n"(O1)
      : "memory");
}

__device__ __forceinline__ void lds_read_tr16_x8(const void* const p[8], u32x2 (&r)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(lds_addr(p[0])), "v"(lds_addr(p[1])), "v"(lds_addr(p[2])), "v"(lds_addr(p[3])), "v"(lds_addr(p[4])),
        "v"(lds_addr(p[5])), "v"(lds_addr(p[6])), "v"(lds_addr(p[7]))
      : "memory");
}

// ---------------------------------------------------------------------------
// Element-type traits: the operand fragment one lane supplies per k-step.
// ---------------------------------------------------------------------------
// bf16 inputs.  The projection x W^T runs on fp16 operands (x converted
// exactly, W log2(e) rounded to fp16): W's rounding moves every exponent, and
// fp16 keeps 3 more bits than bf16 at the same matrix-core rate.  Features,
// states and V stay bf16 (they need bf16's exponent range).
struct TrBF16 {
  typedef bf16 elem;                  // storage type of Q, K, V, O
  typedef u32x4 frag;                 // 8 bf16 (or, for the projection, fp16) values
  static constexpr int KS = 16;       // k per matrix instruction
  static constexpr int VPS = 8;       // values per lane per k-step
  static constexpr bool kF16Proj = true;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
  // projection product on fp16 operands
  static __device__ __forceinline__ f32x16 pmma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
  static __device__ __forceinline__ u32x4 to_proj(u32x4 x) {
    return u32x4{bf16x2_to_f16x2(x[0]), bf16x2_to_f16x2(x[1]), bf16x2_to_f16x2(x[2]), bf16x2_to_f16x2(x[3])};
  }
  static __device__ __forceinline__ float to_f32(elem x) { return (float)x; }
  static __device__ __forceinline__ elem from_f32(float x) { return (elem)x; }
};

struct TrF32 {
  typedef float elem;
  typedef float frag;                 // 1 value
  static constexpr int KS = 2;
  static constexpr int VPS = 1;
  static constexpr bool kF16Proj = false;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 pmma(frag a, frag b, f32x16 c) { return mma(a, b, c); }
  static __device__ __forceinline__ float to_proj(float x) { return x; }
  static __device__ __forceinline__ float to_f32(elem x) { return x; }
  static __device__ __forceinline__ elem from_f32(float x) { return x; }
};

// Fragment (k-step s of a 32-row accumulator block, c-row order) made from
// the accumulator values themselves.  For bf16 the 8 values r = 8s..8s+7 are
// rounded and packed; for f32 the single value r = s is passed through.
template <class Tr> struct CFrag;
template <> struct CFrag<TrBF16> {
  static __device__ __forceinline__ u32x4 make(const f32x16& v, int s) {
    u32x4 f;
    f[0] = pack_bf16(v[8 * s + 0], v[8 * s + 1]);
    f[1] = pack_bf16(v[8 * s + 2], v[8 * s + 3]);
    f[2] = pack_bf16(v[8 * s + 4], v[8 * s + 5]);
    f[3] = pack_bf16(v[8 * s + 6], v[8 * s + 7]);
    return f;
  }
};
template <> struct CFrag<TrF32> {
  static __device__ __forceinline__ float make(const f32x16& v, int s) { return v[s]; }
};

// x summed over aligned groups of G consecutive lanes (G a power of two up
// to 32): DPP lane permutations within rows of 16, a shuffle beyond.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(G >= 1 && G <= 32 && (G & (G - 1)) == 0, "group size");
  if constexpr (G >= 2) x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));   // lanes ^ 1
  if constexpr (G >= 4) x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));   // lanes ^ 2
  if constexpr (G >= 8) x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));  // mirror in 8
  if constexpr (G >= 16) x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false)); // mirror in 16
  if constexpr (G >= 32) x += __shfl_xor(x, 16);
  return x;
}
// x plus its value in the lane 32 apart (both wave halves get the sum)
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x), false, false);
  const unsigned r0 = r[0], r1 = r[1];   // by value: a bit cast of a vector element reads element 0
  return as_f32(r0) + as_f32(r1);
}

// Zero accumulator.
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Accumulator with every element equal to x (a per-lane starting value).
__device__ __forceinline__ f32x16 splat16(float x) {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = x;
  return z;
}

}  // namespace favor
