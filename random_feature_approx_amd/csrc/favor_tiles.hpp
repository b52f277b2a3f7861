// Tile staging and operand-fragment helpers shared by the gfx950 kernels.
#pragma once

#include "favor_device.hpp"

#include <math.h>

namespace favor {

// LDS row stride in bytes for a [rows][D] tile of element size ES: 16 bytes
// of padding move consecutive rows to different LDS banks.
template <int D, int ES> struct Rows {
  static constexpr int CPR = D * ES / 16;      // 16-byte chunks per row
  static constexpr int RS = D * ES + 16;       // padded row stride (bytes)
};

// Load the 16-byte chunks of a [TT][D] tile that thread `tid` owns into
// registers; rows at or beyond nvalid read as zero.
template <class E, int D, int TT, int NT>
struct TileLoader {
  static constexpr int CPR = Rows<D, sizeof(E)>::CPR;
  static constexpr int NCH = (TT * CPR + NT - 1) / NT;
  u32x4 r[NCH];
  __device__ __forceinline__ void load(const E* src, int nvalid, int tid) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      int c = tid + i * NT;
      int row = c / CPR, cc = c % CPR;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c < TT * CPR && row < nvalid)
        v = __builtin_nontemporal_load((const u32x4*)((const char*)src + ((size_t)row * D) * sizeof(E) + cc * 16));
      r[i] = v;
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      int c = tid + i * NT;
      if (c < TT * CPR) {
        int row = c / CPR, cc = c % CPR;
        *(u32x4*)(lds + row * Rows<D, sizeof(E)>::RS + cc * 16) = r[i];
      }
    }
  }
  // Store with the elements converted to the projection operand type.
  __device__ __forceinline__ void store_proj(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      int c = tid + i * NT;
      if (c < TT * CPR) {
        int row = c / CPR, cc = c % CPR;
        u32x4 v = r[i];
        if constexpr (sizeof(E) == 2)
          v = u32x4{bf16x2_to_f16x2(v[0]), bf16x2_to_f16x2(v[1]), bf16x2_to_f16x2(v[2]), bf16x2_to_f16x2(v[3])};
        *(u32x4*)(lds + row * Rows<D, sizeof(E)>::RS + cc * 16) = v;
      }
    }
  }
  // Squared norm of each row, reduced over the CPR consecutive lanes that
  // hold it; the lane holding chunk 0 of a row writes bias(row) to sb.
  __device__ __forceinline__ void row_bias(float* sb, int tid, int nvalid, float half_ln_m) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      int c = tid + i * NT;
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(E) == 2) {
          float a = bf16_lo(r[i][j]), b = bf16_hi(r[i][j]);
          ss = fmaf(a, a, ss);
          ss = fmaf(b, b, ss);
        } else {
          float a = as_f32(r[i][j]);
          ss = fmaf(a, a, ss);
        }
      }
#pragma unroll
      for (int o = 1; o < CPR; o <<= 1) ss += __shfl_xor(ss, o);
      int row = c / CPR;
      if (c < TT * CPR && (c % CPR) == 0)
        sb[row] = row < nvalid ? -(0.5f * ss + half_ln_m) * kLog2e : -INFINITY;
    }
  }
};

// Projection fragment of W (lane = feature f, d-major slots), scaled by
// log2 e and converted to the projection operand type (fp16 for bf16 inputs).
template <class Tr, int D>
__device__ __forceinline__ typename Tr::frag w_frag(const float* wrow, int hh, int s, bool ok) {
  const int d0 = (D / 2) * hh + Tr::VPS * s;
  if constexpr (Tr::VPS == 8) {
    f32x4 a = ok ? *(const f32x4*)(wrow + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 b = ok ? *(const f32x4*)(wrow + d0 + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 f;
    f[0] = pack_f16(a[0] * kLog2e, a[1] * kLog2e);
    f[1] = pack_f16(a[2] * kLog2e, a[3] * kLog2e);
    f[2] = pack_f16(b[0] * kLog2e, b[1] * kLog2e);
    f[3] = pack_f16(b[2] * kLog2e, b[3] * kLog2e);
    return f;
  } else {
    return ok ? wrow[d0] * kLog2e : 0.f;
  }
}

// Operand fragment of a row-major [.][D] tile in LDS for the lane's row,
// d-major slots (k-step s, lane half hh).
template <class Tr, int D>
__device__ __forceinline__ typename Tr::frag row_frag(const char* rowp, int hh, int s) {
  const int d0 = (D / 2) * hh + Tr::VPS * s;
  if constexpr (Tr::VPS == 8) return *(const u32x4*)(rowp + d0 * 2);
  else return *(const float*)(rowp + d0 * 4);
}

// Operand fragment holding, for column `col` (lane%32 of a 32-column block
// starting at col0) of a row-major LDS tile, the 32-row block starting at row0
// in c-row order for k-step s.  bf16: two transposed reads of 4 rows each;
// f32: one element.
template <class Tr, int RS>
__device__ __forceinline__ typename Tr::frag col_frag(const char* base, int row0, int col0, int s, int lane) {
  const int hh = lane >> 5;
  if constexpr (Tr::VPS == 8) {
    const int i16 = lane & 15, g = (lane >> 4) & 1;
    const char* p = base + (row0 + 16 * s + 4 * hh + (i16 >> 2)) * RS + (col0 + 16 * g + 4 * (i16 & 3)) * 2;
    u32x2 lo = lds_read_tr16(p);
    u32x2 hi = lds_read_tr16(p + 8 * RS);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    return *(const float*)(base + (row0 + crow(s, hh)) * RS + (col0 + (lane & 31)) * 4);
  }
}

}  // namespace favor
