// Tile staging and operand-fragment helpers shared by the gfx950 kernels.
#pragma once

#include "favor_device.hpp"

#include <math.h>

namespace favor {

// ---------------------------------------------------------------------------
// Feature maps ("Linear Attention > Kernel Feature Maps", sections 1-4), all
// applied to the projection p = W x:
//   FM_POS   FAVOR+ positive features exp(p - |x|^2/2)/sqrt(m)   (section 4)
//   FM_ELU1  ELU(p) + 1                                           (section 1)
//   FM_RELU  max(0, p)                                            (section 2)
//   FM_TRIG  (1/sqrt(m)) [sin p_i, cos p_i]: 2m features, stored as the m
//            sines then the m cosines                              (section 3)
// The kernels evaluate phi(x) with x = (W s) x + row_bias: W is scaled by
// kWScale when it becomes a matrix operand (log2 e, so FAVOR+ is one exp2;
// 1/(2 pi) for the trig map, whose sine and cosine take revolutions), and
// row_bias is FAVOR+'s -(|x|^2/2 + ln(m)/2) log2 e and 0 otherwise.  Rows
// past the end get a bias of -inf, which every map sends to 0.
// ---------------------------------------------------------------------------
enum { FM_POS = 0, FM_ELU1 = 1, FM_RELU = 2, FM_TRIG = 3 };

template <int FM>
struct FMap {
  static constexpr float kWScale = FM == FM_POS ? kLog2e : (FM == FM_TRIG ? 0.15915494309189535f : 1.f);
  static __device__ __forceinline__ float row_bias(float ss, float half_ln_m) {
    if constexpr (FM == FM_POS) return -(0.5f * ss + half_ln_m) * kLog2e;
    else return 0.f;
  }
  // cosine: the feature is in the second (cosine) half (FM_TRIG);
  // scale: 1/sqrt(m) (FM_TRIG)
  static __device__ __forceinline__ float phi(float x, bool cosine, float scale) {
    if constexpr (FM == FM_POS) {
      return exp2_fast(x);
    } else if constexpr (FM == FM_ELU1) {
      return x > 0.f ? x + 1.f : exp2_fast(x * kLog2e);
    } else if constexpr (FM == FM_RELU) {
      return fmaxf(x, 0.f);
    } else {
      if (x == -INFINITY) return 0.f;
      return scale * (cosine ? __builtin_amdgcn_cosf(x) : __builtin_amdgcn_sinf(x));
    }
  }
};

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
        v = *(const u32x4*)((const char*)src + ((size_t)row * D) * sizeof(E) + cc * 16);
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
  // hold it; the lane holding chunk 0 of a row writes the feature map's
  // row bias to sb (-inf for rows at or beyond nvalid).
  template <int FM = FM_POS>
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
      ss = group_sum<CPR>(ss);
      int row = c / CPR;
      if (c < TT * CPR && (c % CPR) == 0)
        sb[row] = row < nvalid ? FMap<FM>::row_bias(ss, half_ln_m) : -INFINITY;
    }
  }
};

// Projection fragment of W (lane = feature f, d-major slots), scaled by the
// feature map's factor (log2 e for FAVOR+) and converted to the projection
// operand type (fp16 for bf16 inputs).
template <class Tr, int D, int FM = FM_POS>
__device__ __forceinline__ typename Tr::frag w_frag(const float* wrow, int hh, int s, bool ok) {
  constexpr float sc = FMap<FM>::kWScale;
  const int d0 = (D / 2) * hh + Tr::VPS * s;
  if constexpr (Tr::VPS == 8) {
    f32x4 a = ok ? *(const f32x4*)(wrow + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 b = ok ? *(const f32x4*)(wrow + d0 + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 f;
    f[0] = pack_f16(a[0] * sc, a[1] * sc);
    f[1] = pack_f16(a[2] * sc, a[3] * sc);
    f[2] = pack_f16(b[0] * sc, b[1] * sc);
    f[3] = pack_f16(b[2] * sc, b[3] * sc);
    return f;
  } else {
    return ok ? wrow[d0] * sc : 0.f;
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

// ---------------------------------------------------------------------------
// Direct-to-LDS tile pipeline.
//
// Tiles of TT rows x D elements are copied from global memory into LDS with
// global_load_lds_dwordx4 (each lane's 16 bytes land at base + 16 * lane), so
// several tiles can be in flight without holding registers.  Rows are dense
// (ROWB = D * sizeof(E) bytes); the 16-byte chunk c of row r is stored in
// slot c ^ (r & SWZ) of that row, which spreads the rows of a column read
// over the LDS banks.  Waits are explicit: the compiler's own barrier
// (__syncthreads) would drain every outstanding copy.
// ---------------------------------------------------------------------------
#define FAVOR_GLB(p) ((__attribute__((address_space(1))) void*)(p))

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// wait until at most n vector-memory operations of this wave are outstanding
// (n is a multiple of STEP in [0, STEP * MAXK])
template <int STEP, int MAXK>
__device__ __forceinline__ void wait_vmcnt_steps(int k) {
  static_assert(STEP * MAXK < 64, "vmcnt range");
  if constexpr (MAXK >= 3) { if (k >= 3) { wait_vmcnt<3 * STEP>(); return; } }
  if constexpr (MAXK >= 2) { if (k == 2) { wait_vmcnt<2 * STEP>(); return; } }
  if constexpr (MAXK >= 1) { if (k == 1) { wait_vmcnt<STEP>(); return; } }
  wait_vmcnt<0>();
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
// workgroup barrier that does not wait for outstanding global->LDS copies
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Copy n16 16-byte chunks from global src to LDS dst with global->LDS loads
// issued by all NT threads (chunk c lands at dst + 16 c).  Completion is
// waited for with the vector-memory counter.
template <int NT>
__device__ __forceinline__ void dma_copy(char* dst, const char* src, int n16, int tid) {
  const int w = tid >> 6, lane = tid & 63;
  for (int c0 = w * 64; c0 < n16; c0 += NT) {
    const int c = c0 + lane;
    if (c < n16) __builtin_amdgcn_global_load_lds(FAVOR_GLB(src + (size_t)c * 16), LDS_PTR(void, dst + c0 * 16), 16, 0, 0);
  }
}

template <class E, int D, int TT, int NT = 256>
struct DmaTile {
  static constexpr int ROWB = D * (int)sizeof(E);       // bytes per dense row
  static constexpr int CPR = ROWB / 16;                  // chunks per row
  static constexpr int SWZ = (CPR < 8 ? CPR : 8) - 1;
  static constexpr int BYTES = TT * ROWB;
  static constexpr int NW = NT / 64;                     // waves in the workgroup
  static constexpr int NI = TT * CPR / NT;               // copy instructions per wave
  static_assert(NI >= 1 && NI * NT == TT * CPR, "tile must split evenly over the waves");

  // issue this wave's copies of rows [0, TT) of src (row-major, D per row);
  // rows at or beyond nvalid (>= 1) re-read row 0, so every address is valid
  static __device__ __forceinline__ void issue(char* lds, const E* src, int nvalid, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int blk = i * NW + wave;                     // 64-slot block of this instruction
      const int P = blk * 64 + lane;
      const int r = P / CPR, sl = P % CPR;
      const int c = sl ^ (r & SWZ);
      const int rr = r < nvalid ? r : 0;
      const char* g = (const char*)src + (size_t)rr * ROWB + c * 16;
      __builtin_amdgcn_global_load_lds(FAVOR_GLB(g), LDS_PTR(void, lds + blk * 64 * 16), 16, 0, 0);
    }
  }
  // Per-lane plan of this lane's copies, computed once: byte offset in the
  // source tile (and the row-0 fallback used for rows past the end).
  struct Lane {
    int off[NI];     // r * ROWB + c * 16
    int off0[NI];    // c * 16 (row 0)
    int row[NI];
  };
  static __device__ __forceinline__ Lane lane_plan(int wave, int lane) {
    Lane p;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int P = (i * NW + wave) * 64 + lane;
      const int r = P / CPR, c = (P % CPR) ^ (r & SWZ);
      p.off[i] = r * ROWB + c * 16;
      p.off0[i] = c * 16;
      p.row[i] = r;
    }
    return p;
  }
  // copy one tile: src points at its first row (wave-uniform), nvalid >= 1
  static __device__ __forceinline__ void issue_plan(char* lds, const char* src, int nvalid, const Lane& p, int wave) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int off = (nvalid >= TT || p.row[i] < nvalid) ? p.off[i] : p.off0[i];
      __builtin_amdgcn_global_load_lds(FAVOR_GLB(src + off), LDS_PTR(void, lds + (i * NW + wave) * 1024), 16, 0, 0);
    }
  }
  // byte offset of element e of row r
  static __device__ __forceinline__ int at(int r, int e) {
    const int b = e * (int)sizeof(E);
    return r * ROWB + (((b >> 4) ^ (r & SWZ)) << 4) + (b & 15);
  }
  // 16-byte chunk c of row r
  static __device__ __forceinline__ u32x4 chunk(const char* lds, int r, int c) {
    return *(const u32x4*)(lds + r * ROWB + ((c ^ (r & SWZ)) << 4));
  }
};

// Addresses of the two transposed reads of a bf16 col_frag from a swizzled
// dense tile (see col_frag_swz).
template <class DT>
__device__ __forceinline__ void col_frag_swz_addr(const char* base, int row0, int col0, int s, int lane,
                                                  const void*& lo, const void*& hi) {
  const int hh = lane >> 5, i16 = lane & 15, g = (lane >> 4) & 1;
  const int r = row0 + 16 * s + 4 * hh + (i16 >> 2);
  const int off = DT::at(r, col0 + 16 * g + 4 * (i16 & 3));
  lo = base + off;
  hi = base + off + 8 * DT::ROWB;                       // row + 8 keeps (row & SWZ) when SWZ < 8
}

// All NDB x 2 bf16 fragments of a 32-row block of a swizzled dense tile
// (k-steps 0 and 1 of every 32-column block), read in batches that wait for
// themselves; safe while global->LDS copies into other slots are in flight.
template <class DT, int NDB>
__device__ __forceinline__ void col_frags_swz_bf16(const char* base, int row0, int lane, u32x4 (&f)[NDB][2]) {
  if constexpr (NDB == 1) {
    const void *a0, *a1, *a2, *a3;
    col_frag_swz_addr<DT>(base, row0, 0, 0, lane, a0, a1);
    col_frag_swz_addr<DT>(base, row0, 0, 1, lane, a2, a3);
    u32x2 r0, r1, r2, r3;
    lds_read_tr16_x4(a0, a1, a2, a3, r0, r1, r2, r3);
    f[0][0] = u32x4{r0[0], r0[1], r1[0], r1[1]};
    f[0][1] = u32x4{r2[0], r2[1], r3[0], r3[1]};
  } else {
    static_assert(NDB % 2 == 0, "pairs of d blocks");
#pragma unroll
    for (int db = 0; db < NDB; db += 2) {
      const void* a[8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s) col_frag_swz_addr<DT>(base, row0, (db + j) * 32, s, lane, a[4 * j + 2 * s], a[4 * j + 2 * s + 1]);
      u32x2 r[8];
      lds_read_tr16_x8(a, r);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int s = 0; s < 2; ++s)
          f[db + j][s] = u32x4{r[4 * j + 2 * s][0], r[4 * j + 2 * s][1], r[4 * j + 2 * s + 1][0], r[4 * j + 2 * s + 1][1]};
    }
  }
}

// col_frag for a swizzled dense tile (see col_frag).
template <class Tr, class DT>
__device__ __forceinline__ typename Tr::frag col_frag_swz(const char* base, int row0, int col0, int s, int lane) {
  const int hh = lane >> 5;
  if constexpr (Tr::VPS == 8) {
    const int i16 = lane & 15, g = (lane >> 4) & 1;
    const int r = row0 + 16 * s + 4 * hh + (i16 >> 2);
    const int off = DT::at(r, col0 + 16 * g + 4 * (i16 & 3));
    u32x2 lo = lds_read_tr16(base + off);
    u32x2 hi = lds_read_tr16(base + off + 8 * DT::ROWB);   // row + 8 keeps (row & SWZ) when SWZ < 8
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    return *(const float*)(base + DT::at(row0 + crow(s, hh), col0 + (lane & 31)));
  }
}

// Staging pass over a DMA'd tile: convert rows to the projection operand type
// into a padded [TT][RS] tile, and write bias(row) = -(|x|^2/2 + ln(m)/2) log2 e
// (-inf for rows at or beyond nvalid).  Threads own consecutive 16-byte
// chunks, so the CPR chunks of a row sit in consecutive lanes of one wave.
template <class E, int D, int TT, int NT = 256>
__device__ __forceinline__ void prep_proj_tile(const char* raw, char* out, float* bias, int nvalid, float half_ln_m,
                                               int tid) {
  using DT = DmaTile<E, D, TT, NT>;
  constexpr int CPR = DT::CPR;
  constexpr int RS = Rows<D, sizeof(E)>::RS;
#pragma unroll
  for (int i = 0; i < DT::NI; ++i) {                     // TT * CPR chunks over NT threads
    const int c = tid + i * NT;
    const int r = c / CPR, cc = c % CPR;
    u32x4 v = DT::chunk(raw, r, cc);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (sizeof(E) == 2) {
        const float lo = bf16_lo(v[j]), hi = bf16_hi(v[j]);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
        v[j] = pack_f16_sat(lo, hi);
      } else {
        const float x = as_f32(v[j]);
        ss = fmaf(x, x, ss);
      }
    }
    *(u32x4*)(out + r * RS + cc * 16) = v;
    ss = group_sum<CPR>(ss);
    if (cc == 0) bias[r] = r < nvalid ? -(0.5f * ss + half_ln_m) * kLog2e : -INFINITY;
  }
}

}  // namespace favor
