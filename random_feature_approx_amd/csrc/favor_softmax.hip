// Exact softmax attention on gfx950: O = softmax(scale * Q K^T) V, optionally
// masked to keys j <= i.  This is the quadratic attention that FAVOR+
// approximates (the softmax-kernel equation of "Linear Attention > Kernel
// Feature Maps"; the left side of the performer-2020 study notes' reordering
// diagram), kept here as the library's own reference for speed and quality
// comparisons at the same shapes.
//
// One wave owns 32 queries and walks the keys in blocks of 32 with a running
// maximum (online softmax): scores are computed transposed, S^T = K Q^T, so
// each lane holds one query's scores and its running maximum, sum and the
// rescaling of its output column O^T are per-lane scalars.  Four waves share
// 64-key tiles of K and V staged in LDS.
#include "favor_device.hpp"
#include "favor_internal.hpp"
#include "favor_tiles.hpp"

#include <math.h>

namespace favor {

struct SoftmaxArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int L;
  float scale_log2e;     // scale * log2(e): scores go straight into exp2
  int causal;
};

template <class Tr, int D>
struct SmLds {
  using E = typename Tr::elem;
  static constexpr int KB = 64;                          // keys per staged tile
  static constexpr int RS = Rows<D, sizeof(E)>::RS;
  static constexpr int kK = 0, kV = KB * RS;
  static constexpr int kTotal = 2 * KB * RS;
};

template <class Tr, int D>
__global__ __launch_bounds__(256) void k_softmax(SoftmaxArgs a) {
  using E = typename Tr::elem;
  using F = typename Tr::frag;
  using LY = SmLds<Tr, D>;
  constexpr int KB = LY::KB, RS = LY::RS;
  constexpr int NKD = D / Tr::KS;
  constexpr int NDB = D / 32;
  constexpr int NKT = 32 / Tr::KS;
  constexpr int ES = (int)sizeof(E);
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* sK = smem + LY::kK;
  char* sV = smem + LY::kV;

  const int bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
  const size_t hoff = (size_t)bh * a.L * D;
  const E* Qg = (const E*)a.q + hoff;
  const E* Kg = (const E*)a.k + hoff;
  const E* Vg = (const E*)a.v + hoff;
  const int q0 = blockIdx.x * 128;                       // this workgroup's queries
  const int qw = q0 + w * 32;                            // this wave's queries
  const int qi = qw + l32;                               // this lane's query
  const bool qok = qi < a.L;

  // this lane's half of its query row (d-major slots)
  F qf[NKD];
  {
    const E* qrow = Qg + (size_t)(qok ? qi : 0) * D;
#pragma unroll
    for (int s = 0; s < NKD; ++s) {
      const int d0 = (D / 2) * hh + Tr::VPS * s;
      if constexpr (Tr::VPS == 8) qf[s] = qok ? *(const u32x4*)(qrow + d0) : u32x4{0u, 0u, 0u, 0u};
      else qf[s] = qok ? qrow[d0] : 0.f;
    }
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = zero16();
  float mrun = -1e30f, lsum = 0.f;                       // finite start: an all-masked block rescales by 1

  const int kend = a.causal ? min(a.L, q0 + 128) : a.L;  // keys this workgroup needs
  const int nkb = (kend + KB - 1) / KB;
  TileLoader<E, D, KB, 256> lk, lv;
  if (nkb > 0) {
    lk.load(Kg, kend, tid);
    lv.load(Vg, kend, tid);
  }
  for (int kb = 0; kb < nkb; ++kb) {
    const int k0 = kb * KB;
    __syncthreads();                                     // the previous tile is consumed
    lk.store(sK, tid);
    lv.store(sV, tid);
    __syncthreads();
    if (kb + 1 < nkb) {
      lk.load(Kg + (size_t)(k0 + KB) * D, kend - k0 - KB, tid);
      lv.load(Vg + (size_t)(k0 + KB) * D, kend - k0 - KB, tid);
    }
#pragma unroll
    for (int sb = 0; sb < KB / 32; ++sb) {
      const int j0 = k0 + sb * 32;
      if (j0 >= kend || (a.causal && j0 > qw + 31)) continue;   // wave-uniform
      // S^T[j][i] = k_j . q_i (rows = keys, lane = query)
      f32x16 st = zero16();
#pragma unroll
      for (int s = 0; s < NKD; ++s) st = Tr::mma(row_frag<Tr, D>(sK + (sb * 32 + l32) * RS, hh, s), qf[s], st);
      float bmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + crow(r, hh);
        const bool keep = j < kend && (!a.causal || j <= qi);
        st[r] = keep ? st[r] * a.scale_log2e : -INFINITY;
        bmax = fmaxf(bmax, st[r]);
      }
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, bmax),
                                                         __builtin_bit_cast(unsigned, bmax), false, false);
        const unsigned s0 = sw[0], s1 = sw[1];
        bmax = fmaxf(as_f32(s0), as_f32(s1));
      }
      const float mnew = fmaxf(mrun, bmax);
      const float alpha = exp2_fast(mrun - mnew);
      mrun = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[r] = exp2_fast(st[r] - mnew);
        lsum += st[r];
      }
      // O^T[d][i] += V^T[d][j] P^T[j][i]
#pragma unroll
      for (int s2 = 0; s2 < NKT; ++s2) {
        const F pf = CFrag<Tr>::make(st, s2);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = Tr::mma(col_frag<Tr, RS>(sV, sb * 32, db * 32, s2, lane), pf, oacc[db]);
      }
    }
  }
  lsum = half_sum(lsum);
  if (qok) {
    const float inv = 1.f / lsum;
    E* orow = (E*)a.o + hoff + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hh;
        if constexpr (ES == 2) {
          *(u32x2*)(orow + d0) = u32x2{pack_bf16(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                                       pack_bf16(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        } else {
          *(f32x4*)(orow + d0) = f32x4{oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                                       oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
        }
      }
  }
}

template <class Tr, int D>
static hipError_t softmax_t(const Plan& p, const void* q, const void* k, const void* v, void* o, float scale,
                            int causal, hipStream_t s) {
  SoftmaxArgs a{q, k, v, o, p.L, scale * kLog2e, causal};
  const dim3 grid((p.L + 127) / 128, p.BH);
  const size_t lds = SmLds<Tr, D>::kTotal;
  timing_begin(FAVOR_KERNEL_SOFTMAX, s);
  hipLaunchKernelGGL((k_softmax<Tr, D>), grid, dim3(256), lds, s, a);
  timing_end(FAVOR_KERNEL_SOFTMAX, s);
  return hipGetLastError();
}

hipError_t launch_softmax(const Plan& p, const void* q, const void* k, const void* v, void* o, float scale,
                          int causal, hipStream_t s) {
  if (p.dt == FAVOR_BF16) {
    switch (p.D) {
      case 32: return softmax_t<TrBF16, 32>(p, q, k, v, o, scale, causal, s);
      case 64: return softmax_t<TrBF16, 64>(p, q, k, v, o, scale, causal, s);
      case 128: return softmax_t<TrBF16, 128>(p, q, k, v, o, scale, causal, s);
    }
  } else {
    switch (p.D) {
      case 32: return softmax_t<TrF32, 32>(p, q, k, v, o, scale, causal, s);
      case 64: return softmax_t<TrF32, 64>(p, q, k, v, o, scale, causal, s);
      case 128: return softmax_t<TrF32, 128>(p, q, k, v, o, scale, causal, s);
    }
  }
  return kErrPlan;
}

}  // namespace favor
