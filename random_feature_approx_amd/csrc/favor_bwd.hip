// Backward pass of non-causal FAVOR+ on gfx950: gradients of sum(G * O) with
// respect to Q, K and V for an upstream gradient G = dLoss/dO.
//
// With phi = phi(x) = exp(W x - |x|^2/2)/sqrt(m) (the feature-map equation of
// "Linear Attention > Performer: Unbiased Softmax Approximation"),
// M = phi(K)^T V, z = phi(K)^T 1, D_i = phi(q_i).z + eps, o_i = phi(q_i) M / D_i
// (the reassociated form of the same page's In[25] and of the performer-2020
// study notes' key points), the chain rule gives, per token i and key j,
//   y_i = M g_i,  s_i = phi(q_i).y_i  (= g_i.(o_i D_i)),
//   dphi(q_i) = (y_i - z s_i/D_i) / D_i,
//   dM = sum_i phi(q_i) g_i^T / D_i,  dz = -sum_i phi(q_i) s_i / D_i^2,
//   dv_j = dM^T phi(k_j),  dphi(k_j) = dM v_j + dz,
// and through the feature map d phi_f/dx = phi_f (omega_f - x):
//   dx = W^T (dphi * phi) - sum_f(dphi_f phi_f) x.
// For the query side sum_f(dphi_f phi_f) = s_i eps / D_i^2 exactly.
//
// Kernels (one call):
//   k_bprep     W operands: the projection W log2 e (hi and lo parts) and W^T
//   k_bred      token-split reduction of phi(X)^T Y and phi(X)^T c: with X=K,
//               Y=V, c=1 the state M, z; with X=Q, Y=G, c_i = -s_i/D_i and
//               phi scaled by 1/D_i (through the exponent) the gradients dM, dz
//   k_bcombine  fixed-order sum of the partials into the operands below
//   k_bside     per-token side: Q (two passes over the features: D_i and s_i,
//               then dQ) or K (dK and dV)
//
// Precision (bf16 inputs).  The query-side sum y - z s/D cancels strongly
// for some rows, and so does dM v_j + dz on the key side; every operand that
// feeds those differences is carried as a pair of bf16 values (hi + lo,
// two matrix products) -- the projection (fp16 pair), M, dM and phi(Q)/D --
// so they hold about 16 significant bits.  The last products (W^T against
// the feature gradients, dM^T phi(K)) use single bf16 operands; accumulation
// is float32 throughout.
#include "favor_device.hpp"
#include "favor_internal.hpp"
#include "favor_tiles.hpp"

#include <math.h>

namespace favor {

// ---------------------------------------------------------------------------
// precision traits: operands that are split into hi + lo parts
// ---------------------------------------------------------------------------
template <class Tr> struct Bw;
template <> struct Bw<TrBF16> {
  static constexpr int NS = 2;                       // parts per split operand
  // hi and lo bf16 parts of accumulator values 8s..8s+7 (c-row k order)
  static __device__ __forceinline__ void split(const f32x16& v, int s, u32x4 (&f)[2]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = v[8 * s + 2 * k], b = v[8 * s + 2 * k + 1];
      const unsigned hi = pack_bf16(a, b);
      f[0][k] = hi;
      f[1][k] = pack_bf16(a - bf16_lo(hi), b - bf16_hi(hi));
    }
  }
};
template <> struct Bw<TrF32> {
  static constexpr int NS = 1;
  static __device__ __forceinline__ void split(const f32x16& v, int s, float (&f)[1]) { f[0] = v[s]; }
};

// ---------------------------------------------------------------------------
// k_bprep: projection operand W log2 e in the projection type, as hi and lo
// parts for bf16 (fp16 pair) or one float array, in the operand order
// [Hw*M/32][NKG][half][32][16 B] (lane (f, h) of k-group g holds
// d = (D/2) h + (16/WES) g + 0..); and W^T in the element type in the order
// [Hw*M/32][NKT][NDB][half][32][VPS]: lane (c, h) of k-step s and d block db
// holds W[32 fb + crow(VPS s + j, h)][32 db + c] for j < VPS, the c-row
// feature order of a feature accumulator used as the other operand.
// ---------------------------------------------------------------------------
template <class Tr>
__global__ __launch_bounds__(256) void k_bprep(const float* w, void* wph, void* wpl, void* wt, int nrows, int D) {
  using E = typename Tr::elem;
  constexpr int WES = Tr::VPS == 8 ? 2 : 4;
  constexpr int PER = 16 / WES;
  constexpr int VPS = Tr::VPS;
  constexpr int NKT = 32 / Tr::KS;
  const int nkg = D * WES / 32;
  const int NDB = D / 32;
  const int nproj = nrows * D / PER;                   // 16-byte chunks of the projection operand
  const int nt = nrows * D / VPS;                      // VPS-element groups of W^T
  for (int idx = blockIdx.x * 256 + threadIdx.x; idx < nproj + nt; idx += gridDim.x * 256) {
    if (idx < nproj) {
      const int f = idx & 31, h = (idx >> 5) & 1, rest = idx >> 6;
      const int g = rest % nkg, blk = rest / nkg;
      const float* src = w + (size_t)(blk * 32 + f) * D + (D / 2) * h + PER * g;
      if constexpr (WES == 2) {
        unsigned hi[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float a = src[2 * k] * kLog2e, b = src[2 * k + 1] * kLog2e;
          hi[k] = pack_f16(a, b);
          const f16x2 hv = __builtin_bit_cast(f16x2, hi[k]);
          lo[k] = pack_f16(a - (float)hv[0], b - (float)hv[1]);
        }
        ((u32x4*)wph)[idx] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        ((u32x4*)wpl)[idx] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      } else {
        ((f32x4*)wph)[idx] = *(const f32x4*)src * kLog2e;
      }
    } else {
      const int i = idx - nproj;                       // = ((((fbg*NKT + s)*NDB + db)*2 + h)*32 + c)
      const int c = i & 31, h = (i >> 5) & 1;
      int rest = i >> 6;
      const int db = rest % NDB;
      rest /= NDB;
      const int s = rest % NKT, fbg = rest / NKT;      // fbg: feature block over all Hw heads
      E vals[VPS];
#pragma unroll
      for (int j = 0; j < VPS; ++j) vals[j] = (E)w[(size_t)(fbg * 32 + crow(VPS * s + j, h)) * D + db * 32 + c];
      E* dst = (E*)wt + (size_t)i * VPS;
#pragma unroll
      for (int j = 0; j < VPS; ++j) dst[j] = vals[j];
    }
  }
}

// ---------------------------------------------------------------------------
// k_bred: per (token split, feature group, head) partial
//   P[f][d] = sum_t phi(x_t)[f] e_t y_t[d],  Pz[f] = sum_t phi(x_t)[f] e_t c_t
// with e_t = 1, c_t = 1 (WT = false) or e_t = 2^-lg_t, c_t = cw_t (WT).
// Four waves, one 32-feature block each, share 32-token tiles of X and Y
// staged in LDS (double buffered: tile t+1 is loaded into registers while
// tile t is computed).  Lane layout: projection accumulator rows = tokens,
// lanes = features, so phi feeds phi^T Y directly as the first operand.
// ---------------------------------------------------------------------------
struct BRedArgs {
  const void* x;
  const void* y;
  const float* lg;       // [BH][L] (WT)
  const float* cw;       // [BH][L] (WT)
  const void* wph;       // projection operand, hi part (or the float operand)
  const void* wpl;       // lo part (bf16)
  float* part;           // [BH][splits][M][D]
  float* partz;          // [BH][splits][M]
  int L, M, H, Hw, splits, split_len;
};

template <class Tr, int D>
struct BRedLds {
  using E = typename Tr::elem;
  static constexpr int TT = 32;
  static constexpr int RS = Rows<D, sizeof(E)>::RS;
  static constexpr int kX = 0;
  static constexpr int kY = kX + TT * RS;
  static constexpr int kBias = kY + TT * RS;
  static constexpr int kW = kBias + TT * 4;
  static constexpr int BUF = kW + TT * 4;
  static constexpr int kTotal = 2 * BUF;
};

template <class Tr, int D, bool WT>
__global__ __launch_bounds__(256) void k_bred(BRedArgs a) {
  constexpr int NW = 4, NT = 256, TT = 32;
  using E = typename Tr::elem;
  using F = typename Tr::frag;
  using LY = BRedLds<Tr, D>;
  using TL = TileLoader<E, D, TT, NT>;
  using SP = Bw<Tr>;
  constexpr int NKD = D / Tr::KS;
  constexpr int NDB = D / 32;
  constexpr int NKT = 32 / Tr::KS;
  constexpr int RS = LY::RS;
  constexpr int ES = (int)sizeof(E);
  constexpr int CPR = TL::CPR;
  constexpr int WES = Tr::VPS == 8 ? 2 : 4;
  constexpr int NKG = D * WES / 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int split = blockIdx.x, fg = blockIdx.y, bh = blockIdx.z;
  const int head = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
  const int nfb = a.M >> 5;
  const int fb = fg * NW + w;
  const bool active = fb < nfb;
  const E* X = (const E*)a.x + (size_t)bh * a.L * D;
  const E* Y = (const E*)a.y + (size_t)bh * a.L * D;
  const float half_ln_m = 0.5f * logf((float)a.M);

  // projection operand of this wave's feature block (lane = feature f)
  F wf[SP::NS][NKD];
  {
    const int hw = a.Hw == 1 ? 0 : head;
    const int fbg = hw * nfb + (active ? fb : 0);
#pragma unroll
    for (int p = 0; p < SP::NS; ++p) {
      const char* base = (const char*)(p == 0 ? a.wph : a.wpl) + (size_t)fbg * NKG * 2 * 32 * 16;
      if constexpr (WES == 2) {
#pragma unroll
        for (int s = 0; s < NKD; ++s) wf[p][s] = *(const u32x4*)(base + ((s * 2 + hh) * 32 + l32) * 16);
      } else {
#pragma unroll
        for (int g = 0; g < NKG; ++g) {
          const f32x4 v = *(const f32x4*)(base + ((g * 2 + hh) * 32 + l32) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) wf[p][4 * g + j] = v[j];
        }
      }
    }
  }

  f32x16 st[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) st[db] = zero16();
  float zs = 0.f;

  const int t0 = split * a.split_len;
  const int t1 = min(a.L, t0 + a.split_len);
  const int ntiles = t0 < t1 ? (t1 - t0 + TT - 1) / TT : 0;

  TL xl, yl;
  if (ntiles > 0) {
    xl.load(X + (size_t)t0 * D, t1 - t0, tid);
    yl.load(Y + (size_t)t0 * D, t1 - t0, tid);
  }
  for (int tt = 0; tt < ntiles; ++tt) {
    char* buf = smem + (tt & 1) * LY::BUF;
    const int r0 = t0 + tt * TT;
    const int nvalid = min(TT, t1 - r0);
    // stage tile tt: X in the projection type, Y raw, row biases and weights
    xl.store_proj(buf + LY::kX, tid);
    yl.store(buf + LY::kY, tid);
    {
      float* sb = (float*)(buf + LY::kBias);
      float* sw = (float*)(buf + LY::kW);
#pragma unroll
      for (int i = 0; i < TL::NCH; ++i) {
        const int c = tid + i * NT;
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (ES == 2) {
            const float lo = bf16_lo(xl.r[i][j]), hi = bf16_hi(xl.r[i][j]);
            ss = fmaf(lo, lo, fmaf(hi, hi, ss));
          } else {
            const float x = as_f32(xl.r[i][j]);
            ss = fmaf(x, x, ss);
          }
        }
        ss = group_sum<CPR>(ss);
        const int row = c / CPR;
        if (c < TT * CPR && (c % CPR) == 0) {
          float b = -INFINITY, wt = 0.f;
          if (row < nvalid) {
            b = -(0.5f * ss + half_ln_m) * kLog2e;
            wt = 1.f;
            if constexpr (WT) {
              b -= a.lg[(size_t)bh * a.L + r0 + row];
              wt = a.cw[(size_t)bh * a.L + r0 + row];
            }
          }
          sb[row] = b;
          sw[row] = wt;
        }
      }
    }
    __syncthreads();
    if (tt + 1 < ntiles) {
      const int n0 = r0 + TT;
      xl.load(X + (size_t)n0 * D, t1 - n0, tid);
      yl.load(Y + (size_t)n0 * D, t1 - n0, tid);
    }
    if (active) {
      const float* sb = (const float*)(buf + LY::kBias);
      const float* sw = (const float*)(buf + LY::kW);
      f32x16 acc;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 b4 = *(const f32x4*)(sb + 8 * g + 4 * hh);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * g + j] = b4[j];
      }
#pragma unroll
      for (int s = 0; s < NKD; ++s) {
        const F xf = row_frag<Tr, D>(buf + LY::kX + l32 * RS, hh, s);
#pragma unroll
        for (int p = 0; p < SP::NS; ++p) acc = Tr::pmma(xf, wf[p][s], acc);   // P[t][f] + bias[t]
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = exp2_fast(acc[r]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 w4 = *(const f32x4*)(sw + 8 * g + 4 * hh);
#pragma unroll
        for (int j = 0; j < 4; ++j) zs = fmaf(acc[4 * g + j], w4[j], zs);
      }
#pragma unroll
      for (int s2 = 0; s2 < NKT; ++s2) {
        F pf[SP::NS];
        SP::split(acc, s2, pf);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const F yf = col_frag<Tr, RS>(buf + LY::kY, 0, db * 32, s2, lane);
#pragma unroll
          for (int p = 0; p < SP::NS; ++p) st[db] = Tr::mma(pf[p], yf, st[db]);
        }
      }
    }
    // tile tt+1 goes to the other buffer, last read in iteration tt-1
  }

  if (active) {
    float* P = a.part + ((size_t)bh * a.splits + split) * a.M * D;
    float* Pz = a.partz + ((size_t)bh * a.splits + split) * a.M;
    const int f0 = fb * 32;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) P[(size_t)(f0 + crow(r, hh)) * D + db * 32 + l32] = st[db][r];
    const float z = half_sum(zs);
    if (hh == 0) Pz[f0 + l32] = z;
  }
}

// ---------------------------------------------------------------------------
// k_bcombine: fixed-order sum over the splits of a head (8 groups of splits
// per quad of floats, the groups' sums added in order) into
//   rows_hi/rows_lo [BH][M][D] (element type; lo only for bf16),
//   op [BH][M*D] in the apply's operand order (optional),
//   zf [BH][M] float32.
// ---------------------------------------------------------------------------
constexpr int kBSplitGroups = 8;
constexpr int kBQuads = 256 / kBSplitGroups;

template <class E>
struct BOperandOrder {   // same order as the forward apply's state operand
  static constexpr int J = sizeof(E) == 2 ? 8 : 4;
  static constexpr int GF = 2 * J;
  static __device__ __forceinline__ int pos(int f, int d, int D) {
    const int q = f % GF;
    const int slot = sizeof(E) == 2 ? (((q >> 3) << 2) | (q & 3)) : (q & 3);
    return (((f / GF) * 2 + ((f >> 2) & 1)) * D + d) * J + slot;
  }
};

template <class E>
__global__ __launch_bounds__(256) void k_bcombine(const float* part, const float* partz, int splits, int M, int D,
                                                  E* rows_hi, E* rows_lo, E* op, float* zf) {
  __shared__ f32x4 red[kBSplitGroups][kBQuads];
  const int bh = blockIdx.y;
  const int g = threadIdx.x / kBQuads, qi = threadIdx.x % kBQuads;
  const int quad = blockIdx.x * kBQuads + qi;
  const int md4 = M * D / 4, nq = md4 + M / 4;
  const bool active = quad < nq;
  const f32x4* src;
  size_t stride;
  if (quad < md4) {
    src = (const f32x4*)(part + (size_t)bh * splits * M * D) + quad;
    stride = md4;
  } else {
    src = (const f32x4*)(partz + (size_t)bh * splits * M) + (active ? quad - md4 : 0);
    stride = M / 4;
  }
  const int per = (splits + kBSplitGroups - 1) / kBSplitGroups;
  const int s0 = min(splits, g * per), s1 = min(splits, s0 + per);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (active)
    for (int s = s0; s < s1; ++s) acc += src[(size_t)s * stride];
  red[g][qi] = acc;
  __syncthreads();
  if (g != 0 || !active) return;
#pragma unroll
  for (int gg = 1; gg < kBSplitGroups; ++gg) acc += red[gg][qi];
  if (quad < md4) {
    const size_t e0 = (size_t)bh * M * D + (size_t)quad * 4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const E hi = (E)acc[c];
      rows_hi[e0 + c] = hi;
      if (rows_lo) rows_lo[e0 + c] = (E)(acc[c] - (float)hi);
    }
    if (op) {
      const int f = quad * 4 / D, d0 = quad * 4 % D;
#pragma unroll
      for (int c = 0; c < 4; ++c) op[(size_t)bh * M * D + BOperandOrder<E>::pos(f, d0 + c, D)] = (E)acc[c];
    }
  } else {
    *(f32x4*)(zf + (size_t)bh * M + (quad - md4) * 4) = acc;
  }
}

// ---------------------------------------------------------------------------
// k_bside: one wave per 32 tokens (lane = token t, half h), walking all
// feature blocks.  Projection accumulators are P^T[f][t] (rows = features).
//   SIDE_Q: pass 1 accumulates D_t = phi.z + eps and s_t = phi.y (y = M g_t),
//           writes lg_t = log2 D_t and cw_t = -s_t/D_t; pass 2 forms
//           dq_t = (W^T (phi * (y - z s_t/D_t)) - (s_t eps/D_t) q_t) / D_t.
//   SIDE_K: dv_t = dM^T phi,  u = dM v_t + dz,
//           dk_t = W^T (phi * u) - sum_f(phi_f u_f) k_t.
// ---------------------------------------------------------------------------
struct BSideArgs {
  const void* x;          // Q or K
  const void* y;          // G (Q side) or V (K side)
  const void* rows_hi;    // M or dM rows [BH][M][D]
  const void* rows_lo;
  const void* op;         // dM in operand order (K side)
  const float* zf;        // z or dz [BH][M]
  const void* wph;
  const void* wpl;
  const void* wt;         // W^T operand
  void* dx;               // dQ or dK
  void* dy;               // dV (K side)
  float* lg;              // [BH][L] (Q side)
  float* cw;              // [BH][L] (Q side)
  int L, M, H, Hw, tiles_per_head, total;
  float eps;
};

template <class Tr, int D, bool SIDE_Q>
__global__ __launch_bounds__(256) void k_bside(BSideArgs a) {
  using E = typename Tr::elem;
  using F = typename Tr::frag;
  using SP = Bw<Tr>;
  constexpr int NKD = D / Tr::KS;
  constexpr int NDB = D / 32;
  constexpr int NKT = 32 / Tr::KS;
  constexpr int VPS = Tr::VPS;
  constexpr int ES = (int)sizeof(E);
  constexpr int WES = VPS == 8 ? 2 : 4;
  constexpr int NKG = D * WES / 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hh = lane >> 5, l32 = lane & 31;
  const int g = blockIdx.x * 4 + w;
  if (g >= a.total) return;                         // no barriers below
  const int bh = g / a.tiles_per_head, tile = g % a.tiles_per_head;
  const int head = bh % a.H;
  const int nfb = a.M >> 5;
  const int tok = tile * 32 + l32;
  const bool ok = tok < a.L;
  const E* xrow = (const E*)a.x + ((size_t)bh * a.L + (ok ? tok : 0)) * D;
  const E* yrow = (const E*)a.y + ((size_t)bh * a.L + (ok ? tok : 0)) * D;
  const float half_ln_m = 0.5f * logf((float)a.M);

  // this lane's half of its token's row of X (projection type) and of Y
  F xf[NKD], yf[NKD];
  float ss = 0.f;
#pragma unroll
  for (int s = 0; s < NKD; ++s) {
    const int d0 = (D / 2) * hh + VPS * s;
    if constexpr (VPS == 8) {
      const u32x4 xv = ok ? *(const u32x4*)(xrow + d0) : u32x4{0u, 0u, 0u, 0u};
      yf[s] = ok ? *(const u32x4*)(yrow + d0) : u32x4{0u, 0u, 0u, 0u};
      xf[s] = Tr::to_proj(xv);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = bf16_lo(xv[j]), q = bf16_hi(xv[j]);
        ss = fmaf(p, p, fmaf(q, q, ss));
      }
    } else {
      xf[s] = ok ? xrow[d0] : 0.f;
      yf[s] = ok ? yrow[d0] : 0.f;
      ss = fmaf(xf[s], xf[s], ss);
    }
  }
  ss = half_sum(ss);
  const float bias = ok ? -(0.5f * ss + half_ln_m) * kLog2e : -INFINITY;

  const int hw = a.Hw == 1 ? 0 : head;
  const char* wph = (const char*)a.wph + (size_t)hw * nfb * NKG * 2 * 32 * 16;
  const char* wpl = (const char*)a.wpl + (size_t)hw * nfb * NKG * 2 * 32 * 16;
  const E* wt = (const E*)a.wt + (size_t)hw * a.M * D;
  const E* rhi = (const E*)a.rows_hi + (size_t)bh * a.M * D;
  const E* rlo = (const E*)a.rows_lo + (size_t)bh * a.M * D;
  const float* zf = a.zf + (size_t)bh * a.M;

  // phi^T[f][t] of feature block fb (rows f = 32 fb + crow(r, h))
  auto features = [&](int fb) -> f32x16 {
    f32x16 p = zero16();
#pragma unroll
    for (int pp = 0; pp < SP::NS; ++pp) {
      const char* base = (pp == 0 ? wph : wpl) + (size_t)fb * NKG * 2 * 32 * 16;
      if constexpr (WES == 2) {
#pragma unroll
        for (int s = 0; s < NKD; ++s) p = Tr::pmma(*(const u32x4*)(base + ((s * 2 + hh) * 32 + l32) * 16), xf[s], p);
      } else {
#pragma unroll
        for (int gk = 0; gk < NKG; ++gk) {
          const f32x4 v = *(const f32x4*)(base + ((gk * 2 + hh) * 32 + l32) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) p = Tr::pmma(v[j], xf[4 * gk + j], p);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = exp2_fast(p[r] + bias);
    return p;
  };
  // rows-operand product R Y^T for feature block fb (R = M or dM, hi + lo),
  // accumulated onto acc: rows f, lane = token
  auto rows_times_y = [&](int fb, f32x16 acc) -> f32x16 {
    const size_t rb = (size_t)(fb * 32 + l32) * D + (D / 2) * hh;
#pragma unroll
    for (int s = 0; s < NKD; ++s) {
      F rf[SP::NS];
      if constexpr (VPS == 8) {
        rf[0] = *(const u32x4*)(rhi + rb + VPS * s);
        if constexpr (SP::NS == 2) rf[1] = *(const u32x4*)(rlo + rb + VPS * s);
      } else {
        rf[0] = rhi[rb + s];
      }
#pragma unroll
      for (int pp = 0; pp < SP::NS; ++pp) acc = Tr::mma(rf[pp], yf[s], acc);
    }
    return acc;
  };
  // z or dz values of the rows of feature block fb, in accumulator order
  auto zrows = [&](int fb) -> f32x16 {
    f32x16 zr;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v = *(const f32x4*)(zf + fb * 32 + 8 * q4 + 4 * hh);
#pragma unroll
      for (int j = 0; j < 4; ++j) zr[4 * q4 + j] = v[j];
    }
    return zr;
  };
  // acc[db] += W^T gacc (the c-row feature order of gacc)
  auto wt_times = [&](int fb, const f32x16& gacc, f32x16 (&acc)[NDB]) {
#pragma unroll
    for (int s2 = 0; s2 < NKT; ++s2) {
      const F gfr = CFrag<Tr>::make(gacc, s2);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const size_t e = (((((size_t)fb * NKT + s2) * NDB + db) * 2 + hh) * 32 + l32) * VPS;
        F wfr;
        if constexpr (VPS == 8) wfr = *(const u32x4*)(wt + e);
        else wfr = wt[e];
        acc[db] = Tr::mma(wfr, gfr, acc[db]);
      }
    }
  };

  f32x16 dacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dacc[db] = zero16();
  E* drow = (E*)a.dx + ((size_t)bh * a.L + (ok ? tok : 0)) * D;

  if constexpr (SIDE_Q) {
    float den = 0.f, sy = 0.f;
    for (int fb = 0; fb < nfb; ++fb) {
      const f32x16 phi = features(fb);
      const f32x16 zr = zrows(fb);
      const f32x16 y = rows_times_y(fb, zero16());
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        den = fmaf(phi[r], zr[r], den);
        sy = fmaf(phi[r], y[r], sy);
      }
    }
    den = half_sum(den) + a.eps;
    sy = half_sum(sy);
    const float ratio = sy / den;
    if (ok && hh == 0) {
      a.lg[(size_t)bh * a.L + tok] = log2f(den);
      a.cw[(size_t)bh * a.L + tok] = -ratio;
    }
    for (int fb = 0; fb < nfb; ++fb) {
      f32x16 phi = features(fb);
      const f32x16 zr = zrows(fb);
      const f32x16 y = rows_times_y(fb, zero16());
#pragma unroll
      for (int r = 0; r < 16; ++r) phi[r] *= y[r] - zr[r] * ratio;
      wt_times(fb, phi, dacc);
    }
    const float inv = 1.f / den;
    const float rs = sy * a.eps * inv;               // sum_f phi_f (y_f - z_f s/D)
    if (ok) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = db * 32 + 8 * i + 4 * hh;
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = (dacc[db][4 * i + j] - rs * (float)xrow[d0 + j]) * inv;
          if constexpr (ES == 2) {
            *(u32x2*)(drow + d0) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
          } else {
            *(f32x4*)(drow + d0) = f32x4{v[0], v[1], v[2], v[3]};
          }
        }
    }
  } else {
    f32x16 vacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) vacc[db] = zero16();
    const char* opb = (const char*)a.op + (size_t)bh * a.M * D * ES;
    float rs = 0.f;
    for (int fb = 0; fb < nfb; ++fb) {
      f32x16 phi = features(fb);
      // dv^T[d][t] += dM^T phi^T: the state operand in the apply's order
      if constexpr (VPS == 8) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int gi = 2 * fb + s2;
          const F pf = CFrag<Tr>::make(phi, s2);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            vacc[db] = Tr::mma(*(const u32x4*)(opb + ((gi * 2 + hh) * D + db * 32 + l32) * 16), pf, vacc[db]);
        }
      } else {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int gi = 4 * fb + s4;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const f32x4 mf = *(const f32x4*)(opb + ((gi * 2 + hh) * D + db * 32 + l32) * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) vacc[db] = Tr::mma(mf[j], phi[4 * s4 + j], vacc[db]);
          }
        }
      }
      const f32x16 u = rows_times_y(fb, zrows(fb));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        phi[r] *= u[r];
        rs += phi[r];
      }
      wt_times(fb, phi, dacc);
    }
    rs = half_sum(rs);
    if (ok) {
      E* vrow = (E*)a.dy + ((size_t)bh * a.L + tok) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = db * 32 + 8 * i + 4 * hh;
          float v[4], dv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j] = dacc[db][4 * i + j] - rs * (float)xrow[d0 + j];
            dv[j] = vacc[db][4 * i + j];
          }
          if constexpr (ES == 2) {
            *(u32x2*)(drow + d0) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
            *(u32x2*)(vrow + d0) = u32x2{pack_bf16(dv[0], dv[1]), pack_bf16(dv[2], dv[3])};
          } else {
            *(f32x4*)(drow + d0) = f32x4{v[0], v[1], v[2], v[3]};
            *(f32x4*)(vrow + d0) = f32x4{dv[0], dv[1], dv[2], dv[3]};
          }
        }
    }
  }
}

// ===========================================================================
// host side
// ===========================================================================
struct BwdBuffers {
  float *part, *partz, *zf, *lg, *cw;
  void *wph, *wpl, *wt, *rows_hi, *rows_lo, *op;
};

static BwdBuffers bwd_buffers(const Plan& p, char* ws) {
  BwdBuffers b;
  b.part = (float*)(ws + p.boff_part);
  b.partz = (float*)(ws + p.boff_partz);
  b.zf = (float*)(ws + p.boff_zf);
  b.lg = (float*)(ws + p.boff_lg);
  b.cw = (float*)(ws + p.boff_cw);
  b.wph = ws + p.boff_wph;
  b.wpl = ws + p.boff_wpl;
  b.wt = ws + p.boff_wt;
  b.rows_hi = ws + p.boff_rows_hi;
  b.rows_lo = ws + p.boff_rows_lo;
  b.op = ws + p.boff_op;
  return b;
}

template <class Tr, int D>
static hipError_t bwd_noncausal_t(const Plan& p, const BwdTensors& t, hipStream_t s) {
  using E = typename Tr::elem;
  const BwdBuffers b = bwd_buffers(p, t.ws);
  const int nrows = p.Hw * p.M;
  // W operands
  {
    constexpr int WES = Tr::VPS == 8 ? 2 : 4;
    const int n = nrows * D / (16 / WES) + nrows * D / Tr::VPS;
    const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
    timing_begin(FAVOR_KERNEL_BWD_PREP, s);
    hipLaunchKernelGGL((k_bprep<Tr>), dim3(blocks), dim3(256), 0, s, t.w, b.wph, b.wpl, b.wt, nrows, D);
    timing_end(FAVOR_KERNEL_BWD_PREP, s);
  }
  const dim3 rgrid(p.bsplits, p.bfgroups, p.BH);
  const size_t rlds = BRedLds<Tr, D>::kTotal;
  const int nq = (p.M * D + p.M) / 4;
  const dim3 cgrid((nq + kBQuads - 1) / kBQuads, p.BH);
  E* rlo = Tr::VPS == 8 ? (E*)b.rows_lo : nullptr;
  const int tph = (p.L + 31) / 32;
  const int total = p.BH * tph;
  const dim3 sgrid((total + 3) / 4);
  // state M, z from K, V
  {
    BRedArgs a{t.k, t.v, nullptr, nullptr, b.wph, b.wpl, b.part, b.partz, p.L, p.M, p.H, p.Hw, p.bsplits, p.bsplit_len};
    timing_begin(FAVOR_KERNEL_BWD_REDUCE, s);
    hipLaunchKernelGGL((k_bred<Tr, D, false>), rgrid, dim3(256), rlds, s, a);
    timing_end(FAVOR_KERNEL_BWD_REDUCE, s);
    timing_begin(FAVOR_KERNEL_BWD_COMBINE, s);
    hipLaunchKernelGGL((k_bcombine<E>), cgrid, dim3(256), 0, s, b.part, b.partz, p.bsplits, p.M, D, (E*)b.rows_hi, rlo,
                       (E*)nullptr, b.zf);
    timing_end(FAVOR_KERNEL_BWD_COMBINE, s);
  }
  // query side: dQ, and the per-token scale and weight of the next reduction
  {
    BSideArgs a{t.q, t.g, b.rows_hi, b.rows_lo, nullptr, b.zf, b.wph, b.wpl, b.wt, t.dq, nullptr, b.lg, b.cw,
                p.L, p.M, p.H, p.Hw, tph, total, t.eps};
    timing_begin(FAVOR_KERNEL_BWD_Q, s);
    hipLaunchKernelGGL((k_bside<Tr, D, true>), sgrid, dim3(256), 0, s, a);
    timing_end(FAVOR_KERNEL_BWD_Q, s);
  }
  // dM, dz from Q, G
  {
    BRedArgs a{t.q, t.g, b.lg, b.cw, b.wph, b.wpl, b.part, b.partz, p.L, p.M, p.H, p.Hw, p.bsplits, p.bsplit_len};
    timing_begin(FAVOR_KERNEL_BWD_REDUCE, s);
    hipLaunchKernelGGL((k_bred<Tr, D, true>), rgrid, dim3(256), rlds, s, a);
    timing_end(FAVOR_KERNEL_BWD_REDUCE, s);
    timing_begin(FAVOR_KERNEL_BWD_COMBINE, s);
    hipLaunchKernelGGL((k_bcombine<E>), cgrid, dim3(256), 0, s, b.part, b.partz, p.bsplits, p.M, D, (E*)b.rows_hi, rlo,
                       (E*)b.op, b.zf);
    timing_end(FAVOR_KERNEL_BWD_COMBINE, s);
  }
  // key side: dK, dV
  {
    BSideArgs a{t.k, t.v, b.rows_hi, b.rows_lo, b.op, b.zf, b.wph, b.wpl, b.wt, t.dk, t.dv, nullptr, nullptr,
                p.L, p.M, p.H, p.Hw, tph, total, t.eps};
    timing_begin(FAVOR_KERNEL_BWD_K, s);
    hipLaunchKernelGGL((k_bside<Tr, D, false>), sgrid, dim3(256), 0, s, a);
    timing_end(FAVOR_KERNEL_BWD_K, s);
  }
  return hipGetLastError();
}

hipError_t launch_noncausal_bwd(const Plan& p, const BwdTensors& t, hipStream_t s) {
  if (p.dt == FAVOR_BF16) {
    switch (p.D) {
      case 32: return bwd_noncausal_t<TrBF16, 32>(p, t, s);
      case 64: return bwd_noncausal_t<TrBF16, 64>(p, t, s);
      case 128: return bwd_noncausal_t<TrBF16, 128>(p, t, s);
    }
  } else {
    switch (p.D) {
      case 32: return bwd_noncausal_t<TrF32, 32>(p, t, s);
      case 64: return bwd_noncausal_t<TrF32, 64>(p, t, s);
      case 128: return bwd_noncausal_t<TrF32, 128>(p, t, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace favor
