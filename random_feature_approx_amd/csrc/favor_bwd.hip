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
// so they hold about 16 significant bits, and the products of W^T with the
// feature gradients take three products (hi hi, hi lo, lo hi).  dM^T phi(K)
// uses single bf16 operands; accumulation is float32 throughout.
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
__global__ __launch_bounds__(256) void k_bprep(const float* w, void* wph, void* wpl, void* wt, void* wtl, int nrows,
                                               int D, int M, int mt) {
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
      const int R = blk * 32 + f;                      // row of the padded operand (Hw * M rows)
      const bool real = R % M < mt;
      const float* src = w + ((size_t)(R / M) * mt + (real ? R % M : 0)) * D + (D / 2) * h + PER * g;
      const float keep = real ? kLog2e : 0.f;          // rows past m: zero
      if constexpr (WES == 2) {
        unsigned hi[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float a = src[2 * k] * keep, b = src[2 * k + 1] * keep;
          hi[k] = pack_f16(a, b);
          const f16x2 hv = __builtin_bit_cast(f16x2, hi[k]);
          lo[k] = pack_f16(a - (float)hv[0], b - (float)hv[1]);
        }
        ((u32x4*)wph)[idx] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        ((u32x4*)wpl)[idx] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      } else {
        ((f32x4*)wph)[idx] = *(const f32x4*)src * keep;
      }
    } else {
      const int i = idx - nproj;                       // = ((((fbg*NKT + s)*NDB + db)*2 + h)*32 + c)
      const int c = i & 31, h = (i >> 5) & 1;
      int rest = i >> 6;
      const int db = rest % NDB;
      rest /= NDB;
      const int s = rest % NKT, fbg = rest / NKT;      // fbg: feature block over all Hw heads
      E* dst = (E*)wt + (size_t)i * VPS;
      E* dstl = (E*)wtl + (size_t)i * VPS;
#pragma unroll
      for (int j = 0; j < VPS; ++j) {
        const int R = fbg * 32 + crow(VPS * s + j, h);
        const float x = R % M < mt ? w[((size_t)(R / M) * mt + R % M) * D + db * 32 + c] : 0.f;
        const E hi = (E)x;
        dst[j] = hi;
        if (wtl) dstl[j] = (E)(x - (float)hi);         // lo part (bf16)
      }
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
  int mt;                // rows of W per head as given; features past them are padding, phi = 0
};

template <class Tr, int D, int NWR>
struct BRedLds {
  using E = typename Tr::elem;
  // tokens per tile: 64 for eight-wave workgroups (every thread stages one
  // 16-byte chunk per tensor at d = 64), else 32
  static constexpr int TT = NWR == 8 ? 64 : 32;
  static constexpr int RS = Rows<D, sizeof(E)>::RS;
  static constexpr int kX = 0;
  static constexpr int kY = kX + TT * RS;
  static constexpr int kBias = kY + TT * RS;
  static constexpr int kW = kBias + TT * 4;
  static constexpr int BUF = kW + TT * 4;
  static constexpr int kTotal = 2 * BUF;
};

template <class Tr, int D, bool WT, int NW>
__global__ __launch_bounds__(NW * 64) void k_bred(BRedArgs a) {
  constexpr int NT = NW * 64;
  using E = typename Tr::elem;
  using F = typename Tr::frag;
  using LY = BRedLds<Tr, D, NW>;
  constexpr int TT = LY::TT;
  constexpr int NTB = TT / 32;                // 32-token blocks per tile
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
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int nfb = a.M >> 5;
  const int fb = fg * NW + w;
  const bool active = fb < nfb;
  const E* X = (const E*)a.x + (size_t)bh * a.L * D;
  const E* Y = (const E*)a.y + (size_t)bh * a.L * D;
  const float half_ln_m = 0.5f * logf((float)a.mt);

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
  // weighted form: the per-token exponent shift and weight of a tile's rows,
  // loaded with the tile (one tile ahead) by the threads that own the rows
  float plg[TL::NCH], pcw[TL::NCH];
  auto load_tile = [&](int r0) {
    xl.load(X + (size_t)r0 * D, t1 - r0, tid);
    yl.load(Y + (size_t)r0 * D, t1 - r0, tid);
    if constexpr (WT) {
#pragma unroll
      for (int i = 0; i < TL::NCH; ++i) {
        const int c = tid + i * NT, row = c / CPR;
        plg[i] = 0.f;
        pcw[i] = 0.f;
        if (c < TT * CPR && (c % CPR) == 0 && row < t1 - r0) {
          plg[i] = a.lg[(size_t)bh * a.L + r0 + row];
          pcw[i] = a.cw[(size_t)bh * a.L + r0 + row];
        }
      }
    }
  };
  if (ntiles > 0) load_tile(t0);
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
              b -= plg[i];
              wt = pcw[i];
            }
          }
          sb[row] = b;
          sw[row] = wt;
        }
      }
    }
    __syncthreads();
    if (tt + 1 < ntiles) load_tile(r0 + TT);
    if (active) {
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {            // 32-token blocks of the tile
        const float* sb = (const float*)(buf + LY::kBias) + tb * 32;
        const float* sw = (const float*)(buf + LY::kW) + tb * 32;
        f32x16 acc;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 b4 = *(const f32x4*)(sb + 8 * g + 4 * hh);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[4 * g + j] = b4[j];
        }
#pragma unroll
        for (int s = 0; s < NKD; ++s) {
          const F xf = row_frag<Tr, D>(buf + LY::kX + (tb * 32 + l32) * RS, hh, s);
#pragma unroll
          for (int p = 0; p < SP::NS; ++p) acc = Tr::pmma(xf, wf[p][s], acc);   // P[t][f] + bias[t]
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = exp2_fast(acc[r]);
        if (fb * 32 + 32 > a.mt && fb * 32 + l32 >= a.mt) acc = zero16();   // padding feature (lane)
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
            const F yf = col_frag<Tr, RS>(buf + LY::kY, tb * 32, db * 32, s2, lane);
#pragma unroll
            for (int p = 0; p < SP::NS; ++p) st[db] = Tr::mma(pf[p], yf, st[db]);
          }
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
  const void* wt;         // W^T operand (hi)
  const void* wtl;        // W^T operand (lo, bf16)
  void* dx;               // dQ or dK
  void* dy;               // dV (K side)
  float* lg;              // [BH][L] (Q side)
  float* cw;              // [BH][L] (Q side)
  int L, M, H, Hw, tiles_per_head, total;
  float eps;
  int mt;                 // rows of W per head as given; features past them are padding, phi = 0
};

// Work split of the per-token side: TB 32-token blocks per wave and NWB
// waves per workgroup (sharing each LDS image), compiled for bside_waves
// waves per SIMD.  bf16 at d <= 64: one block per wave, eight waves, two per
// SIMD on both sides (no spills; measured on the long workload against two
// blocks per wave in four-wave workgroups: query side 244 -> 226 us, key
// side 225 -> 193 us); elsewhere the register file holds one wave per SIMD.
template <class Tr, int D, bool SIDE_Q>
constexpr int bside_waves() { return (Tr::VPS == 8 && D <= 64) ? 2 : 1; }
template <class Tr, int D>
constexpr int bside_tb() { return 1; }
template <class Tr, int D>
constexpr int bside_nwb() { return (Tr::VPS == 8 && D <= 64) ? 8 : 4; }

// The per-head operands of one 32-feature block, as one workgroup's LDS
// image (16-byte chunks, each region in the order its fragments are read:
// chunk q of lane l at q * 64 + l): the projection operand (hi, lo parts),
// the rows of M or dM (hi, lo), z or dz, dM in the apply's operand order (key
// side) and the W^T operand (hi, lo).  The four waves of a workgroup work on
// one head; the image of block fb + 1 is copied (global -> LDS) while block
// fb is used.
template <class Tr, int D, bool SIDE_Q>
struct BSideImg {
  static constexpr int ES = (int)sizeof(typename Tr::elem);
  static constexpr int NS = Bw<Tr>::NS;
  static constexpr int WES = Tr::VPS == 8 ? 2 : 4;
  static constexpr int NKT = 32 / Tr::KS, NDB = D / 32;
  static constexpr int CWP = (D * WES / 32) * 64;             // projection operand, per part
  static constexpr int RQ = (D / 2) * ES / 16;                // row chunks per lane
  static constexpr int CR = RQ * 64;                          // rows, per part
  static constexpr int CZ = 8;                                // 32 floats
  static constexpr int COP = SIDE_Q ? 0 : (Tr::VPS == 8 ? 2 : 4) * 2 * D;
  static constexpr int CWT = NKT * NDB * 64 * Tr::VPS * ES / 16;   // W^T operand, per part
  static constexpr int kWp = 0, kR = kWp + NS * CWP, kZ = kR + NS * CR, kOp = kZ + CZ, kWt = kOp + COP;
  static constexpr int CHUNKS = kWt + NS * CWT;
  static constexpr int BYTES = CHUNKS * 16;
  // blocks per step of the walk (one barrier per step): two where four images
  // fit the LDS, else one
  static constexpr int G = 4 * BYTES <= 150 * 1024 ? 2 : 1;
  static constexpr int LDS = 2 * G * BYTES;
};

template <class Tr, int D, bool SIDE_Q, int TB, int NWB>
__global__ __launch_bounds__(NWB * 64, (bside_waves<Tr, D, SIDE_Q>() * 4 >= NWB ? bside_waves<Tr, D, SIDE_Q>() * 4 / NWB : 1)) void k_bside(BSideArgs a) {
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
  using IMG = BSideImg<Tr, D, SIDE_Q>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  // workgroup = NWB consecutive groups of TB x 32 tokens of one head; waves
  // past the head's last group take part in the copies and barriers only
  const int wgs_per_head = (a.tiles_per_head + NWB - 1) / NWB;
  const int bh = blockIdx.x / wgs_per_head, tile = (blockIdx.x % wgs_per_head) * NWB + w;
  const bool active = tile < a.tiles_per_head;
  const int head = bh % a.H;
  const int nfb = a.M >> 5;
  const float half_ln_m = 0.5f * logf((float)a.mt);

  // this lane's half of its tokens' rows of X (projection type) and of Y
  int tok[TB];
  bool ok[TB];
  const E* xrow[TB];
  F xf[TB][NKD], yf[TB][NKD];
  float bias[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    tok[tb] = (tile * TB + tb) * 32 + l32;
    ok[tb] = tok[tb] < a.L;
    xrow[tb] = (const E*)a.x + ((size_t)bh * a.L + (ok[tb] ? tok[tb] : 0)) * D;
    const E* yrow = (const E*)a.y + ((size_t)bh * a.L + (ok[tb] ? tok[tb] : 0)) * D;
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < NKD; ++s) {
      const int d0 = (D / 2) * hh + VPS * s;
      if constexpr (VPS == 8) {
        const u32x4 xv = ok[tb] ? *(const u32x4*)(xrow[tb] + d0) : u32x4{0u, 0u, 0u, 0u};
        yf[tb][s] = ok[tb] ? *(const u32x4*)(yrow + d0) : u32x4{0u, 0u, 0u, 0u};
        xf[tb][s] = Tr::to_proj(xv);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = bf16_lo(xv[j]), q = bf16_hi(xv[j]);
          ss = fmaf(p, p, fmaf(q, q, ss));
        }
      } else {
        xf[tb][s] = ok[tb] ? xrow[tb][d0] : 0.f;
        yf[tb][s] = ok[tb] ? yrow[d0] : 0.f;
        ss = fmaf(xf[tb][s], xf[tb][s], ss);
      }
    }
    ss = half_sum(ss);
    bias[tb] = ok[tb] ? -(0.5f * ss + half_ln_m) * kLog2e : -INFINITY;
  }

  const int hw = a.Hw == 1 ? 0 : head;
  const char* wph = (const char*)a.wph + (size_t)hw * nfb * NKG * 2 * 32 * 16;
  const char* wpl = (const char*)a.wpl + (size_t)hw * nfb * NKG * 2 * 32 * 16;
  const E* wt = (const E*)a.wt + (size_t)hw * a.M * D;
  const E* wtlo = (const E*)a.wtl + (size_t)hw * a.M * D;
  const E* rhi = (const E*)a.rows_hi + (size_t)bh * a.M * D;
  const E* rlo = (const E*)a.rows_lo + (size_t)bh * a.M * D;
  const float* zf = a.zf + (size_t)bh * a.M;

  const char* opb = SIDE_Q ? nullptr : (const char*)a.op + (size_t)bh * a.M * D * ES;
  // ---- the LDS image of feature block fb: copy, then fragment reads --------
  // images by position in the walk (not by fb: the query side walks the
  // blocks twice): IMG::G consecutive blocks form a step, steps alternate
  // between two sets of buffers
  constexpr int G = IMG::G;
  auto img = [&](int it) -> char* { return smem + (((it / G) & 1) * G + it % G) * IMG::BYTES; };
  auto copy_region = [&](char* dst, int nchunks, auto src_of) {
    for (int c0 = w * 64; c0 < nchunks; c0 += NWB * 64) {
      const int c = c0 + lane;
      if (c < nchunks) __builtin_amdgcn_global_load_lds(FAVOR_GLB(src_of(c)), LDS_PTR(void, dst + c0 * 16), 16, 0, 0);
    }
  };
  auto copy_image = [&](int fb, int step, bool with_wt) {
    char* im = img(step);
#pragma unroll
    for (int pp = 0; pp < SP::NS; ++pp) {
      const char* wsrc = (pp == 0 ? wph : wpl) + (size_t)fb * IMG::CWP * 16;
      copy_region(im + (IMG::kWp + pp * IMG::CWP) * 16, IMG::CWP, [&](int c) { return wsrc + (size_t)c * 16; });
      const char* rsrc = (const char*)(pp == 0 ? rhi : rlo) + (size_t)fb * 32 * D * ES;
      copy_region(im + (IMG::kR + pp * IMG::CR) * 16, IMG::CR, [&](int c) {
        const int q = c >> 6, ln = c & 63;            // chunk q of lane ln = (row, half)
        return rsrc + (size_t)(ln & 31) * D * ES + (D / 2) * (ln >> 5) * ES + q * 16;
      });
    }
    const char* zsrc = (const char*)(zf + fb * 32);
    copy_region(im + IMG::kZ * 16, IMG::CZ, [&](int c) { return zsrc + (size_t)c * 16; });
    if constexpr (!SIDE_Q) {
      const char* osrc = opb + (size_t)fb * IMG::COP * 16;
      copy_region(im + IMG::kOp * 16, IMG::COP, [&](int c) { return osrc + (size_t)c * 16; });
    }
    if (with_wt) {
#pragma unroll
      for (int pp = 0; pp < SP::NS; ++pp) {
        const char* tsrc = (const char*)(pp == 0 ? wt : wtlo) + (size_t)fb * IMG::CWT * 16;
        copy_region(im + (IMG::kWt + pp * IMG::CWT) * 16, IMG::CWT, [&](int c) { return tsrc + (size_t)c * 16; });
      }
    }
  };
  // projection operand of block fb (hi, lo)
  auto wproj = [&](const char* im, F (&wfr)[SP::NS][NKD]) {
#pragma unroll
    for (int pp = 0; pp < SP::NS; ++pp) {
      const char* base = im + (IMG::kWp + pp * IMG::CWP) * 16;
      if constexpr (WES == 2) {
#pragma unroll
        for (int s = 0; s < NKD; ++s) wfr[pp][s] = *(const u32x4*)(base + (s * 64 + lane) * 16);
      } else {
#pragma unroll
        for (int gk = 0; gk < NKG; ++gk) {
          const f32x4 v = *(const f32x4*)(base + (gk * 64 + lane) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) wfr[pp][4 * gk + j] = v[j];
        }
      }
    }
  };
  // rows operand (M or dM, hi + lo) of block fb: lane (f, h) holds row f,
  // elements (D/2) h + 0 ..
  auto rows = [&](const char* im, F (&rf)[SP::NS][NKD]) {
#pragma unroll
    for (int pp = 0; pp < SP::NS; ++pp) {
      const char* base = im + (IMG::kR + pp * IMG::CR) * 16;
      if constexpr (VPS == 8) {
#pragma unroll
        for (int s = 0; s < NKD; ++s) rf[pp][s] = *(const u32x4*)(base + (s * 64 + lane) * 16);
      } else {
#pragma unroll
        for (int q = 0; q < IMG::RQ; ++q) {
          const f32x4 v = *(const f32x4*)(base + (q * 64 + lane) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) rf[pp][4 * q + j] = v[j];
        }
      }
    }
  };
  // phi^T[f][t] of block fb for token block tb (rows f = 32 fb + crow(r, h));
  // padding features (rows of W past m) are zero
  auto features = [&](const F (&wfr)[SP::NS][NKD], int tb, int fb) -> f32x16 {
    f32x16 p = zero16();
#pragma unroll
    for (int s = 0; s < NKD; ++s)
#pragma unroll
      for (int pp = 0; pp < SP::NS; ++pp) p = Tr::pmma(wfr[pp][s], xf[tb][s], p);
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = exp2_fast(p[r] + bias[tb]);
    if (fb * 32 + 32 > a.mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (fb * 32 + crow(r, hh) >= a.mt) p[r] = 0.f;
    }
    return p;
  };
  auto rows_times_y = [&](const F (&rf)[SP::NS][NKD], int tb, f32x16 acc) -> f32x16 {
#pragma unroll
    for (int s = 0; s < NKD; ++s)
#pragma unroll
      for (int pp = 0; pp < SP::NS; ++pp) acc = Tr::mma(rf[pp][s], yf[tb][s], acc);
    return acc;
  };
  // z or dz values of the rows of feature block fb, in accumulator order
  auto zrows = [&](const char* im) -> f32x16 {
    f32x16 zr;
    const float* zl = (const float*)(im + IMG::kZ * 16);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v = *(const f32x4*)(zl + 8 * q4 + 4 * hh);
#pragma unroll
      for (int j = 0; j < 4; ++j) zr[4 * q4 + j] = v[j];
    }
    return zr;
  };
  // acc[tb][db] += W^T gacc[tb] (c-row feature order), both operands split
  // into hi + lo (three products: hi hi, hi lo, lo hi)
  auto wt_times = [&](const char* im, const f32x16 (&gacc)[TB], f32x16 (&acc)[TB][NDB]) {
#pragma unroll
    for (int s2 = 0; s2 < NKT; ++s2) {
      F gfr[TB][SP::NS];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) SP::split(gacc[tb], s2, gfr[tb]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int e = ((s2 * NDB + db) * 64 + lane) * VPS;   // element within the part
        F wfr[SP::NS];
#pragma unroll
        for (int pp = 0; pp < SP::NS; ++pp)
          wfr[pp] = *(const F*)(im + (IMG::kWt + pp * IMG::CWT) * 16 + e * ES);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          acc[tb][db] = Tr::mma(wfr[0], gfr[tb][0], acc[tb][db]);
          if constexpr (SP::NS == 2) {
            acc[tb][db] = Tr::mma(wfr[0], gfr[tb][1], acc[tb][db]);
            acc[tb][db] = Tr::mma(wfr[1], gfr[tb][0], acc[tb][db]);
          }
        }
      }
    }
  };
  // the input row's values at this lane's output columns d = 32 db + 8 i + 4 h
  // + j, all requested before any output is stored (the stores could alias
  // the input as far as the compiler knows, so loads between them would each
  // wait for a full memory round trip)
  auto x_at_outputs = [&](int tb, float (&xo)[NDB][4][4]) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const E* src = xrow[tb] + db * 32 + 8 * i + 4 * hh;
        if constexpr (ES == 2) {
          const u32x2 x2 = *(const u32x2*)src;
          xo[db][i][0] = bf16_lo(x2[0]);
          xo[db][i][1] = bf16_hi(x2[0]);
          xo[db][i][2] = bf16_lo(x2[1]);
          xo[db][i][3] = bf16_hi(x2[1]);
        } else {
          const f32x4 x4 = *(const f32x4*)src;
#pragma unroll
          for (int j = 0; j < 4; ++j) xo[db][i][j] = x4[j];
        }
      }
  };
  // store 16 values of a d^T accumulator for token block tb (columns d0..d0+3)
  auto store4 = [&](E* row, int d0, const float (&v)[4]) {
    if constexpr (ES == 2) {
      *(u32x2*)(row + d0) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    } else {
      *(f32x4*)(row + d0) = f32x4{v[0], v[1], v[2], v[3]};
    }
  };

  f32x16 dacc[TB][NDB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) dacc[tb][db] = zero16();

  // one step of the block walk: the image of block fb is complete and every
  // wave is done with the other buffer, whose next image is then requested
  // the images of the blocks of step g (positions g G .. g G + G - 1)
  auto copy_step = [&](int g, int nit, auto want_wt) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int it = g * G + i;
      if (it < nit) copy_image(it % nfb, it, want_wt(it));
    }
  };
  // at the first block of a step: its images are complete (own copies waited
  // for, everyone's after the barrier) and every wave is done with the other
  // set of buffers, into which the next step's images are then requested
  auto next_image = [&](int it, int nit, auto want_wt) -> const char* {
    if (it % G == 0) {
      wait_vmcnt<0>();
      raw_barrier();
      copy_step(it / G + 1, nit, want_wt);
    }
    return img(it);
  };
  if constexpr (SIDE_Q) {
    float den[TB], sy[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) den[tb] = sy[tb] = 0.f;
    // two walks over the blocks (den and s, then dq); W^T only in the second
    auto want_wt = [&](int it) { return it >= nfb; };
    copy_step(0, 2 * nfb, want_wt);
    for (int fb = 0; fb < nfb; ++fb) {
      const char* im = next_image(fb, 2 * nfb, want_wt);
      if (!active) continue;
      F wfr[SP::NS][NKD], rf[SP::NS][NKD];
      wproj(im, wfr);
      rows(im, rf);
      const f32x16 zr = zrows(im);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const f32x16 phi = features(wfr, tb, fb);
        const f32x16 y = rows_times_y(rf, tb, zero16());
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          den[tb] = fmaf(phi[r], zr[r], den[tb]);
          sy[tb] = fmaf(phi[r], y[r], sy[tb]);
        }
      }
    }
    float ratio[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      den[tb] = half_sum(den[tb]) + a.eps;
      sy[tb] = half_sum(sy[tb]);
      ratio[tb] = sy[tb] / den[tb];
      if (active && ok[tb] && hh == 0) {
        a.lg[(size_t)bh * a.L + tok[tb]] = log2f(den[tb]);
        a.cw[(size_t)bh * a.L + tok[tb]] = -ratio[tb];
      }
    }
    for (int fb = 0; fb < nfb; ++fb) {
      const char* im = next_image(nfb + fb, 2 * nfb, want_wt);
      if (!active) continue;
      F wfr[SP::NS][NKD], rf[SP::NS][NKD];
      wproj(im, wfr);
      rows(im, rf);
      const f32x16 zr = zrows(im);
      f32x16 gq[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        gq[tb] = features(wfr, tb, fb);
        const f32x16 y = rows_times_y(rf, tb, zero16());
#pragma unroll
        for (int r = 0; r < 16; ++r) gq[tb][r] *= y[r] - zr[r] * ratio[tb];
      }
      wt_times(im, gq, dacc);
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      if (!active || !ok[tb]) continue;
      const float inv = 1.f / den[tb];
      const float rs = sy[tb] * a.eps * inv;           // sum_f phi_f (y_f - z_f s/D)
      E* drow = (E*)a.dx + ((size_t)bh * a.L + tok[tb]) * D;
      float xo[NDB][4][4];
      x_at_outputs(tb, xo);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = db * 32 + 8 * i + 4 * hh;
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = (dacc[tb][db][4 * i + j] - rs * xo[db][i][j]) * inv;
          store4(drow, d0, v);
        }
    }
  } else {
    f32x16 vacc[TB][NDB];
    float rs[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      rs[tb] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) vacc[tb][db] = zero16();
    }
    auto all_wt = [](int) { return true; };
    copy_step(0, nfb, all_wt);
    for (int fb = 0; fb < nfb; ++fb) {
      const char* im = next_image(fb, nfb, all_wt);
      if (!active) continue;
      const char* opl = im + IMG::kOp * 16;             // dM, operand order, this block
      F wfr[SP::NS][NKD], rf[SP::NS][NKD];
      wproj(im, wfr);
      rows(im, rf);
      const f32x16 zr = zrows(im);
      f32x16 gk[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) gk[tb] = features(wfr, tb, fb);
      // dv^T[d][t] += dM^T phi^T: the state operand in the apply's order
      if constexpr (VPS == 8) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const F mf = *(const u32x4*)(opl + ((s2 * 2 + hh) * D + db * 32 + l32) * 16);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) vacc[tb][db] = Tr::mma(mf, CFrag<Tr>::make(gk[tb], s2), vacc[tb][db]);
          }
        }
      } else {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const f32x4 mf = *(const f32x4*)(opl + ((s4 * 2 + hh) * D + db * 32 + l32) * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int tb = 0; tb < TB; ++tb) vacc[tb][db] = Tr::mma(mf[j], gk[tb][4 * s4 + j], vacc[tb][db]);
          }
        }
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const f32x16 u = rows_times_y(rf, tb, zr);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          gk[tb][r] *= u[r];
          rs[tb] += gk[tb][r];
        }
      }
      wt_times(im, gk, dacc);
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const float rsum = half_sum(rs[tb]);
      if (!active || !ok[tb]) continue;
      E* drow = (E*)a.dx + ((size_t)bh * a.L + tok[tb]) * D;
      E* vrow = (E*)a.dy + ((size_t)bh * a.L + tok[tb]) * D;
      float xo[NDB][4][4];
      x_at_outputs(tb, xo);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = db * 32 + 8 * i + 4 * hh;
          float v[4], dv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v[j] = dacc[tb][db][4 * i + j] - rsum * xo[db][i][j];
            dv[j] = vacc[tb][db][4 * i + j];
          }
          store4(drow, d0, v);
          store4(vrow, d0, dv);
        }
    }
  }
}

// ===========================================================================
// host side
// ===========================================================================
struct BwdBuffers {
  float *part, *partz, *zf, *lg, *cw, *acc;
  void *wph, *wpl, *wt, *wtl, *rows_hi, *rows_lo, *op;
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
  b.wtl = ws + p.boff_wtl;
  b.acc = (float*)(ws + p.boff_acc);
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
    hipLaunchKernelGGL((k_bprep<Tr>), dim3(blocks), dim3(256), 0, s, t.w, b.wph, b.wpl, b.wt,
                       Tr::VPS == 8 ? b.wtl : nullptr, nrows, D, p.M, p.mt);
    timing_end(FAVOR_KERNEL_BWD_PREP, s);
  }
  // reduction workgroups: one wave per feature block, the plan's brnw blocks
  // (eight only for bf16 at d <= 64)
  constexpr bool kRed8 = Tr::VPS == 8 && D <= 64;
  if (p.brnw != 4 && !(kRed8 && p.brnw == 8)) return kErrPlan;
  const dim3 rgrid(p.bsplits, p.bfgroups, p.BH);
  constexpr size_t rlds8 = BRedLds<Tr, D, 8>::kTotal, rlds4 = BRedLds<Tr, D, 4>::kTotal;
  auto launch_bred = [&]<bool WT>(const BRedArgs& ra) {
    if constexpr (kRed8) {
      if (p.brnw == 8) {
        hipLaunchKernelGGL((k_bred<Tr, D, WT, 8>), rgrid, dim3(512), rlds8, s, ra);
        return;
      }
    }
    hipLaunchKernelGGL((k_bred<Tr, D, WT, 4>), rgrid, dim3(256), rlds4, s, ra);
  };
  const int nq = (p.M * D + p.M) / 4;
  const dim3 cgrid((nq + kBQuads - 1) / kBQuads, p.BH);
  E* rlo = Tr::VPS == 8 ? (E*)b.rows_lo : nullptr;
  // per-token side: TB 32-token blocks per wave share each operand read,
  // NWB groups of one head per workgroup
  constexpr int TB = bside_tb<Tr, D>(), NWB = bside_nwb<Tr, D>();
  const int tph = (p.L + 32 * TB - 1) / (32 * TB);
  const int total = p.BH * tph;
  const dim3 sgrid(p.BH * ((tph + NWB - 1) / NWB));
  // state M, z from K, V
  {
    BRedArgs a{t.k, t.v, nullptr, nullptr, b.wph, b.wpl, b.part, b.partz, p.L, p.M, p.H, p.Hw, p.bsplits, p.bsplit_len, p.mt};
    timing_begin(FAVOR_KERNEL_BWD_REDUCE, s);
    launch_bred.template operator()<false>(a);
    timing_end(FAVOR_KERNEL_BWD_REDUCE, s);
    timing_begin(FAVOR_KERNEL_BWD_COMBINE, s);
    hipLaunchKernelGGL((k_bcombine<E>), cgrid, dim3(256), 0, s, b.part, b.partz, p.bsplits, p.M, D, (E*)b.rows_hi, rlo,
                       (E*)nullptr, b.zf);
    timing_end(FAVOR_KERNEL_BWD_COMBINE, s);
  }
  // query side: dQ, and the per-token scale and weight of the next reduction
  {
    BSideArgs a{t.q, t.g, b.rows_hi, b.rows_lo, nullptr, b.zf, b.wph, b.wpl, b.wt, b.wtl, t.dq, nullptr, b.lg, b.cw,
                p.L, p.M, p.H, p.Hw, tph, total, t.eps, p.mt};
    timing_begin(FAVOR_KERNEL_BWD_Q, s);
    constexpr size_t lds = BSideImg<Tr, D, true>::LDS;
    hipLaunchKernelGGL((k_bside<Tr, D, true, TB, NWB>), sgrid, dim3(NWB * 64), lds, s, a);
    timing_end(FAVOR_KERNEL_BWD_Q, s);
  }
  // dM, dz from Q, G
  {
    BRedArgs a{t.q, t.g, b.lg, b.cw, b.wph, b.wpl, b.part, b.partz, p.L, p.M, p.H, p.Hw, p.bsplits, p.bsplit_len, p.mt};
    timing_begin(FAVOR_KERNEL_BWD_REDUCE, s);
    launch_bred.template operator()<true>(a);
    timing_end(FAVOR_KERNEL_BWD_REDUCE, s);
    timing_begin(FAVOR_KERNEL_BWD_COMBINE, s);
    hipLaunchKernelGGL((k_bcombine<E>), cgrid, dim3(256), 0, s, b.part, b.partz, p.bsplits, p.M, D, (E*)b.rows_hi, rlo,
                       (E*)b.op, b.zf);
    timing_end(FAVOR_KERNEL_BWD_COMBINE, s);
  }
  // key side: dK, dV
  {
    BSideArgs a{t.k, t.v, b.rows_hi, b.rows_lo, b.op, b.zf, b.wph, b.wpl, b.wt, b.wtl, t.dk, t.dv, nullptr, nullptr,
                p.L, p.M, p.H, p.Hw, tph, total, t.eps, p.mt};
    timing_begin(FAVOR_KERNEL_BWD_K, s);
    constexpr size_t lds = BSideImg<Tr, D, false>::LDS;
    hipLaunchKernelGGL((k_bside<Tr, D, false, TB, NWB>), sgrid, dim3(NWB * 64), lds, s, a);
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
  return kErrPlan;
}

// ===========================================================================
// Causal backward.
//
// With S_i = sum_{j<=i} phi(k_j) v_j^T and z_i = sum_{j<=i} phi(k_j) (the
// prefix sums of case 2 of the performer-2020 study notes), the query side is
// the non-causal one with M, z replaced by S_i, z_i:
//   y_i = S_i g_i,  s_i = phi(q_i).y_i,  D_i = phi(q_i).z_i + eps,
//   dq_i = (A1_i - (s_i/D_i) A2_i - (s_i eps/D_i) q_i) / D_i,
//   A1_i = W^T (phi(q_i) * y_i),  A2_i = W^T (phi(q_i) * z_i);
// the key side uses the suffix sums that the notes' pitfalls section says the
// backward must accumulate in reverse:
//   R_j = sum_{i>=j} phi(q_i) g_i^T / D_i,  r_j = sum_{i>=j} phi(q_i) c_i / D_i,
//   c_i = -s_i/D_i,  dv_j = R_j^T phi(k_j),  dphi(k_j) = R_j v_j + r_j.
// Both sides walk 32-token chunks of a span (one workgroup per span and
// head, one 32-feature block per wave -- eight waves for the bf16 query walks
// at d <= 64, four otherwise -- feature groups in turn),
// starting from the span's exclusive prefix (query side) or suffix (key side)
// of the span aggregates.  Inside a chunk the masked token-by-token terms are
// matrix products with the chunk's 32 x 32 score-like tiles.  The query side
// forms A1 and A2 separately (one pass over the features) with three-term
// split products (hi*hi + hi*lo + lo*hi), which keeps the difference
// A1 - (s/D) A2 accurate; the contributions of the waves and feature groups
// are summed in a fixed order.
// ===========================================================================

// exclusive scan over the spans of a head, in place, one thread per quad of
// floats walking the spans in order: forward a[s] <- sum_{s'<s} a[s'], or
// reverse a[s] <- sum_{s'>s} a[s']
__global__ __launch_bounds__(256) void k_bscan(float* part, float* partz, int spans, int M, int D, int reverse) {
  const int bh = blockIdx.y;
  const int quad = blockIdx.x * 256 + threadIdx.x;
  const int md4 = M * D / 4, nq = md4 + M / 4;
  if (quad >= nq) return;
  f32x4* p;
  size_t stride;
  if (quad < md4) {
    p = (f32x4*)(part + (size_t)bh * spans * M * D) + quad;
    stride = md4;
  } else {
    p = (f32x4*)(partz + (size_t)bh * spans * M) + (quad - md4);
    stride = M / 4;
  }
  // eight spans' loads issued together, then their prefixes stored (a load
  // after a store to the same array would wait for the store's round trip)
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 run = zero;
  for (int k0 = 0; k0 < spans; k0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + j, sp = reverse ? spans - 1 - k : k;
      v[j] = k < spans ? p[(size_t)sp * stride] : zero;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + j, sp = reverse ? spans - 1 - k : k;
      if (k < spans) {
        p[(size_t)sp * stride] = run;
        run += v[j];
      }
    }
  }
}

// DP consecutive values of an output row (16-byte aligned) in 16-byte stores,
// each value rounded to E as a scalar conversion would
template <class E, int DP>
__device__ __forceinline__ void store_row(E* dst, const float (&v)[DP]) {
  if constexpr (sizeof(E) == 2 && DP == 4) {
    E h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (E)v[e];
    *(u32x2*)dst = __builtin_bit_cast(u32x2, h);
  } else if constexpr (sizeof(E) == 2) {
    static_assert(DP % 8 == 0, "whole 16-byte groups");
#pragma unroll
    for (int j = 0; j < DP; j += 8) {
      E h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (E)v[j + e];
      *(u32x4*)(dst + j) = __builtin_bit_cast(u32x4, h);
    }
  } else {
    static_assert(DP % 4 == 0, "whole 16-byte groups");
#pragma unroll
    for (int j = 0; j < DP; j += 4) *(f32x4*)(dst + j) = f32x4{v[j], v[j + 1], v[j + 2], v[j + 3]};
  }
}

// TileLoader::row_bias with a per-row amount subtracted from the FAVOR+ bias
// of each valid row: shift[i] belongs to the row of the thread's chunk i (used
// where the thread holds chunk 0 of the row); rows at or past nvalid get -inf.
template <class E, int D, int TT, int NT>
__device__ __forceinline__ void row_bias_shifted(const TileLoader<E, D, TT, NT>& t, float* sb, int tid, int nvalid,
                                                 float half_ln_m, const float (&shift)[TileLoader<E, D, TT, NT>::NCH]) {
  using TL = TileLoader<E, D, TT, NT>;
  constexpr int CPR = TL::CPR;
#pragma unroll
  for (int i = 0; i < TL::NCH; ++i) {
    const int c = tid + i * NT;
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (sizeof(E) == 2) {
        const float a = bf16_lo(t.r[i][j]), b = bf16_hi(t.r[i][j]);
        ss = fmaf(a, a, ss);
        ss = fmaf(b, b, ss);
      } else {
        const float a = as_f32(t.r[i][j]);
        ss = fmaf(a, a, ss);
      }
    }
    ss = group_sum<CPR>(ss);
    const int row = c / CPR;
    if (c < TT * CPR && (c % CPR) == 0)
      sb[row] = row < nvalid ? FMap<FM_POS>::row_bias(ss, half_ln_m) - shift[i] : -INFINITY;
  }
}

struct BCausalArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* wph;       // projection operand (hi; or the float operand)
  const void* wpl;       // lo (bf16)
  const void* wth;       // W^T operand (hi)
  const void* wtl;       // W^T operand (lo, bf16)
  const float* pre;      // [BH][spans][M][D] exclusive span prefix (query side) or suffix (key side)
  const float* prez;     // [BH][spans][M]
  const float* lg;       // key side: log2 D_i [BH][L]
  const float* cw;       // key side: c_i [BH][L]
  float* lg_out;         // query side outputs
  float* cw_out;
  void* dx;              // dQ (query side) or dK (key side)
  void* dy;              // dV (key side)
  float* acc;            // [BH][L][2D+2] sums carried between feature groups
  int L, M, H, Hw, spans, span_len, fgroups;
  float eps;
  int mt;                // rows of W per head as given; features past them are padding, phi = 0
};

template <class Tr, int D, int NW, bool KEY = false>
struct BCLds {
  using E = typename Tr::elem;
  static constexpr int C = 32;
  static constexpr int RS = Rows<D, sizeof(E)>::RS;
  static constexpr int RSR = D + 4;                     // reduction rows (floats)
  static constexpr int kQ = 0, kK = C * RS, kV = 2 * C * RS, kG = 3 * C * RS;
  static constexpr int kBq = 4 * C * RS, kBk = kBq + C * 4, kC = kBk + C * 4;
  static constexpr int kZ = kC + C * 4;                 // per wave: 32 floats (z or r of its features)
  static constexpr int kRed = kZ + NW * 32 * 4;         // per wave: C x RSR floats
  static constexpr int kRedS = kRed + NW * C * RSR * 4; // per wave: C x 2 floats
  static constexpr int kBase = kRedS + NW * C * 2 * 4;
  // per wave, where it fits next to the rest: the W^T operand fragments of the
  // wave's feature block, [NKT k-steps][NDB d blocks][hi, lo][64 lanes],
  // copied once per feature group, so that the chunk loop reads them from LDS
  // (global loads there would share the in-order load counter with the next
  // chunk's tile prefetch, and waiting for them would wait for the prefetch)
  static constexpr int WTF = (32 / Tr::KS) * (D / 32) * Bw<Tr>::NS;   // fragments per wave
  static constexpr int WTB = WTF * 64 * (int)sizeof(typename Tr::frag);
  static constexpr bool kStageWt = kBase + NW * WTB <= 160 * 1024;
  static constexpr int kWt = kBase;
  static constexpr int kEndWt = kBase + (kStageWt ? NW * WTB : 0);
  // key side, where it fits: a second reduction buffer, so that both per-token
  // outputs (dk, dv) are summed over the waves after one barrier
  static constexpr bool kRed2 = KEY && kEndWt + NW * C * RSR * 4 <= 160 * 1024;
  static constexpr int kRedB = kEndWt;
  static constexpr int kTotal = kEndWt + (kRed2 ? NW * C * RSR * 4 : 0);
};

// B operand over d in c-row order (k-step s2 of d block db) from one row of
// a staged [token][d] tile: d = 32 db + crow(VPS s2 + j, h)
template <class Tr>
__device__ __forceinline__ typename Tr::frag crow_frag(const char* row, int db, int s2, int hh) {
  if constexpr (Tr::VPS == 8) {
    const char* p = row + (32 * db + 16 * s2 + 4 * hh) * 2;
    const u32x2 a = *(const u32x2*)p, b = *(const u32x2*)(p + 16);
    return u32x4{a[0], a[1], b[0], b[1]};
  } else {
    return *(const float*)(row + (32 * db + crow(s2, hh)) * 4);
  }
}

// constant operand [k][n] of k-step s: 1 where pred(k = crow(VPS s + j, h), n = lane) holds
template <class Tr, class P>
__device__ __forceinline__ typename Tr::frag const_frag(int s, int lane, P pred) {
  const int hh = lane >> 5, n = lane & 31;
  if constexpr (Tr::VPS == 8) {
    u32x4 f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned lo = pred(crow(8 * s + 2 * k, hh), n) ? 0x3f80u : 0u;
      const unsigned hi = pred(crow(8 * s + 2 * k + 1, hh), n) ? 0x3f800000u : 0u;
      f[k] = lo | hi;
    }
    return f;
  } else {
    return pred(crow(s, hh), n) ? 1.f : 0.f;
  }
}

// products with split operands: a (split) x b, a x b (split), a x b (both split)
template <class Tr>
__device__ __forceinline__ f32x16 mma_sa(const typename Tr::frag (&a)[Bw<Tr>::NS], typename Tr::frag b, f32x16 c) {
#pragma unroll
  for (int p = 0; p < Bw<Tr>::NS; ++p) c = Tr::mma(a[p], b, c);
  return c;
}
template <class Tr>
__device__ __forceinline__ f32x16 mma_sb(typename Tr::frag a, const typename Tr::frag (&b)[Bw<Tr>::NS], f32x16 c) {
#pragma unroll
  for (int p = 0; p < Bw<Tr>::NS; ++p) c = Tr::mma(a, b[p], c);
  return c;
}
template <class Tr>
__device__ __forceinline__ f32x16 mma_ss(const typename Tr::frag (&a)[Bw<Tr>::NS],
                                         const typename Tr::frag (&b)[Bw<Tr>::NS], f32x16 c) {
  c = Tr::mma(a[0], b[0], c);
  if constexpr (Bw<Tr>::NS == 2) {
    c = Tr::mma(a[0], b[1], c);
    c = Tr::mma(a[1], b[0], c);
  }
  return c;
}

// values of a per-feature array at the accumulator rows crow(r, h)
__device__ __forceinline__ f32x16 rows_of(const float* v, int hh) {
  f32x16 out;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 x = *(const f32x4*)(v + 8 * g + 4 * hh);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * g + j] = x[j];
  }
  return out;
}

// MODE kQ1: the query side's first walk -- D_i = phi(q_i).z_i + eps and
//            s_i = phi(q_i).y_i, written as log2 D_i and c_i = -s_i/D_i;
// MODE kQ2: its second walk -- per feature u = y - z s_i/D_i (float32, where
//            the difference cancels), dq_i = (W^T (phi(q_i) * u) - (s_i eps/D_i) q_i)/D_i;
// MODE kK:  the key side, walking the chunks of a span in reverse;
// MODE kQF: both query walks in one, where the workgroup's waves hold every
//            feature block: per chunk, D_i and s_i are summed over the waves
//            (through LDS, one barrier) before u and dq are formed, with the
//            same arithmetic and summation order as the two walks.
constexpr int kQ1 = 0, kQ2 = 1, kK = 2, kQF = 3;

// Two waves per SIMD for the bf16 query walks at d <= 64 (the second walk
// spills a few registers and runs 30% faster than at one wave), one for the
// key walk, whose state would spill inside the chunk loop.  NW waves per
// workgroup, each owning one 32-feature block: the bf16 query walks at
// d <= 64 run eight (one workgroup per compute unit, all 256 features of
// m = 256 in one walk, so nothing is carried between feature groups), the
// others four.
template <class Tr, int D, int MODE>
constexpr int bcausal_waves() { return (Tr::VPS == 8 && D <= 64 && MODE != kK) ? 2 : 1; }
template <class Tr, int D, int MODE>
constexpr int bcausal_nw() { return (Tr::VPS == 8 && D <= 64 && MODE != kK) ? 8 : 4; }

template <class Tr, int D, int MODE, int NW>
__global__ __launch_bounds__(NW * 64, (bcausal_waves<Tr, D, MODE>())) void k_bcausal(BCausalArgs a) {
  using E = typename Tr::elem;
  using F = typename Tr::frag;
  using SP = Bw<Tr>;
  using LY = BCLds<Tr, D, NW, MODE == kK>;
  constexpr bool QSIDE = MODE != kK;
  constexpr int NT = NW * 64;
  constexpr int C = LY::C;
  constexpr int NKD = D / Tr::KS;
  constexpr int NDB = D / 32;
  constexpr int NKT = 32 / Tr::KS;
  constexpr int VPS = Tr::VPS;
  constexpr int RS = LY::RS, RSR = LY::RSR;
  constexpr int WES = VPS == 8 ? 2 : 4;
  constexpr int NKG = D * WES / 32;
  constexpr int DP = D / 8;                              // outputs per thread in the reductions
  constexpr int AW = 2 * D + 2;                          // floats per token of the carried sums
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* sQ = smem + LY::kQ;
  char* sK = smem + LY::kK;
  char* sV = smem + LY::kV;
  char* sG = smem + LY::kG;
  float* sBq = (float*)(smem + LY::kBq);
  float* sBk = (float*)(smem + LY::kBk);
  float* sC = (float*)(smem + LY::kC);
  float* sRed = (float*)(smem + LY::kRed);
  float* sRedS = (float*)(smem + LY::kRedS);

  const int span = blockIdx.x, bh = blockIdx.y;
  const int head = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  float* sZ = (float*)(smem + LY::kZ) + w * 32;
  const int nfb = a.M >> 5;
  const size_t hoff = (size_t)bh * a.L * D;
  const E* Qg = (const E*)a.q + hoff;
  const E* Kg = (const E*)a.k + hoff;
  const E* Vg = (const E*)a.v + hoff;
  const E* Gg = (const E*)a.g + hoff;
  const int hw = a.Hw == 1 ? 0 : head;
  const float half_ln_m = 0.5f * logf((float)a.mt);
  const int t0 = span * a.span_len;
  const int t1 = min(a.L, t0 + a.span_len);
  const int nch = t0 < t1 ? (t1 - t0 + C - 1) / C : 0;
  const E* wth = (const E*)a.wth + (size_t)hw * a.M * D;
  const E* wtl = (const E*)a.wtl + (size_t)hw * a.M * D;

  F ident[NKT], tri[NKT];
#pragma unroll
  for (int s2 = 0; s2 < NKT; ++s2) {
    ident[s2] = const_frag<Tr>(s2, lane, [](int k, int n) { return k == n; });
    tri[s2] = const_frag<Tr>(s2, lane, [](int k, int n) { return k <= n; });   // key k <= query n
  }
  // W^T operand (hi, lo) of block fb, k-step s2, d block db (lane = d)
  auto wt_global = [&](int fb, int s2, int db, F (&wt)[SP::NS]) {
    const size_t e = (((((size_t)fb * NKT + s2) * NDB + db) * 2 + hh) * 32 + l32) * VPS;
    if constexpr (VPS == 8) {
      wt[0] = *(const u32x4*)(wth + e);
      if constexpr (SP::NS == 2) wt[1] = *(const u32x4*)(wtl + e);
    } else {
      wt[0] = wth[e];
    }
  };
  F* sWt = (F*)(smem + LY::kWt) + (size_t)w * LY::WTF * 64;   // this wave's staged copy
  auto wt_frag = [&](int fb, int s2, int db, F (&wt)[SP::NS]) {
    if constexpr (LY::kStageWt) {
#pragma unroll
      for (int p = 0; p < SP::NS; ++p) wt[p] = sWt[((s2 * NDB + db) * SP::NS + p) * 64 + lane];
    } else {
      wt_global(fb, s2, db, wt);
    }
  };

  for (int fg = 0; fg < a.fgroups; ++fg) {
    const int fb = fg * NW + w;
    const bool valid = fb < nfb;
    const int fbs = valid ? fb : 0;
    // projection operand of this wave's block (lane = feature)
    F wf[SP::NS][NKD];
#pragma unroll
    for (int p = 0; p < SP::NS; ++p) {
      const char* base = (const char*)(p == 0 ? a.wph : a.wpl) + ((size_t)hw * nfb + fbs) * NKG * 2 * 32 * 16;
      if constexpr (WES == 2) {
#pragma unroll
        for (int s = 0; s < NKD; ++s) wf[p][s] = *(const u32x4*)(base + ((s * 2 + hh) * 32 + l32) * 16);
      } else {
#pragma unroll
        for (int gk = 0; gk < NKG; ++gk) {
          const f32x4 v = *(const f32x4*)(base + ((gk * 2 + hh) * 32 + l32) * 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) wf[p][4 * gk + j] = v[j];
        }
      }
    }
    if constexpr (LY::kStageWt && MODE != kQ1) {
      // wave-private copy: a wave's LDS accesses complete in program order,
      // so this overwrites the previous group's copy after its last read
#pragma unroll
      for (int s2 = 0; s2 < NKT; ++s2)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          F wt[SP::NS];
          wt_global(fbs, s2, db, wt);
#pragma unroll
          for (int p = 0; p < SP::NS; ++p) sWt[((s2 * NDB + db) * SP::NS + p) * 64 + lane] = wt[p];
        }
    }
    // state of this block from the span prefix (query side: S^T, rows d, lane f;
    // key side: R^T (rows d, lane f) and R (rows f, lane d)) and z or r
    const float* pre = a.pre + ((size_t)bh * a.spans + span) * a.M * D;
    f32x16 st[NDB], st2[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[db][r] = valid ? pre[(size_t)(fbs * 32 + l32) * D + db * 32 + crow(r, hh)] : 0.f;
        if constexpr (!QSIDE) st2[db][r] = valid ? pre[(size_t)(fbs * 32 + crow(r, hh)) * D + db * 32 + l32] : 0.f;
      }
    float zreg = valid ? a.prez[((size_t)bh * a.spans + span) * a.M + fbs * 32 + l32] : 0.f;
    sZ[l32] = zreg;

    TileLoader<E, D, C, NT> lq, lk, lv, lg_;
    auto chunk0 = [&](int ci) { return t0 + ci * C; };
    // per-token scalars of the first query walk (c_i; log2 D_i for the key
    // side), loaded one chunk ahead with the tiles by the threads that stage them
    float pcw = 0.f;
    const bool sthr = tid >= 64 && tid < 64 + C;
    // key side: log2 D_i of the rows whose chunk 0 this thread stages (the
    // query features enter divided by D_i, as a shift of their row bias)
    float plgr[decltype(lq)::NCH];
    auto prefetch = [&](int ci) {
      const int c0 = chunk0(ci);
      lq.load(Qg + (size_t)c0 * D, t1 - c0, tid);
      lk.load(Kg + (size_t)c0 * D, t1 - c0, tid);
      lv.load(Vg + (size_t)c0 * D, t1 - c0, tid);
      lg_.load(Gg + (size_t)c0 * D, t1 - c0, tid);
      if constexpr (MODE == kQ2 || MODE == kK) {
        const int r = tid - 64;
        pcw = sthr && r < t1 - c0 ? a.cw[(size_t)bh * a.L + c0 + r] : 0.f;
      }
      if constexpr (MODE == kK) {
#pragma unroll
        for (int i = 0; i < decltype(lq)::NCH; ++i) {
          const int c = tid + i * NT, row = c / decltype(lq)::CPR;
          plgr[i] = c < C * decltype(lq)::CPR && c % decltype(lq)::CPR == 0 && row < t1 - c0
                        ? a.lg[(size_t)bh * a.L + c0 + row] : 0.f;
        }
      }
    };
    if (nch > 0) prefetch(QSIDE ? 0 : nch - 1);
    for (int it = 0; it < nch; ++it) {
      const int ci = QSIDE ? it : nch - 1 - it;
      const int c0 = chunk0(ci);
      const int nv = min(C, t1 - c0);
      // No barrier before the staging: every read of the previous chunk's
      // tiles, biases and weights happens in its products, which end at the
      // barrier of its cross-wave sums; what follows that barrier (the sums,
      // the outputs) reads only the reduction buffers, which the next writes
      // reach only after the staging barrier below.
      lq.store_proj(sQ, tid);
      lk.store_proj(sK, tid);
      lv.store(sV, tid);
      lg_.store(sG, tid);
      lk.row_bias(sBk, tid, nv, half_ln_m);
      if constexpr (MODE == kK)
        row_bias_shifted(lq, sBq, tid, nv, half_ln_m, plgr);   // bias - log2 D_i; rows past nv: -inf
      else
        lq.row_bias(sBq, tid, nv, half_ln_m);
      if constexpr (MODE == kQ2 || MODE == kK) {
        // per-token log2 D_i and c_i of the first walk: the key side divides
        // the query features by D_i (bias - log2 D_i) and weights them by c_i;
        // the second query walk uses s_i/D_i = -c_i (rows past nv: 0)
        if (sthr) sC[tid - 64] = pcw;
      }
      __syncthreads();
      if (it + 1 < nch) prefetch(QSIDE ? ci + 1 : ci - 1);

      f32x16 r1[NDB], r2[NDB];                          // per-token partial outputs (rows d, lane token)
      float ps1 = 0.f, ps2 = 0.f;                       // per-token partial scalars
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        r1[db] = zero16();
        r2[db] = zero16();
      }
      // query side: phi(Q)^T, phi(K), Y^T, Z^T of this wave's block (kept
      // across the fused walk's exchange of D_i and s_i)
      f32x16 pq = zero16(), pk = zero16(), y = zero16(), z = zero16();
      if (valid) {
        if constexpr (QSIDE) {
          // phi(Q)^T (rows f, lane i) and phi(K) (rows j, lane f)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 b4 = *(const f32x4*)(sBk + 8 * g + 4 * hh);
#pragma unroll
            for (int j = 0; j < 4; ++j) pk[4 * g + j] = b4[j];
          }
#pragma unroll
          for (int s = 0; s < NKD; ++s) {
            const F qf = row_frag<Tr, D>(sQ + l32 * RS, hh, s);
            const F kf = row_frag<Tr, D>(sK + l32 * RS, hh, s);
#pragma unroll
            for (int p = 0; p < SP::NS; ++p) {
              pq = Tr::pmma(wf[p][s], qf, pq);
              pk = Tr::pmma(kf, wf[p][s], pk);
            }
          }
          const float bq = sBq[l32];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            pq[r] = exp2_fast(pq[r] + bq);
            pk[r] = exp2_fast(pk[r]);
          }
          if (fb * 32 + 32 > a.mt) {                     // padding features: phi = 0
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (fb * 32 + crow(r, hh) >= a.mt) pq[r] = 0.f;
            if (fb * 32 + l32 >= a.mt) pk = zero16();
          }
          // B[j][i] = v_j . g_i for j <= i (rows j, lane i)
          f32x16 bm = zero16();
#pragma unroll
          for (int s = 0; s < NKD; ++s)
            bm = Tr::mma(row_frag<Tr, D>(sV + l32 * RS, hh, s), row_frag<Tr, D>(sG + l32 * RS, hh, s), bm);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (crow(r, hh) > l32) bm[r] = 0.f;
          // Y^T = S^T-operand x G + phi(K)^T B;  Z^T = z + phi(K)^T T (rows f, lane i)
          z = rows_of(sZ, hh);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int s2 = 0; s2 < NKT; ++s2) {
              F sf[SP::NS];
              SP::split(st[db], s2, sf);
              y = mma_sa<Tr>(sf, crow_frag<Tr>(sG + l32 * RS, db, s2, hh), y);
            }
#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2) {
            F kf[SP::NS], bf[SP::NS];
            SP::split(pk, s2, kf);
            SP::split(bm, s2, bf);
            y = mma_ss<Tr>(kf, bf, y);
            z = mma_sa<Tr>(kf, tri[s2], z);
          }
          if constexpr (MODE == kQ1 || MODE == kQF) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              ps1 = fmaf(pq[r], z[r], ps1);
              ps2 = fmaf(pq[r], y[r], ps2);
            }
          }
        }
      }
      // fused walk: D_i and s_i over every wave's features, in wave order
      float fratio = 0.f;
      if constexpr (MODE == kQF) {
        {
          const float a1 = half_sum(ps1), a2s = half_sum(ps2);
          if (hh == 0) {
            sRedS[(w * C + l32) * 2] = a1;
            sRedS[(w * C + l32) * 2 + 1] = a2s;
          }
        }
        wait_lgkm0();
        raw_barrier();
        float d1 = 0.f, d2 = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
          d1 += sRedS[(ww * C + l32) * 2];
          d2 += sRedS[(ww * C + l32) * 2 + 1];
        }
        const float den = d1 + a.eps;
        fratio = -(-(d2 / den));                       // as -c_i of the first walk
      }
      if (valid) {
        if constexpr (QSIDE) {
          if constexpr (MODE == kQ2 || MODE == kQF) {
            // u = y - z s/D in float32, then dq^T += W^T (phi * u) (rows d, lane i)
            const float ratio = MODE == kQF ? fratio : -sC[l32];
            f32x16 gq;
#pragma unroll
            for (int r = 0; r < 16; ++r) gq[r] = pq[r] * (y[r] - z[r] * ratio);
#pragma unroll
            for (int s2 = 0; s2 < NKT; ++s2) {
              F gf[SP::NS];
              SP::split(gq, s2, gf);
#pragma unroll
              for (int db = 0; db < NDB; ++db) {
                F wt[SP::NS];
                wt_frag(fbs, s2, db, wt);
                r1[db] = mma_ss<Tr>(wt, gf, r1[db]);
              }
            }
          }
          // state update: S^T += V^T phi(K), z += phi(K)^T 1
          float zc = 0.f;
#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2) {
            F kf[SP::NS];
            SP::split(pk, s2, kf);
#pragma unroll
            for (int db = 0; db < NDB; ++db) st[db] = mma_sb<Tr>(col_frag<Tr, RS>(sV, 0, db * 32, s2, lane), kf, st[db]);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) zc += pk[r];
          zreg += half_sum(zc);
          sZ[l32] = zreg;                                // read by this wave's next chunk
        } else {
          // phi(K)^T, phi'(Q)^T (rows f, lane token); phi'(Q) (rows i, lane f)
          f32x16 pk = zero16(), pqt = zero16();
#pragma unroll
          for (int s = 0; s < NKD; ++s) {
            const F qf = row_frag<Tr, D>(sQ + l32 * RS, hh, s);
            const F kf = row_frag<Tr, D>(sK + l32 * RS, hh, s);
#pragma unroll
            for (int p = 0; p < SP::NS; ++p) {
              pqt = Tr::pmma(wf[p][s], qf, pqt);
              pk = Tr::pmma(wf[p][s], kf, pk);
            }
          }
          const float bq = sBq[l32], bk = sBk[l32];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            pqt[r] = exp2_fast(pqt[r] + bq);
            pk[r] = exp2_fast(pk[r] + bk);
          }
          if (fb * 32 + 32 > a.mt) {                     // padding features: phi = 0
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (fb * 32 + crow(r, hh) >= a.mt) {
                pqt[r] = 0.f;
                pk[r] = 0.f;
              }
          }
          f32x16 pq = zero16();
#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2) {
            F qf[SP::NS];
            SP::split(pqt, s2, qf);
            pq = mma_sa<Tr>(qf, ident[s2], pq);
          }
          // E[i][j] = g_i . v_j + c_i for i >= j (rows i, lane j)
          f32x16 em = rows_of(sC, hh);
#pragma unroll
          for (int s = 0; s < NKD; ++s)
            em = Tr::mma(row_frag<Tr, D>(sG + l32 * RS, hh, s), row_frag<Tr, D>(sV + l32 * RS, hh, s), em);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (crow(r, hh) < l32) em[r] = 0.f;
          // dphi(K)^T = r + R V^T + phi'(Q)^T E (rows f, lane j)
          f32x16 u = rows_of(sZ, hh);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int s2 = 0; s2 < NKT; ++s2) {
              F rf[SP::NS];
              SP::split(st[db], s2, rf);
              u = mma_sa<Tr>(rf, crow_frag<Tr>(sV + l32 * RS, db, s2, hh), u);
            }
#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2) {
            F qf[SP::NS], ef[SP::NS];
            SP::split(pq, s2, qf);
            SP::split(em, s2, ef);
            u = mma_ss<Tr>(qf, ef, u);
          }
          // scores A2[i][j] = phi'(q_i) . phi(k_j) over this block, i >= j
          f32x16 a2 = zero16();
#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2) a2 = Tr::mma(CFrag<Tr>::make(pqt, s2), CFrag<Tr>::make(pk, s2), a2);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (crow(r, hh) < l32) a2[r] = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            u[r] *= pk[r];
            ps1 += u[r];
          }
#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2) {
            F gf[SP::NS];
            SP::split(u, s2, gf);
            const F kf = CFrag<Tr>::make(pk, s2);
            const F af = CFrag<Tr>::make(a2, s2);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              F wt[SP::NS];
              wt_frag(fbs, s2, db, wt);
              r1[db] = mma_ss<Tr>(wt, gf, r1[db]);                                       // dk^T
              r2[db] = Tr::mma(CFrag<Tr>::make(st2[db], s2), kf, r2[db]);               // R^T phi(K)
              r2[db] = Tr::mma(col_frag<Tr, RS>(sG, 0, db * 32, s2, lane), af, r2[db]); // G^T A2
            }
          }
          // state update: R^T += G^T phi'(Q), R += phi'(Q)^T G, r += phi'(Q)^T c
#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2) {
            F qf[SP::NS];
            SP::split(pq, s2, qf);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const F gcol = col_frag<Tr, RS>(sG, 0, db * 32, s2, lane);
              st[db] = mma_sb<Tr>(gcol, qf, st[db]);
              st2[db] = mma_sa<Tr>(qf, gcol, st2[db]);
            }
          }
          const f32x16 cr = rows_of(sC, hh);
          float rc = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) rc = fmaf(pq[r], cr[r], rc);
          zreg += half_sum(rc);
          sZ[l32] = zreg;
        }
      }

      // what the end of this chunk reads from memory, requested before the
      // sums over the waves so that its latency hides behind them (not
      // earlier: the values would be live across the products, where the
      // register file is full): the input row of the token (dq and dk
      // subtract a multiple of it), the token's log2 D_i and c_i (second query
      // walk) and the sums carried from earlier feature groups
      const bool rt = tid < 8 * C;
      const int tq = rt ? tid >> 3 : 0, d0 = (tid & 7) * DP;
      const bool own = rt && tq < nv;
      const size_t tokq = (size_t)c0 + tq;
      constexpr int NRND = MODE == kQ1 ? 0 : (MODE == kK ? 2 : 1);
      float xrow[DP], carried[NRND > 0 ? NRND * DP : 1], cs1 = 0.f, cs2 = 0.f, lgq = 0.f, cwq = 0.f;
      if constexpr (MODE != kQ1) {
        const E* xr = (QSIDE ? Qg : Kg) + tokq * D + d0;
        const bool need = own && fg + 1 == a.fgroups;
        if constexpr (sizeof(E) == 2 && DP == 4) {
          u32x2 x2 = {0u, 0u};
          if (need) x2 = *(const u32x2*)xr;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            xrow[2 * e] = bf16_lo(x2[e]);
            xrow[2 * e + 1] = bf16_hi(x2[e]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < DP; j += 16 / (int)sizeof(E)) {
            u32x4 x4 = {0u, 0u, 0u, 0u};
            if (need) x4 = *(const u32x4*)(xr + j);
            if constexpr (sizeof(E) == 2) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                xrow[j + 2 * e] = bf16_lo(x4[e]);
                xrow[j + 2 * e + 1] = bf16_hi(x4[e]);
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) xrow[j + e] = as_f32(x4[e]);
            }
          }
        }
        if constexpr (MODE == kQ2) {
          if (own && fg + 1 == a.fgroups) {
            lgq = a.lg[(size_t)bh * a.L + tokq];
            cwq = a.cw[(size_t)bh * a.L + tokq];
          }
        }
      }
      if constexpr (NRND > 0) {
#pragma unroll
        for (int j = 0; j < NRND * DP; ++j) carried[j] = 0.f;
        if (a.fgroups > 1 && fg > 0 && own) {
          const float* ar = a.acc + ((size_t)bh * a.L + tokq) * AW;
#pragma unroll
          for (int rd = 0; rd < NRND; ++rd)
#pragma unroll
            for (int j = 0; j < DP; ++j) carried[rd * DP + j] = ar[rd * D + d0 + j];   // rows 8-byte aligned
        }
      }
      if (a.fgroups > 1 && fg > 0 && own && (MODE == kQ1 || MODE == kK)) {
        const float* as = a.acc + ((size_t)bh * a.L + tokq) * AW + 2 * D;
        cs1 = as[0];
        cs2 = as[1];
      }
      // ---- sums over the waves (fixed order) and the feature groups --------
      // carried sums per token: [0, D) first output, [D, 2D) second, 2D and
      // 2D+1 the two scalars
      float* accrow = a.acc + ((size_t)bh * a.L + c0) * AW;
      // threads 0..255: eight per token of the chunk (rt, tq, d0 above)
      constexpr int NROUND = NRND;
      float v1[DP], v2[DP], sc1 = 0.f, sc2 = 0.f;
      if constexpr (MODE != kQF) {                       // (the fused walk wrote them mid-chunk)
        const float a1 = half_sum(ps1), a2s = half_sum(ps2);
        if (hh == 0) {
          sRedS[(w * C + l32) * 2] = a1;
          sRedS[(w * C + l32) * 2 + 1] = a2s;
        }
      }
      // each round: this wave's partial outputs into a reduction buffer, one
      // barrier, then the sums over the waves in wave order; with a second
      // buffer (key side) both rounds share one barrier
      constexpr bool ONEBAR = NROUND == 2 && LY::kRed2;
      auto red_buf = [&](int round) -> float* {
        if constexpr (ONEBAR) return round == 0 ? sRed : (float*)(smem + LY::kRedB);
        return sRed;
      };
      auto write_round = [&](int round) {
        f32x16 (&rr)[NDB] = round == 0 ? r1 : r2;
        float* rrow = red_buf(round) + (size_t)w * C * RSR + l32 * RSR;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(f32x4*)(rrow + db * 32 + 8 * g + 4 * hh) =
                f32x4{rr[db][4 * g], rr[db][4 * g + 1], rr[db][4 * g + 2], rr[db][4 * g + 3]};
      };
      auto sum_round = [&](int round) {
        float* vv = round == 0 ? v1 : v2;
#pragma unroll
        for (int j = 0; j < DP; ++j) vv[j] = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
          const float* src = red_buf(round) + (size_t)ww * C * RSR + tq * RSR + d0;
#pragma unroll
          for (int j = 0; j < DP; j += 4) {
            const f32x4 x = *(const f32x4*)(src + j);
            vv[j] += x[0];
            vv[j + 1] += x[1];
            vv[j + 2] += x[2];
            vv[j + 3] += x[3];
          }
        }
        if (a.fgroups > 1 && rt && tq < nv) {
          float* ar = accrow + (size_t)tq * AW + round * D + d0;
          if (fg > 0) {
#pragma unroll
            for (int j = 0; j < DP; ++j) vv[j] += carried[round * DP + j];
          }
          if (fg + 1 < a.fgroups) {
#pragma unroll
            for (int j = 0; j < DP; ++j) ar[j] = vv[j];
          }
        }
      };
      // LDS-only barriers from here on: __syncthreads would also wait for
      // the next chunk's tile prefetch and the loads requested above
      if constexpr (ONEBAR) {
        write_round(0);
        write_round(1);
        wait_lgkm0();
        raw_barrier();
        sum_round(0);
        sum_round(1);
      } else {
#pragma unroll
        for (int round = 0; round < NROUND; ++round) {
          write_round(round);
          wait_lgkm0();
          raw_barrier();
          sum_round(round);
          if (round + 1 < NROUND) {                      // before the next round overwrites sRed
            wait_lgkm0();
            raw_barrier();
          }
        }
      }
      if constexpr (NROUND == 0) {                       // the scalars are in LDS
        wait_lgkm0();
        raw_barrier();
      }
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        sc1 += sRedS[(ww * C + tq) * 2];
        sc2 += sRedS[(ww * C + tq) * 2 + 1];
      }
      if (a.fgroups > 1 && rt && tq < nv && (MODE == kQ1 || MODE == kK)) {
        float* as = accrow + (size_t)tq * AW + 2 * D;
        if (fg > 0) {
          sc1 += cs1;
          sc2 += cs2;
        }
        if (fg + 1 < a.fgroups && (tid & 7) == 0) {
          as[0] = sc1;
          as[1] = sc2;
        }
      }
      if (fg + 1 == a.fgroups && rt && tq < nv) {
        const size_t tok = (size_t)c0 + tq;
        if constexpr (MODE == kQ1) {
          if ((tid & 7) == 0) {
            const float den = sc1 + a.eps;
            a.lg_out[(size_t)bh * a.L + tok] = log2f(den);
            a.cw_out[(size_t)bh * a.L + tok] = -(sc2 / den);
          }
        } else if constexpr (MODE == kQ2 || MODE == kQF) {
          float lgv = lgq, cwv = cwq;
          if constexpr (MODE == kQF) {                   // the first walk's outputs, formed here
            const float den = sc1 + a.eps;
            lgv = log2f(den);
            cwv = -(sc2 / den);
            if ((tid & 7) == 0) {
              a.lg_out[(size_t)bh * a.L + tok] = lgv;
              a.cw_out[(size_t)bh * a.L + tok] = cwv;
            }
          }
          const float inv = exp2f(-lgv);
          const float ratio = -cwv;
          float o[DP];
#pragma unroll
          for (int j = 0; j < DP; ++j) o[j] = (v1[j] - ratio * a.eps * xrow[j]) * inv;
          store_row<E, DP>((E*)a.dx + hoff + tok * D + d0, o);
        } else {
          float o[DP];
#pragma unroll
          for (int j = 0; j < DP; ++j) o[j] = v1[j] - sc1 * xrow[j];
          store_row<E, DP>((E*)a.dx + hoff + tok * D + d0, o);
          store_row<E, DP>((E*)a.dy + hoff + tok * D + d0, v2);
        }
      }
    }
  }
}

template <class Tr, int D>
static hipError_t bwd_causal_t(const Plan& p, const BwdTensors& t, hipStream_t s) {
  using E = typename Tr::elem;
  const BwdBuffers b = bwd_buffers(p, t.ws);
  const int nrows = p.Hw * p.M;
  {
    constexpr int WES = Tr::VPS == 8 ? 2 : 4;
    const int n = nrows * D / (16 / WES) + nrows * D / Tr::VPS;
    const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
    timing_begin(FAVOR_KERNEL_BWD_PREP, s);
    hipLaunchKernelGGL((k_bprep<Tr>), dim3(blocks), dim3(256), 0, s, t.w, b.wph, b.wpl, b.wt,
                       Tr::VPS == 8 ? b.wtl : nullptr, nrows, D, p.M, p.mt);
    timing_end(FAVOR_KERNEL_BWD_PREP, s);
  }
  // reduction workgroups: one wave per feature block, the plan's brnw blocks
  // (eight only for bf16 at d <= 64)
  constexpr bool kRed8 = Tr::VPS == 8 && D <= 64;
  if (p.brnw != 4 && !(kRed8 && p.brnw == 8)) return kErrPlan;
  const dim3 rgrid(p.bsplits, p.bfgroups, p.BH);
  constexpr size_t rlds8 = BRedLds<Tr, D, 8>::kTotal, rlds4 = BRedLds<Tr, D, 4>::kTotal;
  auto launch_bred = [&]<bool WT>(const BRedArgs& ra) {
    if constexpr (kRed8) {
      if (p.brnw == 8) {
        hipLaunchKernelGGL((k_bred<Tr, D, WT, 8>), rgrid, dim3(512), rlds8, s, ra);
        return;
      }
    }
    hipLaunchKernelGGL((k_bred<Tr, D, WT, 4>), rgrid, dim3(256), rlds4, s, ra);
  };
  const int nq = (p.M * D + p.M) / 4;
  const dim3 sgrid((nq + 255) / 256, p.BH);
  constexpr int NWQ = bcausal_nw<Tr, D, kQ1>(), NWK = bcausal_nw<Tr, D, kK>();
  static_assert(bcausal_nw<Tr, D, kQ2>() == NWQ && bcausal_nw<Tr, D, kQF>() == NWQ, "one wave count for the query walks");
  const int nfb = p.M / 32;
  const int fgq = (nfb + NWQ - 1) / NWQ, fgk = (nfb + NWK - 1) / NWK;
  if ((fgq > 1 || fgk > 1) && p.boff_acc == p.btotal) return kErrPlan;   // no room for the sums
  if (p.bqnw != NWQ) return kErrPlan;
  BCausalArgs ca{t.q, t.k, t.v, t.g, b.wph, b.wpl, b.wt, b.wtl, b.part, b.partz, b.lg, b.cw, b.lg, b.cw,
                 t.dq, nullptr, b.acc, p.L, p.M, p.H, p.Hw, p.bsplits, p.bsplit_len, fgq, t.eps, p.mt};
  // span aggregates of phi(K) V^T, phi(K) -> exclusive prefixes
  {
    BRedArgs a{t.k, t.v, nullptr, nullptr, b.wph, b.wpl, b.part, b.partz, p.L, p.M, p.H, p.Hw, p.bsplits, p.bsplit_len, p.mt};
    timing_begin(FAVOR_KERNEL_BWD_REDUCE, s);
    launch_bred.template operator()<false>(a);
    timing_end(FAVOR_KERNEL_BWD_REDUCE, s);
    timing_begin(FAVOR_KERNEL_BWD_COMBINE, s);
    hipLaunchKernelGGL(k_bscan, sgrid, dim3(256), 0, s, b.part, b.partz, p.bsplits, p.M, D, 0);
    timing_end(FAVOR_KERNEL_BWD_COMBINE, s);
  }
  // query side: log2 D_i and c_i (the lg and cw arrays), then dQ
  timing_begin(FAVOR_KERNEL_BWD_Q, s);
  const size_t qlds = BCLds<Tr, D, NWQ>::kTotal;
  if (fgq == 1) {                                         // every feature block in one workgroup
    hipLaunchKernelGGL((k_bcausal<Tr, D, kQF, NWQ>), dim3(p.bsplits, p.BH), dim3(NWQ * 64), qlds, s, ca);
  } else {
    hipLaunchKernelGGL((k_bcausal<Tr, D, kQ1, NWQ>), dim3(p.bsplits, p.BH), dim3(NWQ * 64), qlds, s, ca);
    hipLaunchKernelGGL((k_bcausal<Tr, D, kQ2, NWQ>), dim3(p.bsplits, p.BH), dim3(NWQ * 64), qlds, s, ca);
  }
  timing_end(FAVOR_KERNEL_BWD_Q, s);
  // span aggregates of phi'(Q) G^T, phi'(Q) c -> exclusive suffixes
  {
    BRedArgs a{t.q, t.g, b.lg, b.cw, b.wph, b.wpl, b.part, b.partz, p.L, p.M, p.H, p.Hw, p.bsplits, p.bsplit_len, p.mt};
    timing_begin(FAVOR_KERNEL_BWD_REDUCE, s);
    launch_bred.template operator()<true>(a);
    timing_end(FAVOR_KERNEL_BWD_REDUCE, s);
    timing_begin(FAVOR_KERNEL_BWD_COMBINE, s);
    hipLaunchKernelGGL(k_bscan, sgrid, dim3(256), 0, s, b.part, b.partz, p.bsplits, p.M, D, 1);
    timing_end(FAVOR_KERNEL_BWD_COMBINE, s);
  }
  // key side
  ca.dx = t.dk;
  ca.dy = t.dv;
  ca.fgroups = fgk;
  const size_t klds = BCLds<Tr, D, NWK, true>::kTotal;
  timing_begin(FAVOR_KERNEL_BWD_K, s);
  hipLaunchKernelGGL((k_bcausal<Tr, D, kK, NWK>), dim3(p.bsplits, p.BH), dim3(NWK * 64), klds, s, ca);
  timing_end(FAVOR_KERNEL_BWD_K, s);
  return hipGetLastError();
}

hipError_t launch_causal_bwd(const Plan& p, const BwdTensors& t, hipStream_t s) {
  if (p.dt == FAVOR_BF16) {
    switch (p.D) {
      case 32: return bwd_causal_t<TrBF16, 32>(p, t, s);
      case 64: return bwd_causal_t<TrBF16, 64>(p, t, s);
      case 128: return bwd_causal_t<TrBF16, 128>(p, t, s);
    }
  } else {
    switch (p.D) {
      case 32: return bwd_causal_t<TrF32, 32>(p, t, s);
      case 64: return bwd_causal_t<TrF32, 64>(p, t, s);
      case 128: return bwd_causal_t<TrF32, 128>(p, t, s);
    }
  }
  return kErrPlan;
}

}  // namespace favor
