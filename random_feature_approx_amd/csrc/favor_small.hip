// Non-causal FAVOR+ for short sequences (L <= 64 per head, m <= 256,
// d in {32, 64}): the whole head in one workgroup and one launch.
//
// The worked example of the Performer page (In[26]: n = 64, d = 32, m up to
// 512 features) is latency-bound on the general path: a reduction, a combine
// and an apply launch, each with one busy workgroup, and in the apply one wave
// walking all feature blocks of its 32 queries in series.  Here eight waves
// each own one 32-feature block of W and compute, for that block (the
// reassociated form of the Performer page's In[25]):
//   K side:  M_f = phi(K)_f^T V (32 x d) and z_f = phi(K)_f^T 1,
//   Q side:  num_f = phi(Q)_f M_f (L x d) and den_f = phi(Q)_f z_f,
// and the workgroup sums num_f and den_f over the blocks in a fixed order
// (block 0 first) before O = num / (den + eps).  Products as in the general
// kernels: fp16 projection operands for bf16 inputs, bf16 feature and state
// operands, float32 accumulation; float32 inputs on float32 products.
#include "favor_device.hpp"
#include "favor_internal.hpp"
#include "favor_tiles.hpp"

namespace favor {

struct SmallArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* w;
  void* o;
  int L, M, H, Hw, mt;
  float eps;
};

template <class Tr, int D>
struct SmallLds {
  using E = typename Tr::elem;
  static constexpr int T = 64;                          // tokens (at most)
  static constexpr int RS = Rows<D, sizeof(E)>::RS;
  static constexpr int RSR = D + 4;                     // floats per row of the partial outputs
  static constexpr int kQ = 0, kK = T * RS, kV = 2 * T * RS;
  static constexpr int kBq = 3 * T * RS, kBk = kBq + T * 4;
  static constexpr int kZ = kBk + T * 4;                // [8 blocks][32] z
  static constexpr int kRed = kZ + 8 * 32 * 4;          // [8 blocks][32 tokens][RSR]
  static constexpr int kDen = kRed + 8 * 32 * RSR * 4;  // [8 blocks][32 tokens]
  static constexpr int kTotal = kDen + 8 * 32 * 4;
};

template <class Tr, int D>
__global__ __launch_bounds__(512) void k_small_nc(SmallArgs a) {
  using E = typename Tr::elem;
  using F = typename Tr::frag;
  using LY = SmallLds<Tr, D>;
  constexpr int T = LY::T, RS = LY::RS, RSR = LY::RSR;
  constexpr int NKD = D / Tr::KS;                       // projection k-steps over d
  constexpr int NKT = 32 / Tr::KS;                      // k-steps over 32 tokens or features
  constexpr int NDB = D / 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* sBq = (float*)(smem + LY::kBq);
  float* sBk = (float*)(smem + LY::kBk);
  float* sZ = (float*)(smem + LY::kZ);
  float* sRed = (float*)(smem + LY::kRed);
  float* sDen = (float*)(smem + LY::kDen);

  const int bh = blockIdx.x, head = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave's feature block
  const int nfb = a.M >> 5;
  const float half_ln_m = 0.5f * logf((float)a.mt);
  const size_t hoff = (size_t)bh * a.L * D;

  // the head's rows: Q and K in the projection type with their row biases
  // (-inf past L), V as given (rows past L zero)
  {
    TileLoader<E, D, T, 512> lq, lk, lv;
    lq.load((const E*)a.q + hoff, a.L, tid);
    lk.load((const E*)a.k + hoff, a.L, tid);
    lv.load((const E*)a.v + hoff, a.L, tid);
    lq.store_proj(smem + LY::kQ, tid);
    lk.store_proj(smem + LY::kK, tid);
    lv.store(smem + LY::kV, tid);
    lq.row_bias(sBq, tid, a.L, half_ln_m);
    lk.row_bias(sBk, tid, a.L, half_ln_m);
  }
  // this wave's block of W (lane = feature, d-major slots); rows past m
  // (a ragged last block) and blocks past M/32 are zero
  const int wr = w * 32 + l32;
  const bool wok = w < nfb && wr < a.mt;
  const float* wrow = a.w + ((size_t)(a.Hw == 1 ? 0 : head) * a.mt + (wok ? wr : 0)) * D;
  F wf[NKD];
#pragma unroll
  for (int s = 0; s < NKD; ++s) wf[s] = w_frag<Tr, D, FM_POS>(wrow, hh, s, wok);
  __syncthreads();

  // ---- K side: M_f (rows f in c-row order, lane = d) and z_f -----------------
  f32x16 st[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) st[db] = zero16();
  float zs = 0.f;
#pragma unroll
  for (int tb = 0; tb < T / 32; ++tb) {
    f32x16 acc;                                         // P[t][f] + bias[t], lane = f
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = sBk[tb * 32 + crow(r, hh)];
#pragma unroll
    for (int s = 0; s < NKD; ++s)
      acc = Tr::pmma(row_frag<Tr, D>(smem + LY::kK + (tb * 32 + l32) * RS, hh, s), wf[s], acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = wok ? exp2_fast(acc[r]) : 0.f;
#pragma unroll
    for (int s2 = 0; s2 < NKT; ++s2) {
      const F pf = CFrag<Tr>::make(acc, s2);            // lane = f, k = tokens (c-row)
      if constexpr (Tr::VPS == 8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) zs = dot2_bf16(pf[j], 0x3f803f80u, zs);
      } else {
        zs += pf;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        st[db] = Tr::mma(pf, col_frag<Tr, RS>(smem + LY::kV, tb * 32, db * 32, s2, lane), st[db]);
    }
  }
  // features past m: zero state rows (their feature values above were zero
  // only where the lane is the feature; here the rows are features)
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (w * 32 + crow(r, hh) >= a.mt) st[db][r] = 0.f;
  {
    const float z = half_sum(zs);
    if (hh == 0) sZ[w * 32 + l32] = z;                  // zero for features past m (wok false)
  }
  __syncthreads();

  // ---- Q side, per 32-token block: this block's num and den, then the sum
  // over the feature blocks in order ------------------------------------------
  const int ntb = (a.L + 31) / 32;
  for (int tb = 0; tb < ntb; ++tb) {
    f32x16 pt = splat16(sBq[tb * 32 + l32]);            // P^T[f][t] + bias[t], lane = t
#pragma unroll
    for (int s = 0; s < NKD; ++s)
      pt = Tr::pmma(wf[s], row_frag<Tr, D>(smem + LY::kQ + (tb * 32 + l32) * RS, hh, s), pt);
#pragma unroll
    for (int r = 0; r < 16; ++r) pt[r] = exp2_fast(pt[r]);
    f32x16 o[NDB];                                      // O^T[d][t] partial, lane = t
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = zero16();
#pragma unroll
    for (int s2 = 0; s2 < NKT; ++s2) {
      const F bf = CFrag<Tr>::make(pt, s2);             // lane = t, k = features (c-row)
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] = Tr::mma(CFrag<Tr>::make(st[db], s2), bf, o[db]);
    }
    float den = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) den = fmaf(pt[r], sZ[w * 32 + crow(r, hh)], den);
    den = half_sum(den);
    float* rrow = sRed + (w * 32 + l32) * RSR;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(f32x4*)(rrow + db * 32 + 8 * g + 4 * hh) = f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
    if (hh == 0) sDen[w * 32 + l32] = den;
    __syncthreads();
    // 16 threads per token, D/16 outputs each; blocks summed in order
    {
      constexpr int DP = D / 16;
      const int t = tid >> 4, d0 = (tid & 15) * DP;
      float acc[DP];
#pragma unroll
      for (int j = 0; j < DP; ++j) acc[j] = 0.f;
      float dsum = 0.f;
      for (int b = 0; b < nfb; ++b) {
        const float* src = sRed + (b * 32 + t) * RSR + d0;
#pragma unroll
        for (int j = 0; j < DP; ++j) acc[j] += src[j];
        dsum += sDen[b * 32 + t];
      }
      const float inv = 1.0f / (dsum + a.eps);
      const int tok = tb * 32 + t;
      if (tok < a.L) {
        E* orow = (E*)a.o + hoff + (size_t)tok * D + d0;
#pragma unroll
        for (int j = 0; j < DP; ++j) orow[j] = Tr::from_f32(acc[j] * inv);
      }
    }
    __syncthreads();                                    // before the next block reuses the partials
  }
}

bool small_nc_fits(const Plan& p) {
  return !p.causal && p.fmap == FM_POS && p.L <= 64 && p.M <= 256 && (p.D == 32 || p.D == 64);
}

hipError_t launch_small_nc(const Plan& p, const Tensors& t, hipStream_t s) {
  if (!small_nc_fits(p)) return kErrPlan;
  SmallArgs a{t.q, t.k, t.v, t.w, t.o, p.L, p.M, p.H, p.Hw, p.mt, t.eps};
  timing_begin(FAVOR_KERNEL_APPLY, s);
  // (LDS sizes as locals: the launch macro splits template arguments at commas)
  constexpr size_t lb64 = SmallLds<TrBF16, 64>::kTotal, lb32 = SmallLds<TrBF16, 32>::kTotal;
  constexpr size_t lf64 = SmallLds<TrF32, 64>::kTotal, lf32 = SmallLds<TrF32, 32>::kTotal;
  if (p.dt == FAVOR_BF16) {
    if (p.D == 64)
      hipLaunchKernelGGL((k_small_nc<TrBF16, 64>), dim3(p.BH), dim3(512), lb64, s, a);
    else
      hipLaunchKernelGGL((k_small_nc<TrBF16, 32>), dim3(p.BH), dim3(512), lb32, s, a);
  } else {
    if (p.D == 64)
      hipLaunchKernelGGL((k_small_nc<TrF32, 64>), dim3(p.BH), dim3(512), lf64, s, a);
    else
      hipLaunchKernelGGL((k_small_nc<TrF32, 32>), dim3(p.BH), dim3(512), lf32, s, a);
  }
  timing_end(FAVOR_KERNEL_APPLY, s);
  return hipGetLastError();
}

}  // namespace favor
