// Causal FAVOR+ on gfx950.
//
// o_i = phi(q_i)^T S_i / (phi(q_i)^T z_i + eps), S_i = sum_{j<=i} phi(k_j) v_j^T,
// z_i = sum_{j<=i} phi(k_j)   (prefix-sum form of the study notes' case 2;
// the denominator is its analogue of the non-causal normaliser).
//
// L is cut into spans (one workgroup each) and spans into chunks
// of 32 tokens in every scan (a chunk of 64 is carried as two 32-token steps).
//   1. k_reduce (shared with the non-causal path) computes the aggregate
//      [sum phi(k) v^T | sum phi(k)] of every span but the last (whose sum
//      only a prefix past the end would use) in float32.
//   2. k_span_scan turns the aggregates into exclusive prefixes in place, in
//      a fixed order of additions (deterministic).
//   3. k_causal3 (bf16 FAVOR+, d <= 64, m = 256), k_causal2 (other bf16,
//      d <= 64) or k_causal walks the chunks of a span
//      starting from its prefix.  For a
//      chunk c with queries Q_c, keys K_c and values V_c:
//        num = tril(phi(Q_c) phi(K_c)^T) V_c + phi(Q_c) S      (masked tile
//              includes the diagonal)
//        den = rowsum(tril(phi(Q_c) phi(K_c)^T)) + phi(Q_c) z + eps
//        S += phi(K_c)^T V_c,  z += phi(K_c)^T 1.
//      Each wave owns a slice of the features and its slice of S in
//      accumulator registers; the contributions of the slices are summed
//      through LDS.  A feature group that does not fit one workgroup is
//      processed group after group, the partial numerators and denominators
//      kept in float32 in the workspace.
#include "favor_device.hpp"
#include "favor_internal.hpp"
#include "favor_tiles.hpp"

namespace favor {

// ---------------------------------------------------------------------------
// exclusive prefix of the span aggregates, in place:  a[s] <- sum_{s'<s} a[s']
// (the last span's aggregate is neither computed nor read).
// The m*d + m values of a head are handled in quads of 4 floats.  A block is
// kScanGroups groups of threads; group g owns spans [g*per, (g+1)*per) of its
// quad: it first sums them, the groups' sums give each group its starting
// offset (added in group order), and a second pass writes the running
// prefixes.  The order of additions depends only on the span count.
// ---------------------------------------------------------------------------
constexpr int kScanGroups = 8;
constexpr int kScanQuads = 256 / kScanGroups;

__global__ __launch_bounds__(256) void k_span_scan(float* part, float* partz, int spans, int M, int D) {
  __shared__ f32x4 tot[kScanGroups][kScanQuads];
  const int bh = blockIdx.y;
  const int g = threadIdx.x / kScanQuads, qi = threadIdx.x % kScanQuads;
  const int quad = blockIdx.x * kScanQuads + qi;
  const int md4 = M * D / 4, nq = md4 + M / 4;
  const bool active = quad < nq;
  f32x4* p;
  size_t stride;
  if (quad < md4) {
    p = (f32x4*)(part + (size_t)bh * spans * M * D) + quad;
    stride = md4;
  } else {
    p = (f32x4*)(partz + (size_t)bh * spans * M) + (active ? quad - md4 : 0);
    stride = M / 4;
  }
  const int per = (spans + kScanGroups - 1) / kScanGroups;
  const int s0 = min(spans, g * per), s1 = min(spans, s0 + per);
  const int s1a = min(s1, spans - 1);                   // the last span's aggregate is not computed
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 sum = zero;
  // at most 8 spans per group (up to 64 spans): the values stay in registers
  // for the second pass instead of being read again
  f32x4 keep[8];
  const bool kept = s1 - s0 <= 8;
  if (active) {
    for (int s = s0; s < s1; s += 8) {
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = s + j < s1a ? p[(size_t)(s + j) * stride] : zero;
#pragma unroll
      for (int j = 0; j < 8; ++j) sum += v[j];
      if (kept) {
#pragma unroll
        for (int j = 0; j < 8; ++j) keep[j] = v[j];
      }
    }
  }
  tot[g][qi] = sum;
  __syncthreads();
  if (!active) return;
  f32x4 run = zero;
  for (int gg = 0; gg < g; ++gg) run += tot[gg][qi];
  if (kept) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j < s1) {
        p[(size_t)(s0 + j) * stride] = run;
        run += keep[j];
      }
    }
    return;
  }
  for (int s = s0; s < s1; s += 8) {
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = s + j < s1a ? p[(size_t)(s + j) * stride] : zero;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s + j < s1) {
        p[(size_t)(s + j) * stride] = run;
        run += v[j];
      }
    }
  }
}


// The same prefix for at most kScanSmall spans (the usual case): one thread
// per quad loads the span aggregates together and writes the running sums,
// added in span order.
constexpr int kScanSmall = 16;

__global__ __launch_bounds__(256) void k_span_scan_small(float* part, float* partz, int spans, int M, int D) {
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
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 v[kScanSmall];
#pragma unroll
  for (int s = 0; s < kScanSmall; ++s) v[s] = s + 1 < spans ? p[(size_t)s * stride] : zero;
  f32x4 run = zero;
#pragma unroll
  for (int s = 0; s < kScanSmall; ++s) {
    if (s < spans) p[(size_t)s * stride] = run;
    run += v[s];
  }
}

// LDS layout (bytes), computed identically on host and device.
// Tokens per chunk of the generic scan.  32: the per-wave numerators
// (NDB x chunk/32 accumulator tiles) and feature fragments of a 64-token
// chunk spill at d = 128 and hold more registers than needed at d <= 64;
// 32-token chunks measured faster at every d.
template <class Tr, int D>
constexpr int generic_chunk() { return 32; }

template <class Tr, int D, int FBW>
struct CausalLds {
  using E = typename Tr::elem;
  static constexpr int C = generic_chunk<Tr, D>();              // tokens per chunk
  static constexpr int RS = Rows<D, sizeof(E)>::RS;             // Q, K, V rows
  static constexpr int FW = 32 * FBW;                           // features per wave
  static constexpr int RSF = FW * (int)sizeof(E) + 16;          // phi(K) rows
  static constexpr int RSR = (D + 4) * 4;                       // reduction rows (float)
  static constexpr int kQ = 0, kK = C * RS, kV = 2 * C * RS, kPhi = 3 * C * RS;
  static constexpr int kStageEnd = kPhi + 4 * C * RSF;
  static constexpr int kRed = 0, kRedDen = 4 * C * RSR;
  static constexpr int kRedEnd = kRedDen + 4 * C * 4;
  static constexpr int kUnion = kStageEnd > kRedEnd ? kStageEnd : kRedEnd;
  static constexpr int kBq = kUnion, kBk = kBq + C * 4, kZ = kBk + C * 4;
  static constexpr int kTotal = kZ + 4 * FW * 4;
};

// Workgroups per compute unit the generic scan is compiled for: two for
// float32 d <= 64 (at most 256 registers; the d = 64 build then keeps 18
// spilled values outside the chunk loop, and ran 13% faster than at one),
// one otherwise.
template <class Tr, int D>
constexpr int generic_wgs() { return (sizeof(typename Tr::elem) == 4 && D <= 64) ? 2 : 1; }

template <class Tr, int D, int FBW, int FM>
__global__ __launch_bounds__(256, (generic_wgs<Tr, D>())) void k_causal(CausalArgs a) {
  using E = typename Tr::elem;
  using F = typename Tr::frag;
  using LY = CausalLds<Tr, D, FBW>;
  constexpr int C = LY::C;
  constexpr int NTB = C / 32;                 // 32-token blocks per chunk
  constexpr int NKD = D / Tr::KS;
  constexpr int NDB = D / 32;
  constexpr int NKT = 32 / Tr::KS;            // k-steps per 32-token block
  constexpr int RS = LY::RS, RSF = LY::RSF, RSR = LY::RSR, FW = LY::FW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* sQ = smem + LY::kQ;
  char* sK = smem + LY::kK;
  char* sV = smem + LY::kV;
  float* sBq = (float*)(smem + LY::kBq);
  float* sBk = (float*)(smem + LY::kBk);

  const int span = blockIdx.x, bh = blockIdx.y;
  const int head = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
  char* sPhi = smem + LY::kPhi + w * C * RSF;          // this wave's phi(K) [token][feature]
  float* sZ = (float*)(smem + LY::kZ) + w * FW;        // this wave's running z (float)
  float* sRed = (float*)(smem + LY::kRed);
  float* sRedDen = (float*)(smem + LY::kRedDen);
  const int nfb = a.M >> 5;
  const size_t hoff = (size_t)bh * a.L * D;
  const E* Qg = (const E*)a.q + hoff;
  const E* Kg = (const E*)a.k + hoff;
  const E* Vg = (const E*)a.v + hoff;
  E* Og = (E*)a.o + hoff;
  const float* wh = a.w + (size_t)(a.Hw == 1 ? 0 : head) * a.mt * D;
  const float half_ln_m = 0.5f * logf((float)a.mt);
  const float tscale = FM == FM_TRIG ? rsqrtf((float)a.mt) : 1.f;
  const bool ragged = a.mt != a.Mw;
  const int t0 = span * a.span_len;
  const int t1 = min(a.L, t0 + a.span_len);

  for (int fg = 0; fg < a.fgroups; ++fg) {
    const int fb0 = (fg * 4 + w) * FBW;
    F wf[FBW][NKD];
    f32x16 st[FBW][NDB];
    float zreg[FBW];
#pragma unroll
    for (int i = 0; i < FBW; ++i) {
      const bool ok = fb0 + i < nfb;
      const int fbase = (ok ? fb0 + i : 0) * 32;
      const int wr = (FM == FM_TRIG ? fbase % a.Mw : fbase) + l32;    // this lane's row of W
      const bool wok = ok && wr < a.mt;
      const float* wrow = wh + (size_t)(wok ? wr : 0) * D;
#pragma unroll
      for (int s = 0; s < NKD; ++s) wf[i][s] = w_frag<Tr, D, FM>(wrow, hh, s, wok);
      const float* pre = a.prefix + ((size_t)bh * a.spans + span) * a.M * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          st[i][db][r] = ok ? pre[(size_t)(fbase + crow(r, hh)) * D + db * 32 + l32] : 0.f;
      zreg[i] = ok ? a.prefixz[((size_t)bh * a.spans + span) * a.M + fbase + l32] : 0.f;
      sZ[i * 32 + l32] = zreg[i];
    }

    TileLoader<E, D, C, 256> lq, lk, lv;
    if (t0 < t1) {
      lq.load(Qg + (size_t)t0 * D, t1 - t0, tid);
      lk.load(Kg + (size_t)t0 * D, t1 - t0, tid);
      lv.load(Vg + (size_t)t0 * D, t1 - t0, tid);
    }
    for (int c0 = t0; c0 < t1; c0 += C) {
      const int nv = min(C, t1 - c0);
      __syncthreads();                                   // previous reduction finished
      lq.store_proj(sQ, tid);
      lk.store_proj(sK, tid);
      lv.store(sV, tid);
      lq.template row_bias<FM>(sBq, tid, nv, half_ln_m);
      lk.template row_bias<FM>(sBk, tid, nv, half_ln_m);
      __syncthreads();
      if (c0 + C < t1) {
        lq.load(Qg + (size_t)(c0 + C) * D, t1 - c0 - C, tid);
        lk.load(Kg + (size_t)(c0 + C) * D, t1 - c0 - C, tid);
        lv.load(Vg + (size_t)(c0 + C) * D, t1 - c0 - C, tid);
      }

      // ---- feature maps of this wave's features, lane = token -------------
      F pq[FBW][NTB][NKT], pk[FBW][NTB][NKT];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        F qf[NKD], kf[NKD];
#pragma unroll
        for (int s = 0; s < NKD; ++s) {
          qf[s] = row_frag<Tr, D>(sQ + (tb * 32 + l32) * RS, hh, s);
          kf[s] = row_frag<Tr, D>(sK + (tb * 32 + l32) * RS, hh, s);
        }
        const float bq = sBq[tb * 32 + l32], bk = sBk[tb * 32 + l32];
#pragma unroll
        for (int i = 0; i < FBW; ++i) {
          f32x16 aq = zero16(), ak = zero16();
#pragma unroll
          for (int s = 0; s < NKD; ++s) {
            aq = Tr::pmma(wf[i][s], qf[s], aq);          // P^T[f][t]
            ak = Tr::pmma(wf[i][s], kf[s], ak);
          }
          // features past m (a partly filled last group) are exactly zero
          const bool fvalid = fb0 + i < nfb;
          const bool cosine = (fb0 + i) * 32 >= a.Mw;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            aq[r] = fvalid ? FMap<FM>::phi(aq[r] + bq, cosine, tscale) : 0.f;
            ak[r] = fvalid ? FMap<FM>::phi(ak[r] + bk, cosine, tscale) : 0.f;
          }
          if (ragged) {
            // padding features (rows of W past m) get phi(K) = 0, which keeps
            // the state, the key sums and the chunk scores free of them
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int f = (fb0 + i) * 32 + crow(r, hh);
              if ((FM == FM_TRIG ? f % a.Mw : f) >= a.mt) ak[r] = 0.f;
            }
          }
#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2) {
            pq[i][tb][s2] = CFrag<Tr>::make(aq, s2);
            pk[i][tb][s2] = CFrag<Tr>::make(ak, s2);
          }
          // phi(K) into this wave's [token][feature] tile (for the state update)
          char* prow = sPhi + (tb * 32 + l32) * RSF + (i * 32) * (int)sizeof(E);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            if constexpr (Tr::VPS == 8) {
              u32x2 v2 = {pack_bf16(ak[4 * g], ak[4 * g + 1]), pack_bf16(ak[4 * g + 2], ak[4 * g + 3])};
              *(u32x2*)(prow + (8 * g + 4 * hh) * 2) = v2;
            } else {
              f32x4 v4 = {ak[4 * g], ak[4 * g + 1], ak[4 * g + 2], ak[4 * g + 3]};
              *(f32x4*)(prow + (8 * g + 4 * hh) * 4) = v4;
            }
          }
        }
      }

      f32x16 nacc[NDB][NTB];
      float dacc[NTB];
#pragma unroll
      for (int tqb = 0; tqb < NTB; ++tqb) {
        dacc[tqb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) nacc[db][tqb] = zero16();
      }

      // ---- intra-chunk: A^T[tk][tq] = phi(K) phi(Q)^T over this wave's features
#pragma unroll
      for (int tqb = 0; tqb < NTB; ++tqb) {
#pragma unroll
        for (int tkb = 0; tkb <= tqb; ++tkb) {
          f32x16 at = zero16();
#pragma unroll
          for (int i = 0; i < FBW; ++i)
#pragma unroll
            for (int s2 = 0; s2 < NKT; ++s2) at = Tr::mma(pk[i][tkb][s2], pq[i][tqb][s2], at);
          if (tkb == tqb) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (crow(r, hh) > l32) at[r] = 0.f;        // key after query
          }
#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2) {
            F af = CFrag<Tr>::make(at, s2);              // B operand: lane = tq, k = tk (c-row)
            if constexpr (Tr::VPS == 8) {
#pragma unroll
              for (int j = 0; j < 4; ++j) dacc[tqb] = dot2_bf16(af[j], 0x3f803f80u, dacc[tqb]);
            } else {
              dacc[tqb] += af;
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              F vf = col_frag<Tr, RS>(sV, tkb * 32, db * 32, s2, lane);   // V^T[d][tk]
              nacc[db][tqb] = Tr::mma(vf, af, nacc[db][tqb]);
            }
          }
        }
      }

      // ---- inter-chunk: phi(Q) S and phi(Q) z with the state before this chunk
#pragma unroll
      for (int i = 0; i < FBW; ++i) {
        float zf[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 z4 = *(const f32x4*)(sZ + i * 32 + 8 * g + 4 * hh);
#pragma unroll
          for (int j = 0; j < 4; ++j) zf[4 * g + j] = z4[j];
        }
#pragma unroll
        for (int s2 = 0; s2 < NKT; ++s2) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            F sf = CFrag<Tr>::make(st[i][db], s2);           // S^T[d][f] operand
#pragma unroll
            for (int tqb = 0; tqb < NTB; ++tqb) nacc[db][tqb] = Tr::mma(sf, pq[i][tqb][s2], nacc[db][tqb]);
          }
#pragma unroll
          for (int tqb = 0; tqb < NTB; ++tqb) {
            if constexpr (Tr::VPS == 8) {
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const unsigned zz = pack_bf16(zf[8 * s2 + 2 * k], zf[8 * s2 + 2 * k + 1]);
                dacc[tqb] = dot2_bf16(pq[i][tqb][s2][k], zz, dacc[tqb]);
              }
            } else {
              dacc[tqb] = fmaf(pq[i][tqb][s2], zf[s2], dacc[tqb]);
            }
          }
        }
      }

      // ---- state update: S += phi(K)^T V, z += phi(K)^T 1 ------------------
#pragma unroll
      for (int i = 0; i < FBW; ++i) {
        float zc = 0.f;
#pragma unroll
        for (int tkb = 0; tkb < NTB; ++tkb)
#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2) {
            F kt = col_frag<Tr, RSF>(sPhi, tkb * 32, i * 32, s2, lane);    // phi(K)^T[f][t]
            if constexpr (Tr::VPS == 8) {
#pragma unroll
              for (int j = 0; j < 4; ++j) zc = dot2_bf16(kt[j], 0x3f803f80u, zc);
            } else {
              zc += kt;
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              F vf = col_frag<Tr, RS>(sV, tkb * 32, db * 32, s2, lane);
              st[i][db] = Tr::mma(kt, vf, st[i][db]);
            }
          }
        zc = half_sum(zc);
        zreg[i] += zc;
      }
      // publish z for the next chunk (wave-private; read after this wave's
      // next feature maps, so LDS order within the wave suffices)
#pragma unroll
      for (int i = 0; i < FBW; ++i)
        if (hh == 0) sZ[i * 32 + l32] = zreg[i];

      // ---- sum the four waves' contributions -------------------------------
      __syncthreads();                                   // staging area is free
#pragma unroll
      for (int tqb = 0; tqb < NTB; ++tqb) {
        float* rrow = sRed + (size_t)w * C * (RSR / 4) + (tqb * 32 + l32) * (RSR / 4);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 v4 = {nacc[db][tqb][4 * g], nacc[db][tqb][4 * g + 1], nacc[db][tqb][4 * g + 2],
                        nacc[db][tqb][4 * g + 3]};
            *(f32x4*)(rrow + db * 32 + 8 * g + 4 * hh) = v4;
          }
        const float dsum = half_sum(dacc[tqb]);
        if (hh == 0) sRedDen[w * C + tqb * 32 + l32] = dsum;
      }
      __syncthreads();
      {
        constexpr int TPR = 256 / C;                     // threads per output row
        constexpr int DP = D / TPR;                      // outputs per thread
        const int tq = tid / TPR, d0 = (tid % TPR) * DP;
        float acc[DP];
#pragma unroll
        for (int j = 0; j < DP; ++j) acc[j] = 0.f;
        float dsum = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const float* rrow = sRed + (size_t)ww * C * (RSR / 4) + tq * (RSR / 4) + d0;
#pragma unroll
          for (int j = 0; j < DP; j += 4) {
            f32x4 v4 = *(const f32x4*)(rrow + j);
            acc[j] += v4[0];
            acc[j + 1] += v4[1];
            acc[j + 2] += v4[2];
            acc[j + 3] += v4[3];
          }
          dsum += sRedDen[ww * C + tq];
        }
        const int tok = c0 + tq;
        if (tq < nv) {
          const size_t oi = (size_t)tok * D + d0;
          if (a.fgroups > 1) {
            if (fg > 0) {
#pragma unroll
              for (int j = 0; j < DP; ++j) acc[j] += a.num[hoff + oi + j];
              dsum += a.den[(size_t)bh * a.L + tok];
            }
            if (fg + 1 < a.fgroups) {
#pragma unroll
              for (int j = 0; j < DP; ++j) a.num[hoff + oi + j] = acc[j];
              if ((tid % TPR) == 0) a.den[(size_t)bh * a.L + tok] = dsum;
            }
          }
          if (fg + 1 == a.fgroups) {
            const float inv = 1.0f / (dsum + a.eps);
#pragma unroll
            for (int j = 0; j < DP; ++j) Og[oi + j] = (E)(acc[j] * inv);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 chunked scan for d <= 64, chunks of C = 32 tokens.  Same split
// of the features over four waves as k_causal, with every operand read as a
// 16-byte fragment and few enough live registers for two workgroups per
// compute unit at C = 32:
//  - the staged chunk buffers are double-buffered: chunk c+1 is stored while
//    chunk c is computed, and its V tile is rearranged into operand order
//    V^T (lane = d, k-slots = tokens in c-row order) once, after the second
//    barrier of iteration c;
//  - phi(K) is brought from lane = token (the projection's layout, used by
//    the intra-chunk scores) to lane = feature (used by the state update) on
//    the matrix cores: multiplying the fragment by the 32 x 32 identity gives
//    the same values with rows and columns exchanged, exactly;
//  - features past m get a bias of -inf, so their phi is exactly zero.
// ---------------------------------------------------------------------------
template <int D, int C>
struct CausalLds2 {
  static constexpr int RS = Rows<D, 2>::RS;             // padded 16-bit rows
  static constexpr int TILE = C * RS;
  // one chunk buffer: Q and K in the projection type, raw V, V^T, row biases
  static constexpr int kQh = 0, kKh = TILE, kV = 2 * TILE, kVT = 3 * TILE;
  static constexpr int kBq = kVT + C * D * 2, kBk = kBq + C * 4;
  static constexpr int BUF = kBk + C * 4;
  static constexpr int RSR = (D + 4) * 4;                // reduction rows (float)
  static constexpr int kRed = 2 * BUF, kRedDen = kRed + 4 * C * RSR;
  static constexpr int kZ = kRedDen + 4 * C * 4;
  static constexpr int kTotal = kZ + 4 * 64 * 4;          // z of 4 waves x 64 features
};

// FM: the feature map (FMap).  FULL (FAVOR+ only): every feature group
// fills all 4 x FBW blocks (M a multiple of 128 FBW), so no block needs the
// -inf bias of a missing feature block and the projection accumulators start
// at the row biases.  RAG: m is not a multiple of 32; padding features
// (rows of W past m) get phi(K) = 0.
template <int D, int FBW, int C, bool FULL, int FM, bool RAG>
__global__ __launch_bounds__(256, 2) void k_causal2(CausalArgs a) {
  using Tr = TrBF16;
  using E = bf16;
  using F = u32x4;
  using LY = CausalLds2<D, C>;
  constexpr int RS = LY::RS, RSR = LY::RSR;
  constexpr int NTB = C / 32;                  // 32-token blocks per chunk
  constexpr int NKD = D / Tr::KS;
  constexpr int NDB = D / 32;
  constexpr int NVT = 2 * NTB * NDB;           // V^T fragments per chunk
  static_assert(FBW * 32 <= 64, "z slots per wave");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* sRed = (float*)(smem + LY::kRed);
  float* sRedDen = (float*)(smem + LY::kRedDen);

  const int span = blockIdx.x, bh = blockIdx.y;
  const int head = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
  float* sZ = (float*)(smem + LY::kZ) + w * 64;           // this wave's running z
  const int nfb = a.M >> 5;
  const size_t hoff = (size_t)bh * a.L * D;
  const E* Qg = (const E*)a.q + hoff;
  const E* Kg = (const E*)a.k + hoff;
  const E* Vg = (const E*)a.v + hoff;
  E* Og = (E*)a.o + hoff;
  const float* wh = a.w + (size_t)(a.Hw == 1 ? 0 : head) * a.mt * D;
  const float half_ln_m = 0.5f * logf((float)a.mt);
  const float tscale = FM == FM_TRIG ? rsqrtf((float)a.mt) : 1.f;
  const int nfbw = a.Mw >> 5;                              // blocks of distinct rows of W
  const int t0 = span * a.span_len;
  const int t1 = min(a.L, t0 + a.span_len);
  if (t0 >= t1) return;                                    // whole workgroup

  // identity operand: slot j of k-step s2 of lane (n, hh) is 1 where feature
  // crow(8 s2 + j, hh) of the block equals n
  F ident[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned lo = crow(8 * s2 + 2 * k, hh) == l32 ? 0x3f80u : 0u;
      const unsigned hi = crow(8 * s2 + 2 * k + 1, hh) == l32 ? 0x3f80u : 0u;
      ident[s2][k] = lo | (hi << 16);
    }

  TileLoader<E, D, C, 256> lq, lk, lv;
  auto load_chunk = [&](int c0) {
    lq.load(Qg + (size_t)c0 * D, t1 - c0, tid);
    lk.load(Kg + (size_t)c0 * D, t1 - c0, tid);
    lv.load(Vg + (size_t)c0 * D, t1 - c0, tid);
  };
  auto store_chunk = [&](char* buf, int nv) {
    lq.store_proj(buf + LY::kQh, tid);
    lk.store_proj(buf + LY::kKh, tid);
    lv.store(buf + LY::kV, tid);
    lq.template row_bias<FM>((float*)(buf + LY::kBq), tid, nv, half_ln_m);
    lk.template row_bias<FM>((float*)(buf + LY::kBk), tid, nv, half_ln_m);
  };
  // V^T fragment (tb, s2, db): lane (d, hh) holds V[32 tb + crow(8 s2 + j, hh)][32 db + d]
  auto vt_at = [&](const char* buf, int tb, int s2, int db) -> const char* {
    return buf + LY::kVT + (((tb * 2 + s2) * 2 + hh) * D + db * 32 + l32) * 16;
  };
  auto transpose_v = [&](char* buf) {
#pragma unroll
    for (int q = w; q < NVT; q += 4) {
      const int tb = q / (2 * NDB), s2 = (q / NDB) % 2, db = q % NDB;
      const int row = tb * 32 + 16 * s2 + 4 * hh + ((lane & 15) >> 2);
      const int col = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      u32x2 r[2];
      lds_read_tr16_1x2<0, 8 * RS>(lds_addr(buf + LY::kV + row * RS + col * 2), r);
      *(u32x4*)vt_at(buf, tb, s2, db) = u32x4{r[0][0], r[0][1], r[1][0], r[1][1]};
    }
  };


  for (int fg = 0; fg < a.fgroups; ++fg) {
    const int fb0 = (fg * 4 + w) * FBW;
    F wf[FBW][NKD];
    f32x16 st[FBW][NDB];
    float zreg[FBW];
    const float* pre = a.prefix + ((size_t)bh * a.spans + span) * a.M * D;
#pragma unroll
    for (int i = 0; i < FBW; ++i) {
      const bool ok = fb0 + i < nfb;
      const int fbase = (ok ? fb0 + i : 0) * 32;
      const int wr = (FM == FM_TRIG ? fbase % a.Mw : fbase) + l32;    // this lane's row of W
      const bool wok = ok && wr < a.mt;
      const float* wrow = wh + (size_t)(wok ? wr : 0) * D;
#pragma unroll
      for (int s = 0; s < NKD; ++s) wf[i][s] = w_frag<Tr, D, FM>(wrow, hh, s, wok);
    }

    // feature maps of this wave's features for the chunk staged in buf,
    // lane = token; computed one chunk ahead (see the chunk loop)
    F pq[FBW][NTB][2], pk[FBW][NTB][2];
    auto feature_maps = [&](const char* buf) {
      const float* sBq = (const float*)(buf + LY::kBq);
      const float* sBk = (const float*)(buf + LY::kBk);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        F qf[NKD], kf[NKD];
#pragma unroll
        for (int s = 0; s < NKD; ++s) {
          qf[s] = row_frag<Tr, D>(buf + LY::kQh + (tb * 32 + l32) * RS, hh, s);
          kf[s] = row_frag<Tr, D>(buf + LY::kKh + (tb * 32 + l32) * RS, hh, s);
        }
        const float bq0 = sBq[tb * 32 + l32], bk0 = sBk[tb * 32 + l32];
        // FULL: both blocks start from the token's bias (lane = token)
        constexpr bool kInit = FULL && FM == FM_POS;
        const f32x16 bq16 = splat16(kInit ? bq0 : 0.f), bk16 = splat16(kInit ? bk0 : 0.f);
#pragma unroll
        for (int i = 0; i < FBW; ++i) {
          const bool fvalid = fb0 + i < nfb;
          const float bq = fvalid ? bq0 : -INFINITY, bk = fvalid ? bk0 : -INFINITY;
          f32x16 aq = bq16, ak = bk16;
#pragma unroll
          for (int s = 0; s < NKD; ++s) {
            aq = Tr::pmma(wf[i][s], qf[s], aq);          // P^T[f][t]
            ak = Tr::pmma(wf[i][s], kf[s], ak);
          }
          const bool cosine = fb0 + i >= nfbw;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            aq[r] = FMap<FM>::phi(kInit ? aq[r] : aq[r] + bq, cosine, tscale);
            ak[r] = FMap<FM>::phi(kInit ? ak[r] : ak[r] + bk, cosine, tscale);
          }
          if constexpr (RAG) {
            // padding features: phi(K) = 0 keeps the state, the key sums and
            // the chunk scores free of them
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int f = (fb0 + i) * 32 + crow(r, hh);
              if ((FM == FM_TRIG ? f % a.Mw : f) >= a.mt) ak[r] = 0.f;
            }
          }
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            pq[i][tb][s2] = CFrag<Tr>::make(aq, s2);
            pk[i][tb][s2] = CFrag<Tr>::make(ak, s2);
          }
        }
      }
    };

    // prologue: chunk 0 into buffer 0 with its V^T, chunk 1 in registers; the
    // span's prefix state (64 KB per workgroup) is requested after the two
    // chunks, so that staging chunk 0 does not wait for it
    load_chunk(t0);
    __syncthreads();                                     // previous feature group fully done
    store_chunk(smem, min(C, t1 - t0));
    if (t0 + C < t1) load_chunk(t0 + C);
#pragma unroll
    for (int i = 0; i < FBW; ++i) {
      const bool ok = fb0 + i < nfb;
      const int fbase = (ok ? fb0 + i : 0) * 32;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          st[i][db][r] = ok ? pre[(size_t)(fbase + crow(r, hh)) * D + db * 32 + l32] : 0.f;
      zreg[i] = ok ? a.prefixz[((size_t)bh * a.spans + span) * a.M + fbase + l32] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < FBW; ++i) sZ[i * 32 + l32] = zreg[i];
    wait_lgkm0();
    raw_barrier();
    transpose_v(smem);
    feature_maps(smem);

    int c = 0;
    for (int c0 = t0; c0 < t1; c0 += C, ++c) {
      const int nv = min(C, t1 - c0);
      char* cur = smem + (c & 1) * LY::BUF;
      char* nxt = smem + ((c + 1) & 1) * LY::BUF;
      wait_lgkm0();
      raw_barrier();                                     // chunk c staged everywhere; last reduction read
      // The two workgroups on a compute unit interleave on every SIMD; the
      // wave between its staging barrier and its partial sums (matrix-core
      // heavy) issues first, and the other wave's reduction and exponentials
      // fill in behind it (measured 10-15% faster than equal priorities).
      __builtin_amdgcn_s_setprio(1);
      // this chunk's V^T fragments, used by the intra-chunk products and the
      // state update, read once
      F vtf[NTB][2][NDB];
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int db = 0; db < NDB; ++db) vtf[tb][s2][db] = *(const F*)vt_at(cur, tb, s2, db);
      // branch-free so that the whole chunk is one scheduling region: past
      // the end the staged rows are zero and no row is loaded
      store_chunk(nxt, min(C, t1 - c0 - C));
      load_chunk(c0 + 2 * C);


      // ---- numerators per 32-query block: intra-chunk scores, then phi(Q) S
#pragma unroll
      for (int tqb = 0; tqb < NTB; ++tqb) {
        f32x16 nacc[NDB];
        float dacc = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) nacc[db] = zero16();
#pragma unroll
        for (int tkb = 0; tkb <= tqb; ++tkb) {
          f32x16 at = zero16();                          // A^T[tk][tq] over this wave's features
#pragma unroll
          for (int i = 0; i < FBW; ++i)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) at = Tr::mma(pk[i][tkb][s2], pq[i][tqb][s2], at);
          if (tkb == tqb) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (crow(r, hh) > l32) at[r] = 0.f;        // key after query
          }
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const F af = CFrag<Tr>::make(at, s2);        // B operand: lane = tq, k = tk (c-row)
#pragma unroll
            for (int j = 0; j < 4; ++j) dacc = dot2_bf16(af[j], 0x3f803f80u, dacc);
#pragma unroll
            for (int db = 0; db < NDB; ++db) nacc[db] = Tr::mma(vtf[tkb][s2][db], af, nacc[db]);
          }
        }
#pragma unroll
        for (int i = 0; i < FBW; ++i) {
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const f32x4 za = *(const f32x4*)(sZ + i * 32 + 16 * s2 + 4 * hh);
            const f32x4 zb = *(const f32x4*)(sZ + i * 32 + 16 * s2 + 8 + 4 * hh);
            const unsigned zz[4] = {pack_bf16(za[0], za[1]), pack_bf16(za[2], za[3]), pack_bf16(zb[0], zb[1]),
                                    pack_bf16(zb[2], zb[3])};
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              nacc[db] = Tr::mma(CFrag<Tr>::make(st[i][db], s2), pq[i][tqb][s2], nacc[db]);   // S^T phi(Q)^T
#pragma unroll
            for (int k = 0; k < 4; ++k) dacc = dot2_bf16(pq[i][tqb][s2][k], zz[k], dacc);
          }
        }
        // this wave's partial numerators and denominators of the block
        float* rrow = sRed + (size_t)w * C * (RSR / 4) + (tqb * 32 + l32) * (RSR / 4);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 v4 = {nacc[db][4 * g], nacc[db][4 * g + 1], nacc[db][4 * g + 2], nacc[db][4 * g + 3]};
            *(f32x4*)(rrow + db * 32 + 8 * g + 4 * hh) = v4;
          }
        sRedDen[w * C + tqb * 32 + l32] = half_sum(dacc);   // both halves write the same value
      }

      // ---- state update: S += phi(K)^T V, z += phi(K)^T 1 ------------------
#pragma unroll
      for (int i = 0; i < FBW; ++i) {
        float zc = 0.f;
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          f32x16 kt = zero16();                          // phi(K) block, lane = feature
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) kt = Tr::mma(pk[i][tb][s2], ident[s2], kt);
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const F ktf = CFrag<Tr>::make(kt, s2);       // A operand: lane = f, k = t (c-row)
#pragma unroll
            for (int j = 0; j < 4; ++j) zc = dot2_bf16(ktf[j], 0x3f803f80u, zc);
#pragma unroll
            for (int db = 0; db < NDB; ++db) st[i][db] = Tr::mma(ktf, vtf[tb][s2][db], st[i][db]);
          }
        }
        zc = half_sum(zc);
        zreg[i] += zc;
      }
      // z for the next chunk (wave-private; LDS keeps this wave's order; both
      // halves hold the same value)
#pragma unroll
      for (int i = 0; i < FBW; ++i) sZ[i * 32 + l32] = zreg[i];

      __builtin_amdgcn_s_setprio(0);
      wait_lgkm0();
      raw_barrier();                                     // partials complete; the next chunk staged
      // The next chunk's feature maps (matrix cores and exponentials) and its
      // V^T go here, where they overlap the reduction's LDS reads and adds;
      // past the end the staged rows are zero and the result is unused.
      feature_maps(nxt);
      if (c0 + C < t1) transpose_v(nxt);
      {
        constexpr int TPR = 256 / C;                     // threads per output row
        constexpr int DP = D / TPR;                      // outputs per thread
        const int tq = tid / TPR, d0 = (tid % TPR) * DP;
        float acc[DP];
#pragma unroll
        for (int j = 0; j < DP; ++j) acc[j] = 0.f;
        float dsum = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const float* rrow = sRed + (size_t)ww * C * (RSR / 4) + tq * (RSR / 4) + d0;
#pragma unroll
          for (int j = 0; j < DP; j += 4) {
            f32x4 v4 = *(const f32x4*)(rrow + j);
            acc[j] += v4[0];
            acc[j + 1] += v4[1];
            acc[j + 2] += v4[2];
            acc[j + 3] += v4[3];
          }
          dsum += sRedDen[ww * C + tq];
        }
        const int tok = c0 + tq;
        if (tq < nv) {
          const size_t oi = (size_t)tok * D + d0;
          if (a.fgroups > 1) {
            if (fg > 0) {
#pragma unroll
              for (int j = 0; j < DP; ++j) acc[j] += a.num[hoff + oi + j];
              dsum += a.den[(size_t)bh * a.L + tok];
            }
            if (fg + 1 < a.fgroups) {
#pragma unroll
              for (int j = 0; j < DP; ++j) a.num[hoff + oi + j] = acc[j];
              if ((tid % TPR) == 0) a.den[(size_t)bh * a.L + tok] = dsum;
            }
          }
          if (fg + 1 == a.fgroups) {
            const float inv = 1.0f / (dsum + a.eps);
            if constexpr (DP % 8 == 0) {
#pragma unroll
              for (int j = 0; j < DP; j += 8)
                *(u32x4*)(Og + oi + j) = u32x4{pack_bf16(acc[j] * inv, acc[j + 1] * inv),
                                               pack_bf16(acc[j + 2] * inv, acc[j + 3] * inv),
                                               pack_bf16(acc[j + 4] * inv, acc[j + 5] * inv),
                                               pack_bf16(acc[j + 6] * inv, acc[j + 7] * inv)};
            } else {
#pragma unroll
              for (int j = 0; j < DP; ++j) Og[oi + j] = (E)(acc[j] * inv);
            }
          }
        }
      }
    }
  }
}

template <class Tr, int D, int FBW, int FM>
static hipError_t causal_t(const Plan& p, const Tensors& t, hipStream_t s) {
  using LY = CausalLds<Tr, D, FBW>;
  float* part = (float*)(t.ws + p.off_part);
  float* partz = (float*)(t.ws + p.off_partz);
  if (p.fbw != FBW) return kErrPlan;
  CausalArgs a{t.q, t.k, t.v, t.w, t.o, part, partz, (float*)(t.ws + p.off_num), (float*)(t.ws + p.off_den),
               p.L, p.M, p.H, p.Hw, p.splits, p.split_len, p.fgroups, t.eps, p.Mw, p.mt};
  timing_begin(FAVOR_KERNEL_CAUSAL, s);
  hipLaunchKernelGGL((k_causal<Tr, D, FBW, FM>), dim3(p.splits, p.BH), dim3(256), (size_t)LY::kTotal, s, a);
  timing_end(FAVOR_KERNEL_CAUSAL, s);
  return hipGetLastError();
}

template <int D, int FBW, int C, bool FULL, int FM, bool RAG>
static hipError_t causal2_t(const Plan& p, const Tensors& t, hipStream_t s);

// the bf16 32-token scan's variant: ragged m, FAVOR+ with whole feature
// groups (bias-initialised projections), or the general case

template <int D, int FM>
static hipError_t causal2_full(const Plan& p, const Tensors& t, hipStream_t s) {
  if (p.mt != p.Mw) return causal2_t<D, 2, 32, false, FM, true>(p, t, s);
  if constexpr (FM == FM_POS) {
    if (p.M % 256 == 0) return causal2_t<D, 2, 32, true, FM, false>(p, t, s);
  }
  return causal2_t<D, 2, 32, false, FM, false>(p, t, s);
}

// bf16 d <= 64: the 32-token scan with two feature blocks per wave; bf16
// d = 128 and float32: the generic scan
template <int FM>
static hipError_t causal_fmap(const Plan& p, const Tensors& t, hipStream_t s) {
  if (p.dt == FAVOR_BF16) {
    switch (p.D) {
      case 32: return causal2_full<32, FM>(p, t, s);
      case 64: return causal2_full<64, FM>(p, t, s);
      case 128: return causal_t<TrBF16, 128, 1, FM>(p, t, s);
    }
  } else {
    switch (p.D) {
      case 32: return causal_t<TrF32, 32, 1, FM>(p, t, s);
      case 64: return causal_t<TrF32, 64, 1, FM>(p, t, s);
      case 128: return causal_t<TrF32, 128, 1, FM>(p, t, s);
    }
  }
  return kErrPlan;
}

template <int D, int FBW, int C, bool FULL, int FM, bool RAG>
static hipError_t causal2_t(const Plan& p, const Tensors& t, hipStream_t s) {
  using LY = CausalLds2<D, C>;
  float* part = (float*)(t.ws + p.off_part);
  float* partz = (float*)(t.ws + p.off_partz);
  if (p.fbw != FBW) return kErrPlan;
  CausalArgs a{t.q, t.k, t.v, t.w, t.o, part, partz, (float*)(t.ws + p.off_num), (float*)(t.ws + p.off_den),
               p.L, p.M, p.H, p.Hw, p.splits, p.split_len, p.fgroups, t.eps, p.Mw, p.mt};
  timing_begin(FAVOR_KERNEL_CAUSAL, s);
  hipLaunchKernelGGL((k_causal2<D, FBW, C, FULL, FM, RAG>), dim3(p.splits, p.BH), dim3(256), (size_t)LY::kTotal, s, a);
  timing_end(FAVOR_KERNEL_CAUSAL, s);
  return hipGetLastError();
}

hipError_t launch_causal(const Plan& p, const Tensors& t, hipStream_t s) {
  float* part = (float*)(t.ws + p.off_part);
  float* partz = (float*)(t.ws + p.off_partz);
  // the last span's aggregate would only feed a prefix past the end
  hipError_t e = launch_reduce(p, t.k, t.v, t.w, part, partz, s, p.splits - 1);
  if (e != hipSuccess) return e;
  const int nq = (p.M * p.D + p.M) / 4;
  timing_begin(FAVOR_KERNEL_SPAN_SCAN, s);
  if (p.splits <= kScanSmall)
    hipLaunchKernelGGL(k_span_scan_small, dim3((nq + 255) / 256, p.BH), dim3(256), 0, s, part, partz, p.splits, p.M,
                       p.D);
  else
    hipLaunchKernelGGL(k_span_scan, dim3((nq + kScanQuads - 1) / kScanQuads, p.BH), dim3(256), 0, s, part, partz,
                       p.splits, p.M, p.D);
  timing_end(FAVOR_KERNEL_SPAN_SCAN, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.scan3) return launch_causal3(p, t, s);
  if (p.x3) return launch_causal_x3(p, t, s);
  switch (p.fmap) {
    case FM_POS: return causal_fmap<FM_POS>(p, t, s);
    case FM_ELU1: return causal_fmap<FM_ELU1>(p, t, s);
    case FM_RELU: return causal_fmap<FM_RELU>(p, t, s);
    case FM_TRIG: return causal_fmap<FM_TRIG>(p, t, s);
    default: return kErrPlan;
  }
}

}  // namespace favor
