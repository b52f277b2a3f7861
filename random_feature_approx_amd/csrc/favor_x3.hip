// Causal FAVOR+ for float32 inputs on the 16-bit matrix cores, d = 128.
//
// Same arithmetic as the other chunked scans (prefix-sum form of the Performer
// study notes' case 2, the key-points normaliser as denominator): for a
// 32-token chunk with queries Q_c, keys K_c, values V_c and the state S, z
// before it,
//   num = tril(phi(Q_c) phi(K_c)^T) V_c + phi(Q_c) S
//   den = rowsum(tril(phi(Q_c) phi(K_c)^T)) + phi(Q_c) z + eps
//   S += phi(K_c)^T V_c,  z += phi(K_c)^T 1.
//
// Every matrix product runs as three 16-bit products with float32
// accumulation: each float32 operand a is split into a = hi + lo, hi the
// 16-bit rounding of a and lo the 16-bit rounding of a - hi, and
//   a b ~ hi_a hi_b + hi_a lo_b + lo_a hi_b
// (the dropped lo_a lo_b and the rounding of lo leave ~2^-16 of |a b| with
// bf16 halves, ~2^-21 with fp16 halves).  The projection W x takes fp16
// halves: its result is an exponent, so its error is an absolute error of
// the feature; x and W log2 e fit fp16's range (rows with |x|^2 > 2^20 are
// given phi = 0 outright: with every row of W shorter than 256 their
// exponent is below -2^18, far under float32's smallest value).  Features,
// scores, S and V take bf16 halves, which keep float32's exponent range.
// One 16-bit product is 16 times the rate of a float32 one (32x32x16 in ~32
// cycles against 32x32x2 in ~64), so the three of them cost a fifth.
//
// Work split: a workgroup walks one span of tokens, feature group after
// feature group (128 features per group).  In each chunk wave w
//   1. projects its own 32 features of the group for Q and K (lane = token),
//      applies exp2, and publishes phi(Q) and phi(K)^T (transposed on the
//      matrix cores by a permutation matrix, exactly) as split fragments in
//      LDS, with its partial scores over its features and its partial
//      denominator phi(Q) z over them;
//   2. after a barrier, owns the 32 columns d in [32 w, 32 w + 32): sums the
//      four partial score tiles, and computes that column block of
//      tril(A) V + phi(Q) S over all 128 features of the group, then
//      S[:, block] += phi(K)^T V[:, block].
// So a wave's numerator needs no sum with other waves; groups after the
// first add their numerators to the previous groups' in the workspace.
#include "favor_device.hpp"
#include "favor_internal.hpp"
#include "favor_tiles.hpp"

namespace favor {

namespace x3 {

// fourth word of a raw buffer resource on gfx9 (32-bit data format, no swizzle)
constexpr int kX3Word3 = 0x00020000;

__device__ __forceinline__ float f16_lo(unsigned u) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(u & 0xffffu));
}
__device__ __forceinline__ float f16_hi(unsigned u) { return (float)__builtin_bit_cast(_Float16, (unsigned short)(u >> 16)); }

// two floats as fp16 halves: hi = fp16(a), lo = fp16(a - hi)
__device__ __forceinline__ void split_f16(float a, float b, unsigned& hi, unsigned& lo) {
  hi = pack_f16(a, b);
  lo = pack_f16(a - f16_lo(hi), b - f16_hi(hi));
}
// two floats as bf16 halves (a - hi is exact in float32)
__device__ __forceinline__ void split_bf16(float a, float b, unsigned& hi, unsigned& lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - bf16_lo(hi), b - bf16_hi(hi));
}
// k-step s of a 32-row accumulator block (c-row order) as bf16 halves
__device__ __forceinline__ void split_frag(const f32x16& v, int s, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    unsigned h, l;
    split_bf16(v[8 * s + 2 * k], v[8 * s + 2 * k + 1], h, l);
    hi[k] = h;
    lo[k] = l;
  }
}

__device__ __forceinline__ f32x16 mma_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// c + a b with both operands split: hi hi + hi lo + lo hi
__device__ __forceinline__ f32x16 mma3_bf16(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x16 c) {
  c = mma_bf16(al, bh, c);
  c = mma_bf16(ah, bl, c);
  return mma_bf16(ah, bh, c);
}

// k-steps of one W row (lane = feature, d-major slots) as fp16 halves of
// W log2 e, clamped to fp16's range; zero when !ok
template <int D>
__device__ __forceinline__ void w_frags_f16(const float* wrow, int hh, bool ok, u32x4 (&fh)[D / 16], u32x4 (&fl)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const int d0 = (D / 2) * hh + 8 * s;
    const f32x4 p0 = ok ? *(const f32x4*)(wrow + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 p1 = ok ? *(const f32x4*)(wrow + d0 + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    const float v[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      unsigned h, l;
      split_f16(fminf(fmaxf(v[2 * k] * kLog2e, -65504.f), 65504.f),
                fminf(fmaxf(v[2 * k + 1] * kLog2e, -65504.f), 65504.f), h, l);
      fh[s][k] = h;
      fl[s][k] = l;
    }
  }
}

}  // namespace x3
using namespace x3;

template <int D>
struct X3Lds {
  static constexpr int C = 32;                          // tokens per chunk
  static constexpr int NW = 4;                          // waves; 32 features each per group
  static constexpr int RSX = D * 2 + 16;                // fp16 rows of Q and K (odd number of 16-byte chunks)
  static constexpr int FRAG = 64 * 16;                  // one 16-byte fragment per lane
  static constexpr int RAW = C * D * 4;                 // one dense float32 tile as copied from memory
  // staged chunk: Q and K as fp16 halves with their row biases; the copies
  // of the next chunk's Q and K, and V (two chunks: the current one is read
  // while the next one lands)
  static constexpr int kQh = 0, kQl = kQh + C * RSX, kKh = kQl + C * RSX, kKl = kKh + C * RSX;
  static constexpr int kBq = kKl + C * RSX, kBk = kBq + C * 4;
  static constexpr int kRawQ = kBk + C * 4, kRawK = kRawQ + RAW, kRawV = kRawK + RAW;
  // published by the waves in step 1: phi(Q) [k-step of the group][hi, lo],
  // phi(K)^T [feature block][k-step over tokens][hi, lo], partial score tiles
  // [wave][4 x f32x4 per lane], partial denominators [wave][token], and each
  // wave's running key sums [wave][feature]
  static constexpr int kPhiQ = kRawV + 2 * RAW;
  static constexpr int kPhiK = kPhiQ + 2 * NW * 2 * FRAG;
  static constexpr int kA = kPhiK + NW * 2 * 2 * FRAG;
  static constexpr int kDen = kA + NW * 16 * 64 * 4;
  static constexpr int kZ = kDen + NW * C * 4;
  static constexpr int kIdent = kZ + NW * 32 * 4;       // [k-step][lane] permutation fragments
  static constexpr int kTotal = kIdent + 2 * FRAG;
};

// The scan.  CausalArgs as for the other scans; `den` holds one copy of the
// partial denominators per wave ([4][BH][L]) when there are several feature
// groups, so each wave reads back only what it wrote.
template <int D>
__global__ __launch_bounds__(256, 1) void k_causal_x3(CausalArgs a) {
  using LY = X3Lds<D>;
  constexpr int C = LY::C, NW = LY::NW;
  constexpr int NKD = D / 16;                 // projection k-steps
  constexpr int RSX = LY::RSX;
  static_assert(D == 128, "one 32-column block of d per wave");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* sBq = (float*)(smem + LY::kBq);
  float* sBk = (float*)(smem + LY::kBk);

  const int span = blockIdx.x, bh = blockIdx.y;
  const int head = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int nfb = a.M >> 5;
  const size_t hoff = (size_t)bh * a.L * D;
  const float* wh = a.w + (size_t)(a.Hw == 1 ? 0 : head) * a.mt * D;
  const float half_ln_m = 0.5f * logf((float)a.mt);
  const bool ragged = a.mt != a.Mw;
  const int t0 = span * a.span_len;
  const int t1 = min(a.L, t0 + a.span_len);
  const int nch = (t1 - t0 + C - 1) / C;
  if (nch <= 0) return;

  // Buffer resources over the span's output rows and carried numerators:
  // writes past its last token are dropped.  Byte counts fit 32 bits
  // (L d < 2^30).
  const unsigned span_bytes = (unsigned)(t1 - t0) * D * 4u;
  auto rsrc = [&](const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, kX3Word3);
  };
  const auto ro = rsrc((float*)a.o + hoff + (size_t)t0 * D, span_bytes);
  const auto rn = rsrc(a.num + hoff + (size_t)t0 * D, span_bytes);
  const auto rd = rsrc(a.den + ((size_t)w * gridDim.y + bh) * a.L + t0, (unsigned)(t1 - t0) * 4u);

  // Copies of a chunk's Q, K and V rows straight into LDS (dense tiles).
  // Each of the 16 copy instructions of a tile moves 64 x 16 bytes (two
  // rows); wave w issues instructions w, w + 4, ...  Rows past the span
  // re-read the chunk's first row, so every address is valid: their
  // features get a bias of -inf and come out exactly zero.
  const float* Qs = (const float*)a.q + hoff + (size_t)t0 * D;
  const float* Ks = (const float*)a.k + hoff + (size_t)t0 * D;
  const float* Vs = (const float*)a.v + hoff + (size_t)t0 * D;
  auto copy_chunk = [&](int ci) {
    const int nvalid = t1 - (t0 + ci * C);
#pragma unroll
    for (int i = 0; i < LY::RAW / 1024 / NW; ++i) {
      const int blk = i * NW + w;
      const int P = blk * 64 + lane, row = P / 32;
      const size_t off = (size_t)(ci * C + (row < nvalid ? row : 0)) * D + (P % 32) * 4;
      __builtin_amdgcn_global_load_lds(FAVOR_GLB(Qs + off), LDS_PTR(void, smem + LY::kRawQ + blk * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(FAVOR_GLB(Ks + off), LDS_PTR(void, smem + LY::kRawK + blk * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(FAVOR_GLB(Vs + off),
                                       LDS_PTR(void, smem + LY::kRawV + (ci & 1) * LY::RAW + blk * 1024), 16, 0, 0);
    }
  };
  // Q and K rows of the copied chunk as fp16 halves, with the row bias
  // -(|x|^2/2 + ln(m)/2) log2 e (-inf for rows past the span, and for rows
  // with |x|^2 > 2^20, which are zeroed).  Thread t owns
  // the 16-byte chunks (t / 32 + 8 i, t % 32): a row's chunks sit in 32
  // consecutive lanes.
  constexpr int CPR = D * 4 / 16;
  static_assert(CPR == 32 && C * CPR == 4 * 256, "a row's chunks fill half a wave");
  const int srow = tid / CPR, scc = tid % CPR;
  auto stage_rows = [&](int raw, int kh, int kl, float* sb, int nvalid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = srow + 8 * i;
      f32x4 x = *(const f32x4*)(smem + raw + row * D * 4 + scc * 16);
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) ss = fmaf(x[j], x[j], ss);
      ss = group_sum<CPR>(ss);
      const bool big = ss > 1048576.f;
      if (__builtin_amdgcn_ballot_w64(big)) {                // rare: zero such rows
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = big ? 0.f : x[j];
      }
      u32x2 hi, lo;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        unsigned h, l;
        split_f16(x[2 * j], x[2 * j + 1], h, l);
        hi[j] = h;
        lo[j] = l;
      }
      *(u32x2*)(smem + kh + row * RSX + scc * 8) = hi;
      *(u32x2*)(smem + kl + row * RSX + scc * 8) = lo;
      if (scc == 0) sb[row] = (row < nvalid && !big) ? -(0.5f * ss + half_ln_m) * kLog2e : -INFINITY;
    }
  };
  auto stage_chunk = [&](int ci) {
    const int nvalid = t1 - (t0 + ci * C);
    stage_rows(LY::kRawQ, LY::kQh, LY::kQl, sBq, nvalid);
    stage_rows(LY::kRawK, LY::kKh, LY::kKl, sBk, nvalid);
  };

  // permutation matrix taking phi(K) (lane = token, k-slots = features in
  // c-row order) to phi(K)^T (lane = feature): k-step s2, slot j of lane half
  // h holds feature crow(8 s2 + j, h); lane f gets a 1 where that equals f.
  // Kept in LDS (two fragments) and read where it is used.
  if (tid < 128) {
    const int s2 = tid >> 6;
    u32x4 id;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned lo = crow(8 * s2 + 2 * k, hh) == l32 ? 0x3f80u : 0u;
      const unsigned hi = crow(8 * s2 + 2 * k + 1, hh) == l32 ? 0x3f80u : 0u;
      id[k] = lo | (hi << 16);
    }
    *(u32x4*)(smem + LY::kIdent + tid * 16) = id;
  }
  char* phiq = smem + LY::kPhiQ;
  char* phik = smem + LY::kPhiK;
  float* sA = (float*)(smem + LY::kA);
  float* sDen = (float*)(smem + LY::kDen);
  float* sZ = (float*)(smem + LY::kZ) + w * 32;

  for (int fg = 0; fg < a.fgroups; ++fg) {
    // ---- this wave's feature block: W rows as fp16 halves of W log2 e ----
    const int fb = fg * NW + w;
    const bool fvalid = fb < nfb;
    u32x4 wfh[NKD], wfl[NKD];
    {
      const int wr = fb * 32 + l32;
      const bool wok = fvalid && wr < a.mt;
      w_frags_f16<D>(wh + (size_t)(wok ? wr : 0) * D, hh, wok, wfh, wfl);
    }
    // ---- this wave's column block of S (all features of the group) and the
    // key sums of its own features, from the span's prefix ----
    f32x16 st[NW];
    const float* pre = a.prefix + ((size_t)bh * a.spans + span) * a.M * D;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int fbj = fg * NW + j;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        st[j][r] = fbj < nfb ? pre[(size_t)(fbj * 32 + crow(r, hh)) * D + w * 32 + l32] : 0.f;
    }
    float zown = fvalid ? a.prefixz[((size_t)bh * a.spans + span) * a.M + fb * 32 + l32] : 0.f;
    if (hh == 0) sZ[l32] = zown;

    // A wave stages exactly the Q and K rows it copies (rows 2 w + 8 i and
    // 2 w + 8 i + 1), so the copies of chunk ci + 2 are issued as soon as the
    // wave has staged chunk ci + 1, a whole chunk before they are needed;
    // the V tile of a chunk is read by every wave and has two slots.
    copy_chunk(0);
    wait_vmcnt<0>();
    stage_chunk(0);
    if (nch > 1) {
      wait_lgkm0();                           // the staging reads of chunk 0 done
      copy_chunk(1);
    }
    for (int ci = 0; ci < nch; ++ci) {
      wait_lgkm0();
      raw_barrier();                          // chunk ci staged, its V landed; last chunk's step 2 done
      const float* sV = (const float*)(smem + LY::kRawV + (ci & 1) * LY::RAW);

      // ---- step 1: own features --------------------------------------------
      // projections P^T[f][t] (lane = token), started at the row biases
      f32x16 aq = splat16(sBq[l32]), ak = splat16(sBk[l32]);
#pragma unroll
      for (int s = 0; s < NKD; ++s) {
        const int xo = l32 * RSX + ((D / 2) * hh + 8 * s) * 2;
        const u32x4 qh = *(const u32x4*)(smem + LY::kQh + xo), ql = *(const u32x4*)(smem + LY::kQl + xo);
        const u32x4 kh = *(const u32x4*)(smem + LY::kKh + xo), kl = *(const u32x4*)(smem + LY::kKl + xo);
        aq = mma_f16(wfl[s], qh, aq);
        ak = mma_f16(wfl[s], kh, ak);
        aq = mma_f16(wfh[s], ql, aq);
        ak = mma_f16(wfh[s], kl, ak);
        aq = mma_f16(wfh[s], qh, aq);
        ak = mma_f16(wfh[s], kh, ak);
      }
      if (fvalid) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          aq[r] = exp2_fast(aq[r]);
          ak[r] = exp2_fast(ak[r]);
        }
      } else {
        aq = zero16();                        // a feature block past m (last group)
        ak = zero16();
      }
      if (ragged) {
        // padding features (rows of W past m): phi(K) = 0 keeps them out of
        // the state, the key sums and the scores
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (fb * 32 + crow(r, hh) >= a.mt) ak[r] = 0.f;
      }
      // partial denominator over own features with z before this chunk
      float dq = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 z4 = *(const f32x4*)(sZ + 8 * g + 4 * hh);
#pragma unroll
        for (int j = 0; j < 4; ++j) dq = fmaf(aq[4 * g + j], z4[j], dq);
      }
      u32x4 pqh[2], pql[2], pkh[2], pkl[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        split_frag(aq, s2, pqh[s2], pql[s2]);
        *(u32x4*)(phiq + ((2 * w + s2) * 2 + 0) * LY::FRAG + lane * 16) = pqh[s2];
        *(u32x4*)(phiq + ((2 * w + s2) * 2 + 1) * LY::FRAG + lane * 16) = pql[s2];
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) split_frag(ak, s2, pkh[s2], pkl[s2]);
      // partial scores A^T[tk][tq] over own features (lane = tq), causal mask
      {
        f32x16 at = zero16();
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) at = mma3_bf16(pkh[s2], pkl[s2], pqh[s2], pql[s2], at);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (crow(r, hh) > l32) at[r] = 0.f;
          dq += at[r];
        }
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(sA + ((w * 4 + g) * 64 + lane) * 4) = f32x4{at[4 * g], at[4 * g + 1], at[4 * g + 2], at[4 * g + 3]};
      }
      dq = half_sum(dq);
      if (hh == 0) sDen[w * C + l32] = dq;
      // phi(K)^T on the matrix cores (exact: one nonzero product per value),
      // the hi halves, then the lo halves; their sums update z
      float zc = 0.f;
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        f32x16 tt = zero16();
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          tt = mma_bf16(part == 0 ? pkh[s2] : pkl[s2], *(const u32x4*)(smem + LY::kIdent + (s2 * 64 + lane) * 16), tt);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4 kt;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            kt[k] = pack_bf16(tt[8 * s2 + 2 * k], tt[8 * s2 + 2 * k + 1]);
            zc = dot2_bf16(kt[k], 0x3f803f80u, zc);
          }
          *(u32x4*)(phik + ((w * 2 + s2) * 2 + part) * LY::FRAG + lane * 16) = kt;
        }
      }
      zown += half_sum(zc);
      if (hh == 0) sZ[l32] = zown;           // read again only by this wave, after this chunk

      // V^T fragments of this wave's column block, as bf16 halves: lane = d,
      // k-slots = tokens in c-row order
      u32x4 vth[2], vtl[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float vv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) vv[j] = sV[(16 * s2 + 8 * (j >> 2) + 4 * hh + (j & 3)) * D + w * 32 + l32];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          unsigned h, l;
          split_bf16(vv[2 * k], vv[2 * k + 1], h, l);
          vth[s2][k] = h;
          vtl[s2][k] = l;
        }
      }
      wait_lgkm0();
      raw_barrier();                          // every wave's step 1 published

      // ---- step 2: own column block over the group's features ----------------
      if (ci + 1 < nch) {
        wait_vmcnt<0>();                      // this wave's copies of chunk ci + 1 (and older stores)
        stage_chunk(ci + 1);                  // the staging area is no longer read this chunk
      }
      // earlier feature groups' numerators and denominators of these rows
      // (loaded before the next copies, so waiting for them does not wait
      // for the copies)
      const unsigned orow = (unsigned)(ci * C + l32) * D * 4u;
      u32x4 prev[4];
      float prevd = 0.f;
      const bool carry_in = a.fgroups > 1 && fg > 0;
      if (carry_in) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          prev[g] = __builtin_amdgcn_raw_buffer_load_b128(rn, (int)(orow + (w * 32 + 8 * g + 4 * hh) * 4u), 0, 0);
        prevd = as_f32(__builtin_amdgcn_raw_buffer_load_b32(rd, (int)((ci * C + l32) * 4u), 0, 0));
      }
      if (ci + 2 < nch) {
        wait_lgkm0();                         // own staging reads done before the copies overwrite them
        copy_chunk(ci + 2);                   // V slot ci & 1: chunk ci's V was read before the barrier
      }
      f32x16 af = zero16();
#pragma unroll
      for (int ww = 0; ww < NW; ++ww)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v4 = *(const f32x4*)(sA + ((ww * 4 + g) * 64 + lane) * 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) af[4 * g + j] += v4[j];
        }
      f32x16 nacc = zero16();
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 ah, al;
        split_frag(af, s2, ah, al);
        nacc = mma3_bf16(vth[s2], vtl[s2], ah, al, nacc);          // [d][tq]
      }
#pragma unroll
      for (int j = 0; j < NW; ++j)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4 sh, sl;
          split_frag(st[j], s2, sh, sl);                            // S^T[d][f]
          const u32x4 qh = *(const u32x4*)(phiq + ((2 * j + s2) * 2 + 0) * LY::FRAG + lane * 16);
          const u32x4 ql = *(const u32x4*)(phiq + ((2 * j + s2) * 2 + 1) * LY::FRAG + lane * 16);
          nacc = mma3_bf16(sh, sl, qh, ql, nacc);
        }
#pragma unroll
      for (int j = 0; j < NW; ++j)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const u32x4 kh = *(const u32x4*)(phik + ((j * 2 + s2) * 2 + 0) * LY::FRAG + lane * 16);
          const u32x4 kl = *(const u32x4*)(phik + ((j * 2 + s2) * 2 + 1) * LY::FRAG + lane * 16);
          st[j] = mma3_bf16(kh, kl, vth[s2], vtl[s2], st[j]);      // S[f][d] += phi(K)^T V
        }
      float den = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) den += sDen[ww * C + l32];

      // ---- output rows of this chunk: lane = token, values = d ---------------
      if (a.fgroups > 1) {
        if (carry_in) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j) nacc[4 * g + j] += as_f32(prev[g][j]);
          den += prevd;
        }
        if (fg + 1 < a.fgroups) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{as_u32(nacc[4 * g]), as_u32(nacc[4 * g + 1]), as_u32(nacc[4 * g + 2]), as_u32(nacc[4 * g + 3])},
                rn, (int)(orow + (w * 32 + 8 * g + 4 * hh) * 4u), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(as_u32(den), rd, (int)((ci * C + l32) * 4u), 0, 0);
        }
      }
      if (fg + 1 == a.fgroups) {
        const float inv = __builtin_amdgcn_rcpf(den + a.eps);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          __builtin_amdgcn_raw_buffer_store_b128(
              u32x4{as_u32(nacc[4 * g] * inv), as_u32(nacc[4 * g + 1] * inv), as_u32(nacc[4 * g + 2] * inv),
                    as_u32(nacc[4 * g + 3] * inv)},
              ro, (int)(orow + (w * 32 + 8 * g + 4 * hh) * 4u), 0, 0);
      }
    }
  }
}

// ===========================================================================
// Span aggregates for the float32 scan on the same split products:
//   part[f][d] = sum_t phi(k_t)[f] v_t[d],  partz[f] = sum_t phi(k_t)[f]
// over the tokens of a span (the K-side reduction of the Performer page's
// linear-attention form, restricted to the span).  Eight waves each own 32
// features; 32-token tiles of K and V are copied into LDS (two slots), and
// each tile is prepared once for all waves: K as fp16 halves with its row
// biases, V as bf16-half V^T fragments.  Per tile a wave issues 24 fp16
// products (projection, lane = feature, so phi(K)^T needs no transpose) and
// 24 bf16 products (state update).
// ===========================================================================
template <int D>
struct RedX3Lds {
  static constexpr int TT = 32;                         // tokens per tile
  static constexpr int NW = 8;
  static constexpr int NDB = D / 32;
  static constexpr int RAW = TT * D * 4;                // one dense float32 tile
  static constexpr int RSX = D * 2 + 16;                // fp16 rows of K (odd number of 16-byte chunks)
  static constexpr int FRAG = 64 * 16;
  static constexpr int kKh = 0, kKl = TT * RSX;
  static constexpr int kVT = 2 * TT * RSX;              // [d block][k-step][hi, lo][lane] fragments
  static constexpr int kBias = kVT + NDB * 2 * 2 * FRAG;
  static constexpr int PREP = kBias + TT * 4;
  static constexpr int kRaw = 2 * PREP;                 // two prepared tiles, then two raw K|V slots
  static constexpr int kTotal = kRaw + 2 * 2 * RAW;
};

template <int D>
__global__ __launch_bounds__(512, 1) void k_reduce_x3(RedArgs a) {
  using LY = RedX3Lds<D>;
  constexpr int TT = LY::TT, NW = LY::NW, NT = NW * 64, NKD = D / 16, NDB = LY::NDB, RSX = LY::RSX;
  constexpr int CPR = D * 4 / 16;                       // 16-byte chunks per float32 row
  static_assert(D == 128 && TT * CPR == 2 * NT && NDB * 2 == NW, "tile split over the threads");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int split = blockIdx.x, fg = blockIdx.y, bh = blockIdx.z;
  const int head = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nfb = a.M >> 5;
  const int fb = fg * NW + w;
  const bool fvalid = fb < nfb;
  const float* K = (const float*)a.k + (size_t)bh * a.L * D;
  const float* V = (const float*)a.v + (size_t)bh * a.L * D;
  const float* wh = a.w + (size_t)(a.Hw == 1 ? 0 : head) * a.mt * D;
  const float half_ln_m = 0.5f * logf((float)a.mt);
  const int f = fb * 32 + l32;                          // this lane's feature
  const bool wok = fvalid && f < a.mt;

  u32x4 wfh[NKD], wfl[NKD];
  w_frags_f16<D>(wh + (size_t)(wok ? f : 0) * D, hh, wok, wfh, wfl);
  f32x16 st[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) st[db] = zero16();
  float zs = 0.f;

  const int t0 = split * a.split_len;
  const int t1 = min(a.L, t0 + a.split_len);
  const int ntiles = t0 < t1 ? (t1 - t0 + TT - 1) / TT : 0;

  // copies of tile tt into raw slot tt & 1 (rows past the span re-read the
  // tile's first row); each wave issues 2 of the 16 1-KB blocks of K and of V
  auto copy = [&](int tt) {
    const int r0 = t0 + tt * TT, nvalid = t1 - r0;
    char* slot = smem + LY::kRaw + (tt & 1) * 2 * LY::RAW;
#pragma unroll
    for (int i = 0; i < LY::RAW / 1024 / NW; ++i) {
      const int blk = i * NW + w;
      const int P = blk * 64 + lane, row = P / CPR;
      const size_t off = (size_t)(r0 + (row < nvalid ? row : 0)) * D + (P % CPR) * 4;
      __builtin_amdgcn_global_load_lds(FAVOR_GLB(K + off), LDS_PTR(void, slot + blk * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(FAVOR_GLB(V + off), LDS_PTR(void, slot + LY::RAW + blk * 1024), 16, 0, 0);
    }
  };
  // raw slot tt & 1 -> prepared buffer tt & 1
  auto prepare = [&](int tt) {
    const char* raw = smem + LY::kRaw + (tt & 1) * 2 * LY::RAW;
    char* pb = smem + (tt & 1) * LY::PREP;
    float* bias = (float*)(pb + LY::kBias);
    const int nvalid = t1 - (t0 + tt * TT);
#pragma unroll
    for (int i = 0; i < 2; ++i) {                       // K: chunks (tid / 32 + 16 i, tid % 32)
      const int row = tid / CPR + (NT / CPR) * i, cc = tid % CPR;
      f32x4 x = *(const f32x4*)(raw + row * D * 4 + cc * 16);
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) ss = fmaf(x[j], x[j], ss);
      ss = group_sum<CPR>(ss);
      const bool big = ss > 1048576.f;
      if (__builtin_amdgcn_ballot_w64(big)) {          // rare: zero such rows
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = big ? 0.f : x[j];
      }
      u32x2 hi, lo;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        unsigned h, l;
        split_f16(x[2 * j], x[2 * j + 1], h, l);
        hi[j] = h;
        lo[j] = l;
      }
      *(u32x2*)(pb + LY::kKh + row * RSX + cc * 8) = hi;
      *(u32x2*)(pb + LY::kKl + row * RSX + cc * 8) = lo;
      if (cc == 0) bias[row] = (row < nvalid && !big) ? -(0.5f * ss + half_ln_m) * kLog2e : -INFINITY;
    }
    {                                                   // V^T fragment w (d block w / 2, k-step w % 2), lane
      const int db = w >> 1, s2 = w & 1;
      const float* rv = (const float*)(raw + LY::RAW);
      float vv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) vv[j] = rv[(16 * s2 + 8 * (j >> 2) + 4 * hh + (j & 3)) * D + db * 32 + l32];
      u32x4 vh, vl;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        unsigned h, l;
        split_bf16(vv[2 * k], vv[2 * k + 1], h, l);
        vh[k] = h;
        vl[k] = l;
      }
      *(u32x4*)(pb + LY::kVT + (w * 2 + 0) * LY::FRAG + lane * 16) = vh;
      *(u32x4*)(pb + LY::kVT + (w * 2 + 1) * LY::FRAG + lane * 16) = vl;
    }
  };

  if (ntiles > 0) {
    copy(0);
    wait_vmcnt<0>();
    raw_barrier();
    prepare(0);
    if (ntiles > 1) copy(1);
  }
  for (int tt = 0; tt < ntiles; ++tt) {
    wait_vmcnt<0>();                          // this wave's copies of tile tt + 1 landed
    wait_lgkm0();                             // this wave's preparation of tile tt written
    raw_barrier();                            // ... everywhere; tile tt - 1 fully consumed
    if (tt + 1 < ntiles) prepare(tt + 1);
    if (fvalid) {
      const char* pb = smem + (tt & 1) * LY::PREP;
      const float* sb = (const float*)(pb + LY::kBias);
      // P[t][f] + bias[t]: lane = feature, values = tokens (c-row order)
      f32x16 acc;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 b4 = *(const f32x4*)(sb + 8 * g + 4 * hh);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[4 * g + j] = b4[j];
      }
#pragma unroll
      for (int s = 0; s < NKD; ++s) {
        const int xo = l32 * RSX + ((D / 2) * hh + 8 * s) * 2;
        const u32x4 kh = *(const u32x4*)(pb + LY::kKh + xo), kl = *(const u32x4*)(pb + LY::kKl + xo);
        acc = mma_f16(kl, wfh[s], acc);
        acc = mma_f16(kh, wfl[s], acc);
        acc = mma_f16(kh, wfh[s], acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = wok ? exp2_fast(acc[r]) : 0.f;
      u32x4 ph[2], pl[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        split_frag(acc, s2, ph[s2], pl[s2]);
#pragma unroll
        for (int k = 0; k < 4; ++k) zs = dot2_bf16(pl[s2][k], 0x3f803f80u, dot2_bf16(ph[s2][k], 0x3f803f80u, zs));
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const u32x4 vh = *(const u32x4*)(pb + LY::kVT + ((db * 2 + s2) * 2 + 0) * LY::FRAG + lane * 16);
          const u32x4 vl = *(const u32x4*)(pb + LY::kVT + ((db * 2 + s2) * 2 + 1) * LY::FRAG + lane * 16);
          st[db] = mma3_bf16(ph[s2], pl[s2], vh, vl, st[db]);   // S[f][d]
        }
    }
    if (tt + 2 < ntiles) copy(tt + 2);        // raw slot tt & 1 was prepared before the barrier
  }

  if (fvalid) {
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

hipError_t launch_reduce_x3(const Plan& p, const void* k, const void* v, const float* w, float* part, float* partz,
                            hipStream_t s, int nsplit) {
  if (!p.x3 || p.D != 128 || p.rnw != RedX3Lds<128>::NW || p.rfbw != 1) return kErrPlan;
  RedArgs a{k, v, w, part, partz, p.L, p.M, p.H, p.Hw, p.splits, p.split_len, p.Mw, p.mt};
  timing_begin(FAVOR_KERNEL_REDUCE, s);
  hipLaunchKernelGGL(k_reduce_x3<128>, dim3(nsplit, p.rfgroups, p.BH), dim3(RedX3Lds<128>::NW * 64),
                     (size_t)RedX3Lds<128>::kTotal, s, a);
  timing_end(FAVOR_KERNEL_REDUCE, s);
  return hipGetLastError();
}

hipError_t launch_causal_x3(const Plan& p, const Tensors& t, hipStream_t s) {
  if (!p.x3 || p.D != 128 || p.fbw != 1 || p.fgroups != (p.M / 32 + 3) / 4) return kErrPlan;
  float* part = (float*)(t.ws + p.off_part);
  float* partz = (float*)(t.ws + p.off_partz);
  CausalArgs a{t.q, t.k, t.v, t.w, t.o, part, partz, (float*)(t.ws + p.off_num), (float*)(t.ws + p.off_den),
               p.L, p.M, p.H, p.Hw, p.splits, p.split_len, p.fgroups, t.eps, p.Mw, p.mt};
  timing_begin(FAVOR_KERNEL_CAUSAL, s);
  hipLaunchKernelGGL(k_causal_x3<128>, dim3(p.splits, p.BH), dim3(256), (size_t)X3Lds<128>::kTotal, s, a);
  timing_end(FAVOR_KERNEL_CAUSAL, s);
  return hipGetLastError();
}

}  // namespace favor
