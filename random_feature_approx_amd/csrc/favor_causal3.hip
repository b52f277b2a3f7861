// Causal FAVOR+ chunk scan for the common shape: bf16, d in {32, 64},
// m = 256, positive features (FAVOR+), two workgroups per compute unit.
//
// Same arithmetic as the scans in favor_causal.hip (prefix-sum form of the
// Performer study notes' case 2, with the key-points normaliser as
// denominator): for a 32-token chunk c with queries Q_c, keys K_c, values V_c
// and the state S, z before it,
//   num = tril(phi(Q_c) phi(K_c)^T) V_c + phi(Q_c) S
//   den = rowsum(tril(phi(Q_c) phi(K_c)^T)) + phi(Q_c) z + eps
//   S += phi(K_c)^T V_c,  z += phi(K_c)^T 1.
// Four waves each own 64 of the 256 features and their 64 x d slice of S in
// registers; a chunk's output is the sum of the four waves' partials.
//
// The kernel is bound by vector (VALU) instructions, not by the matrix cores
// (a wave issues ~10 vector instructions per matrix instruction), so it is
// built to issue few of them:
//   * the feature map's row bias -(|x|^2/2 + ln(m)/2) log2 e enters the
//     projection as one more k-step of the matrix product: each staged fp16
//     row of Q and K carries the bias as two fp16 halves (hi + lo, exact to
//     ~2^-17) in extra columns, and the matching W columns are 1, so the
//     matrix cores return the base-2 exponent without any per-value add or
//     accumulator initialisation;
//   * the running key sum z is kept in LDS as packed bf16, written once per
//     feature by the lane that owns it, so that phi(Q) z reads ready operand
//     pairs;
//   * row norms are bf16 dot products of the packed input pairs;
//   * loads and stores go through buffer resources that end at the span's
//     last token (reads past it return zero, writes past it are dropped), so
//     the chunk loop has no branches.
// Chunks are double-buffered as in the generic scan: two barriers per chunk,
// the next chunk's feature maps overlapping the cross-wave sum of this one.
#include "favor_device.hpp"
#include "favor_internal.hpp"
#include "favor_tiles.hpp"

namespace favor {

// fourth word of a raw buffer resource on gfx9 (32-bit data format, no swizzle)
constexpr int kBufWord3 = 0x00020000;

struct Causal3Args {
  const void* q;
  const void* k;
  const void* v;
  const float* w;
  void* o;
  const float* prefix;    // [BH][spans][256][D] exclusive span prefixes of S
  const float* prefixz;   // [BH][spans][256]
  int L, H, Hw, spans, span_len;
  float eps;
};

template <int D>
struct Causal3Lds {
  static constexpr int C = 32;                           // tokens per chunk
  // fp16 rows of Q and K: D values, then 16 bias columns ([hi, lo, 0, ...]),
  // padded to an odd number of 16-byte chunks so that 16 consecutive rows
  // start in 16 different LDS bank groups (fragment reads: lane = row)
  static constexpr int RSX0 = (D + 16) * 2;
  static constexpr int RSX = (RSX0 / 16) % 2 ? RSX0 : RSX0 + 16;
  static constexpr int RS = Rows<D, 2>::RS;              // raw V rows (padded)
  static constexpr int kQh = 0, kKh = C * RSX, kV = 2 * C * RSX, kVT = kV + C * RS;
  static constexpr int BUF = kVT + C * D * 2;            // one chunk buffer
  // partial numerators of the four waves [C][D] (rows padded by 16 bytes),
  // then the denominators as [C][4 waves]
  static constexpr int RSR = (D + 4) * 4;
  static constexpr int kRed = 2 * BUF, kDen = kRed + 4 * C * RSR;
  // packed bf16 key sums, per wave [feature block][k-step][lane half][8]
  static constexpr int kZp = kDen + C * 16;
  static constexpr int kTotal = kZp + 4 * 128;
  static_assert(BUF % 16 == 0 && kDen % 16 == 0, "16-byte aligned buffers");
};

template <int D>
__global__ __launch_bounds__(256, 2) void k_causal3(Causal3Args a) {
  using Tr = TrBF16;
  using E = bf16;
  using F = u32x4;
  using LY = Causal3Lds<D>;
  constexpr int C = LY::C, RS = LY::RS, RSX = LY::RSX, RSR = LY::RSR;
  constexpr int NKD = D / Tr::KS;             // projection k-steps over d
  constexpr int NDB = D / 32;                 // 32-wide d blocks
  constexpr int NVT = 2 * NDB;                // V^T fragments per chunk
  constexpr int FBW = 2;                      // feature blocks per wave
  constexpr int M = 256;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int span = blockIdx.x, bh = blockIdx.y;
  const int head = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
  char* sZp = smem + LY::kZp + w * 128;                    // this wave's packed key sums
  const size_t hoff = (size_t)bh * a.L * D;
  const E* Qg = (const E*)a.q + hoff;
  const E* Kg = (const E*)a.k + hoff;
  const E* Vg = (const E*)a.v + hoff;
  E* Og = (E*)a.o + hoff;
  const float* wh = a.w + (size_t)(a.Hw == 1 ? 0 : head) * M * D;
  const float half_ln_m = 0.5f * logf((float)M);
  const int t0 = span * a.span_len;
  const int t1 = min(a.L, t0 + a.span_len);
  if (t0 >= t1) return;                                    // whole workgroup
  const int nch = (t1 - t0 + C - 1) / C;
  const int fb0 = w * FBW;

  // identity operand: slot j of k-step s2 of lane (n, hh) is 1 where feature
  // crow(8 s2 + j, hh) of the block equals n (multiplying a fragment by it
  // exchanges its rows and columns exactly)
  F ident[2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned lo = crow(8 * s2 + 2 * k, hh) == l32 ? 0x3f80u : 0u;
      const unsigned hi = crow(8 * s2 + 2 * k + 1, hh) == l32 ? 0x3f80u : 0u;
      ident[s2][k] = lo | (hi << 16);
    }

  // projection operand W log2(e) (fp16) of this wave's features, and the
  // bias k-step: columns [1, 1, 0, ...] in lane half 0, zero in half 1
  F wf[FBW][NKD];
#pragma unroll
  for (int i = 0; i < FBW; ++i) {
    const float* wrow = wh + (size_t)((fb0 + i) * 32 + l32) * D;
#pragma unroll
    for (int s = 0; s < NKD; ++s) wf[i][s] = w_frag<Tr, D, FM_POS>(wrow, hh, s, true);
  }
  const F wbias = {hh == 0 ? 0x3C003C00u : 0u, 0u, 0u, 0u};

  // ---- staging ---------------------------------------------------------------
  // Buffer resources over the span: reads past its last token return zero,
  // writes past it (or before its first) are dropped.
  const int span_bytes = (t1 - t0) * D * 2;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(Qg + (size_t)t0 * D), (short)0, span_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(Kg + (size_t)t0 * D), (short)0, span_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(Vg + (size_t)t0 * D), (short)0, span_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((void*)(Og + (size_t)t0 * D), (short)0, span_bytes, kBufWord3);
  // this thread's 16-byte chunk of a [C][D] tile (threads past C * CPR
  // repeat the first ones: same loads, same values written)
  constexpr int CPR = D * 2 / 16;
  const int sc = tid % (C * CPR), srow = sc / CPR, scc = sc % CPR;
  u32x4 gq, gk, gv;
  auto load_chunk = [&](int ci) {
    const int off = (ci * C + srow) * D * 2 + scc * 16;
    gq = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
    gk = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    gv = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
  };
  auto buf_of = [&](int ci) -> char* { return smem + (ci & 1) * LY::BUF; };
  // Q, K rows converted to fp16 with their bias columns; V raw.  The bias
  // is split as hi = fp16(b), lo = fp16(b - hi); rows past the span get
  // hi = -inf, lo = 0, so their features are exactly zero.  Each row's bias
  // chunk [hi, lo, 0 x 6] is written by the row's lane 0 and its zero chunk
  // by lane 1; the other lanes write their own data chunk a second time
  // (same value, own address), so that no two lanes of one write touch the
  // same address.
  // per-lane chunk masks of the staging (bias chunk / bias or zero chunk),
  // held as plain bit masks in registers: the compiler would otherwise turn
  // the masked words into selects on VCC, which issue several times slower
  // on gfx950 than bitwise operations
  unsigned m0 = scc == 0 ? ~0u : 0u, m1 = scc <= 1 ? ~0u : 0u;
  asm volatile("" : "+v"(m0), "+v"(m1));
  auto store_chunk = [&](int ci) {
    char* buf = buf_of(ci);
    const bool valid = t0 + ci * C + srow < t1;
    float ssq = 0.f, ssk = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ssq = dot2_bf16(gq[j], gq[j], ssq);
      ssk = dot2_bf16(gk[j], gk[j], ssk);
    }
    *(u32x4*)(buf + LY::kV + srow * RS + scc * 16) = gv;
    ssq = group_sum<CPR>(ssq);
    ssk = group_sum<CPR>(ssk);
    const float bq = FMap<FM_POS>::row_bias(ssq, half_ln_m), bk = FMap<FM_POS>::row_bias(ssk, half_ln_m);
    // (fp16 range: biases down to -131008 are exact, i.e. |x|^2 up to ~1.8e5;
    // below that every feature underflows to zero in float32 anyway unless
    // |w| exceeds ~200)
    const float bqh = (float)(_Float16)fmaxf(bq, -65504.f), bkh = (float)(_Float16)fmaxf(bk, -65504.f);
    // bitwise selects: computed for every lane, so no branch is formed.
    // Rows with |x|^2 > 2^20 take the padding rows' -inf as well: their
    // features are exactly what float32 gives, zero, whenever every row of W
    // is shorter than 256.  Their data words are zeroed, which also covers
    // entries past fp16's range (|x|^2 > 2^32 then): the conversion below
    // does not saturate.
    unsigned mvq = 0u - (unsigned)(valid && !(ssq > 1048576.f));   // all ones: a real row
    unsigned mvk = 0u - (unsigned)(valid && !(ssk > 1048576.f));
    asm volatile("" : "+v"(mvq), "+v"(mvk));
    u32x4 hq, hk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      hq[j] = pack_f16(bf16_lo(gq[j]), bf16_hi(gq[j])) & mvq;
      hk[j] = pack_f16(bf16_lo(gk[j]), bf16_hi(gk[j])) & mvk;
    }
    *(u32x4*)(buf + LY::kQh + srow * RSX + scc * 16) = hq;
    *(u32x4*)(buf + LY::kKh + srow * RSX + scc * 16) = hk;
    const unsigned cq = (pack_f16(bqh, fmaxf(bq - bqh, -65504.f)) & mvq) | (0xFC00u & ~mvq);   // pad: -inf, 0
    const unsigned ck = (pack_f16(bkh, fmaxf(bk - bkh, -65504.f)) & mvk) | (0xFC00u & ~mvk);
    const int boff = scc <= 1 ? D * 2 + scc * 16 : scc * 16;
    *(u32x4*)(buf + LY::kQh + srow * RSX + boff) =
        u32x4{(cq & m0) | (hq[0] & ~m1), hq[1] & ~m1, hq[2] & ~m1, hq[3] & ~m1};
    *(u32x4*)(buf + LY::kKh + srow * RSX + boff) =
        u32x4{(ck & m0) | (hk[0] & ~m1), hk[1] & ~m1, hk[2] & ~m1, hk[3] & ~m1};
  };
  // V^T fragment (s2, db): lane (d, hh) holds V[crow(8 s2 + j, hh)][32 db + d]
  auto vt_at = [&](const char* buf, int s2, int db) -> const char* {
    return buf + LY::kVT + ((s2 * 2 + hh) * D + db * 32 + l32) * 16;
  };
  auto transpose_v = [&](char* buf) {
    // NVT fragments over the waves (D = 32: waves 2, 3 repeat 0, 1)
    const int q = w % NVT;
    const int s2 = q / NDB, db = q % NDB;
    const int row = 16 * s2 + 4 * hh + ((lane & 15) >> 2);
    const int col = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    u32x2 r[2];
    lds_read_tr16_1x2<0, 8 * RS>(lds_addr(buf + LY::kV + row * RS + col * 2), r);
    *(u32x4*)vt_at(buf, s2, db) = u32x4{r[0][0], r[0][1], r[1][0], r[1][1]};
  };

  // ---- feature maps, lane = token: phi of this wave's 64 features ------------
  F pq[FBW][2], pk[FBW][2];
  auto feature_maps = [&](const char* buf) {
    const char* qrow = buf + LY::kQh + l32 * RSX;
    const char* krow = buf + LY::kKh + l32 * RSX;
    F qf[NKD], kf[NKD];
#pragma unroll
    for (int s = 0; s < NKD; ++s) {
      qf[s] = row_frag<Tr, D>(qrow, hh, s);
      kf[s] = row_frag<Tr, D>(krow, hh, s);
    }
    const F qb = *(const F*)(qrow + D * 2 + 16 * hh), kb = *(const F*)(krow + D * 2 + 16 * hh);
    const f32x16 bq = Tr::pmma(wbias, qb, zero16());      // the row biases
    const f32x16 bk = Tr::pmma(wbias, kb, zero16());
    f32x16 aq[FBW], ak[FBW];
#pragma unroll
    for (int i = 0; i < FBW; ++i) {
      aq[i] = bq;
      ak[i] = bk;
#pragma unroll
      for (int s = 0; s < NKD; ++s) {
        aq[i] = Tr::pmma(wf[i][s], qf[s], aq[i]);         // + P^T[f][t]
        ak[i] = Tr::pmma(wf[i][s], kf[s], ak[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < FBW; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        aq[i][r] = exp2_fast(aq[i][r]);
        ak[i][r] = exp2_fast(ak[i][r]);
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        pq[i][s2] = CFrag<Tr>::make(aq[i], s2);
        pk[i][s2] = CFrag<Tr>::make(ak[i], s2);
      }
    }
    // Issue order: the dependent projection chains of the first feature
    // block, then the second block's chains with the first block's
    // exponentials between their matrix instructions (a wave issues in
    // order, so exponentials placed after a chain would wait for all of it)
    __builtin_amdgcn_sched_group_barrier(0x008, 2 + 2 * NKD, 0);   // biases, block 0
#pragma unroll
    for (int s = 0; s < NKD; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);           // block 1, k-step s
      __builtin_amdgcn_sched_group_barrier(0x400, 32 / NKD, 0);    // block 0 exponentials
    }
  };

  // ---- the span's prefix state ----------------------------------------------
  // packed key sum of feature f = l32 of block i: k-step f/16, lane half
  // (f/4)%2, slot 4 ((f/8)%2) + f%4 (c-row order)
  const int zslot = (((l32 >> 4) * 2 + ((l32 >> 2) & 1)) * 16) + (4 * ((l32 >> 3) & 1) + (l32 & 3)) * 2;
  f32x16 st[FBW][NDB];
  float zreg[FBW];
  {
    const float* pre = a.prefix + ((size_t)bh * a.spans + span) * M * D;
    const float* prez = a.prefixz + ((size_t)bh * a.spans + span) * M;
#pragma unroll
    for (int i = 0; i < FBW; ++i) {
      const int fbase = (fb0 + i) * 32;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[i][db][r] = pre[(size_t)(fbase + crow(r, hh)) * D + db * 32 + l32];
      zreg[i] = prez[fbase + l32];
    }
  }
  auto write_z = [&]() {                               // both lane halves: the same value
#pragma unroll
    for (int i = 0; i < FBW; ++i) *(unsigned short*)(sZp + i * 64 + zslot) = (unsigned short)pack_bf16(zreg[i], 0.f);
  };

  // ---- chunk c: partial numerators and denominators, then the state update ---
  auto chunk_products = [&](const F (&vtf)[2][NDB]) {
    float* sRed = (float*)(smem + LY::kRed);
    f32x16 nacc[NDB];
    float dacc = 0.f;
    // intra-chunk scores A^T[tk][tq] over this wave's features, key after query masked
    f32x16 at = zero16();
#pragma unroll
    for (int i = 0; i < FBW; ++i)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) at = Tr::mma(pk[i][s2], pq[i][s2], at);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (crow(r, hh) > l32) at[r] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const F af = CFrag<Tr>::make(at, s2);              // B operand: lane = tq, k = tk (c-row)
#pragma unroll
      for (int j = 0; j < 4; ++j) dacc = dot2_bf16(af[j], 0x3f803f80u, dacc);
#pragma unroll
      for (int db = 0; db < NDB; ++db) nacc[db] = Tr::mma(vtf[s2][db], af, s2 == 0 ? zero16() : nacc[db]);
    }
    // inter-chunk: S^T phi(Q)^T and phi(Q) z with the state before this chunk
#pragma unroll
    for (int i = 0; i < FBW; ++i) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const F zz = *(const F*)(sZp + i * 64 + (s2 * 2 + hh) * 16);
#pragma unroll
        for (int db = 0; db < NDB; ++db) nacc[db] = Tr::mma(CFrag<Tr>::make(st[i][db], s2), pq[i][s2], nacc[db]);
#pragma unroll
        for (int k = 0; k < 4; ++k) dacc = dot2_bf16(pq[i][s2][k], zz[k], dacc);
      }
    }
    // this wave's partials
    float* rrow = sRed + (w * C + l32) * (RSR / 4);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4 = {nacc[db][4 * g], nacc[db][4 * g + 1], nacc[db][4 * g + 2], nacc[db][4 * g + 3]};
        *(f32x4*)(rrow + db * 32 + 8 * g + 4 * hh) = v4;
      }
    ((float*)(smem + LY::kDen))[l32 * 4 + w] = half_sum(dacc);   // both halves: the same value
    // state update: S += phi(K)^T V, z += phi(K)^T 1
#pragma unroll
    for (int i = 0; i < FBW; ++i) {
      float zc = 0.f;
      f32x16 kt = zero16();                              // phi(K) block, lane = feature
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) kt = Tr::mma(pk[i][s2], ident[s2], kt);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const F ktf = CFrag<Tr>::make(kt, s2);           // A operand: lane = f, k = t (c-row)
#pragma unroll
        for (int j = 0; j < 4; ++j) zc = dot2_bf16(ktf[j], 0x3f803f80u, zc);
#pragma unroll
        for (int db = 0; db < NDB; ++db) st[i][db] = Tr::mma(ktf, vtf[s2][db], st[i][db]);
      }
      zreg[i] += half_sum(zc);
    }
    write_z();                                         // wave-private; LDS keeps this wave's order
  };

  // ---- chunk c: sum of the four waves' partials, normalise, store ------------
  auto chunk_output = [&](int ci) {
    const float* sRed = (const float*)(smem + LY::kRed);
    constexpr int TPR = 256 / C;                       // threads per output row
    constexpr int DP = D / TPR;                        // outputs per thread
    const int tq = tid / TPR, d0 = (tid % TPR) * DP;
    float acc[DP];
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {                   // waves in order
      const float* rrow = sRed + (ww * C + tq) * (RSR / 4) + d0;
#pragma unroll
      for (int j = 0; j < DP; j += 4) {
        const f32x4 v4 = *(const f32x4*)(rrow + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[j + e] = ww == 0 ? v4[e] : acc[j + e] + v4[e];
      }
    }
    const f32x4 d4 = *(const f32x4*)((const float*)(smem + LY::kDen) + tq * 4);
    const float dsum = ((d4[0] + d4[1]) + d4[2]) + d4[3];
    const float inv = __builtin_amdgcn_rcpf(dsum + a.eps);
    // rows past the span: offsets outside the output resource, dropped
    const int off = ((ci * C + tq) * D + d0) * 2;
    if constexpr (DP == 8) {
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv),
                pack_bf16(acc[4] * inv, acc[5] * inv), pack_bf16(acc[6] * inv, acc[7] * inv)},
          ro, off, 0, 0);
    } else {
      static_assert(DP == 4, "outputs per thread");
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)},
                                            ro, off, 0, 0);
    }
  };

  // ---- prologue: chunk 0 staged with its V^T and feature maps; chunk 1 loaded
  load_chunk(0);
  store_chunk(0);
  load_chunk(1);
  write_z();
  wait_lgkm0();
  raw_barrier();                                       // chunk 0 staged
  transpose_v(buf_of(0));
  feature_maps(buf_of(0));

  for (int ci = 0; ci < nch; ++ci) {
    char* cur = buf_of(ci);
    wait_lgkm0();
    raw_barrier();                                     // chunk ci staged with V^T; last partials read
    // the wave between this barrier and its partial sums (matrix-core heavy)
    // issues first; the co-resident workgroup's vector work fills in
    __builtin_amdgcn_s_setprio(1);
    F vtf[2][NDB];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < NDB; ++db) vtf[s2][db] = *(const F*)vt_at(cur, s2, db);
    store_chunk(ci + 1);                               // past the span: zero rows
    load_chunk(ci + 2);
    chunk_products(vtf);
    __builtin_amdgcn_s_setprio(0);
    wait_lgkm0();
    raw_barrier();                                     // partials complete; chunk ci+1 staged
    feature_maps(buf_of(ci + 1));
    transpose_v(buf_of(ci + 1));
    chunk_output(ci);
  }
}

hipError_t launch_causal3(const Plan& p, const Tensors& t, hipStream_t s) {
  if (!p.scan3 || p.M != 256 || p.fgroups != 1 || (p.D != 64 && p.D != 32)) return kErrPlan;
  float* part = (float*)(t.ws + p.off_part);
  float* partz = (float*)(t.ws + p.off_partz);
  Causal3Args a{t.q, t.k, t.v, t.w, t.o, part, partz, p.L, p.H, p.Hw, p.splits, p.split_len, t.eps};
  timing_begin(FAVOR_KERNEL_CAUSAL, s);
  if (p.D == 64)
    hipLaunchKernelGGL(k_causal3<64>, dim3(p.splits, p.BH), dim3(256), (size_t)Causal3Lds<64>::kTotal, s, a);
  else
    hipLaunchKernelGGL(k_causal3<32>, dim3(p.splits, p.BH), dim3(256), (size_t)Causal3Lds<32>::kTotal, s, a);
  timing_end(FAVOR_KERNEL_CAUSAL, s);
  return hipGetLastError();
}

}  // namespace favor
