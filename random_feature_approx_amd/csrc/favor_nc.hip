// Non-causal FAVOR+ on gfx950: the fused feature map, the K-side state
// reduction, its fixed-order combine, and the Q-side apply.
//
// Formulas (see include/favor.h for the sources):
//   phi(x) = exp(W x - |x|^2/2) / sqrt(m)
//          = exp2(x . (W log2 e) - (|x|^2/2 + ln(m)/2) log2 e)
//   M = phi(K)^T V,  z = phi(K)^T 1,  O = phi(Q) M / (phi(Q) z + eps)
//
// Every step runs on the matrix cores except the exponentials, the norms and
// the final division: the projection x W^T is a 32x32 MFMA block per 32
// tokens x 32 features, its accumulator is exponentiated in registers and
// fed, without leaving registers, as the operand of the next contraction
// (phi^T V on the K side, M^T phi^T on the Q side).
#include "favor_device.hpp"
#include "favor_internal.hpp"
#include "favor_tiles.hpp"

#include <math.h>
#include <type_traits>

namespace favor {

// ===========================================================================
// favor_features: Phi = phi(X), float32 [BH, L, M]
// ===========================================================================
struct FeatArgs {
  const void* x;
  const float* w;
  float* phi;
  int L, M, H, Hw;
  int Mw;               // feature rows per head (M, or M/2 for the trig map), a multiple of 32
  int mt;               // rows of W per head as given (Mw rounded m up to 32)
};

template <class Tr, int D, int FM>
__global__ __launch_bounds__(256) void k_features(FeatArgs a) {
  using E = typename Tr::elem;
  using F = typename Tr::frag;
  constexpr int NKD = D / Tr::KS;
  const int bh = blockIdx.y, head = bh % a.H;
  const int lane = lane_id(), w = wave_id(), hh = lane >> 5, l32 = lane & 31;
  const int tok = blockIdx.x * 128 + w * 32 + l32;
  const bool tok_ok = tok < a.L;
  const E* xrow = (const E*)a.x + ((size_t)bh * a.L + (tok_ok ? tok : 0)) * D;
  const float* wh = a.w + (size_t)(a.Hw == 1 ? 0 : head) * a.mt * D;
  F xf[NKD];
  float ss = 0.f;
#pragma unroll
  for (int s = 0; s < NKD; ++s) {
    const int d0 = (D / 2) * hh + Tr::VPS * s;
    if constexpr (Tr::VPS == 8) {
      u32x4 v = tok_ok ? *(const u32x4*)(xrow + d0) : u32x4{0u, 0u, 0u, 0u};
      xf[s] = Tr::to_proj(v);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float p = bf16_lo(v[j]), q = bf16_hi(v[j]);
        ss = fmaf(p, p, fmaf(q, q, ss));
      }
    } else {
      float v = tok_ok ? xrow[d0] : 0.f;
      xf[s] = v;
      ss = fmaf(v, v, ss);
    }
  }
  ss = half_sum(ss);
  const float bias = FMap<FM>::row_bias(ss, 0.5f * logf((float)a.mt));
  const float tscale = FM == FM_TRIG ? rsqrtf((float)a.mt) : 1.f;
  const int nfbw = a.Mw >> 5;
  const int outw = FM == FM_TRIG ? 2 * a.mt : a.mt;       // features per row of Phi
  float* out = a.phi + ((size_t)bh * a.L + (tok_ok ? tok : 0)) * outw;
  for (int fb = 0; fb < (a.M >> 5); ++fb) {
    const int wr = (FM == FM_TRIG ? fb % nfbw : fb) * 32 + l32;    // this lane's row of W
    const bool wok = wr < a.mt;
    const float* wrow = wh + (size_t)(wok ? wr : 0) * D;
    const bool cosine = fb >= nfbw;
    f32x16 acc = zero16();
#pragma unroll
    for (int s = 0; s < NKD; ++s) acc = Tr::pmma(w_frag<Tr, D, FM>(wrow, hh, s, wok), xf[s], acc);
    if (tok_ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = FMap<FM>::phi(acc[4 * i + j] + bias, cosine, tscale);
        if (FM == FM_TRIG || a.mt != a.Mw) {
          // one feature at a time: rows past m are padding, and the trig map
          // stores the page's order (2i the sine of omega_i, 2i+1 its cosine)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int f = fb * 32 + 8 * i + 4 * hh + j;
            const int r = cosine ? f - a.Mw : f;
            if (r < a.mt) out[FM == FM_TRIG ? (cosine ? 2 * r + 1 : 2 * r) : f] = v[j];
          }
        } else {
          *(f32x4*)(out + fb * 32 + 8 * i + 4 * hh) = v;
        }
      }
    }
  }
}

// ===========================================================================
// K-side reduction: per (token split, feature group, head) partial
//   M_part[f][d] = sum_t phi(k_t)[f] v_t[d],  z_part[f] = sum_t phi(k_t)[f]
// Wave w of the workgroup owns FBW blocks of 32 features; all four waves
// share the K and V tiles staged in LDS.
// ===========================================================================
// Pipeline shape of the K-side kernels: tiles of TT tokens copied into a
// ring of STAGES raw K|V tiles; each tile is prepared once (K in the
// projection type with its row biases, and for bf16 V rearranged into
// operand order V^T) into one of two prepared buffers.
template <class Tr, int D, int NT>
struct RedLds {
  using E = typename Tr::elem;
  static constexpr bool kVT = Tr::VPS == 8;
  static constexpr int ROWB = D * (int)sizeof(E);
  // 32 tokens for long rows; otherwise 64, or enough rows to give every
  // thread one 16-byte chunk
  static constexpr int TT = ROWB >= 256 ? 32 : (NT * 16 / ROWB > 64 ? NT * 16 / ROWB : 64);
  using DT = DmaTile<E, D, TT, NT>;
  static constexpr int PAIR = 2 * DT::BYTES;
  // tile t+2 is copied while tile t is computed: with V^T the raw slot of
  // tile t is free by then (two slots), otherwise V is read raw (three)
  static constexpr int STAGES = kVT ? 2 : 3;
  static constexpr int RS = Rows<D, sizeof(E)>::RS;
  static constexpr int kKh = 0;                          // converted K, padded rows
  static constexpr int kV = kKh + TT * RS;               // V^T (bf16)
  static constexpr int kBias = kV + (kVT ? TT * D * 2 : 0);
  static constexpr int PREP = kBias + TT * 4;
  static constexpr int kRing = 2 * PREP;                 // [STAGES][K tile | V tile]
  static constexpr int kTotal = kRing + STAGES * PAIR;
};

// NW waves per workgroup, each owning FBW blocks of 32 features.  One barrier
// per tile: after it, tile t+2 is copied, tile t+1 is prepared and tile t is
// computed from its prepared buffer, so the copies, the preparation (LDS and
// a little VALU work) and the matrix products of different tiles overlap.
template <class Tr, int D, int NW, int FBW, int FM>
__global__ __launch_bounds__(NW * 64) void k_reduce(RedArgs a) {
  constexpr int NT = NW * 64;
  using E = typename Tr::elem;
  using F = typename Tr::frag;
  using LY = RedLds<Tr, D, NT>;
  using DT = typename LY::DT;
  constexpr int TT = LY::TT, S = LY::STAGES;
  constexpr int NKD = D / Tr::KS;           // k-steps over d
  constexpr int NDB = D / 32;               // 32-wide d blocks
  constexpr int NKT = 32 / Tr::KS;          // k-steps over a 32-token block
  constexpr int RS = LY::RS;
  constexpr int ES = (int)sizeof(E);
  constexpr int CPR = DT::CPR;
  constexpr int NVT = (TT / 32) * 2 * NDB;  // V^T fragments per tile (bf16)
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int split = blockIdx.x, fg = blockIdx.y, bh = blockIdx.z;
  const int head = bh % a.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
  const int nfb = a.M >> 5;
  const int fb0 = (fg * NW + w) * FBW;
  const E* K = (const E*)a.k + (size_t)bh * a.L * D;
  const E* V = (const E*)a.v + (size_t)bh * a.L * D;
  const float* wh = a.w + (size_t)(a.Hw == 1 ? 0 : head) * a.mt * D;
  const float half_ln_m = 0.5f * logf((float)a.mt);
  const int nfbw = a.Mw >> 5;
  const float tscale = FM == FM_TRIG ? rsqrtf((float)a.mt) : 1.f;
  const bool ragged = a.mt != a.Mw;

  F wf[FBW][NKD];
  bool wok[FBW];
#pragma unroll
  for (int i = 0; i < FBW; ++i) {
    const bool ok = fb0 + i < nfb;
    const int fbw_ = ok ? fb0 + i : 0;
    const int wr = (FM == FM_TRIG ? fbw_ % nfbw : fbw_) * 32 + l32;   // this lane's row of W
    wok[i] = ok && wr < a.mt;
    const float* wrow = wh + (size_t)(wok[i] ? wr : 0) * D;
#pragma unroll
    for (int s = 0; s < NKD; ++s) wf[i][s] = w_frag<Tr, D, FM>(wrow, hh, s, wok[i]);
  }
  // Non-causal: these fragments are also the apply's projection operand, in
  // its operand order [Hw*M/32 feature blocks][k-group g][lane half h][feature
  // f][16 bytes] (lane (f, h) of k-group g holds d = (D/2) h + (16/size) g + 0..,
  // the d-major k order of the projection; rows of W past mt are zero); the
  // first split's workgroup of each head stores them.
  if (a.wp != nullptr && split == 0 && (a.Hw == 1 ? bh == 0 : bh < a.H)) {
    constexpr int NKG = Tr::VPS == 8 ? NKD : NKD / 4;   // 16-byte chunks per lane and block
    const size_t hw = a.Hw == 1 ? 0 : head;
#pragma unroll
    for (int i = 0; i < FBW; ++i) {
      if (fb0 + i < nfb) {
        const size_t blk = hw * nfb + fb0 + i;
#pragma unroll
        for (int g = 0; g < NKG; ++g) {
          u32x4 c;
          if constexpr (Tr::VPS == 8) {
            c = wf[i][g];
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = as_u32(wf[i][4 * g + j]);
          }
          ((u32x4*)a.wp)[((blk * NKG + g) * 2 + hh) * 32 + l32] = c;
        }
      }
    }
  }
  f32x16 st[FBW][NDB];
  float zs[FBW];
#pragma unroll
  for (int i = 0; i < FBW; ++i) {
    zs[i] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) st[i][db] = zero16();
  }

  const int t0 = split * a.split_len;
  const int t1 = min(a.L, t0 + a.split_len);
  const int ntiles = t0 < t1 ? (t1 - t0 + TT - 1) / TT : 0;

  const typename DT::Lane dplan = DT::lane_plan(w, lane);
  auto ring = [&](int tt) -> char* { return smem + LY::kRing + (tt % S) * LY::PAIR; };
  auto prep_buf = [&](int tt) -> char* { return smem + (tt & 1) * LY::PREP; };
  auto issue = [&](int tt) {
    char* slot = ring(tt);
    const int r0 = t0 + tt * TT;
    DT::issue_plan(slot, (const char*)(K + (size_t)r0 * D), t1 - r0, dplan, w);
    DT::issue_plan(slot + DT::BYTES, (const char*)(V + (size_t)r0 * D), t1 - r0, dplan, w);
  };
  // preparation of a tile, in two halves around the products of the
  // previous one: read the raw K chunks; then convert them to the projection
  // type with row biases (-inf past the end) and rearrange V into V^T
  u32x4 kraw[DT::NI];
  auto prep_read = [&](int tt) {
    const char* raw = ring(tt);
#pragma unroll
    for (int i = 0; i < DT::NI; ++i) {
      const int c = tid + i * NT;
      kraw[i] = DT::chunk(raw, c / CPR, c % CPR);
    }
  };
  auto prep_write = [&](int tt) {
    const char* raw = ring(tt);
    char* pb = prep_buf(tt);
    float* bias = (float*)(pb + LY::kBias);
    const int nvalid = min(TT, t1 - (t0 + tt * TT));
#pragma unroll
    for (int i = 0; i < DT::NI; ++i) {
      const int c = tid + i * NT;
      const int r = c / CPR, cc = c % CPR;
      u32x4 v = kraw[i];
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (ES == 2) {
          const float lo = bf16_lo(v[j]), hi = bf16_hi(v[j]);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
          v[j] = pack_f16_sat(lo, hi);
        } else {
          const float x = as_f32(v[j]);
          ss = fmaf(x, x, ss);
        }
      }
      *(u32x4*)(pb + LY::kKh + r * RS + cc * 16) = v;
      ss = group_sum<CPR>(ss);
      if (cc == 0) bias[r] = r < nvalid ? FMap<FM>::row_bias(ss, half_ln_m) : -INFINITY;
    }
    if constexpr (LY::kVT) {
      const char* rawv = raw + DT::BYTES;
#pragma unroll
      for (int q = w; q < NVT; q += NW) {
        const int tb = q / (2 * NDB), s2 = (q / NDB) % 2, db = q % NDB;
        const int off = DT::at(tb * 32 + 16 * s2 + 4 * hh + ((lane & 15) >> 2),
                               db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
        u32x2 r2[2];
        lds_read_tr16_1x2<0, 8 * DT::ROWB>(lds_addr(rawv + off), r2);   // rows +8 keep the swizzle
        *(u32x4*)(pb + LY::kV + (((tb * 2 + s2) * 2 + hh) * D + db * 32 + l32) * 16) =
            u32x4{r2[0][0], r2[0][1], r2[1][0], r2[1][1]};
      }
    }
  };

  if (ntiles > 0) {
    issue(0);
    if (ntiles > 1) issue(1);
    // W rows (loaded first) and tile 0 complete: at most tile 1 outstanding
    wait_vmcnt_steps<2 * DT::NI, 1>(ntiles > 1 ? 1 : 0);
    raw_barrier();
    prep_read(0);
    prep_write(0);
  }
  constexpr int NSUB = TT / 32;
  for (int tt = 0; tt < ntiles; ++tt) {
    wait_vmcnt<0>();                          // tile tt+1 landed (this wave's copies)
    wait_lgkm0();                             // this wave's preparation of tile tt written
    raw_barrier();                            // ... everywhere; tile tt-1 fully consumed
    if (tt + 2 < ntiles) issue(tt + 2);
    const bool more = tt + 1 < ntiles;
    if (more) prep_read(tt + 1);
    // matrix work of tile tt at raised issue priority: the other workgroup's
    // preparation (vector and LDS work) fills in behind it (measured ~5%)
    __builtin_amdgcn_s_setprio(1);
    const char* pb = prep_buf(tt);
    const float* sBias = (const float*)(pb + LY::kBias);
    // projections of every 32-token block of the tile first, then their
    // exponentials and contractions, so matrix and vector work interleave
    f32x16 acc[FBW][NSUB];
#pragma unroll
    for (int tb = 0; tb < NSUB; ++tb) {
      F kf[NKD];
#pragma unroll
      for (int s = 0; s < NKD; ++s)
        kf[s] = *(const F*)(pb + LY::kKh + (tb * 32 + l32) * RS + ((D / 2) * hh + Tr::VPS * s) * ES);
#pragma unroll
      for (int i = 0; i < FBW; ++i) {
        // the accumulator starts at each token's bias, so the projection
        // lands directly on the base-2 exponent
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 b4 = *(const f32x4*)(sBias + tb * 32 + 8 * g + 4 * hh);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][tb][4 * g + j] = b4[j];
        }
#pragma unroll
        for (int s = 0; s < NKD; ++s) acc[i][tb] = Tr::pmma(kf[s], wf[i][s], acc[i][tb]);   // P[t][f] + bias[t]
      }
    }
#pragma unroll
    for (int tb = 0; tb < NSUB; ++tb) {
      F vf[NDB][NKT];
      if constexpr (LY::kVT) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2)
            vf[db][s2] = *(const F*)(pb + LY::kV + (((tb * 2 + s2) * 2 + hh) * D + db * 32 + l32) * 16);
      } else {
        const char* rawv = ring(tt) + DT::BYTES;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2) vf[db][s2] = col_frag_swz<Tr, DT>(rawv, tb * 32, db * 32, s2, lane);
      }
#pragma unroll
      for (int i = 0; i < FBW; ++i) {
        if (fb0 + i < nfb) {
          f32x16 e = acc[i][tb];
          const bool cosine = fb0 + i >= nfbw;
#pragma unroll
          for (int r = 0; r < 16; ++r) e[r] = FMap<FM>::phi(e[r], cosine, tscale);

#pragma unroll
          for (int s2 = 0; s2 < NKT; ++s2) {
            F pf = CFrag<Tr>::make(e, s2);
            if constexpr (Tr::VPS == 8) {
#pragma unroll
              for (int j = 0; j < 4; ++j) zs[i] = dot2_bf16(pf[j], 0x3f803f80u, zs[i]);
            } else {
              zs[i] += pf;
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) st[i][db] = Tr::mma(pf, vf[db][s2], st[i][db]);
          }
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (more) prep_write(tt + 1);
  }

  // the partials are linear in phi: features of padding rows of W (m not a
  // multiple of 32) are written as exact zeros
  float* P = a.part + ((size_t)bh * a.splits + split) * a.M * D;
  float* Pz = a.partz + ((size_t)bh * a.splits + split) * a.M;
#pragma unroll
  for (int i = 0; i < FBW; ++i) {
    if (fb0 + i < nfb) {
      const int f0 = (fb0 + i) * 32;
      if (ragged) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int f = f0 + crow(r, hh);
            if ((FM == FM_TRIG ? f % a.Mw : f) >= a.mt) st[i][db][r] = 0.f;
          }
        if (!wok[i]) zs[i] = 0.f;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) P[(size_t)(f0 + crow(r, hh)) * D + db * 32 + l32] = st[i][db][r];
      float z = half_sum(zs[i]);
      if (hh == 0) Pz[f0 + l32] = z;
    }
  }
}

// ===========================================================================
// Combine: sum the partial states of a head in a fixed order (deterministic)
// and store the state in the operand order of the apply step.
// ===========================================================================
// Position of state element (f, d) in operand order [group][half][d][slot]:
// the features of a lane's k-slots sit next to each other, so the apply step
// reads its state operand with one 16-byte load per lane and a wave reads
// contiguous memory.  bf16: group of 16 features (one 32x32x16 k-step),
// f = 16 g + 8 a + 4 h + b -> slot j = 4 a + b of lane half h;  float: group
// of 8 features (four 32x32x2 k-steps), f = 8 g + 4 h + b -> slot b.
template <class E>
struct OperandOrder {
  static constexpr int J = sizeof(E) == 2 ? 8 : 4;   // slots per lane and group
  static constexpr int GF = 2 * J;                  // features per group
  static __device__ __forceinline__ int slot(int f) {
    const int q = f % GF;
    return sizeof(E) == 2 ? (((q >> 3) << 2) | (q & 3)) : (q & 3);
  }
  static __device__ __forceinline__ int half(int f) { return (f >> 2) & 1; }
  static __device__ __forceinline__ int mpos(int f, int d, int D) { return (((f / GF) * 2 + half(f)) * D + d) * J + slot(f); }
  static __device__ __forceinline__ int zpos(int f) { return ((f / GF) * 2 + half(f)) * J + slot(f); }
};

// The m*d + m values of a head's state are handled in quads of 4 floats;
// a block is NG groups of threads, group g summing splits [g*per, (g+1)*per)
// of its quad in order (per = ceil(splits / NG)), and the groups' sums are
// added in group order.  NG grows with the split count (1 up to 8 splits, 8
// from 33 on), so that a thread has up to 8 loads in flight and a block
// covers 256 / NG quads; the order of additions depends only on the split
// count.
constexpr int combine_groups(int splits) { return splits <= 8 ? 1 : splits <= 16 ? 2 : splits <= 32 ? 4 : 8; }

// grid.y = BH: slice bh combines head bh's partial states.
template <class E, int NG>
__global__ __launch_bounds__(256) void k_combine(const float* part, const float* partz, E* mstate, E* zstate,
                                                 int splits, int M, int D) {
  constexpr int kQuadsPerBlock = 256 / NG;
  __shared__ f32x4 red[NG][kQuadsPerBlock];
  const int bh = blockIdx.y;
  const int g = threadIdx.x / kQuadsPerBlock, qi = threadIdx.x % kQuadsPerBlock;
  const int quad = blockIdx.x * kQuadsPerBlock + qi;
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
  const int per = (splits + NG - 1) / NG;
  const int s0 = min(splits, g * per), s1 = min(splits, s0 + per);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    for (int s = s0; s < s1; s += 8) {
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = s + j < s1 ? src[(size_t)(s + j) * stride] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += v[j];
    }
  }
  if constexpr (NG > 1) {
    red[g][qi] = acc;
    __syncthreads();
    if (g != 0) return;
#pragma unroll
    for (int gg = 1; gg < NG; ++gg) acc += red[gg][qi];
  }
  if (!active) return;
  using OO = OperandOrder<E>;
  if (quad < md4) {
    const int f = quad * 4 / D, d0 = quad * 4 % D;
    E* dst = mstate + (size_t)bh * M * D;
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[OO::mpos(f, d0 + c, D)] = (E)acc[c];
  } else {
    const int f0 = (quad - md4) * 4;
    E* dst = zstate + (size_t)bh * M;
#pragma unroll
    for (int c = 0; c < 4; ++c) dst[OO::zpos(f0 + c)] = (E)acc[c];
  }
}

// ===========================================================================
// Q-side apply: O = phi(Q) M / (phi(Q) z + eps).
// A workgroup of 8 waves walks a contiguous range of "groups" (8 waves x TB x
// 32 tokens of one head).  The projection operand, M and z of the current
// head sit in LDS in chunks of FCH features, all in operand order, copied
// with global->LDS loads; with a single chunk they are loaded once per head.
// Output is computed transposed, O^T = M^T phi(Q)^T, so each lane owns one
// token and divides by its own denominator.  The rows of Q for the next
// group are loaded while the current group is computed.
// ===========================================================================
struct ApplyArgs {
  const void* q;
  const void* wp;       // projection operand (written by the first split of k_reduce)
  const void* mstate;   // [BH] x operand-ordered M (m x d), operand type
  const void* zstate;   // [BH] x operand-ordered z (m), operand type
  void* o;
  int L, M, H, Hw;
  float eps;
  int groups_per_head, groups_total, steps, fch, nbuf;
  int stage_off;        // LDS offset of the per-wave output staging areas (LEAN: Q slots)
  int ostage_off;       // LEAN, 16-bit: LDS offset of the per-wave output rounds
  int Mw;               // feature rows per head (M, or M/2 for the trig map), a multiple of 32
  int mt;               // rows of W per head as given (padding features have zero state rows)
};

// NW waves per workgroup, TB 32-token blocks per wave.  LEAN: no Q prefetch,
// one feature block per scheduling region and no output staging, so that a
// wave fits 128 registers (four waves per SIMD).
template <class Tr, int D, int TB, int NW, bool LEAN, int FM>
__global__ __launch_bounds__(NW * 64) void k_apply(ApplyArgs a) {
  using E = typename Tr::elem;
  using F = typename Tr::frag;
  constexpr int NT = NW * 64;
  constexpr int NKD = D / Tr::KS;
  constexpr int NDB = D / 32;
  constexpr int ES = sizeof(E);
  constexpr int WES = Tr::VPS == 8 ? 2 : 4;
  constexpr int NKG = D * WES / 32;
  constexpr bool QV = Tr::VPS == 8;                  // raw Q kept as 16-byte vectors (bf16)
  using QRaw = typename std::conditional<QV, u32x4, float>::type;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int FCH = a.fch;
  // one buffer (W operand, M, z) per head in flight: with two, the next
  // group's head is copied while the current group is computed
  const int BUFB = FCH * D * WES + FCH * D * ES + FCH * ES;
  char* sW = smem;
  char* sM = sW + FCH * D * WES;
  char* sZ = sM + FCH * D * ES;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hh = lane >> 5, l32 = lane & 31;
  const int nch = (a.M + FCH - 1) / FCH;
  const float half_ln_m = 0.5f * logf((float)a.mt);
  const float tscale = FM == FM_TRIG ? rsqrtf((float)a.mt) : 1.f;
  const int g0 = blockIdx.x * a.steps;
  const int g1 = min(a.groups_total, g0 + a.steps);

  auto load_q = [&](int g, QRaw (&raw)[TB][NKD]) {
    const int bh = g / a.groups_per_head;
    const int tbase = (g % a.groups_per_head) * (NW * TB * 32) + w * TB * 32;
    const E* Q = (const E*)a.q + (size_t)bh * a.L * D;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int tok = tbase + tb * 32 + l32;
      const bool ok = tok < a.L;
      const E* qrow = Q + (size_t)(ok ? tok : 0) * D;
#pragma unroll
      for (int s = 0; s < NKD; ++s) {
        const int d0 = (D / 2) * hh + Tr::VPS * s;
        if constexpr (QV)
          raw[tb][s] = ok ? __builtin_nontemporal_load((const u32x4*)(qrow + d0)) : u32x4{0u, 0u, 0u, 0u};
        else
          raw[tb][s] = ok ? __builtin_nontemporal_load(qrow + d0) : 0.f;
      }
    }
  };
  // all waves finished with the previous contents; copy; copies landed everywhere
  auto issue_state = [&](char* buf, int bh, int f0, int nf) {
    const int head = bh % a.H;
    char* w_ = buf;
    char* m_ = w_ + FCH * D * WES;
    char* z_ = m_ + FCH * D * ES;
    dma_copy<NT>(w_, (const char*)a.wp + ((size_t)(a.Hw == 1 ? 0 : head) * a.M + f0) * D * WES, nf * D * WES / 16, tid);
    dma_copy<NT>(m_, (const char*)a.mstate + ((size_t)bh * a.M + f0) * D * ES, nf * D * ES / 16, tid);
    dma_copy<NT>(z_, (const char*)a.zstate + ((size_t)bh * a.M + f0) * ES, nf * ES / 16, tid);
  };
  auto reload = [&](int bh, int f0, int nf) {
    __syncthreads();
    issue_state(sW, bh, f0, nf);
    wait_vmcnt<0>();
    __syncthreads();
  };
  int cb = 0, loaded0 = -1, loaded1 = -1;             // head held by each buffer

  QRaw qnext[TB][NKD];
  if (!LEAN && g0 < g1) load_q(g0, qnext);
  // LEAN: each wave copies its next 32 Q rows into its own LDS slot with
  // global->LDS loads while the current group is computed (no registers held)
  using QT = DmaTile<E, D, 32, 64>;
  char* qslot = smem + a.stage_off + w * QT::BYTES;
  // copy addresses are recomputed per group (a few integer operations) rather
  // than held in registers for the whole kernel
  auto issue_q = [&](int g) {
    const int bh = g / a.groups_per_head;
    const int tbase = (g % a.groups_per_head) * (NW * TB * 32) + w * TB * 32;
    const E* Q = (const E*)a.q + (size_t)bh * a.L * D;
    const bool any = tbase < a.L;                        // rows past the end re-read row 0
    // the lane index comes from an opaque instruction so that the per-lane
    // offsets are recomputed here rather than kept live (and spilled) across
    // the group loop: a spill reload waits for every outstanding memory
    // operation, this group's output stores included
    int lane_now;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_now));
    QT::issue(qslot, Q + (size_t)(any ? tbase : 0) * D, any ? a.L - tbase : 1, 0, lane_now);
  };
  if constexpr (LEAN) {
    if (g0 < g1) issue_q(g0);
  }
  int cur_bh = -1;
  for (int g = g0; g < g1; ++g) {
    const int bh = g / a.groups_per_head;
    const int tbase = (g % a.groups_per_head) * (NW * TB * 32) + w * TB * 32;
    if (a.nbuf == 2) {
      if ((cb == 0 ? loaded0 : loaded1) != bh) {
        if ((cb == 0 ? loaded1 : loaded0) == bh) {
          cb ^= 1;                                       // copied during the previous group
          wait_vmcnt<0>();
          __syncthreads();
        } else {
          reload(bh, 0, a.M);                            // (sW points at buffer cb)
          if (cb == 0) loaded0 = bh; else loaded1 = bh;
        }
        sW = smem + cb * BUFB;
        sM = sW + FCH * D * WES;
        sZ = sM + FCH * D * ES;
      }
      if (g + 1 < g1) {
        const int nbh = (g + 1) / a.groups_per_head;
        if (nbh != bh && (cb == 0 ? loaded1 : loaded0) != nbh) {
          // the other buffer was last read before a barrier every wave has passed
          issue_state(smem + (cb ^ 1) * BUFB, nbh, 0, a.M);
          if (cb == 0) loaded1 = nbh; else loaded0 = nbh;
        }
      }
    } else if (nch == 1 && bh != cur_bh) {
      reload(bh, 0, a.M);
    }
    cur_bh = bh;

    QRaw qraw[TB][NKD];
    if constexpr (LEAN) {
      static_assert(TB == 1 && QV, "one 32-row block per wave");
      // this wave's rows of group g landed (for later groups the wait before
      // the previous group's output stores covered it)
      if (g == g0) wait_vmcnt<0>();
#pragma unroll
      for (int s = 0; s < NKD; ++s) qraw[0][s] = QT::chunk(qslot, l32, ((D / 2) * hh + Tr::VPS * s) * ES / 16);
      wait_lgkm0();                                      // read before the slot is refilled
      if (g + 1 < g1) issue_q(g + 1);
    } else {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int s = 0; s < NKD; ++s) qraw[tb][s] = qnext[tb][s];
      if (g + 1 < g1) load_q(g + 1, qnext);
    }

    F qf[TB][NKD];
    float bias[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < NKD; ++s) {
        if constexpr (QV) {
          const u32x4 v = qraw[tb][s];
          qf[tb][s] = Tr::to_proj(v);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p = bf16_lo(v[j]), q = bf16_hi(v[j]);
            ss = fmaf(p, p, fmaf(q, q, ss));
          }
        } else {
          qf[tb][s] = qraw[tb][s];
          ss = fmaf(qraw[tb][s], qraw[tb][s], ss);
        }
      }
      ss = half_sum(ss);
      bias[tb] = FMap<FM>::row_bias(ss, half_ln_m);
    }
    // LEAN FAVOR+: the accumulator starts at the token's bias through one
    // float32 32x32x2 product (A = 1/2 in every lane, B = the lane's bias in
    // both k rows: exactly bias[t] in every row of column t), so the matrix
    // cores return the base-2 exponent without a per-value add or copy
    constexpr bool kBiasK = LEAN && FM == FM_POS && Tr::VPS == 8;

    f32x16 oacc[TB][NDB];
    float den[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      den[tb] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[tb][db] = zero16();
    }

    for (int ch = 0; ch < nch; ++ch) {
      const int f0 = ch * FCH;
      const int nf = min(FCH, a.M - f0);
      if (nch > 1) reload(bh, f0, nf);
      // two feature blocks per step: one scheduling region, so the projection
      // of one block overlaps the exponentials of the other
      auto do_fb = [&](const int fb) {
        F wfr[NKD];
        if constexpr (WES == 2) {
#pragma unroll
          for (int s = 0; s < NKD; ++s) wfr[s] = *(const u32x4*)(sW + (((fb * NKG + s) * 2 + hh) * 32 + l32) * 16);
        } else {
#pragma unroll
          for (int gk = 0; gk < NKG; ++gk) {
            const f32x4 v = *(const f32x4*)(sW + (((fb * NKG + gk) * 2 + hh) * 32 + l32) * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) wfr[4 * gk + j] = v[j];
          }
        }
        f32x16 pacc[TB];
        const bool cosine = f0 + fb * 32 >= a.Mw;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          // non-LEAN: the accumulator starts at the token's bias (every row of
          // lane t is token t), so the projection returns P^T[f][t] + bias[t];
          // LEAN adds the bias afterwards (the 16 copies would not fit its
          // 128 registers: spilled values reloaded in the group loop wait for
          // every outstanding copy and store)
          if constexpr (kBiasK) pacc[tb] = __builtin_amdgcn_mfma_f32_32x32x2f32(0.5f, bias[tb], zero16(), 0, 0, 0);
          else pacc[tb] = LEAN ? zero16() : splat16(bias[tb]);
#pragma unroll
          for (int s = 0; s < NKD; ++s) pacc[tb] = Tr::pmma(wfr[s], qf[tb][s], pacc[tb]);   // P^T[f][t], lane = t
          // (LEAN with other feature maps: their bias is 0, no add)
          constexpr bool kAdd = LEAN && !kBiasK && FM == FM_POS;
#pragma unroll
          for (int r = 0; r < 16; ++r) pacc[tb][r] = FMap<FM>::phi(kAdd ? pacc[tb][r] + bias[tb] : pacc[tb][r], cosine, tscale);
        }
        if constexpr (Tr::VPS == 8) {
          // group gi = 2 fb + s2 holds 16 features; lane (d, hh) reads 8 of them
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int gi = 2 * fb + s2;
            const u32x4 zf = *(const u32x4*)(sZ + (gi * 2 + hh) * 16);
            F mf[NDB];
#pragma unroll
            for (int db = 0; db < NDB; ++db) mf[db] = *(const u32x4*)(sM + ((gi * 2 + hh) * D + db * 32 + l32) * 16);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
              F pf = CFrag<Tr>::make(pacc[tb], s2);
#pragma unroll
              for (int k = 0; k < 4; ++k) den[tb] = dot2_bf16(pf[k], zf[k], den[tb]);
#pragma unroll
              for (int db = 0; db < NDB; ++db) oacc[tb][db] = Tr::mma(mf[db], pf, oacc[tb][db]);
            }
          }
        } else {
          // group gi = 4 fb + s4 holds 8 features; lane (d, hh) reads 4 of them
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            const int gi = 4 * fb + s4;
            const f32x4 zf = *(const f32x4*)(sZ + (gi * 2 + hh) * 16);
            f32x4 mf[NDB];
#pragma unroll
            for (int db = 0; db < NDB; ++db) mf[db] = *(const f32x4*)(sM + ((gi * 2 + hh) * D + db * 32 + l32) * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int s = 4 * s4 + j;
#pragma unroll
              for (int tb = 0; tb < TB; ++tb) {
                den[tb] = fmaf(pacc[tb][s], zf[j], den[tb]);
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[tb][db] = Tr::mma(mf[db][j], pacc[tb][s], oacc[tb][db]);
              }
            }
          }
        }
      };
      const int nfbc = nf >> 5;
      int fb = 0;
      // LEAN: the feature-block loop at raised issue priority, so that the
      // waves in their matrix/exponential phase issue ahead of those copying
      // Q or storing output (measured ~3% on the long workload)
      if constexpr (LEAN) __builtin_amdgcn_s_setprio(1);
      if constexpr (!LEAN && (Tr::VPS == 8 || D <= 64)) {   // registers allow it
        for (; fb + 1 < nfbc; fb += 2) {
          do_fb(fb);
          do_fb(fb + 1);
        }
      }
      for (; fb < nfbc; ++fb) do_fb(fb);
      if constexpr (LEAN) __builtin_amdgcn_s_setprio(0);
    }

    // Rows of at most 128 bytes go through this wave's LDS staging area so
    // that every store instruction writes whole rows (8 lanes per row)
    // instead of 16 bytes in each of 32 rows; longer rows are stored directly.
    E* O = (E*)a.o + (size_t)bh * a.L * D;
    constexpr bool kStage = !LEAN && D * ES <= 128;
    // LEAN: the next group's rows (copy issued at this group's start) are
    // waited for here, before this group's stores join the queue
    if constexpr (LEAN) wait_vmcnt<0>();
    constexpr int RSO = D * ES + 16;
    constexpr int CPRO = D * ES / 16;
    char* stage = smem + a.stage_off + w * 32 * RSO;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      if constexpr (LEAN && ES == 2) {
        // Whole rows per store: the lane halves first swap 4-value groups so
        // that each lane holds 16-byte pieces of its row, then rounds of RPR
        // rows pass through this wave's small LDS area and come back with 8
        // (d = 64) or 4 (d = 32) lanes per row, every store instruction
        // writing RPR consecutive rows (one contiguous KB).
        constexpr int RB = D * ES, CPO = RB / 16, RPR = 64 / CPO, RSS = RB + 16;
        const float inv = 1.0f / (half_sum(den[tb]) + a.eps);
        u32x4 piece[NDB][2];                             // d = 32 db + 16 j + 8 hh, 8 values
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const unsigned a0 = pack_bf16(oacc[tb][db][8 * j] * inv, oacc[tb][db][8 * j + 1] * inv);
            const unsigned a1 = pack_bf16(oacc[tb][db][8 * j + 2] * inv, oacc[tb][db][8 * j + 3] * inv);
            const unsigned b0 = pack_bf16(oacc[tb][db][8 * j + 4] * inv, oacc[tb][db][8 * j + 5] * inv);
            const unsigned b1 = pack_bf16(oacc[tb][db][8 * j + 6] * inv, oacc[tb][db][8 * j + 7] * inv);
            // rows 8j..8j+3 of half 0 are d 16j..16j+3, of half 1 d 16j+4..16j+7;
            // rows 8j+4..8j+7: d 16j+8..16j+11 (half 0), 16j+12..16j+15 (half 1).
            // Half 0 keeps a and sends b; half 1 sends a and keeps b.
            const unsigned send0 = hh ? a0 : b0, send1 = hh ? a1 : b1;
            const auto s0 = __builtin_amdgcn_permlane32_swap(send0, send0, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(send1, send1, false, false);
            const unsigned r0 = hh ? s0[0] : s0[1], r1 = hh ? s1[0] : s1[1];   // the other half's values
            piece[db][j] = hh ? u32x4{r0, r1, b0, b1} : u32x4{a0, a1, r0, r1};
          }
        char* ost = smem + a.ostage_off + w * RPR * RSS;
        const int row0 = tbase + tb * 32;
#pragma unroll
        for (int rd = 0; rd < 32 / RPR; ++rd) {
          if (l32 >= rd * RPR && l32 < (rd + 1) * RPR) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
              for (int j = 0; j < 2; ++j)
                *(u32x4*)(ost + (l32 - rd * RPR) * RSS + (db * 4 + 2 * j + hh) * 16) = piece[db][j];
          }
          const int r = lane / CPO, c = lane % CPO;
          const u32x4 v = *(const u32x4*)(ost + r * RSS + c * 16);
          const int tok = row0 + rd * RPR + r;
          if (tok < a.L) *(u32x4*)(O + (size_t)tok * D + c * 8) = v;
          wait_lgkm0();                                  // read before the next round's writes
        }
        continue;
      } else if constexpr (!kStage) {
        const int tok = tbase + tb * 32 + l32;
        const float inv = 1.0f / (half_sum(den[tb]) + a.eps);
        if (tok < a.L) {
          E* orow = O + (size_t)tok * D;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int d0 = db * 32 + 8 * i + 4 * hh;
              if constexpr (ES == 2) {
                u32x2 pk = {pack_bf16(oacc[tb][db][4 * i] * inv, oacc[tb][db][4 * i + 1] * inv),
                            pack_bf16(oacc[tb][db][4 * i + 2] * inv, oacc[tb][db][4 * i + 3] * inv)};
                *(u32x2*)(orow + d0) = pk;
              } else {
                f32x4 v = {oacc[tb][db][4 * i] * inv, oacc[tb][db][4 * i + 1] * inv, oacc[tb][db][4 * i + 2] * inv,
                           oacc[tb][db][4 * i + 3] * inv};
                *(f32x4*)(orow + d0) = v;
              }
            }
        }
        continue;
      }
      const float inv = 1.0f / (half_sum(den[tb]) + a.eps);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = db * 32 + 8 * i + 4 * hh;
          if constexpr (ES == 2) {
            u32x2 pk = {pack_bf16(oacc[tb][db][4 * i] * inv, oacc[tb][db][4 * i + 1] * inv),
                        pack_bf16(oacc[tb][db][4 * i + 2] * inv, oacc[tb][db][4 * i + 3] * inv)};
            *(u32x2*)(stage + l32 * RSO + d0 * ES) = pk;
          } else {
            f32x4 v = {oacc[tb][db][4 * i] * inv, oacc[tb][db][4 * i + 1] * inv, oacc[tb][db][4 * i + 2] * inv,
                       oacc[tb][db][4 * i + 3] * inv};
            *(f32x4*)(stage + l32 * RSO + d0 * ES) = v;
          }
        }
#pragma unroll
      for (int k = 0; k < 32 * CPRO / 64; ++k) {
        const int c = k * 64 + lane, row = c / CPRO, cc = c % CPRO;
        const u32x4 v = *(const u32x4*)(stage + row * RSO + cc * 16);
        const int tok = tbase + tb * 32 + row;
        if (tok < a.L) *(u32x4*)((char*)(O + (size_t)tok * D) + cc * 16) = v;
      }
    }
  }
}

// ===========================================================================
// host launchers
// ===========================================================================
// Call f.template operator()<FM>() for the plan's feature map.
template <class Fn>
static hipError_t with_fmap(int fmap, Fn&& f) {
  switch (fmap) {
    case FM_POS: return f.template operator()<FM_POS>();
    case FM_ELU1: return f.template operator()<FM_ELU1>();
    case FM_RELU: return f.template operator()<FM_RELU>();
    case FM_TRIG: return f.template operator()<FM_TRIG>();
  }
  return kErrPlan;
}

template <class Tr, int D>
static hipError_t features_t(const Plan& p, const void* x, const float* w, float* phi, hipStream_t s) {
  FeatArgs a{x, w, phi, p.L, p.M, p.H, p.Hw, p.Mw, p.mt};
  dim3 grid((p.L + 127) / 128, p.BH);
  return with_fmap(p.fmap, [&]<int FM>() {
    timing_begin(FAVOR_KERNEL_FEATURES, s);
    hipLaunchKernelGGL((k_features<Tr, D, FM>), grid, dim3(256), 0, s, a);
    timing_end(FAVOR_KERNEL_FEATURES, s);
    return hipGetLastError();
  });
}

hipError_t launch_features(const Plan& p, const void* x, const float* w, float* phi, hipStream_t s) {
  if (p.dt == FAVOR_BF16) {
    switch (p.D) {
      case 32: return features_t<TrBF16, 32>(p, x, w, phi, s);
      case 64: return features_t<TrBF16, 64>(p, x, w, phi, s);
      case 128: return features_t<TrBF16, 128>(p, x, w, phi, s);
    }
  } else {
    switch (p.D) {
      case 32: return features_t<TrF32, 32>(p, x, w, phi, s);
      case 64: return features_t<TrF32, 64>(p, x, w, phi, s);
      case 128: return features_t<TrF32, 128>(p, x, w, phi, s);
    }
  }
  return kErrPlan;
}

template <class Tr, int D>
hipError_t launch_reduce_t(const Plan& p, const void* k, const void* v, const float* w, float* part, float* partz,
                           hipStream_t s, int nsplit, void* wp) {
  RedArgs a{k, v, w, part, partz, p.L, p.M, p.H, p.Hw, p.splits, p.split_len, p.Mw, p.mt, wp};
  // 8 waves of one feature block each, or 4 where a wave's registers exceed
  // half a SIMD's (two blocks per wave, sharing each K/V fragment read, ran
  // slower: half as many waves to hide the latency of each block's chain)
  constexpr int FBW = 1;
  constexpr int NW = (Tr::VPS == 1 && D == 128) ? 4 : 8;
  if (p.rnw != NW || p.rfbw != FBW) return kErrPlan;
  dim3 grid(nsplit, p.rfgroups, p.BH);
  const size_t lds = RedLds<Tr, D, NW * 64>::kTotal;
  return with_fmap(p.fmap, [&]<int FM>() {
    timing_begin(FAVOR_KERNEL_REDUCE, s);
    hipLaunchKernelGGL((k_reduce<Tr, D, NW, FBW, FM>), grid, dim3(NW * 64), lds, s, a);
    timing_end(FAVOR_KERNEL_REDUCE, s);
    return hipGetLastError();
  });
}

hipError_t launch_reduce(const Plan& p, const void* k, const void* v, const float* w, float* part, float* partz,
                         hipStream_t s, int nsplit, void* wp) {  // also used for the causal span aggregates
  if (nsplit < 0 || nsplit > p.splits) nsplit = p.splits;
  if (nsplit == 0) return hipSuccess;
  if (p.x3) return launch_reduce_x3(p, k, v, w, part, partz, s, nsplit);
  if (p.dt == FAVOR_BF16) {
    switch (p.D) {
      case 32: return launch_reduce_t<TrBF16, 32>(p, k, v, w, part, partz, s, nsplit, wp);
      case 64: return launch_reduce_t<TrBF16, 64>(p, k, v, w, part, partz, s, nsplit, wp);
      case 128: return launch_reduce_t<TrBF16, 128>(p, k, v, w, part, partz, s, nsplit, wp);
    }
  } else {
    switch (p.D) {
      case 32: return launch_reduce_t<TrF32, 32>(p, k, v, w, part, partz, s, nsplit, wp);
      case 64: return launch_reduce_t<TrF32, 64>(p, k, v, w, part, partz, s, nsplit, wp);
      case 128: return launch_reduce_t<TrF32, 128>(p, k, v, w, part, partz, s, nsplit, wp);
    }
  }
  return kErrPlan;
}

template <class Tr, int D, int TB, int NW, bool LEAN>
static hipError_t apply_t(const Plan& p, const Tensors& t, const void* wp, const void* mstate, const void* zstate,
                          hipStream_t s) {
  using E = typename Tr::elem;
  constexpr int WES = Tr::VPS == 8 ? 2 : 4;
  const int gsz = NW * TB * 32;
  const int gph = (p.L + gsz - 1) / gsz;
  const int total = p.BH * gph;
  const size_t buf = (size_t)p.fch * D * WES + (size_t)p.fch * D * sizeof(E) + (size_t)p.fch * sizeof(E);
  // output staging rows (non-LEAN, rows up to 128 bytes) or the LEAN Q slots
  const size_t stage = LEAN ? (size_t)NW * 32 * D * sizeof(E)
                            : (D * sizeof(E) <= 128 ? (size_t)NW * 32 * (D * sizeof(E) + 16) : 0);
  // LEAN, 16-bit: per wave, rounds of 64 / (row bytes / 16) rows of D + 8 elements
  const size_t ostage = (LEAN && sizeof(E) == 2) ? (size_t)NW * (64 / (D * sizeof(E) / 16)) * (D * sizeof(E) + 16) : 0;
  const int nbuf = (p.fch >= p.M && 2 * buf + stage + ostage <= 150 * 1024) ? 2 : 1;
  const size_t stage_off = (nbuf * buf + 15) / 16 * 16;
  ApplyArgs a{t.q, wp, mstate, zstate, t.o, p.L, p.M, p.H, p.Hw, t.eps, gph, total, p.apply_steps, p.fch, nbuf,
              (int)stage_off, (int)(stage_off + stage), p.Mw, p.mt};
  const int nblk = (total + p.apply_steps - 1) / p.apply_steps;
  const size_t lds = stage_off + stage + ostage;
  if (TB * 32 != p.apply_tile || NW != p.apply_nw) return kErrPlan;
  return with_fmap(p.fmap, [&]<int FM>() {
    timing_begin(FAVOR_KERNEL_APPLY, s);
    hipLaunchKernelGGL((k_apply<Tr, D, TB, NW, LEAN, FM>), dim3(nblk), dim3(NW * 64), lds, s, a);
    timing_end(FAVOR_KERNEL_APPLY, s);
    return hipGetLastError();
  });
}

static hipError_t launch_apply(const Plan& p, const Tensors& t, const void* wp, const void* mstate,
                               const void* zstate, hipStream_t s) {
  if (p.dt == FAVOR_BF16) {
    switch (p.D) {
      case 32: return apply_t<TrBF16, 32, 1, 16, true>(p, t, wp, mstate, zstate, s);
      case 64: return apply_t<TrBF16, 64, 1, 16, true>(p, t, wp, mstate, zstate, s);
      case 128: return apply_t<TrBF16, 128, 1, 8, false>(p, t, wp, mstate, zstate, s);
    }
  } else {
    switch (p.D) {
      case 32: return apply_t<TrF32, 32, 1, 8, false>(p, t, wp, mstate, zstate, s);
      case 64: return apply_t<TrF32, 64, 1, 8, false>(p, t, wp, mstate, zstate, s);
      case 128: return apply_t<TrF32, 128, 1, 8, false>(p, t, wp, mstate, zstate, s);
    }
  }
  return kErrPlan;
}

hipError_t launch_noncausal(const Plan& p, const Tensors& t, hipStream_t s) {
  if (small_nc_fits(p)) return launch_small_nc(p, t, s);
  float* part = (float*)(t.ws + p.off_part);
  float* partz = (float*)(t.ws + p.off_partz);
  void* wp = t.ws + p.off_wprep;
  void* mstate = t.ws + p.off_mstate;
  void* zstate = t.ws + p.off_zstate;
  // the reduction also writes the apply's projection operand (wp)
  hipError_t e = launch_reduce(p, t.k, t.v, t.w, part, partz, s, -1, wp);
  if (e != hipSuccess) return e;
  const int nq = (p.M * p.D + p.M) / 4;
  const int ng = combine_groups(p.splits);
  const dim3 cgrid((nq + 256 / ng - 1) / (256 / ng), p.BH);
  auto launch_combine = [&]<int NG>() {
    if (p.dt == FAVOR_BF16)
      hipLaunchKernelGGL((k_combine<bf16, NG>), cgrid, dim3(256), 0, s, part, partz, (bf16*)mstate, (bf16*)zstate,
                         p.splits, p.M, p.D);
    else
      hipLaunchKernelGGL((k_combine<float, NG>), cgrid, dim3(256), 0, s, part, partz, (float*)mstate, (float*)zstate,
                         p.splits, p.M, p.D);
  };
  timing_begin(FAVOR_KERNEL_COMBINE, s);
  switch (ng) {
    case 1: launch_combine.template operator()<1>(); break;
    case 2: launch_combine.template operator()<2>(); break;
    case 4: launch_combine.template operator()<4>(); break;
    default: launch_combine.template operator()<8>(); break;
  }
  timing_end(FAVOR_KERNEL_COMBINE, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_apply(p, t, wp, mstate, zstate, s);
}

}  // namespace favor
