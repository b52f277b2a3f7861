// Random projection W drawn on the device from a seed.
//
// The Performer page's code cell draws a fresh projection for every call;
// the orthogonal variant (performer-2020 notes, key points) stacks blocks of
// mutually orthogonal rows, each row given an independent chi(d) length so
// that rows stay marginally N(0, I).  Definition (also in favor.h):
//   * Philox4x64-10 (Salmon et al., "Parallel random numbers: as easy as 1,
//     2, 3", SC 2011) keyed by (seed, 0); the block at counter
//     (c, row, head, purpose) yields four 64-bit words w, each mapped to
//     u = (w >> 11) + 1/2 times 2^-53, and the pairs (u0, u1), (u2, u3) give
//     four normals by Box-Muller, sqrt(-2 ln u_a) (cos 2 pi u_b, sin 2 pi u_b):
//     normal j of (row, head, purpose) is component j % 4 of block j / 4;
//   * orthogonal: block b of a head is G_b[i][j] = normal j of
//     (b d + i, head, 0); its QR decomposition with a positive diagonal gives
//     Q, whose column i is row b d + i of W, scaled by the norm of d normals
//     of (b d + i, head, 1);
//   * independent: W[h][f][j] = normal j of (f, h, 0);
//   * every row times `scale`; rows past m are not drawn.
// The orthogonalisation is modified Gram-Schmidt on the columns of G_b in
// float64 (the QR factor with a positive diagonal is unique, so it equals
// the Householder factor after the sign fix up to rounding).
#include "favor_device.hpp"
#include "favor_internal.hpp"

#include <math.h>

namespace favor {

struct U64x4 {
  unsigned long long x[4];
};

__device__ __forceinline__ U64x4 philox4x64_10(unsigned long long c0, unsigned long long c1, unsigned long long c2,
                                               unsigned long long c3, unsigned long long k0, unsigned long long k1) {
  constexpr unsigned long long M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr unsigned long long W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const unsigned long long hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const unsigned long long hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const unsigned long long n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  return U64x4{{c0, c1, c2, c3}};
}

// the four normals of block c of (row, head, purpose)
__device__ __forceinline__ void normals4(unsigned long long seed, int head, int purpose, int row, int c, double (&z)[4]) {
  const U64x4 w = philox4x64_10((unsigned long long)c, (unsigned long long)row, (unsigned long long)head,
                                (unsigned long long)purpose, seed, 0ull);
  double u[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] = ((double)(w.x[k] >> 11) + 0.5) * 0x1.0p-53;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const double r = sqrt(-2.0 * log(u[2 * p]));
    double s, co;
    sincospi(2.0 * u[2 * p + 1], &s, &co);
    z[2 * p] = r * co;
    z[2 * p + 1] = r * s;
  }
}

// independent rows: one thread per group of four entries
__global__ __launch_bounds__(256) void k_draw_iid(unsigned long long seed, int Hw, int m, int d, float scale,
                                                  float* W) {
  const int ng = (d + 3) / 4;
  const long long total = (long long)Hw * m * ng;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const int c = (int)(i % ng);
    const long long r = i / ng;
    const int f = (int)(r % m), h = (int)(r / m);
    double z[4];
    normals4(seed, h, 0, f, c, z);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (4 * c + k < d) W[((size_t)h * m + f) * d + 4 * c + k] = (float)(scale * z[k]);
  }
}

// one workgroup per (block, head): G in LDS column by column (stride d + 1
// doubles), modified Gram-Schmidt, lengths, rows written out
__global__ __launch_bounds__(256) void k_draw_orth(unsigned long long seed, int m, int d, float scale, float* W) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  double* G = (double*)smem;                         // G[j * (d + 1) + i] = G_b[i][j]
  double* red = G + (size_t)d * (d + 1);             // 256 partial sums
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int S = d + 1;
  const int ng = (d + 3) / 4;
  for (int q = tid; q < d * ng; q += 256) {
    const int i = q / ng, c = q % ng;
    double z[4];
    normals4(seed, h, 0, b * d + i, c, z);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (4 * c + k < d) G[(4 * c + k) * S + i] = z[k];
  }
  __syncthreads();
  for (int k = 0; k < d; ++k) {
    double* ck = G + k * S;
    double part = 0.0;
    for (int i = tid; i < d; i += 256) part += ck[i] * ck[i];
    red[tid] = part;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    const double inv = 1.0 / sqrt(red[0]);
    __syncthreads();                                 // every thread has read the norm
    for (int i = tid; i < d; i += 256) ck[i] *= inv;
    __syncthreads();
    // remove column k from the later columns: thread t owns column k + 1 + t
    for (int j = k + 1 + tid; j < d; j += 256) {
      double* cj = G + j * S;
      double dot = 0.0;
      for (int i = 0; i < d; ++i) dot += ck[i] * cj[i];
      for (int i = 0; i < d; ++i) cj[i] -= dot * ck[i];
    }
    __syncthreads();
  }
  // lengths and output: row b d + t of W is column t of Q
  double* len = red;                                  // reuse: d <= 256 lengths
  for (int t = tid; t < d; t += 256) {
    double ss = 0.0;
    for (int c = 0; c < ng; ++c) {
      double z[4];
      normals4(seed, h, 1, b * d + t, c, z);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (4 * c + k < d) ss += z[k] * z[k];
    }
    len[t] = sqrt(ss);
  }
  __syncthreads();
  for (int q = tid; q < d * d; q += 256) {
    const int t = q / d, j = q % d;
    const int f = b * d + t;
    if (f < m) W[((size_t)h * m + f) * d + j] = (float)(scale * len[t] * G[t * S + j]);
  }
}

hipError_t launch_draw(unsigned long long seed, int Hw, int m, int d, int orthogonal, float scale, float* W,
                       hipStream_t s) {
  timing_begin(FAVOR_KERNEL_DRAW, s);
  if (orthogonal) {
    const size_t lds = ((size_t)d * (d + 1) + 256) * sizeof(double);
    hipLaunchKernelGGL(k_draw_orth, dim3((m + d - 1) / d, Hw), dim3(256), lds, s, seed, m, d, scale, W);
  } else {
    const long long total = (long long)Hw * m * ((d + 3) / 4);
    const long long blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_draw_iid, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, seed, Hw, m, d,
                       scale, W);
  }
  timing_end(FAVOR_KERNEL_DRAW, s);
  return hipGetLastError();
}

}  // namespace favor
