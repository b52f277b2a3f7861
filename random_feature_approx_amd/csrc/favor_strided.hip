// Strided layouts and value widths d_v != d at the boundary.
//
// The attention kernels read contiguous [B, H, L, d] tensors.  A call with
// other strides (for example the token-major [B, L, H, d] layout) or with
// values of another width is served by gathering the inputs into contiguous
// workspace buffers, running the contiguous path, and scattering the output
// back.  The output is linear in V (O = phi(Q) (phi(K)^T V) / (phi(Q) (phi(K)^T 1)
// + eps), Performer page In[25]), so a value width d_v != d is handled in
// column chunks of width d: chunk c holds columns [c d, c d + d) of V (zero
// past d_v) and yields the same columns of O.  Each chunk recomputes the
// features; the denominators are identical across chunks.
#include "favor_device.hpp"
#include "favor_internal.hpp"

namespace favor {

// dst[r][0..n) = src row r's columns [c0, c0 + n) (zero beyond `width`), for
// the rows r = (b, h, t) of a [B, H, L] grid; src row (b, h, t) starts at
// b*sb + h*sh + t*st elements.  One thread per destination element.
template <class E>
__global__ __launch_bounds__(256) void k_gather(const E* __restrict__ src, E* __restrict__ dst, int H, int L,
                                                long long sb, long long sh, long long st, int c0, int width, int n,
                                                long long total) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const int c = (int)(i % n);
    const long long r = i / n;
    const int t = (int)(r % L);
    const long long bh = r / L;
    const int h = (int)(bh % H);
    const long long b = bh / H;
    const int col = c0 + c;
    dst[i] = col < width ? src[b * sb + h * sh + t * st + col] : (E)0.f;
  }
}

// dst row (b, h, t) columns [c0, c0 + n) = src[r][0..n) (n <= the chunk width)
template <class E>
__global__ __launch_bounds__(256) void k_scatter(const E* __restrict__ src, E* __restrict__ dst, int H, int L,
                                                 long long sb, long long sh, long long st, int c0, int n, int srow,
                                                 long long total) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const int c = (int)(i % n);
    const long long r = i / n;
    const int t = (int)(r % L);
    const long long bh = r / L;
    const int h = (int)(bh % H);
    const long long b = bh / H;
    dst[b * sb + h * sh + t * st + c0 + c] = src[r * srow + c];
  }
}

static int grid_for(long long total) {
  const long long b = (total + 255) / 256;
  return (int)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

template <class E>
static hipError_t gather_t(const void* src, void* dst, const Plan& p, const long long* s, int c0, int width, int n,
                           hipStream_t st) {
  const long long total = (long long)p.BH * p.L * n;
  hipLaunchKernelGGL((k_gather<E>), dim3(grid_for(total)), dim3(256), 0, st, (const E*)src, (E*)dst, p.H, p.L, s[0],
                     s[1], s[2], c0, width, n, total);
  return hipGetLastError();
}

template <class E>
static hipError_t scatter_t(const void* src, void* dst, const Plan& p, const long long* s, int c0, int n, int srow,
                            hipStream_t st) {
  const long long total = (long long)p.BH * p.L * n;
  hipLaunchKernelGGL((k_scatter<E>), dim3(grid_for(total)), dim3(256), 0, st, (const E*)src, (E*)dst, p.H, p.L, s[0],
                     s[1], s[2], c0, n, srow, total);
  return hipGetLastError();
}

hipError_t gather_rows(const void* src, void* dst, const Plan& p, const long long* strides, int c0, int width, int n,
                       hipStream_t s) {
  return p.dt == FAVOR_BF16 ? gather_t<bf16>(src, dst, p, strides, c0, width, n, s)
                            : gather_t<float>(src, dst, p, strides, c0, width, n, s);
}

hipError_t scatter_rows(const void* src, void* dst, const Plan& p, const long long* strides, int c0, int n, int srow,
                        hipStream_t s) {
  return p.dt == FAVOR_BF16 ? scatter_t<bf16>(src, dst, p, strides, c0, n, srow, s)
                            : scatter_t<float>(src, dst, p, strides, c0, n, srow, s);
}

}  // namespace favor
