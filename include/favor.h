/*
 * favor.h -- C ABI of the MI355X (gfx950) FAVOR+ attention library.
 *
 * FAVOR+ replaces softmax attention by positive random features:
 *   phi(x) = exp(W x - |x|^2/2) / sqrt(m)      (feature-map equation of
 *            "Linear Attention > Performer: Unbiased Softmax Approximation";
 *            section 4 of "Linear Attention > Kernel Feature Maps")
 * and computes attention in the reassociated order
 *   O = phi(Q) (phi(K)^T V) / (phi(Q) (phi(K)^T 1) + eps)
 * (code cell In[25] of the Performer page; key points and the reordering
 * diagram of the performer-2020 study notes), or, causally, with the running
 * m x d state S_i = sum_{j<=i} phi(k_j) v_j^T (case 2 of the study notes).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers on the current HIP device,
 *    owned by the caller; the library never allocates, frees or keeps them.
 *  - Q, K, V, O, X are contiguous row-major [B, H, L, d]; Phi is [B, H, L, m].
 *  - W is float32 [Hw, m, d] (row i of a head is omega_i) with Hw = 1 (one
 *    projection shared by all heads) or Hw = H (one per head).  W is used as
 *    given: the library samples nothing and applies no 1/sqrt(d) temperature;
 *    a caller who wants one pre-scales Q and K.
 *  - dtype FAVOR_BF16: Q, K, V, X and O are bfloat16.  The projection x W^T
 *    runs on fp16 matrix-core operands: x is converted exactly (magnitudes
 *    under 2^-14 keep an absolute error below 2^-25; entries past fp16's
 *    65504 saturate there, and since the row bias -|x|^2/2 is taken from
 *    the unsaturated values, FAVOR+ features of such rows come out 0, as in
 *    exact arithmetic; the other feature maps see the saturated entries) and
 *    W log2(e) is rounded to fp16 (nearest even).  Features phi
 *    and the m x d states enter the other products as bf16 (nearest even);
 *    every product accumulates in float32, and states and sums are float32.
 *    FAVOR_F32: float32 storage, sums and states; products on the float32
 *    matrix cores, except in the causal FAVOR+ path at d = 128, where each
 *    product is three 16-bit products with float32 accumulation: operands
 *    split into hi + lo halves (fp16 for the projection W x, bf16 for
 *    features, scores, states and V), hi*hi + hi*lo + lo*hi, about 2^-16
 *    of each product's size for bf16 halves and 2^-21 for fp16 halves;
 *    rows with |x|^2 > 2^20 get phi = 0 there (exactly what float32 gives
 *    when every row of W is shorter than 256).  The environment variable
 *    FAVOR_F32_MFMA=1 selects float32 products for that path as well.
 *  - Supported shapes: d in {32, 64, 128}; 1 <= m <= 512 (the kernels work
 *    in blocks of 32 features; for m not a multiple of 32 the missing
 *    features are padding whose key-side features are set to exactly 0, so
 *    they add nothing to any sum, forward and backward); L >= 1;
 *    B, H >= 1; B*H <= 65534 and
 *    L*max(d,m) < 2^30 (offsets between heads are 64-bit, offsets inside
 *    one head 32-bit); otherwise FAVOR_ERR_SHAPE.
 *  - stream is a hipStream_t passed as void* (NULL = default stream).  Calls
 *    only enqueue work; results are valid once the stream has been
 *    synchronised.
 *  - Errors are returned, never thrown.  Arguments are validated before
 *    anything is enqueued: a non-OK return means nothing was launched, except
 *    FAVOR_ERR_HIP, which reports a launch failure (hipGetLastError), and
 *    FAVOR_ERR_INTERNAL, which reports a disagreement between the call's
 *    work split and the compiled kernels (a library bug).  Entry points that
 *    launch kernels first clear the calling thread's pending HIP error
 *    (hipGetLastError), so that the status reflects their own launches only:
 *    a caller who needs an earlier error must read it before the call.
 *    Pointer values other than NULL cannot be checked on the host.
 *  - Calls are thread-safe as long as concurrent calls use distinct
 *    workspaces.
 */
#ifndef FAVOR_H
#define FAVOR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FAVOR_F32 = 0, FAVOR_BF16 = 1 } favor_dtype;

typedef enum {
  FAVOR_OK = 0,
  FAVOR_ERR_NULL = 1,         /* a required pointer is NULL                      */
  FAVOR_ERR_SHAPE = 2,        /* B, H, L < 1, Hw not in {1, H}, or size overflow  */
  FAVOR_ERR_UNSUPPORTED = 3,  /* d, m or dtype outside the supported set         */
  FAVOR_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required         */
  FAVOR_ERR_HIP = 5,          /* the HIP runtime reported an error               */
  FAVOR_ERR_INTERNAL = 6      /* library bug; please report                      */
} favor_status;

/* Version of this ABI (incremented on incompatible changes). */
int favor_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* favor_status_string(favor_status s);

/*
 * Bytes of device workspace that favor_attn_noncausal (causal = 0) or
 * favor_attn_causal (causal = 1) needs for these shapes on the current
 * device (the split of L over workgroups depends on its compute-unit
 * count).  Returns 0 when the arguments are invalid.  The size covers both
 * Hw = 1 and Hw = H.  The workspace holds float32 partial states and the
 * projection operand prepared from W; it has no meaning between calls and
 * needs no initialisation.  Its base must be 256-byte aligned.
 */
size_t favor_workspace_bytes(int B, int H, int L, int d, int m, int causal, favor_dtype dtype);

/*
 * Phi = phi(X) for every row of X: Phi[b,h,l,:] = exp(W_h x - |x|^2/2)/sqrt(m)
 * (Performer page, feature-map equation), written as float32.  Used to check
 * the fused feature map; the attention entry points never store features.
 */
favor_status favor_features(const void* X, const float* W, int Hw, float* Phi,
                            int B, int H, int L, int d, int m,
                            favor_dtype dtype, void* stream);

/*
 * Non-causal FAVOR+ attention (Performer page, In[25]; study notes, key
 * points): per (b, h), the state M = phi(K)^T V (m x d) and key sum
 * z = phi(K)^T 1 are reduced over L, then O = (phi(Q) M) / (phi(Q) z + eps),
 * eps added to the denominator only.  Deterministic: the reduction order
 * depends only on the shapes and the device's compute-unit count.
 */
favor_status favor_attn_noncausal(const void* Q, const void* K, const void* V,
                                  const float* W, int Hw, void* O,
                                  int B, int H, int L, int d, int m, float eps,
                                  favor_dtype dtype, void* ws, size_t ws_bytes,
                                  void* stream);

/*
 * Causal FAVOR+ attention (study notes, case 2): with S_i = sum_{j<=i}
 * phi(k_j) v_j^T and z_i = sum_{j<=i} phi(k_j) (the diagonal included),
 * o_i = phi(q_i)^T S_i / (phi(q_i)^T z_i + eps).  The denominator is the
 * causal analogue of the non-causal one (the notes give the numerator
 * only).  Computed in chunks of 32 tokens by every scan (a chunk length C
 * of 64 is the same computation carried as two 32-token steps, identical
 * up to rounding order): inside a chunk the masked chunk-by-chunk score
 * tile is multiplied by V; across chunks the m x d state is carried as a
 * prefix sum, across spans of the sequence by an exclusive scan of the
 * spans' states.  Deterministic as above.
 */
favor_status favor_attn_causal(const void* Q, const void* K, const void* V,
                               const float* W, int Hw, void* O,
                               int B, int H, int L, int d, int m, float eps,
                               favor_dtype dtype, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * Feature maps ("Linear Attention > Kernel Feature Maps", sections 1-4), all
 * applied to the projection p = W x (with W the d x d identity, m = d, the
 * first two act on x itself as the page writes them):
 *   FAVOR_FMAP_POSITIVE  FAVOR+: exp(p - |x|^2/2)/sqrt(m)         (section 4)
 *   FAVOR_FMAP_ELU1      ELU(p) + 1: p + 1 for p > 0, exp(p) else  (section 1)
 *   FAVOR_FMAP_RELU      max(0, p)                                 (section 2)
 *   FAVOR_FMAP_TRIG      random Fourier features, 2m of them:
 *                        (1/sqrt(m)) [sin p_1, cos p_1, ..., sin p_m, cos p_m]
 *                        (section 3; they estimate exp(-|q-k|^2/2))
 * The trig features are not positive: the denominator phi(q).sum phi(k) + eps
 * can come near zero (the performer-2020 notes' pitfalls); results are then
 * ill-conditioned but computed as defined.  bf16 inputs: W's scaled copy is
 * rounded to fp16 for the projection as for FAVOR+ (scale 1, or 1/(2 pi)
 * for the trig map, whose sine and cosine take revolutions).
 */
typedef enum {
  FAVOR_FMAP_POSITIVE = 0,
  FAVOR_FMAP_ELU1 = 1,
  FAVOR_FMAP_RELU = 2,
  FAVOR_FMAP_TRIG = 3
} favor_feature_map;

/* Workspace of favor_attn_fmap for these shapes (m = rows of W). */
size_t favor_workspace_bytes_fmap(int B, int H, int L, int d, int m, int causal,
                                  favor_feature_map fmap, favor_dtype dtype);

/* Phi = phi(X) for the chosen map, float32 [B, H, L, m] or, for the trig
 * map, [B, H, L, 2m] in the page's interleaved order. */
favor_status favor_features_fmap(const void* X, const float* W, int Hw, float* Phi,
                                 int B, int H, int L, int d, int m,
                                 favor_feature_map fmap, favor_dtype dtype, void* stream);

/*
 * Attention (non-causal or causal, as favor_attn) with the chosen feature
 * map: O = phi(Q) (phi(K)^T V) / (phi(Q) (phi(K)^T 1) + eps), causally with
 * prefix sums.  Same arguments, shapes, errors and workspace rules as
 * favor_attn, workspace from favor_workspace_bytes_fmap; m counts the rows
 * of W (the trig map uses 2m features).
 */
favor_status favor_attn_fmap(const void* Q, const void* K, const void* V,
                             const float* W, int Hw, void* O,
                             int B, int H, int L, int d, int m, float eps, int causal,
                             favor_feature_map fmap, favor_dtype dtype, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * Attention with arbitrary layouts and a value width d_v that may differ
 * from d (the page's code cell In[25] allows d_v != d_k).  Each tensor is
 * described by its pointer and three element strides, for its batch, head
 * and token dimensions (the last dimension is contiguous): Q, K are
 * [B, H, L, dk], V and O are [B, H, L, dv] in that index order; for example
 * a token-major [B, L, H, d] tensor has strides {L*H*d, d, H*d}.  dk must be
 * a supported d; dv is any width from 1 to 65536.  Inputs that are not
 * contiguous (and V, O when dv != dk) are gathered into, or scattered from,
 * contiguous copies in the workspace; values are processed in column chunks
 * of width dk (O is linear in V), each chunk recomputing the features.
 * Workspace: favor_workspace_bytes_strided bytes (256-byte aligned).  O must
 * not overlap the inputs.  Errors as favor_attn; negative strides are
 * rejected with FAVOR_ERR_SHAPE.
 */
size_t favor_workspace_bytes_strided(int B, int H, int L, int dk, int dv, int m, int causal,
                                     favor_feature_map fmap, favor_dtype dtype);

favor_status favor_attn_strided(const void* Q, const long long* q_strides,
                                const void* K, const long long* k_strides,
                                const void* V, const long long* v_strides,
                                const float* W, int Hw, void* O, const long long* o_strides,
                                int B, int H, int L, int dk, int dv, int m, float eps, int causal,
                                favor_feature_map fmap, favor_dtype dtype, void* ws, size_t ws_bytes,
                                void* stream);

/* Dispatcher: favor_attn_causal when causal != 0, else favor_attn_noncausal. */
favor_status favor_attn(const void* Q, const void* K, const void* V,
                        const float* W, int Hw, void* O,
                        int B, int H, int L, int d, int m, float eps, int causal,
                        favor_dtype dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * favor_attn for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels, with the workspace taken from a static
 * device array of FAVOR_NOALLOC_SCRATCH_BYTES that the library holds on each
 * device it runs on (from the first such call on that device until the
 * process ends).  The call allocates nothing; the caller still provides Q,
 * K, V, W and O.  A call whose workspace (favor_workspace_bytes) exceeds the
 * scratch returns FAVOR_ERR_WORKSPACE and launches nothing.  Every call on
 * one device shares that device's scratch: calls that may overlap on one
 * device (concurrent streams, threads) race and must be serialised by the
 * caller.  Results equal favor_attn's bit for bit.
 */
#define FAVOR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
favor_status favor_attn_noalloc(const void* Q, const void* K, const void* V,
                                const float* W, int Hw, void* O,
                                int B, int H, int L, int d, int m, float eps, int causal,
                                favor_dtype dtype, void* stream);

/*
 * Backward pass of non-causal attention: the gradients dQ, dK, dV of
 * sum(dO * O) for the O that favor_attn_noncausal computes from the same
 * Q, K, V, W, eps (upstream gradient dO, all [B, H, L, d] in dtype; W gets
 * no gradient: it is a fixed random projection).  The pages give no
 * formulas for it; this is the chain rule through the reassociated form
 * (Performer page, In[25]) and the feature-map equation, where
 * d phi_f / dx = phi_f (omega_f - x).  Nothing from the forward call is
 * reused: the state M, z is recomputed from K and V.
 * Precision: with bf16 inputs the state M, its gradient, the features of Q
 * divided by their denominators and the projection W log2(e) enter their
 * products as pairs of bf16 (fp16 for W) values, hi + lo, about 16
 * significant bits, because the gradient takes differences of nearly equal
 * sums; gradients are returned rounded to bf16.
 * Workspace: favor_bwd_workspace_bytes(B, H, L, d, m, 0, dtype) bytes,
 * 256-byte aligned, no initialisation; it also covers Hw = H.  Same shape
 * support and error behaviour as the forward.
 */
size_t favor_bwd_workspace_bytes(int B, int H, int L, int d, int m, int causal, favor_dtype dtype);

favor_status favor_attn_noncausal_bwd(const void* Q, const void* K, const void* V,
                                      const float* W, int Hw, const void* dO,
                                      void* dQ, void* dK, void* dV,
                                      int B, int H, int L, int d, int m, float eps,
                                      favor_dtype dtype, void* ws, size_t ws_bytes,
                                      void* stream);

/*
 * Backward pass of causal attention: dQ, dK, dV of sum(dO * O) for the O of
 * favor_attn_causal (study notes, case 2, with the causal denominator).  The
 * query side uses the prefix sums S_i, z_i; the key side the suffix sums
 * R_j = sum_{i>=j} phi(q_i) g_i^T / D_i and r_j = sum_{i>=j} phi(q_i) c_i / D_i
 * (c_i = -phi(q_i).S_i g_i / D_i), accumulated in reverse as the study notes'
 * pitfalls section says the causal backward must be.  Computed in 32-token
 * chunks over spans of the sequence; precision as favor_attn_noncausal_bwd,
 * with the query side's two feature sums formed from split (hi + lo)
 * operands.  Workspace: favor_bwd_workspace_bytes(B, H, L, d, m, 1, dtype).
 */
favor_status favor_attn_causal_bwd(const void* Q, const void* K, const void* V,
                                   const float* W, int Hw, const void* dO,
                                   void* dQ, void* dK, void* dV,
                                   int B, int H, int L, int d, int m, float eps,
                                   favor_dtype dtype, void* ws, size_t ws_bytes,
                                   void* stream);

/*
 * Draw the random projection W [Hw, m, d] (float32, device memory owned by
 * the caller) from a seed on the device, as the Performer page's code draws
 * a fresh projection for every call; orthogonal != 0 gives the orthogonal
 * random features of the performer-2020 notes' key points.  Definition:
 * Philox4x64-10 (Salmon et al., SC 2011) keyed by (seed, 0); block
 * (c, row, head, purpose) gives four 64-bit words w, u = ((w >> 11) + 1/2)
 * 2^-53, and Box-Muller on (u0, u1), (u2, u3) gives normals 4c .. 4c+3 of
 * (row, head, purpose).  Orthogonal: block b of head h is the d x d matrix
 * G[i][j] = normal j of (b d + i, h, 0); row b d + i of W is column i of the
 * Q factor of G (QR with a positive diagonal), times the norm of d normals
 * of (b d + i, h, 1).  Otherwise W[h][f][j] = normal j of (f, h, 0).  Every
 * row is multiplied by scale (1: rows N(0, I); 1/sqrt(d): the page code's
 * randn / sqrt(d)).  Deterministic for a given seed and shape.  Shapes:
 * Hw >= 1, 1 <= m <= 65536, 1 <= d <= 128.
 */
favor_status favor_draw_projection(unsigned long long seed, int Hw, int m, int d, int orthogonal,
                                   float scale, float* W, void* stream);

/*
 * Exact softmax attention O = softmax(scale * Q K^T) V, optionally masked
 * to keys j <= i: the quadratic attention FAVOR+ approximates (softmax-kernel
 * equation of "Linear Attention > Kernel Feature Maps"; the left side of the
 * reordering diagram of the performer-2020 study notes, which write the
 * scale as 1/sqrt(d)).  The library's own reference for speed and quality
 * comparisons at equal shapes; it needs no workspace.  Q, K, V, O as for
 * favor_attn (d in {32, 64, 128}); scores, the running maximum and the sums
 * are float32, probabilities enter the value product in the input dtype.
 */
favor_status favor_softmax_attn(const void* Q, const void* K, const void* V, void* O,
                                int B, int H, int L, int d, float scale, int causal,
                                favor_dtype dtype, void* stream);

/*
 * Kernel timing (for benchmarks and profiling; host-side only, allocates no
 * device memory).  favor_timing_start(k, capacity) creates `capacity` pairs
 * of HIP timing events; every later launch of kernel k by this library
 * records one pair around itself on the launch's own stream, until the pool
 * is used up.  favor_timing_stop(k, ms, max, &n) waits for the recorded
 * events, writes the duration of each timed launch in milliseconds to
 * ms[0..min(n, max)-1] in launch order, sets n to the number of timed
 * launches, and destroys the events.  Not thread-safe: use from one host
 * thread while no other thread calls the library.
 */
typedef enum {
  FAVOR_KERNEL_FEATURES = 0,   /* fused feature map (favor_features)            */
  FAVOR_KERNEL_REDUCE = 1,     /* K-side state reduction / causal span totals    */
  FAVOR_KERNEL_COMBINE = 2,    /* non-causal combine of the partial states       */
  FAVOR_KERNEL_APPLY = 3,      /* non-causal Q-side apply (heads of <= 64 tokens: the one-launch kernel) */
  FAVOR_KERNEL_SPAN_SCAN = 4,  /* causal exclusive prefix over spans              */
  FAVOR_KERNEL_CAUSAL = 5,     /* causal chunked scan                             */
  FAVOR_KERNEL_BWD_PREP = 6,   /* backward: W operands                            */
  FAVOR_KERNEL_BWD_REDUCE = 7, /* backward: state and state-gradient reductions   */
  FAVOR_KERNEL_BWD_COMBINE = 8,/* backward: combine of their partials             */
  FAVOR_KERNEL_BWD_Q = 9,      /* backward: query side (dQ)                       */
  FAVOR_KERNEL_BWD_K = 10,     /* backward: key side (dK, dV)                     */
  FAVOR_KERNEL_SOFTMAX = 11,   /* exact softmax attention (favor_softmax_attn)    */
  FAVOR_KERNEL_DRAW = 12,      /* projection sampler (favor_draw_projection)     */
  FAVOR_KERNEL_COUNT = 13
} favor_kernel;

favor_status favor_timing_start(favor_kernel k, int capacity);
favor_status favor_timing_stop(favor_kernel k, double* ms, int max_launches, int* launches);
const char* favor_kernel_name(favor_kernel k);

#ifdef __cplusplus
}
#endif

#endif /* FAVOR_H */
