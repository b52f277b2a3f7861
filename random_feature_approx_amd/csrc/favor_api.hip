// C ABI of the FAVOR+ library: argument validation, the work split (plan),
// workspace layout and dispatch to the kernels.  See include/favor.h.
#include "favor_internal.hpp"

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

namespace favor {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int device_cu_count() {
  static std::atomic<int> cached[64];                 // zero-initialised (static storage)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
  if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Size limits: every offset between heads is 64-bit; offsets inside one head
// are 32-bit byte offsets, so L * max(d, m) must stay below 2^30 (a head's
// float32 features fit 4 GiB); B * H is a grid dimension (y or z, at most
// 65535 on this device), accepted up to 65534.
static favor_status check_shapes(int B, int H, int L, int d, int m, int Hw, favor_dtype dt) {
  if (B < 1 || H < 1 || L < 1) return FAVOR_ERR_SHAPE;
  if (Hw != 1 && Hw != H) return FAVOR_ERR_SHAPE;
  if (dt != FAVOR_F32 && dt != FAVOR_BF16) return FAVOR_ERR_UNSUPPORTED;
  if (d != 32 && d != 64 && d != 128) return FAVOR_ERR_UNSUPPORTED;
  if (m < 1 || m > 512) return FAVOR_ERR_UNSUPPORTED;
  if ((int64_t)L * (d > m ? d : m) >= ((int64_t)1 << 30)) return FAVOR_ERR_SHAPE;
  if ((int64_t)B * H > 65534) return FAVOR_ERR_SHAPE;
  return FAVOR_OK;
}

// Status of a launch sequence.  A pending HIP error left by the caller's own
// work is cleared before launching (see favor.h), so hipGetLastError after
// the launches reports this call's launches only.
static favor_status launch_status(hipError_t e) {
  if (e == hipSuccess) return FAVOR_OK;
  if (e == hipErrorNotSupported) return FAVOR_ERR_UNSUPPORTED;
  if (e == kErrPlan) return FAVOR_ERR_INTERNAL;
  return FAVOR_ERR_HIP;
}
static void clear_pending_error() { (void)hipGetLastError(); }

bool make_plan(Plan& p, int B, int H, int L, int d, int m, int Hw, int causal, favor_dtype dt, int num_cus,
               int fmap) {
  if (check_shapes(B, H, L, d, m, Hw, dt) != FAVOR_OK || num_cus <= 0) return false;
  if (fmap < FAVOR_FMAP_POSITIVE || fmap > FAVOR_FMAP_TRIG) return false;
  p.fmap = fmap;
  p.mt = m;
  p.Mw = (m + 31) / 32 * 32;                // padding features up to a multiple of 32
  m = fmap == FAVOR_FMAP_TRIG ? 2 * p.Mw : p.Mw;   // features: a sine and a cosine per row of W
  p.B = B; p.H = H; p.L = L; p.D = d; p.M = m; p.Hw = Hw; p.causal = causal ? 1 : 0; p.dt = dt;
  p.BH = B * H;
  p.esize = dt == FAVOR_BF16 ? 2 : 4;
  // the float32 FAVOR+ scan for d = 128 on split 16-bit products
  // (k_causal_x3, one workgroup per compute unit, and its span
  // aggregates k_reduce_x3, eight waves); FAVOR_F32_MFMA=1 keeps
  // the float32 matrix-core scan instead (comparisons and tuning)
  {
    const char* env = getenv("FAVOR_F32_MFMA");
    const bool f32_mfma = env && atoi(env) > 0;
    p.x3 = (causal && dt == FAVOR_F32 && fmap == FAVOR_FMAP_POSITIVE && d == 128 && !f32_mfma) ? 1 : 0;
  }
  // reduction split: about two workgroups per compute unit, ranges of at
  // least 256 tokens, whole 64-token tiles (two 32-token chunks of the
  // causal scans).
  // the bf16 scan for d <= 64 (every feature map) owns two feature blocks
  // per wave; the generic scan (bf16 d = 128 and float32) one
  p.fbw = (dt == FAVOR_BF16 && d <= 64) ? 2 : 1;
  const int nfb = m / 32;
  p.fgroups = (nfb + 4 * p.fbw - 1) / (4 * p.fbw);
  p.rfbw = 1;   // two blocks per wave (4 waves) measured slower: fewer waves to hide latency
  p.rnw = (dt == FAVOR_F32 && d == 128 && !p.x3) ? 4 : 8;
  p.rfgroups = (nfb + p.rnw * p.rfbw - 1) / (p.rnw * p.rfbw);
  // the causal scan for bf16 FAVOR+ with d <= 64 and m = 256 (k_causal3)
  p.scan3 = (causal && dt == FAVOR_BF16 && fmap == FAVOR_FMAP_POSITIVE && p.mt == 256 && (d == 32 || d == 64)) ? 1 : 0;
  const int target = p.x3 ? num_cus : 2 * num_cus;
  // non-causal: reduction workgroups = BH * splits * rfgroups; causal: the
  // chunk scan runs one workgroup per (span, head) and walks feature groups
  // in turn, so spans alone fill the device.
  const int per_head = causal ? p.BH : p.BH * p.rfgroups;
  // at most one round of resident workgroups: a few extra workgroups would
  // run as a second, mostly empty round
  int splits = target / per_head;
  const int max_splits = (L + 255) / 256;
  // the causal backward's query walks run one span workgroup of eight waves
  // per compute unit (bf16, d <= 64) or two of four waves
  p.bqnw = (dt == FAVOR_BF16 && d <= 64) ? 8 : 4;
  int bwd_splits = ((p.bqnw == 8 ? 1 : 2) * num_cus) / per_head;
  // FAVOR_SPANS (testing and tuning): the number of causal spans per head
  if (causal) {
    const char* env = getenv("FAVOR_SPANS");
    const int forced = env ? atoi(env) : 0;
    if (forced > 0) splits = bwd_splits = forced;
  }
  if (bwd_splits > max_splits) bwd_splits = max_splits;
  if (bwd_splits < 1) bwd_splits = 1;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int len = (L + splits - 1) / splits;
  len = (len + 63) / 64 * 64;
  p.split_len = len;
  p.splits = (L + len - 1) / len;
  // apply: one workgroup per compute unit walking groups of NW waves x TB x
  // 32 tokens of one head (bf16, d <= 64: 16 waves of one block each, four
  // per SIMD; otherwise 8 waves)
  const bool lean = dt == FAVOR_BF16 && d <= 64;
  p.apply_nw = lean ? 16 : 8;
  p.apply_tile = 32;
  const int gsz = p.apply_nw * p.apply_tile;
  const int gph = (L + gsz - 1) / gsz;
  const int total = p.BH * gph;
  p.apply_steps = (total + num_cus - 1) / num_cus;
  if (p.apply_steps < 1) p.apply_steps = 1;
  p.apply_groups = (total + p.apply_steps - 1) / p.apply_steps;
  const int wes = dt == FAVOR_BF16 ? 2 : 4;         // projection operand bytes
  // LDS for the apply's per-head operands: what the 160 KB leave after the
  // lean kernel's per-wave Q slots and output rounds (16 waves), else 96 KB
  const int lean_extra = lean ? 16 * 32 * d * 2 + 16 * (64 / (d * 2 / 16)) * (d * 2 + 16) : 0;
  const int budget = lean ? 160 * 1024 - lean_extra - 1024 : 98304;
  int fch = budget / (d * wes + d * p.esize + p.esize);   // projection operand, M and z per feature
  fch = fch / 32 * 32;
  p.fch = fch < m ? fch : m;
  // workspace
  size_t off = 0;
  p.off_part = off;
  off += align256((size_t)p.BH * p.splits * m * d * sizeof(float));
  p.off_partz = off;
  off += align256((size_t)p.BH * p.splits * m * sizeof(float));
  // projection operand, sized for one projection per head (Hw = H) so that
  // the size does not depend on Hw
  p.off_wprep = off;
  off += align256((size_t)H * m * d * (dt == FAVOR_BF16 ? 2 : 4));
  p.off_mstate = off;
  off += align256((size_t)p.BH * m * d * p.esize);
  p.off_zstate = off;
  off += align256((size_t)p.BH * m * p.esize);
  // causal with several feature groups: float32 partial numerators and
  // denominators carried from one group to the next
  p.off_num = off;
  if (causal && p.fgroups > 1) off += align256((size_t)p.BH * L * d * sizeof(float));
  p.off_den = off;
  // (k_causal_x3: one copy per wave)
  if (causal && p.fgroups > 1) off += align256((size_t)p.BH * L * sizeof(float) * (p.x3 ? 4 : 1));
  p.total = off;
  // backward reductions: one wave per feature block, eight waves per
  // workgroup (one workgroup per compute unit) for bf16 at d <= 64 with more
  // than four blocks, else four (about two per compute unit); the causal
  // backward reduces over the spans of the forward's chunk scan
  p.brnw = (dt == FAVOR_BF16 && d <= 64 && nfb > 4) ? 8 : 4;
  p.bfgroups = (nfb + p.brnw - 1) / p.brnw;
  if (causal) {
    int bl = (L + bwd_splits - 1) / bwd_splits;
    bl = (bl + 63) / 64 * 64;
    p.bsplit_len = bl;
    p.bsplits = (L + bl - 1) / bl;
  } else {
    const int per = p.BH * p.bfgroups;
    const int btarget = (p.brnw == 8 ? 1 : 2) * num_cus;
    int bs = (btarget + per - 1) / per;
    if (bs > max_splits) bs = max_splits;
    if (bs < 1) bs = 1;
    int bl = (L + bs - 1) / bs;
    bl = (bl + 63) / 64 * 64;
    p.bsplit_len = bl;
    p.bsplits = (L + bl - 1) / bl;
  }
  size_t bo = 0;
  p.boff_part = bo;
  bo += align256((size_t)p.BH * p.bsplits * m * d * sizeof(float));
  p.boff_partz = bo;
  bo += align256((size_t)p.BH * p.bsplits * m * sizeof(float));
  p.boff_zf = bo;
  bo += align256((size_t)p.BH * m * sizeof(float));
  p.boff_lg = bo;
  bo += align256((size_t)p.BH * L * sizeof(float));
  p.boff_cw = bo;
  bo += align256((size_t)p.BH * L * sizeof(float));
  p.boff_wph = bo;                                   // sized for Hw = H
  bo += align256((size_t)H * m * d * (size_t)wes);
  p.boff_wpl = bo;
  bo += align256((size_t)H * m * d * (size_t)wes);
  p.boff_wt = bo;
  bo += align256((size_t)H * m * d * p.esize);
  p.boff_wtl = bo;
  bo += align256((size_t)H * m * d * p.esize);
  p.boff_rows_hi = bo;
  bo += align256((size_t)p.BH * m * d * p.esize);
  p.boff_rows_lo = bo;
  bo += align256((size_t)p.BH * m * d * p.esize);
  p.boff_op = bo;
  bo += align256((size_t)p.BH * m * d * p.esize);
  // causal walks with more than one feature group (the key walk's workgroup
  // holds four blocks, a query walk's bqnw): float32 per-token sums carried
  // from one group to the next (2 d + 2 per token)
  p.boff_acc = bo;
  if (causal && (nfb > 4 || nfb > p.bqnw)) bo += align256((size_t)p.BH * L * (2 * d + 2) * sizeof(float));
  p.btotal = bo;
  return true;
}

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
namespace {
struct Timer {
  hipEvent_t* ev = nullptr;   // 2 * cap events
  int cap = 0, used = 0;
  bool open = false;          // a begin is waiting for its end
};
Timer g_timers[FAVOR_KERNEL_COUNT];
}  // namespace

void timing_begin(favor_kernel k, hipStream_t s) {
  Timer& t = g_timers[k];
  if (t.ev && t.used < t.cap) {
    hipEventRecord(t.ev[2 * t.used], s);
    t.open = true;
  }
}

void timing_end(favor_kernel k, hipStream_t s) {
  Timer& t = g_timers[k];
  if (t.open) {
    hipEventRecord(t.ev[2 * t.used + 1], s);
    ++t.used;
    t.open = false;
  }
}

// ---------------------------------------------------------------------------
// Static scratch for favor_attn_noalloc: one array per device (each device
// that loads the library holds its own copy until the process ends).  The
// array's name is only a host-side handle; kernels get the device address
// that hipGetSymbolAddress returns, looked up once per device with that
// device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[FAVOR_NOALLOC_SCRATCH_BYTES];
static void* g_scratch_addr[64];
static std::mutex g_scratch_mu;

static void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_addr[dev] = p;
  }
  return g_scratch_addr[dev];
}

}  // namespace favor

using namespace favor;

// Enumeration arguments at the boundary.  A C caller may pass any int; C++
// may only load values inside an enumeration's range, so every exported
// function reads its enumeration arguments through their object
// representation and rejects values outside the declared ones before any
// other use.
template <class E>
static int enum_bits(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "enumerations are int-sized");
  int v;
  memcpy(&v, &e, sizeof v);
  return v;
}
static bool dtype_ok(const favor_dtype& dt) {
  const int v = enum_bits(dt);
  return v == FAVOR_F32 || v == FAVOR_BF16;
}
static bool fmap_ok(const favor_feature_map& f) {
  const int v = enum_bits(f);
  return v >= FAVOR_FMAP_POSITIVE && v <= FAVOR_FMAP_TRIG;
}
static bool kernel_ok(const favor_kernel& k) {
  const int v = enum_bits(k);
  return v >= 0 && v < FAVOR_KERNEL_COUNT;
}

extern "C" {

int favor_abi_version(void) { return 1; }

const char* favor_status_string(favor_status s) {
  if (enum_bits(s) < FAVOR_OK || enum_bits(s) > FAVOR_ERR_INTERNAL) return "unknown status";
  switch (s) {
    case FAVOR_OK: return "ok";
    case FAVOR_ERR_NULL: return "null pointer argument";
    case FAVOR_ERR_SHAPE: return "invalid shape";
    case FAVOR_ERR_UNSUPPORTED: return "unsupported d, m or dtype";
    case FAVOR_ERR_WORKSPACE: return "workspace missing or too small";
    case FAVOR_ERR_HIP: return "HIP runtime error";
    case FAVOR_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

size_t favor_workspace_bytes(int B, int H, int L, int d, int m, int causal, favor_dtype dtype) {
  if (!dtype_ok(dtype)) return 0;
  Plan p;
  if (!make_plan(p, B, H, L, d, m, 1, causal, dtype, device_cu_count())) return 0;
  return p.total;
}

size_t favor_workspace_bytes_fmap(int B, int H, int L, int d, int m, int causal, favor_feature_map fmap,
                                  favor_dtype dtype) {
  if (!fmap_ok(fmap)) return 0;
  if (!dtype_ok(dtype)) return 0;
  Plan p;
  if (!make_plan(p, B, H, L, d, m, 1, causal, dtype, device_cu_count(), (int)fmap)) return 0;
  return p.total;
}

favor_status favor_features_fmap(const void* X, const float* W, int Hw, float* Phi, int B, int H, int L, int d,
                                 int m, favor_feature_map fmap, favor_dtype dtype, void* stream) {
  if (!fmap_ok(fmap)) return FAVOR_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype)) return FAVOR_ERR_UNSUPPORTED;
  if (!X || !W || !Phi) return FAVOR_ERR_NULL;
  favor_status st = check_shapes(B, H, L, d, m, Hw, dtype);
  if (st != FAVOR_OK) return st;
  if ((int)fmap < FAVOR_FMAP_POSITIVE || (int)fmap > FAVOR_FMAP_TRIG) return FAVOR_ERR_UNSUPPORTED;
  Plan p;
  if (!make_plan(p, B, H, L, d, m, Hw, 0, dtype, device_cu_count(), (int)fmap)) return FAVOR_ERR_HIP;
  clear_pending_error();
  return launch_status(launch_features(p, X, W, Phi, (hipStream_t)stream));
}

favor_status favor_features(const void* X, const float* W, int Hw, float* Phi, int B, int H, int L, int d, int m,
                            favor_dtype dtype, void* stream) {
  if (!dtype_ok(dtype)) return FAVOR_ERR_UNSUPPORTED;
  return favor_features_fmap(X, W, Hw, Phi, B, H, L, d, m, FAVOR_FMAP_POSITIVE, dtype, stream);
}

static favor_status attn_common(const void* Q, const void* K, const void* V, const float* W, int Hw, void* O, int B,
                                int H, int L, int d, int m, float eps, int causal, favor_dtype dtype, void* ws,
                                size_t ws_bytes, void* stream, int fmap = FAVOR_FMAP_POSITIVE) {
  if (!Q || !K || !V || !W || !O) return FAVOR_ERR_NULL;
  favor_status st = check_shapes(B, H, L, d, m, Hw, dtype);
  if (st != FAVOR_OK) return st;
  if (fmap < FAVOR_FMAP_POSITIVE || fmap > FAVOR_FMAP_TRIG) return FAVOR_ERR_UNSUPPORTED;
  Plan p;
  if (!make_plan(p, B, H, L, d, m, Hw, causal, dtype, device_cu_count(), fmap)) return FAVOR_ERR_HIP;
  if (!ws || ws_bytes < p.total || ((uintptr_t)ws & 255) != 0) return FAVOR_ERR_WORKSPACE;
  Tensors t{Q, K, V, W, O, eps, (char*)ws};
  clear_pending_error();
  return launch_status(causal ? launch_causal(p, t, (hipStream_t)stream) : launch_noncausal(p, t, (hipStream_t)stream));
}

favor_status favor_attn_noncausal(const void* Q, const void* K, const void* V, const float* W, int Hw, void* O, int B,
                                  int H, int L, int d, int m, float eps, favor_dtype dtype, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (!dtype_ok(dtype)) return FAVOR_ERR_UNSUPPORTED;
  return attn_common(Q, K, V, W, Hw, O, B, H, L, d, m, eps, 0, dtype, ws, ws_bytes, stream);
}

favor_status favor_attn_causal(const void* Q, const void* K, const void* V, const float* W, int Hw, void* O, int B,
                               int H, int L, int d, int m, float eps, favor_dtype dtype, void* ws, size_t ws_bytes,
                               void* stream) {
  if (!dtype_ok(dtype)) return FAVOR_ERR_UNSUPPORTED;
  return attn_common(Q, K, V, W, Hw, O, B, H, L, d, m, eps, 1, dtype, ws, ws_bytes, stream);
}

static void timer_free(Timer& t) {
  if (t.ev) {
    for (int i = 0; i < 2 * t.cap; ++i) hipEventDestroy(t.ev[i]);
    delete[] t.ev;
  }
  t = Timer();
}

size_t favor_bwd_workspace_bytes(int B, int H, int L, int d, int m, int causal, favor_dtype dtype) {
  if (!dtype_ok(dtype)) return 0;
  Plan p;
  if (!make_plan(p, B, H, L, d, m, 1, causal, dtype, device_cu_count())) return 0;
  return p.btotal;
}

// ---------------------------------------------------------------------------
// strided layouts and value widths d_v != d (gather, contiguous path, scatter)
// ---------------------------------------------------------------------------
static size_t strided_extra(const Plan& p) { return align256((size_t)p.BH * p.L * p.D * p.esize); }

size_t favor_workspace_bytes_strided(int B, int H, int L, int dk, int dv, int m, int causal, favor_feature_map fmap,
                                     favor_dtype dtype) {
  if (!fmap_ok(fmap)) return 0;
  if (!dtype_ok(dtype)) return 0;
  Plan p;
  if (dv < 1 || !make_plan(p, B, H, L, dk, m, 1, causal, dtype, device_cu_count(), (int)fmap)) return 0;
  return align256(p.total) + 4 * strided_extra(p);
}

static bool contiguous(const long long* s, int H, int L, int d) {
  return s[2] == d && s[1] == (long long)L * d && s[0] == (long long)H * L * d;
}

favor_status favor_attn_strided(const void* Q, const long long* q_strides, const void* K, const long long* k_strides,
                                const void* V, const long long* v_strides, const float* W, int Hw, void* O,
                                const long long* o_strides, int B, int H, int L, int dk, int dv, int m, float eps,
                                int causal, favor_feature_map fmap, favor_dtype dtype, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!fmap_ok(fmap)) return FAVOR_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype)) return FAVOR_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !W || !O || !q_strides || !k_strides || !v_strides || !o_strides) return FAVOR_ERR_NULL;
  favor_status st = check_shapes(B, H, L, dk, m, Hw, dtype);
  if (st != FAVOR_OK) return st;
  if (dv < 1 || dv > 65536) return FAVOR_ERR_SHAPE;
  if ((int)fmap < FAVOR_FMAP_POSITIVE || (int)fmap > FAVOR_FMAP_TRIG) return FAVOR_ERR_UNSUPPORTED;
  for (const long long* sp : {q_strides, k_strides, v_strides, o_strides})
    for (int i = 0; i < 3; ++i)
      if (sp[i] < 0) return FAVOR_ERR_SHAPE;
  Plan p;
  if (!make_plan(p, B, H, L, dk, m, Hw, causal, dtype, device_cu_count(), (int)fmap)) return FAVOR_ERR_HIP;
  const size_t inner = align256(p.total), ex = strided_extra(p);
  if (!ws || ws_bytes < inner + 4 * ex || ((uintptr_t)ws & 255) != 0) return FAVOR_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  clear_pending_error();
  char* base = (char*)ws;
  char* qc = base + inner;
  char* kc = qc + ex;
  char* vc = kc + ex;
  char* oc = vc + ex;
  const bool qcont = contiguous(q_strides, H, L, dk), kcont = contiguous(k_strides, H, L, dk);
  const bool same_w = dv == dk;
  const bool vcont = same_w && contiguous(v_strides, H, L, dk), ocont = same_w && contiguous(o_strides, H, L, dk);
  hipError_t e = hipSuccess;
  const void* qp = Q;
  const void* kp = K;
  if (!qcont) {
    e = gather_rows(Q, qc, p, q_strides, 0, dk, dk, s);
    qp = qc;
  }
  if (e == hipSuccess && !kcont) {
    e = gather_rows(K, kc, p, k_strides, 0, dk, dk, s);
    kp = kc;
  }
  for (int c0 = 0; e == hipSuccess && c0 < dv; c0 += dk) {
    const void* vp = V;
    void* op = O;
    if (!vcont) {
      e = gather_rows(V, vc, p, v_strides, c0, dv, dk, s);
      vp = vc;
    }
    if (!ocont) op = oc;
    if (e != hipSuccess) break;
    Tensors t{qp, kp, vp, W, op, eps, base};
    e = causal ? launch_causal(p, t, s) : launch_noncausal(p, t, s);
    if (e == hipSuccess && !ocont) e = scatter_rows(oc, O, p, o_strides, c0, dv - c0 < dk ? dv - c0 : dk, dk, s);
  }
  return launch_status(e);
}

favor_status favor_draw_projection(unsigned long long seed, int Hw, int m, int d, int orthogonal, float scale,
                                   float* W, void* stream) {
  if (!W) return FAVOR_ERR_NULL;
  if (Hw < 1 || m < 1 || m > 65536 || d < 1 || d > 128) return FAVOR_ERR_SHAPE;
  if ((int64_t)Hw * m * d >= ((int64_t)1 << 31)) return FAVOR_ERR_SHAPE;
  clear_pending_error();
  return launch_status(launch_draw(seed, Hw, m, d, orthogonal ? 1 : 0, scale, W, (hipStream_t)stream));
}

favor_status favor_softmax_attn(const void* Q, const void* K, const void* V, void* O, int B, int H, int L, int d,
                                float scale, int causal, favor_dtype dtype, void* stream) {
  if (!dtype_ok(dtype)) return FAVOR_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !O) return FAVOR_ERR_NULL;
  favor_status st = check_shapes(B, H, L, d, 32, 1, dtype);
  if (st != FAVOR_OK) return st;
  Plan p{};
  p.B = B; p.H = H; p.L = L; p.D = d; p.BH = B * H; p.dt = dtype;
  p.esize = dtype == FAVOR_BF16 ? 2 : 4;
  clear_pending_error();
  return launch_status(launch_softmax(p, Q, K, V, O, scale, causal ? 1 : 0, (hipStream_t)stream));
}

static favor_status bwd_common(const void* Q, const void* K, const void* V, const float* W, int Hw, const void* dO,
                               void* dQ, void* dK, void* dV, int B, int H, int L, int d, int m, float eps, int causal,
                               favor_dtype dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!Q || !K || !V || !W || !dO || !dQ || !dK || !dV) return FAVOR_ERR_NULL;
  favor_status st = check_shapes(B, H, L, d, m, Hw, dtype);
  if (st != FAVOR_OK) return st;
  Plan p;
  if (!make_plan(p, B, H, L, d, m, Hw, causal, dtype, device_cu_count())) return FAVOR_ERR_HIP;
  if (!ws || ws_bytes < p.btotal || ((uintptr_t)ws & 255) != 0) return FAVOR_ERR_WORKSPACE;
  BwdTensors t{Q, K, V, W, dO, dQ, dK, dV, eps, (char*)ws};
  clear_pending_error();
  return launch_status(causal ? launch_causal_bwd(p, t, (hipStream_t)stream) : launch_noncausal_bwd(p, t, (hipStream_t)stream));
}

favor_status favor_attn_noncausal_bwd(const void* Q, const void* K, const void* V, const float* W, int Hw,
                                      const void* dO, void* dQ, void* dK, void* dV, int B, int H, int L, int d,
                                      int m, float eps, favor_dtype dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype)) return FAVOR_ERR_UNSUPPORTED;
  return bwd_common(Q, K, V, W, Hw, dO, dQ, dK, dV, B, H, L, d, m, eps, 0, dtype, ws, ws_bytes, stream);
}

favor_status favor_attn_causal_bwd(const void* Q, const void* K, const void* V, const float* W, int Hw,
                                   const void* dO, void* dQ, void* dK, void* dV, int B, int H, int L, int d, int m,
                                   float eps, favor_dtype dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(dtype)) return FAVOR_ERR_UNSUPPORTED;
  return bwd_common(Q, K, V, W, Hw, dO, dQ, dK, dV, B, H, L, d, m, eps, 1, dtype, ws, ws_bytes, stream);
}

favor_status favor_timing_start(favor_kernel k, int capacity) {
  if (!kernel_ok(k)) return FAVOR_ERR_SHAPE;
  if (capacity < 1) return FAVOR_ERR_SHAPE;
  Timer& t = g_timers[k];
  timer_free(t);
  t.ev = new hipEvent_t[2 * (size_t)capacity];
  for (int i = 0; i < 2 * capacity; ++i) {
    // timing only: no system-scope fence at each record (its cache writeback
    // and invalidate would otherwise be timed with the kernel)
    if (hipEventCreateWithFlags(&t.ev[i], hipEventDisableSystemFence) != hipSuccess) {
      for (int j = 0; j < i; ++j) hipEventDestroy(t.ev[j]);
      delete[] t.ev;
      t = Timer();
      return FAVOR_ERR_HIP;
    }
  }
  t.cap = capacity;
  return FAVOR_OK;
}

favor_status favor_timing_stop(favor_kernel k, double* ms, int max_launches, int* launches) {
  if (!kernel_ok(k)) return FAVOR_ERR_SHAPE;
  if (!launches || (max_launches > 0 && !ms)) return FAVOR_ERR_NULL;
  Timer& t = g_timers[k];
  favor_status st = FAVOR_OK;
  for (int i = 0; i < t.used; ++i) {
    float e = 0.f;
    if (hipEventSynchronize(t.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&e, t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess) {
      st = FAVOR_ERR_HIP;
      break;
    }
    if (i < max_launches) ms[i] = e;
  }
  *launches = t.used;
  timer_free(t);
  return st;
}

const char* favor_kernel_name(favor_kernel k) {
  if (!kernel_ok(k)) return "unknown";
  switch (k) {
    case FAVOR_KERNEL_FEATURES: return "k_features";
    case FAVOR_KERNEL_REDUCE: return "k_reduce";
    case FAVOR_KERNEL_COMBINE: return "k_combine";
    case FAVOR_KERNEL_APPLY: return "k_apply";
    case FAVOR_KERNEL_SPAN_SCAN: return "k_span_scan";
    case FAVOR_KERNEL_CAUSAL: return "k_causal";
    case FAVOR_KERNEL_BWD_PREP: return "k_bprep";
    case FAVOR_KERNEL_BWD_REDUCE: return "k_bred";
    case FAVOR_KERNEL_BWD_COMBINE: return "k_bcombine";
    case FAVOR_KERNEL_BWD_Q: return "k_bside_q";
    case FAVOR_KERNEL_BWD_K: return "k_bside_k";
    case FAVOR_KERNEL_SOFTMAX: return "k_softmax";
    case FAVOR_KERNEL_DRAW: return "k_draw";
    default: return "unknown";
  }
}

favor_status favor_attn(const void* Q, const void* K, const void* V, const float* W, int Hw, void* O, int B, int H,
                        int L, int d, int m, float eps, int causal, favor_dtype dtype, void* ws, size_t ws_bytes,
                        void* stream) {
  if (!dtype_ok(dtype)) return FAVOR_ERR_UNSUPPORTED;
  return attn_common(Q, K, V, W, Hw, O, B, H, L, d, m, eps, causal, dtype, ws, ws_bytes, stream);
}

favor_status favor_attn_noalloc(const void* Q, const void* K, const void* V, const float* W, int Hw, void* O,
                                int B, int H, int L, int d, int m, float eps, int causal, favor_dtype dtype,
                                void* stream) {
  if (!dtype_ok(dtype)) return FAVOR_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !W || !O) return FAVOR_ERR_NULL;
  favor_status st = check_shapes(B, H, L, d, m, Hw, dtype);
  if (st != FAVOR_OK) return st;
  Plan p;
  if (!make_plan(p, B, H, L, d, m, Hw, causal, dtype, device_cu_count())) return FAVOR_ERR_HIP;
  if (p.total > FAVOR_NOALLOC_SCRATCH_BYTES) return FAVOR_ERR_WORKSPACE;    // nothing launched
  void* ws = scratch_address();
  if (!ws) return FAVOR_ERR_HIP;
  return attn_common(Q, K, V, W, Hw, O, B, H, L, d, m, eps, causal, dtype, ws, FAVOR_NOALLOC_SCRATCH_BYTES, stream);
}

favor_status favor_attn_fmap(const void* Q, const void* K, const void* V, const float* W, int Hw, void* O, int B,
                             int H, int L, int d, int m, float eps, int causal, favor_feature_map fmap,
                             favor_dtype dtype, void* ws, size_t ws_bytes, void* stream) {
  if (!fmap_ok(fmap)) return FAVOR_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype)) return FAVOR_ERR_UNSUPPORTED;
  return attn_common(Q, K, V, W, Hw, O, B, H, L, d, m, eps, causal, dtype, ws, ws_bytes, stream, (int)fmap);
}

}  // extern "C"
