// Host-side plan and launcher declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "../../include/favor.h"

namespace favor {

// What a launcher returns when the plan and the compiled kernels disagree (a
// library bug, reported as FAVOR_ERR_INTERNAL).  The launches themselves use
// plan-computed grids, so a launch reporting this code is a library bug too.
constexpr hipError_t kErrPlan = hipErrorInvalidConfiguration;

// How one call is split over workgroups, and where its scratch lives inside
// the caller's workspace.  Computed only from the shapes and the device's
// compute-unit count, so workspace sizing and the call agree.
struct Plan {
  int B, H, L, D, M, Hw, causal;
  favor_dtype dt;
  int fmap;             // feature map (FM_POS, FM_ELU1, FM_RELU, FM_TRIG)
  int mt;               // rows of W per head as given (m)
  int Mw;               // m rounded up to a multiple of 32 (padding features are zero)
                        // M (features) is Mw, or 2 Mw for the trig map
  int BH;
  int esize;            // bytes per element of Q, K, V, O
  // K-side reduction (non-causal state, or causal span aggregates)
  int splits;           // token ranges per head
  int split_len;        // tokens per range (multiple of 64)
  int rnw;              // waves per reduction workgroup
  int rfbw;             // 32-feature blocks per reduction wave
  int rfgroups;         // reduction feature groups per head (workgroups sharing K, V tiles)
  // causal chunk scan
  int scan3;            // the pipelined one-workgroup-per-CU scan (bf16, d <= 64, m = 256, FAVOR+)
  int x3;               // float32 FAVOR+ with d = 128: the scan on split 16-bit products (k_causal_x3)
  int fgroups;          // feature groups walked in turn by one workgroup
  int fbw;              // 32-feature blocks per wave
  // Q-side apply (non-causal)
  int apply_tile;       // tokens per wave per step
  int apply_nw;         // waves per apply workgroup
  int apply_groups;     // total workgroups
  int apply_steps;      // groups per workgroup
  int fch;              // features per LDS chunk
  // workspace offsets (bytes)
  size_t off_part, off_partz, off_wprep, off_mstate, off_zstate, off_num, off_den, total;
  // backward pass: its reductions (4 waves of one feature block each) and
  // its workspace (a separate layout, sized by favor_bwd_workspace_bytes)
  int bsplits, bsplit_len, bfgroups;
  int bqnw;              // causal backward: waves of a query-walk workgroup
  int brnw;              // backward reductions: waves (feature blocks) per workgroup
  size_t boff_part, boff_partz, boff_zf, boff_lg, boff_cw, boff_wph, boff_wpl, boff_wt, boff_wtl, boff_rows_hi,
      boff_rows_lo, boff_op, boff_acc, btotal;
};

bool make_plan(Plan& p, int B, int H, int L, int d, int m, int Hw, int causal, favor_dtype dt, int num_cus,
               int fmap = 0);
int device_cu_count();

struct Tensors {
  const void* q;
  const void* k;
  const void* v;
  const float* w;
  void* o;
  float eps;
  char* ws;
};

struct BwdTensors {
  const void* q;
  const void* k;
  const void* v;
  const float* w;
  const void* g;        // upstream gradient dLoss/dO
  void* dq;
  void* dk;
  void* dv;
  float eps;
  char* ws;
};

// Arguments of the K-side reductions (k_reduce, k_reduce_x3).
struct RedArgs {
  const void* k;
  const void* v;
  const float* w;
  float* part;   // [BH][splits][M][D]
  float* partz;  // [BH][splits][M]
  int L, M, H, Hw, splits, split_len;
  int Mw;        // feature rows per head (M, or M/2 for the trig map), a multiple of 32
  int mt;        // rows of W per head as given; features of rows >= mt are padding, set to 0
  void* wp;      // non-causal: the apply's projection operand, written by the split-0
                 // workgroups from the W fragments they load (nullptr: not written)
};

// Arguments of the causal chunk scans (k_causal, k_causal2, k_causal_x3).
struct CausalArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* w;
  void* o;
  const float* prefix;    // [BH][spans][M][D] exclusive prefixes of S
  const float* prefixz;   // [BH][spans][M]
  float* num;             // [BH][L][D] partial numerators (fgroups > 1)
  float* den;             // [BH][L]
  int L, M, H, Hw, spans, span_len, fgroups;
  float eps;
  int Mw;                 // feature rows per head (M, or M/2 for the trig map), a multiple of 32
  int mt;                 // rows of W per head as given; features of rows >= mt are padding
};

// Non-causal attention of short heads in one launch (favor_small.hip):
// L <= 64, m <= 256, d in {32, 64}, FAVOR+.
bool small_nc_fits(const Plan& p);
hipError_t launch_small_nc(const Plan& p, const Tensors& t, hipStream_t s);

// Kernel timing hooks (see favor_timing_start): record the next free event
// pair of kernel k around a launch on stream s.
void timing_begin(favor_kernel k, hipStream_t s);
void timing_end(favor_kernel k, hipStream_t s);

hipError_t launch_features(const Plan& p, const void* x, const float* w, float* phi, hipStream_t s);
hipError_t launch_noncausal(const Plan& p, const Tensors& t, hipStream_t s);
hipError_t launch_causal(const Plan& p, const Tensors& t, hipStream_t s);
hipError_t launch_causal3(const Plan& p, const Tensors& t, hipStream_t s);
hipError_t launch_causal_x3(const Plan& p, const Tensors& t, hipStream_t s);
hipError_t launch_reduce_x3(const Plan& p, const void* k, const void* v, const float* w, float* part, float* partz,
                            hipStream_t s, int nsplit);
hipError_t gather_rows(const void* src, void* dst, const Plan& p, const long long* strides, int c0, int width, int n,
                       hipStream_t s);
hipError_t scatter_rows(const void* src, void* dst, const Plan& p, const long long* strides, int c0, int n, int srow,
                        hipStream_t s);
hipError_t launch_draw(unsigned long long seed, int Hw, int m, int d, int orthogonal, float scale, float* W,
                       hipStream_t s);
hipError_t launch_softmax(const Plan& p, const void* q, const void* k, const void* v, void* o, float scale,
                          int causal, hipStream_t s);
hipError_t launch_noncausal_bwd(const Plan& p, const BwdTensors& t, hipStream_t s);
hipError_t launch_causal_bwd(const Plan& p, const BwdTensors& t, hipStream_t s);
// nsplit: how many token ranges to reduce (the first nsplit of p.splits;
// -1: all).  The causal scans never read the last span's aggregate.
// wp: non-causal only, the apply's projection operand (written by the
// reduction; nullptr for the causal span aggregates)
hipError_t launch_reduce(const Plan& p, const void* k, const void* v, const float* w, float* part, float* partz,
                         hipStream_t s, int nsplit = -1, void* wp = nullptr);

}  // namespace favor
