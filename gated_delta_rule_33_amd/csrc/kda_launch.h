// Host-side launchers of the KDA forward kernels (one per kernel family).
// Each validates nothing: kda_api.cpp checks every argument before calling.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kda.h"
#include "kda_common.h"

namespace kda {

enum class InType { F32, BF16 };
enum class OutType { F32, BF16 };

// Everything the kernels of one call need, resolved on the host.
struct CallArgs {
  int64_t B, T, H, K, V;
  InType in;
  OutType out;
  float scale;
  int l2norm;
  int n_max;                   // segments per row with packed input (0: fixed rows)
  int64_t nc_fixed;            // chunks per row without segment_ids: ceil(T / 64)
  int64_t cmax, smax;          // chunk / segment capacities of the tables and records
  const void *q, *k, *v, *g, *beta;
  int gate_mode;               // 0: g is the log decay; 1: log sigmoid(z); 2: lower_bound * sigmoid(z)
  float lower_bound;
  const float *a_log, *dt_bias;   // gate parameters ([H], [H,K]) or NULL
  const float* init;
  const int32_t* seg_ids;
  void* o;
  float* fin;
  float* trans;                // [B,H,K,K] transition of each row's first segment, or NULL
  bool trans_only;             // launch_recur: compute the transition instead of o / states
  // Workspace carve-up.
  TableHeader* hdr;
  SegEntry* segs;
  ChunkEntry* chunks;
  RowInfo* rows;
  char* records;
  int64_t record_bytes;
  FusedCtl* fused_ctl;         // fused forward: scheduling words, then one ready word per record
  uint32_t* fused_ready;
  float* fused_lane_state;     // fused forward: state slices of suspended recurrence lanes [B*H*K*V]
  int n_xcd;                   // XCDs of the device (0: unknown, no fused forward)
  hipStream_t stream;
};

// Short convolution of x [B,T,D] with weight [D,W] (layer step before the kernel).
struct ConvArgs {
  int64_t B, T, D;
  int W;
  bool bf16;                  // x and y are bf16 (else fp32)
  const void* x;
  const float* weight;
  const int32_t* seg;         // [B,T] or NULL
  void* y;
  hipStream_t stream;
};
// Gated RMSNorm over rows of V values (output stage after the kernel).
struct NormArgs {
  int64_t rows, V;
  bool o_bf16, gate_bf16, y_bf16;
  const void *o, *gate;
  const float* weight;        // [V]
  float eps;
  void* y;
  hipStream_t stream;
};

// Context-parallel glue over B rows cut into P slices (one call covers all
// slices).  nm = state slots per row (max_segments, or 1 without segment ids).
struct CpArgs {
  int64_t B, T, H, K, V;
  int P, nm;
  const int32_t* seg;         // [B,T] or NULL (plan)
  int32_t* plan;              // [B,P,4]: carried, first global segment, local segments, overflow
  const float* init;          // [B,nm,H,K,V] caller's start states or NULL (gather)
  float* carry;               // [B*P,H,K,V] chain states (chain: out; gather: in, NULL = zeros)
  float* local;               // [B*P,nm,H,K,V] per-slice states (gather: out; chain, scatter: in)
  const float* trans;         // [B*P,H,K,K] (chain)
  float* fin;                 // [B,nm,H,K,V] (scatter: out)
  bool grads;                 // gather: final-state gradients; scatter: initial-state gradients (first slice)
  hipStream_t stream;
};

// The backward: gradients of the plain forward (g is the log decay).
struct BwdArgs {
  int64_t B, T, H, K, V;
  InType in;
  bool do_bf16;               // d_o is bf16 (else fp32)
  float scale;
  int l2norm;
  int n_max;                  // segments per row with packed input (0: fixed rows)
  int64_t nc_fixed, cmax, smax;
  const void *q, *k, *v, *g, *beta, *d_o;
  const float *init, *d_final;
  float *dq, *dk, *dv, *dg, *dbeta, *d_init;
  TableHeader* hdr;
  SegEntry* segs;
  ChunkEntry* chunks;
  float *rec, *hs, *dhs;      // chunk records, states entering and gradients leaving each 16-row chunk
  float *ds, *dds;            // Delta and dDelta of each 16-row chunk
  hipStream_t stream;
};

int64_t record_bytes(InType in, int64_t K, int64_t V);
int64_t bwd_record_floats(int64_t K, int64_t V);

hipError_t launch_prep(const CallArgs& a);
hipError_t launch_intra(const CallArgs& a);
// The fused forward (bf16, no segment ids, K = V = 128) on devices whose XCDs
// hold 32 compute units each.
bool fused_supported(const CallArgs& a);
hipError_t launch_fused(const CallArgs& a);
int xcd_count();
hipError_t launch_recur(const CallArgs& a);
hipError_t launch_zero_states(const CallArgs& a);
hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t stream);
hipError_t launch_short_conv(const ConvArgs& a);
hipError_t launch_gated_rmsnorm(const NormArgs& a);
// stage 0: chunk quantities, 1: forward states, 2: reverse state recurrence,
// 3: per-chunk input gradients (launched in that order).
hipError_t launch_bwd(const BwdArgs& a, int stage);
hipError_t launch_cp_plan(const CpArgs& a);
hipError_t launch_cp_gather(const CpArgs& a);
hipError_t launch_cp_chain(const CpArgs& a);
hipError_t launch_cp_scatter(const CpArgs& a);
hipError_t launch_cp_chain_bwd(const CpArgs& a);
int cu_count();

}  // namespace kda
