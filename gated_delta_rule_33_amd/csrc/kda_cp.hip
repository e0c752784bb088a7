// Context-parallel state chaining for the KDA forward, the single-GPU part of
// the context parallelism of the page "feat(kda): integrate KDA attention with
// tokamax backend and CP support" (Context Parallelism Support: the kernel
// derives per-rank sequence metadata from segment_ids and coordinates the
// recurrent state across ranks; its tests check that splitting T over 2 or 4
// ranks reproduces the unsplit forward, also with packed segments that cross
// a split or start exactly at one).
//
// Each row of T tokens is cut into P slices of L = T / P tokens (slice r of
// row b is "rank" r's share; on one GPU the B*P slices are the rows of one
// batched call).  Because the recurrence is affine in the state a segment
// starts from, rank r can run its slice with a zero state for the segment it
// continues (its "carried" segment) and fix the result afterwards:
//   pass 1   forward on every slice: end state E_r (carried state = 0) and
//            the transition M_r (d end state / d carried start state);
//   chain    C_0 = 0, C_{r+1} = E_r + [slice r carried] M_r C_r, kept only
//            where slice r+1 continues slice r's last segment;
//   pass 2   the recurrence again on the same chunk records, with C_r as the
//            carried segment's start state.
// Across GPUs the chain is P-1 point-to-point hops of one state; here one
// kernel runs every hop.  The kernels below are that glue: the per-slice
// segment plan, the routing of per-segment states between the global layout
// [B, N, H, K, V] and the per-slice layout [B*P, N, H, K, V], and the chain.
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kPlanThreads = 256;

// One workgroup per row: slice by slice, count the segment starts (a token
// with a non-zero id that differs from its predecessor's) and decide whether
// the slice's first token continues the previous slice's segment.
__global__ __launch_bounds__(kPlanThreads) void cp_plan_kernel(const int32_t* __restrict__ seg, int64_t T, int P,
                                                               int n_max, int32_t* __restrict__ plan) {
  __shared__ int part[kPlanThreads / kWave];
  const int64_t b = blockIdx.x;
  const int64_t L = T / P;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int before = 0;   // segment starts in earlier slices (thread 0's copy is the one used)
  for (int r = 0; r < P; ++r) {
    const int64_t t0 = (int64_t)r * L;
    int starts = 0;
    if (seg != nullptr) {
      for (int64_t t = t0 + tid; t < t0 + L; t += kPlanThreads) {
        const int32_t s = seg[b * T + t];
        starts += (s != 0 && (t == 0 || seg[b * T + t - 1] != s)) ? 1 : 0;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) starts += __shfl_xor(starts, off);
    if (lane == 0) part[wave] = starts;
    __syncthreads();
    if (tid == 0) {
      int in_slice = 0;
      for (int i = 0; i < kPlanThreads / kWave; ++i) in_slice += part[i];
      int carried, base, count;
      if (seg == nullptr) {
        carried = r > 0 ? 1 : 0;
        base = 0;
        count = 1;
      } else {
        const int32_t s0 = seg[b * T + t0];
        carried = (r > 0 && s0 != 0 && seg[b * T + t0 - 1] == s0) ? 1 : 0;
        base = before - carried;
        count = carried + in_slice;
      }
      int32_t* e = plan + (b * P + r) * 4;
      e[0] = carried;
      e[1] = base;
      e[2] = count;
      e[3] = (base + count > n_max) ? 1 : 0;
      before += in_slice;
    }
    __syncthreads();
  }
}

constexpr int kCopyThreads = 256;

// One workgroup per (slice, local segment, head) state.  Start states (not
// ends): the slice's local segment l starts from the chain's state if the
// slice continues it (zero when carry is NULL), else from the caller's state
// of its global segment.  Final-state gradients (ends): the slice's last
// local segment, when the next slice continues it, takes the chain's
// gradient (zero when carry is NULL); any other takes the caller's gradient
// of its global segment.  Unused slots get zero.
__global__ __launch_bounds__(kCopyThreads) void cp_gather_kernel(const int32_t* __restrict__ plan,
                                                                 const float* __restrict__ init,
                                                                 const float* __restrict__ carry,
                                                                 float* __restrict__ local, int P, int nm, int64_t H,
                                                                 int64_t KV, int ends) {
  const int64_t id = blockIdx.x;
  const int64_t h = id % H, l = (id / H) % nm, rho = id / (H * nm), b = rho / P, r = rho % P;
  const int32_t* e = plan + rho * 4;
  const float* src = nullptr;
  const bool chained = ends ? (l == e[2] - 1 && r + 1 < P && plan[(rho + 1) * 4] != 0) : (l == 0 && e[0] != 0);
  if (chained) {
    src = carry ? carry + (rho * H + h) * KV : nullptr;
  } else if (l < e[2] && e[1] + l < nm && init != nullptr) {
    src = init + ((b * nm + e[1] + l) * H + h) * KV;
  }
  const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
  f32x4* d4 = reinterpret_cast<f32x4*>(local + id * KV);
  for (int64_t i = threadIdx.x; i < KV / 4; i += kCopyThreads) d4[i] = src ? s4[i] : f32x4{0, 0, 0, 0};
}

// One workgroup per (row, global segment slot, head): the final state of
// global segment s is the one of the last slice that holds it (the gradient
// of its initial state, with `first`, the one of the first slice); slots of
// segments that do not occur get zero.
__global__ __launch_bounds__(kCopyThreads) void cp_scatter_kernel(const int32_t* __restrict__ plan,
                                                                  const float* __restrict__ local,
                                                                  float* __restrict__ fin, int P, int nm, int64_t H,
                                                                  int64_t KV, int first) {
  const int64_t id = blockIdx.x;
  const int64_t h = id % H, s = (id / H) % nm, b = id / (H * nm);
  const float* src = nullptr;
  for (int i = 0; i < P; ++i) {
    const int r = first ? i : P - 1 - i;
    const int32_t* e = plan + (b * P + r) * 4;
    if (e[1] <= s && s < e[1] + e[2]) {
      const int64_t l = s - e[1];
      if (l < nm) src = local + (((b * P + r) * nm + l) * H + h) * KV;
      break;
    }
  }
  const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
  f32x4* d4 = reinterpret_cast<f32x4*>(fin + id * KV);
  for (int64_t i = threadIdx.x; i < KV / 4; i += kCopyThreads) d4[i] = src ? s4[i] : f32x4{0, 0, 0, 0};
}

constexpr int kChainThreads = 256;
constexpr int kChainCols = 16;

// One workgroup per (row, head, 16-column tile of the state): the hops of
// the chain in slice order, C_{r+1} = E_r + [r carried] M_r C_r, in fp32.
// C_r of the tile stays in LDS; thread t owns OPT adjacent outputs of one
// state row.
template <int K>
__global__ __launch_bounds__(kChainThreads) void cp_chain_kernel(const int32_t* __restrict__ plan,
                                                                 const float* __restrict__ fin1,
                                                                 const float* __restrict__ trans,
                                                                 float* __restrict__ carry, int P, int nm, int64_t H,
                                                                 int64_t V) {
  constexpr int OPT = K * kChainCols / kChainThreads;   // outputs per thread
  constexpr int TPR = kChainCols / OPT;                 // threads per state row
  __shared__ float cur[K][kChainCols];
  const int64_t ntile = V / kChainCols;
  const int64_t id = blockIdx.x;
  const int64_t tile = id % ntile, h = (id / ntile) % H, b = id / (ntile * H);
  const int tid = threadIdx.x, row = tid / TPR, c0 = (tid % TPR) * OPT;
  const int64_t v0 = tile * kChainCols;
  const int64_t KV = (int64_t)K * V;
  auto carry_at = [&](int r) { return carry + ((b * P + r) * H + h) * KV + (int64_t)row * V + v0 + c0; };
#pragma unroll
  for (int j = 0; j < OPT; ++j) {
    cur[row][c0 + j] = 0.f;
    carry_at(0)[j] = 0.f;
  }
  __syncthreads();
  for (int r = 1; r < P; ++r) {
    const int32_t* e = plan + (b * P + r) * 4;
    const int32_t* ep = plan + (b * P + r - 1) * 4;
    float acc[OPT];
    if (e[0] && ep[2] >= 1 && ep[2] <= nm) {
      // The previous slice ends inside the segment this one continues, so it
      // holds at least one local segment; its last one is that segment (a
      // slice with more segments than state slots has no such state).
      const float* E = fin1 + (((b * P + r - 1) * nm + (ep[2] - 1)) * H + h) * KV + (int64_t)row * V + v0 + c0;
#pragma unroll
      for (int j = 0; j < OPT; ++j) acc[j] = E[j];
      if (ep[0]) {
        const float* M = trans + ((b * P + r - 1) * H + h) * (int64_t)K * K + (int64_t)row * K;
        for (int k = 0; k < K; ++k) {
          const float mk = M[k];
#pragma unroll
          for (int j = 0; j < OPT; ++j) acc[j] += mk * cur[k][c0 + j];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < OPT; ++j) acc[j] = 0.f;
    }
    __syncthreads();   // every read of C_r is done
#pragma unroll
    for (int j = 0; j < OPT; ++j) {
      cur[row][c0 + j] = acc[j];
      carry_at(r)[j] = acc[j];
    }
    __syncthreads();
  }
}

// The reverse chain for the gradients: X_r, the gradient of the state that
// leaves slice r, is zero for the last slice and, going back,
//     X_r = [slice r+1 continues] (dInit_{r+1} + M_{r+1}^T X_{r+1}),
// where dInit_{r+1} is the gradient the slice's own backward found for the
// state its continued segment starts from (with a zero gradient for the state
// it hands on) and M_{r+1} its transition.  Same tiling as the forward chain.
template <int K>
__global__ __launch_bounds__(kChainThreads) void cp_chain_bwd_kernel(const int32_t* __restrict__ plan,
                                                                     const float* __restrict__ dinit,
                                                                     const float* __restrict__ trans,
                                                                     float* __restrict__ xg, int P, int nm, int64_t H,
                                                                     int64_t V) {
  constexpr int OPT = K * kChainCols / kChainThreads;
  constexpr int TPR = kChainCols / OPT;
  __shared__ float cur[K][kChainCols];
  const int64_t ntile = V / kChainCols;
  const int64_t id = blockIdx.x;
  const int64_t tile = id % ntile, h = (id / ntile) % H, b = id / (ntile * H);
  const int tid = threadIdx.x, row = tid / TPR, c0 = (tid % TPR) * OPT;
  const int64_t v0 = tile * kChainCols;
  const int64_t KV = (int64_t)K * V;
  auto x_at = [&](int r) { return xg + ((b * P + r) * H + h) * KV + (int64_t)row * V + v0 + c0; };
#pragma unroll
  for (int j = 0; j < OPT; ++j) {
    cur[row][c0 + j] = 0.f;
    x_at(P - 1)[j] = 0.f;
  }
  __syncthreads();
  for (int r = P - 2; r >= 0; --r) {
    const int64_t nx = b * P + r + 1;
    float acc[OPT];
    if (plan[nx * 4] != 0) {
      // dInit of the continued segment (local segment 0 of slice r+1) ...
      const float* D = dinit + ((nx * nm) * H + h) * KV + (int64_t)row * V + v0 + c0;
#pragma unroll
      for (int j = 0; j < OPT; ++j) acc[j] = D[j];
      // ... plus M^T X_{r+1}: column `row` of M
      const float* M = trans + (nx * H + h) * (int64_t)K * K + row;
      for (int k = 0; k < K; ++k) {
        const float mk = M[(int64_t)k * K];
#pragma unroll
        for (int j = 0; j < OPT; ++j) acc[j] += mk * cur[k][c0 + j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < OPT; ++j) acc[j] = 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < OPT; ++j) {
      cur[row][c0 + j] = acc[j];
      x_at(r)[j] = acc[j];
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_cp_plan(const CpArgs& a) {
  hipLaunchKernelGGL(cp_plan_kernel, dim3((unsigned)a.B), dim3(kPlanThreads), 0, a.stream, a.seg, a.T, a.P, a.nm,
                     a.plan);
  return hipGetLastError();
}

hipError_t launch_cp_gather(const CpArgs& a) {
  const int64_t n = a.B * a.P * a.nm * a.H;
  hipLaunchKernelGGL(cp_gather_kernel, dim3((unsigned)n), dim3(kCopyThreads), 0, a.stream, a.plan, a.init, a.carry,
                     a.local, a.P, a.nm, a.H, a.K * a.V, a.grads ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_cp_scatter(const CpArgs& a) {
  const int64_t n = a.B * a.nm * a.H;
  hipLaunchKernelGGL(cp_scatter_kernel, dim3((unsigned)n), dim3(kCopyThreads), 0, a.stream, a.plan, a.local, a.fin,
                     a.P, a.nm, a.H, a.K * a.V, a.grads ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_cp_chain_bwd(const CpArgs& a) {
  const dim3 grid((unsigned)(a.B * a.H * (a.V / kChainCols)));
  if (a.K == 64)
    hipLaunchKernelGGL(cp_chain_bwd_kernel<64>, grid, dim3(kChainThreads), 0, a.stream, a.plan, a.local, a.trans,
                       a.carry, a.P, a.nm, a.H, a.V);
  else if (a.K == 128)
    hipLaunchKernelGGL(cp_chain_bwd_kernel<128>, grid, dim3(kChainThreads), 0, a.stream, a.plan, a.local, a.trans,
                       a.carry, a.P, a.nm, a.H, a.V);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_cp_chain(const CpArgs& a) {
  const dim3 grid((unsigned)(a.B * a.H * (a.V / kChainCols)));
  if (a.K == 64)
    hipLaunchKernelGGL(cp_chain_kernel<64>, grid, dim3(kChainThreads), 0, a.stream, a.plan, a.local, a.trans, a.carry,
                       a.P, a.nm, a.H, a.V);
  else if (a.K == 128)
    hipLaunchKernelGGL(cp_chain_kernel<128>, grid, dim3(kChainThreads), 0, a.stream, a.plan, a.local, a.trans,
                       a.carry, a.P, a.nm, a.H, a.V);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kda
