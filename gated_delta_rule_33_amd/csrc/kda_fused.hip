// Fused KDA forward for bf16 inputs without segment ids: the intra-chunk
// items and the inter-chunk recurrence of the chunk form of the "Delta Rule
// formulation" (page "feat(kda): integrate KDA attention with tokamax backend
// and CP support", Implementation Details) in one persistent kernel, so that
// the per-(chunk, head) records pass from their producer to their consumers
// on one XCD, through its L2 while they stay there.  The pages' own answer to
// the same problem is a fused forward ("Add packed KDA forward megakernel",
// Summary); this is its MI355X form.  Producers are not held back to the
// recurrence's pace, and an XCD's L2 holds about ten chunks of its heads'
// records, so most records are still written back to HBM and read again;
// with one producer workgroup per CU beside a lane the kernel is bound by
// producing and stays behind the two-kernel schedule.
//
// Layout of the work.  Two workgroups of four waves run on every compute unit
// (about 66 KB of LDS each).  The first to arrive on a CU runs recurrence
// lanes: one (row, head, 16 value columns) each, chunk by chunk, four waves
// each doing both the chain and the read-out of its token block (the state
// update of kda_delta.h); the second produces records
// (the intra-chunk item of kda_intra_item.h) from a queue.  A sequence-head
// (b, h) belongs to XCD (b H + h) mod n_xcd: its lanes and its records are
// handled only by workgroups whose hardware XCC_ID is that XCD, so producer
// and consumers of a record share one L2.  Queues are per XCD and ordered
// chunk-major, so every XCD produces the first chunks of all its heads first.
//
// Hand-over.  A producer's four waves wait for their record stores to be
// acknowledged (s_waitcnt vmcnt(0)), meet at a barrier, and one lane sets
// the record's ready word with an agent-scope store; a consumer wave polls
// that word with agent-scope loads (which bypass the CU's L1) and reads the
// record only after seeing it set.  The record lines are first touched by
// the consumer's CU after the flag, so its L1 holds no stale copy.
//
// Progress does not depend on how many workgroups are resident at once (the
// dispatcher may hold some back, e.g. while other kernels occupy compute
// units).  Producing an item never waits.  A recurrence lane checks, at the
// end of every chunk, that the record it will need after the next one is
// ready; if not, it stores its state slice to the workspace and steps out,
// and its workgroup claims unclaimed items of its XCD's queue and produces
// them itself until the records are ready, then resumes the lane.  Only once
// every item has been claimed by a running workgroup (whose production
// completes without waiting) does a workgroup wait for a record.  Every wait
// is still bounded: after kSpinLimit polls the wave gives up, raises
// KDA_FLAG_FUSED_TIMEOUT and goes on (results are then undefined, but the
// kernel ends).
#include "kda_delta.h"
#include "kda_intra_item.h"

namespace kda {
namespace {

using namespace detail;

constexpr uint32_t kSpinLimit = 1u << 20;
constexpr int kVT = 16;         // value columns per recurrence lane
constexpr int kOutLd = 20;      // row pitch of the output staging tile

__device__ __forceinline__ unsigned read_xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v;
}
// Compute unit within its XCD from HW_ID: CU [11:8], SH [12], SE [15:13].
__device__ __forceinline__ unsigned read_cu_slot() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(v));
  return (((v >> 13) & 7u) << 5) | (((v >> 12) & 1u) << 4) | ((v >> 8) & 15u);
}

struct FusedParams {
  IntraParams ip;        // inputs, records, table header (flags)
  int64_t n_sh;          // sequence-heads B * H
  int64_t nc;            // chunks per row
  int n_xcd;
  const float* init;
  float* fin;
  void* o;
  FusedCtl* ctl;
  uint32_t* ready;       // one word per record
  float* lane_state;     // a suspended lane's state slice, [n_sh * V/16][K * 16]
};

__device__ __forceinline__ void wait_ready(const uint32_t* word, TableHeader* hdr) {
  uint32_t spins = 0;
  while (__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
    if (++spins >= kSpinLimit) {
      atomicOr(&hdr->flags, KDA_FLAG_FUSED_TIMEOUT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

__device__ __forceinline__ bool is_ready(const uint32_t* word) {
  return __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

// The queue of one XCD: its sequence-heads xcd, xcd + n_xcd, ... (hx of
// them), chunk-major.  Ticket q is chunk q / hx of the (q % hx)-th of them.
// Record indices stay below 2^30 here, so the arithmetic is 32-bit.
struct XcdQueue {
  int xcd;
  int64_t hx;
  __device__ int64_t item(const FusedParams& p, int64_t q) const {   // -1 past the end
    const uint32_t qq = (uint32_t)q, hh = (uint32_t)hx, H = (uint32_t)p.ip.H, nc = (uint32_t)p.nc;
    if (hh == 0 || q >= (int64_t)hh * nc) return -1;
    const uint32_t n = qq / hh;
    const uint32_t sh = (uint32_t)xcd + (uint32_t)p.n_xcd * (qq - n * hh);
    const uint32_t b = sh / H;
    return (int64_t)((b * nc + n) * H + (sh - b * H));
  }
};

// Produces one record with the calling workgroup's four waves from the rows
// `in` and publishes it, loading the rows of the item next_item() names into
// `next` meanwhile (see intra4_item).
template <int K, int V, class NextItem>
__device__ __forceinline__ void produce(const FusedParams& p, int64_t item, char* lds, const ItemRows<K>& in,
                                        const NextItem& next_item, ItemRows<K>& next) {
  intra4_item<K, V, false>(p.ip, item, lds, in, next_item, next);
  __builtin_amdgcn_s_waitcnt(0);   // this wave's record stores are acknowledged
  block_sync();
  if (threadIdx.x == 0) __hip_atomic_store(p.ready + item, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Four consecutive outputs.  Plain stores: a lane's 16 value columns fill
// half of each 128-byte line of fp32 o, and L2 joins the two halves (the
// neighbouring tile's lane writes the other); streamed partial lines would
// each be written back at the cost of a whole line.
__device__ __forceinline__ void store_out4(float* o, int64_t i, const f32x4& x) {
  *reinterpret_cast<f32x4*>(o + i) = x;
}
__device__ __forceinline__ void store_out4(uint16_t* o, int64_t i, const f32x4& x) {
  uint32_t w[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const __bf16 a = to_bf16(x[2 * j]), b = to_bf16(x[2 * j + 1]);
    w[j] = (uint32_t)*reinterpret_cast<const uint16_t*>(&a) | ((uint32_t)*reinterpret_cast<const uint16_t*>(&b) << 16);
  }
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2*>(o + i) = u32x2{w[0], w[1]};
}

// One recurrence lane: sequence-head sh (row b, head h), value columns
// 16 j .. 16 j + 15, the row's chunks from n_start on, in order.  Records
// n_start and n_start + 1 must be ready.  Returns the chunk count when done,
// or the chunk n to resume at when record n + 1 is not ready yet at the end
// of chunk n - 1; the state entering chunk n is then in the lane's slice of
// p.lane_state (a lane starting at n_start > 0 reads its state from there).
// Per chunk, with S the
// K x 16 state slice entering it: Delta = U - W S (wave w: tokens 16w ..),
// S <- diag(exp(G_C)) S + Kt^T Delta (wave w: its key-channel blocks),
// O = scale Qg S + scale Aqk Delta.  S and Delta pass between the waves
// through LDS; each wave's share of a record is loaded into its registers
// one chunk ahead, after the record's ready word is set.
template <class TO, int K, int V>
__device__ __forceinline__ int64_t recur_lane(const FusedParams& p, int64_t sh, int j, char* lds, int* s_word,
                                              int64_t n_start) {
  using P = Prec<uint16_t>;
  using PS = typename P::S;
  using PD = typename P::D;
  using PW = typename P::W;
  using PK = typename P::Kt;
  using PQ = typename P::Qg;
  using PA = typename P::Aq;
  using L = RecordLayout<uint16_t, K, V>;
  constexpr int NCB = K / 64;
  constexpr int KB = K / 32;
  using DL = DeltaLds<uint16_t>;
  constexpr int TS = tile_bytes<PS>();
  static_assert(KB * TS + sizeof(DL) + 4 * 16 * kOutLd * 4 <= sizeof(Intra4Smem<K, V>), "lane LDS");
  char* s_state = lds;
  DL& s_delta = *reinterpret_cast<DL*>(s_state + KB * TS);
  float* s_out = reinterpret_cast<float*>(s_state + KB * TS + sizeof(DL));   // [4][16 * kOutLd]

  const int lane = opaque((int)threadIdx.x) & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int m = lane & 15, gq = lane >> 4;
  const int64_t H = p.ip.H, T = p.ip.T;
  const int64_t b = sh / H, h = sh % H;
  const int64_t n_chunks = p.nc;
  TableHeader* hdr = p.ip.hdr;
  auto rec_index = [&](int64_t n) { return (b * p.nc + n) * H + h; };
  auto record = [&](int64_t n) { return p.ip.records + rec_index(n) * p.ip.record_bytes; };

  TO* out = static_cast<TO*>(p.o);
  const int v0 = kVT * j;
  PW wn[KB];
  f32x4 u;
  PK kt[NCB][2];
  f32x4 gc[NCB];
  float ks[NCB];
  PQ qg[KB];
  PA aq[2];
  auto load_w = [&](const char* r) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) wn[kb].load(r + L::kWn + (int64_t)(w * KB + kb) * tile_bytes<PW>(), lane);
    u = reinterpret_cast<const f32x4*>(r + L::kU + (int64_t)(w * (V / 16) + j) * 1024)[lane];
  };
  auto load_kt = [&](const char* r) {
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kt[c][kb].load(r + L::kKt + (int64_t)((w * NCB + c) * 2 + kb) * tile_bytes<PK>(), lane);
      gc[c] = reinterpret_cast<const f32x4*>(r + L::kGc)[4 * (w * NCB + c) + gq];
      ks[c] = reinterpret_cast<const float*>(r + L::kKs)[w * NCB + c + vector_zero()];
    }
  };
  auto load_q = [&](const char* r) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qg[kb].load(r + L::kQg + (int64_t)(w * KB + kb) * tile_bytes<PQ>(), lane);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      if (kb <= w / 2) aq[kb].load(r + L::kAqk + (int64_t)aqk_tile(w, kb) * tile_bytes<PA>(), lane);
  };

  // State slice: lane (column v0 + m, rows 16cb + 4gq + i) of its blocks,
  // from the initial state, or from the saved slice when resuming.
  float* saved = p.lane_state + ((sh * (V / kVT) + j) * K) * kVT;
  f32x4 st[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const int c0 = 16 * (w * NCB + c) + 4 * gq;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st[c][i] = n_start > 0 ? saved[(c0 + i) * kVT + m]
                             : (p.init ? p.init[((b * H + h) * K + c0 + i) * V + v0 + m] : 0.f);
    float x[4] = {st[c][0], st[c][1], st[c][2], st[c][3]};
    const int cb = w * NCB + c;
    PS::store_half(s_state + (cb / 2) * TS, lane, cb & 1, x);
  }
  if (n_start < n_chunks) {
    wait_ready(p.ready + rec_index(n_start), hdr);
    const char* r0 = record(n_start);
    load_w(r0);
    load_kt(r0);
    load_q(r0);
  }
  block_sync();

  for (int64_t n = n_start; n < n_chunks; ++n) {
    const int64_t t0 = n * kChunk;
    const int len = (int)min<int64_t>(kChunk, T - t0);
    const bool has_next = n + 1 < n_chunks;
    const char* rn1 = record(has_next ? n + 1 : n);

    PS sf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sf[kb].load(s_state + kb * TS, lane);
    {
      f32x4 d0 = u, d1 = {0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < KB; kb += 2) {
        mma(d0, wn[kb], sf[kb]);
        if (kb + 1 < KB) mma(d1, wn[kb + 1], sf[kb + 1]);
      }
      float x[4] = {d0[0] + d1[0], d0[1] + d1[1], d0[2] + d1[2], d0[3] + d1[3]};
      delta_store(s_delta, w, lane, x);
    }
    if (has_next) wait_ready(p.ready + rec_index(n + 1), hdr);
    load_w(rn1);
    block_sync();   // B1

    DeltaOperands<uint16_t> du;
    du.load(s_delta, lane);
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      state_update<uint16_t>(st[c], gc[c], ks[c], kt[c], du);
      float x[4] = {st[c][0], st[c][1], st[c][2], st[c][3]};
      const int cb = w * NCB + c;
      PS::store_half(s_state + (cb / 2) * TS, lane, cb & 1, x);
    }
    load_kt(rn1);
    PD dd[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) dd[kb].load(s_delta.d + kb * DL::TD, lane);

    f32x4 o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < KB; kb += 2) {
      mma(o0, qg[kb], sf[kb]);
      if (kb + 1 < KB) mma(o1, qg[kb + 1], sf[kb + 1]);
    }
    mma(o1, aq[0], dd[0]);
    if (w >= 2) mma(o0, aq[1], dd[1]);
    load_q(rn1);
    float* tl = s_out + w * (16 * kOutLd);
#pragma unroll
    for (int i = 0; i < 4; ++i) tl[(4 * gq + i) * kOutLd + m] = o0[i] + o1[i];
    const int r = lane >> 2, q4 = 4 * (lane & 3);
    const f32x4 x = *reinterpret_cast<const f32x4*>(tl + r * kOutLd + q4);
    if (16 * w + r < len) store_out4(out, ((b * T + t0 + 16 * w + r) * H + h) * V + v0 + q4, x);
    // Is the record after the next one ready?  One lane looks; the answer
    // reaches every wave through the barrier.
    const bool look = n + 2 < n_chunks;
    if (threadIdx.x == 0) *s_word = (look && !is_ready(p.ready + rec_index(n + 2))) ? 1 : 0;
    block_sync();   // B2
    if (look && __builtin_amdgcn_readfirstlane(*s_word) != 0) {
      // Step out: the state entering chunk n + 1 to the workspace; the
      // workgroup produces records and resumes the lane at chunk n + 1.
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const int c0 = 16 * (w * NCB + c) + 4 * gq;
#pragma unroll
        for (int i = 0; i < 4; ++i) saved[(c0 + i) * kVT + m] = st[c][i];
      }
      __builtin_amdgcn_s_waitcnt(0);
      block_sync();
      return n + 1;
    }
  }

  if (p.fin) {
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int c0 = 16 * (w * NCB + c) + 4 * gq;
#pragma unroll
      for (int i = 0; i < 4; ++i) p.fin[((b * H + h) * K + c0 + i) * V + v0 + m] = st[c][i];
    }
  }
  return n_chunks;
}

// A workgroup of role 0 holds a recurrence lane (ticket t) and runs it from
// chunk n whenever records n and n + 1 are ready; when they are not, it
// produces an item of the queue instead, and waits for them only once the
// queue is empty.  Returns when no lane is left.
template <class TO, int K, int V>
__device__ __forceinline__ void run_lanes(const FusedParams& p, const XcdQueue& qu, char* smem_raw, int* s_task) {
  constexpr int NV = V / kVT;
  FusedCtl* ctl = p.ctl;
  const int xcd = qu.xcd;
  int64_t t = -1, n = 0;
  for (;;) {
    if (t < 0) {
      if (threadIdx.x == 0) *s_task = (int)atomicAdd(&ctl->lane_ticket[xcd], 1u);
      block_sync();
      t = __builtin_amdgcn_readfirstlane(*s_task);
      block_sync();
      n = 0;
      if (t >= qu.hx * NV) return;
    }
    const int64_t sh = xcd + p.n_xcd * (t / NV);
    const int64_t base = ((sh / p.ip.H) * p.nc + n) * p.ip.H + sh % p.ip.H;
    if (threadIdx.x == 0) {
      int v = -1;
      if (!is_ready(p.ready + base)) v = 0;
      else if (n + 1 < p.nc && !is_ready(p.ready + base + p.ip.H)) v = 1;
      *s_task = v;
    }
    block_sync();
    const int v = __builtin_amdgcn_readfirstlane(*s_task);
    block_sync();
    if (v < 0) {
      n = recur_lane<TO, K, V>(p, sh, (int)(t % NV), smem_raw, s_task, n);
      block_sync();
      if (n >= p.nc) t = -1;
      continue;
    }
    const int64_t need = base + v * p.ip.H;   // the record the lane waits for
    if (threadIdx.x == 0) *s_task = (int)qu.item(p, (int64_t)atomicAdd(&ctl->item_ticket[xcd], 1u));
    block_sync();
    const int64_t item = __builtin_amdgcn_readfirstlane(*s_task);
    block_sync();
    if (item >= 0) {
      ItemRows<K> in = load_item_rows<K>(p.ip, item), unused;
      produce<K, V>(p, item, smem_raw, in, NoNextItem{}, unused);
      block_sync();
      continue;
    }
    // Every item is claimed by a running workgroup, whose production
    // completes without waiting.
    wait_ready(p.ready + need, p.ip.hdr);
  }
}

// Production only, until the queue is empty.
template <int K, int V>
__device__ __forceinline__ void produce_all(const FusedParams& p, const XcdQueue& qu, char* smem_raw, int* s_task) {
  for (;;) {
    if (threadIdx.x == 0) *s_task = (int)qu.item(p, (int64_t)atomicAdd(&p.ctl->item_ticket[qu.xcd], 1u));
    block_sync();
    const int64_t item = __builtin_amdgcn_readfirstlane(*s_task);
    block_sync();
    if (item < 0) return;
    ItemRows<K> in = load_item_rows<K>(p.ip, item), unused;
    produce<K, V>(p, item, smem_raw, in, NoNextItem{}, unused);
    block_sync();
  }
}

template <class TO, int K, int V>
__global__ __launch_bounds__(256, 2) void kda_fused_kernel(FusedParams p) {
  extern __shared__ __align__(16) char smem_raw[];
  __shared__ int s_task;
  XcdQueue qu;
  qu.xcd = (int)(read_xcc_id() % (unsigned)p.n_xcd);
  // Sequence-heads of this XCD: xcd, xcd + n_xcd, ...
  qu.hx = p.n_sh > qu.xcd ? (p.n_sh - qu.xcd + p.n_xcd - 1) / p.n_xcd : 0;
  if (threadIdx.x == 0) s_task = (int)atomicAdd(&p.ctl->cu_arrivals[qu.xcd][read_cu_slot()], 1u);
  block_sync();
  const int role = __builtin_amdgcn_readfirstlane(s_task);   // uniform: read through LDS
  block_sync();
  if (role == 0) run_lanes<TO, K, V>(p, qu, smem_raw, &s_task);
  produce_all<K, V>(p, qu, smem_raw, &s_task);
}

// Zeroes the control block and the ready words (n words from ctl on) and the
// table header's flags (no tables without segment ids) before the fused
// kernel runs; a kernel rather than a memset, so that the call can be
// captured in a graph.
__global__ void kda_fused_reset_kernel(uint32_t* ctl, int64_t n, TableHeader* hdr) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) ctl[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) hdr->flags = 0u;
}

template <class TO, int K, int V>
hipError_t launch_fused_t(const CallArgs& a) {
  FusedParams p;
  p.ip = IntraParams{a.q, a.k, a.v, a.g, a.beta, a.gate_mode, a.lower_bound, a.a_log, a.dt_bias, a.B, a.T, a.H,
                     a.scale, a.l2norm, a.nc_fixed, 0, a.hdr, a.chunks, a.records, a.record_bytes};
  p.n_sh = a.B * a.H;
  p.nc = a.nc_fixed;
  p.n_xcd = a.n_xcd;
  p.init = a.init;
  p.fin = a.fin;
  p.o = a.o;
  p.ctl = a.fused_ctl;
  p.ready = a.fused_ready;
  p.lane_state = a.fused_lane_state;
  const int64_t n_words = (int64_t)(sizeof(FusedCtl) / 4) + a.B * a.nc_fixed * a.H;
  hipLaunchKernelGGL(kda_fused_reset_kernel, dim3((unsigned)std::min<int64_t>(1024, (n_words + 255) / 256)),
                     dim3(256), 0, a.stream, reinterpret_cast<uint32_t*>(a.fused_ctl), n_words, a.hdr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t smem = sizeof(Intra4Smem<K, V>);
  auto kern = kda_fused_kernel<TO, K, V>;
  static bool smem_set[64] = {false};   // per device
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64 || !smem_set[dev]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) smem_set[dev] = true;
  }
  hipLaunchKernelGGL(kern, dim3(2 * (unsigned)cu_count()), dim3(256), smem, a.stream, p);
  return hipGetLastError();
}

}  // namespace

bool fused_supported(const CallArgs& a) {
  // Record indices and queue tickets travel as 32-bit words.
  return a.in == InType::BF16 && a.n_max == 0 && a.gate_mode >= 0 && a.trans == nullptr && a.K == 128 &&
         a.V == 128 && a.n_xcd > 0 && cu_count() == 32 * a.n_xcd && a.fused_ctl != nullptr &&
         a.fused_lane_state != nullptr && a.B * a.nc_fixed * a.H < ((int64_t)1 << 30);
}

hipError_t launch_fused(const CallArgs& a) {
  if (a.out == OutType::F32) return launch_fused_t<float, 128, 128>(a);
  return launch_fused_t<uint16_t, 128, 128>(a);
}

}  // namespace kda
