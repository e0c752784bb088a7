// Inter-chunk recurrence and output of the KDA forward.
//
// One workgroup owns one sequence (a row, or a packed segment), one head and
// one 16-wide tile of value channels, and walks that sequence's chunks in
// order.  Columns of the state never mix (the delta rule contracts over the
// key axis only), so value tiles are independent recurrences.  Per chunk,
// with S the K x 16 state slice entering the chunk (fp32, in registers):
//   Delta = U - W S                            (wave w: tokens 16w..16w+15)
//   S    <- diag(exp(G_C)) S + Kt^T Delta      (wave w: its key-channel blocks)
//   O     = scale Qg S + scale Aqk Delta       (wave w: tokens 16w..16w+15)
// following the chunk form of the "Delta Rule formulation" on the page
// "feat(kda): integrate KDA attention with tokamax backend and CP support"
// (Implementation Details).  The S and Delta operands are exchanged between
// the four waves through LDS; all other operands come from the per-chunk
// records the intra-chunk kernel wrote.
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kVT = 16;   // value channels per workgroup

// An operand kept in LDS as rows n (value channel) of k-contiguous values.
template <class F> struct LdsPlane;

template <> struct LdsPlane<FragP> {   // hi and lo bf16 planes
  template <int ROWS, int PITCH>
  static constexpr int bytes() { return 2 * ROWS * PITCH * 2; }
  template <int ROWS, int PITCH>
  __device__ static void write4(char* base, int row, int col, const float x[4]) {
    __bf16* hi = reinterpret_cast<__bf16*>(base);
    __bf16* lo = hi + ROWS * PITCH;
    bf16x4 vh, vl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 h = to_bf16(x[i]);
      vh[i] = h;
      vl[i] = to_bf16(x[i] - from_bf16(h));
    }
    *reinterpret_cast<bf16x4*>(hi + row * PITCH + col) = vh;
    *reinterpret_cast<bf16x4*>(lo + row * PITCH + col) = vl;
  }
  template <int ROWS, int PITCH>
  __device__ static FragP read(const char* base, int row, int kb, int g) {
    const __bf16* hi = reinterpret_cast<const __bf16*>(base);
    const __bf16* lo = hi + ROWS * PITCH;
    const int o0 = row * PITCH + 32 * kb + 4 * g, o1 = o0 + 16;
    const bf16x4 h0 = *reinterpret_cast<const bf16x4*>(hi + o0), h1 = *reinterpret_cast<const bf16x4*>(hi + o1);
    const bf16x4 l0 = *reinterpret_cast<const bf16x4*>(lo + o0), l1 = *reinterpret_cast<const bf16x4*>(lo + o1);
    FragP f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.hi[i] = h0[i]; f.hi[4 + i] = h1[i];
      f.lo[i] = l0[i]; f.lo[4 + i] = l1[i];
    }
    return f;
  }
};

template <> struct LdsPlane<FragF> {   // one fp32 plane
  template <int ROWS, int PITCH>
  static constexpr int bytes() { return ROWS * PITCH * 4; }
  template <int ROWS, int PITCH>
  __device__ static void write4(char* base, int row, int col, const float x[4]) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + row * PITCH + col) = f32x4{x[0], x[1], x[2], x[3]};
  }
  template <int ROWS, int PITCH>
  __device__ static FragF read(const char* base, int row, int kb, int g) {
    const float* p = reinterpret_cast<const float*>(base);
    const int o0 = row * PITCH + 32 * kb + 4 * g;
    FragF f;
    f.a = *reinterpret_cast<const f32x4*>(p + o0);
    f.b = *reinterpret_cast<const f32x4*>(p + o0 + 16);
    return f;
  }
};

__device__ __forceinline__ void store_out(float* o, int64_t i, float x) { o[i] = x; }
__device__ __forceinline__ void store_out(uint16_t* o, int64_t i, float x) {
  const __bf16 h = to_bf16(x);
  o[i] = *reinterpret_cast<const uint16_t*>(&h);
}

// Every operand one wave reads from a chunk record, held in registers so
// that the next chunk's loads are in flight while this chunk computes.
template <class TI, int K, int V>
struct ChunkOps {
  using P = Prec<TI>;
  static constexpr int NCB = K / 16 / 4;
  f32x4 u;
  typename P::W wn[K / 32];
  typename P::Kt kt[NCB][2];
  typename P::Q qg[K / 32];
  typename P::Q aqk[2];
  f32x4 gc[NCB];
  __device__ __forceinline__ void load(const char* rec, int w, int j, int lane, int gq) {
    using L = RecordLayout<TI, K, V>;
    u = reinterpret_cast<const f32x4*>(rec + L::kU)[(w * (V / 16) + j) * kWave + lane];
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
      wn[kb].load(rec + L::kWn + (int64_t)(w * (K / 32) + kb) * tile_bytes<typename P::W>(), lane);
      qg[kb].load(rec + L::kQg + (int64_t)(w * (K / 32) + kb) * tile_bytes<typename P::Q>(), lane);
    }
#pragma unroll
    for (int u_ = 0; u_ < NCB; ++u_) {
      const int cb = w * NCB + u_;
      gc[u_] = *reinterpret_cast<const f32x4*>(rec + L::kGc + 4 * (16 * cb + 4 * gq));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        kt[u_][kb].load(rec + L::kKt + (int64_t)(cb * 2 + kb) * tile_bytes<typename P::Kt>(), lane);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      if (kb <= w / 2) aqk[kb].load(rec + L::kAqk + (int64_t)(w * 2 + kb) * tile_bytes<typename P::Q>(), lane);
  }
};

struct RecurParams {
  int64_t B, T, H;
  int64_t nc_fixed;
  int packed, n_max;
  int64_t n_seq_heads_fixed;   // B * H when not packed
  const TableHeader* hdr;
  const SegEntry* segs;
  const ChunkEntry* chunks;
  const char* records;
  int64_t record_bytes;
  const float* init;
  float* fin;
  void* o;
};

template <class TI, class TO, int K, int V>
__global__ __launch_bounds__(kThreads) void kda_recur_kernel(RecurParams p) {
  using PS = typename Prec<TI>::S;
  using PD = typename Prec<TI>::D;
  constexpr int NV = V / kVT;
  constexpr int SP = K + 8;        // LDS row pitch of the state operand
  constexpr int DP = kChunk + 8;   // LDS row pitch of the Delta operand
  constexpr int S_BYTES = LdsPlane<PS>::template bytes<kVT, SP>();
  constexpr int NCB = K / 16 / 4;  // key-channel blocks of the state per wave
  __shared__ __align__(16) char s_state[2][S_BYTES];
  __shared__ __align__(16) char s_delta[LdsPlane<PD>::template bytes<kVT, DP>()];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = lane & 15, gq = lane >> 4;
  const int64_t H = p.H;

  // XCD-aware decode: the NV value tiles of one (sequence, head) sit on
  // workgroup ids with equal id % 8, which the dispatcher places on one XCD,
  // so they share that XCD's L2 copy of the chunk records.
  const int64_t id = blockIdx.x;
  const int64_t seq_head = (id / (8 * NV)) * 8 + id % 8;
  const int j = (int)((id / 8) % NV);
  const int64_t n_seq_heads = p.packed ? (int64_t)p.hdr->n_segments * H : p.n_seq_heads_fixed;
  if (seq_head >= n_seq_heads) return;
  const int64_t h = seq_head % H, sq = seq_head / H;

  int64_t b, slot, n_chunks, chunk0 = 0;
  if (p.packed) {
    const SegEntry se = p.segs[sq];
    b = se.b;
    slot = ((int64_t)se.b * p.n_max + se.local) * H + h;
    n_chunks = se.n_chunks;
    chunk0 = se.chunk_begin;
  } else {
    b = sq;
    slot = b * H + h;
    n_chunks = p.nc_fixed;
  }
  TO* out = static_cast<TO*>(p.o);
  const int v0 = kVT * j;

  // State slice: wave w holds key-channel blocks cb = w*NCB .. +NCB-1, lane
  // (column v0 + m, rows 16cb + 4gq + i).
  f32x4 st[NCB];
#pragma unroll
  for (int u = 0; u < NCB; ++u) {
    const int c0 = 16 * (w * NCB + u) + 4 * gq;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st[u][i] = p.init ? p.init[(slot * K + c0 + i) * V + v0 + m] : 0.f;
    float x[4] = {st[u][0], st[u][1], st[u][2], st[u][3]};
    LdsPlane<PS>::template write4<kVT, SP>(s_state[0], m, c0, x);
  }
  __syncthreads();

  // Chunk n's record index, first token and length.
  auto chunk_info = [&](int64_t n, int64_t& rec_idx, int64_t& t0, int& len) {
    if (p.packed) {
      const ChunkEntry ce = p.chunks[chunk0 + n];
      rec_idx = (chunk0 + n) * H + h;
      t0 = ce.t0;
      len = ce.len;
    } else {
      rec_idx = (b * p.nc_fixed + n) * H + h;
      t0 = n * kChunk;
      len = (int)min<int64_t>(kChunk, p.T - t0);
    }
  };

  // The operands of chunk n + 1 (clamped to the last chunk) are loaded while
  // chunk n computes; `cur` is loop-carried, so those loads cannot sink.
  ChunkOps<TI, K, V> cur;
  int64_t t0 = 0, t0n = 0;
  int len = 0, lenn = 0;
  int buf = 0;
  if (n_chunks > 0) {
    int64_t rec_idx;
    chunk_info(0, rec_idx, t0, len);
    cur.load(p.records + rec_idx * p.record_bytes, w, j, lane, gq);
  }
  for (int64_t n = 0; n < n_chunks; ++n) {
    ChunkOps<TI, K, V> nxt;
    {
      int64_t rec_idx;
      chunk_info(n + 1 < n_chunks ? n + 1 : n, rec_idx, t0n, lenn);
      nxt.load(p.records + rec_idx * p.record_bytes, w, j, lane, gq);
    }

    // Delta = U - W S for tokens 16w..16w+15
    f32x4 d = cur.u;
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
      const PS s = LdsPlane<PS>::template read<kVT, SP>(s_state[buf], m, kb, gq);
      mma(d, cur.wn[kb], s);
    }
    {
      float x[4] = {d[0], d[1], d[2], d[3]};
      LdsPlane<PD>::template write4<kVT, DP>(s_delta, m, 16 * w + 4 * gq, x);
    }
    __syncthreads();

    // S <- diag(exp(G_C)) S + Kt^T Delta
#pragma unroll
    for (int u = 0; u < NCB; ++u) {
      const int cb = w * NCB + u, c0 = 16 * cb + 4 * gq;
#pragma unroll
      for (int i = 0; i < 4; ++i) st[u][i] *= cur.gc[u][i];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const PD dd = LdsPlane<PD>::template read<kVT, DP>(s_delta, m, kb, gq);
        mma(st[u], cur.kt[u][kb], dd);
      }
      float x[4] = {st[u][0], st[u][1], st[u][2], st[u][3]};
      LdsPlane<PS>::template write4<kVT, SP>(s_state[buf ^ 1], m, c0, x);
    }

    // O = scale Qg S + scale Aqk Delta for tokens 16w..16w+15
    f32x4 ov = {0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
      const PS s = LdsPlane<PS>::template read<kVT, SP>(s_state[buf], m, kb, gq);
      mma(ov, cur.qg[kb], s);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb > w / 2) continue;
      const PD dd = LdsPlane<PD>::template read<kVT, DP>(s_delta, m, kb, gq);
      mma(ov, cur.aqk[kb], dd);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * gq + i;
      if (r < len) store_out(out, ((b * p.T + t0 + r) * H + h) * V + v0 + m, ov[i]);
    }
    __syncthreads();
    buf ^= 1;
    cur = nxt;
    t0 = t0n;
    len = lenn;
  }

  if (p.fin) {
#pragma unroll
    for (int u = 0; u < NCB; ++u) {
      const int c0 = 16 * (w * NCB + u) + 4 * gq;
#pragma unroll
      for (int i = 0; i < 4; ++i) p.fin[(slot * K + c0 + i) * V + v0 + m] = st[u][i];
    }
  }
}

template <class TI, class TO, int K, int V>
hipError_t launch_recur_t(const CallArgs& a) {
  constexpr int NV = V / kVT;
  RecurParams p{a.B, a.T, a.H, a.nc_fixed, a.n_max > 0, a.n_max, a.B * a.H, a.hdr, a.segs, a.chunks,
                a.records, a.record_bytes, a.init, a.fin, a.o};
  const int64_t seq_heads = (a.n_max > 0 ? a.smax : a.B) * a.H;
  if (seq_heads <= 0) return hipSuccess;
  const int64_t groups = (seq_heads + 7) / 8;
  const int64_t grid = groups * 8 * NV;
  hipLaunchKernelGGL((kda_recur_kernel<TI, TO, K, V>), dim3((unsigned)grid), dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

template <class TI, class TO>
hipError_t launch_recur_kv(const CallArgs& a) {
  if (a.K == 64 && a.V == 64) return launch_recur_t<TI, TO, 64, 64>(a);
  if (a.K == 64 && a.V == 128) return launch_recur_t<TI, TO, 64, 128>(a);
  if (a.K == 128 && a.V == 64) return launch_recur_t<TI, TO, 128, 64>(a);
  if (a.K == 128 && a.V == 128) return launch_recur_t<TI, TO, 128, 128>(a);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_recur(const CallArgs& a) {
  if (a.in == InType::BF16)
    return a.out == OutType::F32 ? launch_recur_kv<uint16_t, float>(a) : launch_recur_kv<uint16_t, uint16_t>(a);
  return a.out == OutType::F32 ? launch_recur_kv<float, float>(a) : launch_recur_kv<float, uint16_t>(a);
}

}  // namespace kda
