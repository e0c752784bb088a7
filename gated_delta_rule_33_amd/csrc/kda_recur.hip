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
// the four compute waves through LDS; all other operands come from the
// per-chunk records the intra-chunk kernel wrote, staged into LDS by
// producer waves.
//
// Wave roles.  A wave that issues direct-to-LDS loads moves about 10 bytes
// per clock: the rate is per issuing wave (per SIMD), so a compute wave that
// loads its own operands spends most of a step stalled on issue.  Here a
// workgroup carries TPW value tiles of one (sequence, head): compute waves
// 4t .. 4t+3 run tile t, producer wave 4 TPW + i fills stage i (the record
// operands of token block / key-channel group i, shared by the tiles; only U
// differs per tile) and the last wave pulls records a few chunks ahead into
// L2.  Waves are spread round-robin over the SIMDs, so SIMD i hosts compute
// wave i of every tile and producer i.  Two tiles per workgroup halve the
// staged bytes per tile and let the two compute groups hide each other's
// latencies; that pays when there are many (sequence, head) pairs, while one
// tile per workgroup spreads few of them over all CUs.  Three barriers per chunk:
//   B1 after the Delta phase, B15 after the state update, B2 after the
//   output phase.
// A stage group is refilled as soon as the barrier after its last reader
// has passed, and the producer waits for it before the barrier that opens
// its next reader: Wn/U (read before B1) refill after B1 and land by B2;
// Kt/Gc (read between B1 and B15) refill after B15 and land by the next B1;
// Qg/Aqk (read between B15 and B2) refill after B2 and land by the next B15.
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kVT = 16;   // value channels per workgroup
constexpr int kComputeWaves = 4;   // per value tile
template <int TPW>
struct Roles {
  static constexpr int kProducer0 = kComputeWaves * TPW;   // producer of stage i: kProducer0 + i
  static constexpr int kPrefetchWave = kProducer0 + kComputeWaves;
  static constexpr int kThreads = (kPrefetchWave + 1) * kWave;
};
constexpr int kPrefetchAhead = 0;   // extra chunks between the L2 prefetch and the use of a record

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

// Output stores are non-temporal: o is not read again by this forward, and
// streaming it past the caches leaves them to the chunk records.
__device__ __forceinline__ void store_out(float* o, int64_t i, float x) { __builtin_nontemporal_store(x, o + i); }
__device__ __forceinline__ void store_out(uint16_t* o, int64_t i, float x) {
  const __bf16 h = to_bf16(x);
  __builtin_nontemporal_store(*reinterpret_cast<const uint16_t*>(&h), o + i);
}
// Four consecutive outputs o[i .. i + 3] (i a multiple of 4).
__device__ __forceinline__ void store_out4(float* o, int64_t i, const f32x4& x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(o + i));
}
__device__ __forceinline__ void store_out4(uint16_t* o, int64_t i, const f32x4& x) {
  uint32_t w[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const __bf16 a = to_bf16(x[2 * j]), b = to_bf16(x[2 * j + 1]);
    w[j] = (uint32_t)*reinterpret_cast<const uint16_t*>(&a) | ((uint32_t)*reinterpret_cast<const uint16_t*>(&b) << 16);
  }
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2*>(o + i));
}
// The output tile of a wave (lane (g, n) holding token rows 4g + i, column n)
// goes through a padded LDS tile of its own, so each lane stores four
// consecutive columns of one row; row stride 20 keeps both sides free of
// bank conflicts.
constexpr int kOutLd = 20;

// The record operands compute wave w uses in one chunk, staged in its own LDS
// block by its producer wave with direct-to-LDS loads.
//   Wn  : -W rows 16w..16w+15, all K          (K/32 tiles)
//   U   : U rows 16w..16w+15, per value tile   (TPW x 1 KB)
//   Kt  : key-channel blocks cb = w*NCB+u      (NCB x 2 tiles)
//   Qg  : Qg rows 16w..16w+15, all K          (K/32 tiles)
//   Aqk : Aqk row block w, token blocks <= w/2 (1 or 2 tiles)
//   Gc  : exp(G_C) for this wave's key-channel blocks (16 NCB floats)
template <class TI, int K, int V, int TPW>
struct Stage {
  using P = Prec<TI>;
  using L = RecordLayout<TI, K, V>;
  static constexpr int NCB = K / 64;
  static constexpr int kWnBytes = (K / 32) * tile_bytes<typename P::W>();
  static constexpr int kKtBytes = NCB * 2 * tile_bytes<typename P::Kt>();
  static constexpr int kQgBytes = (K / 32) * tile_bytes<typename P::Qg>();
  static constexpr int kAqkTile = tile_bytes<typename P::Aq>();
  static constexpr int oWn = 0;
  static constexpr int oU = oWn + kWnBytes;
  static constexpr int oKt = oU + TPW * 1024;
  static constexpr int oQg = oKt + kKtBytes;
  static constexpr int oAqk = oQg + kQgBytes;
  static constexpr int oGc = oAqk + 2 * kAqkTile;
  static constexpr int kBytes = oGc + 64 * NCB;
  // Load instructions (1 KB each) per group.
  static constexpr int nW = kWnBytes / 1024 + TPW;   // Wn and U
  static constexpr int nKt = kKtBytes / 1024 + 1;   // Kt and Gc
  static constexpr int nQ1 = (kQgBytes + kAqkTile) / 1024;       // Qg and Aqk, waves 0 and 1
  static constexpr int nQ2 = (kQgBytes + 2 * kAqkTile) / 1024;   // waves 2 and 3

  __device__ static void issue_w(char* stg, const char* rec, int w, int j0, int lane) {
    dma_copy<kWnBytes>(stg + oWn, rec + L::kWn + (int64_t)w * kWnBytes, lane);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      dma_copy<1024>(stg + oU + 1024 * t, rec + L::kU + (int64_t)(w * (V / 16) + j0 + t) * 1024, lane);
  }
  __device__ static void issue_kt(char* stg, const char* rec, int w, int lane) {
    dma_copy<kKtBytes>(stg + oKt, rec + L::kKt + (int64_t)w * kKtBytes, lane);
    if (lane < 4 * NCB) dma16(stg + oGc, rec + L::kGc + 64 * (w * NCB) + 16 * lane);
  }
  __device__ static void issue_q(char* stg, const char* rec, int w, int lane) {
    dma_copy<kQgBytes>(stg + oQg, rec + L::kQg + (int64_t)w * kQgBytes, lane);
    const char* a = rec + L::kAqk + (int64_t)(2 * w) * kAqkTile;
    if (w >= 2)
      dma_copy<2 * kAqkTile>(stg + oAqk, a, lane);
    else
      dma_copy<kAqkTile>(stg + oAqk, a, lane);
  }
};

struct RecurParams {
  int64_t B, T, H;
  int64_t nc_fixed;
  int packed, n_max;
  int64_t n_seq_heads_fixed;   // B * H when not packed
  const TableHeader* hdr;
  const SegEntry* segs;
  const char* records;
  int64_t record_bytes;
  const float* init;
  float* fin;
  void* o;
  float* trans;   // [B,H,K,K] transition of each row's carried state, or NULL
};

template <class TI, class TO, int K, int V, int TPW>
__global__ __launch_bounds__(Roles<TPW>::kThreads) void kda_recur_kernel(RecurParams p) {
  using P = Prec<TI>;
  using PS = typename P::S;
  using PD = typename P::D;
  using SG = Stage<TI, K, V, TPW>;
  constexpr int kProducer0 = Roles<TPW>::kProducer0;
  constexpr int kPrefetchWave = Roles<TPW>::kPrefetchWave;
  constexpr int NV = V / kVT;
  constexpr int NVW = NV / TPW;     // workgroups per (sequence, head)
  constexpr int SP = K + 8;        // LDS row pitch of the state operand
  constexpr int DP = kChunk + 8;   // LDS row pitch of the Delta operand
  constexpr int NCB = SG::NCB;     // key-channel blocks of the state per wave
  __shared__ __align__(16) char s_stage[kComputeWaves][SG::kBytes];
  __shared__ __align__(16) char s_state_t[TPW][LdsPlane<PS>::template bytes<kVT, SP>()];
  __shared__ __align__(16) char s_delta_t[TPW][LdsPlane<PD>::template bytes<kVT, DP>()];
  __shared__ __align__(16) char s_sink[1024];   // discarded data of the L2 prefetches

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, gq = lane >> 4;
  const int64_t H = p.H;

  // XCD-aware decode: the NVW workgroups of one (sequence, head) sit on
  // workgroup ids with equal id % 8, which the dispatcher places on one XCD,
  // so they share that XCD's L2 copy of the chunk records.  Workgroup jw
  // carries value tiles j0 = TPW jw .. j0 + TPW - 1.
  const int64_t id = blockIdx.x;
  const int64_t seq_head = (id / (8 * NVW)) * 8 + id % 8;
  const int jw = (int)((id / 8) % NVW), j0 = TPW * jw;
  const int64_t n_seq_heads = p.packed ? (int64_t)p.hdr->n_segments * H : p.n_seq_heads_fixed;
  if (seq_head >= n_seq_heads) return;
  const int64_t h = seq_head % H, sq = seq_head / H;

  // Chunk n of a sequence starts at token t_begin + 64 n; its record is
  // (first_chunk + n) * H + h.
  int64_t b, slot, n_chunks, first_chunk, t_begin, seq_len;
  if (p.packed) {
    const SegEntry se = p.segs[sq];
    b = se.b;
    slot = ((int64_t)se.b * p.n_max + se.local) * H + h;
    n_chunks = se.n_chunks;
    first_chunk = se.chunk_begin;
    t_begin = se.t0;
    seq_len = se.len;
  } else {
    b = sq;
    slot = b * H + h;
    n_chunks = p.nc_fixed;
    first_chunk = b * p.nc_fixed;
    t_begin = 0;
    seq_len = p.T;
  }
  auto record = [&](int64_t n) { return p.records + ((first_chunk + n) * H + h) * p.record_bytes; };

  // ---- L2 prefetch wave: walks kPrefetchAhead chunks ahead and touches this
  // workgroup's 1/NVW share of each record (every 64-byte segment once), so
  // the record is in this XCD's L2 when the producers of all NVW workgroups
  // stage it.
  if (wave == kPrefetchWave) {
    using L = RecordLayout<TI, K, V>;
    constexpr int SEGS = (int)(L::kBytes / 64);
    constexpr int SHARE = (SEGS + NVW - 1) / NVW;
    auto prefetch = [&](int64_t n) {
      const char* r = record(n);
#pragma unroll
      for (int i = 0; i < (SHARE + kWave - 1) / kWave; ++i) {
        const int e = i * kWave + lane, seg = jw * SHARE + e;
        if (e < SHARE && seg < SEGS) dma16(s_sink, r + 64 * (int64_t)seg);
      }
    };
    for (int64_t n = 1; n <= kPrefetchAhead && n < n_chunks; ++n) prefetch(n);
    block_sync();
    for (int64_t n = 0; n < n_chunks; ++n) {
      if (n + kPrefetchAhead + 1 < n_chunks) prefetch(n + kPrefetchAhead + 1);
      block_sync();
      block_sync();
      block_sync();
    }
    vm_wait<0>();
    return;
  }

  // ---- producer waves.  Waits: direct-to-LDS loads of one wave complete in
  // issue order, so a group has landed once no more than the number of loads
  // issued after it are outstanding.
  if (wave >= kProducer0) {
    const int w = wave - kProducer0;
    char* stg = s_stage[w];
    const bool two_aqk = w >= 2;
    if (n_chunks > 0) {
      const char* r0 = record(0);
      SG::issue_w(stg, r0, w, j0, lane);
      SG::issue_kt(stg, r0, w, lane);
      SG::issue_q(stg, r0, w, lane);
      vm_wait<0>();
    }
    block_sync();
    for (int64_t n = 0; n < n_chunks; ++n) {
      const bool more = n + 1 < n_chunks;
      const char* rn = record(n);
      const char* rn1 = more ? record(n + 1) : rn;
      // Delta phase reads Wn/U(n).  Qg/Aqk(n) go out; Kt/Gc(n) must land.
      if (n > 0) {
        SG::issue_q(stg, rn, w, lane);
        if (two_aqk) vm_wait<SG::nQ2>(); else vm_wait<SG::nQ1>();
      }
      block_sync();   // B1
      // State update reads Kt/Gc(n).  Wn/U(n+1) go out; Qg/Aqk(n) must land.
      if (more) {
        SG::issue_w(stg, rn1, w, j0, lane);
        vm_wait<SG::nW>();
      } else {
        vm_wait<0>();
      }
      block_sync();   // B15
      // Output phase reads Qg/Aqk(n).  Kt/Gc(n+1) go out; Wn/U(n+1) must land.
      if (more) {
        SG::issue_kt(stg, rn1, w, lane);
        vm_wait<SG::nKt>();
      }
      block_sync();   // B2
    }
    vm_wait<0>();
    return;
  }

  // ---- compute waves of tile tl
  const int tl = wave / kComputeWaves, w = wave % kComputeWaves;
  const char* stg = s_stage[w];
  TO* out = static_cast<TO*>(p.o);
  const int v0 = kVT * (j0 + tl);
  char* s_state = s_state_t[tl];
  char* s_delta = s_delta_t[tl];

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
    LdsPlane<PS>::template write4<kVT, SP>(s_state, m, c0, x);
  }
  block_sync();

  for (int64_t n = 0; n < n_chunks; ++n) {
    const int64_t t0 = t_begin + n * kChunk;
    const int len = (int)min<int64_t>(kChunk, seq_len - n * kChunk);

    // Delta = U - W S for tokens 16w..16w+15; the S operand stays in
    // registers for the output phase.
    PS sf[K / 32];
    typename P::W wn[K / 32];
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) {
      wn[kb].load(stg + SG::oWn + kb * tile_bytes<typename P::W>(), lane);
      sf[kb] = LdsPlane<PS>::template read<kVT, SP>(s_state, m, kb, gq);
    }
    f32x4 d = reinterpret_cast<const f32x4*>(stg + SG::oU + 1024 * tl)[lane];
#pragma unroll
    for (int kb = 0; kb < K / 32; ++kb) mma(d, wn[kb], sf[kb]);
    {
      float x[4] = {d[0], d[1], d[2], d[3]};
      LdsPlane<PD>::template write4<kVT, DP>(s_delta, m, 16 * w + 4 * gq, x);
    }
    block_sync();   // B1

    // S <- diag(exp(G_C)) S + Kt^T Delta (with one tile per workgroup the
    // Delta operand stays in registers for the output phase)
    PD dd[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) dd[kb] = LdsPlane<PD>::template read<kVT, DP>(s_delta, m, kb, gq);
#pragma unroll
    for (int u = 0; u < NCB; ++u) {
      const int cb = w * NCB + u, c0 = 16 * cb + 4 * gq;
      const f32x4 gc = reinterpret_cast<const f32x4*>(stg + SG::oGc)[4 * u + gq];
      typename P::Kt kt[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kt[kb].load(stg + SG::oKt + (u * 2 + kb) * tile_bytes<typename P::Kt>(), lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) st[u][i] *= gc[i];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma(st[u], kt[kb], dd[kb]);
      float x[4] = {st[u][0], st[u][1], st[u][2], st[u][3]};
      LdsPlane<PS>::template write4<kVT, SP>(s_state, m, c0, x);
    }
    block_sync();   // B15

    // O = scale Qg S + scale Aqk Delta for tokens 16w..16w+15
    f32x4 ov = {0, 0, 0, 0};
    if constexpr (TPW == 1) {
      typename P::Qg qg[K / 32];
      typename P::Aq aq[2];
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) qg[kb].load(stg + SG::oQg + kb * tile_bytes<typename P::Qg>(), lane);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb <= w / 2) aq[kb].load(stg + SG::oAqk + kb * SG::kAqkTile, lane);
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) mma(ov, qg[kb], sf[kb]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb <= w / 2) mma(ov, aq[kb], dd[kb]);
    } else {
      // Four waves per SIMD leave 128 registers: operands are loaded as they
      // are used and Delta is re-read (it stays in LDS until the next chunk's
      // Delta phase).
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) {
        typename P::Qg qg;
        qg.load(stg + SG::oQg + kb * tile_bytes<typename P::Qg>(), lane);
        mma(ov, qg, sf[kb]);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb > w / 2) continue;
        typename P::Aq aq;
        aq.load(stg + SG::oAqk + kb * SG::kAqkTile, lane);
        const PD d2 = LdsPlane<PD>::template read<kVT, DP>(s_delta, m, kb, gq);
        mma(ov, aq, d2);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * gq + i;
      if (r < len) store_out(out, ((b * p.T + t0 + r) * H + h) * V + v0 + m, ov[i]);
    }
    block_sync();   // B2
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

// One value tile per workgroup, operands straight to registers.  Each
// compute wave's share of a record (its token block of Wn, U, Qg and Aqk,
// its key-channel blocks of Kt and exp(G_C)) is read by that wave alone, so
// it is loaded into the wave's registers one chunk ahead, each group right
// after its last use; only S and Delta pass through LDS.  Two barriers per
// chunk: B1 after the Delta phase (Delta visible), B2 at the end (the new
// state visible, the Delta buffer free).  The fifth wave pulls the next
// chunk's record into L2 (further ahead, the lines wait in L2 longer and
// more of them are evicted before use).
//
// With kTrans the same loop carries, instead of the state, the transition of
// a row's first segment: the recurrence is affine in the state a segment
// starts from, S_end = M S_start + (S_end for S_start = 0), and M is the
// chunk product of diag(exp(G_C)) - Kt^T W, i.e. the loop above with U = 0
// and S_start = I, with no read-out.  Its columns (K of them, one 16-wide
// tile per workgroup) index the key channels of S_start.  It exists only
// where one segment runs from the row's first token to its last (every row
// without segment ids); the caller zero-fills the others.  This is the
// transfer matrix a context-parallel rank passes on with its end state.
template <class TI, class TO, int K, int V, bool kTrans>
__global__ __launch_bounds__((kComputeWaves + 1) * kWave) void kda_recur_reg_kernel(RecurParams p) {
  using P = Prec<TI>;
  using PS = typename P::S;
  using PD = typename P::D;
  using PW = typename P::W;
  using PK = typename P::Kt;
  using PQ = typename P::Qg;
  using PA = typename P::Aq;
  using L = RecordLayout<TI, K, V>;
  constexpr int kPrefetchWave = kComputeWaves;
  constexpr int NCOL = kTrans ? K : V;   // columns of the carried matrix
  constexpr int NV = NCOL / kVT;   // workgroups per (sequence, head)
  constexpr int NCB = K / 64;      // key-channel blocks of the state per wave
  constexpr int KB = K / 32;       // 32-deep key slabs
  // S and Delta as operand tiles in fragment order (k = key channel / token):
  // the accumulator rows a wave holds are one half of the same lane's
  // fragment, and each lane reads its fragment as whole 16-byte words.
  constexpr int TS = tile_bytes<PS>(), TD = tile_bytes<PD>();
  __shared__ __align__(16) char s_state[KB * TS];
  __shared__ __align__(16) char s_delta[2 * TD];
  __shared__ __align__(16) char s_sink[1024];   // discarded data of the L2 prefetches
  __shared__ __align__(16) float s_out[kComputeWaves][kChunk / kComputeWaves * kOutLd];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, gq = lane >> 4;
  const int64_t H = p.H;

  // XCD-aware decode: the NV workgroups of one (sequence, head) sit on
  // workgroup ids with equal id % 8, which the dispatcher places on one XCD,
  // so they share that XCD's L2 copy of the chunk records.
  const int64_t id = blockIdx.x;
  const int64_t seq_head = (id / (8 * NV)) * 8 + id % 8;
  const int j = (int)((id / 8) % NV);
  const int64_t n_seq_heads = p.packed ? (int64_t)p.hdr->n_segments * H : p.n_seq_heads_fixed;
  if (seq_head >= n_seq_heads) return;
  const int64_t h = seq_head % H, sq = seq_head / H;

  int64_t b, slot, n_chunks, first_chunk, t_begin, seq_len;
  if (p.packed) {
    const SegEntry se = p.segs[sq];
    if (kTrans && (se.t0 != 0 || se.len != p.T)) return;   // no segment spans this row
    b = se.b;
    slot = ((int64_t)se.b * p.n_max + se.local) * H + h;
    n_chunks = se.n_chunks;
    first_chunk = se.chunk_begin;
    t_begin = se.t0;
    seq_len = se.len;
  } else {
    b = sq;
    slot = b * H + h;
    n_chunks = p.nc_fixed;
    first_chunk = b * p.nc_fixed;
    t_begin = 0;
    seq_len = p.T;
  }
  auto record = [&](int64_t n) { return p.records + ((first_chunk + n) * H + h) * p.record_bytes; };

  // ---- L2 prefetch wave: touches this workgroup's 1/NV share of the record
  // kPrefetchAhead chunks ahead (every 64-byte segment once).
  if (wave == kPrefetchWave) {
    constexpr int SEGS = (int)((kTrans ? L::kQg : L::kBytes) / 64);   // the transition reads Wn and Kt only
    constexpr int SHARE = (SEGS + NV - 1) / NV;
    auto prefetch = [&](int64_t n) {
      const char* r = record(n);
#pragma unroll
      for (int i = 0; i < (SHARE + kWave - 1) / kWave; ++i) {
        const int e = i * kWave + lane, seg = j * SHARE + e;
        if (e < SHARE && seg < SEGS) dma16(s_sink, r + 64 * (int64_t)seg);
      }
    };
    for (int64_t n = 1; n <= kPrefetchAhead && n < n_chunks; ++n) prefetch(n);
    block_sync();
    for (int64_t n = 0; n < n_chunks; ++n) {
      if (n + kPrefetchAhead + 1 < n_chunks) prefetch(n + kPrefetchAhead + 1);
      block_sync();   // B1
      block_sync();   // B2
    }
    vm_wait<0>();
    return;
  }

  // ---- compute wave w: token block w, key-channel blocks w*NCB .. +NCB-1
  const int w = wave;
  TO* out = static_cast<TO*>(p.o);
  const int v0 = kVT * j;
  PW wn[KB];
  f32x4 u;
  PK kt[NCB][2];
  f32x4 gc[NCB];
  PQ qg[KB];
  PA aq[2];
  auto load_w = [&](const char* r) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) wn[kb].load(r + L::kWn + (int64_t)(w * KB + kb) * tile_bytes<PW>(), lane);
    if constexpr (kTrans) u = f32x4{0, 0, 0, 0};
    else u = reinterpret_cast<const f32x4*>(r + L::kU + (int64_t)(w * (V / 16) + j) * 1024)[lane];
  };
  auto load_kt = [&](const char* r) {
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kt[c][kb].load(r + L::kKt + (int64_t)((w * NCB + c) * 2 + kb) * tile_bytes<PK>(), lane);
      gc[c] = reinterpret_cast<const f32x4*>(r + L::kGc)[4 * (w * NCB + c) + gq];
    }
  };
  auto load_q = [&](const char* r) {
    if constexpr (kTrans) return;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qg[kb].load(r + L::kQg + (int64_t)(w * KB + kb) * tile_bytes<PQ>(), lane);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      if (kb <= w / 2) aq[kb].load(r + L::kAqk + (int64_t)(2 * w + kb) * tile_bytes<PA>(), lane);
  };

  // State slice: lane (column v0 + m, rows 16cb + 4gq + i) of its blocks.
  f32x4 st[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const int c0 = 16 * (w * NCB + c) + 4 * gq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kTrans) st[c][i] = (c0 + i == v0 + m) ? 1.f : 0.f;
      else st[c][i] = p.init ? p.init[(slot * K + c0 + i) * V + v0 + m] : 0.f;
    }
    float x[4] = {st[c][0], st[c][1], st[c][2], st[c][3]};
    const int cb = w * NCB + c;
    PS::store_half(s_state + (cb / 2) * TS, lane, cb & 1, x);
  }
  if (n_chunks > 0) {
    const char* r0 = record(0);
    load_w(r0);
    load_kt(r0);
    load_q(r0);
  }
  block_sync();

  for (int64_t n = 0; n < n_chunks; ++n) {
    const int64_t t0 = t_begin + n * kChunk;
    const int len = (int)min<int64_t>(kChunk, seq_len - n * kChunk);
    const char* rn1 = record(n + 1 < n_chunks ? n + 1 : n);

    // Delta = U - W S for tokens 16w..16w+15; the S operand stays in
    // registers for the output phase.  Two accumulators halve the
    // dependent chain.
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
      PD::store_half(s_delta + (w / 2) * TD, lane, w & 1, x);
    }
    load_w(rn1);
    block_sync();   // B1

    // S <- diag(exp(G_C)) S + Kt^T Delta
    PD dd[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) dd[kb].load(s_delta + kb * TD, lane);
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      f32x4 a0, a1 = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) a0[i] = st[c][i] * gc[c][i];
      mma(a0, kt[c][0], dd[0]);
      mma(a1, kt[c][1], dd[1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) st[c][i] = a0[i] + a1[i];
      float x[4] = {st[c][0], st[c][1], st[c][2], st[c][3]};
      const int cb = w * NCB + c;
      PS::store_half(s_state + (cb / 2) * TS, lane, cb & 1, x);
    }
    load_kt(rn1);

    if constexpr (!kTrans) {
      // O = scale Qg S + scale Aqk Delta for tokens 16w..16w+15
      f32x4 o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < KB; kb += 2) {
        mma(o0, qg[kb], sf[kb]);
        if (kb + 1 < KB) mma(o1, qg[kb + 1], sf[kb + 1]);
      }
      mma(o1, aq[0], dd[0]);
      if (w >= 2) mma(o0, aq[1], dd[1]);
      load_q(rn1);
      float* tl = s_out[w];
#pragma unroll
      for (int i = 0; i < 4; ++i) tl[(4 * gq + i) * kOutLd + m] = o0[i] + o1[i];
      const int r = lane >> 2, q4 = 4 * (lane & 3);
      const f32x4 x = *reinterpret_cast<const f32x4*>(tl + r * kOutLd + q4);
      if (16 * w + r < len) store_out4(out, ((b * p.T + t0 + 16 * w + r) * H + h) * V + v0 + q4, x);
    }
    block_sync();   // B2
  }

  if constexpr (kTrans) {
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int c0 = 16 * (w * NCB + c) + 4 * gq;
#pragma unroll
      for (int i = 0; i < 4; ++i) p.trans[((b * H + h) * K + c0 + i) * K + v0 + m] = st[c][i];
    }
  } else if (p.fin) {
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int c0 = 16 * (w * NCB + c) + 4 * gq;
#pragma unroll
      for (int i = 0; i < 4; ++i) p.fin[(slot * K + c0 + i) * V + v0 + m] = st[c][i];
    }
  }
}

// The same loop with its two halves on separate waves.  Per chunk, only
// Delta and the state update are on the chain from one chunk to the next;
// the read-out O = scale Qg S + scale Aqk Delta is not.  Four chain waves
// (Delta for tokens 16w.., the update of key-channel blocks w NCB..) and
// four read-out waves (O for tokens 16w..) share the workgroup, a chain
// wave and a read-out wave on each SIMD, so that the read-out's matrix work
// and latencies fill the chain's waits instead of lengthening each chunk.
// The state is double-buffered in LDS: the read-out of chunk n reads S_n
// between the barriers B1(n) and B2(n) while the chain writes S_{n+1} into
// the other buffer; Delta_n is read by both between the same barriers.
// Operand loads, precisions and sums are those of the kernel above.  While
// the chain computes Delta_n, the read-out waves pull this workgroup's share
// of record n + 2 into L2 (the chain loads record n + 1's operands then).
template <class TI, class TO, int K, int V>
__global__ __launch_bounds__(2 * kComputeWaves * kWave) void kda_recur_split_kernel(RecurParams p) {
  using P = Prec<TI>;
  using PS = typename P::S;
  using PD = typename P::D;
  using PW = typename P::W;
  using PK = typename P::Kt;
  using PQ = typename P::Qg;
  using PA = typename P::Aq;
  using L = RecordLayout<TI, K, V>;
  constexpr int NV = V / kVT;
  constexpr int NCB = K / 64;
  constexpr int KB = K / 32;
  constexpr int TS = tile_bytes<PS>(), TD = tile_bytes<PD>();
  __shared__ __align__(16) char s_state[2][KB * TS];
  __shared__ __align__(16) char s_delta[2 * TD];
  __shared__ __align__(16) float s_out[kComputeWaves][kChunk / kComputeWaves * kOutLd];
  __shared__ __align__(16) char s_sink[1024];   // discarded data of the L2 prefetches

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = wave & (kComputeWaves - 1);
  const bool readout = wave >= kComputeWaves;
  const int m = lane & 15, gq = lane >> 4;
  const int64_t H = p.H;

  // XCD-aware decode, as above.
  const int64_t id = blockIdx.x;
  const int64_t seq_head = (id / (8 * NV)) * 8 + id % 8;
  const int j = (int)((id / 8) % NV);
  const int64_t n_seq_heads = p.packed ? (int64_t)p.hdr->n_segments * H : p.n_seq_heads_fixed;
  if (seq_head >= n_seq_heads) return;
  const int64_t h = seq_head % H, sq = seq_head / H;

  int64_t b, slot, n_chunks, first_chunk, t_begin, seq_len;
  if (p.packed) {
    const SegEntry se = p.segs[sq];
    b = se.b;
    slot = ((int64_t)se.b * p.n_max + se.local) * H + h;
    n_chunks = se.n_chunks;
    first_chunk = se.chunk_begin;
    t_begin = se.t0;
    seq_len = se.len;
  } else {
    b = sq;
    slot = b * H + h;
    n_chunks = p.nc_fixed;
    first_chunk = b * p.nc_fixed;
    t_begin = 0;
    seq_len = p.T;
  }
  auto record = [&](int64_t n) { return p.records + ((first_chunk + n) * H + h) * p.record_bytes; };
  const int v0 = kVT * j;

  if (!readout) {
    // ---- chain wave w
    PW wn[KB];
    f32x4 u;
    PK kt[NCB][2];
    f32x4 gc[NCB];
    auto load_w = [&](const char* r) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) wn[kb].load(r + L::kWn + (int64_t)(w * KB + kb) * tile_bytes<PW>(), lane);
      u = reinterpret_cast<const f32x4*>(r + L::kU + (int64_t)(w * (V / 16) + j) * 1024)[lane];
    };
    auto load_kt = [&](const char* r) {
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          kt[c][kb].load(r + L::kKt + (int64_t)((w * NCB + c) * 2 + kb) * tile_bytes<PK>(), lane);
        gc[c] = reinterpret_cast<const f32x4*>(r + L::kGc)[4 * (w * NCB + c) + gq];
      }
    };
    f32x4 st[NCB];
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int c0 = 16 * (w * NCB + c) + 4 * gq;
#pragma unroll
      for (int i = 0; i < 4; ++i) st[c][i] = p.init ? p.init[(slot * K + c0 + i) * V + v0 + m] : 0.f;
      float x[4] = {st[c][0], st[c][1], st[c][2], st[c][3]};
      const int cb = w * NCB + c;
      PS::store_half(s_state[0] + (cb / 2) * TS, lane, cb & 1, x);
    }
    if (n_chunks > 0) {
      load_w(record(0));
      load_kt(record(0));
    }
    block_sync();   // B0
    for (int64_t n = 0; n < n_chunks; ++n) {
      const char* rn1 = record(n + 1 < n_chunks ? n + 1 : n);
      const char* cur = s_state[n & 1];
      // Delta = U - W S for tokens 16w..16w+15
      {
        PS sf[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sf[kb].load(cur + kb * TS, lane);
        f32x4 d0 = u, d1 = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < KB; kb += 2) {
          mma(d0, wn[kb], sf[kb]);
          if (kb + 1 < KB) mma(d1, wn[kb + 1], sf[kb + 1]);
        }
        float x[4] = {d0[0] + d1[0], d0[1] + d1[1], d0[2] + d1[2], d0[3] + d1[3]};
        PD::store_half(s_delta + (w / 2) * TD, lane, w & 1, x);
      }
      load_w(rn1);
      block_sync();   // B1
      // S <- diag(exp(G_C)) S + Kt^T Delta, into the other buffer
      PD dd[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) dd[kb].load(s_delta + kb * TD, lane);
      char* nxt = s_state[(n + 1) & 1];
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        f32x4 a0, a1 = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) a0[i] = st[c][i] * gc[c][i];
        mma(a0, kt[c][0], dd[0]);
        mma(a1, kt[c][1], dd[1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) st[c][i] = a0[i] + a1[i];
        float x[4] = {st[c][0], st[c][1], st[c][2], st[c][3]};
        const int cb = w * NCB + c;
        PS::store_half(nxt + (cb / 2) * TS, lane, cb & 1, x);
      }
      load_kt(rn1);
      block_sync();   // B2
    }
    if (p.fin) {
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const int c0 = 16 * (w * NCB + c) + 4 * gq;
#pragma unroll
        for (int i = 0; i < 4; ++i) p.fin[(slot * K + c0 + i) * V + v0 + m] = st[c][i];
      }
    }
    return;
  }

  // ---- read-out wave w: O = scale Qg S + scale Aqk Delta for tokens 16w..16w+15
  TO* out = static_cast<TO*>(p.o);
  PQ qg[KB];
  PA aq[2];
  auto load_q = [&](const char* r) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qg[kb].load(r + L::kQg + (int64_t)(w * KB + kb) * tile_bytes<PQ>(), lane);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      if (kb <= w / 2) aq[kb].load(r + L::kAqk + (int64_t)(2 * w + kb) * tile_bytes<PA>(), lane);
  };
  // Every 64-byte segment of the workgroup's 1/NV share of a record, once,
  // split over the four read-out waves.
  auto prefetch = [&](int64_t n) {
    constexpr int SEGS = (int)(L::kBytes / 64);
    constexpr int SHARE = (SEGS + NV - 1) / NV;
    constexpr int PER = (SHARE + kComputeWaves - 1) / kComputeWaves;
    const char* r = record(n);
#pragma unroll
    for (int i = 0; i < (PER + kWave - 1) / kWave; ++i) {
      const int e = i * kWave + lane, seg = j * SHARE + w * PER + e;
      if (e < PER && w * PER + e < SHARE && seg < SEGS) dma16(s_sink, r + 64 * (int64_t)seg);
    }
  };
  if (n_chunks > 0) load_q(record(0));
  if (n_chunks > 1) prefetch(1);
  block_sync();   // B0
  for (int64_t n = 0; n < n_chunks; ++n) {
    const int64_t t0 = t_begin + n * kChunk;
    const int len = (int)min<int64_t>(kChunk, seq_len - n * kChunk);
    const char* rn1 = record(n + 1 < n_chunks ? n + 1 : n);
    if (n + 2 < n_chunks) prefetch(n + 2);
    block_sync();   // B1: Delta_n and S_n in LDS
    const char* cur = s_state[n & 1];
    PS sf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sf[kb].load(cur + kb * TS, lane);
    PD dd[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) dd[kb].load(s_delta + kb * TD, lane);
    f32x4 o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < KB; kb += 2) {
      mma(o0, qg[kb], sf[kb]);
      if (kb + 1 < KB) mma(o1, qg[kb + 1], sf[kb + 1]);
    }
    mma(o1, aq[0], dd[0]);
    if (w >= 2) mma(o0, aq[1], dd[1]);
    load_q(rn1);
    float* tl = s_out[w];
#pragma unroll
    for (int i = 0; i < 4; ++i) tl[(4 * gq + i) * kOutLd + m] = o0[i] + o1[i];
    const int r = lane >> 2, q4 = 4 * (lane & 3);
    const f32x4 x = *reinterpret_cast<const f32x4*>(tl + r * kOutLd + q4);
    if (16 * w + r < len) store_out4(out, ((b * p.T + t0 + 16 * w + r) * H + h) * V + v0 + q4, x);
    block_sync();   // B2
  }
  vm_wait<0>();   // the prefetches' LDS writes land before the workgroup ends
}

template <class TI, class TO, int K, int V, int TPW>
hipError_t launch_recur_w(const RecurParams& p, int64_t seq_heads, hipStream_t stream) {
  constexpr int NVW = V / kVT / TPW;
  const int64_t grid = (seq_heads + 7) / 8 * 8 * NVW;
  hipLaunchKernelGGL((kda_recur_kernel<TI, TO, K, V, TPW>), dim3((unsigned)grid), dim3(Roles<TPW>::kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <class TI, class TO, int K, int V>
hipError_t launch_recur_t(const CallArgs& a) {
  RecurParams p{a.B, a.T, a.H, a.nc_fixed, a.n_max > 0, a.n_max, a.B * a.H, a.hdr, a.segs,
                a.records, a.record_bytes, a.init, a.fin, a.o, a.trans};
  const int64_t seq_heads = (a.n_max > 0 ? a.smax : a.B) * a.H;
  if (seq_heads <= 0) return hipSuccess;
  if (a.trans_only) {
    // Rows without a segment that spans them keep the zero transition.
    if (a.n_max > 0) {
      const hipError_t e = launch_fill_zero(a.trans, a.B * a.H * a.K * a.K, a.stream);
      if (e != hipSuccess) return e;
    }
    const int64_t tgrid = (seq_heads + 7) / 8 * 8 * (K / kVT);
    hipLaunchKernelGGL((kda_recur_reg_kernel<TI, TO, K, V, true>), dim3((unsigned)tgrid),
                       dim3((kComputeWaves + 1) * kWave), 0, a.stream, p);
    return hipGetLastError();
  }
  // One split workgroup per CU while they fit in one round; then the
  // register-direct kernel (two per CU); then two tiles per workgroup.
  const int64_t grid = (seq_heads + 7) / 8 * 8 * (V / kVT);
  if (grid <= (int64_t)cu_count()) {
    hipLaunchKernelGGL((kda_recur_split_kernel<TI, TO, K, V>), dim3((unsigned)grid), dim3(2 * kComputeWaves * kWave),
                       0, a.stream, p);
    return hipGetLastError();
  }
  if (seq_heads * (V / kVT) > 2 * (int64_t)cu_count()) return launch_recur_w<TI, TO, K, V, 2>(p, seq_heads, a.stream);
  hipLaunchKernelGGL((kda_recur_reg_kernel<TI, TO, K, V, false>), dim3((unsigned)grid), dim3((kComputeWaves + 1) * kWave), 0,
                     a.stream, p);
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
