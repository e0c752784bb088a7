// Inter-chunk recurrence and output of the KDA forward.
//
// One workgroup owns one sequence (a row, or a packed segment), one head and
// one or two 16-wide tiles of value channels, and walks that sequence's
// chunks in order.  Columns of the state never mix (the delta rule contracts
// over the key axis only), so value tiles are independent recurrences.  Per
// chunk, with S the K x 16 state slice entering the chunk (fp32):
//   Delta = U - W S                            (tokens 16w..16w+15 per wave)
//   S    <- diag(exp(G_C)) S + Kt^T Delta      (key-channel blocks per wave)
//   O     = scale Qg S + scale Aqk Delta       (tokens 16w..16w+15 per wave)
// following the chunk form of the "Delta Rule formulation" on the page
// "feat(kda): integrate KDA attention with tokamax backend and CP support"
// (Implementation Details).  S and Delta pass between waves through LDS;
// every other operand is read straight into registers from the per-chunk
// records the intra-chunk kernel wrote, one chunk ahead, while a prefetch
// wave pulls later records into L2.
#include "kda_delta.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kVT = 16;   // value channels per workgroup
constexpr int kComputeWaves = 4;   // per value tile

// Four consecutive outputs o[i .. i + 3] (i a multiple of 4), as plain
// stores or, with kStream, non-temporal ones (o is not read again by this
// forward: streaming it past L2 leaves L2 to the chunk records).  Streaming
// pays only where each store instruction covers whole 128-byte lines:
// partial lines are written back separately, each at the cost of a line.
template <bool kStream>
__device__ __forceinline__ void store_out4(float* o, int64_t i, const f32x4& x) {
  if constexpr (kStream) __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(o + i));
  else *reinterpret_cast<f32x4*>(o + i) = x;
}
template <bool kStream>
__device__ __forceinline__ void store_out4(uint16_t* o, int64_t i, const f32x4& x) {
  uint32_t w[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const __bf16 a = to_bf16(x[2 * j]), b = to_bf16(x[2 * j + 1]);
    w[j] = (uint32_t)*reinterpret_cast<const uint16_t*>(&a) | ((uint32_t)*reinterpret_cast<const uint16_t*>(&b) << 16);
  }
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (kStream) __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2*>(o + i));
  else *reinterpret_cast<u32x2*>(o + i) = u32x2{w[0], w[1]};
}
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
  int64_t n_units;   // split kernel: units of work (sequence, head, value tiles) of the grid's numbering
};

// The transition of a row's first segment, for context parallelism: the
// recurrence is affine in the state a segment starts from, S_end = M S_start
// + (S_end for S_start = 0), and M is the chunk product of diag(exp(G_C)) -
// Kt^T W, i.e. the state recurrence with U = 0 and S_start = I, with no
// read-out.  Its columns (K of them, one 16-wide tile per workgroup) index
// the key channels of S_start.  It exists only where one segment runs from
// the row's first token to its last (every row without segment ids); the
// caller zero-fills the others.  This is the transfer matrix a
// context-parallel rank passes on with its end state.
//
// Four compute waves (wave w: Delta for tokens 16w.., the update of
// key-channel blocks w K/64..), each loading its share of a record (its token
// block of Wn, its key blocks of Kt and exp(G_C)) into registers one chunk
// ahead; S and Delta pass through LDS.  Two barriers per chunk: B1 after the
// Delta phase (Delta visible), B2 at the end (the new state visible, the
// Delta buffer free).  The fifth wave pulls the next chunk's Wn and Kt into
// L2.
template <class TI, int K, int V>
__global__ __launch_bounds__((kComputeWaves + 1) * kWave) void kda_recur_trans_kernel(RecurParams p) {
  using P = Prec<TI>;
  using PS = typename P::S;
  using PW = typename P::W;
  using PK = typename P::Kt;
  using L = RecordLayout<TI, K, V>;
  constexpr int kPrefetchWave = kComputeWaves;
  constexpr int NV = K / kVT;      // workgroups per (sequence, head)
  constexpr int NCB = K / 64;      // key-channel blocks of the state per wave
  constexpr int KB = K / 32;       // 32-deep key slabs
  constexpr int TS = tile_bytes<PS>();
  __shared__ __align__(16) char s_state[KB * TS];
  __shared__ __align__(16) DeltaLds<TI> s_delta;
  __shared__ __align__(16) char s_sink[1024];   // discarded data of the L2 prefetches

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

  int64_t b, n_chunks, first_chunk;
  if (p.packed) {
    const SegEntry se = p.segs[sq];
    if (se.t0 != 0 || se.len != p.T) return;   // no segment spans this row
    b = se.b;
    n_chunks = se.n_chunks;
    first_chunk = se.chunk_begin;
  } else {
    b = sq;
    n_chunks = p.nc_fixed;
    first_chunk = b * p.nc_fixed;
  }
  auto record = [&](int64_t n) { return p.records + ((first_chunk + n) * H + h) * p.record_bytes; };

  // ---- L2 prefetch wave: this workgroup's 1/NV share of the record's Wn and
  // Kt (one load per 128-byte L2 line), one chunk ahead.
  if (wave == kPrefetchWave) {
    constexpr int SEGS = (int)(L::kQg / 128);   // L2 lines of 128 bytes
    constexpr int SHARE = (SEGS + NV - 1) / NV;
    auto prefetch = [&](int64_t n) {
      const char* r = record(n);
#pragma unroll
      for (int i = 0; i < (SHARE + kWave - 1) / kWave; ++i) {
        const int e = i * kWave + lane, seg = j * SHARE + e;
        if (e < SHARE && seg < SEGS) dma16(s_sink, r + 128 * (int64_t)seg);
      }
    };
    block_sync();
    for (int64_t n = 0; n < n_chunks; ++n) {
      if (n + 1 < n_chunks) prefetch(n + 1);
      block_sync();   // B1
      block_sync();   // B2
    }
    vm_wait<0>();
    return;
  }

  // ---- compute wave w: token block w, key-channel blocks w*NCB .. +NCB-1
  const int w = wave;
  const int v0 = kVT * j;   // first column of M this workgroup carries
  PW wn[KB];
  PK kt[NCB][2];
  f32x4 gc[NCB];
  float ks[NCB];
  auto load_w = [&](const char* r) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) wn[kb].load(r + L::kWn + (int64_t)(w * KB + kb) * tile_bytes<PW>(), lane);
  };
  auto load_kt = [&](const char* r) {
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kt[c][kb].load(r + L::kKt + (int64_t)((w * NCB + c) * 2 + kb) * tile_bytes<PK>(), lane);
      gc[c] = reinterpret_cast<const f32x4*>(r + L::kGc)[4 * (w * NCB + c) + gq];
      ks[c] = L::kScaledKt ? reinterpret_cast<const float*>(r + L::kKs)[w * NCB + c + vector_zero()] : 1.f;
    }
  };

  // M's slice: lane (column v0 + m, rows 16cb + 4gq + i) of its blocks, from I.
  f32x4 st[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const int c0 = 16 * (w * NCB + c) + 4 * gq;
#pragma unroll
    for (int i = 0; i < 4; ++i) st[c][i] = (c0 + i == v0 + m) ? 1.f : 0.f;
    float x[4] = {st[c][0], st[c][1], st[c][2], st[c][3]};
    const int cb = w * NCB + c;
    PS::store_half(s_state + (cb / 2) * TS, lane, cb & 1, x);
  }
  if (n_chunks > 0) {
    load_w(record(0));
    load_kt(record(0));
  }
  block_sync();

  for (int64_t n = 0; n < n_chunks; ++n) {
    const char* rn1 = record(n + 1 < n_chunks ? n + 1 : n);
    // Delta = -W M for tokens 16w..16w+15 (two accumulators halve the chain)
    PS sf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sf[kb].load(s_state + kb * TS, lane);
    {
      f32x4 d0 = {0, 0, 0, 0}, d1 = {0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < KB; kb += 2) {
        mma(d0, wn[kb], sf[kb]);
        if (kb + 1 < KB) mma(d1, wn[kb + 1], sf[kb + 1]);
      }
      float x[4] = {d0[0] + d1[0], d0[1] + d1[1], d0[2] + d1[2], d0[3] + d1[3]};
      delta_store(s_delta, w, lane, x);
    }
    load_w(rn1);
    block_sync();   // B1

    // M <- diag(exp(G_C)) M + Kt^T Delta
    DeltaOperands<TI> dd;
    dd.load(s_delta, lane);
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      state_update<TI>(st[c], gc[c], ks[c], kt[c], dd);
      float x[4] = {st[c][0], st[c][1], st[c][2], st[c][3]};
      const int cb = w * NCB + c;
      PS::store_half(s_state + (cb / 2) * TS, lane, cb & 1, x);
    }
    load_kt(rn1);
    block_sync();   // B2
  }

#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const int c0 = 16 * (w * NCB + c) + 4 * gq;
#pragma unroll
    for (int i = 0; i < 4; ++i) p.trans[((b * H + h) * K + c0 + i) * K + v0 + m] = st[c][i];
  }
}

// The same loop with its two halves on separate waves, over NT value tiles
// per workgroup.  Per chunk, only Delta and the state update are on the
// chain from one chunk to the next; the read-out O = scale Qg S + scale Aqk
// Delta is not.  Four chain waves (Delta for tokens 16w.., the update of
// key-channel blocks w NCB..) and four read-out waves (O for tokens 16w..)
// share the workgroup, a chain wave and a read-out wave on each SIMD, so
// that the read-out's matrix work and latencies fill the chain's waits.
// The state is double-buffered in LDS: the read-out of chunk n reads S_n
// between the barriers B1(n) and B2(n) while the chain writes S_{n+1} into
// the other buffer; Delta_n is read by both between the same barriers.
// Each wave loads its share of a record once and applies it to all NT
// tiles (with NT = 2 the record bytes per value column halve and the
// read-out writes whole 128-byte lines of o).  Operand loads, precisions and
// sums are those of the kernel above.  A ninth wave pulls this workgroup's
// share of record n + 2 into L2 during chunk n (the chain loads record
// n + 1's operands then); it is a wave of its own because a wave's memory
// counter completes in order, so a wave that also loaded operands would
// wait for its prefetches before them.
constexpr int kSplitWaves = 2 * kComputeWaves + 1;
template <class TI, class TO, int K, int V, int NT>
__global__ __launch_bounds__(kSplitWaves * kWave) void kda_recur_split_kernel(RecurParams p) {
  using P = Prec<TI>;
  using PS = typename P::S;
  using PD = typename P::D;
  using PW = typename P::W;
  using PK = typename P::Kt;
  using PQ = typename P::Qg;
  using PA = typename P::Aq;
  using L = RecordLayout<TI, K, V>;
  constexpr int NV = V / (kVT * NT);   // workgroups per (sequence, head)
  constexpr int NCB = K / 64;
  constexpr int KB = K / 32;
  constexpr int TS = tile_bytes<PS>();
  constexpr int OLD = kVT * NT + 4;    // row pitch of the output staging tile
  __shared__ __align__(16) char s_state[2][NT][KB * TS];
  __shared__ __align__(16) DeltaLds<TI> s_delta[NT];
  __shared__ __align__(16) float s_out[kComputeWaves][kChunk / kComputeWaves * OLD];
  __shared__ __align__(16) char s_sink[1024];   // discarded data of the L2 prefetches

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = wave & (kComputeWaves - 1);
  const bool readout = wave >= kComputeWaves && wave < 2 * kComputeWaves;
  const bool prefetcher = wave == 2 * kComputeWaves;
  const int m = lane & 15, gq = lane >> 4;
  const int64_t H = p.H;

  // Units of work: (sequence, head, NT value tiles), numbered XCD-aware as
  // above (the NV units of a (sequence, head) share id % 8, so they share an
  // L2).  Workgroup g takes units g, g + gridDim.x, ...: with gridDim.x a
  // multiple of 8 NV each workgroup keeps one column j and one XCD, and the
  // sequence-head grows with every step, so the first one past the last
  // ends the walk.  Each unit's first records are loaded during the last
  // chunks of the one before.
  const int64_t n_seq_heads = p.packed ? (int64_t)p.hdr->n_segments * H : p.n_seq_heads_fixed;
  struct Unit {
    int64_t slot, first_chunk;
    int h, b, n_chunks, t_begin, seq_len, j;
    bool valid;
  };
  auto decode = [&](int64_t id) {
    Unit u;
    const int64_t seq_head = (id / (8 * NV)) * 8 + id % 8;
    u.j = (int)((id / 8) % NV);
    u.valid = id < p.n_units && seq_head < n_seq_heads;
    if (!u.valid) return u;
    u.h = (int)(seq_head % H);
    const int64_t sq = seq_head / H;
    if (p.packed) {
      const SegEntry se = p.segs[sq];
      u.b = se.b;
      u.slot = ((int64_t)se.b * p.n_max + se.local) * H + u.h;
      u.n_chunks = se.n_chunks;
      u.first_chunk = se.chunk_begin;
      u.t_begin = se.t0;
      u.seq_len = se.len;
    } else {
      u.b = (int)sq;
      u.slot = sq * H + u.h;
      u.n_chunks = (int)p.nc_fixed;
      u.first_chunk = sq * p.nc_fixed;
      u.t_begin = 0;
      u.seq_len = (int)p.T;
    }
    return u;
  };
  int64_t uid = blockIdx.x;
  Unit cur = decode(uid);
  if (!cur.valid) return;
  Unit nxt = decode(uid + gridDim.x);
  auto record = [&](const Unit& u, int64_t n) {
    return p.records + ((u.first_chunk + n) * H + u.h) * p.record_bytes;
  };
  // The record after chunk n of the current unit: its next chunk, else the
  // next unit's first (else chunk n again, loaded and not used).
  auto record_after = [&](int64_t n) {
    return n + 1 < cur.n_chunks ? record(cur, n + 1) : (nxt.valid ? record(nxt, 0) : record(cur, n));
  };
  auto advance = [&] {
    cur = nxt;
    uid += gridDim.x;
    nxt = decode(uid + gridDim.x);
  };

  if (prefetcher) {
    // ---- one 16-byte load in every 128-byte L2 line of the workgroup's
    //      1/NV share of a record, two records ahead in its sequence of records
    auto prefetch = [&](const char* r, int jj) {
      constexpr int SEGS = (int)(L::kBytes / 128);   // L2 lines of 128 bytes
      constexpr int SHARE = (SEGS + NV - 1) / NV;
#pragma unroll
      for (int i = 0; i < (SHARE + kWave - 1) / kWave; ++i) {
        const int e = i * kWave + lane, seg = jj * SHARE + e;
        if (e < SHARE && seg < SEGS) dma16(s_sink, r + 128 * (int64_t)seg);
      }
    };
    if (cur.n_chunks > 1) prefetch(record(cur, 1), cur.j);
    for (;;) {
      block_sync();   // B0
      for (int64_t n = 0; n < cur.n_chunks; ++n) {
        const int64_t a = n + 2;
        if (a < cur.n_chunks) prefetch(record(cur, a), cur.j);
        else if (nxt.valid && a - cur.n_chunks < nxt.n_chunks) prefetch(record(nxt, a - cur.n_chunks), nxt.j);
        block_sync();   // B1
        block_sync();   // B2
      }
      if (!nxt.valid) break;
      advance();
    }
    vm_wait<0>();   // the prefetches' LDS writes land before the workgroup ends
    return;
  }

  if (!readout) {
    // ---- chain wave w
    PW wn[KB];
    f32x4 u[NT];
    PK kt[NCB][2];
    f32x4 gc[NCB];
    float ks[NCB];
    auto load_w = [&](const char* r, int jj) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) wn[kb].load(r + L::kWn + (int64_t)(w * KB + kb) * tile_bytes<PW>(), lane);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        u[t] = reinterpret_cast<const f32x4*>(r + L::kU + (int64_t)(w * (V / 16) + NT * jj + t) * 1024)[lane];
    };
    auto load_kt = [&](const char* r) {
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          kt[c][kb].load(r + L::kKt + (int64_t)((w * NCB + c) * 2 + kb) * tile_bytes<PK>(), lane);
        gc[c] = reinterpret_cast<const f32x4*>(r + L::kGc)[4 * (w * NCB + c) + gq];
        ks[c] = L::kScaledKt ? reinterpret_cast<const float*>(r + L::kKs)[w * NCB + c + vector_zero()] : 1.f;
      }
    };
    load_w(record(cur, 0), cur.j);
    load_kt(record(cur, 0));
    for (;;) {
      const int v0 = kVT * NT * cur.j;   // first value column of tile 0
      f32x4 st[NT][NCB];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int c = 0; c < NCB; ++c) {
          const int c0 = 16 * (w * NCB + c) + 4 * gq;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            st[t][c][i] = p.init ? p.init[(cur.slot * K + c0 + i) * V + v0 + 16 * t + m] : 0.f;
          float x[4] = {st[t][c][0], st[t][c][1], st[t][c][2], st[t][c][3]};
          const int cb = w * NCB + c;
          PS::store_half(s_state[0][t] + (cb / 2) * TS, lane, cb & 1, x);
        }
      }
      block_sync();   // B0
      for (int64_t n = 0; n < cur.n_chunks; ++n) {
        const char* rn1 = record_after(n);
        const int jn = n + 1 < cur.n_chunks || !nxt.valid ? cur.j : nxt.j;
        // Delta = U - W S for tokens 16w..16w+15, tile by tile
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const char* cs = s_state[n & 1][t];
          PS sf[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) sf[kb].load(cs + kb * TS, lane);
          __builtin_amdgcn_sched_barrier(0);   // every operand read issued before the products
          f32x4 d0 = u[t], d1 = {0, 0, 0, 0};
#pragma unroll
          for (int kb = 0; kb < KB; kb += 2) {
            mma(d0, wn[kb], sf[kb]);
            if (kb + 1 < KB) mma(d1, wn[kb + 1], sf[kb + 1]);
          }
          float x[4] = {d0[0] + d1[0], d0[1] + d1[1], d0[2] + d1[2], d0[3] + d1[3]};
          delta_store(s_delta[t], w, lane, x);
        }
        load_w(rn1, jn);
        block_sync();   // B1
        // S <- diag(exp(G_C)) S + Kt^T Delta, into the other buffer
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          DeltaOperands<TI> dd;
          dd.load(s_delta[t], lane);
          char* ns = s_state[(n + 1) & 1][t];
#pragma unroll
          for (int c = 0; c < NCB; ++c) {
            state_update<TI>(st[t][c], gc[c], ks[c], kt[c], dd);
            float x[4] = {st[t][c][0], st[t][c][1], st[t][c][2], st[t][c][3]};
            const int cb = w * NCB + c;
            PS::store_half(ns + (cb / 2) * TS, lane, cb & 1, x);
          }
        }
        load_kt(rn1);
        block_sync();   // B2
      }
      if (p.fin) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int c = 0; c < NCB; ++c) {
            const int c0 = 16 * (w * NCB + c) + 4 * gq;
#pragma unroll
            for (int i = 0; i < 4; ++i) p.fin[(cur.slot * K + c0 + i) * V + v0 + 16 * t + m] = st[t][c][i];
          }
        }
      }
      if (!nxt.valid) break;
      advance();
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
      if (kb <= w / 2) aq[kb].load(r + L::kAqk + (int64_t)aqk_tile(w, kb) * tile_bytes<PA>(), lane);
  };
  float* tl = s_out[w];
  load_q(record(cur, 0));
  for (;;) {
    const int v0 = kVT * NT * cur.j;
    block_sync();   // B0
    for (int64_t n = 0; n < cur.n_chunks; ++n) {
      const int64_t t0 = cur.t_begin + n * kChunk;
      const int len = (int)min<int64_t>(kChunk, cur.seq_len - n * kChunk);
      const char* rn1 = record_after(n);
      block_sync();   // B1: Delta_n and S_n in LDS
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const char* cs = s_state[n & 1][t];
        PS sf[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sf[kb].load(cs + kb * TS, lane);
        PD dd[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dd[kb].load(s_delta[t].d + kb * DeltaLds<TI>::TD, lane);
        __builtin_amdgcn_sched_barrier(0);   // every operand read issued before the products
        f32x4 o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < KB; kb += 2) {
          mma(o0, qg[kb], sf[kb]);
          if (kb + 1 < KB) mma(o1, qg[kb + 1], sf[kb + 1]);
        }
        mma(o1, aq[0], dd[0]);
        if (w >= 2) mma(o0, aq[1], dd[1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) tl[(4 * gq + i) * OLD + 16 * t + m] = o0[i] + o1[i];
      }
      load_q(rn1);
      // Rows of the tile from LPR lanes each, 4 consecutive columns per lane:
      // every store instruction writes whole row pieces of the tile's 16 NT
      // columns (with NT = 2 whole 128-byte lines of fp32 o, streamed; with
      // one tile a line is shared by two workgroups, and plain stores let L2
      // join its halves).
      constexpr int LPR = kVT * NT / 4;   // lanes per row
      constexpr int RPI = kWave / LPR;    // rows per store instruction
      const int q = 4 * (lane % LPR);
#pragma unroll
      for (int r0 = 0; r0 < kChunk / kComputeWaves; r0 += RPI) {
        const int r = r0 + lane / LPR;
        const f32x4 x = *reinterpret_cast<const f32x4*>(tl + r * OLD + q);
        if (16 * w + r < len)
          store_out4<NT == 2>(out, (((int64_t)cur.b * p.T + t0 + 16 * w + r) * H + cur.h) * V + v0 + q, x);
      }
      block_sync();   // B2
    }
    if (!nxt.valid) break;
    advance();
  }
}


template <class TI, class TO, int K, int V>
hipError_t launch_recur_t(const CallArgs& a) {
  RecurParams p{a.B, a.T, a.H, a.nc_fixed, a.n_max > 0, a.n_max, a.B * a.H, a.hdr, a.segs,
                a.records, a.record_bytes, a.init, a.fin, a.o, a.trans, 0};
  const int64_t seq_heads = (a.n_max > 0 ? a.smax : a.B) * a.H;
  if (seq_heads <= 0) return hipSuccess;
  if (a.trans_only) {
    // Rows without a segment that spans them keep the zero transition.
    if (a.n_max > 0) {
      const hipError_t e = launch_fill_zero(a.trans, a.B * a.H * a.K * a.K, a.stream);
      if (e != hipSuccess) return e;
    }
    const int64_t tgrid = (seq_heads + 7) / 8 * 8 * (K / kVT);
    hipLaunchKernelGGL((kda_recur_trans_kernel<TI, K, V>), dim3((unsigned)tgrid),
                       dim3((kComputeWaves + 1) * kWave), 0, a.stream, p);
    return hipGetLastError();
  }
  // One value tile per split workgroup while one workgroup per CU covers
  // every tile: then each chunk's step is as short as it gets.  Beyond, two
  // tiles per workgroup: the step is longer (the matrix work per SIMD
  // doubles) but each record operand is loaded once for both tiles, which
  // wins once the workgroups take several rounds; and a grid of one
  // workgroup per CU (a multiple of 8 NV units) that walks the units, so
  // that a unit's first records load under the last chunks of the one
  // before instead of opening every unit.
  const int64_t tiles = (seq_heads + 7) / 8 * 8 * (V / kVT);
  const int64_t cus = cu_count();
  if (tiles <= cus) {
    p.n_units = tiles;
    hipLaunchKernelGGL((kda_recur_split_kernel<TI, TO, K, V, 1>), dim3((unsigned)tiles), dim3(kSplitWaves * kWave), 0,
                       a.stream, p);
  } else {
    p.n_units = tiles / 2;
    const int64_t step = 8 * (V / (2 * kVT));
    const int64_t grid = std::min<int64_t>(p.n_units, std::max<int64_t>(step, cus / step * step));
    hipLaunchKernelGGL((kda_recur_split_kernel<TI, TO, K, V, 2>), dim3((unsigned)grid),
                       dim3(kSplitWaves * kWave), 0, a.stream, p);
  }
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
