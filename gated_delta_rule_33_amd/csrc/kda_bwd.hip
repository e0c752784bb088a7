// KDA backward: gradients of the chunked forward with respect to q, k, v, g,
// beta and the initial state, given dL/do and dL/d(final state).
//
// The forward is the gated delta rule of the page "feat(kda): integrate KDA
// attention with tokamax backend and CP support" (Implementation Details,
// Delta Rule formulation); that page's CP gradient-equivalence test and the
// tokamax pages' follow-ups treat the backward as its own pass.  Per chunk of
// C rows with S the state entering it (G = in-chunk cumsum of g, Gamma =
// exp(G), Gamma_C = exp(G of the last row)):
//     A   = strictly lower  beta_r sum_c k_rc k_ic exp(G_rc - G_ic)
//     Aqk = lower           sum_c q_rc k_ic exp(G_rc - G_ic)
//     T = (I + A)^-1,  W = T diag(beta) (K * Gamma),  U = T diag(beta) V
//     Delta = U - W S,  O = scale (Q * Gamma) S + scale Aqk Delta
//     S'  = diag(Gamma_C) S + Kt^T Delta,  Kt = K * exp(G_C - G)
// and its reverse, given dO and dS' (= dL/dS'):
//     dDelta = scale Aqk^T dO + Kt dS'
//     dS     = diag(Gamma_C) dS' + scale (Q * Gamma)^T dO - W^T dDelta
// (a recurrence run from the last chunk back), then per chunk the local
// products dQg = scale dO S^T, dAqk = scale dO Delta^T, dKt = Delta dS'^T,
// dW = -dDelta S^T, dU = dDelta, dT = dW Kb^T + dU Vb^T, dKb = T^T dW,
// dVb = T^T dU, dA = -T^T dT T^T, and the exponent-factor terms of A and Aqk
// back onto q, k and G; dg is the reverse in-chunk cumsum of dG.
//
// Chunks here are 16 rows: exp(G_r - G_0) <= 1 and exp(G_0 - G_i) <= exp(64)
// for any 16-row span up to 64, which leaves a wide margin below FLT_MAX for
// the sums these factors enter, so every product splits at the chunk's first
// row; a chunk with a larger span (possible only at the edge of the safe
// gate's [-5, 0), or without it) takes exp(G_r - G_i) per element.  The result does not depend on
// the chunk size.  Everything is fp32 (bf16 inputs are exact in fp32).
//
// Kernels, in order: bwd_chunk (one workgroup per chunk and head: G, A, Aqk,
// T, W, U, Kt, Qg into a chunk record), bwd_states (the forward recurrence
// again, keeping the state entering every chunk), bwd_dstates (the reverse
// recurrence, keeping dS' of every chunk and the initial-state gradients),
// bwd_local (one workgroup per chunk and head: all input gradients).
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kBC = 16;            // rows per backward chunk
constexpr int kBThreads = 256;
constexpr float kSpanMax = 64.f;   // exp(64) ~ 6e27: room for sums of O(1e10) below FLT_MAX

// Chunk record (floats) per (slot, head).
template <int K, int V>
struct BRec {
  static constexpr int64_t kG = 0;                    // [16][K]  in-chunk cumsum of g
  static constexpr int64_t kKt = kG + kBC * K;        // [16][K]  k exp(G_C - G)
  static constexpr int64_t kQg = kKt + kBC * K;       // [16][K]  q exp(G)
  static constexpr int64_t kW = kQg + kBC * K;        // [16][K]
  static constexpr int64_t kU = kW + kBC * K;         // [16][V]
  static constexpr int64_t kAqk = kU + kBC * V;       // [16][16]
  static constexpr int64_t kT = kAqk + kBC * kBC;     // [16][16]
  static constexpr int64_t kGc = kT + kBC * kBC;      // [K]      exp(G_C)
  static constexpr int64_t kInfo = kGc + K;           // [4]      unsafe-span flag
  static constexpr int64_t kFloats = (kInfo + 4 + 63) / 64 * 64;
};

struct BwdParams {
  int64_t B, T, H;
  int64_t nc64;                 // 64-token chunks per row without segment ids
  int packed, n_max, l2norm;
  float scale;
  const TableHeader* hdr;
  const SegEntry* segs;
  const ChunkEntry* chunks;
  const void *q, *k, *v, *g, *beta, *d_o;
  const float *init, *d_final;
  float *dq, *dk, *dv, *dg, *dbeta, *d_init;
  float* rec;                   // [slots][H][BRec::kFloats]
  float* hs;                    // [slots][H][K][V] state entering each chunk
  float* dhs;                   // [slots][H][K][V] dL/d(state leaving each chunk)
};

// A 16-row chunk: slot s is sub-chunk s % 4 of 64-token chunk s / 4.
struct BSlot {
  int64_t b, t0;
  int len;
};

__device__ bool slot_info(const BwdParams& p, int64_t slot, BSlot* s) {
  if (p.packed) {
    const int64_t c = slot / 4;
    if (c >= p.hdr->n_chunks) return false;
    const ChunkEntry ce = p.chunks[c];
    const int len = ce.len - kBC * (int)(slot % 4);
    if (len <= 0) return false;
    s->b = ce.b;
    s->t0 = ce.t0 + kBC * (slot % 4);
    s->len = min(kBC, len);
  } else {
    const int64_t per_row = 4 * p.nc64;
    s->b = slot / per_row;
    s->t0 = kBC * (slot % per_row);
    if (s->t0 >= p.T) return false;
    s->len = (int)min<int64_t>(kBC, p.T - s->t0);
  }
  return true;
}

// A sequence (segment, or row without segment ids): its first slot, its
// number of 16-row chunks, its row, and its state slot.
struct BSeq {
  int64_t b, slot0, n16, state, t0;
};

__device__ bool seq_info(const BwdParams& p, int64_t sq, int64_t h, BSeq* s) {
  if (p.packed) {
    if (sq >= p.hdr->n_segments) return false;
    const SegEntry se = p.segs[sq];
    s->b = se.b;
    s->slot0 = 4 * (int64_t)se.chunk_begin;
    s->n16 = (se.len + kBC - 1) / kBC;
    s->state = ((int64_t)se.b * p.n_max + se.local) * p.H + h;
    s->t0 = se.t0;
  } else {
    if (sq >= p.B) return false;
    s->b = sq;
    s->slot0 = sq * 4 * p.nc64;
    s->n16 = (p.T + kBC - 1) / kBC;
    s->state = sq * p.H + h;
    s->t0 = 0;
  }
  return true;
}

__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bits_to_f32(p[i]); }

// Sum over the 16 lanes of an aligned lane group.
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// ---------------------------------------------------------------- bwd_chunk
template <class TI, int K, int V>
__global__ __launch_bounds__(kBThreads) void bwd_chunk_kernel(BwdParams p) {
  using R = BRec<K, V>;
  const int64_t slot = blockIdx.x / p.H, h = blockIdx.x % p.H;
  BSlot si;
  if (!slot_info(p, slot, &si)) return;
  __shared__ float sk[kBC][K], sq[kBC][K], sG[kBC][K], sv[kBC][V];
  __shared__ float skf[kBC][K], skb[kBC][K], sqf[kBC][K];
  __shared__ float sA[kBC][kBC + 1], sT[kBC][kBC + 1], sbeta[kBC];
  __shared__ int s_unsafe;
  const int tid = threadIdx.x;
  const TI* q = static_cast<const TI*>(p.q);
  const TI* k = static_cast<const TI*>(p.k);
  const TI* v = static_cast<const TI*>(p.v);
  const TI* g = static_cast<const TI*>(p.g);
  const TI* beta = static_cast<const TI*>(p.beta);
  float* rec = p.rec + (slot * p.H + h) * R::kFloats;
  if (tid == 0) s_unsafe = 0;
  for (int e = tid; e < kBC * K; e += kBThreads) {
    const int r = e / K, c = e % K;
    const int64_t off = ((si.b * p.T + si.t0 + r) * p.H + h) * K + c;
    const bool live = r < si.len;
    sk[r][c] = live ? ld(k, off) : 0.f;
    sq[r][c] = live ? ld(q, off) : 0.f;
    sG[r][c] = live ? ld(g, off) : 0.f;
  }
  for (int e = tid; e < kBC * V; e += kBThreads) {
    const int r = e / V, j = e % V;
    sv[r][j] = r < si.len ? ld(v, ((si.b * p.T + si.t0 + r) * p.H + h) * V + j) : 0.f;
  }
  if (tid < kBC) sbeta[tid] = tid < si.len ? ld(beta, (si.b * p.T + si.t0 + tid) * p.H + h) : 0.f;
  __syncthreads();
  if (p.l2norm) {
    // 16 lanes per row: sum of squares, then divide
    const int r = tid / 16, sub = tid % 16;
    float sqq = 0.f, skk = 0.f;
    for (int c = sub; c < K; c += 16) {
      sqq += sq[r][c] * sq[r][c];
      skk += sk[r][c] * sk[r][c];
    }
    sqq = sum16(sqq);
    skk = sum16(skk);
    const float iq = 1.f / sqrtf(sqq + 1e-6f), ik = 1.f / sqrtf(skk + 1e-6f);
    for (int c = sub; c < K; c += 16) {
      sq[r][c] *= iq;
      sk[r][c] *= ik;
    }
  }
  // in-chunk cumsum of g, one channel per thread
  for (int c = tid; c < K; c += kBThreads) {
    float run = 0.f;
    for (int r = 0; r < kBC; ++r) {
      run += sG[r][c];
      sG[r][c] = run;
    }
    if (sG[0][c] - sG[si.len - 1][c] > kSpanMax) s_unsafe = 1;
  }
  __syncthreads();
  const bool unsafe = s_unsafe != 0;
  const int last = si.len - 1;
  for (int e = tid; e < kBC * K; e += kBThreads) {
    const int r = e / K, c = e % K;
    const float G = sG[r][c], G0 = sG[0][c], GC = sG[last][c];
    skf[r][c] = sk[r][c] * __expf(G - G0);
    skb[r][c] = unsafe ? 0.f : sk[r][c] * __expf(G0 - G);
    sqf[r][c] = sq[r][c] * __expf(G - G0);
    rec[R::kG + e] = G;
    rec[R::kKt + e] = sk[r][c] * __expf(GC - G);
    rec[R::kQg + e] = sq[r][c] * __expf(G);
    if (r == 0) rec[R::kGc + c] = __expf(GC);
  }
  __syncthreads();
  {
    // A and Aqk, one (r, i) pair per thread
    const int r = tid / kBC, i = tid % kBC;
    float a = 0.f, aq = 0.f;
    if (i <= r) {
      if (!unsafe) {
        for (int c = 0; c < K; ++c) {
          a += skf[r][c] * skb[i][c];
          aq += sqf[r][c] * skb[i][c];
        }
      } else {
        for (int c = 0; c < K; ++c) {
          const float e = __expf(sG[r][c] - sG[i][c]);
          a += sk[r][c] * sk[i][c] * e;
          aq += sq[r][c] * sk[i][c] * e;
        }
      }
    }
    sA[r][i] = i < r ? sbeta[r] * a : 0.f;
    rec[R::kAqk + r * kBC + i] = aq;
  }
  __syncthreads();
  // T = (I + A)^-1 by forward substitution, one column per thread
  if (tid < kBC) {
    const int j = tid;
    for (int r = 0; r < kBC; ++r) {
      float t = r == j ? 1.f : 0.f;
      for (int i = j; i < r; ++i) t -= sA[r][i] * sT[i][j];
      sT[r][j] = r >= j ? t : 0.f;
    }
  }
  // Kb = diag(beta) (K * Gamma) in place of q, which A and Aqk no longer need
  for (int e = tid; e < kBC * K; e += kBThreads) {
    const int r = e / K, c = e % K;
    sq[r][c] = sbeta[r] * sk[r][c] * __expf(sG[r][c]);
  }
  __syncthreads();
  rec[R::kT + tid] = sT[tid / kBC][tid % kBC];
  // W = T Kb, U = T diag(beta) V
  for (int e = tid; e < kBC * K; e += kBThreads) {
    const int r = e / K, c = e % K;
    float w = 0.f;
    for (int i = 0; i <= r; ++i) w += sT[r][i] * sq[i][c];
    rec[R::kW + e] = w;
  }
  for (int e = tid; e < kBC * V; e += kBThreads) {
    const int r = e / V, j = e % V;
    float u = 0.f;
    for (int i = 0; i <= r; ++i) u += sT[r][i] * sbeta[i] * sv[i][j];
    rec[R::kU + e] = u;
  }
  if (tid == 0) rec[R::kInfo] = unsafe ? 1.f : 0.f;
}

// ---------------------------------------------------- recurrences (helpers)
// Per-chunk operands of one 16-column state tile, staged through registers
// one chunk ahead and stored into the LDS buffer of the next chunk.
template <int K, int V, bool kRev>
struct Stage {
  static constexpr int NW = kBC * K / 4 / kBThreads;   // float4 of W (and Kt, Qg) per thread
  f32x4 w[NW], kt[NW], qg[NW];
  float u, aq, gc, dout;
  __device__ void fetch(const float* rec, int tid, int tile, const float* dorow_f, const uint16_t* dorow_b,
                        int64_t do_stride, int len) {
    using R = BRec<K, V>;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      w[i] = reinterpret_cast<const f32x4*>(rec + R::kW)[tid + i * kBThreads];
      kt[i] = reinterpret_cast<const f32x4*>(rec + R::kKt)[tid + i * kBThreads];
      if (kRev) qg[i] = reinterpret_cast<const f32x4*>(rec + R::kQg)[tid + i * kBThreads];
    }
    const int r = tid / kBC, j = tid % kBC;
    u = kRev ? 0.f : rec[R::kU + r * V + tile * kBC + j];
    aq = kRev ? rec[R::kAqk + tid] : 0.f;
    gc = tid < K ? rec[R::kGc + tid] : 0.f;
    dout = 0.f;
    if (kRev && r < len) dout = dorow_f ? dorow_f[r * do_stride + tile * kBC + j]
                                        : bits_to_f32(dorow_b[r * do_stride + tile * kBC + j]);
  }
  __device__ void store(float (*sW)[K], float (*sKt)[K], float (*sQg)[K], float (*sX)[kBC], float (*sAq)[kBC],
                        float* sGc, float (*sdO)[kBC], int tid) const {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      reinterpret_cast<f32x4*>(&sW[0][0])[tid + i * kBThreads] = w[i];
      reinterpret_cast<f32x4*>(&sKt[0][0])[tid + i * kBThreads] = kt[i];
      if (kRev) reinterpret_cast<f32x4*>(&sQg[0][0])[tid + i * kBThreads] = qg[i];
    }
    const int r = tid / kBC, j = tid % kBC;
    if (!kRev) sX[r][j] = u;
    if (kRev) {
      sAq[r][j] = aq;
      sdO[r][j] = dout;
    }
    if (tid < K) sGc[tid] = gc;
  }
};

// ---------------------------------------------------------------- bwd_states
// One workgroup per (sequence, head, 16 value columns): S from the initial
// state through every chunk, writing the state entering each chunk.
template <int K, int V>
__global__ __launch_bounds__(kBThreads) void bwd_states_kernel(BwdParams p) {
  using R = BRec<K, V>;
  constexpr int NV = V / kBC;
  const int64_t id = blockIdx.x;
  const int tile = (int)(id % NV);
  const int64_t sh = id / NV, h = sh % p.H, sq = sh / p.H;
  BSeq s;
  if (!seq_info(p, sq, h, &s)) return;
  __shared__ float S[K][kBC];
  __shared__ float sW[2][kBC][K], sKt[2][kBC][K], sU[2][kBC][kBC], sGc[2][K], sD[kBC][kBC];
  const int tid = threadIdx.x;
  const int cr = tid / 2, j0 = (tid % 2) * 8;   // state rows owned in the update (K = 128; K = 64 uses tid < 128)
  for (int e = tid; e < K * kBC; e += kBThreads) {
    const int c = e / kBC, j = e % kBC;
    S[c][j] = p.init ? p.init[s.state * K * V + c * V + tile * kBC + j] : 0.f;
  }
  auto rec = [&](int64_t n) { return p.rec + ((s.slot0 + n) * p.H + h) * R::kFloats; };
  Stage<K, V, false> st;
  st.fetch(rec(0), tid, tile, nullptr, nullptr, 0, 0);
  st.store(sW[0], sKt[0], nullptr, sU[0], nullptr, sGc[0], nullptr, tid);
  __syncthreads();
  for (int64_t n = 0; n < s.n16; ++n) {
    const int cur = (int)(n & 1);
    if (n + 1 < s.n16) st.fetch(rec(n + 1), tid, tile, nullptr, nullptr, 0, 0);
    float* hs = p.hs + ((s.slot0 + n) * p.H + h) * K * V + tile * kBC;
    for (int e = tid; e < K * kBC; e += kBThreads) hs[(e / kBC) * V + e % kBC] = S[e / kBC][e % kBC];
    {
      const int r = tid / kBC, j = tid % kBC;
      float d = sU[cur][r][j];
      for (int c = 0; c < K; ++c) d -= sW[cur][r][c] * S[c][j];
      sD[r][j] = d;
    }
    __syncthreads();
    if (cr < K) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        float x = sGc[cur][cr] * S[cr][j0 + jj];
        for (int r = 0; r < kBC; ++r) x += sKt[cur][r][cr] * sD[r][j0 + jj];
        S[cr][j0 + jj] = x;
      }
    }
    if (n + 1 < s.n16) st.store(sW[cur ^ 1], sKt[cur ^ 1], nullptr, sU[cur ^ 1], nullptr, sGc[cur ^ 1], nullptr, tid);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- bwd_dstates
// One workgroup per (sequence, head, 16 value columns): dS' from the final
// state's gradient back through every chunk, writing dS' of each chunk and
// the gradient of the sequence's initial state.
template <class TO, int K, int V>
__global__ __launch_bounds__(kBThreads) void bwd_dstates_kernel(BwdParams p) {
  using R = BRec<K, V>;
  constexpr int NV = V / kBC;
  const int64_t id = blockIdx.x;
  const int tile = (int)(id % NV);
  const int64_t sh = id / NV, h = sh % p.H, sq = sh / p.H;
  BSeq s;
  if (!seq_info(p, sq, h, &s)) return;
  __shared__ float S[K][kBC];   // dS'
  __shared__ float sW[2][kBC][K], sKt[2][kBC][K], sQg[2][kBC][K];
  __shared__ float sAq[2][kBC][kBC], sdO[2][kBC][kBC], sGc[2][K], sD[kBC][kBC];
  const int tid = threadIdx.x;
  const int cr = tid / 2, j0 = (tid % 2) * 8;
  const TO* d_o = static_cast<const TO*>(p.d_o);
  for (int e = tid; e < K * kBC; e += kBThreads) {
    const int c = e / kBC, j = e % kBC;
    S[c][j] = p.d_final ? p.d_final[s.state * K * V + c * V + tile * kBC + j] : 0.f;
  }
  auto rec = [&](int64_t n) { return p.rec + ((s.slot0 + n) * p.H + h) * R::kFloats; };
  auto fetch = [&](Stage<K, V, true>& st, int64_t n) {
    const int64_t t0 = s.t0 + n * kBC;
    const int len = (int)min<int64_t>(kBC, (p.packed ? p.segs[sq].len : p.T) - n * kBC);
    const TO* row = d_o + ((s.b * p.T + t0) * p.H + h) * V;
    if constexpr (sizeof(TO) == 4)
      st.fetch(rec(n), tid, tile, reinterpret_cast<const float*>(row), nullptr, p.H * V, len);
    else
      st.fetch(rec(n), tid, tile, nullptr, reinterpret_cast<const uint16_t*>(row), p.H * V, len);
  };
  Stage<K, V, true> st;
  fetch(st, s.n16 - 1);
  st.store(sW[0], sKt[0], sQg[0], nullptr, sAq[0], sGc[0], sdO[0], tid);
  __syncthreads();
  for (int64_t m = 0; m < s.n16; ++m) {
    const int64_t n = s.n16 - 1 - m;
    const int cur = (int)(m & 1);
    if (n > 0) fetch(st, n - 1);
    float* dhs = p.dhs + ((s.slot0 + n) * p.H + h) * K * V + tile * kBC;
    for (int e = tid; e < K * kBC; e += kBThreads) dhs[(e / kBC) * V + e % kBC] = S[e / kBC][e % kBC];
    {
      // dDelta = scale Aqk^T dO + Kt dS'
      const int i = tid / kBC, j = tid % kBC;
      float d = 0.f;
      for (int r = 0; r < kBC; ++r) d += sAq[cur][r][i] * sdO[cur][r][j];
      d *= p.scale;
      for (int c = 0; c < K; ++c) d += sKt[cur][i][c] * S[c][j];
      sD[i][j] = d;
    }
    __syncthreads();
    if (cr < K) {
      // dS = diag(Gamma_C) dS' + scale Qg^T dO - W^T dDelta
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        float a = 0.f, b = 0.f;
        for (int r = 0; r < kBC; ++r) {
          a += sQg[cur][r][cr] * sdO[cur][r][j0 + jj];
          b += sW[cur][r][cr] * sD[r][j0 + jj];
        }
        S[cr][j0 + jj] = sGc[cur][cr] * S[cr][j0 + jj] + p.scale * a - b;
      }
    }
    if (n > 0) st.store(sW[cur ^ 1], sKt[cur ^ 1], sQg[cur ^ 1], nullptr, sAq[cur ^ 1], sGc[cur ^ 1], sdO[cur ^ 1], tid);
    __syncthreads();
  }
  if (p.d_init)
    for (int e = tid; e < K * kBC; e += kBThreads) {
      const int c = e / kBC, j = e % kBC;
      p.d_init[s.state * K * V + c * V + tile * kBC + j] = S[c][j];
    }
}

// ---------------------------------------------------------------- bwd_local
// One workgroup per (chunk, head): every input gradient of the chunk's rows.
// Thread t owns row r = t / 16 and key channels c = t % 16 + 16 m.
template <class TI, class TO, int K, int V>
__global__ __launch_bounds__(kBThreads) void bwd_local_kernel(BwdParams p) {
  using R = BRec<K, V>;
  constexpr int VT = 32;           // value columns per pass over the states
  constexpr int MC = K / kBC;      // key channels per thread
  const int64_t slot = blockIdx.x / p.H, h = blockIdx.x % p.H;
  BSlot si;
  if (!slot_info(p, slot, &si)) return;
  const float* rec = p.rec + (slot * p.H + h) * R::kFloats;
  const float* hS = p.hs + (slot * p.H + h) * K * V;
  const float* dhS = p.dhs + (slot * p.H + h) * K * V;
  __shared__ float sG[kBC][K], sKt[kBC][K], sQg[kBC][K], sW[kBC][K], sKb[kBC][K];
  __shared__ float sk[kBC][K], sq[kBC][K], skf[kBC][K], skb[kBC][K], sqf[kBC][K];
  __shared__ float sU[kBC][V], sv[kBC][V], sdO[kBC][V];
  __shared__ float sHH[2 * K * VT];   // h and dh tiles; afterwards dW, dKt, dQg and dG
  __shared__ float sD[kBC][VT], sdD[kBC][VT];
  __shared__ float sAqk[kBC][kBC + 1], sT[kBC][kBC + 1], sX[kBC][kBC + 1], sdA[kBC][kBC + 1];
  __shared__ float sdAqk[kBC][kBC + 1], sdT[kBC][kBC + 1], sGc[K], sdgc[K], sbeta[kBC];
  static_assert(4 * kBC * K <= 2 * K * VT, "dW, dKt, dQg and dG must fit the state tiles");
  float (*sh)[VT] = reinterpret_cast<float (*)[VT]>(sHH);
  float (*sdh)[VT] = reinterpret_cast<float (*)[VT]>(sHH + K * VT);
  const int tid = threadIdx.x, r = tid / kBC, cc = tid % kBC;
  const TI* q = static_cast<const TI*>(p.q);
  const TI* k = static_cast<const TI*>(p.k);
  const TI* v = static_cast<const TI*>(p.v);
  const TI* beta = static_cast<const TI*>(p.beta);
  const TO* d_o = static_cast<const TO*>(p.d_o);
  const bool unsafe = rec[R::kInfo] != 0.f;
  const int len = si.len, last = len - 1;
  auto tok = [&](int row) { return (si.b * p.T + si.t0 + row) * p.H + h; };

  // ---- the record and the inputs
  for (int e = tid; e < kBC * K; e += kBThreads) {
    const int rr = e / K, c = e % K;
    sG[rr][c] = rec[R::kG + e];
    sKt[rr][c] = rec[R::kKt + e];
    sQg[rr][c] = rec[R::kQg + e];
    sW[rr][c] = rec[R::kW + e];
    sk[rr][c] = rr < len ? ld(k, tok(rr) * K + c) : 0.f;
    sq[rr][c] = rr < len ? ld(q, tok(rr) * K + c) : 0.f;
  }
  for (int e = tid; e < kBC * V; e += kBThreads) {
    const int rr = e / V, j = e % V;
    sU[rr][j] = rec[R::kU + e];
    sv[rr][j] = rr < len ? ld(v, tok(rr) * V + j) : 0.f;
    sdO[rr][j] = rr < len ? ld(d_o, tok(rr) * V + j) : 0.f;
  }
  sAqk[r][cc] = rec[R::kAqk + tid];
  sT[r][cc] = rec[R::kT + tid];
  for (int c = tid; c < K; c += kBThreads) {
    sGc[c] = rec[R::kGc + c];
    sdgc[c] = 0.f;
  }
  if (tid < kBC) sbeta[tid] = tid < len ? ld(beta, tok(tid)) : 0.f;
  __syncthreads();
  // the L2 norm of q and k, 16 lanes per row (norms kept for the chain rule)
  float nq = 1.f, nk = 1.f;
  {
    float sqq = 0.f, skk = 0.f;
    for (int c = cc; c < K; c += kBC) {
      sqq += sq[r][c] * sq[r][c];
      skk += sk[r][c] * sk[r][c];
    }
    sqq = sum16(sqq);
    skk = sum16(skk);
    if (p.l2norm) {
      nq = sqrtf(sqq + 1e-6f);
      nk = sqrtf(skk + 1e-6f);
    }
    for (int c = cc; c < K; c += kBC) {
      sq[r][c] /= nq;
      sk[r][c] /= nk;
    }
  }
  __syncthreads();
  for (int e = tid; e < kBC * K; e += kBThreads) {
    const int rr = e / K, c = e % K;
    const float G = sG[rr][c], G0 = sG[0][c];
    skf[rr][c] = sk[rr][c] * __expf(G - G0);
    skb[rr][c] = unsafe ? 0.f : sk[rr][c] * __expf(G0 - G);
    sqf[rr][c] = sq[rr][c] * __expf(G - G0);
    sKb[rr][c] = sbeta[rr] * sk[rr][c] * __expf(G);
  }

  // ---- passes over the value columns: Delta = U - W h, dDelta = scale Aqk^T dO
  // + Kt dh, and every product that contracts over V
  float aQg[MC] = {}, aKt[MC] = {}, aW[MC] = {};
  float aAqk = 0.f, aT = 0.f, dbv = 0.f;
  for (int j0 = 0; j0 < V; j0 += VT) {
    __syncthreads();
    for (int e = tid; e < K * VT; e += kBThreads) {
      const int c = e / VT, j = e % VT;
      sh[c][j] = hS[c * V + j0 + j];
      sdh[c][j] = dhS[c * V + j0 + j];
    }
    __syncthreads();
    for (int e = tid; e < kBC * VT; e += kBThreads) {
      const int rr = e / VT, j = e % VT;
      float d = sU[rr][j0 + j], dd = 0.f;
      for (int c = 0; c < K; ++c) d -= sW[rr][c] * sh[c][j];
      for (int i = 0; i < kBC; ++i) dd += sAqk[i][rr] * sdO[i][j0 + j];
      dd *= p.scale;
      for (int c = 0; c < K; ++c) dd += sKt[rr][c] * sdh[c][j];
      sD[rr][j] = d;
      sdD[rr][j] = dd;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const int c = cc + kBC * m;
      float x = 0.f, y = 0.f, z = 0.f;
      for (int j = 0; j < VT; ++j) {
        x += sdO[r][j0 + j] * sh[c][j];
        y += sD[r][j] * sdh[c][j];
        z += sdD[r][j] * sh[c][j];
      }
      aQg[m] += p.scale * x;   // dQg = scale dO h^T
      aKt[m] += y;             // dKt = Delta dh^T
      aW[m] -= z;              // dW = -dDelta h^T
    }
    {
      float x = 0.f, y = 0.f;
      for (int j = 0; j < VT; ++j) {
        x += sdO[r][j0 + j] * sD[cc][j];
        y += sdD[r][j] * sbeta[cc] * sv[cc][j0 + j];
      }
      aAqk += p.scale * x;     // dAqk = scale dO Delta^T
      aT += y;                 // dT  = dDelta Vb^T (+ dW Kb^T below)
    }
    // dVb = T^T dDelta: dv = beta dVb, and dbeta gets v . dVb
    for (int jj = cc; jj < VT; jj += kBC) {
      float x = 0.f;
      for (int rr = r; rr < kBC; ++rr) x += sT[rr][r] * sdD[rr][jj];
      if (r < len) p.dv[tok(r) * V + j0 + jj] = sbeta[r] * x;
      dbv += sv[r][j0 + jj] * x;
    }
    for (int c = tid; c < K; c += kBThreads) {
      float x = 0.f;
      for (int j = 0; j < VT; ++j) x += sdh[c][j] * sh[c][j];
      sdgc[c] += x;            // d Gamma_C = rowsum(dh * h)
    }
  }
  __syncthreads();
  float* dWl = sHH;                 // [16][K]
  float* dKtl = sHH + kBC * K;
  float* dQgl = sHH + 2 * kBC * K;
  float* dGl = sHH + 3 * kBC * K;
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    const int c = cc + kBC * m;
    dWl[r * K + c] = aW[m];
    dKtl[r * K + c] = aKt[m];
    dQgl[r * K + c] = aQg[m];
  }
  __syncthreads();
  {
    float x = 0.f;
    for (int c = 0; c < K; ++c) x += dWl[r * K + c] * sKb[cc][c];
    sdT[r][cc] = aT + x;
    sdAqk[r][cc] = r >= cc ? aAqk : 0.f;
  }
  __syncthreads();
  {
    // X = T^T dT
    float x = 0.f;
    for (int a = r; a < kBC; ++a) x += sT[a][r] * sdT[a][cc];
    sX[r][cc] = x;
  }
  __syncthreads();
  {
    // dA = -(T^T dT T^T), strictly lower
    float x = 0.f;
    for (int b = 0; b <= cc; ++b) x += sX[r][b] * sT[cc][b];
    sdA[r][cc] = cc < r ? -x : 0.f;
  }
  __syncthreads();

  // ---- per (row, channel): the terms of A and Aqk back onto q, k and G
  const float br = sbeta[r];
  float dqh[MC], dkh[MC], dbeta_p = 0.f;
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    const int c = cc + kBC * m;
    const float G = sG[r][c], GC = sG[last][c];
    float RA = 0.f, RAq = 0.f, CA = 0.f, CAq = 0.f;
    if (!unsafe) {
      for (int i = 0; i < kBC; ++i) {
        RA += sdA[r][i] * skb[i][c];
        RAq += sdAqk[r][i] * skb[i][c];
        CA += sdA[i][r] * sbeta[i] * skf[i][c];
        CAq += sdAqk[i][r] * sqf[i][c];
      }
      const float fr = __expf(G - sG[0][c]), bk = __expf(sG[0][c] - G);
      RA *= fr;
      RAq *= fr;
      CA *= bk;
      CAq *= bk;
    } else {
      for (int i = 0; i < kBC; ++i) {
        const float e = __expf(G - sG[i][c]), ei = __expf(sG[i][c] - G);
        if (i <= r) {
          RA += sdA[r][i] * sk[i][c] * e;
          RAq += sdAqk[r][i] * sk[i][c] * e;
        }
        if (i >= r) {
          CA += sdA[i][r] * sbeta[i] * sk[i][c] * ei;
          CAq += sdAqk[i][r] * sq[i][c] * ei;
        }
      }
    }
    float dKb = 0.f;
    for (int i = r; i < kBC; ++i) dKb += sT[i][r] * dWl[i * K + c];
    const float e = __expf(G), ec = __expf(GC - G), kh = sk[r][c], qh = sq[r][c];
    const float dQg = dQgl[r * K + c], dKt = dKtl[r * K + c];
    dqh[m] = dQg * e + RAq;
    dkh[m] = dKb * br * e + dKt * ec + br * RA + CA + CAq;
    dbeta_p += kh * e * dKb + kh * RA;
    float dG = dQg * qh * e + dKb * br * kh * e - dKt * kh * ec + br * kh * RA - kh * CA + qh * RAq - kh * CAq;
    if (r == last) {
      float x = 0.f;
      for (int i = 0; i < kBC; ++i) x += dKtl[i * K + c] * sKt[i][c];
      dG += x + sdgc[c] * sGc[c];
    }
    dGl[r * K + c] = r < len ? dG : 0.f;
  }
  // dbeta: the V part and the K part, summed over the row's 16 lanes
  const float db = sum16(dbv + dbeta_p);
  if (cc == 0 && r < len) p.dbeta[tok(r)] = db;
  // dq, dk through the L2 norm: dx = (dx^ - x^ (x^ . dx^)) / n
  float pq = 0.f, pk = 0.f;
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    pq += sq[r][cc + kBC * m] * dqh[m];
    pk += sk[r][cc + kBC * m] * dkh[m];
  }
  pq = sum16(pq);
  pk = sum16(pk);
  if (r < len) {
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const int c = cc + kBC * m;
      const float dq = p.l2norm ? (dqh[m] - sq[r][c] * pq) / nq : dqh[m];
      const float dk = p.l2norm ? (dkh[m] - sk[r][c] * pk) / nk : dkh[m];
      p.dq[tok(r) * K + c] = dq;
      p.dk[tok(r) * K + c] = dk;
    }
  }
  __syncthreads();
  // dg = reverse in-chunk cumsum of dG
  for (int c = tid; c < K; c += kBThreads) {
    float run = 0.f;
    for (int rr = last; rr >= 0; --rr) {
      run += dGl[rr * K + c];
      p.dg[tok(rr) * K + c] = run;
    }
  }
}

template <class TI, class TO, int K, int V>
hipError_t launch_bwd_t(const BwdArgs& a) {
  BwdParams p{};
  p.B = a.B; p.T = a.T; p.H = a.H;
  p.nc64 = a.nc_fixed;
  p.packed = a.n_max > 0;
  p.n_max = a.n_max;
  p.l2norm = a.l2norm;
  p.scale = a.scale;
  p.hdr = a.hdr; p.segs = a.segs; p.chunks = a.chunks;
  p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta; p.d_o = a.d_o;
  p.init = a.init; p.d_final = a.d_final;
  p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dg = a.dg; p.dbeta = a.dbeta; p.d_init = a.d_init;
  p.rec = a.rec; p.hs = a.hs; p.dhs = a.dhs;
  const int64_t slots = 4 * a.cmax;
  const dim3 blk(kBThreads);
  hipLaunchKernelGGL((bwd_chunk_kernel<TI, K, V>), dim3((unsigned)(slots * a.H)), blk, 0, a.stream, p);
  const int64_t seqs = (p.packed ? a.smax : a.B) * a.H * (V / kBC);
  hipLaunchKernelGGL((bwd_states_kernel<K, V>), dim3((unsigned)seqs), blk, 0, a.stream, p);
  hipLaunchKernelGGL((bwd_dstates_kernel<TO, K, V>), dim3((unsigned)seqs), blk, 0, a.stream, p);
  hipLaunchKernelGGL((bwd_local_kernel<TI, TO, K, V>), dim3((unsigned)(slots * a.H)), blk, 0, a.stream, p);
  return hipGetLastError();
}

template <class TI, class TO>
hipError_t launch_bwd_kv(const BwdArgs& a) {
  if (a.K == 64 && a.V == 64) return launch_bwd_t<TI, TO, 64, 64>(a);
  if (a.K == 64 && a.V == 128) return launch_bwd_t<TI, TO, 64, 128>(a);
  if (a.K == 128 && a.V == 64) return launch_bwd_t<TI, TO, 128, 64>(a);
  if (a.K == 128 && a.V == 128) return launch_bwd_t<TI, TO, 128, 128>(a);
  return hipErrorInvalidValue;
}

}  // namespace

int64_t bwd_record_floats(int64_t K, int64_t V) {
  if (K == 64 && V == 64) return BRec<64, 64>::kFloats;
  if (K == 64 && V == 128) return BRec<64, 128>::kFloats;
  if (K == 128 && V == 64) return BRec<128, 64>::kFloats;
  return BRec<128, 128>::kFloats;
}

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.in == InType::BF16)
    return a.do_bf16 ? launch_bwd_kv<uint16_t, uint16_t>(a) : launch_bwd_kv<uint16_t, float>(a);
  return a.do_bf16 ? launch_bwd_kv<float, uint16_t>(a) : launch_bwd_kv<float, float>(a);
}

}  // namespace kda
