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
// gate's [-5, 0), or without it) takes exp(G_r - G_i) per element.  The
// result does not depend on the chunk size.  Everything is fp32 (bf16 inputs
// are exact in fp32), the products on fp32 matrix-core tiles.
//
// Kernels, in order: bwd_chunk (one workgroup per chunk and head: G, A, Aqk,
// T, W, U, Kt, Qg into a chunk record), bwd_states (the forward recurrence
// again, keeping the state entering every 64-token chunk and Delta of every
// chunk), bwd_dstates
// (the reverse recurrence, keeping dS' and dDelta of every chunk and the
// initial-state gradients), bwd_local (one workgroup per chunk and head: all
// input gradients).
#include <type_traits>
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kBC = 16;            // rows per backward chunk
constexpr int kBThreads = 256;
// The recurrences: four compute waves and the waves filling their operand
// ring (two for the states, three for their gradients).  One wave moves
// about 10 bytes per clock from L2 into LDS, so a single one set the pace of
// every chunk.
constexpr int kStatesThreads = 6 * kWave, kDStatesThreads = 7 * kWave;
constexpr float kSpanMax = 64.f;   // exp(64) ~ 6e27: room for sums of O(1e10) below FLT_MAX
constexpr int kTP = 20;            // LDS row stride of 16x16 tiles (bank-conflict free fragment reads)

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
  float* hs;                    // [slots / 4][H][K][V] state entering each 64-token chunk
  float* dhs;                   // [slots][H][K][V] dL/d(state leaving each chunk)
  float* ds;                    // [slots][H][16][V] Delta of each chunk
  float* dds;                   // [slots][H][16][V] dDelta of each chunk
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
    if (s->b >= p.B || s->t0 >= p.T) return false;
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

// fp32 matrix-core tiles (v_mfma_f32_16x16x4_f32).  A 16-deep slab of a
// product C (16x16) += A (16x16) B (16x16) is four instructions: for the j-th,
// lane l = 16 g + n supplies A[n][4g + j] and B[4g + j][n], so one f32x4 per
// operand and lane covers the slab.  The accumulator lane l holds C[4g + i][n]
// (i = 0..3), which is also the B operand of a 16-deep slab over its rows.
__device__ __forceinline__ void mma16(f32x4& c, const f32x4& a, const f32x4& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
}
// A operand of a row-major X (rows m0.., k = k0 + 4g + j); also the B operand
// of X^T (cols m0..).
__device__ __forceinline__ f32x4 opa(const float* X, int ld, int m0, int k0, int lane) {
  return *reinterpret_cast<const f32x4*>(X + (int64_t)(m0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4));
}
// B operand of a row-major Y (k = k0 + 4g + j, cols n0..); also the A operand
// of Y^T (rows n0..).
__device__ __forceinline__ f32x4 opb(const float* Y, int ld, int k0, int n0, int lane) {
  const float* q = Y + (int64_t)(k0 + 4 * (lane >> 4)) * ld + n0 + (lane & 15);
  return f32x4{q[0], q[ld], q[2 * ld], q[3 * ld]};
}

// Rows 0..15 of a [rows][W] input (row r at src + r * row_stride elements)
// into fp32 LDS rows of stride LD, zero past len: 16-byte loads (eight bf16
// or four fp32 per lane) instead of one element per lane.
__device__ __forceinline__ void cvt16(const uint16_t* src, float* x) {
  const uint4 u = *reinterpret_cast<const uint4*>(src);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void cvt16(const float* src, float* x) {
  const f32x4 u = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = u[i];
}
template <int W, int LD, class T>
__device__ __forceinline__ void load_rows(float* dst, const T* src, int64_t row_stride, int len, int tid,
                                          const float* div = nullptr) {
  constexpr int E = 16 / (int)sizeof(T), PER_ROW = W / E;
  for (int e = tid; e < kBC * PER_ROW; e += kBThreads) {
    const int r = e / PER_ROW, c = (e % PER_ROW) * E;
    float x[E];
    if (r < len) {
      cvt16(src + r * row_stride + c, x);
      if (div)   // each row divided by its own factor
#pragma unroll
        for (int i = 0; i < E; ++i) x[i] /= div[r];
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) x[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < E; i += 4) *reinterpret_cast<f32x4*>(dst + r * LD + c + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
  }
}

// ---------------------------------------------------------------- bwd_chunk
// One workgroup (four waves) per (chunk, head): the chunk quantities into
// the chunk record.  A = beta (kf kb^T) and Aqk = qf kb^T with kf = k exp(G -
// G_0), kb = k exp(G_0 - G), qf = q exp(G - G_0) (or exp(G_r - G_i) per
// element past the span limit), T = (I + A)^-1 = (I - A)(I + A^2)(I + A^4)
// (I + A^8) (A is strictly lower, so A^16 = 0), W = T Kb, U = T Vb: all on
// fp32 matrix-core tiles, 16x16 intermediates through LDS.
template <class TI, int K, int V>
__global__ __launch_bounds__(kBThreads) void bwd_chunk_kernel(BwdParams p) {
  using R = BRec<K, V>;
  constexpr int NKB = K / 16, NVB = V / 16;
  // Rows padded by four floats, 16x16 tiles to a stride of 20: the fragment
  // reads (one row per lane, or four rows per lane group) then fall on
  // distinct banks.
  constexpr int KP = K + 4, VP = V + 4, TP = kTP;
  const int64_t slot = blockIdx.x / p.H, h = blockIdx.x % p.H;
  BSlot si;
  if (!slot_info(p, slot, &si)) return;
  __shared__ __align__(16) float sk[kBC][KP], sq[kBC][KP], sG[kBC][KP], sv[kBC][VP];
  __shared__ __align__(16) float sA[kBC][TP], sP1[kBC][TP], sP2[kBC][TP], sT[kBC][TP];
  __shared__ float sbeta[kBC];
  __shared__ int s_unsafe;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = 4 * (lane >> 4), n = lane & 15;
  const TI* q = static_cast<const TI*>(p.q);
  const TI* k = static_cast<const TI*>(p.k);
  const TI* v = static_cast<const TI*>(p.v);
  const TI* g = static_cast<const TI*>(p.g);
  const TI* beta = static_cast<const TI*>(p.beta);
  float* rec = p.rec + (slot * p.H + h) * R::kFloats;
  if (tid == 0) s_unsafe = 0;
  {
    const int64_t t0 = (si.b * p.T + si.t0) * p.H + h;   // first row's token index (times H, plus h)
    load_rows<K, KP>(&sk[0][0], k + t0 * K, p.H * K, si.len, tid);
    load_rows<K, KP>(&sq[0][0], q + t0 * K, p.H * K, si.len, tid);
    load_rows<K, KP>(&sG[0][0], g + t0 * K, p.H * K, si.len, tid);
    load_rows<V, VP>(&sv[0][0], v + t0 * V, p.H * V, si.len, tid);
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
    const float G = sG[r][c], GC = sG[last][c];
    rec[R::kG + e] = G;
    rec[R::kKt + e] = sk[r][c] * __expf(GC - G);
    rec[R::kQg + e] = sq[r][c] * __expf(G);
    if (r == 0) rec[R::kGc + c] = __expf(GC);
  }
  __syncthreads();
  if (wave < 2) {
    // wave 0: A, wave 1: Aqk (contraction over K)
    f32x4 c = {0, 0, 0, 0};
    if (!unsafe) {
      // operands formed on the fly: left = (k | q) exp(G - G_0), right kb = k exp(G_0 - G)
      const float* left = wave == 0 ? &sk[0][0] : &sq[0][0];
#pragma unroll 4
      for (int s = 0; s < NKB; ++s) {
        const f32x4 x = opa(left, KP, 0, 16 * s, lane), kk = opa(&sk[0][0], KP, 0, 16 * s, lane);
        const f32x4 gr = opa(&sG[0][0], KP, 0, 16 * s, lane), g0 = opa(&sG[0][0], 0, 0, 16 * s, lane);
        f32x4 a, b;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a[j] = x[j] * __expf(gr[j] - g0[j]);
          b[j] = kk[j] * __expf(g0[j] - gr[j]);
        }
        mma16(c, a, b);
      }
    } else {
      const float* left = wave == 0 ? &sk[0][0] : &sq[0][0];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = g4 + i;
        float x = 0.f;
        if (n <= r)
          for (int cc = 0; cc < K; ++cc) x += left[r * KP + cc] * sk[n][cc] * __expf(sG[r][cc] - sG[n][cc]);
        c[i] = x;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = g4 + i;
      if (wave == 0) sA[r][n] = n < r ? sbeta[r] * c[i] : 0.f;
      else rec[R::kAqk + r * kBC + n] = n <= r ? c[i] : 0.f;
    }
  }
  // Kb = diag(beta) (K * Gamma) in place of q, which A and Aqk no longer need
  __syncthreads();
  for (int e = tid; e < kBC * K; e += kBThreads) {
    const int r = e / K, c = e % K;
    sq[r][c] = sbeta[r] * sk[r][c] * __expf(sG[r][c]);
  }
  if (wave == 0) {
    // T = (I - A)(I + A^2)(I + A^4)(I + A^8): squares and products, one wave
    auto mul = [&](const float (*X)[TP], const float (*Y)[TP]) {
      f32x4 c = {0, 0, 0, 0};
      mma16(c, opa(&X[0][0], TP, 0, 0, lane), opb(&Y[0][0], TP, 0, 0, lane));
      return c;
    };
    auto put = [&](float (*X)[TP], const f32x4& c, float diag) {
#pragma unroll
      for (int i = 0; i < 4; ++i) X[g4 + i][n] = c[i] + (g4 + i == n ? diag : 0.f);
    };
    // sP1 = A^2; sT = I - A; sP2 = (I - A)(I + A^2)
    put(sP1, mul(sA, sA), 0.f);
#pragma unroll
    for (int i = 0; i < 4; ++i) sT[g4 + i][n] = (g4 + i == n ? 1.f : 0.f) - sA[g4 + i][n];
    lds_wait();
    {
      f32x4 c = mul(sT, sP1);   // (I - A) A^2
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] += sT[g4 + i][n];
      put(sP2, c, 0.f);         // (I - A)(I + A^2)
    }
    lds_wait();
    put(sA, mul(sP1, sP1), 0.f);   // A^4 (A no longer needed)
    lds_wait();
    {
      f32x4 c = mul(sP2, sA);   // X (A^4)
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] += sP2[g4 + i][n];
      put(sT, c, 0.f);          // X (I + A^4)
    }
    lds_wait();
    put(sP1, mul(sA, sA), 0.f);    // A^8
    lds_wait();
    {
      f32x4 c = mul(sT, sP1);
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] += sT[g4 + i][n];
      lds_wait();
      put(sT, c, 0.f);          // T
    }
  }
  __syncthreads();
  rec[R::kT + tid] = sT[tid / kBC][tid % kBC];
  // W = T Kb, U = T Vb: K/16 + V/16 output tiles, taken by the waves in
  // pairs of adjacent column blocks and stored through an LDS tile of 16 x 32
  // (k's and G's buffers are free by now; row stride 36 keeps both sides free
  // of bank conflicts), so that each lane stores 16 bytes and each
  // instruction whole 128-byte lines.  Stored straight from the accumulator
  // layout, each wave wrote half lines that another wave completed, which
  // cost this kernel about a third of its time.
  constexpr int NP = (NKB + NVB) / 2, SL = 2 * kBC + 4;
  constexpr bool kAlias = 2 * kBC * SL <= kBC * KP;
  __shared__ __align__(16) float sStage[kAlias ? 4 : 4 * kBC * SL];
  float* stage = kAlias ? (wave < 2 ? &sk[0][0] : &sG[0][0]) + (wave & 1) * (kBC * SL) : sStage + wave * (kBC * SL);
  for (int pr = wave; pr < NP; pr += 4) {
    const bool isW = pr < NKB / 2;
    const int t0 = isW ? 2 * pr : 2 * (pr - NKB / 2);   // first column block of the pair
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x4 c = {0, 0, 0, 0};
      if (isW) {
        mma16(c, opa(&sT[0][0], TP, 0, 0, lane), opb(&sq[0][0], KP, 0, 16 * (t0 + h2), lane));
      } else {
        f32x4 b = opb(&sv[0][0], VP, 0, 16 * (t0 + h2), lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] *= sbeta[g4 + j];
        mma16(c, opa(&sT[0][0], TP, 0, 0, lane), b);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) stage[(g4 + i) * SL + 16 * h2 + n] = c[i];
    }
    float* dst = rec + (isW ? R::kW : R::kU) + 16 * t0;
    const int ldr = isW ? K : V;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = (lane >> 3) + 8 * hh, c4 = 4 * (lane & 7);
      *reinterpret_cast<f32x4*>(dst + r * ldr + c4) = *reinterpret_cast<const f32x4*>(stage + r * SL + c4);
    }
  }
  if (tid == 0) rec[R::kInfo] = unsafe ? 1.f : 0.f;
}

// ------------------------------------------------- recurrence operand ring
// The recurrences read each chunk's operands from an LDS image that the
// workgroup's fill waves load with direct-to-LDS loads LEAD chunks ahead,
// so the compute waves issue no global loads in their loop.  Images of
// [16][K] operands store 16-byte unit u of row r at unit u ^ (r & 15): the
// fragment reads (a row of four columns per lane, or four rows of one column
// per lane group) then fall on distinct banks.
__device__ __forceinline__ int swz(int r, int u) { return u ^ (r & 15); }

// One wave: rows 0..15 of a row-major [16][K] fp32 operand into an image.
template <int K>
__device__ __forceinline__ void dma_rows(float* dst, const float* src, int lane) {
  constexpr int UPR = K / 4;   // 16-byte units per row
#pragma unroll
  for (int i = 0; i < K / 16; ++i) {
    const int pos = 64 * i + lane, r = pos / UPR;
    dma16(dst + 256 * i, src + r * K + 4 * swz(r, pos % UPR));
  }
}
// Images of [16][16] blocks hold row r at position 4 (r & 3) + (r >> 2): a
// lane group's four rows 4g + i then lie 16 banks apart.
__device__ __forceinline__ int blk_pos(int r) { return 4 * (r & 3) + (r >> 2); }
// One wave: a [16][16] fp32 block (row stride ld) into such an image (lane l
// fills position l / 4, the inverse of blk_pos being the same permutation).
__device__ __forceinline__ void dma_block16(float* dst, const float* src, int ld, int lane) {
  dma16(dst, src + blk_pos(lane >> 2) * ld + 4 * (lane & 3));
}
// Fragments of an image: A operand of X (16 x K image), rows 0..15, k = 16 cb
// + 4g + j; and B operand of X (k = 4g + j, columns 16 cb ..), i.e. the A
// operand of X^T.
template <int K>
__device__ __forceinline__ f32x4 img_opa(const float* X, int cb, int lane) {
  const int n = lane & 15;
  return *reinterpret_cast<const f32x4*>(X + n * K + 4 * swz(n, 4 * cb + (lane >> 4)));
}
template <int K>
__device__ __forceinline__ f32x4 img_opb(const float* X, int cb, int lane) {
  const int n = lane & 15, g4 = 4 * (lane >> 4);
  f32x4 x;
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = X[(g4 + j) * K + 4 * swz(g4 + j, 4 * cb + (n >> 2)) + (n & 3)];
  return x;
}

// Allow n (0 .. LEAD - 1, wave-uniform) chunks of PER direct loads each to
// stay outstanding.
template <int PER, int LEAD>
__device__ __forceinline__ void wait_chunks(int64_t n) {
  static_assert(LEAD >= 2 && LEAD <= 4 && (LEAD - 1) * PER < 64, "vmcnt is six bits");
  if constexpr (LEAD >= 4) {
    if (n >= 3) return vm_wait<3 * PER>();
  }
  if constexpr (LEAD >= 3) {
    if (n >= 2) return vm_wait<2 * PER>();
  }
  if (n >= 1) vm_wait<PER>();
  else vm_wait<0>();
}

// A fill wave: issue(c) loads its part of chunk c's image (PER direct loads)
// into slot c % LEAD.  Chunk
// c + 1 is complete before barrier c (the compute waves read it right after),
// and chunk c + LEAD is issued after it, into the slot of chunk c, which no
// wave reads past barrier c.  One barrier precedes the loop (chunk 0 ready).
template <int PER, int LEAD, class IssueFn>
__device__ void ring_fill(IssueFn issue, int64_t n) {
  for (int64_t c = 0; c < LEAD && c < n; ++c) issue(c);
  wait_chunks<PER, LEAD>(min<int64_t>(LEAD, n) - 1);
  block_sync();
  for (int64_t c = 0; c < n; ++c) {
    wait_chunks<PER, LEAD>(max<int64_t>(0, min<int64_t>(c + LEAD, n) - (c + 2)));
    block_sync();
    if (c + LEAD < n) issue(c + LEAD);
  }
  vm_wait<0>();
}

// A wave stores an accumulator tile (lane (g, n) holding rows 4g + i, column
// n) to a row-major matrix with row stride ld: through a padded LDS tile of
// its own, so that each lane writes one 16-byte piece of a row (one
// instruction instead of four).  Row stride 20 keeps both the scattered
// writes and the 16-byte reads free of bank conflicts.
constexpr int kTileLd = kTP;
__device__ __forceinline__ void store_tile(float* dst, int64_t ld, const f32x4& c, float* lds, int lane) {
  const int g4 = 4 * (lane >> 4), n = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) lds[(g4 + i) * kTileLd + n] = c[i];
  const int r = lane >> 2, q4 = 4 * (lane & 3);
  const f32x4 x = *reinterpret_cast<const f32x4*>(lds + r * kTileLd + q4);
  *reinterpret_cast<f32x4*>(dst + r * ld + q4) = x;
}

// ---------------------------------------------------------------- bwd_states
// One workgroup (four compute waves and the ring's fill waves) per (sequence, head,
// 16 value columns): the state from the initial state through every chunk,
// writing the state that enters each 64-token chunk (the local kernel
// rebuilds the three after it) and Delta of every chunk.  The 16-column
// state is K/16 accumulator tiles; wave w holds tiles w, w + 4 (rows
// 16 cb ..), which are also the B operands of its slabs of W S.  Per chunk: each wave's partial
// W S goes through LDS (double buffered, one barrier), every wave sums the
// four in the same order into Delta = U - W S, and updates its tiles
// S <- diag(Gamma_C) S + Kt^T Delta.  Operands of chunk c + 1 are read from
// the ring into registers right after barrier c.
template <int K, int V>
struct StatesImg {
  float w[kBC * K], kt[kBC * K], gc[K], u[kBC * kBC];
  static constexpr int kLead = 4;                 // images in flight (ring slots)
};

template <int K, int V>
struct StatesOps {
  static constexpr int TPW = K / 64;   // state tiles per wave
  f32x4 w[TPW], kt[TPW], gc[TPW], u;
  __device__ void load(const StatesImg<K, V>& m, int wave, int lane) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int cb = wave + 4 * t;
      w[t] = img_opa<K>(m.w, cb, lane);                  // W[n][16 cb + 4g + j]
      kt[t] = img_opb<K>(m.kt, cb, lane);                // (Kt^T)[16 cb + n][4g + j]
      gc[t] = *reinterpret_cast<const f32x4*>(m.gc + 16 * cb + 4 * (lane >> 4));
    }
    const int g4 = 4 * (lane >> 4), n = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = m.u[blk_pos(g4 + i) * kBC + n];
  }
};

template <int K, int V>
__global__ __launch_bounds__(kStatesThreads) void bwd_states_kernel(BwdParams p) {
  using R = BRec<K, V>;
  using Img = StatesImg<K, V>;
  using Ops = StatesOps<K, V>;
  constexpr int NV = V / kBC, TPW = Ops::TPW;
  // The NV workgroups of one (sequence, head) get ids of equal id % 8, which
  // the dispatcher places on one XCD: they share its L2 copy of the records.
  const int64_t id = blockIdx.x;
  const int tile = (int)((id / 8) % NV);
  const int64_t sh = (id / (8 * NV)) * 8 + id % 8, h = sh % p.H, sq = sh / p.H;
  BSeq s;
  if (!seq_info(p, sq, h, &s)) return;
  __shared__ __align__(16) Img ring[Img::kLead];
  __shared__ __align__(16) float sP[2][4][kBC][kTP];
  __shared__ __align__(16) float sX[4][TPW][kBC * kTileLd];   // per-wave store staging
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = 4 * (lane >> 4), n = lane & 15;
  auto rec = [&](int64_t c) { return p.rec + ((s.slot0 + c) * p.H + h) * R::kFloats; };
  if (wave == 4) {   // W and exp(G_C): K/16 + 1 loads a chunk (lane 0 always issues)
    ring_fill<K / 16 + 1, Img::kLead>(
        [&](int64_t c) {
          Img& m = ring[c % Img::kLead];
          dma_rows<K>(m.w, rec(c) + R::kW, lane);
          if (lane < K / 4) dma16(m.gc, rec(c) + R::kGc + 4 * lane);
        },
        s.n16);
    return;
  }
  if (wave == 5) {   // Kt and the workgroup's 16 columns of U: K/16 + 1 loads a chunk
    ring_fill<K / 16 + 1, Img::kLead>(
        [&](int64_t c) {
          Img& m = ring[c % Img::kLead];
          dma_rows<K>(m.kt, rec(c) + R::kKt, lane);
          dma_block16(m.u, rec(c) + R::kU + tile * kBC, V, lane);
        },
        s.n16);
    return;
  }
  f32x4 st[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st[t][i] = p.init ? p.init[s.state * K * V + (int64_t)(16 * (wave + 4 * t) + g4 + i) * V + tile * kBC + n] : 0.f;
  auto step = [&](int64_t c, const Ops& cur, Ops& next) {
    if ((c & 3) == 0) {   // checkpoint: the state entering a 64-token chunk (slot0 is a multiple of 4)
      float* hs = p.hs + (((s.slot0 + c) >> 2) * p.H + h) * K * V + tile * kBC;
#pragma unroll
      for (int t = 0; t < TPW; ++t) store_tile(hs + (int64_t)16 * (wave + 4 * t) * V, V, st[t], sX[wave][t], lane);
    }
    f32x4 d = {0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < TPW; ++t) mma16(d, cur.w[t], st[t]);
    const int buf = (int)(c & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) sP[buf][wave][g4 + i][n] = d[i];
    block_sync();
    f32x4 delta;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      delta[i] = cur.u[i] - (sP[buf][0][g4 + i][n] + sP[buf][1][g4 + i][n] + sP[buf][2][g4 + i][n] +
                             sP[buf][3][g4 + i][n]);
    if (c + 1 < s.n16) next.load(ring[(c + 1) % Img::kLead], wave, lane);
    if (wave == 0) {
      float* dst = p.ds + ((s.slot0 + c) * p.H + h) * kBC * V + tile * kBC + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(g4 + i) * V] = delta[i];
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = cur.gc[t][i] * st[t][i];
      mma16(x, cur.kt[t], delta);
      st[t] = x;
    }
  };
  Ops o0, o1;
  block_sync();
  if (s.n16 > 0) o0.load(ring[0], wave, lane);
  for (int64_t c = 0; c < s.n16; c += 2) {
    step(c, o0, o1);
    if (c + 1 < s.n16) step(c + 1, o1, o0);
  }
}

// ---------------------------------------------------------------- bwd_dstates
// One workgroup (four compute waves and the ring's fill waves) per (sequence, head,
// 16 value columns): dS' from the final state's gradient back through every
// chunk, writing dS' of each chunk and the gradient of the sequence's
// initial state.  Same tiling as bwd_states: per chunk the waves' partial
// Kt dS' (and scale Aqk^T dO, added by wave 0) are summed into dDelta through
// LDS, then each wave updates its tiles dS = diag(Gamma_C) dS' + scale Qg^T dO
// - W^T dDelta.  The ring holds the chunk's Kt, Qg, W, Gamma_C, Aqk and the
// workgroup's 16 columns of the chunk's dO rows.
template <class TO, int K, int V>
struct DStatesImg {
  float kt[kBC * K], qg[kBC * K], w[kBC * K], gc[K], aq[kBC * kBC];
  TO dout[kBC * kBC];
  static constexpr int kLead = 4;
};

template <int K, int V>
struct DStatesOps {
  static constexpr int TPW = K / 64;
  f32x4 kt[TPW], qgt[TPW], wt[TPW], gc[TPW], aq, dout;
  template <class TO>
  __device__ void load(const DStatesImg<TO, K, V>& m, int len, int wave, int lane) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int cb = wave + 4 * t;
      kt[t] = img_opa<K>(m.kt, cb, lane);                // Kt[n][16 cb + 4g + j]
      qgt[t] = img_opb<K>(m.qg, cb, lane);               // (Qg^T)[16 cb + n][4g + j]
      wt[t] = img_opb<K>(m.w, cb, lane);                 // (W^T)[16 cb + n][4g + j]
      gc[t] = *reinterpret_cast<const f32x4*>(m.gc + 16 * cb + 4 * (lane >> 4));
    }
    const int g4 = 4 * (lane >> 4), n = lane & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      aq[j] = m.aq[blk_pos(g4 + j) * kBC + n];             // (Aqk^T)[n][4g + j]
      dout[j] = g4 + j < len ? ld(m.dout, blk_pos(g4 + j) * kBC + n) : 0.f;
    }
  }
};

template <class TO, int K, int V>
__global__ __launch_bounds__(kDStatesThreads) void bwd_dstates_kernel(BwdParams p) {
  using R = BRec<K, V>;
  using Img = DStatesImg<TO, K, V>;
  using Ops = DStatesOps<K, V>;
  constexpr int NV = V / kBC, TPW = Ops::TPW;
  // The NV workgroups of one (sequence, head) get ids of equal id % 8, which
  // the dispatcher places on one XCD: they share its L2 copy of the records.
  const int64_t id = blockIdx.x;
  const int tile = (int)((id / 8) % NV);
  const int64_t sh = (id / (8 * NV)) * 8 + id % 8, h = sh % p.H, sq = sh / p.H;
  BSeq s;
  if (!seq_info(p, sq, h, &s)) return;
  __shared__ __align__(16) Img ring[Img::kLead];
  __shared__ __align__(16) float sP[2][4][kBC][kTP];
  __shared__ __align__(16) float sX[4][TPW][kBC * kTileLd];   // per-wave store staging
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g4 = 4 * (lane >> 4), n = lane & 15;
  const TO* d_o = static_cast<const TO*>(p.d_o);
  const int64_t seq_len = p.packed ? p.segs[sq].len : p.T;
  // Step m handles chunk n16 - 1 - m.
  auto chunk_len = [&](int64_t c) { return (int)min<int64_t>(kBC, seq_len - c * kBC); };
  // step m's image holds chunk n16 - 1 - m
  auto rec = [&](int64_t m) { return p.rec + ((s.slot0 + s.n16 - 1 - m) * p.H + h) * R::kFloats; };
  if (wave == 4) {   // Kt: K/16 loads a chunk
    ring_fill<K / 16, Img::kLead>([&](int64_t m) { dma_rows<K>(ring[m % Img::kLead].kt, rec(m) + R::kKt, lane); },
                                  s.n16);
    return;
  }
  if (wave == 5) {   // Qg: K/16 loads a chunk
    ring_fill<K / 16, Img::kLead>([&](int64_t m) { dma_rows<K>(ring[m % Img::kLead].qg, rec(m) + R::kQg, lane); },
                                  s.n16);
    return;
  }
  if (wave == 6) {   // W, exp(G_C), Aqk and the dO columns: K/16 + 3 loads a chunk
    ring_fill<K / 16 + 3, Img::kLead>(
        [&](int64_t m) {
          Img& im = ring[m % Img::kLead];
          const int64_t c = s.n16 - 1 - m;
          const float* r = rec(m);
          dma_rows<K>(im.w, r + R::kW, lane);
          if (lane < K / 4) dma16(im.gc, r + R::kGc + 4 * lane);   // lane 0 always issues
          dma_block16(im.aq, r + R::kAqk, kBC, lane);
          // 16 columns of each present dO row, LPR lanes of 16 bytes a row,
          // rows permuted as in every [16][16] image
          constexpr int LPR = kBC * (int)sizeof(TO) / 16;
          const int row = lane / LPR < kBC ? blk_pos(lane / LPR) : kBC;
          if (row < chunk_len(c))   // row 0 (position 0) always present: every chunk issues its loads
            dma16(im.dout, d_o + ((s.b * p.T + s.t0 + c * kBC + row) * p.H + h) * V + tile * kBC +
                               (lane % LPR) * (16 / (int)sizeof(TO)));
        },
        s.n16);
    return;
  }
  f32x4 st[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st[t][i] = p.d_final ? p.d_final[s.state * K * V + (int64_t)(16 * (wave + 4 * t) + g4 + i) * V + tile * kBC + n]
                           : 0.f;
  auto step = [&](int64_t m, const Ops& cur, Ops& next) {
    const int64_t c = s.n16 - 1 - m;
    float* dhs = p.dhs + ((s.slot0 + c) * p.H + h) * K * V + tile * kBC;
    f32x4 d = {0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      store_tile(dhs + (int64_t)16 * (wave + 4 * t) * V, V, st[t], sX[wave][t], lane);
      mma16(d, cur.kt[t], st[t]);
    }
    if (wave == 0) {
      f32x4 e = {0, 0, 0, 0};
      mma16(e, cur.aq, cur.dout);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] += p.scale * e[i];
    }
    const int buf = (int)(m & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) sP[buf][wave][g4 + i][n] = d[i];
    block_sync();
    f32x4 dd;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dd[i] = sP[buf][0][g4 + i][n] + sP[buf][1][g4 + i][n] + sP[buf][2][g4 + i][n] + sP[buf][3][g4 + i][n];
    if (m + 1 < s.n16) next.load(ring[(m + 1) % Img::kLead], chunk_len(c - 1), wave, lane);
    if (wave == 0) {
      float* dst = p.dds + ((s.slot0 + c) * p.H + h) * kBC * V + tile * kBC + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(g4 + i) * V] = dd[i];
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      f32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
      mma16(a, cur.qgt[t], cur.dout);
      mma16(b, cur.wt[t], dd);
#pragma unroll
      for (int i = 0; i < 4; ++i) st[t][i] = cur.gc[t][i] * st[t][i] + p.scale * a[i] - b[i];
    }
  };
  Ops o0, o1;
  block_sync();
  if (s.n16 > 0) o0.load(ring[0], chunk_len(s.n16 - 1), wave, lane);
  for (int64_t m = 0; m < s.n16; m += 2) {
    step(m, o0, o1);
    if (m + 1 < s.n16) step(m + 1, o1, o0);
  }
  if (p.d_init)
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p.d_init[s.state * K * V + (int64_t)(16 * (wave + 4 * t) + g4 + i) * V + tile * kBC + n] = st[t][i];
}

// ---------------------------------------------------------------- bwd_local
// One workgroup (four waves) per (chunk, head): every input gradient of the
// chunk's rows.  Delta and dDelta come from the recurrences; the state h
// entering the chunk is rebuilt per 16x16 tile from the state entering its
// 64-token chunk and the updates of the 16-token chunks before it there.
// Phase B (contraction over V; wave w takes key blocks w, w + 4, ...): dQg =
// scale dO h^T, dKt = Delta dh^T, dW = -dDelta h^T and d Gamma_C =
// rowsum(dh * h); besides, wave 0 dAqk = scale dO Delta^T, wave 1
// dT = dDelta Vb^T, waves 2-3 dVb = T^T dDelta (dv, and dbeta's V part).
// Phase C: dT += dW Kb^T, dA = -T^T dT T^T.  Phase D (key blocks again): dKb =
// T^T dW and the exponent-factor sums of A and Aqk, assembled per (row,
// channel) into dq, dk, dbeta and dG; dg = reverse in-chunk cumsum of dG.
template <class TI, class TO, int K, int V>
__global__ __launch_bounds__(kBThreads) __attribute__((amdgpu_waves_per_eu(3))) void bwd_local_kernel(BwdParams p) {
  using R = BRec<K, V>;
  constexpr int NKB = K / 16, NVB = V / 16, MX = K > V ? K : V;
  // Chunk-major ids: the heads of one chunk are neighbours (their input rows
  // are contiguous), and with H a multiple of 8 the four 16-token chunks of
  // a (64-token chunk, head) land on one XCD, sharing the state they start
  // from in its L2.
  const int64_t slot = blockIdx.x / p.H, h = blockIdx.x % p.H;
  const int sub = (int)(slot & 3);   // the chunk's place in its 64-token chunk
  BSlot si;
  if (!slot_info(p, slot, &si)) return;
  const float* rec = p.rec + (slot * p.H + h) * R::kFloats;
  const float* hS = p.hs + ((slot >> 2) * p.H + h) * K * V;
  const float* dhS = p.dhs + (slot * p.H + h) * K * V;
  __shared__ __align__(16) float sG[kBC][K], sk[kBC][K], sq[kBC][K];
  __shared__ __align__(16) float sVG[kBC * MX];        // v [16][V], then the dT partials, then dG [16][K]
  __shared__ __align__(16) float sOW[kBC * MX];        // dO [16][V], later dW [16][K]
  __shared__ __align__(16) float sT[kBC][kBC], sAqk[kBC][kBC], sdA[kBC][kBC], sdAqk[kBC][kBC], sdT[kBC][kBC];
  __shared__ __align__(16) float sX[kBC][kBC];
  // Per-wave partial sums (one writer each), combined in wave order: no
  // atomics, so every run adds in the same order.
  __shared__ float sdgc[K], sred[4][kBC][4];
  static_assert(4 * kBC * kBC <= kBC * MX, "the dT partials fit v's buffer");
  float (*sdTp)[kBC][kBC] = reinterpret_cast<float (*)[kBC][kBC]>(sVG);
  __shared__ float sbeta[kBC], snq[kBC], snk[kBC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = 4 * (lane >> 4), n = lane & 15;
  const TI* q = static_cast<const TI*>(p.q);
  const TI* k = static_cast<const TI*>(p.k);
  const TI* v = static_cast<const TI*>(p.v);
  const TI* beta = static_cast<const TI*>(p.beta);
  const TO* d_o = static_cast<const TO*>(p.d_o);
  const bool unsafe = rec[R::kInfo] != 0.f;
  const int len = si.len, last = len - 1;
  auto tok = [&](int row) { return (si.b * p.T + si.t0 + row) * p.H + h; };
  float* sv = sVG;
  float* sdO = sOW;
  // Delta and dDelta of the chunk, as the recurrences left them (rows past
  // the chunk are zero).  Every wave reads them for each of its key blocks:
  // with V <= K they are staged for phase B in the buffers of k and q, which
  // phase B does not use (both are loaded again, normalised, after it).
  constexpr bool kStageD = V <= K;
  const float* gD = p.ds + (slot * p.H + h) * kBC * V;
  const float* gdD = p.dds + (slot * p.H + h) * kBC * V;
  const float* sD = kStageD ? &sk[0][0] : gD;
  const float* sdD = kStageD ? &sq[0][0] : gdD;

  // ---- inputs
  {
    const int64_t t0 = tok(0);
    load_rows<K, K>(&sG[0][0], rec + R::kG, K, kBC, tid);
    load_rows<K, K>(&sk[0][0], k + t0 * K, p.H * K, len, tid);
    load_rows<K, K>(&sq[0][0], q + t0 * K, p.H * K, len, tid);
    load_rows<V, V>(sv, v + t0 * V, p.H * V, len, tid);
    load_rows<V, V>(sdO, d_o + t0 * V, p.H * V, len, tid);
  }
  sT[tid / kBC][tid % kBC] = rec[R::kT + tid];
  sAqk[tid / kBC][tid % kBC] = rec[R::kAqk + tid];
  for (int e = tid; e < 4 * kBC * 4; e += kBThreads) (&sred[0][0][0])[e] = 0.f;
  if (tid < kBC) sbeta[tid] = tid < len ? ld(beta, tok(tid)) : 0.f;
  __syncthreads();
  {
    // the L2 norm of q and k, 16 lanes per row
    const int r = tid / kBC, cc = tid % kBC;
    float sqq = 0.f, skk = 0.f;
    for (int c = cc; c < K; c += kBC) {
      sqq += sq[r][c] * sq[r][c];
      skk += sk[r][c] * sk[r][c];
    }
    sqq = sum16(sqq);
    skk = sum16(skk);
    const float nq = p.l2norm ? sqrtf(sqq + 1e-6f) : 1.f, nk = p.l2norm ? sqrtf(skk + 1e-6f) : 1.f;
    if constexpr (!kStageD) {
      for (int c = cc; c < K; c += kBC) {
        sq[r][c] /= nq;
        sk[r][c] /= nk;
      }
    }
    if (cc == 0) {
      snq[r] = nq;
      snk[r] = nk;
    }
  }
  __syncthreads();
  if constexpr (kStageD) {
    load_rows<V, V>(&sk[0][0], gD, V, kBC, tid);
    load_rows<V, V>(&sq[0][0], gdD, V, kBC, tid);
    __syncthreads();
  }

  // ---- phase B: products over V
  // d Gamma_C = rowsum(dh * h) comes along: lane (g, n) holds h and dh of
  // channel 16 cb + n, columns 16 s + 4g .. +3.  That is also the
  // accumulator layout of the h^T tile, so h is rebuilt there as
  // h^T <- h^T diag(Gamma_C) + Delta^T Kt for each earlier 16-token chunk
  // of the 64-token chunk, as the states kernel advanced it.
  f32x4 cQ[2], cKt[2], cW[2];
  // One instance per number NE of earlier 16-token chunks in the 64-token
  // chunk (0..3, wave-uniform), so each loads exactly the operands it uses
  // and no branch sits between a load and its use.
  auto phase_b = [&](auto ne_tag) {
    constexpr int NE = decltype(ne_tag)::value, NA = NE > 0 ? NE : 1;
    for (int u = 0; u < 2; ++u) {
      const int cb = wave + 4 * u;
      cQ[u] = cKt[u] = cW[u] = f32x4{0, 0, 0, 0};
      if (cb >= NKB) continue;
      // the earlier chunks' Kt and Gamma_C of this key block
      f32x4 ktp[NA];
      float gcp[NA];
      const float* dsp[NA];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int64_t se = slot - NE + e;
        const float* r = p.rec + (se * p.H + h) * R::kFloats;
        ktp[e] = opb(r + R::kKt, K, 0, 16 * cb, lane);      // Kt[4g + j][16 cb + n]
        gcp[e] = r[R::kGc + 16 * cb + n];
        dsp[e] = p.ds + (se * p.H + h) * kBC * V;
      }
      struct VOps {
        f32x4 bh, bdh, d, dd, dl[NA];
      };
      auto load_v = [&](int s, VOps& o) {
        o.bh = opa(hS, V, 16 * cb, 16 * s, lane);
        o.bdh = opa(dhS, V, 16 * cb, 16 * s, lane);
        o.d = opa(sD, V, 0, 16 * s, lane);
        o.dd = opa(sdD, V, 0, 16 * s, lane);
#pragma unroll
        for (int e = 0; e < NE; ++e) o.dl[e] = opb(dsp[e], V, 0, 16 * s, lane);   // (Delta^T)[16 s + n][4g + j]
      };
      float gsum = 0.f;
      auto use_v = [&](int s, const VOps& o) {
        f32x4 bh = o.bh;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
#pragma unroll
          for (int i = 0; i < 4; ++i) bh[i] *= gcp[e];
          mma16(bh, o.dl[e], ktp[e]);
        }
        mma16(cQ[u], opa(sdO, V, 0, 16 * s, lane), bh);
        mma16(cKt[u], o.d, o.bdh);
        mma16(cW[u], o.dd, bh);
        gsum += bh[0] * o.bdh[0] + bh[1] * o.bdh[1] + bh[2] * o.bdh[2] + bh[3] * o.bdh[3];
      };
      // value blocks in pairs, the next block's operands in flight (NVB is even)
      VOps va, vb;
      load_v(0, va);
#pragma unroll 1
      for (int s = 0; s < NVB; s += 2) {
        load_v(s + 1, vb);
        use_v(s, va);
        if (s + 2 < NVB) load_v(s + 2, va);
        use_v(s + 1, vb);
      }
      gsum += __shfl_xor(gsum, 16);
      gsum += __shfl_xor(gsum, 32);
      if (lane < 16) sdgc[16 * cb + n] = gsum;
    }
  };
  switch (sub) {
    case 0: phase_b(std::integral_constant<int, 0>{}); break;
    case 1: phase_b(std::integral_constant<int, 1>{}); break;
    case 2: phase_b(std::integral_constant<int, 2>{}); break;
    default: phase_b(std::integral_constant<int, 3>{}); break;
  }
  if (wave == 0) {
    f32x4 c = {0, 0, 0, 0};
    for (int s = 0; s < NVB; ++s) mma16(c, opa(sdO, V, 0, 16 * s, lane), opa(sD, V, 0, 16 * s, lane));
#pragma unroll
    for (int i = 0; i < 4; ++i) sdAqk[g4 + i][n] = g4 + i >= n ? p.scale * c[i] : 0.f;
  } else if (wave == 1) {
    f32x4 c = {0, 0, 0, 0};
    for (int s = 0; s < NVB; ++s) {
      f32x4 b = opa(sv, V, 0, 16 * s, lane);
      const float bn = sbeta[n];
      b = f32x4{b[0] * bn, b[1] * bn, b[2] * bn, b[3] * bn};
      mma16(c, opa(sdD, V, 0, 16 * s, lane), b);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sdT[g4 + i][n] = c[i];
  } else {
    for (int vb = wave - 2; vb < NVB; vb += 2) {
      f32x4 c = {0, 0, 0, 0};
      mma16(c, opb(&sT[0][0], kBC, 0, 0, lane), opb(sdD, V, 0, 16 * vb, lane));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = g4 + i, j = 16 * vb + n;
        if (r < len) p.dv[tok(r) * V + j] = sbeta[r] * c[i];
        const float x = sum16(sv[r * V + j] * c[i]);
        if (n == 0) sred[wave][r][3] += x;
      }
    }
  }
  __syncthreads();
  if constexpr (kStageD) {   // k and q again, normalised as before
    const int64_t t0 = tok(0);
    load_rows<K, K>(&sk[0][0], k + t0 * K, p.H * K, len, tid, p.l2norm ? snk : nullptr);
    load_rows<K, K>(&sq[0][0], q + t0 * K, p.H * K, len, tid, p.l2norm ? snq : nullptr);
  }
  // dW goes through LDS (its transposes are needed); dKt and dQg stay in the
  // registers of the lanes that use them
  float* sdW = sOW;
  for (int u = 0; u < 2; ++u) {
    const int cb = wave + 4 * u;
    if (cb >= NKB) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) sdW[(g4 + i) * K + 16 * cb + n] = -cW[u][i];
  }
  __syncthreads();

  // ---- phase C: dT += dW Kb^T (as dT^T = Kb dW^T, summed over the waves' key blocks), dA
  {
    f32x4 c = {0, 0, 0, 0};
    for (int u = 0; u < 2; ++u) {
      const int cb = wave + 4 * u;
      if (cb >= NKB) continue;
      const int i = n, c0 = 16 * cb + g4;
      f32x4 a;
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = sbeta[i] * sk[i][c0 + j] * __expf(sG[i][c0 + j]);
      mma16(c, a, opa(sdW, K, 0, 16 * cb, lane));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sdTp[wave][n][g4 + i] = c[i];
  }
  __syncthreads();
  {
    const int r = tid / kBC, cc = tid % kBC;
    sX[r][cc] = sdT[r][cc] + sdTp[0][r][cc] + sdTp[1][r][cc] + sdTp[2][r][cc] + sdTp[3][r][cc];
  }
  __syncthreads();
  {
    const int r = tid / kBC, cc = tid % kBC;
    float x = 0.f;
    for (int a = r; a < kBC; ++a) x += sT[a][r] * sX[a][cc];
    sdT[r][cc] = x;   // now X = T^T dT
  }
  __syncthreads();
  {
    const int r = tid / kBC, cc = tid % kBC;
    float x = 0.f;
    for (int b = 0; b <= cc; ++b) x += sdT[r][b] * sT[cc][b];
    sdA[r][cc] = cc < r ? -x : 0.f;
  }
  __syncthreads();

  // ---- phase D: per key block, the terms of A and Aqk back onto q, k and G
  float* sdG = sVG;
  float dqh[2][4], dkh[2][4];
  float pq[4] = {0, 0, 0, 0}, pk[4] = {0, 0, 0, 0}, pb[4] = {0, 0, 0, 0};
  for (int u = 0; u < 2; ++u) {
    const int cb = wave + 4 * u;
    if (cb >= NKB) continue;
    const int c = 16 * cb + n;                  // this lane's channel in the C layout
    f32x4 cKb = {0, 0, 0, 0}, RA = {0, 0, 0, 0}, RAq = {0, 0, 0, 0}, CA = {0, 0, 0, 0}, CAq = {0, 0, 0, 0};
    mma16(cKb, opb(&sT[0][0], kBC, 0, 0, lane), opb(sdW, K, 0, 16 * cb, lane));
    if (!unsafe) {
      // B operands kb[4g+j][c] = k exp(G0 - G), beta kf = beta k exp(G - G0), qf = q exp(G - G0)
      f32x4 kb, bkf, qf;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = g4 + j;
        const float d = sG[r][c] - sG[0][c];
        kb[j] = sk[r][c] * __expf(-d);
        bkf[j] = sbeta[r] * sk[r][c] * __expf(d);
        qf[j] = sq[r][c] * __expf(d);
      }
      mma16(RA, opa(&sdA[0][0], kBC, 0, 0, lane), kb);
      mma16(RAq, opa(&sdAqk[0][0], kBC, 0, 0, lane), kb);
      mma16(CA, opb(&sdA[0][0], kBC, 0, 0, lane), bkf);
      mma16(CAq, opb(&sdAqk[0][0], kBC, 0, 0, lane), qf);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = sG[g4 + i][c] - sG[0][c];
        const float fr = __expf(d), bk = __expf(-d);
        RA[i] *= fr;
        RAq[i] *= fr;
        CA[i] *= bk;
        CAq[i] *= bk;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = g4 + i;
        for (int x = 0; x < kBC; ++x) {
          const float e = __expf(sG[r][c] - sG[x][c]), ei = __expf(sG[x][c] - sG[r][c]);
          if (x <= r) {
            RA[i] += sdA[r][x] * sk[x][c] * e;
            RAq[i] += sdAqk[r][x] * sk[x][c] * e;
          }
          if (x >= r) {
            CA[i] += sdA[x][r] * sbeta[x] * sk[x][c] * ei;
            CAq[i] += sdAqk[x][r] * sq[x][c] * ei;
          }
        }
      }
    }
    const float GC = sG[last][c];
    // the last row's G_C terms: sum over the chunk's rows of dKt * Kt (this
    // lane holds rows 4g .. 4g+3 of channel c; the four lane groups add up),
    // and d Gamma_C Gamma_C
    float lastx = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) lastx += cKt[u][i] * rec[R::kKt + (g4 + i) * K + c];
    lastx += __shfl_xor(lastx, 16);
    lastx += __shfl_xor(lastx, 32);
    lastx += sdgc[c] * __expf(GC);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = g4 + i;
      const float G = sG[r][c], e = __expf(G), ec = __expf(GC - G), kh = sk[r][c], qh = sq[r][c], br = sbeta[r];
      const float dQg = p.scale * cQ[u][i], dKt = cKt[u][i], dKb = cKb[i];
      dqh[u][i] = dQg * e + RAq[i];
      dkh[u][i] = dKb * br * e + dKt * ec + br * RA[i] + CA[i] + CAq[i];
      pb[i] += kh * e * dKb + kh * RA[i];
      float dG = dQg * qh * e + dKb * br * kh * e - dKt * kh * ec + br * kh * RA[i] - kh * CA[i] + qh * RAq[i] -
                 kh * CAq[i];
      if (r == last) dG += lastx;
      sdG[r * K + c] = r < len ? dG : 0.f;
      pq[i] += qh * dqh[u][i];
      pk[i] += kh * dkh[u][i];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = sum16(pq[i]), b = sum16(pk[i]), c = sum16(pb[i]);
    if (n == 0) {
      sred[wave][g4 + i][0] = a;
      sred[wave][g4 + i][1] = b;
      sred[wave][g4 + i][2] = c;
    }
  }
  __syncthreads();
  for (int u = 0; u < 2; ++u) {
    const int cb = wave + 4 * u;
    if (cb >= NKB) continue;
    const int c = 16 * cb + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = g4 + i;
      if (r >= len) continue;
      const float pqr = sred[0][r][0] + sred[1][r][0] + sred[2][r][0] + sred[3][r][0];
      const float pkr = sred[0][r][1] + sred[1][r][1] + sred[2][r][1] + sred[3][r][1];
      const float dq = p.l2norm ? (dqh[u][i] - sq[r][c] * pqr) / snq[r] : dqh[u][i];
      const float dk = p.l2norm ? (dkh[u][i] - sk[r][c] * pkr) / snk[r] : dkh[u][i];
      p.dq[tok(r) * K + c] = dq;
      p.dk[tok(r) * K + c] = dk;
    }
  }
  if (tid < len) {
    float x = 0.f;
    for (int w = 0; w < 4; ++w) x += sred[w][tid][2] + sred[w][tid][3];
    p.dbeta[tok(tid)] = x;
  }
  for (int c = tid; c < K; c += kBThreads) {
    float run = 0.f;
    for (int r = last; r >= 0; --r) {
      run += sdG[r * K + c];
      p.dg[tok(r) * K + c] = run;
    }
  }
}

template <class TI, class TO, int K, int V>
hipError_t launch_bwd_t(const BwdArgs& a, int stage) {
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
  p.rec = a.rec; p.hs = a.hs; p.dhs = a.dhs; p.ds = a.ds; p.dds = a.dds;
  const int64_t slots = 4 * a.cmax;
  const dim3 blk(kBThreads);
  const int64_t seqs = ((p.packed ? a.smax : a.B) * a.H + 7) / 8 * 8 * (V / kBC);
  switch (stage) {
    case 0: hipLaunchKernelGGL((bwd_chunk_kernel<TI, K, V>), dim3((unsigned)(slots * a.H)), blk, 0, a.stream, p); break;
    case 1: hipLaunchKernelGGL((bwd_states_kernel<K, V>), dim3((unsigned)seqs), dim3(kStatesThreads), 0, a.stream, p); break;
    case 2:
      hipLaunchKernelGGL((bwd_dstates_kernel<TO, K, V>), dim3((unsigned)seqs), dim3(kDStatesThreads), 0, a.stream, p);
      break;
    case 3: hipLaunchKernelGGL((bwd_local_kernel<TI, TO, K, V>), dim3((unsigned)(slots * a.H)), blk, 0, a.stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class TI, class TO>
hipError_t launch_bwd_kv(const BwdArgs& a, int stage) {
  if (a.K == 64 && a.V == 64) return launch_bwd_t<TI, TO, 64, 64>(a, stage);
  if (a.K == 64 && a.V == 128) return launch_bwd_t<TI, TO, 64, 128>(a, stage);
  if (a.K == 128 && a.V == 64) return launch_bwd_t<TI, TO, 128, 64>(a, stage);
  if (a.K == 128 && a.V == 128) return launch_bwd_t<TI, TO, 128, 128>(a, stage);
  return hipErrorInvalidValue;
}

}  // namespace

int64_t bwd_record_floats(int64_t K, int64_t V) {
  if (K == 64 && V == 64) return BRec<64, 64>::kFloats;
  if (K == 64 && V == 128) return BRec<64, 128>::kFloats;
  if (K == 128 && V == 64) return BRec<128, 64>::kFloats;
  return BRec<128, 128>::kFloats;
}

hipError_t launch_bwd(const BwdArgs& a, int stage) {
  if (a.in == InType::BF16)
    return a.do_bf16 ? launch_bwd_kv<uint16_t, uint16_t>(a, stage) : launch_bwd_kv<uint16_t, float>(a, stage);
  return a.do_bf16 ? launch_bwd_kv<float, uint16_t>(a, stage) : launch_bwd_kv<float, float>(a, stage);
}

}  // namespace kda
