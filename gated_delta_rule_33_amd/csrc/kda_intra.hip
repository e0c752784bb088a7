// Intra-chunk kernel of the KDA forward: everything that does not depend on
// the recurrent state, per (chunk, head) item.
//
// Notation (rows r, i = tokens of the chunk, c = key channel):
//   G_r   = sum_{j<=r} g_j, the running log decay inside the chunk
//   A[r,i]   = beta_r sum_c k_rc k_ic exp(G_rc - G_ic)   i < r
//   Aqk[r,i] = sum_c q_rc k_ic exp(G_rc - G_ic)          i <= r
//   T = (I + A)^-1, W = T diag(beta) (K * exp(G)), U = T diag(beta) V
// Unrolling the delta rule of the page "feat(kda): integrate KDA attention
// with tokamax backend and CP support" (Implementation Details, "Delta Rule
// formulation") over a chunk gives, with S0 the state entering the chunk,
//   Delta = U - W S0,  O = scale [ (Q * exp(G)) S0 + Aqk Delta ],
//   S_C = diag(exp(G_C)) S0 + (K * exp(G_C - G))^T Delta,
// which the recurrence kernel evaluates.  This kernel writes the S0-free
// operands of those three lines.  The triangular solve replaces the
// row-by-row stacking solver described for the TPU megakernel (tokamax packed
// forward page, 2026-09-29 follow-ups) by 16x16 diagonal inversions plus
// matrix-core block merges.
//
// Overflow-free exponentials: exp(G_r - G_i) is split at a reference row f
// (the first row of r's 16-row block) as exp(G_r - G_f) * exp(G_f - G_i).
// Both factors are <= 1 whenever i precedes f.  Inside the diagonal block the
// second factor can exceed 1 by up to exp(span), span = G_f - G_{f+15}; the
// split is used while span <= 64 (always true under the safe-gate bound
// g >= -5 of the chunk_kda options, where span <= 75 is possible only at the
// very edge) and the block is evaluated pair by pair otherwise.
#include <cstring>

#include "kda_intra_item.h"

namespace kda {
namespace {

using namespace detail;

constexpr int kIntraWaves = 8;                       // two per SIMD
constexpr int kIntraThreads = kIntraWaves * kWave;

// Rows of W elements kept in LDS with their 16-byte chunks XOR-swizzled by the
// row index, so that 16 lanes reading one chunk of 16 different rows hit 16
// different bank groups.  Direct-to-LDS loads write 64 consecutive 16-byte
// slots per instruction; each lane picks the global chunk that belongs in its
// slot, which is how the swizzle is applied on the way in.
template <class TI, int W>
struct SwzRows {
  static constexpr int E = 16 / (int)sizeof(TI);   // elements per chunk
  static constexpr int NCH = W / E;                  // chunks per row
  __device__ static __forceinline__ int idx(int r, int c) {
    return r * W + (((c / E) ^ (r % NCH)) * E) + (c % E);
  }
};

template <class TI, int K, int V>
struct IntraSmem {
  static constexpr bool kDB = sizeof(TI) == 2;   // g/v double-buffered (fits LDS for bf16)
  static constexpr int NB = kDB ? 2 : 1;
  // bf16 inputs: the decayed keys X of the column operands are tabulated once
  // per item (fp32 inputs compute them pair by pair, for lack of LDS).
  static constexpr bool kXT = sizeof(TI) == 2;
  static constexpr int kGVW = K > V ? K : V;      // g (width K) and later v (width V) share a buffer
  static constexpr int kGP = K + 4;               // row pitch (floats) of G and X
  static constexpr int kMP = 68;                  // row pitch of M (T below the diagonal, A^T above)
  static constexpr int kPairs = 10;               // (row block, column block) pairs with I <= R
  TI q[kChunk * K];
  TI k[kChunk * K];
  TI gv[NB][kChunk * kGVW];
  float G[kChunk * kGP];
  float beta[kChunk];
  float M[kChunk * kMP];
  alignas(16) float nk[kChunk];
  // Per-channel decay factors (bf16 inputs): exp(G_f(R) - G_l(I)) for the ten
  // pairs, exp(G_f(R)) for the four row blocks (f = first, l = last row),
  // then exp(G_C - G_l(I)) for the four column blocks.
  static constexpr int kTabRows = kPairs + 8;
  alignas(16) float tab[kXT ? kTabRows * K : 4];
  // Partial A / Aqk tiles of the upper key-channel half: 10 (row block, column
  // block) tiles x {A, Aqk} x 64 lanes x 4.  They reuse the q buffer (dead by
  // then) when it is large enough (fp32 inputs with K = 128), else the scratch.
  static constexpr int kRedFloats = 10 * 2 * kWave * 4;
  static constexpr bool kRedInQ = sizeof(TI) * kChunk * K >= sizeof(float) * kRedFloats;
  // Scratch used in turn by the running-sum partials, the X table and the
  // partial tiles.
  static constexpr int kPartFloats = 2 * kIntraThreads;
  static constexpr int kXFloats = kXT ? kChunk * kGP : 0;
  static constexpr int kScratch0 = kPartFloats > kXFloats ? kPartFloats : kXFloats;
  static constexpr int kScratch = (!kRedInQ && kRedFloats > kScratch0) ? kRedFloats : kScratch0;
  alignas(16) float scratch[kScratch];
  __device__ float* part() { return scratch; }
  __device__ float* X() { return scratch; }
  __device__ float* red_buf() { return kRedInQ ? reinterpret_cast<float*>(q) : scratch; }
};

__device__ __forceinline__ float ld1(const float* p) { return *p; }
// Two consecutive elements (even offset) as floats.
__device__ __forceinline__ void ld2(const float* p, float& a, float& b) {
  const float2 v = *reinterpret_cast<const float2*>(p);
  a = v.x;
  b = v.y;
}
__device__ __forceinline__ void ld2(const uint16_t* p, float& a, float& b) {
  const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
  a = __uint_as_float(v << 16);
  b = __uint_as_float(v & 0xffff0000u);
}
__device__ __forceinline__ float ld1(const uint16_t* p) { return bits_to_f32(*p); }

// The eight elements of a swizzled row at the fragment k-order of k-tile kb.
template <class TI, int W>
__device__ __forceinline__ void row8(const TI* base, int r, int kb, int g, float x[8]) {
  using S = SwzRows<TI, W>;
  const f32x4 a = ld4(base + S::idx(r, 32 * kb + 4 * g)), b = ld4(base + S::idx(r, 32 * kb + 16 + 4 * g));
  x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
  x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}
// The same for an fp32 row with a padded pitch.
__device__ __forceinline__ void row8f(const float* rowp, int kb, int g, float x[8]) {
  const f32x4 a = ld4(rowp + 32 * kb + 4 * g), b = ld4(rowp + 32 * kb + 16 + 4 * g);
  x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
  x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}

// This wave's share of the direct-to-LDS loads of a 64 x W tile whose row r
// starts at src + r * row_stride.  Rows >= len are not loaded (their LDS rows
// are zeroed after the wait).  Asynchronous: completion is awaited with
// wait_loads() before the data is read.
template <class TI, int W>
__device__ __forceinline__ void issue_rows(TI* lds, const TI* src, int64_t row_stride, int len, int w, int lane) {
  using S = SwzRows<TI, W>;
  constexpr int BLOCKS = kChunk * S::NCH / kWave;   // 1 KB blocks
#pragma unroll
  for (int bi = w; bi < BLOCKS; bi += kIntraWaves) {
    const int L = bi * kWave + lane, r = L / S::NCH, pch = L % S::NCH, cv = pch ^ (r % S::NCH);
    if (r < len)
      dma16(lds + bi * kWave * S::E, src + r * row_stride + cv * S::E);
  }
}

// Wait for every outstanding vector memory operation of this wave.
__device__ __forceinline__ void wait_loads() { vm_wait<0>(); }

// One workgroup per CU, looping over (chunk, head) items.  The inputs of the
// next item are loaded into LDS (direct-to-LDS, asynchronous) while the
// current item computes: k, g and beta after the A products (second buffers),
// q once the current q is dead (after the A products), v into the g buffer
// once g has been summed (issued after the A products too).
template <class TI, int K, int V>
__global__ __launch_bounds__(kIntraThreads, 1) void kda_intra_kernel(IntraParams p) {
  using S = IntraSmem<TI, K, V>;
  using SK = SwzRows<TI, K>;
  using SV = SwzRows<TI, V>;
  using PA = typename Prec<TI>::A;
  using PT = typename Prec<TI>::T;
  using PX = typename Prec<TI>::X;
  using PV = typename Prec<TI>::V;
  using PW = typename Prec<TI>::W;
  using PK = typename Prec<TI>::Kt;
  using PQ = typename Prec<TI>::Qg;
  using PAq = typename Prec<TI>::Aq;
  using L = RecordLayout<TI, K, V>;
  extern __shared__ __align__(16) char smem_raw[];
  S& sm = *reinterpret_cast<S*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Row block of the intra-chunk products and half of the key channels this
  // wave takes: waves s and s + 4 share SIMD s and get row blocks s and 3 - s,
  // so every SIMD carries the same share of the triangle.
  const int R = w < 4 ? w : 7 - w, chalf = w / 4;
  const TI* gq_ = static_cast<const TI*>(p.q);
  const TI* gk_ = static_cast<const TI*>(p.k);
  const TI* gv_ = static_cast<const TI*>(p.v);
  const TI* gg_ = static_cast<const TI*>(p.g);
  const TI* gb_ = static_cast<const TI*>(p.beta);
  const int64_t H = p.H;
  const int64_t n_items = p.packed ? (int64_t)p.hdr->n_chunks * H : p.B * p.nc_fixed * H;
  // No tables without segments: the flags start clear (debug builds clear
  // them before the launch, since their checks may raise flags meanwhile).
  if (!KDA_DEBUG_CHECKS && !p.packed && blockIdx.x == 0 && tid == 0) p.hdr->flags = 0;
  if ((int64_t)blockIdx.x >= n_items) return;

  // beta of the next item travels as raw input bits in one register per lane
  // (lane = token), loaded unconditionally from a clamped token and widened
  // only after the wait for the item's loads: a load whose value is used at
  // once would make the compiler wait for every load in flight, the
  // direct-to-LDS prefetches included.
  TI beta_next = TI(0);
  // The gate parameters of the next item for this thread's two running-sum
  // channels (raw A_log of its head, dt_bias of the channels), likewise.
  constexpr int kSumPairs = K / 2;
  const int c_sum = 2 * (tid % kSumPairs);
  float alog_next = 0.f, db0_next = 0.f, db1_next = 0.f;
  auto issue_k = [&](const ItemInfo& it) {
    issue_rows<TI, K>(sm.k, gk_ + (it.tok0 * H + it.h) * K, H * K, it.len, w, lane);
  };
  auto issue_gb = [&](const ItemInfo& it, int buf) {
    issue_rows<TI, K>(sm.gv[buf], gg_ + (it.tok0 * H + it.h) * K, H * K, it.len, w, lane);
    beta_next = gb_[(it.tok0 + min(lane, it.len - 1)) * H + it.h];
    if (p.gate_mode) {
      if (p.a_log) alog_next = p.a_log[it.h];
      if (p.dt_bias) {
        db0_next = p.dt_bias[it.h * K + c_sum];
        db1_next = p.dt_bias[it.h * K + c_sum + 1];
      }
    }
  };
  auto issue_q = [&](const ItemInfo& it) {
    issue_rows<TI, K>(sm.q, gq_ + (it.tok0 * H + it.h) * K, H * K, it.len, w, lane);
  };

  // Items are walked from the last one back: the records of the first
  // chunks, which the recurrence reads first, are then the most recently
  // written and still in L2 and the memory-side cache when it starts.
  {
    const ItemInfo first = item_info(p, item_pos(p, n_items - 1 - (int64_t)blockIdx.x));
    issue_k(first);
    issue_gb(first, 0);
    issue_q(first);
  }

  int it_no = 0;
  const ItemPos stride = item_pos(p, gridDim.x);
  ItemPos pos = item_pos(p, n_items - 1 - (int64_t)blockIdx.x);
  for (int64_t idx = blockIdx.x; idx < n_items; idx += gridDim.x, ++it_no) {
    const int64_t item = n_items - 1 - idx;
    const int cb = S::kDB ? (it_no & 1) : 0;
    const ItemInfo cur = item_info(p, pos);
    const int len = cur.len;
    const int64_t h = cur.h;
    const bool has_next = idx + gridDim.x < n_items;
    const ItemPos npos = item_retreat(p, pos, stride);
    const ItemInfo nxt = has_next ? item_info(p, npos) : cur;
    pos = npos;
    char* rec = p.records + item * p.record_bytes;
    TI* kbuf = sm.k;
    TI* gvbuf = sm.gv[cb];
    const int tid = opaque(threadIdx.x), lane = tid & 63;
    const int m = lane & 15, gq = lane >> 4;

    // ---- this item's q, k, g, beta have landed; zero the rows past the chunk
    wait_loads();
    block_sync();
    if (w == 0) sm.beta[lane] = lane < len ? ld1(&beta_next) : 0.f;   // zero past the chunk
    if (len < kChunk) {
      for (int e = tid; e < (kChunk - len) * K; e += kIntraThreads) {
        const int r = len + e / K, c = e % K;
        sm.q[SK::idx(r, c)] = TI(0);
        kbuf[SK::idx(r, c)] = TI(0);
        gvbuf[SK::idx(r, c)] = TI(0);
      }
    }
    block_sync();

    // ---- running sum of g over the chunk, per channel
    {   // two channels per thread, rows in PARTS parts of RP
      constexpr int PAIRS = kSumPairs, PARTS = kIntraThreads / PAIRS, RP = kChunk / PARTS;
      const int c = 2 * (tid % PAIRS), part = tid / PAIRS, r0 = part * RP;
      float g0[RP], g1[RP];
#pragma unroll
      for (int i = 0; i < RP; ++i) ld2(gvbuf + SK::idx(r0 + i, c), g0[i], g1[i]);   // all reads in flight
      if (KDA_DEBUG_CHECKS && !p.gate_mode) {   // g is the log decay: g <= 0 is a precondition
        bool pos = false;
#pragma unroll
        for (int i = 0; i < RP; ++i) pos = pos || (r0 + i < len && (g0[i] > 0.f || g1[i] > 0.f));
        flag_if_any(&p.hdr->flags, pos, KDA_FLAG_GATE_POSITIVE);
      }
      if (p.gate_mode) {
        // In-kernel gate: z = exp(A_log_h) (g + dt_bias_hc); the log decay is
        // lower_bound * sigmoid(z) under the safe gate, else log sigmoid(z).
        // Rows past the chunk keep g = 0.
        const float ea = __expf(alog_next);
#pragma unroll
        for (int i = 0; i < RP; ++i) {
          if (r0 + i >= len) continue;
          g0[i] = gate_log_decay(p.gate_mode, p.lower_bound, ea * (g0[i] + db0_next));
          g1[i] = gate_log_decay(p.gate_mode, p.lower_bound, ea * (g1[i] + db1_next));
        }
      }
#pragma unroll
      for (int i = 1; i < RP; ++i) {
        g0[i] += g0[i - 1];
        g1[i] += g1[i - 1];
      }
      *reinterpret_cast<float2*>(&sm.part()[part * K + c]) = float2{g0[RP - 1], g1[RP - 1]};
      block_sync();
      float o0 = 0.f, o1 = 0.f;
      float2 pv[PARTS - 1];
#pragma unroll
      for (int pp = 0; pp < PARTS - 1; ++pp) pv[pp] = *reinterpret_cast<const float2*>(&sm.part()[pp * K + c]);
#pragma unroll
      for (int pp = 0; pp < PARTS - 1; ++pp)
        if (pp < part) {
          o0 += pv[pp].x;
          o1 += pv[pp].y;
        }
#pragma unroll
      for (int i = 0; i < RP; ++i)
        *reinterpret_cast<float2*>(&sm.G[(r0 + i) * S::kGP + c]) = float2{g0[i] + o0, g1[i] + o1};
    }
    block_sync();   // g consumed: the buffer may receive v

    // ---- bf16 inputs: X[i][c] = k_ic exp(G_l,c - G_ic) with l the last row of
    //      i's block (every factor <= 1), and the per-channel factors
    //      exp(G_f(R) - G_l(I)) (pairs I <= R) and exp(G_f(R)).  A column
    //      operand of the pair (R, I) is then X * exp(G_f(R) - G_l(I)) =
    //      k_i exp(G_f(R) - G_i), and exp(G_r) = exp(G_r - G_f(R)) exp(G_f(R)).
    if constexpr (S::kXT) {
      float* X = sm.X();
      constexpr int XIT = kChunk * K / 4 / kIntraThreads;
      static_assert(XIT * kIntraThreads * 4 == kChunk * K, "whole passes");
      f32x4 gr[XIT], gl[XIT], kx[XIT];
#pragma unroll
      for (int it = 0; it < XIT; ++it) {   // all reads first
        const int e4 = tid + it * kIntraThreads, r = e4 / (K / 4), c = (e4 % (K / 4)) * 4, l = (r | 15);
        gr[it] = ld4(sm.G + r * S::kGP + c);
        gl[it] = ld4(sm.G + l * S::kGP + c);
        kx[it] = ld4(kbuf + SK::idx(r, c));
      }
#pragma unroll
      for (int it = 0; it < XIT; ++it) {
        const int e4 = tid + it * kIntraThreads, r = e4 / (K / 4), c = (e4 % (K / 4)) * 4;
        f32x4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = kx[it][j] * __expf(gl[it][j] - gr[it][j]);
        *reinterpret_cast<f32x4*>(X + r * S::kGP + c) = x;
      }
      constexpr int TIT = (S::kTabRows * K + kIntraThreads - 1) / kIntraThreads;
      float ga[TIT], gb[TIT];
#pragma unroll
      for (int it = 0; it < TIT; ++it) {
        const int e = tid + it * kIntraThreads, t = e / K, c = e % K;
        int ra = 0, rb = kChunk - 1;   // exp(G_ra - G_rb)
        if (t < S::kPairs) {
          const int R2 = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3, I2 = t - R2 * (R2 + 1) / 2;
          ra = 16 * R2;
          rb = 16 * I2 + 15;
        } else if (t < S::kPairs + 4) {
          ra = 16 * (t - S::kPairs);
          rb = -1;
        } else {
          ra = kChunk - 1;
          rb = 16 * (t - S::kPairs - 4) + 15;
        }
        const bool ok = e < S::kTabRows * K;
        ga[it] = ok ? sm.G[ra * S::kGP + c] : 0.f;
        gb[it] = (ok && rb >= 0) ? sm.G[rb * S::kGP + c] : 0.f;
      }
#pragma unroll
      for (int it = 0; it < TIT; ++it) {
        const int e = tid + it * kIntraThreads;
        if (e < S::kTabRows * K) sm.tab[e] = __expf(ga[it] - gb[it]);
      }
    }

    // ---- this wave's rows: norms and its block's span (both waves of a row block)
    const int f = 16 * R, r_own = f + m;
    float nqr = 1.f, nkr = 1.f;
    if (p.l2norm) {
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int kb = 0; kb < K / 32; ++kb) {
        float kx[8], qx[8];
        row8<TI, K>(sm.q, r_own, kb, gq, qx);
        row8<TI, K>(kbuf, r_own, kb, gq, kx);
#pragma unroll
        for (int j = 0; j < 8; ++j) { sq += qx[j] * qx[j]; sk += kx[j] * kx[j]; }
      }
      sq += __shfl_xor(sq, 16); sq += __shfl_xor(sq, 32);
      sk += __shfl_xor(sk, 16); sk += __shfl_xor(sk, 32);
      nqr = 1.f / sqrtf(sq + 1e-6f);
      nkr = 1.f / sqrtf(sk + 1e-6f);
    }
    if (gq == 0 && chalf == 0) sm.nk[r_own] = nkr;
    float span = 0.f;
    for (int c = lane; c < K; c += kWave) span = fmaxf(span, sm.G[f * S::kGP + c] - sm.G[(f + 15) * S::kGP + c]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) span = fmaxf(span, __shfl_xor(span, off));
    // wave-uniform (the reduction above leaves it in every lane); stated so,
    // the block loop below branches on scalars instead of masking lanes
    const bool diag_split = __builtin_amdgcn_readfirstlane(span <= kSpanMax ? 1 : 0) != 0;
    block_sync();   // nk, X and the factor table visible

    // ---- A and Aqk for row block R over key-channel half chalf: tiles (I, R)
    //      hold D[i][r], I <= R; the two halves are summed through LDS below.
    //      The per-row L2-norm factors multiply the 16x16 results, not the
    //      operands.
    f32x4 accKK[4], accQK[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) { accKK[I] = f32x4{0, 0, 0, 0}; accQK[I] = f32x4{0, 0, 0, 0}; }
    {
      const int r = r_own;
      const float sqr = p.scale * nqr;
      constexpr int KBH = K / 64;   // 32-channel slabs per half
#pragma unroll
      for (int kbi = 0; kbi < KBH; ++kbi) {
        const int kb = chalf * KBH + kbi;
        float gr[8], gf[8], kx[8], qx[8], xk[8], xq[8], er[8];
        row8f(sm.G + r * S::kGP, kb, gq, gr);
        row8f(sm.G + f * S::kGP, kb, gq, gf);
        row8<TI, K>(kbuf, r, kb, gq, kx);
        row8<TI, K>(sm.q, r, kb, gq, qx);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          er[j] = __expf(gr[j] - gf[j]);
          xk[j] = kx[j] * er[j];
          xq[j] = qx[j] * er[j];
        }
        PA fkr, fqr;
        fkr.set(xk);
        fqr.set(xq);
        {   // scale * q * exp(G) for this wave's rows: the output's inter-chunk operand
          float xg[8];
          if constexpr (S::kXT) {
            float ef[8];
            row8f(sm.tab + (S::kPairs + R) * K, kb, gq, ef);
#pragma unroll
            for (int j = 0; j < 8; ++j) xg[j] = sqr * qx[j] * er[j] * ef[j];
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) xg[j] = sqr * qx[j] * __expf(gr[j]);
          }
          PQ qf;
          qf.set(xg);
          qf.store(rec + L::kQg + (int64_t)(R * (K / 32) + kb) * tile_bytes<PQ>(), lane);
        }
        // bf16 inputs: the column operands' table rows for every I <= R
        // are read before any is used
        float xi[4][8], di[4][8];
        if constexpr (S::kXT) {
#pragma unroll
          for (int I = 0; I < 4; ++I) {
            if (I > R) continue;
            row8f(sm.X() + (16 * I + m) * S::kGP, kb, gq, xi[I]);
            row8f(sm.tab + (R * (R + 1) / 2 + I) * K, kb, gq, di[I]);
          }
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (I > R || (I == R && !diag_split)) continue;
          const int i = 16 * I + m;
          float xc[8];
          if constexpr (S::kXT) {
#pragma unroll
            for (int j = 0; j < 8; ++j) xc[j] = xi[I][j] * di[I][j];
          } else {
            float gi[8], ki[8];
            row8f(sm.G + i * S::kGP, kb, gq, gi);
            row8<TI, K>(kbuf, i, kb, gq, ki);
#pragma unroll
            for (int j = 0; j < 8; ++j) xc[j] = ki[j] * __expf(gf[j] - gi[j]);
          }
          PA fkc;
          fkc.set(xc);
          mma(accKK[I], fkc, fkr);
          mma(accQK[I], fkc, fqr);
        }
      }
      if (p.l2norm) {   // D[i][r] * nk_i * (nk_r | nq_r); lane: column r, rows i = 16I + 4gq + ii
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (I > R) continue;
          const f32x4 nki = ld4(sm.nk + 16 * I + 4 * gq);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            accKK[I][ii] *= nki[ii] * nkr;
            accQK[I][ii] *= nki[ii] * nqr;
          }
        }
      }
      if (!diag_split) {
        // Pair-by-pair evaluation of the diagonal block: exp(G_r - G_i) <= 1.
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int i = f + 4 * gq + ii;
          float sk_ = 0.f, sq_ = 0.f;
          if (i <= r) {
            const float nki = sm.nk[i];
            for (int c = chalf * (K / 2); c < (chalf + 1) * (K / 2); ++c) {
              const float e = __expf(sm.G[r * S::kGP + c] - sm.G[i * S::kGP + c]);
              const float kk = ld1(kbuf + SK::idx(i, c)) * nki * e;
              sk_ += ld1(kbuf + SK::idx(r, c)) * nkr * kk;
              sq_ += ld1(sm.q + SK::idx(r, c)) * nqr * kk;
            }
          }
#pragma unroll
          for (int I = 0; I < 4; ++I)
            if (I == R) { accKK[I][ii] = sk_; accQK[I][ii] = sq_; }
        }
      }
    }
    // This item's v and the next item's k, g and beta go out here, where the
    // other wave of each SIMD has VALU work to fill the issue stalls.
    issue_rows<TI, V>(gvbuf, gv_ + (cur.tok0 * H + h) * V, H * V, len, w, lane);
    if (S::kDB && has_next) issue_gb(nxt, cb ^ 1);

    // ---- Kt = (k * exp(G_C - G))^T as operand tiles [c-block][token k-tile].
    //      bf16 inputs: from X, Kt[c][r] = X[r][c] exp(G_C - G_l(I(r))), by the
    //      waves of the lower channel half, whose share of the products above
    //      is the smaller one; fp32 inputs: beside the solve below.
    constexpr int NKT = (K / 16) * 2;
    if constexpr (S::kXT) {
      if (w < 4) {
        for (int t = w; t < NKT; t += 4) {
          const int cbk = t >> 1, kb = t & 1, c = 16 * cbk + m;
          const float e0 = sm.tab[(S::kPairs + 4 + 2 * kb) * K + c], e1 = sm.tab[(S::kPairs + 5 + 2 * kb) * K + c];
          float xv[8], n8[8], x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {   // all reads first
            const int r = 32 * kb + kperm(gq, j);
            xv[j] = sm.X()[r * S::kGP + c];
            n8[j] = sm.nk[r];
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = xv[j] * n8[j] * (j < 4 ? e0 : e1);
          PK fr;
          fr.set(x);
          fr.store(rec + L::kKt + (int64_t)(cbk * 2 + kb) * tile_bytes<PK>(), lane);
        }
      }
    }

    // ---- the two channel halves exchange partial tiles: the upper half
    //      completes A (into M), the lower half completes Aqk (into the record)
    {
      float* red = sm.red_buf();
      const int slot0 = R * (R + 1) / 2;   // tiles (R, 0..R)
      block_sync();   // everyone is done with q (fp32 inputs reuse it here)
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        if (I > R) continue;
        if (chalf == 1)
          reinterpret_cast<f32x4*>(red)[((slot0 + I) * 2 + 0) * kWave + lane] = accKK[I];
        else
          reinterpret_cast<f32x4*>(red)[((slot0 + I) * 2 + 1) * kWave + lane] = accQK[I];
      }
      block_sync();
      const int r = r_own;
      if (chalf == 0) {
        // A[r][i] = beta_r * D[i][r] (i < r), stored transposed above the diagonal of M.
        const float br = sm.beta[r];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (I > R) continue;
          const f32x4 part = reinterpret_cast<const f32x4*>(red)[((slot0 + I) * 2 + 0) * kWave + lane];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int i = 16 * I + 4 * gq + ii;
            const float a = br * (accKK[I][ii] + part[ii]);
            if (I < R || i < r) sm.M[i * S::kMP + r] = a;
          }
        }
      } else {
        // scale * Aqk, rows of block R: the D[i][r] tiles (I, R) are the operand layout
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (I > R) continue;
          const f32x4 part = reinterpret_cast<const f32x4*>(red)[((slot0 + I) * 2 + 1) * kWave + lane];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int i = 16 * I + 4 * gq + ii;
            accQK[I][ii] = (I < R || i <= r) ? p.scale * (accQK[I][ii] + part[ii]) : 0.f;
          }
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb > R / 2) continue;   // all zero: not stored
          float x[8];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            x[ii] = (2 * kb <= R) ? accQK[2 * kb][ii] : 0.f;
            x[4 + ii] = (2 * kb + 1 <= R) ? accQK[2 * kb + 1][ii] : 0.f;
          }
          PAq af;
          af.set(x);
          af.store(rec + L::kAqk + (int64_t)aqk_tile(R, kb) * tile_bytes<PAq>(), lane);
        }
      }
    }
    block_sync();   // q and the partial tiles are dead: the next item's q streams in
    if (has_next) issue_q(nxt);

    // ---- Kt = (k * exp(G_C - G))^T as operand tiles [c-block][token k-tile];
    //      independent of T, so waves 4-7 build them while waves 0-3 solve
    auto kt_tile = [&](int t) {
      const int cbk = t >> 1, kb = t & 1, c = 16 * cbk + m;
      const float gc = sm.G[(kChunk - 1) * S::kGP + c];
      float x[8], kv8[8], g8[8], n8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {   // all reads first
        const int r = 32 * kb + kperm(gq, j);
        kv8[j] = ld1(kbuf + SK::idx(r, c));
        g8[j] = sm.G[r * S::kGP + c];
        n8[j] = sm.nk[r];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = kv8[j] * n8[j] * __expf(gc - g8[j]);
      PK fr;
      fr.set(x);
      fr.store(rec + L::kKt + (int64_t)(cbk * 2 + kb) * tile_bytes<PK>(), lane);
    };

    // ---- T = (I + A)^-1 by 16x16 blocks on the fp32 matrix path.  M holds
    //      A^T above the diagonal; T goes below it, diagonal included.
    //      Operand fragments of a 16x16 block X: A layout, lane (m, g) element
    //      s = X[m][4g + s]; B layout, lane (n, g) element s = X[4g + s][n],
    //      which is also the accumulator layout.
    //      With fp32 inputs waves 4-7 build the Kt tiles meanwhile.
    const int g4 = 4 * gq;
    // A layout of the block (R0, J0) of A, J0 < R0: A[16R0 + m][16J0 + 4g + s]
    auto a_of_A = [&](int R0, int J0, float x[4]) {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) x[s2] = sm.M[(16 * J0 + g4 + s2) * S::kMP + 16 * R0 + m];
    };
    // B layout of the block (J0, I0) of T, J0 >= I0 (diagonal blocks masked)
    auto b_of_T = [&](int J0, int I0, float x[4]) {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const float t = sm.M[(16 * J0 + g4 + s2) * S::kMP + 16 * I0 + m];
        x[s2] = (J0 > I0 || g4 + s2 >= m) ? t : 0.f;
      }
    };
    // A layout of the block (R0, K0) of T, R0 >= K0 (diagonal blocks masked)
    auto a_of_T = [&](int R0, int K0, float x[4]) {
      const f32x4 t = ld4(sm.M + (16 * R0 + m) * S::kMP + 16 * K0 + g4);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) x[s2] = (R0 > K0 || g4 + s2 <= m) ? t[s2] : 0.f;
    };
    auto as4 = [](const f32x4& c, float x[4]) { x[0] = c[0]; x[1] = c[1]; x[2] = c[2]; x[3] = c[3]; };
    // -c stored as the block (R0, I0) of T
    auto store_negT = [&](int R0, int I0, const f32x4& c) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sm.M[(16 * R0 + g4 + ii) * S::kMP + 16 * I0 + m] = -c[ii];
    };

    // Diagonal blocks, wave w < 4 takes block w: with L the strictly lower
    // block of A, (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8) since L^16 = 0.
    // The A layout of X^T is the B layout of X, so the squares are formed in
    // both orientations, each from the other's accumulators.
    if (w < 4) {
      float aL[4], bL[4];
      {
        const f32x4 t = ld4(sm.M + (f + m) * S::kMP + f + g4);   // L[4g+s][m] = M[f+m][f+4g+s]
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          bL[s2] = (g4 + s2 > m) ? t[s2] : 0.f;
          const float u = sm.M[(f + g4 + s2) * S::kMP + f + m];   // L[m][4g+s]
          aL[s2] = (m > g4 + s2) ? u : 0.f;
        }
      }
      const f32x4 z = {0, 0, 0, 0};
      f32x4 L2 = z, L2t = z, L4 = z, L4t = z, L8t = z;
      mma16_f32(L2, aL, bL);     // L L
      mma16_f32(L2t, bL, aL);    // L^T L^T: accumulators = A layout of L^2
      float x[4], y[4];
      as4(L2t, x); as4(L2, y);
      mma16_f32(L4, x, y);       // L^2 L^2
      as4(L2, x); as4(L2t, y);
      mma16_f32(L4t, x, y);      // (L^T)^4: A layout of L^4
      as4(L4, x); as4(L4t, y);
      mma16_f32(L8t, x, y);      // (L^T)^8: A layout of L^8
      f32x4 P;
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) P[s2] = (g4 + s2 == m ? 1.f : 0.f) - bL[s2];   // I - L
      as4(L2t, x); as4(P, y);
      mma16_f32(P, x, y);        // (I + L^2)(I - L)
      as4(L4t, x); as4(P, y);
      mma16_f32(P, x, y);
      as4(L8t, x); as4(P, y);
      mma16_f32(P, x, y);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        if (g4 + ii >= m) sm.M[(f + g4 + ii) * S::kMP + f + m] = P[ii];
    } else if constexpr (!S::kXT) {
      for (int t = w - 4; t < NKT / 2; t += 4) kt_tile(t);
    }
    block_sync();

    // Off-diagonal blocks in two levels: T_10 and T_32 from the diagonal
    // blocks, then T_20, T_21, T_30, T_31 from those, T_RI = -T_RR sum_J A_RJ T_JI.
    f32x4 y0 = {0, 0, 0, 0}, y1 = {0, 0, 0, 0};
    if (w < 4) {
      float a[4], b[4];
      if (w == 0) {          // T_10 = -D_1 A_10 D_0; then A_20 D_0 for T_20
        f32x4 t = {0, 0, 0, 0}, u = {0, 0, 0, 0};
        b_of_T(0, 0, b);
        a_of_A(1, 0, a); mma16_f32(t, a, b);
        a_of_A(2, 0, a); mma16_f32(y0, a, b);
        a_of_T(1, 1, a); as4(t, b); mma16_f32(u, a, b);
        store_negT(1, 0, u);
      } else if (w == 1) {   // T_32 = -D_3 A_32 D_2; then A_21 D_1 and A_31 D_1 for T_31
        f32x4 t = {0, 0, 0, 0}, u = {0, 0, 0, 0};
        b_of_T(2, 2, b);
        a_of_A(3, 2, a); mma16_f32(t, a, b);
        b_of_T(1, 1, b);
        a_of_A(2, 1, a); mma16_f32(y0, a, b);
        a_of_A(3, 1, a); mma16_f32(y1, a, b);
        a_of_T(3, 3, a); as4(t, b); mma16_f32(u, a, b);
        store_negT(3, 2, u);
      } else if (w == 2) {   // A_21 D_1 for T_21
        b_of_T(1, 1, b);
        a_of_A(2, 1, a); mma16_f32(y0, a, b);
      } else {               // A_20 D_0 and A_30 D_0 for T_30
        b_of_T(0, 0, b);
        a_of_A(2, 0, a); mma16_f32(y0, a, b);
        a_of_A(3, 0, a); mma16_f32(y1, a, b);
      }
    } else if constexpr (!S::kXT) {
      for (int t = NKT / 2 + w - 4; t < 3 * NKT / 4; t += 4) kt_tile(t);
    }
    block_sync();
    if (w < 4) {
      float a[4], b[4];
      f32x4 u = {0, 0, 0, 0};
      if (w == 0) {          // T_20 = -D_2 (A_20 D_0 + A_21 T_10)
        a_of_A(2, 1, a); b_of_T(1, 0, b); mma16_f32(y0, a, b);
        a_of_T(2, 2, a); as4(y0, b); mma16_f32(u, a, b);
        store_negT(2, 0, u);
      } else if (w == 1) {   // T_31 = -(T_32 A_21 D_1 + D_3 A_31 D_1)
        a_of_T(3, 2, a); as4(y0, b); mma16_f32(u, a, b);
        a_of_T(3, 3, a); as4(y1, b); mma16_f32(u, a, b);
        store_negT(3, 1, u);
      } else if (w == 2) {   // T_21 = -D_2 A_21 D_1
        a_of_T(2, 2, a); as4(y0, b); mma16_f32(u, a, b);
        store_negT(2, 1, u);
      } else {               // T_30 = -(T_32 (A_20 D_0 + A_21 T_10) + D_3 (A_30 D_0 + A_31 T_10))
        b_of_T(1, 0, b);
        a_of_A(2, 1, a); mma16_f32(y0, a, b);
        a_of_A(3, 1, a); mma16_f32(y1, a, b);
        a_of_T(3, 2, a); as4(y0, b); mma16_f32(u, a, b);
        a_of_T(3, 3, a); as4(y1, b); mma16_f32(u, a, b);
        store_negT(3, 0, u);
      }
    } else if constexpr (!S::kXT) {
      for (int t = 3 * NKT / 4 + w - 4; t < NKT; t += 4) kt_tile(t);
    }
    block_sync();

    // ---- T fragments (row r of block rb, k = i): T and T diag(beta); T[r][i] = 0 for i > r
    auto t_frag = [&](int rb, int kb, bool with_beta) {
      const int r = 16 * rb + m;
      float x[8];
      const f32x4 a = ld4(sm.M + r * S::kMP + 32 * kb + 4 * gq), c4 = ld4(sm.M + r * S::kMP + 32 * kb + 16 + 4 * gq);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 32 * kb + kperm(gq, j);
        const float tv = j < 4 ? a[j] : c4[j - 4];
        x[j] = (i <= r) ? (with_beta ? tv * sm.beta[i] : tv) : 0.f;
      }
      PT fr;
      fr.set(x);
      return fr;
    };
    // With bf16 inputs the twelve fragments W and U use ((rb, kb) with
    // kb <= rb / 2, without and with beta) are built once, into the dead
    // partial-tile buffer, instead of by every wave.
    constexpr bool kTShared = !S::kRedInQ && 12 * tile_bytes<PT>() <= S::kRedFloats * 4;
    char* tfr = reinterpret_cast<char*>(sm.red_buf());
    auto t_index = [](int rb, int kb, bool with_beta) { return (with_beta ? 6 : 0) + (rb < 2 ? rb : 2 * rb - 2) + kb; };
    auto t_get = [&](int rb, int kb, bool with_beta) {
      if constexpr (kTShared) {
        PT f;
        f.load(tfr + t_index(rb, kb, with_beta) * tile_bytes<PT>(), lane);
        return f;
      } else {
        return t_frag(rb, kb, with_beta);
      }
    };

    if constexpr (kTShared) {
      for (int tt = w; tt < 12; tt += kIntraWaves) {
        const int pr = tt % 6, rb = pr < 2 ? pr : (pr + 2) / 2, kb = pr < 2 ? 0 : pr & 1;
        t_frag(rb, kb, tt >= 6).store(tfr + tt * tile_bytes<PT>(), lane);
      }
    }
    block_sync();
    if (tid < K) reinterpret_cast<float*>(rec + L::kGc)[tid] = __expf(sm.G[(kChunk - 1) * S::kGP + tid]);

    // ---- -W: W^T tiles D[c][r] for key-channel block cb = w and every row
    //      block; a W operand tile spans two channel blocks, so each wave
    //      writes its half of every lane's fragment
    if (w < K / 16) {
      PX xf[2];
      const int c = 16 * w + m;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 32 * kb + kperm(gq, j);
          x[j] = sm.beta[i] * ld1(kbuf + SK::idx(i, c)) * sm.nk[i] * __expf(sm.G[i * S::kGP + c]);
        }
        xf[kb].set(x);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb > rb / 2) continue;
          mma(acc, xf[kb], t_get(rb, kb, false));
        }
        const float wv[4] = {-acc[0], -acc[1], -acc[2], -acc[3]};
        PW::store_half(rec + L::kWn + (int64_t)(rb * (K / 32) + w / 2) * tile_bytes<PW>(), lane, w & 1, wv);
      }
    }

    // ---- U = T diag(beta) V for value block vb = w: v has landed in the g buffer
    wait_loads();
    block_sync();   // k is dead: the next item's keys stream in
    if (has_next) issue_k(nxt);
    if (len < kChunk)
      for (int e = tid; e < (kChunk - len) * V; e += kIntraThreads) gvbuf[SV::idx(len + e / V, e % V)] = TI(0);
    block_sync();
    if (w < V / 16) {
      PV vf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = ld1(gvbuf + SV::idx(32 * kb + kperm(gq, j), 16 * w + m));
        vf[kb].set(x);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb > rb / 2) continue;
          mma(acc, t_get(rb, kb, true), vf[kb]);
        }
        reinterpret_cast<f32x4*>(rec + L::kU)[(rb * (V / 16) + w) * kWave + lane] = acc;
      }
    }
    block_sync();   // k and the g/v buffer are free
    if (!S::kDB && has_next) issue_gb(nxt, 0);
  }
}


// The next item of a workgroup that takes its items from a counter: thread 0
// draws a ticket when the item starts (the atomic's latency passes under the
// item's first phases: its answer is needed only before the third barrier);
// tickets past the n_items - gridDim.x items left after every workgroup's
// first mean none.  Items are handed out from the last down, as with a fixed
// stride, so the first chunks still run last.
struct TicketNextItem {
  int64_t* s_next;
  TableHeader* hdr;
  int64_t n_items, grid;
  uint32_t ticket;   // thread 0's
  __device__ void draw() {   // only while items outnumber workgroups (else the counter is not zeroed)
    if (threadIdx.x == 0 && n_items > grid) ticket = atomicAdd(&hdr->item_ticket, 1u);
  }
  __device__ void publish() const {
    if (threadIdx.x == 0) {
      const int64_t t = grid + (int64_t)ticket;
      *s_next = n_items > grid && t < n_items ? n_items - 1 - t : -1;
    }
  }
  __device__ int64_t operator()() const { return uniform_i64(s_next); }
  __device__ ItemInfo info(const IntraParams& p, int64_t item) const { return item_info(p, item_pos(p, item)); }
};

// bf16 inputs: workgroups of four waves, two per CU (about 66 KB of LDS
// each), each running item n_items - 1 - blockIdx.x first and then the
// items its tickets name (the counter is zeroed before the launch), so that
// workgroups that run faster take more items: the per-item time varies
// between compute units, and a fixed share of eight items per workgroup
// left the last workgroups finishing 40 µs after the first.  A workgroup
// loads the next item's rows while it finishes the current one.
template <int K, int V>
__global__ __launch_bounds__(256, 2) void kda_intra4_kernel(IntraParams p) {
  extern __shared__ __align__(16) char smem_raw[];
  __shared__ int64_t s_next;
  const int64_t n_items = p.packed ? (int64_t)p.hdr->n_chunks * p.H : p.B * p.nc_fixed * p.H;
  // No tables without segments: the flags start clear (debug builds clear
  // them before the launch, since their checks may raise flags meanwhile).
  if (!KDA_DEBUG_CHECKS && !p.packed && blockIdx.x == 0 && threadIdx.x == 0) p.hdr->flags = 0;
  int64_t item = n_items - 1 - (int64_t)blockIdx.x;
  if (item < 0) return;
  TicketNextItem nxi{&s_next, p.hdr, n_items, (int64_t)gridDim.x, 0u};
  ItemRows<K> in = load_item_rows<K>(p, item), nx;
  for (;;) {
    nxi.draw();
    intra4_item<K, V>(p, item, smem_raw, in, nxi, nx);
    const int64_t next = uniform_i64(&s_next);
    if (next < 0) break;
    block_sync();
    in = nx;
    item = next;
  }
}

template <int K, int V>
hipError_t launch_intra4_t(const CallArgs& a) {
  IntraParams p{a.q, a.k, a.v, a.g, a.beta, a.gate_mode, a.lower_bound, a.a_log, a.dt_bias, a.B, a.T, a.H,
                a.scale, a.l2norm, a.nc_fixed,
                a.n_max > 0, a.hdr, a.chunks, a.records, a.record_bytes};
  const size_t smem = sizeof(Intra4Smem<K, V>);
  auto kern = kda_intra4_kernel<K, V>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  const int64_t items = (a.n_max > 0 ? a.cmax : a.B * a.nc_fixed) * a.H;
  if (items <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>(items, 2 * (int64_t)cu_count());
  if (a.n_max == 0 && items > (int64_t)grid) {   // with segment ids the table kernel zeroes the item counter
    e = launch_fill_zero(reinterpret_cast<float*>(&a.hdr->item_ticket), 1, a.stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), smem, a.stream, p);
  return hipGetLastError();
}

template <class TI, int K, int V>
hipError_t launch_intra_t(const CallArgs& a) {
  IntraParams p{a.q, a.k, a.v, a.g, a.beta, a.gate_mode, a.lower_bound, a.a_log, a.dt_bias, a.B, a.T, a.H,
                a.scale, a.l2norm, a.nc_fixed,
                a.n_max > 0, a.hdr, a.chunks, a.records, a.record_bytes};
  const size_t smem = sizeof(IntraSmem<TI, K, V>);
  auto kern = kda_intra_kernel<TI, K, V>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  const int64_t items = (a.n_max > 0 ? a.cmax : a.B * a.nc_fixed) * a.H;
  if (items <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>(items, cu_count());
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kIntraThreads), smem, a.stream, p);
  return hipGetLastError();
}

}  // namespace

int64_t record_bytes(InType in, int64_t K, int64_t V) {
#define KDA_RB(TI, KK, VV) if (K == KK && V == VV) return RecordLayout<TI, KK, VV>::kBytes;
  if (in == InType::BF16) {
    KDA_RB(uint16_t, 64, 64) KDA_RB(uint16_t, 64, 128) KDA_RB(uint16_t, 128, 64) KDA_RB(uint16_t, 128, 128)
  } else {
    KDA_RB(float, 64, 64) KDA_RB(float, 64, 128) KDA_RB(float, 128, 64) KDA_RB(float, 128, 128)
  }
#undef KDA_RB
  return -1;
}

hipError_t launch_intra(const CallArgs& a) {
#define KDA_LI(TI, KK, VV) if (a.K == KK && a.V == VV) return launch_intra_t<TI, KK, VV>(a);
#define KDA_LI4(KK, VV) if (a.K == KK && a.V == VV) return launch_intra4_t<KK, VV>(a);
  if (a.in == InType::BF16) {
    KDA_LI4(64, 64) KDA_LI4(64, 128) KDA_LI4(128, 64) KDA_LI4(128, 128)
  } else {
    KDA_LI(float, 64, 64) KDA_LI(float, 64, 128) KDA_LI(float, 128, 64) KDA_LI(float, 128, 128)
  }
#undef KDA_LI
#undef KDA_LI4
  return hipErrorInvalidValue;
}

// XCDs of the current device: 8 on a gfx950 device with 256 compute units
// (32 per XCD); 0 (unknown) elsewhere, which keeps the fused forward off.
int xcd_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    hipDeviceProp_t prop;
    int n = -1;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
        prop.multiProcessorCount % 32 == 0 && prop.multiProcessorCount / 32 <= 8)
      n = prop.multiProcessorCount / 32;
    cached[dev] = n;
  }
  return cached[dev] > 0 ? cached[dev] : 0;
}

// Compute units of the current device (cached per device).
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace kda
