// Intra-chunk kernel of the KDA forward: everything that does not depend on
// the recurrent state, for one (chunk, head) per workgroup.
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
#include "kda_launch.h"

namespace kda {
namespace {

constexpr float kSpanMax = 64.f;

template <class TI, int K, int V>
struct IntraSmem {
  static constexpr int kQP = K + 8;   // row pitch (elements) of q, k
  static constexpr int kVP = V + 8;   // row pitch of v
  static constexpr int kGP = K + 4;   // row pitch (floats) of G / exp(G)
  static constexpr int kMP = 68;      // row pitch of M (T below the diagonal, A^T above)
  TI q[kChunk * kQP];
  TI k[kChunk * kQP];
  TI v[kChunk * kVP];
  float G[kChunk * kGP];
  float M[kChunk * kMP];
  float beta[kChunk];
  float nq[kChunk], nk[kChunk];
  float part[512];
  int span_bits[4];
};

__device__ __forceinline__ float ldf(const float* p, int i) { return p[i]; }
__device__ __forceinline__ float ldf(const uint16_t* p, int i) { return bits_to_f32(p[i]); }

// 16B vector copy of input rows into LDS; rows >= len are zero.
template <class TI, int W_, int PITCH>
__device__ __forceinline__ void load_rows(TI* dst, const TI* src, int64_t row_stride, int len, int tid) {
  constexpr int E = 16 / sizeof(TI);
  constexpr int PER_ROW = W_ / E;
  for (int idx = tid; idx < kChunk * PER_ROW; idx += kThreads) {
    const int r = idx / PER_ROW, cv = idx % PER_ROW;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < len) val = *reinterpret_cast<const uint4*>(src + r * row_stride + cv * E);
    *reinterpret_cast<uint4*>(dst + r * PITCH + cv * E) = val;
  }
}

// 16-deep fp32 product on the matrix cores: element s of lane group g holds k = 4g + s.
__device__ __forceinline__ void mma16_f32(f32x4& c, const float a[4], const float b[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
}

struct IntraParams {
  const void *q, *k, *v, *g, *beta;
  int64_t B, T, H;
  float scale;
  int l2norm;
  int64_t nc_fixed;          // chunks per row (fixed rows)
  int packed;
  TableHeader* hdr;
  const ChunkEntry* chunks;
  char* records;
  int64_t record_bytes;
};

template <class TI, int K, int V>
__global__ __launch_bounds__(kThreads) void kda_intra_kernel(IntraParams p) {
  using S = IntraSmem<TI, K, V>;
  using PA = typename Prec<TI>::A;
  using PT = typename Prec<TI>::T;
  using PX = typename Prec<TI>::X;
  using PV = typename Prec<TI>::V;
  using PW = typename Prec<TI>::W;
  using PK = typename Prec<TI>::Kt;
  using PQ = typename Prec<TI>::Q;
  using L = RecordLayout<TI, K, V>;
  extern __shared__ __align__(16) char smem_raw[];
  S& sm = *reinterpret_cast<S*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m = lane & 15, gq = lane >> 4;
  const TI* gq_ = static_cast<const TI*>(p.q);
  const TI* gk_ = static_cast<const TI*>(p.k);
  const TI* gv_ = static_cast<const TI*>(p.v);
  const TI* gg_ = static_cast<const TI*>(p.g);
  const TI* gb_ = static_cast<const TI*>(p.beta);
  const int64_t H = p.H;
  const int64_t n_items = p.packed ? (int64_t)p.hdr->n_chunks * H : p.B * p.nc_fixed * H;
  if (!p.packed && blockIdx.x == 0 && tid == 0) p.hdr->flags = 0;   // no tables without segments

  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int64_t h = item % H, chunk = item / H;
    int64_t b, t0;
    int len;
    if (p.packed) {
      const ChunkEntry ce = p.chunks[chunk];
      b = ce.b; t0 = ce.t0; len = ce.len;
    } else {
      b = chunk / p.nc_fixed;
      t0 = (chunk % p.nc_fixed) * kChunk;
      len = (int)min<int64_t>(kChunk, p.T - t0);
    }
    char* rec = p.records + item * p.record_bytes;
    const int64_t tok0 = b * p.T + t0;

    // ---- load the chunk (rows >= len are zero: they then contribute nothing)
    load_rows<TI, K, S::kQP>(sm.q, gq_ + (tok0 * H + h) * K, H * K, len, tid);
    load_rows<TI, K, S::kQP>(sm.k, gk_ + (tok0 * H + h) * K, H * K, len, tid);
    load_rows<TI, V, S::kVP>(sm.v, gv_ + (tok0 * H + h) * V, H * V, len, tid);
    if (tid < kChunk) sm.beta[tid] = tid < len ? load_in(gb_, (tok0 + tid) * H + h) : 0.f;
    if (tid < 4) sm.span_bits[tid] = 0;

    // ---- running sum of g over the chunk, per channel
    {
      constexpr int RP = kChunk / (kThreads / K);   // rows per thread
      const int c = tid % K, part = tid / K, r0 = part * RP;
      float run = 0.f;
      for (int r = r0; r < r0 + RP; ++r) {
        const float gv = r < len ? load_in(gg_, ((tok0 + r) * H + h) * K + c) : 0.f;
        run += gv;
        sm.G[r * S::kGP + c] = run;
      }
      sm.part[part * K + c] = run;
      __syncthreads();
      float off = 0.f;
      for (int pp = 0; pp < part; ++pp) off += sm.part[pp * K + c];
      if (part > 0)
        for (int r = r0; r < r0 + RP; ++r) sm.G[r * S::kGP + c] += off;
    }
    __syncthreads();

    // ---- q/k normalisation factors and the diagonal-block spans
    {
      const int r = tid >> 2, qtr = tid & 3;
      float sq = 0.f, sk = 0.f;
      if (p.l2norm) {
        for (int c = qtr * (K / 4); c < (qtr + 1) * (K / 4); ++c) {
          const float a = ldf(sm.q, r * S::kQP + c), bb = ldf(sm.k, r * S::kQP + c);
          sq += a * a;
          sk += bb * bb;
        }
        sq += __shfl_xor(sq, 1); sq += __shfl_xor(sq, 2);
        sk += __shfl_xor(sk, 1); sk += __shfl_xor(sk, 2);
      }
      if (qtr == 0) {
        sm.nq[r] = p.l2norm ? 1.f / sqrtf(sq + 1e-6f) : 1.f;
        sm.nk[r] = p.l2norm ? 1.f / sqrtf(sk + 1e-6f) : 1.f;
      }
      for (int e = tid; e < 4 * K; e += kThreads) {
        const int blk = e / K, c = e % K;
        const float span = sm.G[(16 * blk) * S::kGP + c] - sm.G[(16 * blk + 15) * S::kGP + c];
        atomicMax(&sm.span_bits[blk], __float_as_int(fmaxf(span, 0.f)));
      }
    }
    __syncthreads();

    // ---- A and Aqk for row block R = w: tiles (I, R) with D[i][r], I <= R
    const int R = w, f = 16 * R;
    f32x4 accKK[4], accQK[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) { accKK[I] = f32x4{0, 0, 0, 0}; accQK[I] = f32x4{0, 0, 0, 0}; }
    const bool diag_split = __int_as_float(sm.span_bits[R]) <= kSpanMax;
    {
      const int r = f + m;
      const float nqr = sm.nq[r], nkr = sm.nk[r];
      for (int kb = 0; kb < K / 32; ++kb) {
        float xk[8], xq[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = 32 * kb + kperm(gq, j);
          const float e = __expf(sm.G[r * S::kGP + c] - sm.G[f * S::kGP + c]);
          xk[j] = ldf(sm.k, r * S::kQP + c) * nkr * e;
          xq[j] = ldf(sm.q, r * S::kQP + c) * nqr * e;
        }
        PA fkr, fqr;
        fkr.set(xk);
        fqr.set(xq);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          if (I > R || (I == R && !diag_split)) continue;
          const int i = 16 * I + m;
          const float nki = sm.nk[i];
          float xc[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int c = 32 * kb + kperm(gq, j);
            xc[j] = ldf(sm.k, i * S::kQP + c) * nki * __expf(sm.G[f * S::kGP + c] - sm.G[i * S::kGP + c]);
          }
          PA fkc;
          fkc.set(xc);
          mma(accKK[I], fkc, fkr);
          mma(accQK[I], fkc, fqr);
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
            for (int c = 0; c < K; ++c) {
              const float e = __expf(sm.G[r * S::kGP + c] - sm.G[i * S::kGP + c]);
              const float kk = ldf(sm.k, i * S::kQP + c) * nki * e;
              sk_ += ldf(sm.k, r * S::kQP + c) * nkr * kk;
              sq_ += ldf(sm.q, r * S::kQP + c) * nqr * kk;
            }
          }
#pragma unroll
          for (int I = 0; I < 4; ++I)
            if (I == R) { accKK[I][ii] = sk_; accQK[I][ii] = sq_; }
        }
      }
      // A[r][i] = beta_r * D[i][r] (i < r), stored transposed above the diagonal of M.
      const float br = sm.beta[r];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        if (I > R) continue;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int i = 16 * I + 4 * gq + ii;
          if (i < r) sm.M[i * S::kMP + r] = br * accKK[I][ii];
          accQK[I][ii] = (i <= r) ? p.scale * accQK[I][ii] : 0.f;
        }
      }
    }
    __syncthreads();

    // ---- T = (I + A)^-1: invert the four 16x16 diagonal blocks (wave w: block w)
    if (lane < 16) {
      const int j = lane;
      float t[16], acc[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) acc[s] = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        t[r] = (r == j) ? 1.f : (r < j ? 0.f : -acc[r]);
#pragma unroll
        for (int s = r + 1; s < 16; ++s) acc[s] += sm.M[(f + r) * S::kMP + f + s] * t[r];   // A[f+s][f+r]
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r >= j) sm.M[(f + r) * S::kMP + f + j] = t[r];
    }
    __syncthreads();
    // ---- off-diagonal blocks by distance: T_RI = -T_RR sum_{J=I}^{R-1} A_RJ T_JI
    for (int d = 1; d < 4; ++d) {
      const int RR = w + d, II = w;
      if (RR < 4) {
        f32x4 mm = {0, 0, 0, 0};
        for (int J = II; J < RR; ++J) {
          float a[4], bb[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            a[s] = sm.M[(16 * J + 4 * gq + s) * S::kMP + 16 * RR + m];   // A[16RR+m][16J+4gq+s]
            // T[16J+4gq+s][16II+m]; above the diagonal of a diagonal block M holds A^T, T is 0
            bb[s] = (J > II || 4 * gq + s >= m) ? sm.M[(16 * J + 4 * gq + s) * S::kMP + 16 * II + m] : 0.f;
          }
          mma16_f32(mm, a, bb);
        }
        float a[4], bb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          a[s] = (m >= 4 * gq + s) ? sm.M[(16 * RR + m) * S::kMP + 16 * RR + 4 * gq + s] : 0.f;  // T_RR[m][4gq+s]
          bb[s] = mm[s];
        }
        f32x4 res = {0, 0, 0, 0};
        mma16_f32(res, a, bb);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sm.M[(16 * RR + 4 * gq + ii) * S::kMP + 16 * II + m] = -res[ii];
      }
      __syncthreads();
    }

    // ---- Kt = (k * exp(G_C - G))^T as operand tiles [c-block][token k-tile]
    for (int t = w; t < (K / 16) * 2; t += 4) {
      const int cb = t >> 1, kb = t & 1, c = 16 * cb + m;
      const float gc = sm.G[(kChunk - 1) * S::kGP + c];
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 32 * kb + kperm(gq, j);
        x[j] = ldf(sm.k, r * S::kQP + c) * sm.nk[r] * __expf(gc - sm.G[r * S::kGP + c]);
      }
      PK fr;
      fr.set(x);
      fr.store(rec + L::kKt + (int64_t)(cb * 2 + kb) * tile_bytes<PK>(), lane);
    }
    __syncthreads();
    // exp(G) in place of G from here on.
    for (int e = tid; e < kChunk * K; e += kThreads) {
      const int r = e / K, c = e % K;
      sm.G[r * S::kGP + c] = __expf(sm.G[r * S::kGP + c]);
    }
    __syncthreads();
    if (tid < K) reinterpret_cast<float*>(rec + L::kGc)[tid] = sm.G[(kChunk - 1) * S::kGP + tid];

    // ---- -W = -(T diag(beta) (K * exp(G))), computed as W^T tiles D[c][r] for rows r of block w
    {
      const int r = 16 * w + m;
      PT tf[2];
      PT tb[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float xt[8], xtb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 32 * kb + kperm(gq, j);
          const float tv = (i <= r) ? sm.M[r * S::kMP + i] : 0.f;
          xt[j] = tv;
          xtb[j] = tv * sm.beta[i];
        }
        tf[kb].set(xt);
        tb[kb].set(xtb);
      }
      const int nkb = w / 2 + 1;   // T[r][i] = 0 for i > r
      for (int kb2 = 0; kb2 < K / 32; ++kb2) {
        f32x4 acc2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int cb = 2 * kb2 + hh, c = 16 * cb + m;
          acc2[hh] = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (kb >= nkb) continue;
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int i = 32 * kb + kperm(gq, j);
              x[j] = sm.beta[i] * ldf(sm.k, i * S::kQP + c) * sm.nk[i] * sm.G[i * S::kGP + c];
            }
            PX xf;
            xf.set(x);
            mma(acc2[hh], xf, tf[kb]);
          }
        }
        float wv[8];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) { wv[ii] = -acc2[0][ii]; wv[4 + ii] = -acc2[1][ii]; }
        PW wf;
        wf.set(wv);
        wf.store(rec + L::kWn + (int64_t)(w * (K / 32) + kb2) * tile_bytes<PW>(), lane);
      }
      // ---- U = T diag(beta) V, rows of block w, output-tile layout
      for (int vb = 0; vb < V / 16; ++vb) {
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb >= nkb) continue;
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 32 * kb + kperm(gq, j);
            x[j] = ldf(sm.v, i * S::kVP + 16 * vb + m);
          }
          PV vf;
          vf.set(x);
          mma(acc, tb[kb], vf);
        }
        reinterpret_cast<f32x4*>(rec + L::kU)[(w * (V / 16) + vb) * kWave + lane] = acc;
      }
      // ---- scale * q * exp(G), rows of block w
      const float nqr = sm.nq[r];
      for (int kb = 0; kb < K / 32; ++kb) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = 32 * kb + kperm(gq, j);
          x[j] = p.scale * ldf(sm.q, r * S::kQP + c) * nqr * sm.G[r * S::kGP + c];
        }
        PQ qf;
        qf.set(x);
        qf.store(rec + L::kQg + (int64_t)(w * (K / 32) + kb) * tile_bytes<PQ>(), lane);
      }
      // ---- scale * Aqk, rows of block w: D[i][r] tiles (I, w) are the operand layout
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float x[8];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          x[ii] = (2 * kb <= R) ? accQK[2 * kb][ii] : 0.f;
          x[4 + ii] = (2 * kb + 1 <= R) ? accQK[2 * kb + 1][ii] : 0.f;
        }
        PQ af;
        af.set(x);
        af.store(rec + L::kAqk + (int64_t)(w * 2 + kb) * tile_bytes<PQ>(), lane);
      }
    }
    __syncthreads();   // LDS is reused by the next item
  }
}

template <class TI, int K, int V>
hipError_t launch_intra_t(const CallArgs& a) {
  IntraParams p{a.q, a.k, a.v, a.g, a.beta, a.B, a.T, a.H, a.scale, a.l2norm, a.nc_fixed,
                a.n_max > 0, a.hdr, a.chunks, a.records, a.record_bytes};
  const size_t smem = sizeof(IntraSmem<TI, K, V>);
  auto kern = kda_intra_kernel<TI, K, V>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  const int64_t items = (a.n_max > 0 ? a.cmax : a.B * a.nc_fixed) * a.H;
  if (items <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>(items, 1 << 20);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), smem, a.stream, p);
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
  if (a.in == InType::BF16) {
    KDA_LI(uint16_t, 64, 64) KDA_LI(uint16_t, 64, 128) KDA_LI(uint16_t, 128, 64) KDA_LI(uint16_t, 128, 128)
  } else {
    KDA_LI(float, 64, 64) KDA_LI(float, 64, 128) KDA_LI(float, 128, 64) KDA_LI(float, 128, 128)
  }
#undef KDA_LI
  return hipErrorInvalidValue;
}

}  // namespace kda
