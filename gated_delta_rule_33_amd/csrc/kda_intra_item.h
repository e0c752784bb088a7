// The bf16 intra-chunk item (everything of one (chunk, head) that does not
// depend on the recurrent state) as a device function, shared by the
// standalone intra-chunk kernel and the fused forward, with the item
// decoding and small helpers both use.
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
// which the recurrence evaluates; the item writes the S0-free operands of
// those three lines to its record (RecordLayout in kda_common.h).
#pragma once
#include "kda_launch.h"

namespace kda {
namespace detail {

constexpr float kSpanMax = 64.f;   // natural-log span limit of the split diagonal block
constexpr float kLog2e = 1.4426950408889634f;
// 2^x on the hardware exponential (G differences below are in log2 units).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// A copy of x the compiler cannot see through.  Per-lane addresses derived
// from it inside an item loop are recomputed per item instead of being
// hoisted out of the loop, where they would all stay live and spill.
__device__ __forceinline__ int opaque(int x) {
  int y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  return y;
}
// Activated log decay of the in-kernel gate for z = exp(A_log) (g + dt_bias):
// mode 2 (safe gate) lower_bound * sigmoid(z), mode 1 log sigmoid(z) in the
// form min(z, 0) - log(1 + exp(-|z|)), which neither overflows nor cancels.
// Hardware exp, log and reciprocal (about one ulp each): the absolute error
// of g stays near 1e-7, far below what the bf16 operands carry.
__device__ __forceinline__ float gate_log_decay(int mode, float lower_bound, float z) {
  if (mode == 2) return lower_bound * __builtin_amdgcn_rcpf(1.f + __expf(-z));
  return fminf(z, 0.f) - __logf(1.f + __expf(-fabsf(z)));
}

// Four consecutive elements as floats.
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld4(const uint16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
               __uint_as_float(v.y & 0xffff0000u)};
}
// 16-deep fp32 product on the matrix cores: element s of lane group g holds k = 4g + s.
__device__ __forceinline__ void mma16_f32(f32x4& c, const float a[4], const float b[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
}

struct IntraParams {
  const void *q, *k, *v, *g, *beta;
  int gate_mode;               // 0: g is the log decay; 1: log sigmoid(z); 2: lower_bound * sigmoid(z)
  float lower_bound;
  const float *a_log, *dt_bias;
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

struct ItemInfo {
  int64_t h, tok0;   // head, first token's row index b * T + t0
  int len;
};

// Position of an item = chunk * H + h, with chunk = b * nc_fixed + ci for
// fixed rows.  Integer division is a long instruction sequence on the GPU,
// so it is done once per workgroup; the item loop advances the position by
// a constant stride with carries.
struct ItemPos {
  int64_t chunk, h, b, ci;
};

__device__ __forceinline__ ItemPos item_pos(const IntraParams& p, int64_t item) {
  ItemPos q;
  q.h = item % p.H;
  q.chunk = item / p.H;
  q.b = p.packed ? 0 : q.chunk / p.nc_fixed;
  q.ci = p.packed ? 0 : q.chunk % p.nc_fixed;
  return q;
}

// q moved back by d (a position used as a stride: d.chunk whole chunks and
// d.h heads, d.ci < nc_fixed after d.b whole rows), with borrows instead of
// an integer division per item.
__device__ __forceinline__ ItemPos item_retreat(const IntraParams& p, ItemPos q, const ItemPos& d) {
  q.h -= d.h;
  q.chunk -= d.chunk;
  q.b -= d.b;
  q.ci -= d.ci;
  if (q.h < 0) {
    q.h += p.H;
    q.chunk -= 1;
    q.ci -= 1;
  }
  if (!p.packed && q.ci < 0) {
    q.ci += p.nc_fixed;
    q.b -= 1;
  }
  return q;
}

__device__ __forceinline__ ItemInfo item_info(const IntraParams& p, const ItemPos& q) {
  ItemInfo it;
  it.h = q.h;
  if (p.packed) {
    const ChunkEntry ce = p.chunks[q.chunk];
    it.tok0 = (int64_t)ce.b * p.T + ce.t0;
    it.len = ce.len;
  } else {
    const int64_t t0 = q.ci * kChunk;
    it.tok0 = q.b * p.T + t0;
    it.len = (int)min<int64_t>(kChunk, p.T - t0);
  }
  return it;
}

// ---------------------------------------------------------------------------
// bf16 inputs: one (chunk, head) item per workgroup of four waves, wave R
// owning the 16-row block R.  The arithmetic is that of the kernel above (the
// same exponent splits, operand precisions and record), organised for
// throughput: each wave keeps its rows of q, k and the running sum G in
// registers in operand-fragment order (lane (m, g): row 16R + m, channels
// 32 kb + kperm(g, j)), the running sum over the 16 rows of a block is a DPP
// scan within the wave, and the workgroup needs about 66 KB of LDS, so two
// items are in flight per compute unit and one item's barrier waits are
// filled by the other's work.
template <int K, int V>
struct Intra4Smem {
  static constexpr int KB = K / 32;
  static constexpr int XP = K + 4;    // row pitch (floats) of X
  static constexpr int MP = 68;       // row pitch of M
  static constexpr int VP = V + 8;    // row pitch (bf16) of the value rows
  float Gf[4][K];      // G of the first row of each 16-row block
  float Gl[4][K];      // G of the last row of each block
  float d[10][K];      // exp(G_f(R) - G_l(I)), I <= R, at row R (R + 1) / 2 + I
  float ktf[4][K];     // exp(G_C - G_l(I))
  float gff[4][K];     // exp(G_f(R))
  float beta[64];
  float nk[64];        // key norm factors (1 without the in-kernel L2 norm)
  union {
    float tot[4][K];   // per-block sums of g (running-sum phase)
    float M[64 * MP];  // A^T above the diagonal, T = (I + A)^-1 below it
  };
  union {
    float X[64 * XP];            // k exp(G_l(I) - G), rows of the chunk (A, Aqk and Kt)
    float KG[64 * XP];           // then nk k exp(G) (W)
    uint16_t v[64 * VP];         // then the value rows (U)
  };
};

template <int D>
__device__ __forceinline__ float dpp_shr(float x) {   // lane m - D of the same 16-lane row, 0 for m < D
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 | D, 0xF, 0xF, true));
}

// Elements 0..3 and 4..7 of a fragment at float offset o of a row: channels
// o + 4g .. +3 and o + 16 + 4g .. +3.
__device__ __forceinline__ void frag_rd(const float* row, int o, int g, float x[8]) {
  const f32x4 a = ld4(row + o + 4 * g), b = ld4(row + o + 16 + 4 * g);
#pragma unroll
  for (int j = 0; j < 4; ++j) { x[j] = a[j]; x[4 + j] = b[j]; }
}
__device__ __forceinline__ void frag_wr(float* row, int o, int g, const float x[8]) {
  *reinterpret_cast<f32x4*>(row + o + 4 * g) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(row + o + 16 + 4 * g) = f32x4{x[4], x[5], x[6], x[7]};
}
// Eight bf16 inputs at channels o + 4g .. +3 and o + 16 + 4g .. +3 of a row in memory, widened.
__device__ __forceinline__ void frag_ld_bf16(const uint16_t* row, int o, int g, float x[8]) {
  const uint2 a = *reinterpret_cast<const uint2*>(row + o + 4 * g);
  const uint2 b = *reinterpret_cast<const uint2*>(row + o + 16 + 4 * g);
  x[0] = __uint_as_float(a.x << 16); x[1] = __uint_as_float(a.x & 0xffff0000u);
  x[2] = __uint_as_float(a.y << 16); x[3] = __uint_as_float(a.y & 0xffff0000u);
  x[4] = __uint_as_float(b.x << 16); x[5] = __uint_as_float(b.x & 0xffff0000u);
  x[6] = __uint_as_float(b.y << 16); x[7] = __uint_as_float(b.y & 0xffff0000u);
}

// The raw inputs of one lane of an item: its row of q, k and g (bf16 pairs in
// fragment order: channels 32 kb + 4 gq .. +3 in [kb][0], 32 kb + 16 + 4 gq
// .. +3 in [kb][1]) and its beta, with `keep` all ones, or for rows past
// the chunk's end the first row's values with `keep` zero (applied when the
// rows are widened, so that nothing waits for the loads before then).  Kept
// packed (50 registers), so that the next item's can be in flight while the
// current item finishes.
template <int K>
struct ItemRows {
  uint2 q[K / 32][2], k[K / 32][2], g[K / 32][2];
  uint32_t beta, keep;
  ItemInfo it;   // the item's head, first token and length
};

template <int K>
__device__ __forceinline__ ItemRows<K> load_item_rows(const IntraParams& p, const ItemInfo& it) {
  constexpr int KB = K / 32;
  const int tid = opaque((int)threadIdx.x) & 255;
  const int m = tid & 15, gq = (tid >> 4) & 3, r_own = 16 * (tid >> 6) + m;
  ItemRows<K> x;
  x.it = it;
  // Rows past the chunk's end read the chunk's first row (always present),
  // so that no load is conditional.
  const bool row_ok = r_own < it.len;
  x.keep = row_ok ? 0xffffffffu : 0u;
  const int64_t tok = it.tok0 + (row_ok ? r_own : 0);
  const int64_t off = (tok * p.H + it.h) * K;
  const uint16_t* qr = static_cast<const uint16_t*>(p.q) + off;
  const uint16_t* kr = static_cast<const uint16_t*>(p.k) + off;
  const uint16_t* gr = static_cast<const uint16_t*>(p.g) + off;
  auto ld = [&](const uint16_t* r, int o) { return *reinterpret_cast<const uint2*>(r + o); };
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int o = 32 * kb + 16 * hf + 4 * gq;
      x.q[kb][hf] = ld(qr, o);
      x.k[kb][hf] = ld(kr, o);
      x.g[kb][hf] = ld(gr, o);
    }
  }
  x.beta = (uint32_t) static_cast<const uint16_t*>(p.beta)[tok * p.H + it.h];
  return x;
}

template <int K>
__device__ __forceinline__ ItemRows<K> load_item_rows(const IntraParams& p, int64_t item) {
  return load_item_rows<K>(p, item_info(p, item_pos(p, item)));
}

// An int64 that every lane of the wave holds alike (read from LDS), as a scalar.
__device__ __forceinline__ int64_t uniform_i64(const int64_t* lds) {
  const int64_t v = *lds;
  const int lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)(uint64_t)v);
  const int hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

__device__ __forceinline__ void widen8(const uint2 a[2], uint32_t keep, float x[8]) {
  const uint32_t w[4] = {a[0].x & keep, a[0].y & keep, a[1].x & keep, a[1].y & keep};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// No next item (see intra4_item).
struct NoNextItem {
  __device__ void publish() const {}
  __device__ int64_t operator()() const { return -1; }
  __device__ ItemInfo info(const IntraParams& p, int64_t item) const { return item_info(p, item_pos(p, item)); }
};

// One (chunk, head) item by the four waves of the calling workgroup, in the
// LDS at smem_raw (sizeof(Intra4Smem<K, V>) bytes), from the rows `in` that
// this lane loaded with load_item_rows.  Once this item's own rows are no
// longer needed, next_item() (called by every lane, after the item's first
// barriers, with a result alike in all lanes) names the next item this
// workgroup will run, next_item.info(p, item) its head, tokens and length,
// (next_item.publish(), called by every lane before the item's third
// barrier, lets thread 0 put that answer in LDS), and that item's rows are
// loaded into `next` (nothing for -1), so that their
// latency overlaps the rest of this item.  kEarlyV issues the item's value
// loads before the solve instead of after it (16 more registers live through
// the solve).  The caller separates consecutive items with a barrier.
template <int K, int V, bool kEarlyV = true, class NextItem>
__device__ __forceinline__ void intra4_item(const IntraParams& p, int64_t item, char* smem_raw,
                                            const ItemRows<K>& in, const NextItem& next_item, ItemRows<K>& next) {
  using S = Intra4Smem<K, V>;
  using P = Prec<uint16_t>;
  using PA = typename P::A;
  using PT = typename P::T;
  using PX = typename P::X;
  using PV = typename P::V;
  using PW = typename P::W;
  using PK = typename P::Kt;
  using PQ = typename P::Qg;
  using PAq = typename P::Aq;
  using L = RecordLayout<uint16_t, K, V>;
  constexpr int KB = K / 32;
  constexpr int CBW = K / 64;   // key-channel blocks of W per wave
  constexpr int VBW = V / 64;   // value blocks of U per wave
  S& sm = *reinterpret_cast<S*>(smem_raw);

  const int tid = opaque((int)threadIdx.x) & 255, lane = tid & 63;
  const int R = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, gq = lane >> 4;
  const int f = 16 * R, r_own = f + m;
  const int64_t H = p.H;
  const ItemInfo it = in.it;
  const int len = it.len;
  const int64_t h = it.h;
  char* rec = p.records + item * p.record_bytes;
  const bool row_ok = r_own < len;

  // ---- this lane's row of q, k and g (fragment order) and beta
  float qx[KB][8], kx[KB][8], gx[KB][8];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    widen8(in.q[kb], in.keep, qx[kb]);
    widen8(in.k[kb], in.keep, kx[kb]);
    widen8(in.g[kb], in.keep, gx[kb]);
  }
  const float beta_own = bits_to_f32((uint16_t)(in.beta & in.keep));
  if (KDA_DEBUG_CHECKS && p.gate_mode == 0) {   // g is the log decay: g <= 0 is a precondition
    bool pos = false;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) pos = pos || gx[kb][j] > 0.f;
    flag_if_any(&p.hdr->flags, pos, KDA_FLAG_GATE_POSITIVE);
  }
  if (p.gate_mode && row_ok) {
    // In-kernel gate: z = exp(A_log_h) (g + dt_bias_hc), log decay lower_bound
    // * sigmoid(z) under the safe gate, else log sigmoid(z).
    const float ea = p.a_log ? __expf(p.a_log[h]) : 1.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float db[8];   // dt_bias is only float-aligned: element loads
#pragma unroll
      for (int j = 0; j < 8; ++j) db[j] = p.dt_bias ? p.dt_bias[h * K + 32 * kb + kperm(gq, j)] : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) gx[kb][j] = gate_log_decay(p.gate_mode, p.lower_bound, ea * (gx[kb][j] + db[j]));
    }
  }

  // ---- running sum of g over the rows: inclusive scan over the block's 16
  //      rows (lanes m of one 16-lane row), then the sums of earlier blocks.
  //      G is carried in log2 units (G log2 e) from here on, so each
  //      exponential below is one hardware exp2.
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = gx[kb][j] * kLog2e;
      x += dpp_shr<1>(x);
      x += dpp_shr<2>(x);
      x += dpp_shr<4>(x);
      x += dpp_shr<8>(x);
      gx[kb][j] = x;
    }
    if (m == 15) frag_wr(sm.tot[R], 32 * kb, gq, gx[kb]);
  }
  block_sync();   // B0: block sums
#pragma unroll
  for (int J = 0; J < 3; ++J) {
    if (J >= R) break;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float t[8];
      frag_rd(sm.tot[J], 32 * kb, gq, t);
#pragma unroll
      for (int j = 0; j < 8; ++j) gx[kb][j] += t[j];
    }
  }
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    if (m == 0) frag_wr(sm.Gf[R], 32 * kb, gq, gx[kb]);
    if (m == 15) frag_wr(sm.Gl[R], 32 * kb, gq, gx[kb]);
  }
  block_sync();   // B1: first and last rows of every block

  // ---- per-wave factor rows (read back only by this wave until B2):
  //      d(R, I) for I <= R, exp(G_f(R)); and for block R the row
  //      exp(G_C - G_l(R)) used by every wave after B2
#pragma unroll
  for (int cc = 0; cc < K / kWave; ++cc) {
    const int c = lane + kWave * cc;
    const float gf = sm.Gf[R][c], gl = sm.Gl[R][c], gc = sm.Gl[3][c];
#pragma unroll
    for (int I = 0; I < 4; ++I)
      if (I <= R) sm.d[R * (R + 1) / 2 + I][c] = exp2_hw(gf - sm.Gl[I][c]);
    sm.gff[R][c] = exp2_hw(gf);
    sm.ktf[R][c] = exp2_hw(gc - gl);
    if (R == 3) reinterpret_cast<float*>(rec + L::kGc)[c] = exp2_hw(gc);
  }
  // Norms of this lane's row (all four lane groups hold a quarter of its channels).
  float nqr = 1.f, nkr = 1.f;
  if (p.l2norm) {
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) { sq += qx[kb][j] * qx[kb][j]; sk += kx[kb][j] * kx[kb][j]; }
    sq += __shfl_xor(sq, 16); sq += __shfl_xor(sq, 32);
    sk += __shfl_xor(sk, 16); sk += __shfl_xor(sk, 32);
    nqr = 1.f / sqrtf(sq + 1e-6f);
    nkr = 1.f / sqrtf(sk + 1e-6f);
  }
  if (gq == 0) {
    sm.beta[r_own] = beta_own;
    sm.nk[r_own] = nkr;
  }
  // Span of the block's running sum: the split exp(G_r - G_f) exp(G_f - G_i)
  // inside the diagonal block is used while it is at most kSpanMax.
  float span = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    float gfr[8], glr[8];
    frag_rd(sm.Gf[R], 32 * kb, gq, gfr);
    frag_rd(sm.Gl[R], 32 * kb, gq, glr);
#pragma unroll
    for (int j = 0; j < 8; ++j) span = fmaxf(span, gfr[j] - glr[j]);
  }
  span = fmaxf(span, __shfl_xor(span, 16));
  span = fmaxf(span, __shfl_xor(span, 32));
  const bool diag_split = __builtin_amdgcn_readfirstlane(span <= kSpanMax * kLog2e ? 1 : 0) != 0;
  f32x4 accKK[4], accQK[4];
#pragma unroll
  for (int I = 0; I < 4; ++I) { accKK[I] = f32x4{0, 0, 0, 0}; accQK[I] = f32x4{0, 0, 0, 0}; }
  if (!diag_split) {
    // Pair-by-pair evaluation of the diagonal block, exp(G_r - G_i) <= 1
    // (before the rows' q, k and G leave the registers): row r - dd's keys
    // and running sums come from lane m - dd of the same 16-lane row, each
    // lane group sums its quarter of the channels.  Norm factors are applied
    // with the other tiles below.
    // Lane (m, gq) keeps D[i][r = f + m] for i = f + 4 gq + ii, i.e. the
    // step dd = m - 4 gq - ii (each step's sums are alike in the four lane
    // groups of a column).
    f32x4 dKK = {0, 0, 0, 0}, dQK = {0, 0, 0, 0};
#define KDA_DIAG_STEP(DD)                                                              \
    {                                                                                  \
      float pk = 0.f, pq = 0.f;                                                        \
      _Pragma("unroll") for (int kb = 0; kb < KB; ++kb)                                \
      _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                  \
        const float ki = DD == 0 ? kx[kb][j] : dpp_shr<DD>(kx[kb][j]);                 \
        const float gi = DD == 0 ? gx[kb][j] : dpp_shr<DD>(gx[kb][j]);                 \
        const float t = ki * exp2_hw(gx[kb][j] - gi);                                  \
        pk += kx[kb][j] * t;                                                           \
        pq += qx[kb][j] * t;                                                           \
      }                                                                                \
      pk += __shfl_xor(pk, 16); pk += __shfl_xor(pk, 32);                              \
      pq += __shfl_xor(pq, 16); pq += __shfl_xor(pq, 32);                              \
      _Pragma("unroll") for (int ii = 0; ii < 4; ++ii) {                               \
        const bool mine = m - (DD) == 4 * gq + ii;                                     \
        dKK[ii] = mine ? pk : dKK[ii];                                                 \
        dQK[ii] = mine ? pq : dQK[ii];                                                 \
      }                                                                                \
    }
    KDA_DIAG_STEP(0) KDA_DIAG_STEP(1) KDA_DIAG_STEP(2) KDA_DIAG_STEP(3)
    KDA_DIAG_STEP(4) KDA_DIAG_STEP(5) KDA_DIAG_STEP(6) KDA_DIAG_STEP(7)
    KDA_DIAG_STEP(8) KDA_DIAG_STEP(9) KDA_DIAG_STEP(10) KDA_DIAG_STEP(11)
    KDA_DIAG_STEP(12) KDA_DIAG_STEP(13) KDA_DIAG_STEP(14) KDA_DIAG_STEP(15)
#undef KDA_DIAG_STEP
#pragma unroll
    for (int I = 0; I < 4; ++I)
      if (I == R) {
        accKK[I] = dKK;
        accQK[I] = dQK;
      }
  }
  // Row operands k exp(G_r - G_f), q exp(G_r - G_f) (every factor <= 1); the
  // output's operand scale nq q exp(G_r) goes to the record; the column table
  // X = k exp(G_l - G) (every factor <= 1) to LDS.
  PA fkr[KB], fqr[KB];
  lds_wait();   // this wave's exp(G_f) row
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    float gfr[8], glr[8], efr[8];
    frag_rd(sm.Gf[R], 32 * kb, gq, gfr);
    frag_rd(sm.Gl[R], 32 * kb, gq, glr);
    frag_rd(sm.gff[R], 32 * kb, gq, efr);
    float xk[8], xq[8], xg[8], xx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float er = exp2_hw(gx[kb][j] - gfr[j]);
      xk[j] = kx[kb][j] * er;
      xq[j] = qx[kb][j] * er;
      xg[j] = p.scale * nqr * xq[j] * efr[j];
      xx[j] = kx[kb][j] * exp2_hw(glr[j] - gx[kb][j]);
    }
    fkr[kb].set(xk);
    fqr[kb].set(xq);
    PQ qf;
    qf.set(xg);
    qf.store(rec + L::kQg + (int64_t)(R * KB + kb) * tile_bytes<PQ>(), lane);
    frag_wr(sm.X + r_own * S::XP, 32 * kb, gq, xx);
  }
  next_item.publish();
  block_sync();   // B2: X, nk, beta, factor rows
  // The next item's rows (this item's are dead from here on), issued before
  // this item's larger stores.
  {
    const int64_t nx = next_item();
    if (nx >= 0) next = load_item_rows<K>(p, next_item.info(p, nx));
  }

  // ---- A and Aqk for row block R: tiles (I, R) hold D[i][r], I <= R
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      if (I > R || (I == R && !diag_split)) continue;
      float xi[8], di[8], xc[8];
      frag_rd(sm.X + (16 * I + m) * S::XP, 32 * kb, gq, xi);
      frag_rd(sm.d[R * (R + 1) / 2 + I], 32 * kb, gq, di);
#pragma unroll
      for (int j = 0; j < 8; ++j) xc[j] = xi[j] * di[j];
      PA fkc;
      fkc.set(xc);
      mma(accKK[I], fkc, fkr[kb]);
      mma(accQK[I], fkc, fqr[kb]);
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
  // A[r][i] = beta_r D[i][r] (i < r) goes above the diagonal of M, transposed;
  // scale Aqk (i <= r) to the record: the D[i][r] tiles (I, R) are its operand layout.
  {
    const float br = beta_own;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      if (I > R) continue;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * I + 4 * gq + ii;
        if (I < R || i < r_own) sm.M[i * S::MP + r_own] = br * accKK[I][ii];
        accQK[I][ii] = (I < R || i <= r_own) ? p.scale * accQK[I][ii] : 0.f;
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
  // Kt = (k exp(G_C - G))^T tiles [c-block][token slab] from columns of X:
  // k_r exp(G_C - G_r) = X_r exp(G_C - G_l(I(r))).  The waves with fewer A
  // tiles above take more channel blocks: 4, 3, 1, 0 of 8 (K = 128) or
  // 2, 1, 1, 0 of 4 (K = 64).  Each 16-key block is stored as fp16 times
  // 2^s, s putting its largest magnitude in [2^14, 2^15), with 2^-s beside.
  constexpr int NCBK = K / 16;
  auto kt_bound = [](int w) { return NCBK == 8 ? (w == 0 ? 0 : w == 1 ? 4 : w == 2 ? 7 : 8)
                                               : (w == 0 ? 0 : w == 1 ? 2 : w == 2 ? 3 : 4); };
  const int kt_begin = kt_bound(R), kt_end = kt_bound(R + 1);
#pragma unroll
  for (int u = 0; u < NCBK / 2; ++u) {
    const int cb = kt_begin + u, c = 16 * cb + m;
    if (cb >= kt_end) break;
    float kt[2][8];
    float mx = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float xv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xv[j] = sm.X[(32 * kb + kperm(gq, j)) * S::XP + c];   // all reads first
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 32 * kb + kperm(gq, j);
        kt[kb][j] = xv[j] * sm.ktf[r >> 4][c] * sm.nk[r];
        mx = fmaxf(mx, fabsf(kt[kb][j]));
      }
    }
    // max = f 2^e with f in [1/2, 1): 2^(15 - e) brings it into [2^14, 2^15)
    // (for 0, inf and NaN the exponent reads 0, and the values pass as they are).
    const int e = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_frexp_expf(wave_max(mx)));
    const int sh = min(max(15 - e, -100), 100);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = ldexpf(kt[kb][j], sh);
      PK fr;
      fr.set(y);
      fr.store(rec + L::kKt + (int64_t)(cb * 2 + kb) * tile_bytes<PK>(), lane);
    }
    if (lane == 0) reinterpret_cast<float*>(rec + L::kKs)[cb] = ldexpf(1.f, -sh);
  }
  block_sync();   // B3: A^T in M; X is dead
  // W's operand rows nk k exp(G) take X's place (read as columns after the
  // solve), rebuilt from the row operand pair k exp(G - G_f) (hi + lo, about
  // 16 significant bits; the operand is rounded to a pair again).  beta is
  // applied on the T side, which W and U share.
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    float efr[8], kg[8];
    frag_rd(sm.gff[R], 32 * kb, gq, efr);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      kg[j] = nkr * ((float)fkr[kb].hi[j] + (float)fkr[kb].lo[j]) * efr[j];
    frag_wr(sm.KG + r_own * S::XP, 32 * kb, gq, kg);
  }

  // ---- the value rows (16R + l / VPR + 4t, 16-byte piece l % VPR): loaded
  //      here (kEarlyV), so that the solve and -W cover their latency, else
  //      after the solve, and stored to LDS once KG is dead.  Rows past the
  //      chunk's end read the first row (no conditional load) and store zeros.
  constexpr int VPR = V / 8;                  // 16-byte pieces per value row
  constexpr int VT = 16 * VPR / kWave;        // pieces per lane
  uint4 vv[VT];
  auto load_v = [&] {
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      const int e = lane + kWave * t, r = f + e / VPR, pc = e % VPR;
      vv[t] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v) +
                                              ((it.tok0 + (r < len ? r : 0)) * H + h) * V + 8 * pc);
    }
  };
  if constexpr (kEarlyV) load_v();

  // ---- T = (I + A)^-1 by 16x16 blocks on the fp32 matrix path (as above)
  const int g4 = 4 * gq;
  auto a_of_A = [&](int R0, int J0, float x[4]) {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) x[s2] = sm.M[(16 * J0 + g4 + s2) * S::MP + 16 * R0 + m];
  };
  auto b_of_T = [&](int J0, int I0, float x[4]) {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const float t = sm.M[(16 * J0 + g4 + s2) * S::MP + 16 * I0 + m];
      x[s2] = (J0 > I0 || g4 + s2 >= m) ? t : 0.f;
    }
  };
  auto a_of_T = [&](int R0, int K0, float x[4]) {
    const f32x4 t = ld4(sm.M + (16 * R0 + m) * S::MP + 16 * K0 + g4);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) x[s2] = (R0 > K0 || g4 + s2 <= m) ? t[s2] : 0.f;
  };
  auto as4 = [](const f32x4& c, float x[4]) { x[0] = c[0]; x[1] = c[1]; x[2] = c[2]; x[3] = c[3]; };
  auto store_negT = [&](int R0, int I0, const f32x4& c) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) sm.M[(16 * R0 + g4 + ii) * S::MP + 16 * I0 + m] = -c[ii];
  };
  {   // diagonal block R: (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8)
    float aL[4], bL[4];
    const f32x4 t = ld4(sm.M + (f + m) * S::MP + f + g4);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      bL[s2] = (g4 + s2 > m) ? t[s2] : 0.f;
      const float u = sm.M[(f + g4 + s2) * S::MP + f + m];
      aL[s2] = (m > g4 + s2) ? u : 0.f;
    }
    const f32x4 z = {0, 0, 0, 0};
    f32x4 L2 = z, L2t = z, L4 = z, L4t = z, L8t = z;
    mma16_f32(L2, aL, bL);
    mma16_f32(L2t, bL, aL);
    float x[4], y[4];
    as4(L2t, x); as4(L2, y);
    mma16_f32(L4, x, y);
    as4(L2, x); as4(L2t, y);
    mma16_f32(L4t, x, y);
    as4(L4, x); as4(L4t, y);
    mma16_f32(L8t, x, y);
    f32x4 Pm;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) Pm[s2] = (g4 + s2 == m ? 1.f : 0.f) - bL[s2];
    as4(L2t, x); as4(Pm, y);
    mma16_f32(Pm, x, y);
    as4(L4t, x); as4(Pm, y);
    mma16_f32(Pm, x, y);
    as4(L8t, x); as4(Pm, y);
    mma16_f32(Pm, x, y);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
      if (g4 + ii >= m) sm.M[(f + g4 + ii) * S::MP + f + m] = Pm[ii];
  }
  block_sync();   // B4
  f32x4 y0 = {0, 0, 0, 0}, y1 = {0, 0, 0, 0};
  {
    float a[4], b[4];
    if (R == 0) {
      f32x4 t = {0, 0, 0, 0}, u = {0, 0, 0, 0};
      b_of_T(0, 0, b);
      a_of_A(1, 0, a); mma16_f32(t, a, b);
      a_of_A(2, 0, a); mma16_f32(y0, a, b);
      a_of_T(1, 1, a); as4(t, b); mma16_f32(u, a, b);
      store_negT(1, 0, u);
    } else if (R == 1) {
      f32x4 t = {0, 0, 0, 0}, u = {0, 0, 0, 0};
      b_of_T(2, 2, b);
      a_of_A(3, 2, a); mma16_f32(t, a, b);
      b_of_T(1, 1, b);
      a_of_A(2, 1, a); mma16_f32(y0, a, b);
      a_of_A(3, 1, a); mma16_f32(y1, a, b);
      a_of_T(3, 3, a); as4(t, b); mma16_f32(u, a, b);
      store_negT(3, 2, u);
    } else if (R == 2) {
      b_of_T(1, 1, b);
      a_of_A(2, 1, a); mma16_f32(y0, a, b);
    } else {
      b_of_T(0, 0, b);
      a_of_A(2, 0, a); mma16_f32(y0, a, b);
      a_of_A(3, 0, a); mma16_f32(y1, a, b);
    }
  }
  block_sync();   // B5
  {
    float a[4], b[4];
    f32x4 u = {0, 0, 0, 0};
    if (R == 0) {
      a_of_A(2, 1, a); b_of_T(1, 0, b); mma16_f32(y0, a, b);
      a_of_T(2, 2, a); as4(y0, b); mma16_f32(u, a, b);
      store_negT(2, 0, u);
    } else if (R == 1) {
      a_of_T(3, 2, a); as4(y0, b); mma16_f32(u, a, b);
      a_of_T(3, 3, a); as4(y1, b); mma16_f32(u, a, b);
      store_negT(3, 1, u);
    } else if (R == 2) {
      a_of_T(2, 2, a); as4(y0, b); mma16_f32(u, a, b);
      store_negT(2, 1, u);
    } else {
      b_of_T(1, 0, b);
      a_of_A(2, 1, a); mma16_f32(y0, a, b);
      a_of_A(3, 1, a); mma16_f32(y1, a, b);
      a_of_T(3, 2, a); as4(y0, b); mma16_f32(u, a, b);
      a_of_T(3, 3, a); as4(y1, b); mma16_f32(u, a, b);
      store_negT(3, 0, u);
    }
  }
  block_sync();   // B6: T complete
  if constexpr (!kEarlyV) load_v();

  // ---- T diag(beta) fragments (row block rb, token slab kb <= rb / 2):
  //      T[r][i] beta_i, the operand both W and U take
  auto t_frag = [&](int rb, int kb) {
    const int r = 16 * rb + m;
    float x[8];
    const f32x4 a = ld4(sm.M + r * S::MP + 32 * kb + 4 * gq), c4 = ld4(sm.M + r * S::MP + 32 * kb + 16 + 4 * gq);
    const f32x4 b0 = ld4(sm.beta + 32 * kb + 4 * gq), b1 = ld4(sm.beta + 32 * kb + 16 + 4 * gq);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = 32 * kb + kperm(gq, j);
      const float tv = j < 4 ? a[j] * b0[j] : c4[j - 4] * b1[j - 4];
      x[j] = (i <= r) ? tv : 0.f;
    }
    PT fr;
    fr.set(x);
    return fr;
  };
  PT tf[6];   // (rb, kb): (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
  tf[0] = t_frag(0, 0); tf[1] = t_frag(1, 0); tf[2] = t_frag(2, 0);
  tf[3] = t_frag(2, 1); tf[4] = t_frag(3, 0); tf[5] = t_frag(3, 1);
  auto t_idx = [](int rb, int kb) { return rb < 2 ? rb : 2 * rb - 2 + kb; };

  // ---- -W = -(T diag(beta)) (K exp(G)): W^T tiles D[c][r] from columns of KG
#pragma unroll
  for (int u = 0; u < CBW; ++u) {
    const int cb = CBW * R + u, c = 16 * cb + m;
    PX xf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float xw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xw[j] = sm.KG[(32 * kb + kperm(gq, j)) * S::XP + c];
      xf[kb].set(xw);
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb > rb / 2) continue;
        mma(acc, xf[kb], tf[t_idx(rb, kb)]);
      }
      const float wv[4] = {-acc[0], -acc[1], -acc[2], -acc[3]};
      PW::store_half(rec + L::kWn + (int64_t)(rb * KB + cb / 2) * tile_bytes<PW>(), lane, cb & 1, wv);
    }
  }
  block_sync();   // B7: KG is dead; the value rows take its place
#pragma unroll
  for (int t = 0; t < VT; ++t) {
    const int e = lane + kWave * t, r = f + e / VPR, pc = e % VPR;
    *reinterpret_cast<uint4*>(sm.v + r * S::VP + 8 * pc) = r < len ? vv[t] : uint4{0, 0, 0, 0};
  }
  block_sync();   // B8
#pragma unroll
  for (int u = 0; u < VBW; ++u) {
    const int vb = VBW * R + u;
    PV vf[2];   // the bf16 values as they are (no conversion)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        vf[kb].v[j] = __builtin_bit_cast(__bf16, sm.v[(32 * kb + kperm(gq, j)) * S::VP + 16 * vb + m]);
    }
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb > rb / 2) continue;
        mma(acc, tf[t_idx(rb, kb)], vf[kb]);
      }
      reinterpret_cast<f32x4*>(rec + L::kU)[(rb * (V / 16) + vb) * kWave + lane] = acc;
    }
  }
}

}  // namespace detail
}  // namespace kda
