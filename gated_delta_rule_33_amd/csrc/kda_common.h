// Device-side building blocks shared by the KDA forward kernels (gfx950).
//
// Matrix products run on the CDNA4 matrix cores with 16x16 output tiles:
//   bf16 operands: v_mfma_f32_16x16x32_bf16 (one instruction per 32-deep slab)
//   fp32 operands: v_mfma_f32_16x16x4_f32   (eight instructions per slab)
// Output tile layout (both): lane l holds column n = l % 16 and the four rows
// m = 4*(l/16) + i, i = 0..3.
// Operand fragments for a 16 x 32 slab: lane l holds row (A) or column (B)
// l % 16 and eight k-indices chosen by its lane group g = l / 16.  Only the
// pairing of A and B elements matters to the sum, so every fragment here
// uses the k-order
//     element j of group g  <->  k = 4g + j          (j < 4)
//                                 k = 16 + 4g + j-4  (j >= 4)
// With that order, two output tiles stacked along m (rows 0-15 and 16-31 of
// a 32-row block) are, lane for lane, an operand fragment whose k runs over
// those 32 rows: a product's result feeds the next product without any
// shuffle or LDS transpose.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

constexpr int kChunk = 64;      // tokens per chunk
constexpr int kSub = 16;        // rows per sub-block of the intra-chunk products
constexpr int kWave = 64;
constexpr int kThreads = 256;   // four waves per workgroup

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Direct-to-LDS loads.  One instruction moves 16 bytes per lane from each
// lane's global address to LDS at (M0 = wave-uniform LDS base) + 16 * lane,
// i.e. 1 KB per wave.  It is issued from inline assembly so that the compiler
// does not treat every later LDS read as dependent on it (it cannot tell the
// LDS blocks apart and would drain all such loads before any LDS read); the
// issuing code waits for the data itself with vm_wait before reading it.  The
// compiler's own waits for its register loads only become longer by it: it
// does not count these loads, so it never assumes fewer are outstanding.
// s_nop covers the M0-write-to-LDS-DMA hazard.
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void dma16(void* lds_base, const void* lane_src) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)lds_base);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(lane_src), "{m0}"(m0) : "memory");
}
// Copy BYTES (a multiple of 1 KB) from src to the LDS block at dst, one wave.
template <int BYTES>
__device__ __forceinline__ void dma_copy(char* dst, const char* src, int lane) {
  static_assert(BYTES % 1024 == 0, "whole 1 KB blocks");
#pragma unroll
  for (int i = 0; i < BYTES / 1024; ++i) dma16(dst + 1024 * i, src + 1024 * i + 16 * lane);
}
// Wait until at most N vector memory operations of this wave are outstanding
// (s_waitcnt vmcnt(N), expcnt and lgkmcnt left open).  The asm statement keeps
// the compiler from moving LDS reads above the wait.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
// Wait for every outstanding LDS operation of this wave (lgkmcnt(0)).
__device__ __forceinline__ void lds_wait() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
  asm volatile("" ::: "memory");
}

// Workgroup barrier for data exchanged through LDS: this wave's LDS reads and
// writes complete, then all waves meet.  __syncthreads() would also wait for
// every outstanding global load of the wave (its workgroup-scope fence counts
// the LDS side of direct-to-LDS loads), which would drain the prefetches that
// are meant to stay in flight across the barrier; those are awaited with
// vm_wait by the code that reads their data.
__device__ __forceinline__ void block_sync() {
  lds_wait();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// k index (0..31) held in element j of lane group g.
__device__ __forceinline__ int kperm(int g, int j) { return (j < 4) ? 4 * g + j : 12 + 4 * g + j; }

__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }   // round to nearest even
__device__ __forceinline__ float from_bf16(__bf16 x) { return (float)x; }

__device__ __forceinline__ float bits_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Two floats rounded to bf16 (nearest even) with one packed conversion.
__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b) { return __builtin_convertvector(f32x2{a, b}, bf16x2); }
// The pair a, b split as hi + lo: hi = bf16(x), lo = bf16(x - hi); two packed
// conversions, the hi values widened back with one shift and one mask.
__device__ __forceinline__ void split_bf16x2(float a, float b, bf16x2& hi, bf16x2& lo) {
  hi = to_bf16x2(a, b);
  const uint32_t hb = __builtin_bit_cast(uint32_t, hi);
  lo = to_bf16x2(a - __uint_as_float(hb << 16), b - __uint_as_float(hb & 0xffff0000u));
}

// Two floats rounded to fp16 (nearest even) with one packed conversion.
__device__ __forceinline__ f16x2 to_f16x2(float a, float b) { return __builtin_convertvector(f32x2{a, b}, f16x2); }

// A zero in a vector register that the compiler cannot see through: a load
// whose address it offsets stays a vector-memory load (counted by vmcnt,
// which barriers here do not wait for) even where the address is uniform.
__device__ __forceinline__ int vector_zero() {
  int y;
  asm volatile("v_mov_b32 %0, 0" : "=v"(y));
  return y;
}

// Largest value of x >= 0 over the wave, as a wave-uniform value: DPP
// shifts within each 16-lane row leave the row's largest in its lane 15,
// two row broadcasts carry those to lane 63 (lanes a DPP move has no source
// for read 0, which leaves a maximum of non-negative values alone).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_move<0x111, 0xF>(x));   // row_shr:1
  x = fmaxf(x, dpp_move<0x112, 0xF>(x));   // row_shr:2
  x = fmaxf(x, dpp_move<0x114, 0xF>(x));   // row_shr:4
  x = fmaxf(x, dpp_move<0x118, 0xF>(x));   // row_shr:8
  x = fmaxf(x, dpp_move<0x142, 0xA>(x));   // row_bcast:15 into rows 1 and 3
  x = fmaxf(x, dpp_move<0x143, 0xC>(x));   // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Input element loads (the raw input types are float and bf16 bits).
__device__ __forceinline__ float load_in(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_in(const uint16_t* p, int64_t i) { return bits_to_f32(p[i]); }

// ----------------------------------------------------------------------------
// Operand fragments.  Three precisions:
//   FragB  one bf16 per element (8 bits of significand)
//   FragP  a bf16 pair hi + lo with hi = bf16(x), lo = bf16(x - hi): about 16
//          bits of significand with the range of fp32
//   FragF  fp32 elements, multiplied on the fp32 matrix path
// Products: B*B 1 instruction, P*B / B*P 2, P*P 3 (the lo*lo term is below
// the pair's own rounding), F*F 8.  Two fp16 forms for the state update of
// the recurrence (FragH, FragHP below): H*HP 2.
struct FragB {
  bf16x8 v;
  static constexpr int kBytesPerLane = 16;
  __device__ __forceinline__ void set(const float x[8]) {
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const bf16x2 h = to_bf16x2(x[j], x[j + 1]);
      v[j] = h[0];
      v[j + 1] = h[1];
    }
  }
  __device__ __forceinline__ void load(const void* tile, int lane) {
    v = reinterpret_cast<const bf16x8*>(tile)[lane];
  }
  __device__ __forceinline__ void store(void* tile, int lane) const {
    reinterpret_cast<bf16x8*>(tile)[lane] = v;
  }
  // Elements 4 half .. 4 half + 3 of this lane's fragment in a tile (the
  // other half is written by whoever holds it).
  __device__ static __forceinline__ void store_half(void* tile, int lane, int half, const float x[4]) {
    bf16x4 h;
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const bf16x2 p = to_bf16x2(x[j], x[j + 1]);
      h[j] = p[0];
      h[j + 1] = p[1];
    }
    reinterpret_cast<bf16x4*>(tile)[2 * lane + half] = h;
  }
};

struct FragP {
  bf16x8 hi, lo;
  static constexpr int kBytesPerLane = 32;
  __device__ __forceinline__ void set(const float x[8]) {
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      bf16x2 h, l;
      split_bf16x2(x[j], x[j + 1], h, l);
      hi[j] = h[0]; hi[j + 1] = h[1];
      lo[j] = l[0]; lo[j + 1] = l[1];
    }
  }
  // Tile storage: the 64 hi vectors, then the 64 lo vectors.
  __device__ __forceinline__ void load(const void* tile, int lane) {
    const bf16x8* t = reinterpret_cast<const bf16x8*>(tile);
    hi = t[lane];
    lo = t[64 + lane];
  }
  __device__ __forceinline__ void store(void* tile, int lane) const {
    bf16x8* t = reinterpret_cast<bf16x8*>(tile);
    t[lane] = hi;
    t[64 + lane] = lo;
  }
  // Elements 4 half .. 4 half + 3 of this lane's fragment, split into a pair.
  __device__ static __forceinline__ void store_half(void* tile, int lane, int half, const float x[4]) {
    bf16x4 h, l;
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      bf16x2 hp, lp;
      split_bf16x2(x[j], x[j + 1], hp, lp);
      h[j] = hp[0]; h[j + 1] = hp[1];
      l[j] = lp[0]; l[j + 1] = lp[1];
    }
    reinterpret_cast<bf16x4*>(tile)[2 * lane + half] = h;
    reinterpret_cast<bf16x4*>(tile)[128 + 2 * lane + half] = l;
  }
};

struct FragF {
  f32x4 a, b;   // elements 0..3 and 4..7
  static constexpr int kBytesPerLane = 32;
  __device__ __forceinline__ void set(const float x[8]) {
    a = f32x4{x[0], x[1], x[2], x[3]};
    b = f32x4{x[4], x[5], x[6], x[7]};
  }
  __device__ __forceinline__ void load(const void* tile, int lane) {
    const f32x4* t = reinterpret_cast<const f32x4*>(tile);
    a = t[2 * lane];
    b = t[2 * lane + 1];
  }
  __device__ __forceinline__ void store(void* tile, int lane) const {
    f32x4* t = reinterpret_cast<f32x4*>(tile);
    t[2 * lane] = a;
    t[2 * lane + 1] = b;
  }
  __device__ static __forceinline__ void store_half(void* tile, int lane, int half, const float x[4]) {
    reinterpret_cast<f32x4*>(tile)[2 * lane + half] = f32x4{x[0], x[1], x[2], x[3]};
  }
};

// One fp16 per element (11 bits of significand), rounded to nearest even.
// Holds the decayed keys Kt of a record, each 16-key block scaled by a power
// of two that brings its largest magnitude into [2^14, 2^15), so neither
// overflow nor subnormals touch it whatever the keys' scale.
struct FragH {
  f16x8 v;
  static constexpr int kBytesPerLane = 16;
  __device__ __forceinline__ void set(const float x[8]) {
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const f16x2 h = to_f16x2(x[j], x[j + 1]);
      v[j] = h[0];
      v[j + 1] = h[1];
    }
  }
  __device__ __forceinline__ void load(const void* tile, int lane) {
    v = reinterpret_cast<const f16x8*>(tile)[lane];
  }
  __device__ __forceinline__ void store(void* tile, int lane) const {
    reinterpret_cast<f16x8*>(tile)[lane] = v;
  }
  // The same values as a bf16 pair (exact: 11 significant bits fit in two
  // bf16 of 8 each, and the range of fp16 lies inside bf16's).
  __device__ __forceinline__ FragP widen() const {
    FragP r;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      bf16x2 h, l;
      split_bf16x2((float)v[j], (float)v[j + 1], h, l);
      r.hi[j] = h[0]; r.hi[j + 1] = h[1];
      r.lo[j] = l[0]; r.lo[j + 1] = l[1];
    }
    return r;
  }
};

// An fp16 pair hi + lo with hi = fp16(x), lo = fp16(x - hi), both rounded to
// nearest even: about 22 bits of significand where x and x - hi are normal
// fp16 numbers (2^-3 <= |x| < 2^15), an absolute error within 2^-25 below;
// its user scales x by a power of two into that range (recurrence state
// update).
struct FragHP {
  f16x8 hi, lo;
  static constexpr int kBytesPerLane = 32;
  __device__ __forceinline__ void set(const float x[8]) {
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const f16x2 hp = to_f16x2(x[j], x[j + 1]);
      const f16x2 lp = to_f16x2(x[j] - (float)hp[0], x[j + 1] - (float)hp[1]);
      hi[j] = hp[0]; hi[j + 1] = hp[1];
      lo[j] = lp[0]; lo[j + 1] = lp[1];
    }
  }
  __device__ __forceinline__ void load(const void* tile, int lane) {
    const f16x8* t = reinterpret_cast<const f16x8*>(tile);
    hi = t[lane];
    lo = t[64 + lane];
  }
  // Elements 4 half .. 4 half + 3 of this lane's fragment, split into a pair.
  __device__ static __forceinline__ void store_half(void* tile, int lane, int half, const float x[4]) {
    f16x4 h, l;
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const f16x2 hp = to_f16x2(x[j], x[j + 1]);
      const f16x2 lp = to_f16x2(x[j] - (float)hp[0], x[j + 1] - (float)hp[1]);
      h[j] = hp[0]; h[j + 1] = hp[1];
      l[j] = lp[0]; l[j + 1] = lp[1];
    }
    reinterpret_cast<f16x4*>(tile)[2 * lane + half] = h;
    reinterpret_cast<f16x4*>(tile)[128 + 2 * lane + half] = l;
  }
};

// Bytes one 16x32 fragment tile occupies in memory.
template <class F>
constexpr int tile_bytes() { return F::kBytesPerLane * kWave; }

__device__ __forceinline__ void mfma_bb(f32x4& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4& c, const FragB& a, const FragB& b) { mfma_bb(c, a.v, b.v); }
__device__ __forceinline__ void mma(f32x4& c, const FragP& a, const FragB& b) {
  mfma_bb(c, a.lo, b.v);
  mfma_bb(c, a.hi, b.v);
}
__device__ __forceinline__ void mma(f32x4& c, const FragB& a, const FragP& b) {
  mfma_bb(c, a.v, b.lo);
  mfma_bb(c, a.v, b.hi);
}
__device__ __forceinline__ void mma(f32x4& c, const FragP& a, const FragP& b) {
  mfma_bb(c, a.lo, b.hi);
  mfma_bb(c, a.hi, b.lo);
  mfma_bb(c, a.hi, b.hi);
}
__device__ __forceinline__ void mfma_hh(f32x4& c, const f16x8& a, const f16x8& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const FragH& a, const FragHP& b) {
  mfma_hh(c, a.v, b.lo);
  mfma_hh(c, a.v, b.hi);
}
__device__ __forceinline__ void mma(f32x4& c, const FragF& a, const FragF& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[j], b.a[j], c, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[j], b.b[j], c, 0, 0, 0);
}

// Operand precisions per role.  bf16 inputs: the products whose rounding
// reaches the output at the 1e-2 level use pairs; T, W and Qg stay single
// bf16 (each costs at most a few 1e-3 of the output's rms on the benchmark
// workloads), V is an exact bf16 input.  The state update takes Kt as
// block-scaled fp16 (half the bytes of a bf16 pair: the recurrence's step is
// bound by the record bytes its waves load) and Delta as a scaled fp16 pair
// (Du).  fp32 inputs: fp32 throughout.
template <class TI> struct Prec;
template <> struct Prec<uint16_t> {
  using A = FragP;   // exp-scaled q/k operands of the intra-chunk products
  using T = FragB;   // (I+A)^-1 as an operand (W and U)
  using X = FragP;   // beta * k * exp(G) for W
  using V = FragB;   // values (exact)
  using W = FragB;   // -W as stored for the recurrence
  using Kt = FragH;  // k * exp(G_C - G) 2^s per 16-key block (state update)
  using Qg = FragB;  // scale * q * exp(G) (output, inter-chunk part)
  using Aq = FragP;  // scale * Aqk (output, intra-chunk part)
  using S = FragP;   // the state as an operand
  using D = FragP;   // the scaled residuals Delta as an operand (output)
  using Du = FragHP; // Delta 2^t as the state update's operand
};
template <> struct Prec<float> {
  using A = FragF; using T = FragF; using X = FragF; using V = FragF; using W = FragF;
  using Kt = FragF; using Qg = FragF; using Aq = FragF; using S = FragF; using D = FragF; using Du = FragF;
};

// ----------------------------------------------------------------------------
// Per-(chunk, head) record the intra-chunk kernel writes and the recurrence
// reads.  All fragment tiles use the k-order above.
//   Wn  : -W, rows = token r (4 blocks), k = key channel c     [4][K/32] tiles
//   Kt  : k * exp(G_C - G) transposed, rows = c, k = token r   [K/16][2] tiles
//   Qg  : scale * q * exp(G), rows = r, k = c                   [4][K/32] tiles
//   Aqk : scale * A_qk (lower incl. diagonal), rows = r, k = i  6 tiles (aqk_tile)
//   U   : T diag(beta) V in output-tile layout, rows = r, cols = value
//         channel, [4][V/16] tiles of 64 lanes x 4 fp32
//   Gc  : exp(G_C), K fp32 (decay of the whole chunk)
//   Ks  : (bf16 inputs) 2^-s of each 16-key block of Kt, K/16 fp32: the
//         stored block is Kt 2^s
// Aqk (lower triangular) as operand tiles (row block rb, 32-token slab kb):
// slab 1 of row blocks 0 and 1 is all zero and not stored, so tile (rb, kb)
// is the record's tile number aqk_tile(rb, kb), 0..5, for kb <= rb / 2.
__host__ __device__ constexpr int aqk_tile(int rb, int kb) { return rb < 2 ? rb : 2 * rb - 2 + kb; }

template <class TI, int K, int V>
struct RecordLayout {
  using P = Prec<TI>;
  static constexpr int64_t kWn = 0;
  static constexpr int64_t kWnBytes = 4 * (K / 32) * tile_bytes<typename P::W>();
  static constexpr int64_t kKt = kWn + kWnBytes;
  static constexpr int64_t kKtBytes = (K / 16) * 2 * tile_bytes<typename P::Kt>();
  static constexpr int64_t kQg = kKt + kKtBytes;
  static constexpr int64_t kQgBytes = 4 * (K / 32) * tile_bytes<typename P::Qg>();
  static constexpr int64_t kAqk = kQg + kQgBytes;
  static constexpr int64_t kAqkBytes = 6 * tile_bytes<typename P::Aq>();   // aqk_tile: no all-zero tiles
  static constexpr int64_t kU = kAqk + kAqkBytes;
  static constexpr int64_t kUBytes = 4 * (V / 16) * kWave * 16;
  static constexpr int64_t kGc = kU + kUBytes;
  static constexpr int64_t kGcBytes = K * 4;
  static constexpr bool kScaledKt = std::is_same<typename P::Kt, FragH>::value;
  static constexpr int64_t kKs = kGc + kGcBytes;
  static constexpr int64_t kKsBytes = kScaledKt ? (K / 16) * 4 : 0;
  static constexpr int64_t kBytes = ((kKs + kKsBytes) + 255) / 256 * 256;
};

// Chunk and segment tables built for packed inputs.
struct ChunkEntry {
  int32_t b, t0, len, seg;   // row, first token, tokens (1..64), global segment index
};
struct SegEntry {
  int32_t b, t0, len, local;     // row, first token, tokens, index within the row
  int32_t chunk_begin, n_chunks; // global chunk index of its first chunk, chunk count
  int32_t pad0, pad1;
};
// Per row of packed input: the state slots its segments fill and the first
// token of its unrecorded segments (T when all are recorded).
struct RowInfo {
  int32_t n_recorded, tail_t0;
};
// Scheduling words of the fused forward (zeroed before every call): arrivals
// per (XCD, compute unit) decide the workgroup's role, and per-XCD tickets
// hand out recurrence lanes and records to produce.
struct FusedCtl {
  uint32_t cu_arrivals[8][256];
  uint32_t lane_ticket[8];
  uint32_t item_ticket[8];
  uint32_t pad[48];
};
// Debug builds (-DKDA_DEBUG_CHECKS=1) check the g <= 0 precondition on the
// device and report a violation in the table header's flags.
#ifndef KDA_DEBUG_CHECKS
#define KDA_DEBUG_CHECKS 0
#endif
// Raises `bit` in the flags word if any lane's `bad` is set.
__device__ __forceinline__ void flag_if_any(uint32_t* flags, bool bad, uint32_t bit) {
  if (bad) atomicOr(flags, bit);
}

struct TableHeader {
  int32_t n_segments;   // recorded segments (all rows)
  int32_t n_chunks;     // chunks of recorded segments
  uint32_t flags;       // KDA_FLAG_* bits
  uint32_t tail_work;   // packed input: some output or final state needs zeroing after the tables
  uint32_t item_ticket; // intra-chunk items handed out past each workgroup's first (zeroed before the kernel)
  int32_t pad[59];      // keeps the header 256 bytes
};

}  // namespace kda
