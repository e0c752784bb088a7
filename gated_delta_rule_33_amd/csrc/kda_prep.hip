// Segment and chunk tables for packed inputs (integer work only).
//
// segment_ids [B,T] are 1-based with 0 = padding (KimiDeltaAttention.__call__,
// page "feat(kda): integrate KDA attention with tokamax backend and CP
// support", Public API).  A segment is a maximal run of equal non-zero ids.
// Each segment is chunked from its own first token (64 tokens per chunk, the
// last chunk partial), which is the natively packed layout the tokamax packed
// forward page describes: no chunk straddles a boundary, and the tail rows of
// a partial chunk are zero.
//
// One workgroup builds the tables row by row with block-wide prefix sums.
// Segments past max_segments in a row are not recorded: it raises
// KDA_FLAG_SEGMENT_OVERFLOW and notes per row where the unrecorded tokens
// begin and how many state slots were filled; a second, grid-wide kernel then
// zeroes the outputs of padding tokens and of unrecorded tokens, and the
// final states of the slots no segment reaches.
// While max_segments fits kLdsSegs, the bounds of a row's segments stay in
// LDS between the passes (each pass otherwise reads back from global memory
// what the one before wrote).
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kPrepThreads = 1024;
constexpr int kPrepTok = 8;     // tokens per thread in the segment scan
constexpr int kLdsSegs = 2048;  // segments per row whose bounds LDS holds

// Inclusive prefix sum over a wave (DPP: shifts within each 16-lane row,
// then the row totals carried on by two row broadcasts).
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ int wave_scan(int x) {
  x = dpp_add<0x111, 0xF>(x);   // row_shr:1
  x = dpp_add<0x112, 0xF>(x);   // row_shr:2
  x = dpp_add<0x114, 0xF>(x);   // row_shr:4
  x = dpp_add<0x118, 0xF>(x);   // row_shr:8
  x = dpp_add<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
  x = dpp_add<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// Inclusive prefix sum over the 1024 threads of the block; *total gets the
// sum.  Each wave scans its lanes, then wave 0 scans the 16 wave sums.
__device__ int block_scan(int x, int* wave_sums, int* total) {
  constexpr int NW = kPrepThreads / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int v = wave_scan(x);
  if (lane == 63) wave_sums[wv] = v;
  __syncthreads();
  if (wv == 0) {
    const int ws = lane < NW ? wave_sums[lane] : 0;
    const int u = wave_scan(ws);
    if (lane < NW) wave_sums[lane] = u - ws;   // exclusive
    if (lane == NW - 1) wave_sums[NW] = u;    // total
  }
  __syncthreads();
  const int res = v + wave_sums[wv];
  *total = wave_sums[NW];
  __syncthreads();
  return res;
}

template <class TO>
__device__ void zero_token(TO* o, int64_t tok, int64_t HV, int t0, int stride) {
  for (int64_t e = t0; e < HV; e += stride) o[tok * HV + e] = TO(0);
}

struct PrepParams {
  const int32_t* ids;
  int64_t B, T, H, K, V;
  int n_max;
  TableHeader* hdr;
  SegEntry* segs;
  ChunkEntry* chunks;
  RowInfo* rows;
  void* o;
  float* fin;
};

__global__ __launch_bounds__(kPrepThreads) void kda_prep_kernel(PrepParams p) {
  const int64_t T = p.T;
  __shared__ int wave_sums[kPrepThreads / 64 + 1];
  __shared__ int l_t0[kLdsSegs], l_end[kLdsSegs];   // per recorded segment of the row
  const bool lds = p.n_max <= kLdsSegs;
  // 16-byte loads of ids where every row starts 16-byte aligned
  const bool vec = ((reinterpret_cast<uintptr_t>(p.ids) | (uintptr_t)(T * 4)) & 15) == 0;
  const int tid = threadIdx.x;
  int seg_base = 0, chunk_base = 0;
  uint32_t flags = 0;
  bool tail_work = false;   // padding, unrecorded segments or unreached state slots
  for (int64_t b = 0; b < p.B; ++b) {
    const int32_t* row = p.ids + b * T;
    // Pass 1: segment starts and ends.  Each thread takes kPrepTok
    // consecutive tokens (all their ids loaded at once), counts the starts
    // among them, and one block scan per kPrepThreads * kPrepTok tokens
    // numbers the segments.
    int row_segs = 0;
    for (int64_t t0 = 0; t0 < T; t0 += (int64_t)kPrepThreads * kPrepTok) {
      const int64_t tb = t0 + (int64_t)tid * kPrepTok;
      // tokens tb - 1 .. tb + kPrepTok (0 outside the row): every load is
      // issued, at a clamped index, and masked after
      int ids[kPrepTok + 2];
      if (vec && tb + kPrepTok <= T) {
        // two 16-byte loads: each wave's load instruction covers 1 KB of ids
        const int4 a = *reinterpret_cast<const int4*>(row + tb);
        const int4 c = *reinterpret_cast<const int4*>(row + tb + 4);
        ids[1] = a.x; ids[2] = a.y; ids[3] = a.z; ids[4] = a.w;
        ids[5] = c.x; ids[6] = c.y; ids[7] = c.z; ids[8] = c.w;
        ids[0] = row[tb > 0 ? tb - 1 : 0];
        ids[kPrepTok + 1] = row[tb + kPrepTok < T ? tb + kPrepTok : T - 1];
      } else {
#pragma unroll
        for (int i = 0; i < kPrepTok + 2; ++i) {
          const int64_t t = tb - 1 + i;
          ids[i] = row[t < 0 ? 0 : (t < T ? t : T - 1)];
        }
      }
#pragma unroll
      for (int i = 0; i < kPrepTok + 2; ++i) {
        const int64_t t = tb - 1 + i;
        ids[i] = (t >= 0 && t < T) ? ids[i] : 0;
      }
      // bit i - 1: token tb + i - 1 starts (smask) or ends (emask) a segment
      uint32_t smask = 0, emask = 0;
      bool padding = false;
#pragma unroll
      for (int i = 1; i <= kPrepTok; ++i) {
        const int64_t t = tb + i - 1;
        const int id = ids[i];
        const bool in = t < T && id != 0;
        padding = padding || (t < T && id == 0);
        smask |= (in && (t == 0 || id != ids[i - 1]) ? 1u : 0u) << (i - 1);
        emask |= (in && (t == T - 1 || ids[i + 1] != id) ? 1u : 0u) << (i - 1);
      }
      if (__syncthreads_or(padding ? 1 : 0)) tail_work = true;
      const int starts = __builtin_popcount(smask);
      int total;
      const int incl = block_scan(starts, wave_sums, &total);
      const int seen = row_segs + incl - starts;   // segments started before this thread's first token
      // only the tokens that start or end a segment do anything
      for (uint32_t ev = smask | emask; ev != 0; ev &= ev - 1) {
        const int bit = __builtin_ctz(ev);
        const int local = seen + __builtin_popcount(smask & ((2u << bit) - 1)) - 1;   // its segment
        if (local >= p.n_max) break;
        const int t = (int)(tb + bit);
        const bool start = (smask >> bit) & 1, end = (emask >> bit) & 1;
        if (lds) {
          if (start) l_t0[local] = t;
          if (end) l_end[local] = t + 1;
        } else {
          SegEntry* se = p.segs + seg_base + local;
          if (start) se->t0 = t;
          if (end) se->len = t + 1;   // end for now; turned into a length below
        }
      }
      row_segs += total;
    }
    __syncthreads();
    const int nrec = min(row_segs, p.n_max);
    if (row_segs > p.n_max) flags |= KDA_FLAG_SEGMENT_OVERFLOW;
    if (row_segs > p.n_max || (p.fin != nullptr && row_segs < p.n_max)) tail_work = true;
    // Pass 2: lengths, chunk counts and first chunk of each recorded
    // segment, and its entry; pass 3: its chunk entries (one thread per
    // segment, right after).
    int last_end = 0;   // end of the row's last recorded segment (thread 0)
    for (int s0 = 0; s0 < nrec; s0 += kPrepThreads) {
      const int s = s0 + tid;
      int st = 0, len = 0, nch = 0;
      if (s < nrec) {
        if (lds) {
          st = l_t0[s];
          len = l_end[s] - st;
        } else {
          st = p.segs[seg_base + s].t0;
          len = p.segs[seg_base + s].len - st;
        }
        nch = (len + kChunk - 1) / kChunk;
      }
      int total;
      const int incl = block_scan(nch, wave_sums, &total);
      if (s < nrec) {
        SegEntry se;
        se.b = (int)b;
        se.t0 = st;
        se.len = len;
        se.local = s;
        se.chunk_begin = chunk_base + incl - nch;
        se.n_chunks = nch;
        se.pad0 = se.pad1 = 0;
        p.segs[seg_base + s] = se;
        for (int c = 0; c < nch; ++c) {
          ChunkEntry ce;
          ce.b = (int)b;
          ce.t0 = st + c * kChunk;
          ce.len = min(kChunk, len - c * kChunk);
          ce.seg = seg_base + s;
          p.chunks[se.chunk_begin + c] = ce;
        }
        if (s == nrec - 1) wave_sums[kPrepThreads / 64] = st + len;
      }
      chunk_base += total;
    }
    __syncthreads();
    if (nrec > 0) last_end = wave_sums[kPrepThreads / 64];
    // Where the row's unrecorded tokens begin (T when every segment is
    // recorded) and how many state slots its segments fill.
    if (tid == 0) {
      RowInfo ri;
      ri.n_recorded = nrec;
      ri.tail_t0 = row_segs > p.n_max ? last_end : (int)T;
      p.rows[b] = ri;
    }
    seg_base += nrec;
    __syncthreads();
  }
  if (tid == 0) {
    p.hdr->n_segments = seg_base;
    p.hdr->n_chunks = chunk_base;
    p.hdr->flags = flags;
    p.hdr->tail_work = tail_work ? 1u : 0u;
    p.hdr->item_ticket = 0u;   // the intra-chunk kernel's item counter
  }
}

// Grid-wide zeroing after the tables: the outputs of padding tokens and of
// tokens of unrecorded segments (a row with more than max_segments
// segments), and the final states of the slots no segment of a row reaches.
// One wave per token or per (row, slot, head) state block.
constexpr int kTailThreads = 256;

template <class TO>
__global__ __launch_bounds__(kTailThreads) void kda_prep_tail_kernel(PrepParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kTailThreads / 64) + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * (kTailThreads / 64);
  if (p.hdr->tail_work == 0) return;   // nothing to zero: no padding, every segment recorded, every slot reached
  const int64_t HV = p.H * p.V, KV = p.K * p.V;
  TO* o = static_cast<TO*>(p.o);
  if (o != nullptr) {
    for (int64_t tok = wave; tok < p.B * p.T; tok += n_waves) {
      const int64_t b = tok / p.T, t = tok % p.T;
      const int id = p.ids[tok];
      if (id == 0 || t >= p.rows[b].tail_t0) zero_token(o, tok, HV, lane, 64);
    }
  }
  if (p.fin != nullptr) {
    for (int64_t blk = wave; blk < p.B * p.n_max * p.H; blk += n_waves) {
      const int64_t b = blk / ((int64_t)p.n_max * p.H), local = (blk / p.H) % p.n_max;
      if (local < p.rows[b].n_recorded) continue;
      f32x4* dst = reinterpret_cast<f32x4*>(p.fin + blk * KV);
      for (int64_t e = lane; e < KV / 4; e += 64) dst[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

__global__ void kda_fill_zero_kernel(float* x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    x[i] = 0.f;
}

}  // namespace

hipError_t launch_prep(const CallArgs& a) {
  PrepParams p{a.seg_ids, a.B, a.T, a.H, a.K, a.V, a.n_max, a.hdr, a.segs, a.chunks, a.rows, a.o, a.fin};
  hipLaunchKernelGGL(kda_prep_kernel, dim3(1), dim3(kPrepThreads), 0, a.stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (a.o == nullptr && a.fin == nullptr)) return e;
  const int64_t waves = std::max<int64_t>(a.B * a.T, a.B * a.n_max * a.H);
  const unsigned tail_groups = (unsigned)std::min<int64_t>(1024, (waves + 3) / 4);
  if (a.out == OutType::F32)
    hipLaunchKernelGGL(kda_prep_tail_kernel<float>, dim3(tail_groups), dim3(kTailThreads), 0, a.stream, p);
  else
    hipLaunchKernelGGL(kda_prep_tail_kernel<uint16_t>, dim3(tail_groups), dim3(kTailThreads), 0, a.stream, p);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t stream) {
  if (n <= 0 || x == nullptr) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>(1024, (n + 255) / 256);
  hipLaunchKernelGGL(kda_fill_zero_kernel, dim3(grid), dim3(256), 0, stream, x, n);
  return hipGetLastError();
}

// final_state (every slot: one per row, or max_segments per row with
// segment ids) and the transition when no segment can occur (T == 0).
hipError_t launch_zero_states(const CallArgs& a) {
  hipError_t e = launch_fill_zero(a.fin, a.smax * a.H * a.K * a.V, a.stream);
  if (e == hipSuccess) e = launch_fill_zero(a.trans, a.B * a.H * a.K * a.K, a.stream);
  return e;
}

}  // namespace kda
