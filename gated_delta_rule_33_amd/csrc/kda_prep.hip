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
// Workgroup 0 builds the tables row by row with block-wide prefix sums; the
// other workgroups write o = 0 for padding tokens.  Segments past max_segments
// in a row are not recorded: workgroup 0 raises KDA_FLAG_SEGMENT_OVERFLOW and
// notes per row where the unrecorded tokens begin and how many state slots
// were filled; a second, grid-wide kernel then zeroes the outputs of the
// unrecorded tokens and the final states of the slots no segment reaches.
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kPrepThreads = 1024;
constexpr int kPrepTok = 8;   // tokens per thread in the segment scan

// Inclusive prefix sum over the 1024 threads of the block; *total gets the sum.
__device__ int block_scan(int x, int* wave_sums, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int v = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(v, d);
    if (lane >= d) v += y;
  }
  if (lane == 63) wave_sums[wv] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < kPrepThreads / 64; ++i) {
      const int s = wave_sums[i];
      wave_sums[i] = run;
      run += s;
    }
    wave_sums[kPrepThreads / 64] = run;
  }
  __syncthreads();
  const int res = v + wave_sums[wv];
  *total = wave_sums[kPrepThreads / 64];
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

template <class TO>
__global__ __launch_bounds__(kPrepThreads) void kda_prep_kernel(PrepParams p) {
  const int64_t T = p.T, HV = p.H * p.V;
  TO* o = static_cast<TO*>(p.o);
  if (blockIdx.x > 0) {
    // Padding tokens: one wave per token (nothing to do without an output).
    if (o == nullptr) return;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)(blockIdx.x - 1) * (kPrepThreads / 64) + (threadIdx.x >> 6);
    const int64_t n_waves = (int64_t)(gridDim.x - 1) * (kPrepThreads / 64);
    for (int64_t tok = wave; tok < p.B * T; tok += n_waves)
      if (p.ids[tok] == 0) zero_token(o, tok, HV, lane, 64);
    return;
  }

  __shared__ int wave_sums[kPrepThreads / 64 + 1];
  const int tid = threadIdx.x;
  int seg_base = 0, chunk_base = 0;
  uint32_t flags = 0;
  for (int64_t b = 0; b < p.B; ++b) {
    const int32_t* row = p.ids + b * T;
    // Pass 1: segment starts and ends.  Each thread takes kPrepTok
    // consecutive tokens (all their ids loaded at once), counts the starts
    // among them, and one block scan per kPrepThreads * kPrepTok tokens
    // numbers the segments.
    int row_segs = 0;
    for (int64_t t0 = 0; t0 < T; t0 += (int64_t)kPrepThreads * kPrepTok) {
      const int64_t tb = t0 + (int64_t)tid * kPrepTok;
      int ids[kPrepTok + 2];   // tokens tb - 1 .. tb + kPrepTok (0 outside the row)
#pragma unroll
      for (int i = 0; i < kPrepTok + 2; ++i) {
        const int64_t t = tb - 1 + i;
        ids[i] = (t >= 0 && t < T) ? row[t] : 0;
      }
      int starts = 0;
#pragma unroll
      for (int i = 1; i <= kPrepTok; ++i) {
        const int64_t t = tb + i - 1;
        starts += (t < T && ids[i] != 0 && (t == 0 || ids[i] != ids[i - 1])) ? 1 : 0;
      }
      int total;
      const int incl = block_scan(starts, wave_sums, &total);
      int seen = row_segs + incl - starts;   // segments started before this thread's first token
#pragma unroll
      for (int i = 1; i <= kPrepTok; ++i) {
        const int64_t t = tb + i - 1;
        if (t >= T) break;
        const int id = ids[i];
        const bool start = id != 0 && (t == 0 || id != ids[i - 1]);
        const bool end = id != 0 && (t == T - 1 || ids[i + 1] != id);
        seen += start ? 1 : 0;
        const int local = seen - 1;   // the segment token t belongs to
        if (id != 0 && local < p.n_max) {
          SegEntry* se = p.segs + seg_base + local;
          if (start) { se->b = (int)b; se->t0 = (int)t; se->local = local; }
          if (end) se->len = (int)(t + 1);   // end for now; turned into a length below
        }
      }
      row_segs += total;
    }
    __syncthreads();
    const int nrec = min(row_segs, p.n_max);
    if (row_segs > p.n_max) flags |= KDA_FLAG_SEGMENT_OVERFLOW;
    // Pass 2: lengths, chunk counts and first chunk of each recorded segment.
    for (int s0 = 0; s0 < nrec; s0 += kPrepThreads) {
      const int s = s0 + tid;
      int nch = 0;
      if (s < nrec) {
        SegEntry* se = p.segs + seg_base + s;
        se->len = se->len - se->t0;
        nch = (se->len + kChunk - 1) / kChunk;
        se->n_chunks = nch;
      }
      int total;
      const int incl = block_scan(nch, wave_sums, &total);
      if (s < nrec) p.segs[seg_base + s].chunk_begin = chunk_base + incl - nch;
      chunk_base += total;
    }
    __syncthreads();
    // Pass 3: chunk entries (one thread per recorded segment).
    for (int s = tid; s < nrec; s += kPrepThreads) {
      const SegEntry se = p.segs[seg_base + s];
      for (int c = 0; c < se.n_chunks; ++c) {
        ChunkEntry ce;
        ce.b = (int)b;
        ce.t0 = se.t0 + c * kChunk;
        ce.len = min(kChunk, se.len - c * kChunk);
        ce.seg = seg_base + s;
        p.chunks[se.chunk_begin + c] = ce;
      }
    }
    // Where the row's unrecorded tokens begin (T when every segment is
    // recorded) and how many state slots its segments fill.
    if (tid == 0) {
      RowInfo ri;
      ri.n_recorded = nrec;
      ri.tail_t0 = (int)T;
      if (row_segs > p.n_max) {
        const SegEntry last = p.segs[seg_base + nrec - 1];
        ri.tail_t0 = last.t0 + last.len;
      }
      p.rows[b] = ri;
    }
    seg_base += nrec;
    __syncthreads();
  }
  if (tid == 0) {
    p.hdr->n_segments = seg_base;
    p.hdr->n_chunks = chunk_base;
    p.hdr->flags = flags;
  }
}

// Grid-wide zeroing after the tables: the outputs of tokens of unrecorded
// segments (a row with more than max_segments segments) and the final states
// of the slots no segment of a row reaches.  One wave per token or per
// (row, slot, head) state block.
constexpr int kTailThreads = 256;

template <class TO>
__global__ __launch_bounds__(kTailThreads) void kda_prep_tail_kernel(PrepParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kTailThreads / 64) + (threadIdx.x >> 6);
  const int64_t n_waves = (int64_t)gridDim.x * (kTailThreads / 64);
  const int64_t HV = p.H * p.V, KV = p.K * p.V;
  TO* o = static_cast<TO*>(p.o);
  if (o != nullptr) {
    for (int64_t tok = wave; tok < p.B * p.T; tok += n_waves) {
      const int64_t b = tok / p.T, t = tok % p.T;
      if (t >= p.rows[b].tail_t0 && p.ids[tok] != 0) zero_token(o, tok, HV, lane, 64);
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
  const int64_t tokens = a.B * a.T;
  const int zero_groups = (int)std::min<int64_t>(256, (tokens + 15) / 16);
  const dim3 grid(1 + zero_groups);
  if (a.out == OutType::F32)
    hipLaunchKernelGGL(kda_prep_kernel<float>, grid, dim3(kPrepThreads), 0, a.stream, p);
  else
    hipLaunchKernelGGL(kda_prep_kernel<uint16_t>, grid, dim3(kPrepThreads), 0, a.stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (a.o == nullptr && a.fin == nullptr)) return e;
  const int64_t waves = std::max<int64_t>(tokens, a.B * a.n_max * a.H);
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
