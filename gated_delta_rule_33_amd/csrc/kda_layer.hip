// The two layer steps around the KDA forward, from the layer pipeline of the
// page "feat(kda): integrate KDA attention with tokamax backend and CP
// support" (Implementation Details, Layer architecture):
//   short convolution  y[b,t,d] = SiLU( sum_{j<W} w[d,j] x[b, t-(W-1)+j, d] ),
//     causal and depthwise over T, applied to q, k and v; a tap reads zero
//     before the start of t's segment (a maximal run of one non-zero segment
//     id, the review notes' segment-aware convolution) and padding tokens
//     give y = 0;
//   output stage       y = w * o / sqrt(mean_V(o^2) + eps) * sigmoid(gate),
//     a per-head RMSNorm over the value channels with a sigmoid output gate.
// Both are memory-bound streams: the convolution keeps a window of the last
// W inputs in registers (eight channels and eight tokens per thread),
// the norm reduces one (token, head) row of V values per wave.
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvTokens = 8;      // tokens per thread
constexpr int kConvCh = 8;          // channels per thread (one 16-byte load of bf16)

typedef float f32x8 __attribute__((ext_vector_type(8)));

// Eight channels as raw words (bf16: one 16-byte load; fp32: two) and widened.
template <class T> struct Raw8;
template <> struct Raw8<uint16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ f32x8 widen() const {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    f32x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[2 * i] = __uint_as_float(u[i] << 16);
      r[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
    return r;
  }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ f32x8 widen() const { return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }
};
__device__ __forceinline__ void store8(float* p, const f32x8& x) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
__device__ __forceinline__ void store8(uint16_t* p, const f32x8& x) {
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = __builtin_bit_cast(uint32_t, to_bf16x2(x[2 * i], x[2 * i + 1]));
  *reinterpret_cast<uint4*>(p) = uint4{u[0], u[1], u[2], u[3]};
}

__device__ __forceinline__ float silu(float a) { return a / (1.f + __expf(-a)); }

// Block (b, token tile, channel group): thread i owns channels 8i..8i+7 of
// the group and walks the tile's 8 tokens, with the W-1 tokens before the
// tile as the initial window.  reach[t] = how many of the taps t, t-1, ...
// lie in t's segment (0 for padding), computed once per tile.
template <class T, int W>
__global__ __launch_bounds__(kConvThreads) void short_conv_kernel(const T* __restrict__ x, const float* __restrict__ w,
                                                                  const int32_t* __restrict__ seg, T* __restrict__ y,
                                                                  int64_t Tlen, int64_t D, int64_t tiles) {
  __shared__ int reach[kConvTokens];
  const int64_t b = blockIdx.x / tiles, t0 = (blockIdx.x % tiles) * kConvTokens;
  const int tid = threadIdx.x;
  if (tid < kConvTokens) {
    const int64_t t = t0 + tid;
    int r = 0;
    if (t < Tlen) {
      if (seg == nullptr) {
        r = (int)min<int64_t>(W, t + 1);
      } else {
        const int32_t sv = seg[b * Tlen + t];
        if (sv != 0) {
          r = 1;
          while (r < W && t - r >= 0 && seg[b * Tlen + t - r] == sv) ++r;
        }
      }
    }
    reach[tid] = r;
  }
  __syncthreads();
  const int64_t d = ((int64_t)blockIdx.y * kConvThreads + tid) * kConvCh;
  if (d >= D) return;
  const T* xr = x + b * Tlen * D + d;
  T* yr = y + b * Tlen * D + d;
  const int n = (int)min<int64_t>(kConvTokens, Tlen - t0);
  // all loads of the tile in flight at once: W-1 tokens of history, then the tile
  Raw8<T> raw[W - 1 + kConvTokens];
#pragma unroll
  for (int k = 0; k < W - 1 + kConvTokens; ++k) {
    const int64_t t = t0 - (W - 1) + k;
    if (t >= 0 && k - (W - 1) < n) raw[k].load(xr + t * D);
    else raw[k] = Raw8<T>{};
  }
  f32x8 wk[W];
#pragma unroll
  for (int j = 0; j < W; ++j)
#pragma unroll
    for (int c = 0; c < kConvCh; ++c) wk[j][c] = w[(d + c) * W + j];
#pragma unroll
  for (int i = 0; i < kConvTokens; ++i) {
    if (i >= n) break;
    const int r = reach[i];
    f32x8 acc = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < W; ++j) {
      // tap j reads token t - (W-1) + j, i.e. W-1-j tokens back: raw[i + j]
      if (W - 1 - j < r) {
        const f32x8 h = raw[i + j].widen();
#pragma unroll
        for (int c = 0; c < kConvCh; ++c) acc[c] += wk[j][c] * h[c];
      }
    }
    f32x8 out;
#pragma unroll
    for (int c = 0; c < kConvCh; ++c) out[c] = r > 0 ? silu(acc[c]) : 0.f;
    store8(yr + (t0 + i) * D, out);
  }
}

template <class T>
hipError_t launch_conv_t(const ConvArgs& a, dim3 grid, int64_t tiles) {
  const T* x = static_cast<const T*>(a.x);
  T* y = static_cast<T*>(a.y);
#define KDA_CONV_W(WW)                                                                                             \
  case WW:                                                                                                         \
    hipLaunchKernelGGL((short_conv_kernel<T, WW>), grid, dim3(kConvThreads), 0, a.stream, x, a.weight, a.seg, y, a.T, \
                       a.D, tiles);                                                                                \
    break;
  switch (a.W) {
    KDA_CONV_W(1) KDA_CONV_W(2) KDA_CONV_W(3) KDA_CONV_W(4) KDA_CONV_W(5) KDA_CONV_W(6) KDA_CONV_W(7) KDA_CONV_W(8)
    default: return hipErrorInvalidValue;
  }
#undef KDA_CONV_W
  return hipGetLastError();
}

// One wave per row of V values: y = w * o / sqrt(mean(o^2) + eps) * sigmoid(gate).
template <int EPL>
__device__ __forceinline__ void load_row(const float* p, int lane, float x[EPL]) {
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] = p[lane * EPL + e];
}
template <int EPL>
__device__ __forceinline__ void load_row(const uint16_t* p, int lane, float x[EPL]) {
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] = bits_to_f32(p[lane * EPL + e]);
}
template <int EPL>
__device__ __forceinline__ void store_row(float* p, int lane, const float x[EPL]) {
#pragma unroll
  for (int e = 0; e < EPL; ++e) p[lane * EPL + e] = x[e];
}
template <int EPL>
__device__ __forceinline__ void store_row(uint16_t* p, int lane, const float x[EPL]) {
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const __bf16 h = to_bf16(x[e]);
    p[lane * EPL + e] = __builtin_bit_cast(uint16_t, h);
  }
}

constexpr int kNormThreads = 256;

template <class TO, class TG, class TY, int EPL>
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(const TO* __restrict__ o, const TG* __restrict__ gate,
                                                                     const float* __restrict__ w, float eps,
                                                                     TY* __restrict__ y, int64_t rows) {
  constexpr int V = EPL * kWave;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kNormThreads / kWave) + (threadIdx.x >> 6);
  if (row >= rows) return;
  float ov[EPL], gv[EPL], wv[EPL];
  load_row<EPL>(o + row * V, lane, ov);
  load_row<EPL>(gate + row * V, lane, gv);
  load_row<EPL>(w, lane, wv);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) ss += ov[e] * ov[e];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv = 1.f / sqrtf(ss / (float)V + eps);
  float out[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[e] = wv[e] * ov[e] * inv / (1.f + __expf(-gv[e]));
  store_row<EPL>(y + row * V, lane, out);
}

template <class TO, class TG, class TY>
hipError_t launch_norm_t(const NormArgs& a) {
  const unsigned grid = (unsigned)((a.rows + kNormThreads / kWave - 1) / (kNormThreads / kWave));
  const TO* o = static_cast<const TO*>(a.o);
  const TG* g = static_cast<const TG*>(a.gate);
  TY* y = static_cast<TY*>(a.y);
  switch (a.V) {
    case 64: hipLaunchKernelGGL((gated_rmsnorm_kernel<TO, TG, TY, 1>), dim3(grid), dim3(kNormThreads), 0, a.stream, o, g, a.weight, a.eps, y, a.rows); break;
    case 128: hipLaunchKernelGGL((gated_rmsnorm_kernel<TO, TG, TY, 2>), dim3(grid), dim3(kNormThreads), 0, a.stream, o, g, a.weight, a.eps, y, a.rows); break;
    case 256: hipLaunchKernelGGL((gated_rmsnorm_kernel<TO, TG, TY, 4>), dim3(grid), dim3(kNormThreads), 0, a.stream, o, g, a.weight, a.eps, y, a.rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class TO, class TG>
hipError_t launch_norm_g(const NormArgs& a) {
  return a.y_bf16 ? launch_norm_t<TO, TG, uint16_t>(a) : launch_norm_t<TO, TG, float>(a);
}
template <class TO>
hipError_t launch_norm_o(const NormArgs& a) {
  return a.gate_bf16 ? launch_norm_g<TO, uint16_t>(a) : launch_norm_g<TO, float>(a);
}

}  // namespace

hipError_t launch_short_conv(const ConvArgs& a) {
  if (a.B == 0 || a.T == 0 || a.D == 0) return hipSuccess;
  const int64_t tiles = (a.T + kConvTokens - 1) / kConvTokens;
  const dim3 grid((unsigned)(a.B * tiles), (unsigned)((a.D / kConvCh + kConvThreads - 1) / kConvThreads));
  return a.bf16 ? launch_conv_t<uint16_t>(a, grid, tiles) : launch_conv_t<float>(a, grid, tiles);
}

hipError_t launch_gated_rmsnorm(const NormArgs& a) {
  if (a.rows == 0) return hipSuccess;
  return a.o_bf16 ? launch_norm_o<uint16_t>(a) : launch_norm_o<float>(a);
}

}  // namespace kda
