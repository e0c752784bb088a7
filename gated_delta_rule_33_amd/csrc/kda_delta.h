// Delta of one chunk between the waves of a recurrence workgroup, and the
// state update S <- diag(exp(G_C)) S + Kt^T Delta that consumes it.
//
// With bf16 inputs the record stores Kt as fp16 scaled by 2^s per 16-key
// block (FragH).  Its partner in the update is Delta as an fp16 pair
// (FragHP) of Delta 2^kDeltaShift.  Where a 32-token slab's largest scaled
// |Delta| lies in [2^-4, 2^15) the pair carries every value to within 2^-22
// of itself or 2^-21 of that largest; a 16-token block with a scaled value
// at or above 2^15 (or not finite), or nonzero values all below 2^-4, marks
// its slab, and the update of that slab takes the bf16 pair of Delta (which
// the output's Aqk Delta product needs anyway) against Kt widened exactly to
// a bf16 pair.  So results never depend on Delta's scale beyond rounding,
// and only the speed does: the fp16 form covers largest |Delta| per slab in
// [2^-8, 2^11), the usual range of the residuals.  fp32 inputs: Delta and
// Kt in fp32, no scaling.
#pragma once
#include "kda_launch.h"

namespace kda {

template <class TI>
struct DeltaLds {
  using P = Prec<TI>;
  static constexpr bool kScaled = std::is_same<typename P::Du, FragHP>::value;
  static constexpr int TD = tile_bytes<typename P::D>();
  static constexpr int TU = kScaled ? tile_bytes<typename P::Du>() : 16;
  char d[2 * TD];    // Delta as operand tiles (32 tokens each): output; the update's fallback
  char du[2 * TU];   // Delta 2^kDeltaShift as the update's operand tiles (bf16 inputs)
  int fits[4];       // per 16-token block: its scaled Delta fits the fp16 pair
};

constexpr int kDeltaShift = 4;

// Chain wave w stores its 16 tokens of Delta (x[i]: token 4 gq + i of the
// block, value column m).
template <class TI>
__device__ __forceinline__ void delta_store(DeltaLds<TI>& dl, int w, int lane, const float x[4]) {
  using DL = DeltaLds<TI>;
  Prec<TI>::D::store_half(dl.d + (w / 2) * DL::TD, lane, w & 1, x);
  if constexpr (DL::kScaled) {
    constexpr float sc = (float)(1 << kDeltaShift);
    const float y[4] = {x[0] * sc, x[1] * sc, x[2] * sc, x[3] * sc};
    FragHP::store_half(dl.du + (w / 2) * DL::TU, lane, w & 1, y);
    const float my = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
    const bool over = __builtin_amdgcn_ballot_w64(!(my < 32768.f)) != 0;   // NaN counts as over
    const bool big = __builtin_amdgcn_ballot_w64(my >= 0.0625f) != 0;
    const bool nonzero = __builtin_amdgcn_ballot_w64(my > 0.f) != 0;
    if (lane == 0) dl.fits[w] = !over && (big || !nonzero) ? 1 : 0;
  }
}

// The update's operands for the 32-token slabs kb = 0 (tokens 0..31) and 1
// (32..63): the fp16 pair when both blocks of the slab fit it (factor
// 2^-kDeltaShift), else the bf16 pair (factor 1).
template <class TI>
struct DeltaOperands {
  using P = Prec<TI>;
  using DL = DeltaLds<TI>;
  typename P::Du du[2];
  typename P::D d[2];
  bool fast[2];
  float f[2];
  __device__ __forceinline__ void load(const DL& dl, int lane) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (DL::kScaled) {
        du[kb].load(dl.du + kb * DL::TU, lane);
        fast[kb] = __builtin_amdgcn_readfirstlane(dl.fits[2 * kb] & dl.fits[2 * kb + 1]) != 0;
        f[kb] = fast[kb] ? 1.f / (float)(1 << kDeltaShift) : 1.f;
        if (!fast[kb]) d[kb].load(dl.d + kb * DL::TD, lane);
      } else {
        fast[kb] = false;
        f[kb] = 1.f;
        d[kb].load(dl.d + kb * DL::TD, lane);
      }
    }
  }
};

// One 16-key block of the state (this lane's 4 rows of a value column):
// s <- s diag(gc) + ks (f0 Kt0^T Delta0 + f1 Kt1^T Delta1) over the two
// slabs, with kt the block's two slab tiles and ks = 2^-s of the block's Kt
// scale (1 for fp32).
template <class TI>
__device__ __forceinline__ void state_update(f32x4& s, const f32x4& gc, float ks, const typename Prec<TI>::Kt kt[2],
                                             const DeltaOperands<TI>& o) {
  f32x4 a[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if constexpr (DeltaLds<TI>::kScaled) {
      if (o.fast[kb]) mma(a[kb], kt[kb], o.du[kb]);
      else mma(a[kb], kt[kb].widen(), o.d[kb]);
    } else {
      mma(a[kb], kt[kb], o.d[kb]);
    }
  }
  const float c0 = ks * o.f[0], c1 = ks * o.f[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = s[i] * gc[i] + (c0 * a[0][i] + c1 * a[1][i]);
}


}  // namespace kda
