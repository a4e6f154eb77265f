// Binning of scores relative to the predicted threshold theta, shared by the
// top-k kernels and the scoring kernel that lists each row's band for them:
// both sides must put a score in the same bin, bit for bit.
#pragma once

#include "common.hpp"

namespace {

// Binning of a score relative to the prediction theta. Scores more than
// |theta|/4 below theta all share bin 0: only the bins around and above the
// boundary are needed, and lumping the bulk lets the histogram skip the
// per-bin work for most tokens. Bin 0 is below every real bin, so the binning
// stays monotone in s. A NaN theta means no shift and no lumping.
struct Shift {
  float th, cut;
  bool on;
};

__device__ __forceinline__ Shift make_shift(float th) {
  Shift sh;
  sh.on = th == th;
  sh.th = th;
  const float a = fabsf(th);
  sh.cut = (sh.on && a > 0.f && a < __builtin_inff()) ? -0.25f * a : -__builtin_inff();
  return sh;
}

// Bins of the one-pass path: the high byte of the order key of fp16(d), the
// same four bins per binade as bin16, computed with fewer instructions: d + 0
// folds -0 onto +0 (equal scores share a bin), and the key's high byte is
// the fp16 high byte with the sign bit flipped (positive d) or all bits
// flipped (negative d). A negative d that rounds to fp16 -0 takes bin 0x7f,
// just below +0: still monotone in d.
__device__ __forceinline__ uint32_t bin_one(float d) {
  const _Float16 h = (_Float16)(d + 0.0f);
  const uint32_t u = __builtin_bit_cast(uint16_t, h);
  const uint32_t neg = (uint32_t)((int32_t)(u << 16) >> 31);   // ~0 for a negative d
  return (u >> 8) ^ 0x80u ^ (neg & 0x7fu);
}

__device__ __forceinline__ uint32_t shifted_bin_one(float x, const Shift& sh) {
  const float d = sh.on ? x - sh.th : x;
  return d < sh.cut ? 0u : bin_one(d);
}

constexpr float kBandFrac = 0.125f;  // band: scores down to about theta - |theta|/8

// Floor the prediction implies: the bin of d = -|theta|/8 (above the lumping
// cut at -|theta|/4); 0 (no constraint) without a finite nonzero theta.
__device__ __forceinline__ uint32_t band_lo(const Shift& sh) {
  const float a = fabsf(sh.th);
  if (!sh.on || !(a > 0.f) || !(a < __builtin_inff())) return 0u;
  return bin_one(-kBandFrac * a);
}

}  // namespace
