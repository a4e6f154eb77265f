// Shared device helpers for the gfx950 kernels of libech (wave64 throughout).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ech.h"

#define ECH_LAUNCH_CHECK()                                   \
  do {                                                       \
    if (hipGetLastError() != hipSuccess) return ECH_EHIP;    \
  } while (0)

namespace ech {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Order-preserving 32-bit key of a float: a < b  <=>  ord(a) < ord(b) for all
// non-NaN values, with -0.0 folded onto +0.0 so equal scores get equal keys.
__device__ __forceinline__ uint32_t ord_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) == 0u) u = 0u;           // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float ord_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Add one to hist[bin] for every active lane with a plain LDS atomic. Merging
// lanes that share a bin first (leader election with ballots) was measured
// slower on gfx950 for every distribution here: the LDS serialises
// same-address atomics cheaply, the ballot loop costs more.
__device__ __forceinline__ void lds_hist_add(int* hist, uint32_t bin, bool active) {
  if (active) atomicAdd(&hist[bin], 1);
}

// A global counter bumped by many lanes: one atomic per wave with the number
// of flagged lanes, instead of one per lane. Atomics on
// one word serialise in one L2 channel, which made per-lane counting cost tens
// of microseconds over 10^5 entries. Call from converged code: every active
// lane takes part in the ballots.
__device__ __forceinline__ void wave_count(int32_t* addr, bool flag) {
  const unsigned long long m = __ballot(flag);
  if (m != 0ull && lane_id() == __builtin_ctzll(m)) atomicAdd(addr, (int)__popcll(m));
}

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// Exclusive prefix sum across a block of NT threads; returns the thread's
// exclusive prefix and writes the block total to *total. `scratch` holds at
// least NT/64 ints of LDS. Contains __syncthreads(): call from all threads.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* scratch, int* total) {
  constexpr int NW = NT / kWave;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  int incl = wave_incl_scan(v);
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    int s = scratch[i];
    wbase += (i < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

template <int NT>
__device__ __forceinline__ int block_sum(int v, int* scratch) {
  int tot;
  (void)block_excl_scan<NT>(v, scratch, &tot);
  return tot;
}

}  // namespace ech
