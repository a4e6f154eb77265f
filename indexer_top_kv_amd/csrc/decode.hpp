// The fp8 decode scores of one wave, shared by the plain scores kernel
// (logits.hip) and the fused scores + early-fetch kernel (fused.hip), so that
// both write the same bit patterns.
//
// The fp8 key stream goes through LDS with direct-to-LDS loads
// (global_load_lds_dwordx4). Every load instruction then reads a contiguous
// 1 KiB (8 whole 128-byte key rows) with the nontemporal hint; register loads
// in the MFMA operand layout cannot, because that layout puts 16 different
// tokens in a wave's 64 lanes, so each of their instructions touches half of
// 16 rows. Measured on MI355X with loads only: 6.2 TB/s for the half-row
// pattern (5.8 with the hint), 7.1 TB/s for whole rows with it.
//
// Each wave is independent (no barrier): it loads its query straight into
// registers, then streams its own TPW tiles of 16 tokens through a private
// ring of NS slots (NS - 1 tiles in flight). Small workgroups that start
// cheaply let the hardware dispatcher balance the work: on MI355X waves with
// equal shares of the stream finish up to 1.6x apart, so a fixed split (one
// persistent workgroup per slot) waits for the slowest. Measured at 32 x
// 131072 tokens: 16 tiles per wave and 4 waves per workgroup were best (8
// tiles: +25%, the start of each workgroup dominates; 32 tiles: +6%, a longer
// tail).
//
// Within a slot, token t's 16-byte chunk c sits at position 8t + (c ^ swz(t)):
// a DMA lane may fetch any chunk of its instruction's 1 KiB, so the
// permutation costs nothing on the global side, and it makes the MFMA-layout
// reads (16 tokens, same chunk) hit distinct banks in every group of 8 and of
// 16 lanes.
#pragma once

#include "score.hpp"

namespace {

constexpr int kDecTile = 16 * kD;   // 2 KiB of fp8 keys per 16-token tile

__device__ __forceinline__ int swz(int t) { return (t & 7) ^ (t >> 3); }

// s_waitcnt vmcnt(n) alone (lgkmcnt and expcnt not waited; gfx9 encoding).
// n is a constant once the tile loop is unrolled, so the switch folds away.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define ECH_W(k) \
  case k:        \
    __builtin_amdgcn_s_waitcnt(((k) & 15) | (((k) >> 4) << 14) | 0x70 | 0xF00); \
    break;
    ECH_W(0) ECH_W(1) ECH_W(2) ECH_W(3) ECH_W(4) ECH_W(5) ECH_W(6) ECH_W(7) ECH_W(8) ECH_W(9) ECH_W(10)
    ECH_W(11) ECH_W(12) ECH_W(13) ECH_W(14) ECH_W(15)
#undef ECH_W
    default:
      __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);
      break;
  }
}

#define ECH_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// A tile's two 16-byte key pieces and its scale, read from LDS; they have
// returned when this returns. Written as asm because the compiler cannot tell
// the ring slots apart: before a plain LDS read it waits for every
// outstanding direct-to-LDS load (vmcnt(0)), which leaves one tile in flight.
// The kernel's own vmcnt wait orders these reads after the loads of their
// slot, and the lgkmcnt wait inside the block also frees the slot for its
// next load. The outputs are early-clobber: a read may return before a later
// read of the block has taken its address.
__device__ __forceinline__ float read_tile(KeyFrag<ECH_KEY_FP8>& f, const uint8_t* p0, const uint8_t* p1,
                                           const float* ps) {
  const uint32_t a0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ECH_LDS(p0)));
  const uint32_t a1 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ECH_LDS(p1)));
  const uint32_t a2 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ECH_LDS(ps)));
  u32x4_t x0, x1;
  float sc;
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %4\n\t"
      "ds_read_b32 %2, %5\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(x1), "=&v"(sc)
      : "v"(a0), "v"(a1), "v"(a2)
      : "memory");
  f.c[0] = uint4{x0.x, x0.y, x0.z, x0.w};
  f.c[1] = uint4{x1.x, x1.y, x1.z, x1.w};
  return sc;
}

// Scores of the TPW*16 tokens wt0 .. wt0+16*TPW-1 of row r (first global
// token g0, len tokens; wt0 < len), through this wave's private LDS ring
// (NS slots of kDecTile bytes) and scale ring (2 x 64 floats). On return,
// lane l holds in keep[j] the score of token wt0 + 64j + l (tokens past the
// row end hold scores of the clamped last token and must not be used).
template <int TPW, int NS>
__device__ __forceinline__ void fp8_wave_scores(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                                const uint8_t* __restrict__ kc, const float* __restrict__ ksc, int r,
                                                int64_t g0, int len, int wt0, uint8_t (*ring)[kDecTile],
                                                float (*sring)[64], float (&keep)[(TPW + 3) / 4]) {
  constexpr int kAux = 2;                   // cache policy of the stream: nontemporal
  // A scale load brings the scales of 4 tiles; while tile it is read, the
  // loads of at most NS - 1 later tiles are out, so 2 scale slots suffice.
  static_assert(NS >= 2 && NS <= 5, "ring depth");
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  // Query fragments and head weights straight into registers (every wave of
  // the row reads the same 16 KiB, mostly from L2); issued before the key
  // stream, so waiting for them never waits for a key load.
  bf16x8_t a[4][4];
  float wv[4][4];
  {
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(q + (size_t)r * kH * kD);
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        a[ht][s] = as_bf16x8(*reinterpret_cast<const uint4*>(qb + (16 * ht + col) * (kD * 2) +
                                                              2 * dim0_of<ECH_KEY_FP8>(grp, s)));
#pragma unroll
      for (int u = 0; u < 4; ++u) wv[ht][u] = w[(size_t)r * kH + 16 * ht + 4 * grp + u];
    }
  }
  const uint8_t* kbase = kc + (size_t)g0 * kD;
  const float* sbase = ksc + g0;
  // DMA lane roles: lane i of half j fetches token 8j + i/8, chunk (i%8) ^ swz.
  const int dt = lane >> 3, dc = lane & 7;
  // Tile u: (every 4th tile) the scales of tiles u..u+3, then both key halves
  // into slot u % NS. Tokens past the row end are clamped to len - 1 (loads
  // stay inside the row; their scores are never stored). Each load is pinned
  // in this order: the waits below count loads in issue order.
  auto issue = [&](int u) {
    if ((u & 3) == 0) {
      const int tc = min(wt0 + u * 16 + lane, len - 1);
      __builtin_amdgcn_global_load_lds(sbase + tc, ECH_LDS(&sring[(u >> 2) & 1][0]), 4, 0, kAux);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int t = 8 * j + dt;
      const int tc = min(wt0 + u * 16 + t, len - 1);
      __builtin_amdgcn_global_load_lds(kbase + (size_t)tc * kD + 16 * (dc ^ swz(t)),
                                       ECH_LDS(&ring[u % NS][1024 * j]), 16, 0, kAux);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto loads_of = [](int u) { return 2 + ((u & 3) == 0 ? 1 : 0); };
#pragma unroll
  for (int u = 0; u < NS - 1 && u < TPW; ++u) issue(u);

  // Tile it's score goes to lane group it % 4, so every 4 tiles leave 64
  // consecutive scores, one per lane. They are stored after the last tile
  // (score stores in the middle of the key stream cost more).
#pragma unroll
  for (int j = 0; j < (TPW + 3) / 4; ++j) keep[j] = 0.f;
#pragma unroll
  for (int it = 0; it < TPW; ++it) {
    if (it + NS - 1 < TPW) issue(it + NS - 1);   // refills the slot read for tile it - 1
    // Loads complete in issue order: tile it's keys (and its scales, issued
    // earlier) are in once at most the loads of the later tiles are out.
    int later = 0;
#pragma unroll
    for (int u = it + 1; u < TPW && u < it + NS; ++u) later += loads_of(u);
    wait_vmcnt(later);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* rd = &ring[it % NS][128 * col];
    KeyFrag<ECH_KEY_FP8> f;
    const float sc = read_tile(f, rd + 16 * (grp ^ swz(col)), rd + 16 * ((4 + grp) ^ swz(col)),
                               &sring[(it >> 2) & 1][16 * (it & 3) + col]);
    bf16x8_t b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s] = key_step<ECH_KEY_FP8>(f, s);
    const float v = tile_score(a, wv, b, sc);
    if ((it & 3) == grp) keep[it >> 2] = v;
  }
}

// Store the wave's first n scores (keep layout above) to dst, through the
// idle ring slot (the last tile waited for every load) so that each lane
// stores 4 consecutive scores: 1 KiB per store instruction.
template <int TPW>
__device__ __forceinline__ void fp8_wave_store(const float (&keep)[(TPW + 3) / 4], uint8_t* ring0, float* dst,
                                               int n) {
  const int lane = threadIdx.x & 63;
  float* sw = reinterpret_cast<float*>(ring0);
#pragma unroll
  for (int j = 0; j < (TPW + 3) / 4; ++j) sw[64 * j + lane] = keep[j];
  if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
#pragma unroll
    for (int i = 4 * lane; i < TPW * 16; i += 256) {
      if (i + 3 < n) {
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4_t*>(sw + i), reinterpret_cast<f32x4_t*>(dst + i));
      } else {
        for (int k = i; k < n; ++k) dst[k] = sw[k];
      }
    }
  } else {
    for (int i = lane; i < n; i += 64) dst[i] = sw[i];
  }
}

}  // namespace
