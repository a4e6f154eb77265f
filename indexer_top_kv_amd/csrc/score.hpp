// MFMA building blocks of the indexer score, shared by every kernel that
// scores tokens (decode rows, causal prefill blocks, the resident tokens of
// the early fetch), so that a (row, token) score is the same bit pattern
// whichever kernel computes it.
//
// Per token the work is a [64 heads x 128] x [128] product: heads are the M
// dimension of v_mfma_f32_16x16x32_bf16 (4 tiles of 16), tokens the N
// dimension (tiles of 16). fp8 e4m3fn keys widen exactly to bf16
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1), so every product is exact and
// only the fp32 accumulation rounds. The epilogue folds ReLU, the head
// weights and the per-token scale:
//   ReLU(s * x) = s * med3(x, 0, s >= 0 ? +inf : -inf),
// then reduces the 64 heads (16 per lane in registers, 4 lane groups by
// lane swaps and adds).
//
// MFMA operand layout used (16x16x32 bf16, wave64): lane l holds A[row l%16]
// and B[col l%16], 8 contraction elements each in lane group l/16; the
// result C[4*(l/16)+v][l%16] is in accumulator register v. Which physical
// dims a lane group holds is free as long as A and B agree, so each lane's
// key loads are 16-byte contiguous pieces of one token row.
#pragma once

#include "common.hpp"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kH = 64;
constexpr int kD = 128;

__device__ __forceinline__ uint32_t cvt_lo(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
}
__device__ __forceinline__ uint32_t cvt_hi(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true));
}

// 8 fp8 bytes (two dwords) -> 8 bf16 in byte order.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t a, uint32_t b) {
  u32x4_t v = {cvt_lo(a), cvt_hi(a), cvt_lo(b), cvt_hi(b)};
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  u32x4_t u = {v.x, v.y, v.z, v.w};
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Contraction dims held by lane group grp in MFMA step s (8 contiguous dims).
//  fp8 keys: a lane loads bytes [64i + 16grp, +16) of the 128-byte key
//            (i = 0, 1); step s = 2i + h uses the h-th 8 of them.
//  bf16 keys: a lane loads bytes [64i + 16grp, +16) of the 256-byte key
//            (i = 0..3) = dims 32i + 8grp .. +8; step s = i.
template <int KDT>
__device__ __forceinline__ int dim0_of(int grp, int s) {
  if (KDT == ECH_KEY_FP8) return 64 * (s >> 1) + 16 * grp + 8 * (s & 1);
  return 32 * s + 8 * grp;
}

template <int KDT>
struct KeyFrag;
template <>
struct KeyFrag<ECH_KEY_FP8> {
  uint4 c[2];
};
template <>
struct KeyFrag<ECH_KEY_BF16> {
  uint4 c[4];
};

template <int KDT>
__device__ __forceinline__ void load_key(KeyFrag<KDT>& f, const uint8_t* row, int grp) {
  if constexpr (KDT == ECH_KEY_FP8) {
    f.c[0] = *reinterpret_cast<const uint4*>(row + 16 * grp);
    f.c[1] = *reinterpret_cast<const uint4*>(row + 64 + 16 * grp);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.c[i] = *reinterpret_cast<const uint4*>(row + 64 * i + 16 * grp);
  }
}

template <int KDT>
__device__ __forceinline__ bf16x8_t key_step(const KeyFrag<KDT>& f, int s) {
  if constexpr (KDT == ECH_KEY_FP8) {
    const uint4 c = f.c[s >> 1];
    return (s & 1) ? fp8x8_to_bf16(c.z, c.w) : fp8x8_to_bf16(c.x, c.y);
  } else {
    return as_bf16x8(f.c[s]);
  }
}

// One 16-token tile on the matrix cores: acc[ht][v] = q[16ht + 4grp + v] . k[col].
__device__ __forceinline__ void tile_mfma(const bf16x8_t (&a)[4][4], const bf16x8_t (&b)[4], f32x4_t (&acc)[4]) {
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) acc[ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) acc[ht] = mfma(a[ht][s], b[s], acc[ht]);
  }
}

// x[l] + x[l^16] + x[l^32] + x[l^48] (the 4 lane groups) in every lane, with
// the same additions in the same order as x + xor16(x), then + xor32 of that.
// v_permlane16/32_swap of a register with itself leaves, in each lane, the
// lane's own value and its partner's in the two outputs, so their sum is the
// pair sum; unlike a shuffle (ds_bpermute) this stays in the VALU and does not
// wait on the LDS crossbar.
__device__ __forceinline__ float lane_group_sum(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Epilogue of a tile: ReLU (with the per-token scale's sign), head weights,
// head sum. Returns the score of token column (lane & 15) in every lane.
__device__ __forceinline__ float tile_epilogue(const f32x4_t (&acc)[4], const float (&wv)[4][4], float sc) {
  const float bound = sc >= 0.f ? __builtin_inff() : -__builtin_inff();
  float part = 0.f;
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
    for (int v = 0; v < 4; ++v) part = fmaf(wv[ht][v], __builtin_amdgcn_fmed3f(acc[ht][v], 0.f, bound), part);
  }
  return lane_group_sum(part) * sc;
}

__device__ __forceinline__ float tile_score(const bf16x8_t (&a)[4][4], const float (&wv)[4][4],
                                            const bf16x8_t (&b)[4], float sc) {
  f32x4_t acc[4];
  tile_mfma(a, b, acc);
  return tile_epilogue(acc, wv, sc);
}

// Load one query row [64][128] bf16 (16 KiB) into LDS, then each wave picks
// up its A fragments and head weights into registers.
template <int KDT>
__device__ __forceinline__ void load_query(const uint16_t* __restrict__ qrow, const float* __restrict__ wrow,
                                           uint4* qs, bf16x8_t (&a)[4][4], float (&wv)[4][4], int col, int grp) {
  const uint4* qg = reinterpret_cast<const uint4*>(qrow);
  for (int i = threadIdx.x; i < kH * kD * 2 / 16; i += blockDim.x) qs[i] = qg[i];
  __syncthreads();
  const uint8_t* qb = reinterpret_cast<const uint8_t*>(qs);
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int off = (16 * ht + col) * (kD * 2) + 2 * dim0_of<KDT>(grp, s);
      a[ht][s] = as_bf16x8(*reinterpret_cast<const uint4*>(qb + off));
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) wv[ht][v] = wrow[16 * ht + 4 * grp + v];
  }
}

}  // namespace
