// Sparse attention over the selected slots of the device cache: the consumer
// of sel_slot. The attention reads a fixed device pool through the index
// tensor the cache step rewrites every step (ECHO Guide blog, "CUDA Graph
// Compatibility via Pre-Allocated Tensor Pointers"), so its launch never
// changes between steps. Rows are DeepSeek-V3.2-style absorbed MLA rows: 576
// bf16 values, all of them the key and the first 512 the value.
//
// Work split. A workgroup takes one (sequence, token span) and every head
// (or half of 128 heads when there are fewer workgroups than CUs): each of
// its waves owns 16 heads. The span's rows are gathered 32
// tokens at a time from HBM into LDS once for all heads, token-major for the
// scores and transposed (value column-major) for the output product, so each
// row crosses HBM once. Per 32-token tile and wave, on the matrix cores
// (v_mfma_f32_16x16x32_bf16):
//   S^T[token][head] = K . Q^T      2 token tiles x 18 contraction steps
//   O^T[col][head]  += V^T . P^T    32 column tiles, contraction = 32 tokens
// S^T leaves each lane one head (lane % 16) and 4+4 tokens, which are exactly
// the 8 contraction elements the same lane supplies as B of the output
// product when the token order inside the contraction is permuted the same
// way in A (the permutation is free as long as A and B agree). So the
// softmax probabilities never leave registers, and the online-softmax
// rescale is one multiply per accumulator (every accumulator of a lane
// belongs to its head). Scores are kept in the base-2 domain.
//
// Spans are merged by a second kernel from per-span (max, sum, unnormalised
// output) partials in the workspace.
#include <algorithm>

#include "common.hpp"
#include "score.hpp"

namespace {

constexpr int kRowV = 576;                 // values per row (key width)
constexpr int kValV = 512;                 // value width
constexpr int kTile = 32;                  // tokens per LDS tile
constexpr int kKs = kRowV / 32;            // contraction steps of the scores (18)
constexpr int kCt = kValV / 16;            // column tiles of the output (32)
constexpr int kKPitch = kRowV * 2 + 16;    // bytes per token row in LDS (bank spread)
constexpr int kVPitch = 72;                // bytes per value column in LDS (32 tokens + pad)
constexpr int kChunks = kRowV * 2 / 16;    // 16-byte pieces per row (72)
constexpr int kVChunks = kValV * 2 / 16;   // of which value (64)
constexpr int kMaxWaves = 8;               // heads <= 128
constexpr size_t kLdsBytes = (size_t)kTile * kKPitch + (size_t)kValV * kVPitch + kTile * 4;

__device__ __forceinline__ float lane_group_max(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Gather the rows of tile tokens [t0, t0 + 32) of this span into registers.
// Each thread takes pieces i = tid + j*NT, token fastest: neighbouring lanes
// then write neighbouring tokens of one value column in the transposed tile
// (2-byte stores without bank conflicts; token-major pieces would put 16
// lanes on 4 banks), and 16-byte row pieces of neighbouring tokens, whose LDS
// rows the pitch spreads over all banks. Every slot id is read first with a
// clamped index and every row piece after, with no branch around a load, so
// a tile costs two memory round trips (a guarded load waits for all loads in
// flight before the next one issues). Invalid tokens read slot 0; the
// result says whether piece 0's token is valid.
template <int NT>
__device__ __forceinline__ uint32_t tile_load(const uint4* __restrict__ cache, const int32_t* __restrict__ sel,
                                              int C, int t0, int t1,
                                              uint4 (&reg)[(kTile * kChunks + NT - 1) / NT]) {
  constexpr int kP = (kTile * kChunks + NT - 1) / NT;
  int slot[kP];
#pragma unroll
  for (int j = 0; j < kP; ++j) {
    const int i = threadIdx.x + j * NT;
    const int t = i % kTile;
    slot[j] = sel[min(t0 + t, t1 - 1)];
  }
  uint32_t ok0 = 0;
#pragma unroll
  for (int j = 0; j < kP; ++j) {
    const int i = threadIdx.x + j * NT;
    const int ch = min(i / kTile, kChunks - 1), t = i % kTile;
    const bool valid = (t0 + t < t1) && slot[j] >= 0 && slot[j] < C;
    if (j == 0) ok0 = valid;
    reg[j] = cache[(size_t)(valid ? slot[j] : 0) * kChunks + ch];
  }
  return ok0;
}

// Pieces beyond the tile (i >= 32 * 72) were loaded from a clamped address
// and are dropped here. Threads 0..31 hold piece 0 of token tid (chunk 0).
template <int NT>
__device__ __forceinline__ void tile_store(uint8_t* __restrict__ lds_k, uint8_t* __restrict__ lds_v,
                                           int* __restrict__ lds_ok, uint32_t ok,
                                           const uint4 (&reg)[(kTile * kChunks + NT - 1) / NT]) {
  constexpr int kP = (kTile * kChunks + NT - 1) / NT;
#pragma unroll
  for (int j = 0; j < kP; ++j) {
    const int i = threadIdx.x + j * NT;
    if (i >= kTile * kChunks) break;
    const int ch = i / kTile, t = i - ch * kTile;
    *reinterpret_cast<uint4*>(lds_k + t * kKPitch + ch * 16) = reg[j];
    if (ch < kVChunks) {
      const uint32_t w[4] = {reg[j].x, reg[j].y, reg[j].z, reg[j].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t v = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
        *reinterpret_cast<uint16_t*>(lds_v + (ch * 8 + e) * kVPitch + t * 2) = v;
      }
    }
  }
  if (threadIdx.x < kTile) lds_ok[threadIdx.x] = (int)ok;
}

// grid (spans, B), block 64 * H/16 threads (NT fixed at compile time).
template <int NT>
__global__ void __launch_bounds__(NT, 1)
    attn_span_kernel(const uint16_t* __restrict__ q, const uint4* __restrict__ cache, int C,
                     const int32_t* __restrict__ sel_slot, int H, int k, int span, float scale2,
                     float* __restrict__ part_o, float2* __restrict__ part_ml) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* lds_k = smem;
  uint8_t* lds_v = smem + kTile * kKPitch;
  int* lds_ok = reinterpret_cast<int*>(lds_v + kValV * kVPitch);
  constexpr int kP = (kTile * kChunks + NT - 1) / NT;

  // blockIdx.x = span * hsplit + head group (hsplit = H / heads per workgroup)
  const int hsplit = H / (NT / 4);
  const int b = blockIdx.y, sp = blockIdx.x / hsplit, nsp = gridDim.x / hsplit;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int h = (blockIdx.x % hsplit) * (NT / 4) + wave * 16 + col;   // this lane's head (S^T, O^T column)
  const int32_t* sel = sel_slot + (size_t)b * k;
  const int t_begin = sp * span, t_end = min(k, t_begin + span);

  // Q^T fragments (B operand of the scores): head h, dims 32 s + 8 grp .. +8.
  bf16x8_t qf[kKs];
  const uint8_t* qrow = reinterpret_cast<const uint8_t*>(q + ((size_t)b * H + h) * kRowV);
#pragma unroll
  for (int s = 0; s < kKs; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + s * 64 + grp * 16));

  f32x4_t acc[kCt];
#pragma unroll
  for (int c = 0; c < kCt; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), l = 0.f;

  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    {
      uint4 reg[kP];
      const uint32_t ok = tile_load<NT>(cache, sel, C, t0, t_end, reg);
      __syncthreads();                                       // the previous tile is consumed
      tile_store<NT>(lds_k, lds_v, lds_ok, ok, reg);
      __syncthreads();
    }

    // scores of the 32 tokens for this wave's 16 heads
    f32x4_t st[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      st[sub] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint8_t* kr = lds_k + (sub * 16 + col) * kKPitch + grp * 16;
#pragma unroll
      for (int s = 0; s < kKs; ++s)
        st[sub] = mfma(as_bf16x8(*reinterpret_cast<const uint4*>(kr + s * 64)), qf[s], st[sub]);
    }
    float sv[8];
    float tmax = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = (j < 4) ? (4 * grp + j) : (16 + 4 * grp + j - 4);
      sv[j] = lds_ok[t] ? st[j >> 2][j & 3] * scale2 : -__builtin_inff();
      tmax = fmaxf(tmax, sv[j]);
    }
    tmax = lane_group_max(tmax);
    // The running max moves only when some head's tile max exceeds it by more
    // than 8 (base 2): weights up to 2^8 stay exact enough in fp32 sums and
    // in bf16, and most tiles then skip the rescale of the accumulators.
    const bool grow = __any(tmax > m + 8.f);
    const float mn = grow ? fmaxf(m, tmax) : m;
    const bool none = (mn == -__builtin_inff());
    const float alpha = none ? 1.f : exp2f(m - mn);
    float psum = 0.f;
    bf16x8_t pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = none ? 0.f : exp2f(sv[j] - mn);
      psum += p;
      pb[j] = (__bf16)p;
    }
    l = l * alpha + lane_group_sum(psum);
    m = mn;
    if (grow) {
#pragma unroll
      for (int c = 0; c < kCt; ++c) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[c][v] *= alpha;
      }
    }
    // O^T += V^T . P^T: A = value column (ct*16 + col) at this lane group's tokens
#pragma unroll
    for (int c = 0; c < kCt; ++c) {
      const uint8_t* vr = lds_v + (c * 16 + col) * kVPitch;
      const uint2 lo = *reinterpret_cast<const uint2*>(vr + 8 * grp);
      const uint2 hi = *reinterpret_cast<const uint2*>(vr + 32 + 8 * grp);
      acc[c] = mfma(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, acc[c]);
    }
  }

  // partials: O^T column c = ct*16 + 4 grp + v of head h
  float* po = part_o + (((size_t)b * nsp + sp) * H + h) * kValV;
#pragma unroll
  for (int c = 0; c < kCt; ++c) *reinterpret_cast<f32x4_t*>(po + c * 16 + 4 * grp) = acc[c];
  if (grp == 0) part_ml[((size_t)b * nsp + sp) * H + h] = make_float2(m, l);
}

// out[b, h, :] and lse[b, h] from the spans' partials. grid (H, B), 128 threads.
// KG = spans whose loads are in flight together (8 for up to 8 spans, else 32).
template <int kG>
__global__ void __launch_bounds__(128)
    attn_merge_kernel(const float* __restrict__ part_o, const float2* __restrict__ part_ml, int H, int nsp,
                      float* __restrict__ out, float* __restrict__ lse) {
  const int h = blockIdx.x, b = blockIdx.y;
  // Every load below is clamped and unguarded, so a group's loads all issue
  // before the first wait; spans past the end are masked in arithmetic.
  float mx = -__builtin_inff();
  for (int s0 = 0; s0 < nsp; s0 += kG) {
    float2 ml[kG];
#pragma unroll
    for (int j = 0; j < kG; ++j) ml[j] = part_ml[((size_t)b * nsp + min(s0 + j, nsp - 1)) * H + h];
#pragma unroll
    for (int j = 0; j < kG; ++j) mx = fmaxf(mx, ml[j].x);          // clamped repeats change nothing
  }
  float den = 0.f;
  f32x4_t o = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (mx != -__builtin_inff()) {
    for (int s0 = 0; s0 < nsp; s0 += kG) {
      f32x4_t v[kG];
      float2 ml[kG];
#pragma unroll
      for (int j = 0; j < kG; ++j) {
        const size_t sj = (size_t)b * nsp + min(s0 + j, nsp - 1);
        v[j] = *reinterpret_cast<const f32x4_t*>(part_o + (sj * H + h) * kValV + 4 * threadIdx.x);
        ml[j] = part_ml[sj * H + h];
      }
#pragma unroll
      for (int j = 0; j < kG; ++j) {
        const float wgt = (s0 + j < nsp) ? exp2f(ml[j].x - mx) : 0.f;   // 0 also for a span that saw nothing
        den += wgt * ml[j].y;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] += wgt * v[j][e];
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] *= inv;
  *reinterpret_cast<f32x4_t*>(out + ((size_t)b * H + h) * kValV + 4 * threadIdx.x) = o;
  if (lse && threadIdx.x == 0)
    lse[(size_t)b * H + h] = den > 0.f ? (mx + log2f(den)) * 0.69314718055994531f : -__builtin_inff();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int spans_for(int B, int k) {
  // about one workgroup per CU over 256 CUs (a workgroup of 8 waves holds a
  // CU's registers), spans of whole 32-token tiles
  const int tiles = (k + kTile - 1) / kTile;
  int nsp = (256 + B - 1) / B;
  nsp = std::max(1, std::min(nsp, tiles));
  const int per = (tiles + nsp - 1) / nsp;
  return (tiles + per - 1) / per;
}

int span_tokens(int B, int k) {
  const int tiles = (k + kTile - 1) / kTile;
  const int nsp = spans_for(B, k);
  return ((tiles + nsp - 1) / nsp) * kTile;
}

}  // namespace

extern "C" size_t ech_sparse_attn_ws_bytes(int B, int H, int k) {
  if (B < 1 || H < 16 || H > 16 * kMaxWaves || H % 16 || k < 1 || k > 65536) return 0;
  const size_t nsp = (size_t)spans_for(B, k);
  const size_t o = nsp * B * H * kValV * sizeof(float);
  return ((o + 255) & ~(size_t)255) + nsp * B * H * sizeof(float2);
}

extern "C" int ech_sparse_attn(const void* q, const void* dev_cache, int32_t C, const int32_t* sel_slot, int B,
                               int H, int k, float sm_scale, float* out, float* lse, void* ws, size_t ws_bytes,
                               void* stream) {
  if (!q || !dev_cache || !sel_slot || !out || !ws) return ECH_EINVAL;
  if (B < 1 || B > 65535 || C < 1 || H < 16 || H > 16 * kMaxWaves || H % 16 || k < 1 || k > 65536)
    return ECH_EINVAL;
  if (!(sm_scale == sm_scale) || !aligned16(q) || !aligned16(dev_cache) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(ws) & 255u))
    return ECH_EINVAL;
  if (ws_bytes < ech_sparse_attn_ws_bytes(B, H, k)) return ECH_EINVAL;
  const int nsp = spans_for(B, k), span = span_tokens(B, k);
  const size_t o = (size_t)nsp * B * H * kValV * sizeof(float);
  float* part_o = static_cast<float*>(ws);
  float2* part_ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + ((o + 255) & ~(size_t)255));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const float scale2 = sm_scale * 1.4426950408889634f;
  // With fewer workgroups than CUs (a few sequences), 128 heads go to two
  // workgroups of 64 per span: twice the workgroups, rows read twice (one
  // sequence: 36 -> 29 us). With more, one workgroup of 128 reads each row
  // once and its 8 waves fill a CU.
  const int hsplit = (H == 16 * kMaxWaves && B * nsp < 256) ? 2 : 1;
  const dim3 grid(nsp * hsplit, B);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* cc = static_cast<const uint4*>(dev_cache);
  switch (H / 16 / hsplit) {
#define ECH_ATTN_CASE(W)                                                                                      \
  case W:                                                                                                     \
    hipLaunchKernelGGL(attn_span_kernel<64 * W>, grid, dim3(64 * W), kLdsBytes, s, qq, cc, C, sel_slot, H, k, \
                       span, scale2, part_o, part_ml);                                                        \
    break;
    ECH_ATTN_CASE(1)
    ECH_ATTN_CASE(2)
    ECH_ATTN_CASE(3)
    ECH_ATTN_CASE(4)
    ECH_ATTN_CASE(5)
    ECH_ATTN_CASE(6)
    ECH_ATTN_CASE(7)
    ECH_ATTN_CASE(8)
#undef ECH_ATTN_CASE
    default:
      return ECH_EINVAL;
  }
  ECH_LAUNCH_CHECK();
  if (nsp <= 8)
    hipLaunchKernelGGL(attn_merge_kernel<8>, dim3(H, B), dim3(kValV / 4), 0, s, part_o, part_ml, H, nsp, out, lse);
  else
    hipLaunchKernelGGL(attn_merge_kernel<32>, dim3(H, B), dim3(kValV / 4), 0, s, part_o, part_ml, H, nsp, out, lse);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}
