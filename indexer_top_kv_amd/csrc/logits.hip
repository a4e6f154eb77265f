// Lightning-indexer scores on gfx950 matrix cores.
//
// logit[r,t] = sum_h w[r,h] * ReLU(q[r,h,:] . k[g,:]), g = tok0 + t, over every
// cached token (ECHO explainer: "Fused indexer kernel (extends DeepGEMM)",
// "Decode: fetch above a predicted threshold"; the lightning-indexer form).
// The MFMA tile, its operand layout and the fused epilogue are in score.hpp.

#include <algorithm>

#include "decode.hpp"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

// ------------------------------------------------------------------ decode
// grid (ceil(max_len / (kWaves*TPW*16)), R). Each wave handles TPW tiles of 16
// tokens; the WG's waves interleave tiles so they stream adjacent 2-4 KiB
// pieces. The tile loop is fully unrolled (TPW is a template parameter):
// in straight-line code the compiler counts the outstanding loads exactly and
// keeps three tiles in flight while one is multiplied, which it does not do
// across a loop back-edge.
template <int KDT, int TPW>
__global__ __launch_bounds__(kThreads) void logits_decode_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ kc,
    const float* __restrict__ ksc, const int64_t* __restrict__ tok0, const int32_t* __restrict__ lens,
    float* __restrict__ out, int64_t ld) {
  constexpr int kRowB = (KDT == ECH_KEY_FP8) ? kD : 2 * kD;
  constexpr int kDepth = 3;   // tiles in flight ahead of the one being multiplied
  const int r = blockIdx.y;
  const int len = lens[r];
  const int wg_t0 = blockIdx.x * (kWaves * TPW * 16);
  if (wg_t0 >= len) return;
  __shared__ uint4 qs[kH * kD * 2 / 16];
  // The WG's scores are buffered here and written once at the end as full
  // coalesced lines: per-tile 64-byte stores interleaved with the key stream
  // cost ~15% of the bandwidth.
  __shared__ float sbuf[kWaves * TPW * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  bf16x8_t a[4][4];
  float wv[4][4];
  load_query<KDT>(q + (size_t)r * kH * kD, w + (size_t)r * kH, qs, a, wv, col, grp);

  const int64_t g0 = tok0[r];
  const uint8_t* kbase = kc + (size_t)g0 * kRowB;
  const float* sbase = (KDT == ECH_KEY_FP8) ? ksc + g0 : nullptr;
  float* orow = out + (size_t)r * ld;
  // This wave's tiles start at wg_t0 + (it * kWaves + wave) * 16. Tokens past
  // the row end are clamped to len - 1 so loads stay inside the row; their
  // scores are never written out.
  const int first = wg_t0 + wave * 16;

  KeyFrag<KDT> f[kDepth + 1];
  float sc[kDepth + 1];
  auto load = [&](int buf, int it) {
    const int tc = min(first + it * kWaves * 16 + col, len - 1);
    load_key<KDT>(f[buf], kbase + (size_t)tc * kRowB, grp);
    sc[buf] = (KDT == ECH_KEY_FP8) ? sbase[tc] : 1.f;
  };
#pragma unroll
  for (int it = 0; it < kDepth && it < TPW; ++it) load(it, it);
#pragma unroll
  for (int it = 0; it < TPW; ++it) {
    if (it + kDepth < TPW) load((it + kDepth) % (kDepth + 1), it + kDepth);
    // Keep the prefetch where it is: without this the scheduler sinks the
    // loads towards their use and the tiles in flight drop to about one.
    __builtin_amdgcn_sched_barrier(0);
    const int buf = it % (kDepth + 1);
    bf16x8_t b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s] = key_step<KDT>(f[buf], s);
    const float v = tile_score(a, wv, b, sc[buf]);
    sbuf[(it * kWaves + wave) * 16 + col] = v;   // the 4 lane groups hold the same sum
  }
  __syncthreads();
  const int n = min(kWaves * TPW * 16, len - wg_t0);
  float* dst = orow + wg_t0;
  if ((ld & 3) == 0) {   // rows 16-byte aligned: float4 stores
    for (int i = 4 * threadIdx.x; i < n; i += 4 * kThreads) {
      if (i + 3 < n) {
        *reinterpret_cast<float4*>(dst + i) = *reinterpret_cast<const float4*>(sbuf + i);
      } else {
        for (int j = i; j < n; ++j) dst[j] = sbuf[j];
      }
    }
  } else {
    for (int i = threadIdx.x; i < n; i += kThreads) dst[i] = sbuf[i];
  }
}

// ------------------------------------------------------------------ decode, fp8 keys
// The wave body (direct-to-LDS key stream, MFMA tile, fused epilogue) is in
// decode.hpp, shared with the fused scores + early-fetch kernel.
template <int TPW, int NS, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void logits_decode_fp8_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ kc,
    const float* __restrict__ ksc, const int64_t* __restrict__ tok0, const int32_t* __restrict__ lens,
    float* __restrict__ out, int64_t ld) {
  const int r = blockIdx.y;
  const int len = lens[r];
  const int wave = WAVES == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wt0 = (blockIdx.x * WAVES + wave) * (TPW * 16);   // this wave's first token
  if (wt0 >= len) return;
  __shared__ __attribute__((aligned(16))) uint8_t ring[WAVES][NS][kDecTile];
  __shared__ __attribute__((aligned(16))) float sring[WAVES][2][64];
  float keep[(TPW + 3) / 4];
  fp8_wave_scores<TPW, NS>(q, w, kc, ksc, r, tok0[r], len, wt0, ring[wave], sring[wave], keep);
  fp8_wave_store<TPW>(keep, &ring[wave][0][0], out + (size_t)r * ld + wt0, min(TPW * 16, len - wt0));
}

template <int WAVES>
hipError_t launch_decode_fp8(int tpw, int R, int max_len, hipStream_t s, const uint16_t* q, const float* w,
                             const uint8_t* kc, const float* ksc, const int64_t* tok0, const int32_t* lens,
                             float* out, int64_t ld) {
  constexpr int kNS = 4;
  const dim3 grid((max_len + WAVES * tpw * 16 - 1) / (WAVES * tpw * 16), R);
  switch (tpw) {
#define ECH_DEC8(T)                                                                                     \
  case T:                                                                                               \
    hipLaunchKernelGGL((logits_decode_fp8_kernel<T, kNS, WAVES>), grid, dim3(WAVES * 64), 0, s, q, w, kc, \
                       ksc, tok0, lens, out, ld);                                                       \
    break;
    ECH_DEC8(1) ECH_DEC8(2) ECH_DEC8(4) ECH_DEC8(8) ECH_DEC8(16)
#undef ECH_DEC8
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KDT>
hipError_t launch_decode(int tpw, dim3 grid, hipStream_t s, const uint16_t* q, const float* w, const uint8_t* kc,
                         const float* ksc, const int64_t* tok0, const int32_t* lens, float* out, int64_t ld) {
  switch (tpw) {
#define ECH_DEC(T)                                                                                          \
  case T:                                                                                                   \
    hipLaunchKernelGGL((logits_decode_kernel<KDT, T>), grid, dim3(kThreads), 0, s, q, w, kc, ksc, tok0, lens, \
                       out, ld);                                                                            \
    break;
    ECH_DEC(1) ECH_DEC(2) ECH_DEC(4) ECH_DEC(8) ECH_DEC(16) ECH_DEC(32)
#undef ECH_DEC
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ causal prefill
// One WG = kWaves query rows (one per wave) x a span of kSpan tokens. Key
// tiles of 64 tokens are widened to bf16 once and staged in LDS (rows padded
// to 272 B so the 16-lane column reads hit distinct banks), double-buffered,
// with the next tile's global loads in flight during the current tile's
// MFMAs; every wave multiplies its row's q against them. Row r sees
// t <= row0 + r.
constexpr int kPTile = 64;                  // tokens per LDS stage
constexpr int kPStride = 2 * kD + 16;       // padded bf16 key row in LDS (bytes)
constexpr int kSpan = 4096;                 // tokens per WG

// Staging of one 64-token key tile, split in two so the global loads of
// tile i+1 are in flight while tile i is multiplied: fetch() issues them into
// registers, commit() widens fp8 to bf16 and writes the LDS tile.
// 256 threads; thread -> token tid/4; fp8: bytes 32*(tid%4) .. +32 (-> 64 B
// bf16); bf16: bytes 64*(tid%4) .. +64.
template <int KDT>
struct Staged {
  uint4 v[KDT == ECH_KEY_FP8 ? 2 : 4];
  float sc;
};

template <int KDT>
__device__ __forceinline__ void stage_fetch(Staged<KDT>& r, const uint8_t* __restrict__ kbase,
                                            const float* __restrict__ sbase, int t0, int nvalid) {
  const int tid = threadIdx.x;
  const int tok = tid >> 2, part = tid & 3;
  const int tsrc = t0 + min(tok, max(nvalid - 1, 0));
  if constexpr (KDT == ECH_KEY_FP8) {
    const uint4* s = reinterpret_cast<const uint4*>(kbase + (size_t)tsrc * kD + 32 * part);
    r.v[0] = s[0];
    r.v[1] = s[1];
    r.sc = sbase[tsrc];
  } else {
    const uint4* s = reinterpret_cast<const uint4*>(kbase + (size_t)tsrc * 2 * kD + 64 * part);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = s[i];
    r.sc = 1.f;
  }
}

template <int KDT>
__device__ __forceinline__ void stage_commit(const Staged<KDT>& r, uint8_t* dst, float* sdst) {
  const int tid = threadIdx.x;
  const int tok = tid >> 2, part = tid & 3;
  uint8_t* d = dst + tok * kPStride;
  if constexpr (KDT == ECH_KEY_FP8) {
    const uint4 x = r.v[0], y = r.v[1];
    u32x4_t o0 = {cvt_lo(x.x), cvt_hi(x.x), cvt_lo(x.y), cvt_hi(x.y)};
    u32x4_t o1 = {cvt_lo(x.z), cvt_hi(x.z), cvt_lo(x.w), cvt_hi(x.w)};
    u32x4_t o2 = {cvt_lo(y.x), cvt_hi(y.x), cvt_lo(y.y), cvt_hi(y.y)};
    u32x4_t o3 = {cvt_lo(y.z), cvt_hi(y.z), cvt_lo(y.w), cvt_hi(y.w)};
    u32x4_t* dd = reinterpret_cast<u32x4_t*>(d + 64 * part);
    dd[0] = o0;
    dd[1] = o1;
    dd[2] = o2;
    dd[3] = o3;
  } else {
    uint4* dd = reinterpret_cast<uint4*>(d + 64 * part);
#pragma unroll
    for (int i = 0; i < 4; ++i) dd[i] = r.v[i];
  }
  if (part == 0) sdst[tok] = r.sc;
}

template <int KDT, int RPW>
__global__ __launch_bounds__(kThreads) void logits_causal_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ kc,
    const float* __restrict__ ksc, int64_t tok0, int64_t row0, int R, float* __restrict__ out, int64_t ld) {
  constexpr int kRowB = (KDT == ECH_KEY_FP8) ? kD : 2 * kD;
  constexpr int kRows = kWaves * RPW;              // query rows per WG
  const int rg = blockIdx.x;                       // row group
  const int span0 = blockIdx.y * kSpan;
  const int r_first = rg * kRows;
  const int r_last = min(R - 1, r_first + kRows - 1);
  const int64_t vis_max = row0 + r_last + 1;       // tokens visible to the last row
  if ((int64_t)span0 >= vis_max) return;
  const int span_end = (int)min<int64_t>(vis_max, (int64_t)span0 + kSpan);

  __shared__ __attribute__((aligned(16))) uint8_t kt[2][kPTile * kPStride];
  __shared__ float st[2][kPTile];
  __shared__ float sres[kRows][kPTile];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  // wave w scores rows r_first + w*RPW + j, j < RPW: every key fragment read
  // from LDS feeds RPW rows' MFMAs
  bool row_ok[RPW];
  int64_t vis[RPW];                                // tokens t < vis are visible
  float* orow[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int r = r_first + wave * RPW + j;
    row_ok[j] = r <= r_last;
    vis[j] = row_ok[j] ? row0 + r + 1 : 0;
    orow[j] = out + (size_t)min(r, R - 1) * ld;
  }

  // A fragments and head weights straight from global memory (q rows are
  // shared by every span of the row group and stay in L2): 16-byte pieces,
  // all loads in flight at once, no staging barrier.
  bf16x8_t a[RPW][4][4];
  float wv[RPW][4][4];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int rr = min(r_first + wave * RPW + j, r_last);
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(q + (size_t)rr * kH * kD);
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int off = (16 * ht + col) * (kD * 2) + 2 * dim0_of<ECH_KEY_BF16>(grp, s);
        a[j][ht][s] = as_bf16x8(*reinterpret_cast<const uint4*>(qb + off));
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) wv[j][ht][v] = w[(size_t)rr * kH + 16 * ht + 4 * grp + v];
    }
  }

  const uint8_t* kbase = kc + (size_t)tok0 * kRowB;
  const float* sbase = (KDT == ECH_KEY_FP8) ? ksc + tok0 : nullptr;
  const int ntiles = (span_end - span0 + kPTile - 1) / kPTile;

  Staged<KDT> nxt;
  stage_fetch<KDT>(nxt, kbase, sbase, span0, span_end - span0);
  stage_commit<KDT>(nxt, kt[0], st[0]);
  __syncthreads();
#pragma unroll 1
  for (int it = 0; it < ntiles; ++it) {
    const int cb = it & 1;
    const int t0 = span0 + it * kPTile;
    const bool more = it + 1 < ntiles;
    // fp8 tiles stay in registers (8 VGPRs) while this tile is multiplied;
    // bf16 tiles are twice as large and are committed at once instead.
    if (more) stage_fetch<KDT>(nxt, kbase, sbase, t0 + kPTile, span_end - (t0 + kPTile));
    if (KDT == ECH_KEY_BF16 && more) stage_commit<KDT>(nxt, kt[cb ^ 1], st[cb ^ 1]);
    bool live = false;
#pragma unroll
    for (int j = 0; j < RPW; ++j) live |= row_ok[j] && t0 < vis[j];
    if (live) {
      // All four sub-tiles for every row of the wave; scores past a row's
      // causal edge are computed but never stored.
#pragma unroll
      for (int sub = 0; sub < kPTile / 16; ++sub) {
        const uint8_t* kr = kt[cb] + (sub * 16 + col) * kPStride;
        bf16x8_t b[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          b[s] = as_bf16x8(*reinterpret_cast<const uint4*>(kr + 2 * dim0_of<ECH_KEY_BF16>(grp, s)));
        const float sc = st[cb][sub * 16 + col];
        // Every row's MFMAs first, issued at raised wave priority; the
        // epilogues at normal priority, so the other wave on the SIMD gets its
        // MFMAs issued while this one runs VALU work (2-3% per block).
        f32x4_t acc[RPW][4];
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < RPW; ++j) tile_mfma(a[j], b, acc[j]);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < RPW; ++j) sres[wave * RPW + j][sub * 16 + col] = tile_epilogue(acc[j], wv[j], sc);
      }
    }
    if (KDT == ECH_KEY_FP8 && more) stage_commit<KDT>(nxt, kt[cb ^ 1], st[cb ^ 1]);
    __syncthreads();
    // One coalesced 256-byte store of each row's 64 scores per tile (four
    // 64-byte partial-line stores cost write bandwidth).
#pragma unroll
    for (int j = 0; j < RPW; ++j)
      if (row_ok[j] && t0 + lane < vis[j]) orow[j][t0 + lane] = sres[wave * RPW + j][lane];
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int ech_index_logits(const void* q, const float* w, const void* kcache, int kdtype,
                                const float* kscale, const int64_t* row_tok0, const int32_t* row_len,
                                int R, int H, int D, int max_len, float* logits, int64_t ld, void* stream) {
  if (!q || !w || !kcache || !row_tok0 || !row_len || !logits) return ECH_EINVAL;
  if (H != kH || D != kD || R < 1 || R > 65535 || max_len < 0 || ld < max_len) return ECH_EINVAL;
  if (kdtype != ECH_KEY_BF16 && kdtype != ECH_KEY_FP8) return ECH_EUNSUPPORTED;
  if (kdtype == ECH_KEY_FP8 && !kscale) return ECH_EINVAL;
  if (!aligned16(q) || !aligned16(kcache)) return ECH_EINVAL;
  if (max_len == 0) return ECH_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Enough WGs to fill 256 CUs; long rows give each wave up to 32 tiles so the
  // per-WG query staging (16 KiB) stays small next to the key stream.
  const int64_t total = (int64_t)R * max_len;
  // Enough WGs to fill 256 CUs several times over; long rows give each wave up
  // to 32 tiles so the per-WG query staging (16 KiB) stays small next to the
  // key stream. Tiles per wave is a power of two (one kernel per value).
  int tpw = 1;
  while (tpw < 32 && total / ((int64_t)2048 * kWaves * 16 * (tpw * 2)) >= 1) tpw *= 2;
  const int per_wg = kWaves * tpw * 16;
  dim3 grid((max_len + per_wg - 1) / per_wg, R);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint8_t* kk = static_cast<const uint8_t*>(kcache);
  const hipError_t e =
      (kdtype == ECH_KEY_FP8)
          ? launch_decode_fp8<4>(std::min(tpw, 16), R, max_len, s, qq, w, kk, kscale, row_tok0, row_len, logits, ld)
          : launch_decode<ECH_KEY_BF16>(tpw, grid, s, qq, w, kk, kscale, row_tok0, row_len, logits, ld);
  return e == hipSuccess ? ECH_OK : ECH_EHIP;
}

extern "C" int ech_index_logits_causal(const void* q, const float* w, const void* kcache, int kdtype,
                                       const float* kscale, int64_t tok0, int64_t row0, int R, int H, int D,
                                       float* logits, int64_t ld, void* stream) {
  if (!q || !w || !kcache || !logits) return ECH_EINVAL;
  if (H != kH || D != kD || R < 1 || tok0 < 0 || row0 < 0) return ECH_EINVAL;
  if (kdtype != ECH_KEY_BF16 && kdtype != ECH_KEY_FP8) return ECH_EUNSUPPORTED;
  if (kdtype == ECH_KEY_FP8 && !kscale) return ECH_EINVAL;
  if (!aligned16(q) || !aligned16(kcache)) return ECH_EINVAL;
  if (ld < row0 + R || row0 + R > (int64_t)INT32_MAX) return ECH_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t vis_max = row0 + R;
  constexpr int kRPW = 2;   // query rows per wave
  dim3 grid((R + kWaves * kRPW - 1) / (kWaves * kRPW), (unsigned)((vis_max + kSpan - 1) / kSpan));
  if (grid.y > 65535) return ECH_EINVAL;
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint8_t* kk = static_cast<const uint8_t*>(kcache);
  if (kdtype == ECH_KEY_FP8)
    hipLaunchKernelGGL((logits_causal_kernel<ECH_KEY_FP8, kRPW>), grid, dim3(kThreads), 0, s, qq, w, kk, kscale,
                       tok0, row0, R, logits, ld);
  else
    hipLaunchKernelGGL((logits_causal_kernel<ECH_KEY_BF16, kRPW>), grid, dim3(kThreads), 0, s, qq, w, kk, kscale,
                       tok0, row0, R, logits, ld);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}
