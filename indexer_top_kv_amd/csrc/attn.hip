// Sparse attention over the selected slots of the device cache: the consumer
// of sel_slot. The attention reads a fixed device pool through the index
// tensor the cache step rewrites every step (ECHO Guide blog, "CUDA Graph
// Compatibility via Pre-Allocated Tensor Pointers"), so its launch never
// changes between steps. Rows are DeepSeek-V3.2-style absorbed MLA rows: 576
// bf16 values, all of them the key and the first 512 the value.
//
// Work split. A workgroup takes one (sequence, token span) and every head
// (or a quarter or half of them when there are fewer workgroups than CUs, the
// head groups of a span on one XCD): each of its waves owns 16 heads of one
// token lane. The span's rows are gathered 32 tokens (one tile per lane) at a
// time from HBM into LDS once for all of the workgroup's heads, so each row
// crosses HBM once. Per
// 32-token tile and wave, on the matrix cores (v_mfma_f32_16x16x32_bf16):
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
// output) partials in the workspace; two token lanes of a workgroup are
// merged in LDS before their span's partial is written.
#include <algorithm>

#include "common.hpp"
#include "score.hpp"

namespace {

constexpr int kRowV = 576;                 // values per row (key width)
constexpr int kValV = 512;                 // value width
constexpr int kTile = 32;                  // tokens per LDS tile
constexpr int kKs = kRowV / 32;            // contraction steps of the scores (18)
constexpr int kCt = kValV / 16;            // column tiles of the output (32)
constexpr int kKPitch = kRowV * 2 + 32;    // bytes per token row in LDS (bank spread)
constexpr int kChunks = kRowV * 2 / 16;    // 16-byte pieces per row (72)
constexpr int kMaxWaves = 8;               // heads <= 128
constexpr int kKD = 4;                     // key fragments in flight per wave
constexpr int kVD = 3;                     // value fragments in flight per wave

#define ECH_ATTN_LDS(p) ((__attribute__((address_space(3))) void*)(p))


__device__ __forceinline__ float lane_group_max(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// ------------------------------------------------------------------ span kernel
// NW waves of NS x 16 heads (NS = 1: 16 heads per wave, two waves per SIMD;
// two sets per wave would share every key fragment read but need 2 x 144
// fragment and 256 accumulator registers, past what a wave can hold without
// spilling). The tile stays token-major in LDS for both products: the value
// operand V^T of O^T += V^T.P^T comes from ds_read_b64_tr_b16 (within each
// 16-lane group, lane i receives element i%4 of the 8-byte pieces addressed
// by lanes 4e + i/4, e = 0..3: with lanes 4j..4j+3 pointing at token j's
// columns c, c+4, c+8, c+12, lane i gets column c+i of 4 tokens), so no
// transposed copy is stored. Rows arrive by direct-to-LDS loads into two tile
// buffers: tile i+1's loads are issued right after the barrier that opens
// tile i and run under its products. They are issued from inline asm, so
// that the compiler, which cannot tell the two buffers apart, does not wait
// for them before every LDS read; they write no register, and each tile opens
// with an explicit wait for all of them and a barrier. Slot ids go through a
// 3-deep LDS ring, loaded one tile further ahead and used only after that
// wait.
//
// LDS reads are software-pipelined: kKD key and kVD value fragments are in
// flight per wave (the scheduler is held to one read per product), where the
// compiler alone would wait for each read before its product. The row pitch
// is 74 chunks: the key reads (16 rows x 64 B per read) then hit every bank
// once per pass; measured on gfx950 with a read probe, 216 B per clock per CU
// at pitch 74 against 125 at 73 and 63 at 72; the transposed value reads
// give ~89 B per clock at any of these pitches.
constexpr int kP2 = kKPitch / 16;            // 74 chunks per token row in LDS (two spare: banks)
constexpr int kPos2 = kTile * kP2;           // 2368 chunk positions per tile
constexpr int kBuf2 = kPos2 * 16;            // 37888 bytes per tile buffer

typedef short v4s_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t tr_pair(const uint8_t* p0, const uint8_t* p1) {
  const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(p0));
  const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(p1));
  typedef short v8s_t __attribute__((ext_vector_type(8)));
  const v8s_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// grid (spans x head groups, B), block 64 * NH * TL threads: NH waves of 16
// heads for each of TL token lanes. With TL = 2 a step brings two tiles into
// LDS and the two waves of a head set take one tile each, with a softmax
// state of their own, merged in LDS at the end: half the spans (and the
// partials the merge reads) for the same waves per CU.
template <int NH, int TL>
__global__ void __launch_bounds__(64 * NH * TL, 1)
    attn_span_kernel(const uint16_t* __restrict__ q, const uint4* __restrict__ cache, int C,
                       const int32_t* __restrict__ sel_slot, int H, int k, int span, float scale2,
                       float* __restrict__ part_o, float2* __restrict__ part_ml) {
  constexpr int NS = 1;
  constexpr int NW = NH * TL;
  constexpr int kStep = TL * kTile;                    // tokens per step
  constexpr int kInstrS = (TL * kPos2 + 63) / 64;      // load instructions per step
  static_assert(kStep <= 64, "one slot id per lane of wave 0");
  __shared__ __align__(16) uint8_t tiles[2][TL * kBuf2];
  __shared__ int slots[3][kStep];   // slot id of each token of a step, -1: nothing to attend
  constexpr int kJ = (kInstrS + NW - 1) / NW;   // load instructions per wave per step
  const int hsplit = H / (16 * NH);
  const int nsp = gridDim.x / hsplit;
  // The head groups of one span run on one XCD, next to each other in
  // dispatch order (workgroups go to the XCDs round robin), so that the
  // rows they all read come from that XCD's L2 after the first read.
  int wg = blockIdx.x + blockIdx.y * gridDim.x;
  const int nwg = gridDim.x * gridDim.y;
  if (hsplit > 1 && nwg % (8 * hsplit) == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
  const int hh = wg % hsplit, b = wg / (hsplit * nsp), sp = (wg / hsplit) % nsp;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int wvu = __builtin_amdgcn_readfirstlane(wave);
  const int hw = wvu % NH, tl = wvu / NH;             // head set and token lane of this wave
  const int h0 = hh * (16 * NH) + hw * 16 + col;
  const int32_t* sel = sel_slot + (size_t)b * k;
  const int t_begin = sp * span, t_end = min(k, t_begin + span);
  const int nsteps = t_end > t_begin ? (t_end - t_begin + kStep - 1) / kStep : 0;
  const bool slot_lane = wave == 0 && lane < kStep;   // the lanes that fetch slot ids

  bf16x8_t qf[NS][kKs];   // Q^T fragments: head h0 + 16 hs, dims 32 s + 8 grp .. +8
  f32x4_t acc[NS][kCt];
  float m[NS], l[NS];

  // slot id of token t0 + lane: a clamped load, then validity in arithmetic
  auto slot_raw = [&](int t0) -> int { return sel[min(t0 + lane, t_end - 1)]; };
  auto slot_ok = [&](int t0, int sl) -> int { return (t0 + lane < t_end && sl >= 0 && sl < C) ? sl : -1; };
  // direct-to-LDS loads of the tile whose slot ids are in slots[si]; the
  // pad chunk of each LDS row and positions past the tile are not loaded
  // The lane's positions are recomputed per tile (a few integer operations)
  // and the LDS addresses are scalar: held across the loop they would take
  // registers the products need.
  auto issue = [&](int si, int buf) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ECH_ATTN_LDS(&tiles[0][0]))) +
                          static_cast<uint32_t>(buf * TL * kBuf2);
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int ins = j * NW + wv;
      const int p = ins * 64 + ln;
      const int t = p / kP2, c = p - t * kP2;
      if (ins < kInstrS && p < TL * kPos2 && c < kChunks) {
        const int sl = slots[si][t];
        const uint4* src = cache + (size_t)max(sl, 0) * kChunks + c;
        const uint32_t lds = lds0 + static_cast<uint32_t>(ins * 1024);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds), "v"(src) : "memory", "m0");
      }
    }
  };
  // the scores, online softmax and value product of the tile in cur
  auto compute = [&](const int* sid, const uint8_t* cur) {
    f32x4_t st[2][NS];   // [16-token half][head set]
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int hs = 0; hs < NS; ++hs) st[sub][hs] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      // 36 key fragments, x = 2 s + half, kKD of them in flight
      const uint8_t* kr = cur + col * kKPitch + grp * 16;
      auto kload = [&](int x) {
        return as_bf16x8(*reinterpret_cast<const uint4*>(kr + (x & 1) * 16 * kKPitch + (x >> 1) * 64));
      };
      bf16x8_t kb[kKD];
#pragma unroll
      for (int x = 0; x < kKD; ++x) kb[x] = kload(x);
#pragma unroll
      for (int x = 0; x < 2 * kKs; ++x) {
        const bf16x8_t kf = kb[x % kKD];
        if (x + kKD < 2 * kKs) kb[x % kKD] = kload(x + kKD);
#pragma unroll
        for (int hs = 0; hs < NS; ++hs) st[x & 1][hs] = mfma(kf, qf[hs][x >> 1], st[x & 1][hs]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kKD, 0);   // DS reads
#pragma unroll
      for (int x = 0; x < 2 * kKs - kKD; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, NS, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NS * kKD, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    bool ok[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) ok[j] = sid[(j < 4) ? (4 * grp + j) : (16 + 4 * grp + j - 4)] >= 0;
    bf16x8_t pb[NS];
    float alpha[NS];
    bool grow[NS];
#pragma unroll
    for (int hs = 0; hs < NS; ++hs) {
      float sv[8];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sv[j] = ok[j] ? st[j >> 2][hs][j & 3] * scale2 : -__builtin_inff();
        tmax = fmaxf(tmax, sv[j]);
      }
      tmax = lane_group_max(tmax);
      // the running max moves only when a head's tile max exceeds it by more
      // than 8 (base 2), as in the 16-head form
      grow[hs] = __any(tmax > m[hs] + 8.f);
      const float mn = grow[hs] ? fmaxf(m[hs], tmax) : m[hs];
      const bool none = (mn == -__builtin_inff());
      alpha[hs] = none ? 1.f : exp2f(m[hs] - mn);
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = none ? 0.f : exp2f(sv[j] - mn);
        psum += p;
        pb[hs][j] = (__bf16)p;
      }
      l[hs] = l[hs] * alpha[hs] + lane_group_sum(psum);
      m[hs] = mn;
    }
#pragma unroll
    for (int hs = 0; hs < NS; ++hs) {
      if (grow[hs]) {
#pragma unroll
        for (int c = 0; c < kCt; ++c)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[hs][c][v] *= alpha[hs];
      }
    }
    // O^T += V^T . P^T: the value operand of tokens {4 grp .. +3, 16 + 4 grp .. +3}
    // (the order of this lane's probabilities) at column c*16 + col
    const uint8_t* vb = cur + (4 * grp + (col >> 2)) * kKPitch + 8 * (col & 3);
    __builtin_amdgcn_sched_barrier(0);
    {
      bf16x8_t vbuf[kVD];
#pragma unroll
      for (int c = 0; c < kVD; ++c) vbuf[c] = tr_pair(vb + c * 32, vb + 16 * kKPitch + c * 32);
#pragma unroll
      for (int c = 0; c < kCt; ++c) {
        const bf16x8_t vf = vbuf[c % kVD];
        if (c + kVD < kCt) vbuf[c % kVD] = tr_pair(vb + (c + kVD) * 32, vb + 16 * kKPitch + (c + kVD) * 32);
#pragma unroll
        for (int hs = 0; hs < NS; ++hs) acc[hs][c] = mfma(vf, pb[hs], acc[hs][c]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVD, 0);
#pragma unroll
      for (int c = 0; c < kCt - kVD; ++c) {
        __builtin_amdgcn_sched_group_barrier(0x008, NS, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NS * kVD, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The first step's slot ids, then its loads, go out before the query
  // fragments (a wait for the slot ids would otherwise wait for them too).
  if (nsteps > 0) {
    if (slot_lane) slots[0][lane] = slot_ok(t_begin, slot_raw(t_begin));
    __syncthreads();
    issue(0, 0);
  }
  int nxt = slot_lane && nsteps > 1 ? slot_raw(t_begin + kStep) : -1;
#pragma unroll
  for (int hs = 0; hs < NS; ++hs) {
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(q + ((size_t)b * H + h0 + 16 * hs) * kRowV);
#pragma unroll
    for (int s = 0; s < kKs; ++s) qf[hs][s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + s * 64 + grp * 16));
#pragma unroll
    for (int c = 0; c < kCt; ++c) acc[hs][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m[hs] = -__builtin_inff();
    l[hs] = 0.f;
  }
  if (nsteps > 0) {
    // one step: its loads have landed (every wave waited, then the barrier),
    // the next step's slot ids are published and its loads issued, then the
    // products of this wave's tile run over them
    for (int i = 0; i < nsteps; ++i) {
      // every load of this wave (the builtin form, so that the compiler knows
      // the query fragments and slot ids are in as well)
      __builtin_amdgcn_s_waitcnt(0x70 | 0xF00);   // vmcnt(0)
      if (slot_lane && i + 1 < nsteps) slots[(i + 1) % 3][lane] = slot_ok(t_begin + (i + 1) * kStep, nxt);
      __syncthreads();
      if (i + 1 < nsteps) issue((i + 1) % 3, (i + 1) & 1);
      if (slot_lane && i + 2 < nsteps) nxt = slot_raw(t_begin + (i + 2) * kStep);
      // a token lane past the span's end has nothing to add (a wave-uniform test)
      if (TL == 1 || t_begin + i * kStep + tl * kTile < t_end)
        compute(&slots[i % 3][tl * kTile], &tiles[i & 1][tl * kBuf2]);
    }
  }

  if constexpr (TL == 2) {
    // The second token lane's state goes through LDS (the tile buffers, free
    // once every wave has left the loop) to the first, which merges it.
    static_assert(NH * (kCt * 64 * 16 + 64 * 8) <= 2 * TL * kBuf2, "merge state fits the tile buffers");
    f32x4_t* xo = reinterpret_cast<f32x4_t*>(&tiles[0][0]) + hw * kCt * 64 + lane;
    float2* xml = reinterpret_cast<float2*>(&tiles[0][0] + NH * kCt * 64 * 16) + hw * 64 + lane;
    __syncthreads();
    if (tl == 1) {
#pragma unroll
      for (int c = 0; c < kCt; ++c) xo[c * 64] = acc[0][c];
      *xml = make_float2(m[0], l[0]);
    }
    __syncthreads();
    if (tl == 1) return;
    const float2 o = *xml;
    const float mn = fmaxf(m[0], o.x);
    if (mn != -__builtin_inff()) {
      const float ra = exp2f(m[0] - mn), rb = exp2f(o.x - mn);   // 0 for a lane that saw nothing
      l[0] = l[0] * ra + o.y * rb;
      m[0] = mn;
#pragma unroll
      for (int c = 0; c < kCt; ++c) {
        const f32x4_t x = xo[c * 64];
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[0][c][v] = acc[0][c][v] * ra + x[v] * rb;
      }
    }
  }

  // partials: O^T column c*16 + 4 grp + v of heads h0 + 16 hs
#pragma unroll
  for (int hs = 0; hs < NS; ++hs) {
    const int h = h0 + 16 * hs;
    float* po = part_o + (((size_t)b * nsp + sp) * H + h) * kValV;
#pragma unroll
    for (int c = 0; c < kCt; ++c) *reinterpret_cast<f32x4_t*>(po + c * 16 + 4 * grp) = acc[hs][c];
    if (grp == 0) part_ml[((size_t)b * nsp + sp) * H + h] = make_float2(m[hs], l[hs]);
  }
}

// out[b, h, :] and lse[b, h] from the spans' partials. grid (H, B), 128 threads.
// KG = spans whose loads are in flight together (2 or 4: the power of two that
// covers the spans; 32 beyond 32 spans, whose merge loops over groups).
// One pass: a group's maxima, sums and outputs are loaded together, and the
// running sums are rescaled when a group raises the maximum.
template <int kG>
__global__ void __launch_bounds__(128)
    attn_merge_kernel(const float* __restrict__ part_o, const float2* __restrict__ part_ml, int H, int nsp,
                      float* __restrict__ out, float* __restrict__ lse) {
  const int h = blockIdx.x, b = blockIdx.y;
  float mx = -__builtin_inff(), den = 0.f;
  f32x4_t o = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsp; s0 += kG) {
    // every load is clamped and unguarded, so all of a group's loads issue
    // before the first wait; spans past the end are masked in arithmetic
    f32x4_t v[kG];
    float2 ml[kG];
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const size_t sj = (size_t)b * nsp + min(s0 + j, nsp - 1);
      v[j] = *reinterpret_cast<const f32x4_t*>(part_o + (sj * H + h) * kValV + 4 * threadIdx.x);
      ml[j] = part_ml[sj * H + h];
    }
    float gmx = mx;
#pragma unroll
    for (int j = 0; j < kG; ++j) gmx = fmaxf(gmx, ml[j].x);   // clamped repeats change nothing
    if (gmx == -__builtin_inff()) continue;                  // nothing attended so far
    const float r = exp2f(mx - gmx);                          // 0 while mx is -inf (den, o are 0)
    den *= r;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] *= r;
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const float wgt = (s0 + j < nsp) ? exp2f(ml[j].x - gmx) : 0.f;   // 0 also for a span that saw nothing
      den += wgt * ml[j].y;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += wgt * v[j][e];
    }
    mx = gmx;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] *= inv;
  *reinterpret_cast<f32x4_t*>(out + ((size_t)b * H + h) * kValV + 4 * threadIdx.x) = o;
  if (lse && threadIdx.x == 0)
    lse[(size_t)b * H + h] = den > 0.f ? (mx + log2f(den)) * 0.69314718055994531f : -__builtin_inff();
}

// The merge for 5 to 32 spans: grid (H, B, 4), 128 threads.
// Workgroup z takes the value columns 128 z .. +127 of one (sequence, head);
// thread t the four columns 4 (t % 32) .. +3 of them over the spans
// t / 32, t / 32 + 4, ... (kPer of them, loads all in flight); the four span
// subsets are combined through LDS. Four times the workgroups of the
// one-group form, a quarter of the loads per thread.
template <int kPer>
__global__ void __launch_bounds__(128)
    attn_merge_split_kernel(const float* __restrict__ part_o, const float2* __restrict__ part_ml, int H, int nsp,
                            float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float s_mx[128], s_den[128];
  __shared__ f32x4_t s_o[128];
  const int h = blockIdx.x, b = blockIdx.y, quarter = blockIdx.z;
  const int tid = threadIdx.x, quad = tid & 31, sub = tid >> 5;
  const int c0 = quarter * 128 + 4 * quad;
  f32x4_t v[kPer];
  float2 ml[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {   // clamped and unguarded: every load issues before the first wait
    const size_t sj = (size_t)b * nsp + min(sub + 4 * j, nsp - 1);
    v[j] = *reinterpret_cast<const f32x4_t*>(part_o + (sj * H + h) * kValV + c0);
    ml[j] = part_ml[sj * H + h];
  }
  float mx = -__builtin_inff(), den = 0.f;
  f32x4_t o = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (sub + 4 * j < nsp) mx = fmaxf(mx, ml[j].x);
  if (mx != -__builtin_inff()) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const float wgt = (sub + 4 * j < nsp) ? exp2f(ml[j].x - mx) : 0.f;   // 0 also for a span that saw nothing
      den += wgt * ml[j].y;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += wgt * v[j][e];
    }
  }
  s_mx[tid] = mx;
  s_den[tid] = den;
  s_o[tid] = o;
  __syncthreads();
  if (sub != 0) return;
  float gmx = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < 4; ++u) gmx = fmaxf(gmx, s_mx[quad + 32 * u]);
  float gden = 0.f;
  f32x4_t go = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (gmx != -__builtin_inff()) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float r = exp2f(s_mx[quad + 32 * u] - gmx);   // 0 for a subset that saw nothing
      gden += r * s_den[quad + 32 * u];
      const f32x4_t x = s_o[quad + 32 * u];
#pragma unroll
      for (int e = 0; e < 4; ++e) go[e] += r * x[e];
    }
  }
  const float inv = gden > 0.f ? 1.f / gden : 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) go[e] *= inv;
  *reinterpret_cast<f32x4_t*>(out + ((size_t)b * H + h) * kValV + c0) = go;
  if (lse && quarter == 0 && quad == 0)
    lse[(size_t)b * H + h] = gden > 0.f ? (gmx + log2f(gden)) * 0.69314718055994531f : -__builtin_inff();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The launch's shape: spans per sequence, tokens per span, head groups per
// span, token lanes per workgroup.
struct Plan {
  int nsp, span, hsplit, tl;
};

// Spans of whole 32-token tiles, about 256 workgroups: one span per CU's
// worth of sequences (ceil(256 / B) per sequence), but at least two tiles
// per span, so that few sequences do not end up with one-tile spans whose
// partials cost more than their rows. When spans x sequences leave CUs
// without a workgroup, the heads of a span are split over up to 4
// workgroups (a divisor of H / 16), which read the span's rows from one
// XCD's L2. Then two token lanes where a workgroup has room for them: eight
// waves of 16 heads become two head groups of four waves with two lanes each
// (as many workgroups, half the spans and partials), and four waves or fewer
// take a second lane: with a workgroup per CU already, half the spans and
// twice the head groups (as many workgroups and waves, half the partials),
// else twice the waves. Measured at 128 heads x 2048 rows (span + merge,
// rocprofv3): 32 sequences 39.8 + 12.2 -> 41.0 + 7.7 us, 16 sequences 29.0 +
// 15.6 -> 30.8 + 6.8 us; one sequence 23.8 -> 22.9 us; four 34.4 us one lane,
// 30.8 with 2 head groups x 2 lanes, 28.5 with 4 x 2 (16 spans).
Plan plan_for(int B, int H, int k) {
  const int tiles = (k + kTile - 1) / kTile, groups = H / 16;
  int nsp = std::min((256 + B - 1) / B, std::max(1, tiles / 2));
  nsp = std::max(1, std::min(nsp, tiles));
  int per = (tiles + nsp - 1) / nsp;
  nsp = (tiles + per - 1) / per;
  int hsplit = 1;
  const int want = std::max(1, 256 / (B * nsp));
  for (int d = std::min(4, groups); d > 1; --d)
    if (groups % d == 0 && d <= want) {
      hsplit = d;
      break;
    }
  int tl = 1;
  const int nh = groups / hsplit;
  if (per >= 2 && nh == kMaxWaves) {
    tl = 2;
    hsplit *= 2;
    nsp = (nsp + 1) / 2;
  } else if (per >= 2 && 2 * nh <= kMaxWaves) {
    tl = 2;
    if (B * nsp * hsplit >= 256) {
      nsp = (nsp + 1) / 2;
      if (nh % 2 == 0) hsplit *= 2;   // as many workgroups as before, as many waves each
    }
  }
  if (tl == 2) {
    // whole steps of two tiles per span
    per = (tiles + nsp - 1) / nsp;
    per += per & 1;
    nsp = (tiles + per - 1) / per;
  }
  return Plan{nsp, per * kTile, hsplit, tl};
}

}  // namespace

extern "C" size_t ech_sparse_attn_ws_bytes(int B, int H, int k) {
  if (B < 1 || H < 16 || H > 16 * kMaxWaves || H % 16 || k < 1 || k > 65536) return 0;
  const size_t nsp = (size_t)plan_for(B, H, k).nsp;
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
  const Plan pl = plan_for(B, H, k);
  const int nsp = pl.nsp, span = pl.span, hsplit = pl.hsplit;
  if (H % (16 * hsplit) || (H / 16 / hsplit) * pl.tl > kMaxWaves) return ECH_EINVAL;
  const size_t o = (size_t)nsp * B * H * kValV * sizeof(float);
  float* part_o = static_cast<float*>(ws);
  float2* part_ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + ((o + 255) & ~(size_t)255));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const float scale2 = sm_scale * 1.4426950408889634f;
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* cc = static_cast<const uint4*>(dev_cache);
  const dim3 grid(nsp * hsplit, B);
  switch ((H / 16 / hsplit) * 16 + pl.tl) {
#define ECH_ATTN_CASE(W, T)                                                                                     \
  case W * 16 + T:                                                                                              \
    hipLaunchKernelGGL((attn_span_kernel<W, T>), grid, dim3(64 * W * T), 0, s, qq, cc, C, sel_slot, H, k, span, \
                       scale2, part_o, part_ml);                                                                \
    break;
    ECH_ATTN_CASE(1, 1)
    ECH_ATTN_CASE(2, 1)
    ECH_ATTN_CASE(3, 1)
    ECH_ATTN_CASE(4, 1)
    ECH_ATTN_CASE(5, 1)
    ECH_ATTN_CASE(6, 1)
    ECH_ATTN_CASE(7, 1)
    ECH_ATTN_CASE(8, 1)
    ECH_ATTN_CASE(1, 2)
    ECH_ATTN_CASE(2, 2)
    ECH_ATTN_CASE(3, 2)
    ECH_ATTN_CASE(4, 2)
#undef ECH_ATTN_CASE
    default:
      return ECH_EINVAL;
  }
  ECH_LAUNCH_CHECK();
  // the merge loads up to kG spans at once: the power of two that covers nsp
  // (clamped repeats past nsp would cost requests), at most 32
  const dim3 mgrid(H, B), mblock(kValV / 4);
  if (nsp <= 2)
    hipLaunchKernelGGL(attn_merge_kernel<2>, mgrid, mblock, 0, s, part_o, part_ml, H, nsp, out, lse);
  else if (nsp <= 4)
    hipLaunchKernelGGL(attn_merge_kernel<4>, mgrid, mblock, 0, s, part_o, part_ml, H, nsp, out, lse);
  else if (nsp <= 8)
    hipLaunchKernelGGL(attn_merge_split_kernel<2>, dim3(H, B, 4), mblock, 0, s, part_o, part_ml, H, nsp, out, lse);
  else if (nsp <= 16)
    hipLaunchKernelGGL(attn_merge_split_kernel<4>, dim3(H, B, 4), mblock, 0, s, part_o, part_ml, H, nsp, out, lse);
  else if (nsp <= 32)
    hipLaunchKernelGGL(attn_merge_split_kernel<8>, dim3(H, B, 4), mblock, 0, s, part_o, part_ml, H, nsp, out, lse);
  else
    hipLaunchKernelGGL(attn_merge_kernel<32>, mgrid, mblock, 0, s, part_o, part_ml, H, nsp, out, lse);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}
