// Exact top-k per score row on gfx950.
//
// ECHO explainer, "Prefill: one-round histogram": a single 256-bin histogram
// pass keyed by the high byte of the score minus the predicted threshold
// theta; the selection must be exact (the explainer's opening summary). The k-th element (s*, t*) of the order
// (score descending, token ascending) defines the set exactly:
//     t selected  <=>  s_t > s*  or  (s_t == s* and t among the first
//                      need_eq tokens with score s*)
// so the kernels find s* and need_eq, then compact in ascending t.
//
//   T1 hist     grid (chunks, R): LDS histogram of bin(t) = high byte of
//               the order key of fp16(fl32(s_t - theta)) per 4096-token chunk.
//               Every step is monotone in s, so higher bins hold strictly
//               larger scores.
//   T2 rowsel   grid (R): sum the chunk histograms, boundary bin b* where the
//               count from the top reaches k, need = k - count above b*.
//   T3 gather   grid (chunks, R): count tokens above b* per chunk; append the
//               b* tokens (score, t) to a per-row candidate list.
//   T4 resolve  grid (R): radix-select need-th largest score among the
//               candidates in LDS (4 rounds of 8 bits of ord(s)); per-chunk
//               counts of ">" and "==" tokens give output offsets. If the
//               boundary bin overflowed the list (no or poor theta), the same
//               radix rounds run over the whole row instead. Writes kth and
//               the EMA update of theta.
//   T5 compact  grid (chunks, R): each chunk writes its selected tokens in
//               ascending order at its offset; rows shorter than k are padded
//               with -1.
// A good theta puts only a few hundred tokens in b* (bins are logarithmic
// around the threshold), so T4 works in LDS and the row is read three times.

#include <algorithm>

#include "common.hpp"

namespace {

constexpr int kChunk = 4096;        // tokens per chunk (T1, T3, T5)
constexpr int kVec = kChunk / (4 * 256);   // float4 loads per thread
constexpr int kT = 256;             // threads for chunk kernels
constexpr int kMaxK = 4096;
constexpr int kMaxChunks = 1024;    // max_len <= 4M

enum RowMode : int { kNormal = 0, kAll = 1, kEmpty = 2 };

struct RowState {
  int mode;
  int bstar;
  int need;
  int cand;      // candidates appended (may exceed the list capacity)
  float spred;   // scores > spred are selected (-inf in kAll mode)
  int pad[3];
};

struct Ws {
  RowState* rs;
  int* hist;     // [R][nch][256]
  int* above;    // [R][nch]
  int* off;      // [R][nch]
  int* take;     // [R][nch]
  int2* cand;    // [R][cap]
  int cap;
  int nch;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int cand_cap(int R) { return R <= 256 ? 16384 : 4096; }

size_t layout(int R, int max_len, Ws* w, char* base) {
  const int nch = std::max(1, (max_len + kChunk - 1) / kChunk);
  const int cap = cand_cap(R);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  size_t o_rs = take(sizeof(RowState) * R);
  size_t o_hist = take(sizeof(int) * (size_t)R * nch * 256);
  size_t o_above = take(sizeof(int) * (size_t)R * nch);
  size_t o_off = take(sizeof(int) * (size_t)R * nch);
  size_t o_take = take(sizeof(int) * (size_t)R * nch);
  size_t o_cand = take(sizeof(int2) * (size_t)R * cap);
  if (w && base) {
    w->rs = reinterpret_cast<RowState*>(base + o_rs);
    w->hist = reinterpret_cast<int*>(base + o_hist);
    w->above = reinterpret_cast<int*>(base + o_above);
    w->off = reinterpret_cast<int*>(base + o_off);
    w->take = reinterpret_cast<int*>(base + o_take);
    w->cand = reinterpret_cast<int2*>(base + o_cand);
    w->cap = cap;
    w->nch = nch;
  }
  return o;
}

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

// The 256 bins are the high byte of the order key of fp16(d): sign, 5
// exponent bits and 2 mantissa bits, i.e. four bins per binade of |d| (the
// high byte of the fp32 key would give one bin per two binades). fp32 -> fp16
// rounding is monotone, so the binning stays monotone in s; overflow goes to
// the infinities, the outermost bins. Finite negative d never reaches bin 0
// (its order key is at least 0x0400), so bin 0 is free for the lumped scores.
__device__ __forceinline__ uint32_t bin16(float d) {
  const _Float16 h = (_Float16)d;
  uint32_t u = __builtin_bit_cast(uint16_t, h);
  if ((u & 0x7fffu) == 0u) u = 0u;               // -0 -> +0
  const uint32_t key = (u & 0x8000u) ? (~u & 0xffffu) : (u | 0x8000u);
  return key >> 8;
}

__device__ __forceinline__ uint32_t shifted_bin(float x, const Shift& sh) {
  if (!sh.on) return bin16(x);
  const float d = x - sh.th;
  return d < sh.cut ? 0u : bin16(d);
}

__device__ __forceinline__ float row_theta(const float* th, int r) {
  return th ? th[r] : __builtin_nanf("");
}

// ------------------------------------------------------------------ T1
// Load a chunk's 16 scores per thread (4 float4, issued before any use);
// element j*4 + e of thread tid is token lo + 4*(j*256 + tid) + e.
__device__ __forceinline__ void load_chunk(const float* row, int lo, int hi, float4 (&v)[kVec]) {
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int t = lo + 4 * (j * kT + (int)threadIdx.x);
    if (t + 3 < hi) {
      // nontemporal: each load instruction covers a contiguous 1 KiB, the
      // pattern where the hint raises the stream rate on MI355X
      typedef float f4v __attribute__((ext_vector_type(4)));
      const f4v x = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(row + t));
      v[j] = make_float4(x.x, x.y, x.z, x.w);
    } else {
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < hi) v[j].x = row[t];
      if (t + 1 < hi) v[j].y = row[t + 1];
      if (t + 2 < hi) v[j].z = row[t + 2];
    }
  }
}

__device__ __forceinline__ float f4(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

__global__ __launch_bounds__(kT) void topk_hist_kernel(const float* __restrict__ logits, int64_t ld,
                                                       const int32_t* __restrict__ lens, int k,
                                                       const float* __restrict__ theta, Ws ws) {
  const int r = blockIdx.y, c = blockIdx.x;
  const int len = lens[r];
  const int lo = c * kChunk;
  if (len <= k || lo >= len) return;
  const int hi = min(lo + kChunk, len);
  __shared__ int h[256];
  h[threadIdx.x] = 0;
  const Shift sh = make_shift(row_theta(theta, r));
  float4 v[kVec];
  load_chunk(logits + (size_t)r * ld, lo, hi, v);
  __syncthreads();
  int lumped = 0;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int t = lo + 4 * (j * kT + (int)threadIdx.x);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = f4(v[j], e);
      const bool ok = t + e < hi;
      const float d = sh.on ? x - sh.th : x;
      const bool lump = ok && d < sh.cut;
      lumped += lump;
      ech::lds_hist_add(h, bin16(d), ok && !lump);
    }
  }
  lumped = ech::wave_sum(lumped);
  if (ech::lane_id() == 0 && lumped) atomicAdd(&h[0], lumped);
  __syncthreads();
  ws.hist[((size_t)r * ws.nch + c) * 256 + threadIdx.x] = h[threadIdx.x];
}

// ------------------------------------------------------------------ T2
// NT threads (1024 for a few long rows, 256 for many rows): thread
// (part, b) sums bin (255 - b) over the chunks c = part, part + NT/256, ...,
// eight independent loads in flight (a loop with one load per iteration
// waits a full memory round trip per chunk).
template <int NT>
__global__ __launch_bounds__(NT) void topk_rowsel_kernel(const int32_t* __restrict__ lens, int k, Ws ws) {
  constexpr int kParts = NT / 256;
  const int r = blockIdx.x;
  const int len = lens[r];
  RowState& st = ws.rs[r];
  if (len <= k) {
    if (threadIdx.x == 0) {
      st.mode = len == 0 ? kEmpty : kAll;
      st.bstar = 0;
      st.need = 0;
      st.cand = 0;
    }
    return;
  }
  const int nch = (len + kChunk - 1) / kChunk;
  __shared__ int part_sum[kParts][256];
  __shared__ int scratch[NT / 64];
  const int b = threadIdx.x & 255, part = threadIdx.x >> 8;
  const int bin = 255 - b;
  const int* h = ws.hist + (size_t)r * ws.nch * 256 + bin;
  int acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int c = part;
  for (; c + 7 * kParts < nch; c += 8 * kParts) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += h[(size_t)(c + kParts * u) * 256];
  }
  for (; c < nch; c += kParts) acc[0] += h[(size_t)c * 256];
  part_sum[part][b] = acc[0] + acc[1] + acc[2] + acc[3] + acc[4] + acc[5] + acc[6] + acc[7];
  __syncthreads();
  // threads 0..255 hold bins 255..0 in order; the rest add zeros after them
  int cnt = 0;
  if (threadIdx.x < 256) {
#pragma unroll
    for (int pp = 0; pp < kParts; ++pp) cnt += part_sum[pp][b];
  }
  int tot;
  const int above = ech::block_excl_scan<NT>(cnt, scratch, &tot);
  if (threadIdx.x < 256 && above < k && above + cnt >= k) {
    st.mode = kNormal;
    st.bstar = bin;
    st.need = k - above;
    st.cand = 0;
  }
}

// ------------------------------------------------------------------ T3
__global__ __launch_bounds__(kT) void topk_gather_kernel(const float* __restrict__ logits, int64_t ld,
                                                         const int32_t* __restrict__ lens,
                                                         const float* __restrict__ theta, Ws ws) {
  const int r = blockIdx.y, c = blockIdx.x;
  const int len = lens[r];
  const int lo = c * kChunk;
  if (lo >= len) return;
  const int hi = min(lo + kChunk, len);
  // scores first, so their latency overlaps that of the row state
  float4 v[kVec];
  load_chunk(logits + (size_t)r * ld, lo, hi, v);
  const RowState st = ws.rs[r];
  if (st.mode != kNormal) return;
  const Shift sh = make_shift(row_theta(theta, r));
  const uint32_t bstar = (uint32_t)st.bstar;
  int2* cand = ws.cand + (size_t)r * ws.cap;
  int* cnt = &ws.rs[r].cand;
  const int lane = ech::lane_id();
  __shared__ int scratch[kT / 64];
  int above = 0;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int t0 = lo + 4 * (j * kT + (int)threadIdx.x);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = t0 + e;
      const bool ok = t < hi;
      const float x = f4(v[j], e);
      const uint32_t b = shifted_bin(x, sh);
      above += (ok && b > bstar) ? 1 : 0;
      const bool is_c = ok && b == bstar;
      const uint64_t m = __ballot(is_c);
      if (m) {
        int base = 0;
        const int leader = __ffsll((unsigned long long)m) - 1;
        if (lane == leader) base = atomicAdd(cnt, __popcll(m));
        base = __shfl(base, leader, 64);
        if (is_c) {
          const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
          if (pos < ws.cap) cand[pos] = make_int2(__float_as_int(x), t);
        }
      }
    }
  }
  const int tot = ech::block_sum<kT>(above, scratch);
  if (threadIdx.x == 0) ws.above[(size_t)r * ws.nch + c] = tot;
}

// ------------------------------------------------------------------ T4
// fn(t, x) for every score of a row, NT threads, four float4 loads in flight
// per thread (a loop with one scalar load per iteration waits a full memory
// round trip each time). Rows are 16-byte aligned (ld % 4 == 0).
template <int NT, typename Fn>
__device__ __forceinline__ void for_each_score(const float* __restrict__ row, int len, Fn fn) {
  constexpr int kU = 4;
  for (int b0 = 0; b0 < len; b0 += 4 * NT * kU) {
    float4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int t = b0 + 4 * (u * NT + (int)threadIdx.x);
      if (t + 3 < len) {
        v[u] = *reinterpret_cast<const float4*>(row + t);
      } else {
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < len) v[u].x = row[t];
        if (t + 1 < len) v[u].y = row[t + 1];
        if (t + 2 < len) v[u].z = row[t + 2];
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int t = b0 + 4 * (u * NT + (int)threadIdx.x);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t + e < len) fn(t + e, f4(v[u], e));
    }
  }
}

// Radix-select helpers over a key set; `hist` is 256 ints of LDS.
// Finds the digit d (bits [shift, shift+8) of ord) at which the count from
// the top reaches `need`; updates need to the rank within that digit.
__device__ __forceinline__ void pick_digit(int* hist, int* sh, int need, int* out_digit, int* out_need) {
  // thread i < 256 owns digit 255 - i
  int cnt = 0, above = 0, tot = 0;
  if (threadIdx.x < 256) cnt = hist[255 - threadIdx.x];
  // block-wide exclusive scan over the first 256 threads (4 waves)
  const int lane = ech::lane_id(), wave = threadIdx.x / 64;
  int incl = ech::wave_incl_scan(cnt);
  if (threadIdx.x < 256 && lane == 63) sh[wave] = incl;
  __syncthreads();
  if (threadIdx.x < 256) {
    int wb = 0;
    for (int i = 0; i < wave; ++i) wb += sh[i];
    above = wb + incl - cnt;
    if (above < need && above + cnt >= need) {
      *out_digit = 255 - threadIdx.x;
      *out_need = need - above;
    }
  }
  (void)tot;
  __syncthreads();
}

template <int NT>
__global__ __launch_bounds__(NT) void topk_resolve_kernel(const float* __restrict__ logits, int64_t ld,
                                                           const int32_t* __restrict__ lens, int k,
                                                           const float* __restrict__ theta_in,
                                                           float* __restrict__ theta_out, float* __restrict__ kth,
                                                           Ws ws) {
  extern __shared__ int2 cl[];                     // candidate list [cap]
  __shared__ int hist[256];
  __shared__ int sh[16];
  __shared__ int gt_c[kMaxChunks];
  __shared__ int eq_c[kMaxChunks];
  __shared__ int s_digit, s_need;
  __shared__ float s_min;

  const int r = blockIdx.x;
  const int len = lens[r];
  RowState& st = ws.rs[r];
  const int mode = st.mode;
  const float th_in = row_theta(theta_in, r);
  const float* row = logits + (size_t)r * ld;
  const int nch = (len + kChunk - 1) / kChunk;

  if (mode == kEmpty) {
    if (threadIdx.x == 0) {
      kth[r] = __builtin_nanf("");
      if (theta_out) theta_out[r] = th_in;
    }
    return;
  }
  for (int c = threadIdx.x; c < nch; c += NT) {
    gt_c[c] = 0;
    eq_c[c] = 0;
  }
  float sstar, spred;
  int need_eq;
  if (mode == kAll) {
    // every visible token is selected; kth is the row minimum
    float m = __builtin_inff();
    for_each_score<NT>(row, len, [&](int, float x) { m = fminf(m, x); });
    for (int d = 32; d > 0; d >>= 1) m = fminf(m, __shfl_xor(m, d, 64));
    float* wmin = reinterpret_cast<float*>(hist);
    if (ech::lane_id() == 0) wmin[threadIdx.x / 64] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      float mm = __builtin_inff();
      for (int i = 0; i < NT / 64; ++i) mm = fminf(mm, wmin[i]);
      s_min = mm;
    }
    __syncthreads();
    sstar = s_min;
    spred = -__builtin_inff();
    need_eq = 0;
    for (int c = threadIdx.x; c < nch; c += NT) gt_c[c] = min(kChunk, len - c * kChunk);
    __syncthreads();
  } else {
    const int cnt = st.cand;
    int need = st.need;
    uint32_t prefix = 0, mask = 0;
    const bool in_lds = cnt <= ws.cap;
    const Shift shf = make_shift(th_in);
    const uint32_t bstar = (uint32_t)st.bstar;
    if (in_lds) {
      const int2* src = ws.cand + (size_t)r * ws.cap;
      for (int i = threadIdx.x; i < cnt; i += NT) cl[i] = src[i];
    }
    __syncthreads();
#pragma unroll 1
    for (int round = 0; round < 4; ++round) {
      const int shift = 24 - 8 * round;
      for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0;
      __syncthreads();
      if (in_lds) {
        for (int i0 = 0; i0 < cnt; i0 += NT) {
          const int i = i0 + threadIdx.x;
          uint32_t key = 0;
          bool act = false;
          if (i < cnt) {
            key = ech::ord_key(__int_as_float(cl[i].x));
            act = (key & mask) == prefix;
          }
          ech::lds_hist_add(hist, (key >> shift) & 255u, act);
        }
      } else {
        for_each_score<NT>(row, len, [&](int, float x) {
          const uint32_t key = ech::ord_key(x);
          const bool act = shifted_bin(x, shf) == bstar && (key & mask) == prefix;
          ech::lds_hist_add(hist, (key >> shift) & 255u, act);
        });
      }
      __syncthreads();
      pick_digit(hist, sh, need, &s_digit, &s_need);
      prefix |= (uint32_t)s_digit << shift;
      mask |= 255u << shift;
      need = s_need;
      __syncthreads();
    }
    sstar = ech::ord_to_float(prefix);
    spred = sstar;
    need_eq = need;
    // per-chunk counts of tokens strictly above s* and equal to s*
    if (in_lds) {
      for (int c = threadIdx.x; c < nch; c += NT) gt_c[c] = ws.above[(size_t)r * ws.nch + c];
      __syncthreads();
      for (int i = threadIdx.x; i < cnt; i += NT) {
        const float x = __int_as_float(cl[i].x);
        const int c = cl[i].y / kChunk;
        if (x > sstar) atomicAdd(&gt_c[c], 1);
        else if (x == sstar) atomicAdd(&eq_c[c], 1);
      }
    } else {
      for_each_score<NT>(row, len, [&](int t, float x) {
        if (x > sstar) atomicAdd(&gt_c[t / kChunk], 1);
        else if (x == sstar) atomicAdd(&eq_c[t / kChunk], 1);
      });
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int run = 0, eq_before = 0;
    int* off = ws.off + (size_t)r * ws.nch;
    int* tk = ws.take + (size_t)r * ws.nch;
    for (int c = 0; c < nch; ++c) {
      const int tkc = max(0, min(eq_c[c], need_eq - eq_before));
      off[c] = run;
      tk[c] = tkc;
      run += gt_c[c] + tkc;
      eq_before += eq_c[c];
    }
    st.spred = spred;
    kth[r] = sstar;
    if (theta_out) theta_out[r] = (th_in == th_in) ? (sstar + th_in) * 0.5f : sstar;
  }
}

// ------------------------------------------------------------------ T5
__global__ __launch_bounds__(kT) void topk_compact_kernel(const float* __restrict__ logits, int64_t ld,
                                                          const int32_t* __restrict__ lens, int k,
                                                          int32_t* __restrict__ idx, Ws ws) {
  const int r = blockIdx.y, c = blockIdx.x;
  const int len = lens[r];
  int32_t* orow = idx + (size_t)r * k;
  if (c == 0) {
    for (int j = min(k, len) + threadIdx.x; j < k; j += kT) orow[j] = -1;
  }
  const int lo = c * kChunk;
  if (lo >= len) return;
  const int hi = min(lo + kChunk, len);
  float4 v[kVec];
  load_chunk(logits + (size_t)r * ld, lo, hi, v);   // before the row state: the latencies overlap
  const RowState st = ws.rs[r];
  if (st.mode == kEmpty) return;
  const float sp = st.spred;
  const int base = ws.off[(size_t)r * ws.nch + c];
  const int te = ws.take[(size_t)r * ws.nch + c];
  __shared__ int scratch[kT / 64];
  int gt_run = 0, eq_run = 0;   // block-uniform running counts
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int t = lo + 4 * (j * kT + (int)threadIdx.x);
    int ngt = 0, neq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = f4(v[j], e);
      const bool ok = t + e < hi;
      ngt += (ok && x > sp) ? 1 : 0;
      neq += (ok && x == sp) ? 1 : 0;
    }
    int tot;
    const int pre = ech::block_excl_scan<kT>(ngt | (neq << 16), scratch, &tot);
    int gt_b = gt_run + (pre & 0xffff);
    int eq_b = eq_run + (pre >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = f4(v[j], e);
      if (t + e >= hi) continue;
      const bool gt = x > sp, eq = x == sp;
      const bool sel = gt || (eq && eq_b < te);
      const int pos = base + gt_b + min(eq_b, te);
      if (sel && pos < k) orow[pos] = t + e;
      gt_b += gt;
      eq_b += eq;
    }
    gt_run += tot & 0xffff;
    eq_run += tot >> 16;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" size_t ech_topk_ws_bytes(int R, int max_len, int k) {
  (void)k;
  if (R < 1 || max_len < 0) return 0;
  return layout(R, max_len, nullptr, nullptr);
}

extern "C" int ech_topk(const float* logits, int64_t ld, const int32_t* row_len, int R, int max_len, int k,
                        const float* theta_in, float* theta_out, int32_t* idx, float* kth, void* ws,
                        size_t ws_bytes, void* stream) {
  if (!logits || !row_len || !idx || !kth || !ws) return ECH_EINVAL;
  if (R < 1 || R > 65535 || k < 1 || k > kMaxK || max_len < 0 || ld < max_len) return ECH_EINVAL;
  if ((int64_t)max_len > (int64_t)kChunk * kMaxChunks) return ECH_EINVAL;
  if (ld % 4 != 0 || !aligned16(logits) || (reinterpret_cast<uintptr_t>(ws) & 255u)) return ECH_EINVAL;
  if (ws_bytes < ech_topk_ws_bytes(R, max_len, k)) return ECH_EINVAL;
  Ws w;
  layout(R, max_len, &w, static_cast<char*>(ws));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 gch(w.nch, R);
  hipLaunchKernelGGL(topk_hist_kernel, gch, dim3(kT), 0, s, logits, ld, row_len, k, theta_in, w);
  ECH_LAUNCH_CHECK();
  // A few long rows (decode) get 1024 threads per row; many rows (a prefill
  // block) get 256, so the per-row kernels fit beside other work on a CU.
  const bool wide = R <= 256;
  if (wide)
    hipLaunchKernelGGL(topk_rowsel_kernel<1024>, dim3(R), dim3(1024), 0, s, row_len, k, w);
  else
    hipLaunchKernelGGL(topk_rowsel_kernel<256>, dim3(R), dim3(256), 0, s, row_len, k, w);
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(topk_gather_kernel, gch, dim3(kT), 0, s, logits, ld, row_len, theta_in, w);
  ECH_LAUNCH_CHECK();
  if (wide)
    hipLaunchKernelGGL(topk_resolve_kernel<1024>, dim3(R), dim3(1024), sizeof(int2) * w.cap, s, logits, ld,
                       row_len, k, theta_in, theta_out, kth, w);
  else
    hipLaunchKernelGGL(topk_resolve_kernel<256>, dim3(R), dim3(256), sizeof(int2) * w.cap, s, logits, ld, row_len,
                       k, theta_in, theta_out, kth, w);
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(topk_compact_kernel, gch, dim3(kT), 0, s, logits, ld, row_len, k, idx, w);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}
