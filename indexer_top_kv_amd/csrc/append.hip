// Appending each sequence's newly decoded token (growing contexts). The host
// copy holds every KV row and is never written back on eviction (ECHO
// explainer, "One layer, one step"), so a new row crosses PCIe once, when it
// is produced: the kernel stores it straight into the pinned host pool
// (zero-copy writes), puts the token's indexer key (and fp8 scale) into the
// key cache and grows the sequence's length. The token is not resident: if a
// later step selects it, that step's recall brings it in.
#include "common.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// grid (B), 64 threads: sequence b's token tok0[b] + len[b].
__global__ void __launch_bounds__(64)
    kv_append_kernel(uint4* __restrict__ host_pool, int64_t P, int row16, uint8_t* __restrict__ kcache, int key16,
                     float* __restrict__ kscale, int32_t* __restrict__ tok2slot,
                     const int64_t* __restrict__ seq_tok0, int32_t* __restrict__ seq_len,
                     const int32_t* __restrict__ seq_cap, const uint4* __restrict__ new_rows,
                     const uint4* __restrict__ new_keys, const float* __restrict__ new_scales,
                     int32_t* __restrict__ ctr) {
  const int b = blockIdx.x;
  const int len = seq_len[b];
  const int64_t g = seq_tok0[b] + len;
  if (len < 0 || len >= seq_cap[b] || g < 0 || g >= P) {   // full (or a bad layout): nothing written
    if (threadIdx.x == 0) atomicOr(&ctr[ECH_CTR_STATUS], ECH_ST_FULL);
    return;
  }
  for (int i = threadIdx.x; i < row16; i += blockDim.x)
    host_pool[g * row16 + i] = new_rows[(int64_t)b * row16 + i];
  uint4* kd = reinterpret_cast<uint4*>(kcache);
  for (int i = threadIdx.x; i < key16; i += blockDim.x) kd[g * key16 + i] = new_keys[(int64_t)b * key16 + i];
  __syncthreads();                                 // every lane has read seq_len[b]
  if (threadIdx.x == 0) {
    if (kscale) kscale[g] = new_scales[b];
    tok2slot[g] = -1;
    seq_len[b] = len + 1;
  }
}

}  // namespace

extern "C" int ech_kv_append(void* host_pool, int64_t P, int64_t row_bytes, void* kcache, int kdtype,
                             float* kscale, int32_t* tok2slot, const int64_t* seq_tok0, int32_t* seq_len,
                             const int32_t* seq_cap, int B, const void* new_rows, const void* new_keys,
                             const float* new_scales, int32_t* ctr, void* stream) {
  if (!host_pool || !kcache || !tok2slot || !seq_tok0 || !seq_len || !seq_cap || !new_rows || !new_keys || !ctr)
    return ECH_EINVAL;
  if (B < 1 || B > 65535 || P < 1 || row_bytes < 16 || row_bytes % 16) return ECH_EINVAL;
  if (kdtype != ECH_KEY_FP8 && kdtype != ECH_KEY_BF16) return ECH_EUNSUPPORTED;
  if (kdtype == ECH_KEY_FP8 && (!kscale || !new_scales)) return ECH_EINVAL;
  if (!aligned16(host_pool) || !aligned16(kcache) || !aligned16(new_rows) || !aligned16(new_keys))
    return ECH_EINVAL;
  void* dptr = nullptr;
  if (hipHostGetDevicePointer(&dptr, host_pool, 0) != hipSuccess || !dptr) {
    (void)hipGetLastError();
    return ECH_EINVAL;
  }
  const int key_bytes = kdtype == ECH_KEY_FP8 ? 128 : 256;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(kv_append_kernel, dim3(B), dim3(64), 0, s, static_cast<uint4*>(dptr), P, (int)(row_bytes / 16),
                     static_cast<uint8_t*>(kcache), key_bytes / 16, kdtype == ECH_KEY_FP8 ? kscale : nullptr,
                     tok2slot, seq_tok0, seq_len, seq_cap, static_cast<const uint4*>(new_rows),
                     static_cast<const uint4*>(new_keys), new_scales, ctr);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}
