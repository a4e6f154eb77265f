// Library-internal: the top-k selection over band lists that a scoring
// kernel wrote (topk.hip), launched by the fused scores entry points
// (fused.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ech {

// Rows r < R: per chunk c of `chunk_tok` tokens (c < ceil(len_r / chunk_tok)
// <= cpr), meta[r * cpr + c] = (n, floor): the chunk's tokens in bins >= floor
// (bins of shifted_bin_one against list_theta[r]), n of them, are
// pool[(r * cpr + c) * slice + i], i < n, (score bits, token), in token
// order; floor 256 lists nothing. A row whose theta_in differs from
// list_theta (bit for bit) is selected from the whole row. Writes idx [R, k],
// kth and theta_out as ech_topk. Arguments are checked by the caller;
// returns ECH_OK or ECH_EHIP.
int topk_lists_launch(const float* logits, int64_t ld, const int32_t* row_len, int R, int max_len, int k,
                      const float* theta_in, float* theta_out, int32_t* idx, float* kth, const int2* meta,
                      const int2* pool, const float* list_theta, int cpr, int slice, int chunk_tok,
                      hipStream_t stream);

// Most chunks per row, and the largest k, topk_lists_launch handles.
constexpr int kListMaxChunks = 4096;
constexpr int kListMaxK = 4096;

}  // namespace ech
