// The commit step of the decoding loop: what one ISD step keeps, per request.
//
// The two-state chain behind tokens per forward (「I-DLM – introspektive Diffusion Language
// Models」 "Speedup Factor Explorer"; the step that cannot verify, 「I-DLM – introspektive
// Diffusion Language Models」 "Inference & ISD"): a hot request verified N-1 drafts and
// keeps the accepted ones plus the next token; a cold one (no valid drafts) keeps one
// exact token.  The block's first slot held the last committed token c at position
// ctx_len, so the cache grows by the number kept and the next token becomes the new c.
// The next step has drafts -- the samples of the [MASK] rows -- only if this step was
// cold or accepted every draft; otherwise they were proposed after a rejected token.
#include "device.h"
#include "launch.h"

namespace isd {
namespace {

__global__ __launch_bounds__(256) void commit_kernel(const CommitLaunch c) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= c.B) return;
  const int N = c.N, nd = N - 1;
  int32_t* d = c.draft_ids + (size_t)b * nd;
  const bool cold = nd > 0 && d[0] < 0;
  const int n = cold ? 0 : min(max(c.n_accept[b], 0), nd);
  if (c.tokens) {
    int32_t* t = c.tokens + (size_t)b * N;
    for (int i = 0; i < N; ++i) t[i] = i < n ? d[i] : (i == n ? c.next_token[b] : -1);
  }
  if (c.counts) c.counts[b] = n + 1;
  c.ctx_lens[b] += n + 1;
  const bool hot_next = cold || n == nd;
  for (int i = 0; i < nd; ++i) d[i] = hot_next ? c.sampled_ids[(size_t)b * N + 1 + i] : -1;
}

}  // namespace

hipError_t launch_commit(const CommitLaunch& c, hipStream_t s) {
  commit_kernel<<<(c.B + 255) / 256, 256, 0, s>>>(c);
  return hipGetLastError();
}

}  // namespace isd
