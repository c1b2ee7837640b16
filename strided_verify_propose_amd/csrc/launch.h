// Host-side launch interface between the C ABI (isd_api.cpp) and the kernels (*.hip).
// Arguments have already been validated (isd_validate.cpp) when these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "launch_types.h"

namespace isd {

hipError_t launch_attention(const AttnLaunch& a, hipStream_t s);
hipError_t launch_kv_pages(const KvPagesLaunch& c, hipStream_t s);
hipError_t launch_kv_sweep(const KvSweepLaunch& c, hipStream_t s);
hipError_t launch_verify(const VerifyLaunch& v, hipStream_t s);        // stats + tail
hipError_t launch_verify_stats(const VerifyLaunch& v, hipStream_t s);  // the stats pass alone
hipError_t launch_verify_tail(const VerifyLaunch& v, hipStream_t s);   // walk, residual, draws
hipError_t launch_lm_head(const LmhLaunch& p, hipStream_t s);        // logits (+ mini-chunk records)
hipError_t launch_lm_head_merge(const LmhLaunch& p, hipStream_t s);  // records -> chunk records
hipError_t launch_commit(const CommitLaunch& c, hipStream_t s);
// Large-tile partial sums, their ordered sum, and the delta on gated rows.
hipError_t launch_proj_big(const ProjLaunch& p, bool packed, hipStream_t s);
hipError_t launch_proj(const ProjLaunch& p, hipStream_t s);
hipError_t launch_lora(const ProjLaunch& p, hipStream_t s);  // the second kernel alone
hipError_t launch_proj_reduce(const ProjLaunch& p, hipStream_t s);  // sum of the K parts
hipError_t launch_proj_packed(const ProjLaunch& p, hipStream_t s);
// Pack [W^T; A^T] (Nout + r rows of K) into fragment order and copy B^T after it.
// kn: w [K, Nout], a [K, r], b [r, Nout] instead of w [Nout, K], a [r, K], b [Nout, r]
hipError_t launch_pack_proj(const uint16_t* w, const uint16_t* a, const uint16_t* b, uint16_t* packed,
                            int K, int Nout, int r, bool kn, hipStream_t s);

}  // namespace isd
