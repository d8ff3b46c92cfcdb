// Internal entries shared by the C ABI's translation units: the argument
// checks of the backward passes (everything but the workspace) and the
// recomputing backward pass of dn_chunk_bwd with a caller-chosen workspace.
#pragma once

#include "dn.h"

namespace dn {

dn_status bwd_check(const dn_shape *s, const void *q, const void *k, const void *v, const float *beta,
                    const float *g, const int32_t *cu_seqlens, const void *dO, const float *dq, const float *dk,
                    const float *dv, const float *dbeta, const float *dg);

dn_status bwd_recompute(const dn_shape *s, const void *q, const void *k, const void *v, const float *beta,
                        const float *g, const float *h0, const int32_t *cu_seqlens, const void *dO,
                        const float *dhT, float *dq, float *dk, float *dv, float *dbeta, float *dg, float *dh0,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

}  // namespace dn
