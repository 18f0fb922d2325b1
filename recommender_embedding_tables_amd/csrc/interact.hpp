// Launchers of the fused pooled-lookup + DLRM dot interaction kernels.
#pragma once

#include "embtab_internal.hpp"

namespace embtab {

// Shapes the kernels take: T + 1 <= 32 vectors per sample, D a multiple of 16
// and at most 256 (a sample's vectors and pair matrix sit in one wave's LDS).
bool interact_supported(const Handle& h);

hipError_t launch_interact_forward(const Handle& h, const int64_t* offsets, const int64_t* ids,
                                   int64_t B, int64_t nnz, bool mean, const float* dense,
                                   float* out, hipStream_t s);

hipError_t launch_interact_backward(const Handle& h, const int64_t* offsets, const int64_t* ids,
                                    int64_t B, int64_t nnz, bool mean, const float* dense,
                                    const float* grad_out, float* grad_dense,
                                    float* grad_pooled, hipStream_t s);

}  // namespace embtab
