// gdn_kernels.h -- internal interface between the C-ABI layer (gdn_api.cpp)
// and the HIP kernels (gdn_fwd.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>

namespace gdn {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* alpha;
    const void* beta;
    const float* state_in;   // may be null (zero state)
    void* out;
    float* state_out;        // may be null
    int B, H, T, dk, dv;
    float scale, eps;
    int qk_l2norm;
    int out_bf16;            // 1: out is bf16, 0: fp32
    int in_f32;              // 1: inputs fp32, 0: bf16
};

// Single-pass launch: one workgroup per (batch, head, value-column tile).
hipError_t launch_fwd_seq(const FwdArgs& a, int chunk, int bv, hipStream_t s);

// Largest value-column tile whose LDS plan fits one workgroup.
int seq_max_bv(int in_f32, int dk, int chunk);

}  // namespace gdn
