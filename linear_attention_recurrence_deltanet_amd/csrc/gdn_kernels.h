// gdn_kernels.h -- internal interface between the C-ABI layer (gdn_api.cpp)
// and the HIP kernels.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>

namespace gdn {

// Arguments common to every forward launch.
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

// Segmented chunk walker (chunk 32 or 64).
struct WalkArgs : FwdArgs {
    void* summA;             // [B*H][nseg-1][dk][dk] segment transitions A_s, operand
                             //   precision (fp16; fp32 for fp32 inputs)   (nseg > 1)
    float* summB;            // [B*H][nseg-1][dk][dv] segment offsets B_s  (nseg > 1)
    float* snap;             // [B*H][dk][dv] copy of state_in            (nseg > 1)
    int nseg;                // segments per sequence (1: no split)
    int seg_chunks;          // chunks per segment
};

// Segmented walker: summary pass (if nseg > 1) then main pass.
hipError_t launch_walk(const WalkArgs& a, int chunk, int waves, hipStream_t s);
// Waves per workgroup (value tile = 16 * waves) that fit on chip; 0: none.
int walk_max_waves(int in_f32, int dk, int chunk);

// Pipelined walker (bf16 inputs, dk 64 or 128, dv a multiple of 64, chunk 32
// or 64): eight waves per workgroup, value tile of 64 columns in the main
// pass; the summary pass covers 64 * pipe_summary_tiles(dk, dv) columns of
// [identity | value] per workgroup.
bool pipe_supported(int in_f32, int dk, int dv, int chunk);
int pipe_summary_tiles(int dk, int dv);
hipError_t launch_pipe(const WalkArgs& a, int chunk, hipStream_t s);

// Single-pass kernel (128-token chunks; fp32 inputs with dk = 128): one
// workgroup per (batch, head, value-column tile of bv).  0: does not fit.
hipError_t launch_fwd_single(const FwdArgs& a, int chunk, int bv, hipStream_t s);
int single_max_bv(int in_f32, int dk, int chunk);

}  // namespace gdn
