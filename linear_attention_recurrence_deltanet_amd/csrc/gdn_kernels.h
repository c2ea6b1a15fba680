// gdn_kernels.h -- internal interface between the C-ABI layer (gdn_api.cpp)
// and the HIP kernels.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>

namespace gdn {

// Record a message for gdn_last_error() on this thread and return status
// (for entry points outside gdn_api.cpp).
int api_fail(int status, const char* msg);

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
    int gate_logits;         // 1: alpha, beta hold logits (gate_log2_alpha, gate_beta)
    const void* out_gate;    // null, or [B*H][T][dv] in the input dtype: out *= gate
    int reverse;             // 1: walk the tokens backward (position t is token T-1-t)
    int accumulate;          // 1: out = (gated) outputs + acc_src, rounded once
    const float* acc_src;    // accumulate: fp32 [B*H][T][dv] to add
    int rev_wg;              // debug: workgroups take their work items in reverse order
};

// Segmented chunk walkers (chunk 32 or 64).  With nseg > 1 the workspace
// holds the segment maps M_out = A_s M_in + B_s:
//   segmented walker (fp32 inputs): segments 0 .. nseg-2, A_s row-major
//     (operand precision: fp16, fp32 for fp32 inputs), B_s row-major;
//   pipelined walker: all nseg segments, A_s fp16 in MFMA fragment order,
//     B_s fp32 in accumulator order, plus Phi (the outputs' linear part) and
//     the outputs from a zero incoming state (fp16), both in fragment order.
struct WalkArgs : FwdArgs {
    void* summA;             // [B*H][nseg(-1)][dk][dk] segment transitions A_s
    float* summB;            // [B*H][nseg(-1)][dk][dv] segment offsets B_s
    float* snap;             // [B*H][dk][dv] copy of state_in
    void* phi;               // pipelined: [B*H][nseg][seg_chunks*chunk][dk] fp16, fragment order
    void* ostage;            // pipelined: [B*H][nseg][seg_chunks*chunk][dv] fp16 partial outputs
    float* sscale;           // pipelined: [B*H][dv/16] power-of-two working scale of each 16
                             // value columns; staged outputs and maps are in units of it
    int nseg;                // segments per sequence (1: no split)
    int seg_chunks;          // chunks per segment
    // pipelined, plain calls: segment 0 walks its value columns from
    // state_in and writes its outputs directly (its tiles of identity columns
    // only are not launched) and leaves its final state, at the working
    // scale, in snap; the correction pass then covers segments 1 .. nseg-1,
    // folding from snap through the maps of segments 1 .. s-1
    int seg0_direct;
    // pipelined: the last fix_split segments are corrected by two workgroups
    // each, one per half of the segment's chunks
    int fix_split;
    // Both directions of a bidirectional call in one segmented launch pair
    // (pipelined walker): the walk launch covers direction 0 (forward, the
    // buffers above) and direction 1 (tokens in reverse from a zero state,
    // the buffers in bw, segments mirrored so that both directions' segment
    // s holds the same tokens); one correction pass writes the sum.
    int bidir;
    struct SegBufs {
        void* summA;
        float* summB;
        void* phi;
        void* ostage;
        float* sscale;
    } bw;
};

// Segmented walker: summary pass (if nseg > 1) then main pass.
hipError_t launch_walk(const WalkArgs& a, int chunk, int waves, hipStream_t s);
// Waves per workgroup (value tile = 16 * waves) that fit on chip; 0: none.
int walk_max_waves(int in_f32, int dk, int chunk);

// Pipelined walker (bf16 inputs, dk 64 or 128, dv a multiple of 64, chunk 32
// or 64): eight waves per workgroup, value tile of 64 columns without
// segments; with segments one walk per segment covers 64 * pipe_seg_tiles(dk,
// dv) columns of [identity | value] per workgroup, and a correction pass
// completes outputs and state.
bool pipe_supported(int in_f32, int dk, int dv, int chunk);
int pipe_seg_tiles(int dk, int dv);
size_t pipe_workspace(int B, int H, int dk, int dv, int chunk, int nseg, int seg_chunks);
hipError_t launch_pipe(const WalkArgs& a, int chunk, hipStream_t s);

// Single-pass kernel (128-token chunks; fp32 inputs with dk = 128): one
// workgroup per (batch, head, value-column tile of bv).  0: does not fit.
hipError_t launch_fwd_single(const FwdArgs& a, int chunk, int bv, hipStream_t s);
int single_max_bv(int in_f32, int dk, int chunk);

// Softmax attention over [sink; window; current] keys (gdn_attn.hip):
// q, out [B*H][Nq][d]; k[s], v[s] [B*H][n[s]][d] for s = sink, window,
// current (bf16); out fp32 or bf16.
struct AttnArgs {
    const void* q;
    const void* k[3];
    const void* v[3];
    int n[3];
    void* out;
    int B, H, Nq, d;
    float scale;
    int out_bf16;
    int nsplit;              // key ranges (1: no split)
    float* part_o;           // nsplit > 1: [nsplit][B*H*Nq][d] unnormalised outputs
    float* part_ml;          // nsplit > 1: [nsplit][B*H*Nq][2] running max (exp2 domain), sum
    int rev_wg;              // debug: workgroups take their work items in reverse order
};
bool attn_supported(int d);
// Key ranges the launch splits into (1 when the workgroups already fill the
// chip), and the workspace they need.
int attn_splits(int B, int H, int Nq, const int n[3]);
size_t attn_workspace(int B, int H, int Nq, int d, int nsplit);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);

// Frame-wise Gated DeltaNet with a normalised readout (gdn_frame.hip): frame
// summaries, a scan over frames, the readout; bf16 inputs.
struct FrameArgs {
    const void* q;           // [B*H][T][dk], T = F * N
    const void* k;           // [B*H][T][dk]
    const void* v;           // [B*H][T][dv]
    const void* alpha;       // [B*H][F] decay per frame (logits if gate_logits)
    const void* beta;        // [B*H][T] write strength (logits if gate_logits)
    const float* state_in;   // [B*H][dk][dv] or null
    const float* z_in;       // [B*H][dk] or null
    void* out;               // [B*H][T][dv] fp32 or bf16
    float* state_out;        // [B*H][dk][dv] or null
    float* z_out;            // [B*H][dk] or null
    const void* out_gate;    // [B*H][T][dv] or null
    int B, H, F, N, dk, dv;
    int gate_logits, qk_l2norm, out_bf16;
    float eps;
    int nsp;                 // token splits of a frame's summaries
    int nts;                 // token splits of the readout
    float* sums;             // workspace: [B*H][F][nsp][dk][dk + dv + 16] partial summaries
    uint16_t* mt_hi;         // workspace: [B*H][F][dv][dk] M_f^T, bf16 hi part
    uint16_t* mt_lo;         // workspace: [B*H][F][dv][dk] bf16 lo part
    float* zf;               // workspace: [B*H][F][dk] z_f
    int rev_wg;              // debug: workgroups take their work items in reverse order
};
// Token splits of the launch plan, and the workspace (bytes) with the
// offsets of mt_hi and zf (mt_lo follows mt_hi at the same distance).
void frame_plan(int B, int H, int F, int N, int dk, int dv, int* nsp, int* nts);
size_t frame_workspace(int B, int H, int F, int N, int dk, int dv, size_t* off_mt, size_t* off_zf);
hipError_t launch_framewise(const FrameArgs& a, hipStream_t s);

}  // namespace gdn
