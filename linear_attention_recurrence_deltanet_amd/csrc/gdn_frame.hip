// gdn_frame.hip -- prologue and epilogue of the frame-wise Gated DeltaNet
// with a normalised readout (SANA-Streaming, section 2.1 "Frame-wise Gated
// DeltaNet for Global Accumulated Memory"; appendix G.3 names the per-frame
// decay, per-token write and output gates, G.4/G.5 the frame-wise update and
// the normalised readout).
//
// The frame-wise update is the token-wise gated delta rule with the frame's
// decay on its first token and no decay on the others; the denominator state
// z is one more state column driven by a value of constant 1.  The scan
// itself is the token-wise pipelined walker, run on
//   values  [v | 1 0 ... 0]      (dv + 64 columns: one 64-column tile more),
//   state   [M | z 0 ... 0]      (dk x (dv + 64), fp32),
//   decay   alpha_f on token f*N, 1 elsewhere (logits: -inf, which maps to 1);
// the prologue writes these into the workspace, the epilogue divides each
// output row by its denominator column, applies the output gate, rounds once
// and unpacks the state.  Both are streaming kernels bound by HBM: 16-byte
// accesses, consecutive lanes on consecutive pieces of a row.  Indices are
// 32-bit: the caller keeps B*H*T*(dv + 64) below 2^31.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr uint16_t kBf16One = 0x3F80;
constexpr uint16_t kBf16NegInf = 0xFF80;

int grid_for(unsigned work) {
    const unsigned g = (work + kThreads - 1) / kThreads;
    return (int)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

__global__ __launch_bounds__(kThreads) void frame_prep_kernel(FrameArgs p) {
    const unsigned T = (unsigned)p.F * p.N, bh = (unsigned)p.B * p.H;
    const unsigned dvp = p.dv + 64;
    const unsigned stride = (unsigned)gridDim.x * kThreads;
    const unsigned tid = (unsigned)blockIdx.x * kThreads + threadIdx.x;

    // values: rows of dvp bf16 in 16-byte pieces
    const unsigned ppr = dvp / 8, vpr = p.dv / 8;
    const uint4* vs = reinterpret_cast<const uint4*>(p.v);
    uint4* va = reinterpret_cast<uint4*>(p.v_aug);
    const unsigned nv = bh * T * ppr;
    for (unsigned e = tid; e < nv; e += stride) {
        const unsigned row = e / ppr;
        const unsigned c = e - row * ppr;
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (c < vpr) w = vs[row * vpr + c];
        else if (c == vpr) w.x = kBf16One;          // the denominator's value column
        va[e] = w;
    }

    // decay: alpha_f on the first token of frame f, 1 on the others
    const uint16_t* al = reinterpret_cast<const uint16_t*>(p.alpha);
    uint16_t* at = reinterpret_cast<uint16_t*>(p.alpha_tok);
    const uint16_t none = p.gate_logits ? kBf16NegInf : kBf16One;
    const unsigned na = bh * T;
    for (unsigned e = tid; e < na; e += stride) {
        const unsigned h = e / T;
        const unsigned t = e - h * T;
        const unsigned f = t / p.N;
        at[e] = (t - f * p.N == 0) ? al[h * p.F + f] : none;
    }

    // state [M | z 0 ...]: only when an incoming state is given
    if (p.state_in || p.z_in) {
        const unsigned spr = dvp / 4, mpr = p.dv / 4;
        const unsigned ns = bh * p.dk * spr;
        const float4* sm = reinterpret_cast<const float4*>(p.state_in);
        float4* sa = reinterpret_cast<float4*>(p.state_aug);
        for (unsigned e = tid; e < ns; e += stride) {
            const unsigned row = e / spr;                 // (head, key index)
            const unsigned c = e - row * spr;
            float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < mpr) {
                if (sm) w = sm[row * mpr + c];
            } else if (c == mpr && p.z_in) {
                w.x = p.z_in[row];
            }
            sa[e] = w;
        }
    }
}

__global__ __launch_bounds__(kThreads) void frame_readout_kernel(FrameArgs p) {
    const unsigned T = (unsigned)p.F * p.N, bh = (unsigned)p.B * p.H;
    const unsigned dvp = p.dv + 64;
    const unsigned stride = (unsigned)gridDim.x * kThreads;
    const unsigned tid = (unsigned)blockIdx.x * kThreads + threadIdx.x;

    // out = numerator / denominator (* gate), one rounding
    const unsigned ppr = p.dv / 4;
    const unsigned no = bh * T * ppr;
    const bool gated = p.out_gate != nullptr;
    for (unsigned e = tid; e < no; e += stride) {
        const unsigned row = e / ppr;
        const unsigned c = e - row * ppr;
        const float* src = p.out_aug + row * dvp;
        const float4 num = *reinterpret_cast<const float4*>(src + 4 * c);
        const float den = src[p.dv];
        float o[4] = {num.x / den, num.y / den, num.z / den, num.w / den};
        if (gated) {
            const uint2 g = reinterpret_cast<const uint2*>(p.out_gate)[e];
            o[0] *= bf16_to_f32((uint16_t)(g.x & 0xffffu));
            o[1] *= bf16_to_f32((uint16_t)(g.x >> 16));
            o[2] *= bf16_to_f32((uint16_t)(g.y & 0xffffu));
            o[3] *= bf16_to_f32((uint16_t)(g.y >> 16));
        }
        if (p.out_bf16) {
            uint2 w;
            w.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
            w.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
            reinterpret_cast<uint2*>(p.out)[e] = w;
        } else {
            reinterpret_cast<float4*>(p.out)[e] = make_float4(o[0], o[1], o[2], o[3]);
        }
    }

    // state: M to state_out, the denominator column to z_out
    if (p.state_out) {
        const unsigned spr = dvp / 4, mpr = p.dv / 4;
        const unsigned ns = bh * p.dk * mpr;
        const float4* sa = reinterpret_cast<const float4*>(p.state_aug);
        float4* so = reinterpret_cast<float4*>(p.state_out);
        for (unsigned e = tid; e < ns; e += stride) {
            const unsigned row = e / mpr;
            so[e] = sa[row * spr + (e - row * mpr)];
        }
    }
    if (p.z_out) {
        const unsigned nz = bh * p.dk;
        for (unsigned e = tid; e < nz; e += stride) p.z_out[e] = p.state_aug[e * dvp + p.dv];
    }
}

}  // namespace

hipError_t launch_frame_prep(const FrameArgs& a, hipStream_t s) {
    const unsigned T = (unsigned)a.F * a.N, bh = (unsigned)a.B * a.H;
    unsigned work = bh * T * ((a.dv + 64) / 8);
    const unsigned st = bh * a.dk * ((a.dv + 64) / 4);
    if (st > work) work = st;
    hipLaunchKernelGGL(frame_prep_kernel, dim3(grid_for(work)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_frame_readout(const FrameArgs& a, hipStream_t s) {
    const unsigned T = (unsigned)a.F * a.N, bh = (unsigned)a.B * a.H;
    unsigned work = bh * T * (a.dv / 4);
    const unsigned st = bh * a.dk * (a.dv / 4);
    if (st > work) work = st;
    hipLaunchKernelGGL(frame_readout_kernel, dim3(grid_for(work)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace gdn
