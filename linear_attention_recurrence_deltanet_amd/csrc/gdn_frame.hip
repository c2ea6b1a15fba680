// gdn_frame.hip -- frame-wise Gated DeltaNet with a normalised readout
// (SANA-Streaming, section 2.1 "Frame-wise Gated DeltaNet for Global
// Accumulated Memory": one state update per frame of N spatial tokens, a decay
// per frame, a write strength per token, an output gate, a numerator and a
// denominator state carried across chunks; section 2.3 "Efficient GDN
// Kernel": frame summaries by reductions over the spatial tokens, a short
// scan over frames, then the frame's queries read against its state).
//
// Per (b, h) and frame f, with unit keys k^ and the frame mean over n < N:
//   G_f = (1/N) sum_n beta_n k^_n k^_n^T          (dk x dk)
//   W_f = (1/N) sum_n beta_n k^_n [v_n | 1]^T     (dk x (dv + 1))
//   [M | z]_f = alpha_f (I - G_f) [M | z]_{f-1} + W_f    (M = S^T, dk x dv)
//   out_n = (M_f^T q_n) / (z_f . q_n) * gate_n
// (the query's normalisation cancels in the ratio, so q is used raw).
//
// Three launches:
//   frame_sum_kernel   summaries [G | W | w] of every (head, frame, token
//                      split): a reduction over tokens on the matrix cores;
//   frame_scan_kernel  the scan over frames, one wave per 16 state columns,
//                      the state in fp32 accumulators;
//   frame_out_kernel   the readout, one 16-byte store per lane and row.
//
// Operand precision.  The reductions over tokens contract over the row index
// of the row-major inputs, while a matrix-core operand holds eight
// consecutive k values per lane; so 16 x 16 blocks of the raw inputs, staged
// in LDS as they lie, are transposed by a product with the identity (exact),
// which leaves each lane the four tokens 4g .. 4g+3 of a block: two blocks
// give the "accumulator order" k set of a 32-token step (see gdn_common.h).
// The per-token factor beta r^2 / N (G) or beta r / N (W) is applied in fp32
// to the transposed keys, which are then split into bf16 hi + lo parts; the
// other operand is the raw bf16 input (exact), so each product costs two
// instructions and carries about 16 significant bits.  The scan multiplies
// G (hi + lo) by the state (hi + lo) in three products.  The readout takes
// M_f^T as bf16 hi + lo against the raw queries.  Everything else is fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr uint16_t kBf16One = 0x3F80;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// 16 x 16 transpose of a bf16 block [row][col] (row stride ld elements) on
// the matrix core: lane (g, c) receives x[4g + i][c], i < 4, exactly.
__device__ __forceinline__ f32x4 tr16(const uint16_t* x, int ld, int lane) {
    const int lc = lane & 15, lg = lane >> 4;
    const u16x4 a = *reinterpret_cast<const u16x4*>(x + lc * ld + 4 * lg);
    u16x4 one;
#pragma unroll
    for (int j = 0; j < 4; ++j) one[j] = (4 * lg + j == lc) ? kBf16One : (uint16_t)0;
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                    __builtin_bit_cast(bf16x4, one), zero4(), 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma_bf16(const u16x8& a, const u16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two fp32 -> two bf16 (round to nearest even), packed: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, bf2));
}
// Two fp32 that hold bf16 values exactly -> their high halves, packed.
__device__ __forceinline__ uint32_t pk_hi16(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
// x0, x1 -> bf16 hi word and lo word with x = hi + lo to about 2^-16.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    hi = pk_bf16(x0, x1);
    lo = pk_bf16(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u));
}
// Eight fp32 values -> bf16 hi and lo fragments.
__device__ __forceinline__ void split8(const float* x, u16x8& hi, u16x8& lo) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 h, l;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t a, b;
        split2(x[2 * j], x[2 * j + 1], a, b);
        h[j] = a;
        l[j] = b;
    }
    hi = __builtin_bit_cast(u16x8, h);
    lo = __builtin_bit_cast(u16x8, l);
}

__device__ __forceinline__ float ld_bf16(const void* base, size_t i) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[i]);
}

// ---------------------------------------------------------------------------
// Phase A: frame summaries.  Grid (nsp, F, B*H); 4 waves per 64-column tile
// of the summary columns [G (dk) | W_v (dv)], all tiles in one workgroup so
// that the frame's keys and values are read from memory once; the last tile
// also forms the 16-column block of w = (1/N) sum beta k^ (value 1 in its
// column 0).  Wave (j, wr) owns rows [wr * dk/4, (wr+1) * dk/4) of tile j.
// Tokens of split sp of the frame are walked 32 at a time: the workgroup
// stages the raw keys (all dk features, for the norms), the values and the
// per-token factors in LDS; each wave then transposes what it needs.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(64 * 4 * ((DK + DV) / 64)) void frame_sum_kernel(FrameArgs p) {
    constexpr int NT = (DK + DV) / 64;
    constexpr int NTH = 256 * NT;
    constexpr int NS = DK + DV + 16;
    constexpr int RB = DK / 64;          // 16-row blocks per wave
    constexpr int KST = DK + 8;          // LDS row stride of the keys (elements)
    constexpr int VST = DV + 8;          // ... and of the values
    constexpr int KP = 32 * DK / 8;      // 16-byte pieces of a 32-token key block
    constexpr int VP = 32 * DV / 8;      // ... and of a value block
    static_assert(KP <= NTH && VP <= NTH, "one piece of each per thread at most");
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][32 * KST];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][32 * VST];
    __shared__ float Ss[2][2][32];       // per-token factor: [buf][G (beta r^2 / N) | W (beta r / N)]

    const int sp = block_x(p.rev_wg), nsp = gridDim.x;
    const int f = block_y(p.rev_wg), bh = block_z(p.rev_wg);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
    const int j = w >> 2, wr = w & 3;    // tile and row group of this wave (wave-uniform)
    const int N = p.N;
    const size_t T = (size_t)p.F * N;
    const int L = (((N + nsp - 1) / nsp) + 31) & ~31;
    const int t0 = sp * L, t1 = min(N, t0 + L);
    const bool gtile = j < DK / 64;
    const bool etile = j == NT - 1;
    const float invN = 1.f / (float)N;
    const size_t row0 = (size_t)bh * T + (size_t)f * N;    // first token row of the frame
    const uint16_t* kg = reinterpret_cast<const uint16_t*>(p.k);
    const uint16_t* vg = reinterpret_cast<const uint16_t*>(p.v);
    const int vcol = 64 * (j - DK / 64);

    f32x4 acc[RB][4], acce[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        acce[rb] = zero4();
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = zero4();
    }

    // registers of the next step's staging; loads through buffer resources
    // that cover exactly this split's tokens, so rows past it (and threads
    // past the pieces) read zero without a branch (a branch around a load
    // makes the wave wait for it)
    const unsigned ntok = (unsigned)(t1 > t0 ? t1 - t0 : 0);
    const rsrc_t rk = make_rsrc(kg + (row0 + t0) * DK, ntok * DK * 2);
    const rsrc_t rbeta = make_rsrc(reinterpret_cast<const uint16_t*>(p.beta) + row0 + t0, ntok * 2);
    const rsrc_t rv = make_rsrc(vg + (row0 + t0) * DV, ntok * DV * 2);
    const bool hask = tid < KP, hasv = tid < VP;
    const int ktk = tid / (DK / 8), kfg = tid % (DK / 8);
    const int vtk = tid / (DV / 8), vfg = tid % (DV / 8);
    uint4 kreg, vreg;
    float breg;
    auto fetch = [&](int ts) {
        const unsigned tk = (unsigned)(ts - t0 + ktk);
        kreg = buf_load16(rk, hask ? tk * DK * 2 + 16 * kfg : kOffNone);
        breg = gate_beta(bf16_to_f32(buf_load2(rbeta, hask ? tk * 2 : kOffNone)), p.gate_logits != 0);
        const unsigned tv = (unsigned)(ts - t0 + vtk);
        vreg = buf_load16(rv, hasv ? tv * DV * 2 + 16 * vfg : kOffNone);
    };
    auto stage = [&](int buf) {
        float ss = 0.f;
        const uint32_t wv[4] = {kreg.x, kreg.y, kreg.z, kreg.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float a = bf16_to_f32((uint16_t)(wv[q] & 0xffffu));
            const float b = bf16_to_f32((uint16_t)(wv[q] >> 16));
            ss += a * a + b * b;
        }
        ss = group_sum<DK / 8>(ss);
        if (hask) {
            *reinterpret_cast<uint4*>(&Ks[buf][ktk * KST + 8 * kfg]) = kreg;
            if (kfg == 0) {
                const float r = p.qk_l2norm ? 1.f / sqrtf(ss + p.eps) : 1.f;
                Ss[buf][0][ktk] = breg * r * r * invN;
                Ss[buf][1][ktk] = breg * r * invN;
            }
        }
        if (hasv) *reinterpret_cast<uint4*>(&Vs[buf][vtk * VST + 8 * vfg]) = vreg;
    };

    const int nsteps = t1 > t0 ? (t1 - t0 + 31) / 32 : 0;
    if (nsteps > 0) {
        fetch(t0);
        stage(0);
    }
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1;
        if (s + 1 < nsteps) fetch(t0 + 32 * (s + 1));
        // transposed operands of this step: acc-order k = tokens {4g+i} of
        // the first 16 and {16+4g+i} of the second 16
        float sc[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[h][i] = Ss[buf][gtile ? 0 : 1][16 * h + 4 * lg + i];
        u16x8 ahi[RB], alo[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int fb = wr * RB + rb;
            float x[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 t = tr16(&Ks[buf][16 * h * KST + 16 * fb], KST, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) x[4 * h + i] = t[i] * sc[h][i];
            }
            split8(x, ahi[rb], alo[rb]);
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            u32x4 bw;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const f32x4 t = gtile ? tr16(&Ks[buf][16 * h * KST + 64 * j + 16 * cb], KST, lane)
                                      : tr16(&Vs[buf][16 * h * VST + vcol + 16 * cb], VST, lane);
                bw[2 * h] = pk_hi16(t[0], t[1]);        // exact: raw bf16 values
                bw[2 * h + 1] = pk_hi16(t[2], t[3]);
            }
            const u16x8 bf = __builtin_bit_cast(u16x8, bw);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                acc[rb][cb] = mma_bf16(ahi[rb], bf, acc[rb][cb]);
                acc[rb][cb] = mma_bf16(alo[rb], bf, acc[rb][cb]);
            }
        }
        if (etile) {
            u16x8 one;
#pragma unroll
            for (int q = 0; q < 8; ++q) one[q] = lc == 0 ? kBf16One : (uint16_t)0;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                acce[rb] = mma_bf16(ahi[rb], one, acce[rb]);
                acce[rb] = mma_bf16(alo[rb], one, acce[rb]);
            }
        }
        if (s + 1 < nsteps) stage(buf ^ 1);
        __syncthreads();
    }

    // partial sums of this split: [B*H][F][nsp][DK][NS]
    float* dst = p.sums + (((size_t)bh * p.F + f) * nsp + sp) * DK * NS;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r0 = 16 * (wr * RB + rb) + 4 * lg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) dst[(size_t)(r0 + i) * NS + 64 * j + 16 * cb + lc] = acc[rb][cb][i];
            if (etile) dst[(size_t)(r0 + i) * NS + DK + DV + lc] = acce[rb][i];
        }
    }
}

// ---------------------------------------------------------------------------
// Phase B: the scan over frames.  One workgroup per (b, h) with one wave per
// 16 columns of M (dv/16 waves).  A column tile lives in accumulators: lane
// (g, c) holds rows 16 rb + 4g + i of column c.  G_f M is formed with M as the
// B operand straight from the accumulators (k in accumulator order) and G_f,
// summed over the token splits and split into bf16 hi + lo, staged in LDS by
// the whole workgroup; the next frame's G is loaded into registers while this
// frame's products run.  The denominator z (one column) is updated on the
// vector ALU from the same LDS copy of G: four threads per row.
// ---------------------------------------------------------------------------
template <int DK>
constexpr int max_splits() { return DK == 128 ? 2 : 4; }

template <int DK, int DV>
__global__ __launch_bounds__(64 * (DV / 16)) void frame_scan_kernel(FrameArgs p) {
    constexpr int NTH = 64 * (DV / 16);
    constexpr int NS = DK + DV + 16;
    constexpr int NRB = DK / 16;
    constexpr int NKS = DK / 32;
    constexpr int GST = DK + 4;                 // LDS row stride (bf16): (DK + 4) / 2 words
    constexpr int NQ = DK * DK / 4;             // float4 pieces of G
    constexpr int QPT = (NQ + NTH - 1) / NTH;
    constexpr int MS = max_splits<DK>();
    constexpr int ZIT = 4 * DK > NTH ? 4 * DK / NTH : 1;   // rows of z per thread group
    __shared__ __attribute__((aligned(16))) uint16_t Gh[DK * GST];
    __shared__ __attribute__((aligned(16))) uint16_t Gl[DK * GST];
    __shared__ float zs[2][DK];

    const int tid = threadIdx.x, ct = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
    const int bh = block_x(p.rev_wg);
    const int nsp = p.nsp;

    f32x4 M[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * lg + i;
            M[rb][i] = p.state_in ? p.state_in[((size_t)bh * DK + row) * DV + 16 * ct + lc] : 0.f;
        }
    if (tid < DK) zs[0][tid] = p.z_in ? p.z_in[(size_t)bh * DK + tid] : 0.f;

    // summaries of frame f: a buffer resource over its nsp partials, so the
    // loads of absent partials (s >= nsp) read zero without a branch
    auto sums_rsrc = [&](int f) {
        return make_rsrc(p.sums + ((size_t)bh * p.F + f) * nsp * DK * NS, (unsigned)(nsp * DK * NS * 4));
    };
    static_assert(NQ % NTH == 0, "whole pieces per thread");
    float4 gq[QPT];
    auto load_g = [&](int f) {
        const rsrc_t r = sums_rsrc(f);
#pragma unroll
        for (int m = 0; m < QPT; ++m) {
            const int idx = tid + NTH * m;
            const int row = idx / (DK / 4), c4 = idx % (DK / 4);
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int s = 0; s < MS; ++s) {
                const uint4 u = buf_load16(r, (unsigned)(((s * DK + row) * NS + 4 * c4) * 4));
                acc.x += __uint_as_float(u.x); acc.y += __uint_as_float(u.y);
                acc.z += __uint_as_float(u.z); acc.w += __uint_as_float(u.w);
            }
            gq[m] = acc;
        }
    };
    if (p.F > 0) load_g(0);

    for (int f = 0; f < p.F; ++f) {
        const int zb = f & 1;
        __syncthreads();                    // the previous frame is done with G and z
#pragma unroll
        for (int m = 0; m < QPT; ++m) {
            const int idx = tid + NTH * m;
            const int row = idx / (DK / 4), c4 = idx % (DK / 4);
            uint32_t h0, l0, h1, l1;
            split2(gq[m].x, gq[m].y, h0, l0);
            split2(gq[m].z, gq[m].w, h1, l1);
            *reinterpret_cast<uint2*>(&Gh[row * GST + 4 * c4]) = make_uint2(h0, h1);
            *reinterpret_cast<uint2*>(&Gl[row * GST + 4 * c4]) = make_uint2(l0, l1);
        }
        __syncthreads();
        const rsrc_t rs = sums_rsrc(f);
        const float a = exp2f(gate_log2_alpha(ld_bf16(p.alpha, (size_t)bh * p.F + f), p.gate_logits != 0));
        // w_f and W_f of every split, issued first (in the order they are
        // used: the wait for w_f leaves W_f in flight) and summed where they
        // are needed, so that their memory latency overlaps the denominator
        // update; the next frame's G is loaded after them
        uint32_t wzr[ZIT][MS];
#pragma unroll
        for (int zi = 0; zi < ZIT; ++zi) {
            const int row = (tid + NTH * zi) >> 2;
#pragma unroll
            for (int s = 0; s < MS; ++s)
                wzr[zi][s] = buf_load4(rs, (tid + NTH * zi < 4 * DK) ? (unsigned)(((s * DK + row) * NS + DK + DV) * 4)
                                                                     : kOffNone);
        }
        // one lane offset per split (the split in it, so that an absent split
        // falls past the range and reads zero); the row, uniform, as the
        // scalar offset
        uint32_t wr[MS][NRB][4];
#pragma unroll
        for (int s = 0; s < MS; ++s) {
            const unsigned wlane = (unsigned)(((s * DK + 4 * lg) * NS + DK + 16 * ct + lc) * 4);
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    wr[s][rb][i] = __builtin_amdgcn_raw_buffer_load_b32(rs, wlane, (unsigned)((16 * rb + i) * NS * 4), 0);
        }
        // denominator: z <- alpha (z - G z) + w, four threads per row
#pragma unroll
        for (int zi = 0; zi < ZIT; ++zi) {
            const int zt = tid + NTH * zi;
            if (zt >= 4 * DK) break;                      // wave-uniform
            const int row = zt >> 2, part = zt & 3;
            float y = 0.f;
#pragma unroll
            for (int c = 0; c < DK / 4; ++c) {
                const int kk = part * (DK / 4) + c;
                const float g = __uint_as_float((uint32_t)Gh[row * GST + kk] << 16) +
                                __uint_as_float((uint32_t)Gl[row * GST + kk] << 16);
                y += g * zs[zb][kk];
            }
            y += __shfl_xor(y, 1, 64);
            y += __shfl_xor(y, 2, 64);
            float wz = 0.f;
#pragma unroll
            for (int s = 0; s < MS; ++s) wz += __uint_as_float(wzr[zi][s]);
            if (part == 0) {
                const float zn = a * (zs[zb][row] - y) + wz;
                zs[zb ^ 1][row] = zn;
                p.zf[((size_t)bh * p.F + f) * DK + row] = zn;
            }
        }
        // W_f, summed over the splits once the denominator update has covered
        // its latency
        float wv[NRB][4];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float w = 0.f;
#pragma unroll
                for (int s = 0; s < MS; ++s) w += __uint_as_float(wr[s][rb][i]);
                wv[rb][i] = w;
            }
        // B operand: the state, hi + lo, k in accumulator order
        u16x8 bhi[NKS], blo[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = M[2 * ks][i];
                x[4 + i] = M[2 * ks + 1][i];
            }
            split8(x, bhi[ks], blo[ks]);
        }
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            f32x4 y = zero4();
            const int grow = 16 * rb + lc;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int k0 = grow * GST + 32 * ks + 4 * lg;
                const u16x4 h0 = *reinterpret_cast<const u16x4*>(&Gh[k0]);
                const u16x4 h1 = *reinterpret_cast<const u16x4*>(&Gh[k0 + 16]);
                const u16x4 l0 = *reinterpret_cast<const u16x4*>(&Gl[k0]);
                const u16x4 l1 = *reinterpret_cast<const u16x4*>(&Gl[k0 + 16]);
                const u16x8 ghi = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
                const u16x8 glo = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
                y = mma_bf16(ghi, bhi[ks], y);
                y = mma_bf16(ghi, blo[ks], y);
                y = mma_bf16(glo, bhi[ks], y);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) M[rb][i] = a * (M[rb][i] - y[i]) + wv[rb][i];
        }
        if (f + 1 < p.F) load_g(f + 1);     // staged at the start of the next frame
        // the frame's state for the readout: M^T as bf16 hi + lo
        const size_t base = (((size_t)bh * p.F + f) * DV + 16 * ct + lc) * DK;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            uint32_t h0, l0, h1, l1;
            split2(M[rb][0], M[rb][1], h0, l0);
            split2(M[rb][2], M[rb][3], h1, l1);
            const size_t o = base + 16 * rb + 4 * lg;
            *reinterpret_cast<uint2*>(p.mt_hi + o) = make_uint2(h0, h1);
            *reinterpret_cast<uint2*>(p.mt_lo + o) = make_uint2(l0, l1);
        }
    }
    __syncthreads();

    // final states
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 4 * lg + i;
            if (p.state_out) p.state_out[((size_t)bh * DK + row) * DV + 16 * ct + lc] = M[rb][i];
        }
    if (tid < DK && p.z_out) p.z_out[(size_t)bh * DK + tid] = zs[p.F & 1][tid];
}

// ---------------------------------------------------------------------------
// Phase C: the readout.  One workgroup of 8 waves per (64 value columns,
// token range, frame, head).  The workgroup
// stages M_f^T hi + lo of 64 value columns in LDS; each wave keeps them as A
// operands (k = key index) with z_f, and walks 16-token blocks of the frame,
// the next block's queries loading while the current one is formed.  The B
// operand is the raw query rows, so the product is out^T and lane (g, c)
// holds columns 4g .. 4g+3 of token c; the denominator z . q of token c is
// summed over the four lanes holding its k slices, which are exactly the
// lanes that hold its outputs.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(512) void frame_out_kernel(FrameArgs p) {
    constexpr int NCG = DV / 64;
    constexpr int NKS = DK / 32;
    constexpr int MST = DK + 8;
    __shared__ __attribute__((aligned(16))) uint16_t Mh[64 * MST];
    __shared__ __attribute__((aligned(16))) uint16_t Ml[64 * MST];
    // One-dimensional grid of NCG x (nts x F x B*H) work items.  Workgroups
    // are dealt to the 8 XCDs round-robin; the NCG column groups of one
    // (token range, frame, head) read the same queries, so they are placed 8
    // apart and share an XCD and its L2 (the items past the last whole
    // multiple of 8 keep the plain order).
    const int nts = p.nts;
    int cg, rest;
    {
        const int n = (int)gridDim.x, lin = block_x(p.rev_wg);
        const int n8 = (n / NCG) / 8 * 8 * NCG;
        if (lin < n8) {
            const int a = lin & 7, bq = lin >> 3;
            cg = bq % NCG;
            rest = a + 8 * (bq / NCG);
        } else {
            cg = lin % NCG;
            rest = lin / NCG;
        }
    }
    const int ts = rest % nts, f = (rest / nts) % p.F, bh = rest / (nts * p.F);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lg = lane >> 4, lc = lane & 15;
    const int N = p.N;
    const size_t T = (size_t)p.F * N;
    const size_t row0 = (size_t)bh * T + (size_t)f * N;
    const uint16_t* qg = reinterpret_cast<const uint16_t*>(p.q);
    const uint16_t* gg = reinterpret_cast<const uint16_t*>(p.out_gate);

    // Prologue: every load it needs -- this column group's M_f^T (hi + lo), z_f
    // and the first block's queries and gate -- is issued before any is
    // used, so the workgroup pays one memory round trip before its first
    // products, not one per kind of operand
    const size_t mb = ((size_t)bh * p.F + f) * DV * DK + (size_t)64 * cg * DK;
    constexpr int MIT = 64 * DK / 8 / 512;          // 16-byte pieces per thread of each of hi, lo
    static_assert(MIT * 512 * 8 == 64 * DK, "whole pieces");
    uint4 mh[MIT], ml[MIT];
#pragma unroll
    for (int j = 0; j < MIT; ++j) {
        const int e = tid + 512 * j, r = e / (DK / 8), c8 = e % (DK / 8);
        mh[j] = *reinterpret_cast<const uint4*>(p.mt_hi + mb + (size_t)r * DK + 8 * c8);
        ml[j] = *reinterpret_cast<const uint4*>(p.mt_lo + mb + (size_t)r * DK + 8 * c8);
    }
    float zq[NKS][8];
    const float* zf = p.zf + ((size_t)bh * p.F + f) * DK;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int q = 0; q < 8; ++q) zq[ks][q] = zf[32 * ks + 8 * lg + q];

    // queries and gate of the frame through buffer resources: rows past the
    // frame read zero without a branch
    const rsrc_t rq = make_rsrc(qg + row0 * DK, (unsigned)(N * DK * 2));
    const rsrc_t rg = make_rsrc(gg ? gg + row0 * DV : qg, gg ? (unsigned)(N * DV * 2) : 0u);
    const int nb = (N + 15) / 16;
    const int stride = 8 * nts;
    int b = ts * 8 + w;
    u16x8 qn[NKS];
    uint2 gn[4];
    auto load_q = [&](int bb) {
        const unsigned t = (unsigned)(bb < nb ? 16 * bb + lc : N);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const uint4 u = buf_load16(rq, t * DK * 2 + (32 * ks + 8 * lg) * 2);
            qn[ks] = __builtin_bit_cast(u16x8, u);
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) gn[ct] = buf_load8(rg, (t * DV + 64 * cg + 16 * ct + 4 * lg) * 2);
    };
    load_q(b);
#pragma unroll
    for (int j = 0; j < MIT; ++j) {
        const int e = tid + 512 * j, r = e / (DK / 8), c8 = e % (DK / 8);
        *reinterpret_cast<uint4*>(&Mh[r * MST + 8 * c8]) = mh[j];
        *reinterpret_cast<uint4*>(&Ml[r * MST + 8 * c8]) = ml[j];
    }
    __syncthreads();
    u16x8 ah[4][NKS], al[4][NKS];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            ah[ct][ks] = *reinterpret_cast<const u16x8*>(&Mh[(16 * ct + lc) * MST + 32 * ks + 8 * lg]);
            al[ct][ks] = *reinterpret_cast<const u16x8*>(&Ml[(16 * ct + lc) * MST + 32 * ks + 8 * lg]);
        }
    for (; b < nb; b += stride) {
        u16x8 qf[NKS];
        uint2 gf[4];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[ks] = qn[ks];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) gf[ct] = gn[ct];
        load_q(b + stride);
        const int t = 16 * b + lc;
        const bool valid = t < N;
        const size_t row = row0 + t;
        float den = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int q = 0; q < 8; ++q) den += zq[ks][q] * bf16_to_f32(qf[ks][q]);
        den += __shfl_xor(den, 16, 64);
        den += __shfl_xor(den, 32, 64);
        const float rden = 1.f / den;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                acc = mma_bf16(ah[ct][ks], qf[ks], acc);
                acc = mma_bf16(al[ct][ks], qf[ks], acc);
            }
            if (valid) {
                const int col = 64 * cg + 16 * ct + 4 * lg;
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = acc[i] * rden;
                if (gg) {
                    const uint2 gv = gf[ct];
                    o[0] *= __uint_as_float(gv.x << 16);
                    o[1] *= __uint_as_float(gv.x & 0xffff0000u);
                    o[2] *= __uint_as_float(gv.y << 16);
                    o[3] *= __uint_as_float(gv.y & 0xffff0000u);
                }
                if (p.out_bf16) {
                    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + row * DV + col) =
                        make_uint2(pk_bf16(o[0], o[1]), pk_bf16(o[2], o[3]));
                } else {
                    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + row * DV + col) =
                        make_float4(o[0], o[1], o[2], o[3]);
                }
            }
        }
    }
}

template <int DK, int DV>
hipError_t launch3(const FrameArgs& a, hipStream_t s) {
    const unsigned bh = (unsigned)a.B * a.H;
    if (a.F > 0) {
        hipLaunchKernelGGL((frame_sum_kernel<DK, DV>), dim3(a.nsp, a.F, bh), dim3(256 * ((DK + DV) / 64)), 0, s, a);
    }
    hipLaunchKernelGGL((frame_scan_kernel<DK, DV>), dim3(bh), dim3(64 * (DV / 16)), 0, s, a);
    if (a.F > 0) {
        hipLaunchKernelGGL((frame_out_kernel<DK, DV>), dim3((unsigned)(DV / 64) * a.nts * a.F * bh), dim3(512), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

void frame_plan(int B, int H, int F, int N, int dk, int dv, int* nsp, int* nts) {
    const long long bhf = (long long)B * H * (F > 0 ? F : 1);
    // summaries: about 384 workgroups, splits of at least 128 tokens
    const long long nt = (dk + dv) / 64;
    long long s = (384 + nt * bhf - 1) / (nt * bhf);
    long long smax = N / 128 > 0 ? N / 128 : 1;
    const long long ms = dk == 128 ? 2 : 4;     // max_splits<DK>() of the scan
    if (smax > ms) smax = ms;
    *nsp = (int)(s < 1 ? 1 : (s > smax ? smax : s));
    // readout: about 1024 workgroups of 8 waves, each wave at least one 16-token
    // block: a workgroup's time is mostly its first memory round trips, so more
    // and shorter token ranges finish sooner (measured against 256 and 512
    // targets: 42.0 and 40.0 -> 40.0 us at d = 64, 92.0 and 91.2 -> 88.8 us at
    // d = 128 per frame-wise call)
    const long long ncg = dv / 64;
    long long r = (1024 + ncg * bhf - 1) / (ncg * bhf);
    long long rmax = (N + 127) / 128;
    *nts = (int)(r < 1 ? 1 : (r > rmax ? rmax : r));
}

size_t frame_workspace(int B, int H, int F, int N, int dk, int dv, size_t* off_mt, size_t* off_zf) {
    int nsp, nts;
    frame_plan(B, H, F, N, dk, dv, &nsp, &nts);
    auto r256 = [](size_t n) { return (n + 255) & ~(size_t)255; };
    const size_t bhf = (size_t)B * H * F;
    const size_t sums = r256(bhf * nsp * dk * (size_t)(dk + dv + 16) * 4);
    const size_t mt = r256(bhf * dv * dk * 2);
    if (off_mt) *off_mt = sums;
    if (off_zf) *off_zf = sums + 2 * mt;
    return sums + 2 * mt + r256(bhf * dk * 4);
}

hipError_t launch_framewise(const FrameArgs& a, hipStream_t s) {
    if (a.dk == 64 && a.dv == 64) return launch3<64, 64>(a, s);
    if (a.dk == 64 && a.dv == 128) return launch3<64, 128>(a, s);
    if (a.dk == 128 && a.dv == 64) return launch3<128, 64>(a, s);
    if (a.dk == 128 && a.dv == 128) return launch3<128, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace gdn
