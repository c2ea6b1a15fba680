// gdn_fwd_single.hip -- chunked Gated DeltaNet forward on gfx950 (MI355X),
// single-pass variant: used for 128-token chunks (whose C x C intermediates
// do not leave room for the per-wave buffers of the segmented walker) and for
// fp32 inputs with 128-wide keys.
//
// The recurrence (token-wise gated delta rule; SANA-Streaming, paperpeel page,
// section 2.1, Gated DeltaNet [35]; state carried across streaming chunks),
// with the state stored transposed, M = S^T [dk][dv]:
//     u_t = beta_t (v_t - alpha_t M^T k_t),   M <- alpha_t M + k_t u_t^T,
//     o_t = M^T q_t                      (q_t, k_t unit-normalised)
//
// is evaluated a chunk of C tokens at a time (UT / WY form).  With
// g_r = sum_{s<=r} log alpha_s inside the chunk, gam = exp(g),
// G_rs = exp(g_r - g_s) (r >= s only, so every exponent is <= 0):
//     A  = diag(beta) strict_tril(K^ K^T .* G)
//     T  = (I + A)^-1 diag(beta),    T2 = T diag(gam)
//     W  = T2 K^ ,   Ut = T V,        U = Ut - W M0
//     O  = diag(gam) Q^ M0 + tril(Q^ K^T .* G) U
//     M  = gam_C M0 + K^T diag(exp(g_C - g)) U
// A partial last chunk behaves exactly as if padded with alpha = 1,
// beta = 0, q = k = v = 0.
//
// One workgroup (4 waves) owns one (batch, head, value-column tile of BV)
// and walks the chunks in order; the fp32 state tile lives in registers for
// the whole sequence (section 2.3 "Efficient GDN Kernel": the state stays on
// chip while q/k/v stream from HBM).  Matrix products run on the matrix
// cores: the Gram products on the raw bf16 inputs (exact operands), every
// product with a computed operand in fp16 (11-bit significand) with fp32
// accumulation; fp32 inputs use fp32 matrix-core products throughout.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

template <class In> struct InTraits;
template <> struct InTraits<uint16_t> {
    typedef OpBF16 Gram;
    __device__ static __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
};
template <> struct InTraits<float> {
    typedef OpF32 Gram;
    __device__ static __forceinline__ float to_f32(float x) { return x; }
};

__device__ __forceinline__ float warp_xor_sum(float v, int width) {
    for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int A_, int B_> struct cmax { static constexpr int v = A_ > B_ ? A_ : B_; };
constexpr int align16(int x) { return (x + 15) & ~15; }

// Compile-time LDS plan of one workgroup.
template <class In, class Op, int DK, int C, int BV>
struct Plan {
    typedef typename Op::elem E;
    static constexpr int NB = C / 16;
    static constexpr int PIN = 16 / (int)sizeof(In);
    static constexpr int PE = 16 / (int)sizeof(E);
    static constexpr int LDQ = DK + PIN;   // qraw / kraw rows
    static constexpr int LDA = C + 4;      // fp32 A / X
    static constexpr int LDT = C + PE;     // T, T2, P, Kt, Vt, Ut, U2t rows
    static constexpr int LDW = DK + PE;    // W, Mt rows
    // region X: phase-disjoint union
    static constexpr int X_IN = 2 * C * LDQ * (int)sizeof(In);
    static constexpr int X_A = C * LDA * 4;
    static constexpr int X_T = 2 * C * LDT * (int)sizeof(E);
    static constexpr int X_W = C * LDW * (int)sizeof(E);
    static constexpr int X_U = 2 * BV * LDT * (int)sizeof(E);
    static constexpr int SZ_X = align16(cmax<cmax<X_IN, X_A>::v, cmax<cmax<X_T, X_W>::v, X_U>::v>::v);
    static constexpr int SZ_KT = align16(DK * LDT * (int)sizeof(E));
    static constexpr int SZ_VT = align16(BV * LDT * (int)sizeof(E));
    static constexpr int SZ_P = align16(C * LDT * (int)sizeof(E));
    static constexpr int SZ_MT = align16(BV * LDW * (int)sizeof(E));
    static constexpr int SZ_VEC = 6 * C * 4;
    static constexpr int OFF_X = 0;
    static constexpr int OFF_KT = OFF_X + SZ_X;
    static constexpr int OFF_VT = OFF_KT + SZ_KT;
    static constexpr int OFF_P = OFF_VT + SZ_VT;
    static constexpr int OFF_MT = OFF_P + SZ_P;
    static constexpr int OFF_VEC = OFF_MT + SZ_MT;
    static constexpr int TOTAL = OFF_VEC + SZ_VEC;
};

template <class In, class Op, int DK, int C, int BV>
constexpr int lds_bytes() { return Plan<In, Op, DK, C, BV>::TOTAL; }

// Q^ operand fragment: raw input row scaled by its r_q, converted to Op.
template <class In, class Op>
__device__ __forceinline__ typename Op::frag qhat_frag(const In* base, int ld, int row0, int kb,
                                                       int lane, float rq) {
    const In* p = base + (row0 + (lane & 15)) * ld + kb + (lane >> 4) * Op::KPER;
    if constexpr (Op::KPER == 1) {
        return Op::from_f32(InTraits<In>::to_f32(p[0]) * rq);
    } else {
        typename Op::frag f;
#pragma unroll
        for (int e = 0; e < Op::KPER; ++e) {
            _Float16 h = (_Float16)(InTraits<In>::to_f32(p[e]) * rq);
            f[e] = __builtin_bit_cast(uint16_t, h);
        }
        return f;
    }
}

// Store 4 consecutive values of a row as Op elements.
template <class E>
__device__ __forceinline__ void st4(E* p, float a, float b, float c, float d) {
    p[0] = (E)a; p[1] = (E)b; p[2] = (E)c; p[3] = (E)d;
}

template <class In, class Op, int DK, int C, int BV>
__global__ __launch_bounds__(256)
void gdn_fwd_single_kernel(FwdArgs p) {
    typedef Plan<In, Op, DK, C, BV> L;
    typedef typename Op::elem E;
    typedef typename InTraits<In>::Gram GOp;
    constexpr int NB = L::NB;
    constexpr int NCB = BV / 16;                  // column blocks per tile
    constexpr int NTO = NB * NCB;                 // O / U tiles  [C x BV]
    constexpr int SO = (NTO + 3) / 4;
    constexpr int NTM = (DK / 16) * NCB;          // state tiles  [DK x BV]
    constexpr int SM = (NTM + 3) / 4;
    constexpr int NTW = (DK / 16) * NB;           // W^T tiles    [DK x C]
    constexpr int SW = (NTW + 3) / 4;
    constexpr int NTG = NB * (NB + 1) / 2;        // lower-triangle Gram tiles
    constexpr int SG = (NTG + 3) / 4;
    constexpr int EPV = 16 / (int)sizeof(In);     // input elements per 16-byte load
    constexpr int VPRQ = DK / EPV;                // 16-byte loads per q/k row
    constexpr int VPRV = BV / EPV;                // 16-byte loads per v tile row

    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    In* qraw = reinterpret_cast<In*>(smem + L::OFF_X);
    In* kraw = qraw + C * L::LDQ;
    float* Am = reinterpret_cast<float*>(smem + L::OFF_X);
    E* Tm = reinterpret_cast<E*>(smem + L::OFF_X);
    E* T2m = Tm + C * L::LDT;
    E* Wm = reinterpret_cast<E*>(smem + L::OFF_X);
    E* Ut = reinterpret_cast<E*>(smem + L::OFF_X);
    E* U2t = Ut + BV * L::LDT;
    E* Kt = reinterpret_cast<E*>(smem + L::OFF_KT);
    E* Vt = reinterpret_cast<E*>(smem + L::OFF_VT);
    E* Pm = reinterpret_cast<E*>(smem + L::OFF_P);
    E* Mt = reinterpret_cast<E*>(smem + L::OFF_MT);
    float* v_rq = reinterpret_cast<float*>(smem + L::OFF_VEC);
    float* v_rk = v_rq + C;
    float* v_g2 = v_rk + C;
    float* v_gam = v_g2 + C;
    float* v_eg = v_gam + C;
    float* v_beta = v_eg + C;
    __shared__ float v_red[4];                    // per-wave maxima for the working scale

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ntile = p.dv / BV;
    const int tile = block_x(p.rev_wg) % ntile;
    const int bh = block_x(p.rev_wg) / ntile;
    const int col0 = tile * BV;
    const int T = p.T, dv = p.dv;
    const TokMap tm = tok_map(T, p.reverse);   // walk position -> token

    const In* qg = reinterpret_cast<const In*>(p.q) + (size_t)bh * T * DK;
    const In* kg = reinterpret_cast<const In*>(p.k) + (size_t)bh * T * DK;
    const In* vg = reinterpret_cast<const In*>(p.v) + (size_t)bh * T * dv;
    const In* ag = reinterpret_cast<const In*>(p.alpha) + (size_t)bh * T;
    const In* bg = reinterpret_cast<const In*>(p.beta) + (size_t)bh * T;

    // P above the diagonal blocks is structurally zero: clear it once.
    for (int e = tid; e < C * C; e += 256) {
        int r = e / C, s = e % C;
        if ((s >> 4) > (r >> 4)) Pm[r * L::LDT + s] = (E)0.f;
    }

    // Initial state tile -> registers (fp32).
    f32x4 Macc[SM];
#pragma unroll
    for (int sl = 0; sl < SM; ++sl) {
        const int t = wave + 4 * sl;
        Macc[sl] = zero4();
        if (t < NTM && p.state_in) {
            const int i0 = (t / NCB) * 16 + 4 * (lane >> 4);
            const int c = (t % NCB) * 16 + (lane & 15);
            const float* sp = p.state_in + (size_t)bh * DK * dv + col0 + c;
#pragma unroll
            for (int i = 0; i < 4; ++i) Macc[sl][i] = sp[(size_t)(i0 + i) * dv];
        }
    }
    // Working scale of the tile (bf16 inputs; the fp32 path keeps 1): a power
    // of two from the largest |M| of the incoming state and the largest |v| of
    // the first chunk in these columns.  The walk runs on M / ws and v / ws
    // (exact) and multiplies outputs and the final state by ws, so the fp16
    // operands formed from M, v and U stay near magnitude 1 whatever the scale
    // of the inputs.
    float ws = 1.f;
    if constexpr (sizeof(In) == 2) {
        float m = 0.f;
#pragma unroll
        for (int sl = 0; sl < SM; ++sl)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(Macc[sl][i]));
        const int n0 = min(C, T);
        for (int it = tid; it < C * VPRV; it += 256) {
            const int r = it / VPRV, part = it % VPRV;
            if (r < n0) {
                const uint4 rv4 = *reinterpret_cast<const uint4*>(vg + (size_t)tm(r) * dv + col0 + part * EPV);
                m = fmaxf(m, maxabs8_bf16(rv4));
            }
        }
        m = wave_max(m);
        if (lane == 0) v_red[wave] = m;
        __syncthreads();
        ws = pow2_scale(fmaxf(fmaxf(v_red[0], v_red[1]), fmaxf(v_red[2], v_red[3])));
    }
    const float wi = 1.f / ws;
    // ... and its operand copy Mt, at the working scale
#pragma unroll
    for (int sl = 0; sl < SM; ++sl) {
        const int t = wave + 4 * sl;
        if (t < NTM) {
            const int i0 = (t / NCB) * 16 + 4 * (lane >> 4);
            const int c = (t % NCB) * 16 + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) Macc[sl][i] *= wi;
            st4(Mt + c * L::LDW + i0, Macc[sl][0], Macc[sl][1], Macc[sl][2], Macc[sl][3]);
        }
    }
    __syncthreads();

    const int nchunks = (T + C - 1) / C;
    for (int ch = 0; ch < nchunks; ++ch) {
        const int t0 = ch * C;
        const int n = min(C, T - t0);

        // ---- phase 1: stage q, k (raw), v^T; per-token norms; decay scan ----
        for (int it = tid; it < C * VPRQ; it += 256) {
            const int r = it / VPRQ, part = it % VPRQ;
            uint4 rq4 = make_uint4(0, 0, 0, 0), rk4 = make_uint4(0, 0, 0, 0);
            if (r < n) {
                rq4 = *reinterpret_cast<const uint4*>(qg + (size_t)tm(t0 + r) * DK + part * EPV);
                rk4 = *reinterpret_cast<const uint4*>(kg + (size_t)tm(t0 + r) * DK + part * EPV);
            }
            const In* qe = reinterpret_cast<const In*>(&rq4);
            const In* ke = reinterpret_cast<const In*>(&rk4);
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                float a = InTraits<In>::to_f32(qe[e]), b = InTraits<In>::to_f32(ke[e]);
                sq += a * a; sk += b * b;
            }
            sq = warp_xor_sum(sq, VPRQ);
            sk = warp_xor_sum(sk, VPRQ);
            const float rq = p.qk_l2norm ? p.scale / sqrtf(sq + p.eps) : p.scale;
            const float rk = p.qk_l2norm ? 1.0f / sqrtf(sk + p.eps) : 1.0f;
            *reinterpret_cast<uint4*>(qraw + r * L::LDQ + part * EPV) = rq4;
            *reinterpret_cast<uint4*>(kraw + r * L::LDQ + part * EPV) = rk4;
#pragma unroll
            for (int e = 0; e < EPV; ++e)
                Kt[(part * EPV + e) * L::LDT + r] = Op::from_f32(InTraits<In>::to_f32(ke[e]) * rk);
            if (part == 0) { v_rq[r] = rq; v_rk[r] = rk; }
        }
        for (int it = tid; it < C * VPRV; it += 256) {
            const int r = it / VPRV, part = it % VPRV;
            uint4 rv4 = make_uint4(0, 0, 0, 0);
            if (r < n)
                rv4 = *reinterpret_cast<const uint4*>(vg + (size_t)tm(t0 + r) * dv + col0 + part * EPV);
            const In* ve = reinterpret_cast<const In*>(&rv4);
#pragma unroll
            for (int e = 0; e < EPV; ++e)
                Vt[(part * EPV + e) * L::LDT + r] = Op::from_f32(InTraits<In>::to_f32(ve[e]) * wi);
        }
        if (wave == 0) {
            constexpr int TPL = C >= 64 ? C / 64 : 1;   // tokens per lane
            float la[TPL], be[TPL];
            float run = 0.f;
#pragma unroll
            for (int e = 0; e < TPL; ++e) {
                const int r = lane * TPL + e;
                // padding rows: alpha = 1, beta = 0
                float l2 = 0.f, b = 0.f;
                if (r < n) {
                    l2 = gate_log2_alpha(InTraits<In>::to_f32(ag[tm(t0 + r)]), p.gate_logits);
                    b = gate_beta(InTraits<In>::to_f32(bg[tm(t0 + r)]), p.gate_logits);
                }
                run += l2;
                la[e] = run;
                be[e] = b;
            }
            float incl = run;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                float y = __shfl_up(incl, o, 64);
                if (lane >= o) incl += y;
            }
            const float excl = incl - run;
            const float gtot = __shfl(incl, 63, 64);
#pragma unroll
            for (int e = 0; e < TPL; ++e) {
                const int r = lane * TPL + e;
                if (r < C) {
                    const float g = excl + la[e];
                    v_g2[r] = g;
                    v_gam[r] = exp2f(g);
                    v_eg[r] = exp2f(gtot - g);
                    v_beta[r] = be[e];
                }
            }
        }
        __syncthreads();

        // ---- phase 2: Gram products (lower triangle) and O = gam .* (Q^ M0) ----
        f32x4 Areg[SG];
#pragma unroll
        for (int sl = 0; sl < SG; ++sl) {
            const int t = wave + 4 * sl;
            Areg[sl] = zero4();
            if (t < NTG) {
                int I = 0;
                while ((I + 1) * (I + 2) / 2 <= t) ++I;
                const int J = t - I * (I + 1) / 2;        // J <= I
                f32x4 kk = zero4(), kq = zero4();
#pragma unroll
                for (int kb = 0; kb < DK; kb += GOp::KSTEP) {
                    auto a = frag_at<GOp>(kraw, L::LDQ, 16 * J, kb, lane);
                    auto bk = frag_at<GOp>(kraw, L::LDQ, 16 * I, kb, lane);
                    auto bq = frag_at<GOp>(qraw, L::LDQ, 16 * I, kb, lane);
                    kk = GOp::mma(a, bk, kk);
                    kq = GOp::mma(a, bq, kq);
                }
                // element i: row s = 16J + 4(lane/16) + i, column r = 16I + lane%16
                const int r = 16 * I + (lane & 15);
                const int s0 = 16 * J + 4 * (lane >> 4);
                const float br = v_beta[r], rkr = v_rk[r], rqr = v_rq[r], gr = v_g2[r];
                float pv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = s0 + i;
                    const float rks = v_rk[s];
                    const float e = (s <= r) ? exp2f(gr - v_g2[s]) : 0.f;
                    Areg[sl][i] = (s < r) ? br * rkr * rks * kk[i] * e : 0.f;
                    pv[i] = rqr * rks * kq[i] * e;
                }
                st4(Pm + r * L::LDT + s0, pv[0], pv[1], pv[2], pv[3]);
            }
        }
        f32x4 Oacc[SO];
#pragma unroll
        for (int sl = 0; sl < SO; ++sl) {
            const int t = wave + 4 * sl;
            Oacc[sl] = zero4();
            if (t < NTO) {
                const int rb = t / NCB, cb = t % NCB;
                const float rq = v_rq[16 * rb + (lane & 15)];
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < DK; kb += Op::KSTEP) {
                    auto a = qhat_frag<In, Op>(qraw, L::LDQ, 16 * rb, kb, lane, rq);
                    auto b = frag_at<Op>(Mt, L::LDW, 16 * cb, kb, lane);
                    acc = Op::mma(a, b, acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) Oacc[sl][i] = acc[i] * v_gam[16 * rb + 4 * (lane >> 4) + i];
            }
        }
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < SG; ++sl) {
            const int t = wave + 4 * sl;
            if (t < NTG) {
                int I = 0;
                while ((I + 1) * (I + 2) / 2 <= t) ++I;
                const int J = t - I * (I + 1) / 2;
                const int r = 16 * I + (lane & 15);
                const int s0 = 16 * J + 4 * (lane >> 4);
                *reinterpret_cast<f32x4*>(Am + r * L::LDA + s0) = Areg[sl];
            }
        }
        __syncthreads();

        // ---- phase 3: X = (I + A)^-1, blocked by 16 ----
        // 3a: diagonal blocks by forward substitution, one lane per column.
        if (tid < NB * 16) {
            const int R0 = (tid >> 4) * 16, j = tid & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = 0.f;
                const float* arow = Am + (R0 + r) * L::LDA + R0;
#pragma unroll
                for (int s = 0; s < r; ++s) acc += arow[s] * x[s];
                x[r] = (r < j) ? 0.f : (r == j ? 1.f : -acc);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Am[(R0 + r) * L::LDA + R0 + j] = x[r];
        }
        __syncthreads();
        // 3b: block rows below: X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj.
        {
            const int a = tid >> 4, bc = tid & 15;
#pragma unroll
            for (int lev = 1; lev < NB; ++lev) {
                float R[NB > 1 ? NB - 1 : 1];
#pragma unroll
                for (int m = 0; m < lev; ++m) {
                    float acc = 0.f;
                    const float* arow = Am + (16 * lev + a) * L::LDA;
                    for (int kk = m; kk < lev; ++kk) {
#pragma unroll
                        for (int c = 0; c < 16; ++c)
                            acc += arow[16 * kk + c] * Am[(16 * kk + c) * L::LDA + 16 * m + bc];
                    }
                    R[m] = acc;
                }
                __syncthreads();
#pragma unroll
                for (int m = 0; m < lev; ++m) Am[(16 * lev + a) * L::LDA + 16 * m + bc] = R[m];
                __syncthreads();
#pragma unroll
                for (int m = 0; m < lev; ++m) {
                    float acc = 0.f;
                    const float* xrow = Am + (16 * lev + a) * L::LDA + 16 * lev;
#pragma unroll
                    for (int c = 0; c < 16; ++c)
                        acc += xrow[c] * Am[(16 * lev + c) * L::LDA + 16 * m + bc];
                    R[m] = -acc;
                }
                __syncthreads();
#pragma unroll
                for (int m = 0; m < lev; ++m) Am[(16 * lev + a) * L::LDA + 16 * m + bc] = R[m];
                __syncthreads();
            }
        }
        // 3c: T = X diag(beta), T2 = T diag(gam), as matrix-core operands.
        {
            constexpr int NQ = C * C / 4 / 256 > 0 ? C * C / 4 / 256 : 1;
            f32x4 xv[NQ];
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
                const int e = (tid + 256 * m) * 4;
                xv[m] = zero4();
                if (e < C * C) {
                    const int r = e / C, s0 = e % C;
                    f32x4 x = *reinterpret_cast<const f32x4*>(Am + r * L::LDA + s0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) xv[m][i] = (s0 + i <= r) ? x[i] : 0.f;
                }
            }
            __syncthreads();
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
                const int e = (tid + 256 * m) * 4;
                if (e < C * C) {
                    const int r = e / C, s0 = e % C;
                    float t[4], t2[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        t[i] = xv[m][i] * v_beta[s0 + i];
                        t2[i] = t[i] * v_gam[s0 + i];
                    }
                    st4(Tm + r * L::LDT + s0, t[0], t[1], t[2], t[3]);
                    st4(T2m + r * L::LDT + s0, t2[0], t2[1], t2[2], t2[3]);
                }
            }
        }
        __syncthreads();

        // ---- phase 4: W^T = K^T T2^T (stored negated), Ut = T V ----
        f32x4 Wreg[SW];
#pragma unroll
        for (int sl = 0; sl < SW; ++sl) {
            const int t = wave + 4 * sl;
            Wreg[sl] = zero4();
            if (t < NTW) {
                const int ib = t / NB, rb = t % NB;
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < C; kb += Op::KSTEP) {
                    auto a = frag_at<Op>(Kt, L::LDT, 16 * ib, kb, lane);
                    auto b = frag_at<Op>(T2m, L::LDT, 16 * rb, kb, lane);
                    acc = Op::mma(a, b, acc);
                }
                Wreg[sl] = acc;
            }
        }
        f32x4 Uacc[SO];
#pragma unroll
        for (int sl = 0; sl < SO; ++sl) {
            const int t = wave + 4 * sl;
            Uacc[sl] = zero4();
            if (t < NTO) {
                const int rb = t / NCB, cb = t % NCB;
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < C; kb += Op::KSTEP) {
                    auto a = frag_at<Op>(Tm, L::LDT, 16 * rb, kb, lane);
                    auto b = frag_at<Op>(Vt, L::LDT, 16 * cb, kb, lane);
                    acc = Op::mma(a, b, acc);
                }
                Uacc[sl] = acc;
            }
        }
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < SW; ++sl) {
            const int t = wave + 4 * sl;
            if (t < NTW) {
                const int ib = t / NB, rb = t % NB;
                const int r = 16 * rb + (lane & 15);
                const int i0 = 16 * ib + 4 * (lane >> 4);
                st4(Wm + r * L::LDW + i0, -Wreg[sl][0], -Wreg[sl][1], -Wreg[sl][2], -Wreg[sl][3]);
            }
        }
        __syncthreads();

        // ---- phase 5: U = Ut - W M0; O += P U; M = gam_C M0 + K^T (eg .* U) ----
#pragma unroll
        for (int sl = 0; sl < SO; ++sl) {
            const int t = wave + 4 * sl;
            if (t < NTO) {
                const int rb = t / NCB, cb = t % NCB;
#pragma unroll
                for (int kb = 0; kb < DK; kb += Op::KSTEP) {
                    auto a = frag_at<Op>(Wm, L::LDW, 16 * rb, kb, lane);
                    auto b = frag_at<Op>(Mt, L::LDW, 16 * cb, kb, lane);
                    Uacc[sl] = Op::mma(a, b, Uacc[sl]);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < SO; ++sl) {
            const int t = wave + 4 * sl;
            if (t < NTO) {
                const int rb = t / NCB, cb = t % NCB;
                const int c = 16 * cb + (lane & 15);
                const int r0 = 16 * rb + 4 * (lane >> 4);
                st4(Ut + c * L::LDT + r0, Uacc[sl][0], Uacc[sl][1], Uacc[sl][2], Uacc[sl][3]);
                st4(U2t + c * L::LDT + r0, Uacc[sl][0] * v_eg[r0], Uacc[sl][1] * v_eg[r0 + 1],
                    Uacc[sl][2] * v_eg[r0 + 2], Uacc[sl][3] * v_eg[r0 + 3]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int sl = 0; sl < SO; ++sl) {
            const int t = wave + 4 * sl;
            if (t < NTO) {
                const int rb = t / NCB, cb = t % NCB;
#pragma unroll
                for (int kb = 0; kb < C; kb += Op::KSTEP) {
                    auto a = frag_at<Op>(Pm, L::LDT, 16 * rb, kb, lane);
                    auto b = frag_at<Op>(Ut, L::LDT, 16 * cb, kb, lane);
                    Oacc[sl] = Op::mma(a, b, Oacc[sl]);
                }
                const int c = col0 + 16 * cb + (lane & 15);
                const int r0 = 16 * rb + 4 * (lane >> 4);
                float ov[4];
                unsigned oe[4];                                   // element within the head
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = r0 + i;
                    oe[i] = r < n ? (unsigned)(tm(t0 + r) * dv + c) : kOffNone;
                    ov[i] = Oacc[sl][i] * ws;
                    if (p.out_gate && r < n)
                        ov[i] *= InTraits<In>::to_f32(reinterpret_cast<const In*>(p.out_gate)[(size_t)bh * T * dv + oe[i]]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (r0 + i >= n) continue;
                    const size_t o = (size_t)bh * T * dv + oe[i];
                    // accumulating: the fp32 plane is added, the sum rounded once
                    if (p.accumulate) ov[i] += p.acc_src[o];
                    if (p.out_bf16)
                        reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16(ov[i]);
                    else
                        reinterpret_cast<float*>(p.out)[o] = ov[i];
                }
            }
        }
        const float gC = v_gam[C - 1];
#pragma unroll
        for (int sl = 0; sl < SM; ++sl) {
            const int t = wave + 4 * sl;
            if (t < NTM) {
                const int ib = t / NCB, cb = t % NCB;
                f32x4 acc = Macc[sl] * gC;
#pragma unroll
                for (int kb = 0; kb < C; kb += Op::KSTEP) {
                    auto a = frag_at<Op>(Kt, L::LDT, 16 * ib, kb, lane);
                    auto b = frag_at<Op>(U2t, L::LDT, 16 * cb, kb, lane);
                    acc = Op::mma(a, b, acc);
                }
                Macc[sl] = acc;
                const int c = 16 * cb + (lane & 15);
                const int i0 = 16 * ib + 4 * (lane >> 4);
                st4(Mt + c * L::LDW + i0, acc[0], acc[1], acc[2], acc[3]);
            }
        }
        __syncthreads();
    }

    if (p.state_out) {
#pragma unroll
        for (int sl = 0; sl < SM; ++sl) {
            const int t = wave + 4 * sl;
            if (t < NTM) {
                const int i0 = (t / NCB) * 16 + 4 * (lane >> 4);
                const int c = (t % NCB) * 16 + (lane & 15);
                float* sp = p.state_out + (size_t)bh * DK * dv + col0 + c;
#pragma unroll
                for (int i = 0; i < 4; ++i) sp[(size_t)(i0 + i) * dv] = Macc[sl][i] * ws;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launch table
// ---------------------------------------------------------------------------
template <class In, class Op, int DK, int C, int BV>
static hipError_t launch_seq(const FwdArgs& a, int grid, hipStream_t s) {
    static_assert(lds_bytes<In, Op, DK, C, BV>() <= 160 * 1024, "LDS plan exceeds 160 KiB");
    hipLaunchKernelGGL((gdn_fwd_single_kernel<In, Op, DK, C, BV>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <class In, class Op, int DK, int C, int BV>
constexpr bool fits() { return lds_bytes<In, Op, DK, C, BV>() <= 160 * 1024; }

template <class In, class Op, int DK, int C>
static hipError_t pick_bv(const FwdArgs& a, int BV, hipStream_t s) {
    const int bh = a.B * a.H;
    if constexpr (fits<In, Op, DK, C, 16>())
        if (BV == 16) return launch_seq<In, Op, DK, C, 16>(a, bh * (a.dv / 16), s);
    if constexpr (fits<In, Op, DK, C, 32>())
        if (BV == 32) return launch_seq<In, Op, DK, C, 32>(a, bh * (a.dv / 32), s);
    if constexpr (fits<In, Op, DK, C, 64>())
        if (BV == 64) return launch_seq<In, Op, DK, C, 64>(a, bh * (a.dv / 64), s);
    return hipErrorInvalidValue;
}

template <class In, class Op>
static hipError_t pick_dk(const FwdArgs& a, int C, int BV, hipStream_t s) {
    if (C == 128) {
        switch (a.dk) {
        case 32: return pick_bv<In, Op, 32, 128>(a, BV, s);
        case 64: return pick_bv<In, Op, 64, 128>(a, BV, s);
        case 128: return pick_bv<In, Op, 128, 128>(a, BV, s);
        default: return hipErrorInvalidValue;
        }
    }
    if constexpr (sizeof(In) == 4) {
        if (a.dk == 128 && C == 64) return pick_bv<In, Op, 128, 64>(a, BV, s);
        if (a.dk == 128 && C == 32) return pick_bv<In, Op, 128, 32>(a, BV, s);
    }
    return hipErrorInvalidValue;
}

template <class In, class Op, int DK, int C>
static int max_bv_of() {
    if constexpr (fits<In, Op, DK, C, 64>()) return 64;
    if constexpr (fits<In, Op, DK, C, 32>()) return 32;
    if constexpr (fits<In, Op, DK, C, 16>()) return 16;
    return 0;
}

template <class In, class Op, int DK>
static int max_bv_c(int C) {
    if (C == 128) return max_bv_of<In, Op, DK, 128>();
    if constexpr (sizeof(In) == 4 && DK == 128) {
        if (C == 64) return max_bv_of<In, Op, DK, 64>();
        if (C == 32) return max_bv_of<In, Op, DK, 32>();
    }
    return 0;
}

int single_max_bv(int in_f32, int dk, int C) {
    // widest value-column tile whose LDS plan fits one workgroup (0: none)
    switch (dk) {
    case 32: return in_f32 ? max_bv_c<float, OpF32, 32>(C) : max_bv_c<uint16_t, OpF16, 32>(C);
    case 64: return in_f32 ? max_bv_c<float, OpF32, 64>(C) : max_bv_c<uint16_t, OpF16, 64>(C);
    case 128: return in_f32 ? max_bv_c<float, OpF32, 128>(C) : max_bv_c<uint16_t, OpF16, 128>(C);
    default: return 0;
    }
}

hipError_t launch_fwd_single(const FwdArgs& a, int C, int BV, hipStream_t s) {
    if (a.in_f32) return pick_dk<float, OpF32>(a, C, BV, s);
    return pick_dk<uint16_t, OpF16>(a, C, BV, s);
}

}  // namespace gdn
