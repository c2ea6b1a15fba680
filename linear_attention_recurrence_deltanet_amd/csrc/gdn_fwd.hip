// gdn_fwd.hip -- chunked Gated DeltaNet forward on gfx950 (MI355X): the
// segmented chunk walker used for 32- and 64-token chunks.
//
// Recurrence (token-wise gated delta rule; SANA-Streaming, paperpeel page,
// section 2.1 with Gated DeltaNet [35]; the state is carried across streaming
// chunks, section 2.1 and appendix G.6).  With the state stored transposed,
// M = S^T of shape [dk][dv]:
//     u_t = beta_t (v_t - alpha_t M^T k_t),  M <- alpha_t M + k_t u_t^T,
//     o_t = M^T q_t                     (q_t, k_t unit-normalised)
//
// Chunk form (C tokens, incoming state M0, g_r = sum_{s<=r} log alpha_s,
// gam = exp(g), G_rs = exp(g_r - g_s) for r >= s only, so exponents are <= 0):
//     A  = diag(beta) strict_tril(K^ K^T .* G)
//     T  = (I + A)^-1 diag(beta),   T2 = T diag(gam)
//     W  = T2 K^,  Ut = T V,  U = Ut - W M0
//     O  = diag(gam) Q^ M0 + tril(Q^ K^T .* G) U
//     M  = gam_C M0 + K^T diag(exp(g_C - g)) U
// A partial chunk behaves as if padded with alpha = 1, beta = 0, q = k = v = 0.
//
// Work decomposition (section 2.3 "Efficient GDN Kernel" keeps the state on
// chip while q/k/v stream from HBM; here re-planned for 64-wide waves):
//  * a workgroup walks the chunks of one sequence segment for one tile of
//    16*NW value columns; wave w owns 16 of those columns, so the
//    state-dependent chain (U, O, the state update) runs inside one wave with
//    the fp32 state in its registers and no workgroup barrier;
//  * the state-independent part of a chunk (norms, decay scan, Gram products,
//    triangular solve, W and Ut) is shared by the waves through LDS; the next
//    chunk's inputs are prefetched into registers meanwhile;
//  * for few heads the sequence is cut into segments.  Because the map from a
//    segment's incoming state to its outgoing state is affine,
//    M_out = A_s M_in + B_s, a summary pass computes (A_s, B_s) for every
//    segment but the last by running the same walk on identity columns (v = 0,
//    M0 = I) and on the value columns (M0 = 0); the main pass then folds the
//    predecessors' maps into its incoming state and walks its segment.
// Matrix products: Gram products on the raw bf16 inputs with bf16 MFMA (exact
// operands); products with a computed operand in fp16 (11-bit significand)
// with fp32 accumulation; fp32 inputs use fp32 MFMA throughout.
#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

template <class In> struct InTraits;
template <> struct InTraits<uint16_t> {
    typedef OpBF16 Gram;
    __device__ static __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
};
template <> struct InTraits<float> {
    typedef OpF32 Gram;
    __device__ static __forceinline__ float to_f32(float x) { return x; }
};

__device__ __forceinline__ float group_sum(float v, int width) {
    for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

constexpr int al16(int x) { return (x + 15) & ~15; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Compile-time LDS plan.
template <class In, class Op, int DK, int C, int NW>
struct WPlan {
    typedef typename Op::elem E;
    static constexpr int BV = 16 * NW, NB = C / 16, NT = 64 * NW;
    static constexpr int SI = (int)sizeof(In), SE = (int)sizeof(E);
    static constexpr int LDQ = DK + 16 / SI;   // raw q / k rows
    static constexpr int LDC = C + 16 / SE;    // rows of C elements
    static constexpr int LDD = DK + 16 / SE;   // rows of DK elements
    static constexpr int LDX = 16 + 16 / SE;   // rows of 16 elements
    static constexpr int LDAD = 20;            // fp32 rows of 16 (+4)
    // region R1: raw q/k (load..Gram) | solve scratch | W (W..chain) | fold A
    static constexpr int R1_IN = 2 * C * LDQ * SI;
    static constexpr int O_AOFF = 0;
    static constexpr int O_TT = al16(O_AOFF + C * LDC * SE);
    static constexpr int O_AD = al16(O_TT + C * LDC * SE);
    static constexpr int O_XD = al16(O_AD + NB * 16 * LDAD * 4);
    static constexpr int R1_SOLVE = al16(O_XD + NB * 16 * LDX * SE);
    static constexpr int R1_W = C * LDD * SE;
    static constexpr int R1_FOLD = DK * LDD * SE;
    static constexpr int SZ_R1 = al16(cmax(cmax(R1_IN, R1_SOLVE), cmax(R1_W, R1_FOLD)));
    static constexpr int OFF_KT = SZ_R1;                                  // K^T  [DK][LDC]
    static constexpr int OFF_VT = OFF_KT + al16(DK * LDC * SE);           // V^T  [BV][LDC]
    static constexpr int OFF_P = OFF_VT + al16(BV * LDC * SE);            // P    [C][LDC]
    static constexpr int OFF_T = OFF_P + al16(C * LDC * SE);              // T    [C][LDC]
    static constexpr int OFF_T2 = OFF_T + al16(C * LDC * SE);             // T2   [C][LDC]
    static constexpr int OFF_VEC = OFF_T2 + al16(C * LDC * SE);           // 6 x C floats
    static constexpr int OFF_WAVE = OFF_VEC + al16(6 * C * 4);
    // per wave: M operand [16][LDD], U and eg.*U operands [16][LDC], Y [16][LDX]
    static constexpr int W_MOP = 0;
    static constexpr int W_UOP = al16(16 * LDD * SE);
    static constexpr int W_U2OP = W_UOP + al16(16 * LDC * SE);
    static constexpr int W_YS = W_U2OP + al16(16 * LDC * SE);
    static constexpr int W_SIZE = W_YS + al16(16 * LDX * SE);
    static constexpr int TOTAL = OFF_WAVE + NW * W_SIZE;
};

template <class In, class Op, int DK, int C, int NW>
constexpr bool walk_fits() { return WPlan<In, Op, DK, C, NW>::TOTAL <= 160 * 1024; }

template <class E>
__device__ __forceinline__ void st4(E* p, float a, float b, float c, float d) {
    p[0] = (E)a; p[1] = (E)b; p[2] = (E)c; p[3] = (E)d;
}

// Q^ operand fragment from the raw input row, scaled by that row's r_q.
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

}  // namespace

// ---------------------------------------------------------------------------
// The walker.  SUMMARY = false: main pass (outputs, final state).
//              SUMMARY = true : segment summaries (A_s, B_s), no outputs.
// ---------------------------------------------------------------------------
template <class In, class Op, int DK, int C, int NW, bool SUMMARY>
__global__ __launch_bounds__(64 * NW)
void gdn_walk_kernel(WalkArgs p) {
    typedef WPlan<In, Op, DK, C, NW> L;
    typedef typename Op::elem E;
    typedef typename InTraits<In>::Gram GOp;
    constexpr int NT = L::NT, BV = L::BV, NB = L::NB;
    constexpr int NTG = NB * (NB + 1) / 2;            // lower-triangle 16x16 Gram tiles
    constexpr int SG = (NTG + NW - 1) / NW;
    constexpr int NDB = DK / 16;                      // 16-row blocks of the state
    constexpr int NTW = NDB * NB;                     // W^T tiles
    constexpr int SW = (NTW + NW - 1) / NW;
    constexpr int EPV = 16 / (int)sizeof(In);         // input elements per 16-byte load
    constexpr int VPRQ = DK / EPV;                    // 16-byte loads per q/k row
    constexpr int VPRV = BV / EPV;                    // 16-byte loads per v row of the tile
    constexpr int QV = C * VPRQ, QPT = (QV + NT - 1) / NT;
    constexpr int VV = C * VPRV, VPT = (VV + NT - 1) / NT;
    constexpr int TPL = C >= 64 ? C / 64 : 1;         // decay tokens per lane of wave 0
    constexpr bool LOADQ = !SUMMARY;

    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    In* qraw = reinterpret_cast<In*>(smem);
    In* kraw = qraw + C * L::LDQ;
    E* Aoff = reinterpret_cast<E*>(smem + L::O_AOFF);
    E* Tt = reinterpret_cast<E*>(smem + L::O_TT);
    float* Adt = reinterpret_cast<float*>(smem + L::O_AD);
    E* Xd = reinterpret_cast<E*>(smem + L::O_XD);
    E* Wn = reinterpret_cast<E*>(smem);
    E* Afold = reinterpret_cast<E*>(smem);
    E* Kt = reinterpret_cast<E*>(smem + L::OFF_KT);
    E* Vt = reinterpret_cast<E*>(smem + L::OFF_VT);
    E* Pm = reinterpret_cast<E*>(smem + L::OFF_P);
    E* Tm = reinterpret_cast<E*>(smem + L::OFF_T);
    E* T2m = reinterpret_cast<E*>(smem + L::OFF_T2);
    float* v_rq = reinterpret_cast<float*>(smem + L::OFF_VEC);
    float* v_rk = v_rq + C;
    float* v_g2 = v_rk + C;
    float* v_gam = v_g2 + C;
    float* v_eg = v_gam + C;
    float* v_beta = v_eg + C;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lc = lane & 15;          // column (or row) within a 16-wide block
    const int lg = lane >> 4;          // lane group 0..3
    char* wbase = smem + L::OFF_WAVE + wave * L::W_SIZE;
    E* Mop = reinterpret_cast<E*>(wbase + L::W_MOP);     // [16 cols][DK]
    E* Uop = reinterpret_cast<E*>(wbase + L::W_UOP);     // [16 cols][C]
    E* U2op = reinterpret_cast<E*>(wbase + L::W_U2OP);   // [16 cols][C]
    E* Ys = reinterpret_cast<E*>(wbase + L::W_YS);       // [16][16]

    const int T = p.T, dv = p.dv;
    const int nseg = p.nseg;
    const int nsum = nseg - 1;
    // workgroup -> (bh, seg, column tile)
    int bh, seg, ctile, ncol;
    if constexpr (SUMMARY) {
        ncol = (DK + dv) / BV;
        ctile = blockIdx.x % ncol;
        const int r = blockIdx.x / ncol;
        seg = r % nsum;
        bh = r / nsum;
    } else {
        ncol = dv / BV;
        ctile = blockIdx.x % ncol;
        const int r = blockIdx.x / ncol;
        seg = r % nseg;
        bh = r / nseg;
    }
    const bool ident = SUMMARY && ctile < DK / BV;       // identity columns of A_s
    const int vcol0 = SUMMARY ? (ident ? 0 : (ctile - DK / BV) * BV) : ctile * BV;
    const int mycol = 16 * wave + lc;                    // this lane's column in the tile

    const int nchunks = (T + C - 1) / C;
    const int ch0 = seg * p.seg_chunks;
    const int ch1 = min(nchunks, ch0 + p.seg_chunks);

    const In* qg = reinterpret_cast<const In*>(p.q) + (size_t)bh * T * DK;
    const In* kg = reinterpret_cast<const In*>(p.k) + (size_t)bh * T * DK;
    const In* vg = reinterpret_cast<const In*>(p.v) + (size_t)bh * T * dv;
    const In* ag = reinterpret_cast<const In*>(p.alpha) + (size_t)bh * T;
    const In* bg = reinterpret_cast<const In*>(p.beta) + (size_t)bh * T;
    const size_t sstride = (size_t)DK * (DK + dv);      // one segment summary
    float* summ_bh = p.summ + (size_t)bh * nsum * sstride;

    // Structurally zero parts of the persistent matrices (upper blocks).
    for (int e = tid; e < C * C; e += NT) {
        const int r = e / C, s = e % C;
        if ((s >> 4) > (r >> 4)) {
            Pm[r * L::LDC + s] = (E)0.f;
            Tm[r * L::LDC + s] = (E)0.f;
            T2m[r * L::LDC + s] = (E)0.f;
        }
    }

    // ---------------- incoming state (fp32 registers + fp16 operand) ------
    f32x4 Macc[NDB];
#pragma unroll
    for (int ib = 0; ib < NDB; ++ib) Macc[ib] = zero4();
    if constexpr (SUMMARY) {
        if (ident) {
            const int cidx = vcol0 + ctile * BV + mycol;     // identity column index
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                for (int i = 0; i < 4; ++i) Macc[ib][i] = (16 * ib + 4 * lg + i == cidx) ? 1.f : 0.f;
        } else if (seg == 0 && p.snap && p.state_in) {
            // snapshot of the incoming state for the main pass (state_in may alias state_out)
            const float* sp = p.state_in + (size_t)bh * DK * dv + vcol0 + mycol;
            float* dp = p.snap + (size_t)bh * DK * dv + vcol0 + mycol;
            for (int i = lg; i < DK; i += 4) dp[(size_t)i * dv] = sp[(size_t)i * dv];
        }
    } else {
        const float* sinp = nseg > 1 ? (p.state_in ? p.snap : nullptr) : p.state_in;
        if (sinp) {
            const float* sp = sinp + (size_t)bh * DK * dv + vcol0 + mycol;
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                for (int i = 0; i < 4; ++i) Macc[ib][i] = sp[(size_t)(16 * ib + 4 * lg + i) * dv];
        }
    }
#pragma unroll
    for (int ib = 0; ib < NDB; ++ib)
        st4(Mop + lc * L::LDD + 16 * ib + 4 * lg, Macc[ib][0], Macc[ib][1], Macc[ib][2], Macc[ib][3]);

    if constexpr (!SUMMARY) {
        // fold the maps of the preceding segments: M <- A_s M + B_s
        for (int s2 = 0; s2 < seg; ++s2) {
            const float* Ag = summ_bh + (size_t)s2 * sstride;
            __syncthreads();                                  // Afold free
            for (int e = tid * 4; e < DK * DK; e += NT * 4) {
                const int i = e / DK, j = e % DK;
                f32x4 a4 = *reinterpret_cast<const f32x4*>(Ag + (size_t)i * (DK + dv) + j);
                st4(Afold + i * L::LDD + j, a4[0], a4[1], a4[2], a4[3]);
            }
            __syncthreads();
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib) {
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i] = Ag[(size_t)(16 * ib + 4 * lg + i) * (DK + dv) + DK + vcol0 + mycol];
#pragma unroll
                for (int kb = 0; kb < DK; kb += Op::KSTEP)
                    acc = Op::mma(frag_at<Op>(Afold, L::LDD, 16 * ib, kb, lane),
                                  frag_at<Op>(Mop, L::LDD, 0, kb, lane), acc);
                Macc[ib] = acc;
            }
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib)
                st4(Mop + lc * L::LDD + 16 * ib + 4 * lg, Macc[ib][0], Macc[ib][1], Macc[ib][2], Macc[ib][3]);
        }
        if (seg > 0) __syncthreads();                         // Afold (region R1) dead
    }

    // ---------------- register prefetch of one chunk ----------------------
    uint4 pq[LOADQ ? QPT : 1], pk[QPT], pv[VPT];
    float pa[TPL], pb[TPL];
    auto prefetch = [&](int ch) {
        const int t0 = ch * C;
        const int n = min(C, T - t0);
#pragma unroll
        for (int it = 0; it < QPT; ++it) {
            const int idx = tid + NT * it;
            const int r = idx / VPRQ, part = idx % VPRQ;
            const bool ok = idx < QV && r < n;
            const size_t off = (size_t)(t0 + r) * DK + part * EPV;
            pk[it] = ok ? *reinterpret_cast<const uint4*>(kg + off) : make_uint4(0, 0, 0, 0);
            if constexpr (LOADQ)
                pq[it] = ok ? *reinterpret_cast<const uint4*>(qg + off) : make_uint4(0, 0, 0, 0);
        }
        if (!ident) {
#pragma unroll
            for (int it = 0; it < VPT; ++it) {
                const int idx = tid + NT * it;
                const int r = idx / VPRV, part = idx % VPRV;
                const bool ok = idx < VV && r < n;
                pv[it] = ok ? *reinterpret_cast<const uint4*>(vg + (size_t)(t0 + r) * dv + vcol0 + part * EPV)
                            : make_uint4(0, 0, 0, 0);
            }
        }
        if (wave == 0) {
#pragma unroll
            for (int e = 0; e < TPL; ++e) {
                const int r = lane * TPL + e;
                const bool ok = r < n;
                pa[e] = ok ? InTraits<In>::to_f32(ag[t0 + r]) : 1.f;
                pb[e] = ok ? InTraits<In>::to_f32(bg[t0 + r]) : 0.f;
            }
        }
    };
    if (ch0 < ch1) prefetch(ch0);

    for (int ch = ch0; ch < ch1; ++ch) {
        const int t0 = ch * C;
        const int n = min(C, T - t0);

        // ---- P1: staged inputs, norms, K^T, V^T, decay scan; prefetch next ----
#pragma unroll
        for (int it = 0; it < QPT; ++it) {
            const int idx = tid + NT * it;
            if (idx < QV) {                           // whole waves in or out
                const int r = idx / VPRQ, part = idx % VPRQ;
                const In* ke = reinterpret_cast<const In*>(&pk[it]);
                float sk = 0.f, sq = 0.f;
#pragma unroll
                for (int e = 0; e < EPV; ++e) { float b = InTraits<In>::to_f32(ke[e]); sk += b * b; }
                if constexpr (LOADQ) {
                    const In* qe = reinterpret_cast<const In*>(&pq[it]);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) { float a = InTraits<In>::to_f32(qe[e]); sq += a * a; }
                    sq = group_sum(sq, VPRQ);
                    *reinterpret_cast<uint4*>(qraw + r * L::LDQ + part * EPV) = pq[it];
                }
                sk = group_sum(sk, VPRQ);
                const float rk = p.qk_l2norm ? 1.0f / sqrtf(sk + p.eps) : 1.0f;
                *reinterpret_cast<uint4*>(kraw + r * L::LDQ + part * EPV) = pk[it];
#pragma unroll
                for (int e = 0; e < EPV; ++e)
                    Kt[(part * EPV + e) * L::LDC + r] = Op::from_f32(InTraits<In>::to_f32(ke[e]) * rk);
                if (part == 0) {
                    v_rk[r] = rk;
                    if constexpr (LOADQ) v_rq[r] = p.qk_l2norm ? p.scale / sqrtf(sq + p.eps) : p.scale;
                }
            }
        }
        if (!ident) {
#pragma unroll
            for (int it = 0; it < VPT; ++it) {
                const int idx = tid + NT * it;
                if (idx < VV) {
                    const int r = idx / VPRV, part = idx % VPRV;
                    const In* ve = reinterpret_cast<const In*>(&pv[it]);
#pragma unroll
                    for (int e = 0; e < EPV; ++e)
                        Vt[(part * EPV + e) * L::LDC + r] = Op::from_f32(InTraits<In>::to_f32(ve[e]));
                }
            }
        }
        if (wave == 0) {
            float la[TPL];
            float run = 0.f;
#pragma unroll
            for (int e = 0; e < TPL; ++e) {
                const int r = lane * TPL + e;
                // log2(0) would make g_r - g_s undefined; 2^-200 is 0 in fp32 anyway
                run += (r < C) ? fmaxf(log2f(pa[e]), -200.f) : 0.f;
                la[e] = run;
            }
            float incl = run;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(incl, o, 64);
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
                    v_beta[r] = pb[e];
                }
            }
        }
        if (ch + 1 < ch1) prefetch(ch + 1);
        __syncthreads();

        // ---- P2: Gram products (lower tiles); O = gam .* (Q^ M0) -------------
        f32x4 Areg[SG];
#pragma unroll
        for (int sl = 0; sl < SG; ++sl) {
            const int t = wave + NW * sl;
            Areg[sl] = zero4();
            if (t < NTG) {
                int I = 0;
                while ((I + 1) * (I + 2) / 2 <= t) ++I;
                const int J = t - I * (I + 1) / 2;        // J <= I
                f32x4 kk = zero4(), kq = zero4();
#pragma unroll
                for (int kb = 0; kb < DK; kb += GOp::KSTEP) {
                    auto a = frag_at<GOp>(kraw, L::LDQ, 16 * J, kb, lane);
                    kk = GOp::mma(a, frag_at<GOp>(kraw, L::LDQ, 16 * I, kb, lane), kk);
                    if constexpr (!SUMMARY) kq = GOp::mma(a, frag_at<GOp>(qraw, L::LDQ, 16 * I, kb, lane), kq);
                }
                // element i: row s = 16J + 4 lg + i, column r = 16I + lc
                const int r = 16 * I + lc;
                const int s0 = 16 * J + 4 * lg;
                const float br = v_beta[r], rkr = v_rk[r], gr = v_g2[r];
                float pv4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = s0 + i;
                    const float rks = v_rk[s];
                    const float e = (s <= r) ? exp2f(gr - v_g2[s]) : 0.f;
                    Areg[sl][i] = (s < r) ? br * rkr * rks * kk[i] * e : 0.f;
                    if constexpr (!SUMMARY) pv4[i] = v_rq[r] * rks * kq[i] * e;
                }
                if constexpr (!SUMMARY) st4(Pm + r * L::LDC + s0, pv4[0], pv4[1], pv4[2], pv4[3]);
            }
        }
        f32x4 Oacc[NB];
        if constexpr (!SUMMARY) {
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                const float rq = v_rq[16 * rb + lc];
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < DK; kb += Op::KSTEP)
                    acc = Op::mma(qhat_frag<In, Op>(qraw, L::LDQ, 16 * rb, kb, lane, rq),
                                  frag_at<Op>(Mop, L::LDD, 0, kb, lane), acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) Oacc[rb][i] = acc[i] * v_gam[16 * rb + 4 * lg + i];
            }
        }
        __syncthreads();                                   // raw q/k dead: R1 -> solve scratch
#pragma unroll
        for (int sl = 0; sl < SG; ++sl) {
            const int t = wave + NW * sl;
            if (t < NTG) {
                int I = 0;
                while ((I + 1) * (I + 2) / 2 <= t) ++I;
                const int J = t - I * (I + 1) / 2;
                if (I == J) {
                    // diagonal block, stored transposed: Adt[I][s][r] = A[r][s]
#pragma unroll
                    for (int i = 0; i < 4; ++i) Adt[(16 * I + 4 * lg + i) * L::LDAD + lc] = Areg[sl][i];
                } else {
                    st4(Aoff + (16 * I + lc) * L::LDC + 16 * J + 4 * lg,
                        Areg[sl][0], Areg[sl][1], Areg[sl][2], Areg[sl][3]);
                }
            }
        }
        __syncthreads();

        // ---- P3: T = (I + A)^-1 diag(beta) ----------------------------------
        // diagonal 16x16 blocks: column elimination, one lane per column
        if (tid < C) {
            const int b = tid >> 4, j = tid & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < 15; ++s) {
                const float* col = Adt + (16 * b + s) * L::LDAD;   // A[16b + r][16b + s], r = 0..15
                const float xs = x[s];
#pragma unroll
                for (int r = s + 1; r < 16; ++r) x[r] -= col[r] * xs;
            }
            const int c = 16 * b + j;
            const float bc = v_beta[c], gc = v_gam[c];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float t = x[r] * bc;
                Tm[(16 * b + r) * L::LDC + c] = (E)t;
                T2m[(16 * b + r) * L::LDC + c] = (E)(t * gc);
                Tt[c * L::LDC + 16 * b + r] = (E)t;
                Xd[(16 * b + r) * L::LDX + j] = (E)x[r];
            }
        }
        __syncthreads();
        // block rows below: T_ij = -X_ii sum_{k=j}^{i-1} A_ik T_kj
#pragma unroll
        for (int lev = 1; lev < NB; ++lev) {
            for (int j = wave; j < lev; j += NW) {
                f32x4 y = zero4();
                for (int k = j; k < lev; ++k)
                    y = mm_k16<Op>(Aoff + (16 * lev) * L::LDC + 16 * k, L::LDC,
                                   Tt + (16 * j) * L::LDC + 16 * k, L::LDC, y, lane);
                // Y (rows c' = 4 lg + i, column c = lc) -> [c][c'] operand
                st4(Ys + lc * L::LDX + 4 * lg, y[0], y[1], y[2], y[3]);
                f32x4 t = mm_k16<Op>(Xd + (16 * lev) * L::LDX, L::LDX, Ys, L::LDX, zero4(), lane);
                const int c = 16 * j + lc;
                const float gc = v_gam[c];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * lev + 4 * lg + i;
                    Tm[r * L::LDC + c] = (E)(-t[i]);
                    T2m[r * L::LDC + c] = (E)(-t[i] * gc);
                }
                st4(Tt + c * L::LDC + 16 * lev + 4 * lg, -t[0], -t[1], -t[2], -t[3]);
            }
            __syncthreads();
        }

        // ---- P4: W^T = K^T T2^T (stored negated), Ut = T V -----------------
#pragma unroll
        for (int sl = 0; sl < SW; ++sl) {
            const int t = wave + NW * sl;
            if (t < NTW) {
                const int ib = t / NB, rb = t % NB;
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < C; kb += Op::KSTEP)
                    acc = Op::mma(frag_at<Op>(Kt, L::LDC, 16 * ib, kb, lane),
                                  frag_at<Op>(T2m, L::LDC, 16 * rb, kb, lane), acc);
                st4(Wn + (16 * rb + lc) * L::LDD + 16 * ib + 4 * lg, -acc[0], -acc[1], -acc[2], -acc[3]);
            }
        }
        f32x4 Uacc[NB];
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            f32x4 acc = zero4();
            if (!ident) {
#pragma unroll
                for (int kb = 0; kb < C; kb += Op::KSTEP)
                    acc = Op::mma(frag_at<Op>(Tm, L::LDC, 16 * rb, kb, lane),
                                  frag_at<Op>(Vt, L::LDC, 16 * wave, kb, lane), acc);
            }
            Uacc[rb] = acc;
        }
        __syncthreads();                                   // W complete

        // ---- P5 (wave-local): U = Ut - W M0; O += P U; M = gam_C M0 + K^T (eg .* U)
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
            for (int kb = 0; kb < DK; kb += Op::KSTEP)
                Uacc[rb] = Op::mma(frag_at<Op>(Wn, L::LDD, 16 * rb, kb, lane),
                                   frag_at<Op>(Mop, L::LDD, 0, kb, lane), Uacc[rb]);
            const int r0 = 16 * rb + 4 * lg;
            if constexpr (!SUMMARY)
                st4(Uop + lc * L::LDC + r0, Uacc[rb][0], Uacc[rb][1], Uacc[rb][2], Uacc[rb][3]);
            st4(U2op + lc * L::LDC + r0, Uacc[rb][0] * v_eg[r0], Uacc[rb][1] * v_eg[r0 + 1],
                Uacc[rb][2] * v_eg[r0 + 2], Uacc[rb][3] * v_eg[r0 + 3]);
        }
        if constexpr (!SUMMARY) {
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
                for (int kb = 0; kb < C; kb += Op::KSTEP)
                    Oacc[rb] = Op::mma(frag_at<Op>(Pm, L::LDC, 16 * rb, kb, lane),
                                       frag_at<Op>(Uop, L::LDC, 0, kb, lane), Oacc[rb]);
                const int c = vcol0 + mycol;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * rb + 4 * lg + i;
                    if (r < n) {
                        const size_t o = ((size_t)bh * T + t0 + r) * dv + c;
                        if (p.out_bf16)
                            reinterpret_cast<uint16_t*>(p.out)[o] = f32_to_bf16(Oacc[rb][i]);
                        else
                            reinterpret_cast<float*>(p.out)[o] = Oacc[rb][i];
                    }
                }
            }
        }
        const float gC = v_gam[C - 1];
#pragma unroll
        for (int ib = 0; ib < NDB; ++ib) {
            f32x4 acc = Macc[ib] * gC;
#pragma unroll
            for (int kb = 0; kb < C; kb += Op::KSTEP)
                acc = Op::mma(frag_at<Op>(Kt, L::LDC, 16 * ib, kb, lane),
                              frag_at<Op>(U2op, L::LDC, 0, kb, lane), acc);
            Macc[ib] = acc;
            st4(Mop + lc * L::LDD + 16 * ib + 4 * lg, acc[0], acc[1], acc[2], acc[3]);
        }
        __syncthreads();                                   // end of chunk: LDS reuse
    }

    // ---------------- results ---------------------------------------------
    if constexpr (SUMMARY) {
        const int col = ident ? ctile * BV + mycol : DK + vcol0 + mycol;
        float* dst = summ_bh + (size_t)seg * sstride + col;
#pragma unroll
        for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[(size_t)(16 * ib + 4 * lg + i) * (DK + dv)] = Macc[ib][i];
    } else {
        if (p.state_out && seg == nseg - 1) {
            float* sp = p.state_out + (size_t)bh * DK * dv + vcol0 + mycol;
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                for (int i = 0; i < 4; ++i) sp[(size_t)(16 * ib + 4 * lg + i) * dv] = Macc[ib][i];
        }
    }
}

// ---------------------------------------------------------------------------
// Launch table
// ---------------------------------------------------------------------------
namespace {

template <class In, class Op, int DK, int C, int NW>
hipError_t launch_walk(const WalkArgs& a, hipStream_t s) {
    static_assert(walk_fits<In, Op, DK, C, NW>(), "LDS plan exceeds 160 KiB");
    const int bh = a.B * a.H;
    if (a.nseg > 1) {
        const int grid = bh * (a.nseg - 1) * ((DK + a.dv) / (16 * NW));
        hipLaunchKernelGGL((gdn_walk_kernel<In, Op, DK, C, NW, true>), dim3(grid), dim3(64 * NW), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int grid = bh * a.nseg * (a.dv / (16 * NW));
    hipLaunchKernelGGL((gdn_walk_kernel<In, Op, DK, C, NW, false>), dim3(grid), dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

template <class In, class Op, int DK, int C>
hipError_t pick_nw(const WalkArgs& a, int nw, hipStream_t s) {
    if constexpr (walk_fits<In, Op, DK, C, 4>())
        if (nw == 4) return launch_walk<In, Op, DK, C, 4>(a, s);
    if constexpr (walk_fits<In, Op, DK, C, 2>())
        if (nw == 2) return launch_walk<In, Op, DK, C, 2>(a, s);
    return hipErrorInvalidValue;
}

template <class In, class Op, int DK>
hipError_t pick_c(const WalkArgs& a, int C, int nw, hipStream_t s) {
    switch (C) {
    case 32: return pick_nw<In, Op, DK, 32>(a, nw, s);
    case 64: return pick_nw<In, Op, DK, 64>(a, nw, s);
    default: return hipErrorInvalidValue;
    }
}

template <class In, class Op, int DK, int C>
int max_nw_of() {
    if constexpr (walk_fits<In, Op, DK, C, 4>()) return 4;
    if constexpr (walk_fits<In, Op, DK, C, 2>()) return 2;
    return 0;
}

template <class In, class Op, int DK>
int max_nw_c(int C) {
    switch (C) {
    case 32: return max_nw_of<In, Op, DK, 32>();
    case 64: return max_nw_of<In, Op, DK, 64>();
    default: return 0;
    }
}

}  // namespace

int walk_max_waves(int in_f32, int dk, int C) {
    switch (dk) {
    case 32: return in_f32 ? max_nw_c<float, OpF32, 32>(C) : max_nw_c<uint16_t, OpF16, 32>(C);
    case 64: return in_f32 ? max_nw_c<float, OpF32, 64>(C) : max_nw_c<uint16_t, OpF16, 64>(C);
    case 128: return in_f32 ? 0 : max_nw_c<uint16_t, OpF16, 128>(C);
    default: return 0;
    }
}

hipError_t launch_walk(const WalkArgs& a, int C, int nw, hipStream_t s) {
    if (a.in_f32) {
        switch (a.dk) {
        case 32: return pick_c<float, OpF32, 32>(a, C, nw, s);
        case 64: return pick_c<float, OpF32, 64>(a, C, nw, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (a.dk) {
    case 32: return pick_c<uint16_t, OpF16, 32>(a, C, nw, s);
    case 64: return pick_c<uint16_t, OpF16, 64>(a, C, nw, s);
    case 128: return pick_c<uint16_t, OpF16, 128>(a, C, nw, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
