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

constexpr int al16(int x) { return (x + 15) & ~15; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Compile-time LDS plan.
template <class In, class Op, int DK, int C, int NW>
struct WPlan {
    typedef typename Op::elem E;
    static constexpr int BV = 16 * NW, NB = C / 16, NT = 64 * NW;
    static constexpr int SE = (int)sizeof(E);
    static constexpr int LDC = C + 16 / SE;    // rows of C elements
    static constexpr int LDD = DK + 16 / SE;   // rows of DK elements
    static constexpr int LDV = BV + 16 / SE;   // rows of BV elements
    static constexpr int LDX = 16 + 16 / SE;   // rows of 16 elements
    static constexpr int LDAD = 20;            // fp32 rows of 16 (+4)
    // region R1, phase-disjoint: normalised q^, k^ and v rows (load..P3a) |
    // W (P4..P5) | a folded segment map (before the walk)
    static constexpr int O_QH = 0;
    static constexpr int O_KH = al16(O_QH + C * LDD * SE);
    static constexpr int O_VR = al16(O_KH + C * LDD * SE);
    static constexpr int R1_IN = al16(O_VR + C * LDV * SE);
    static constexpr int R1_W = C * LDD * SE;
    static constexpr int R1_FOLD = DK * LDD * SE;
    static constexpr int SZ_R1 = al16(cmax(R1_IN, cmax(R1_W, R1_FOLD)));
    // triangular-solve scratch (written by the Gram pass, read by the solve)
    static constexpr int O_AOFF = SZ_R1;                                  // A off-diag blocks
    static constexpr int O_TT = al16(O_AOFF + C * LDC * SE);              // T column-major
    static constexpr int O_AD = al16(O_TT + C * LDC * SE);                // A diag blocks^T fp32
    static constexpr int O_XD = al16(O_AD + NB * 16 * LDAD * 4);          // diag inverses
    static constexpr int OFF_KT = al16(O_XD + NB * 16 * LDX * SE);        // K^T  [DK][LDC]
    static constexpr int OFF_P = OFF_KT + al16(DK * LDC * SE);            // P    [C][LDC]
    static constexpr int OFF_T = OFF_P + al16(C * LDC * SE);              // T    [C][LDC]
    static constexpr int OFF_T2 = OFF_T + al16(C * LDC * SE);             // T2   [C][LDC]
    static constexpr int OFF_VEC = OFF_T2 + al16(C * LDC * SE);           // 4 x C floats
    static constexpr int TOTAL = OFF_VEC + al16(4 * C * 4);
};

template <class In, class Op, int DK, int C, int NW>
constexpr bool walk_fits() { return WPlan<In, Op, DK, C, NW>::TOTAL <= 160 * 1024; }

// Four consecutive elements, one store (p is 8-byte aligned for fp16,
// 16-byte aligned for fp32 at every call site).
template <class E>
__device__ __forceinline__ void st4(E* p, float a, float b, float c, float d) {
    if constexpr (sizeof(E) == 2) {
        *reinterpret_cast<f16x4*>(p) = f16x4{(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
    } else {
        *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
    }
}

// 16 bytes of input (8 bf16 or 4 fp32) -> scaled Op elements in LDS, one
// vector store (dst is 16-byte aligned for bf16 -> fp16 and fp32 -> fp32).
template <class In, class E>
__device__ __forceinline__ void put16(E* dst, const uint4& raw, float scale) {
    const In* e = reinterpret_cast<const In*>(&raw);
    if constexpr (sizeof(In) == 2) {
        f16x8 h;
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = (_Float16)(InTraits<In>::to_f32(e[i]) * scale);
        *reinterpret_cast<f16x8*>(dst) = h;
    } else {
        f32x4 f;
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = InTraits<In>::to_f32(e[i]) * scale;
        *reinterpret_cast<f32x4*>(dst) = f;
    }
}

template <class In>
__device__ __forceinline__ float sumsq16(const uint4& raw) {
    const In* e = reinterpret_cast<const In*>(&raw);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16 / (int)sizeof(In); ++i) { const float x = InTraits<In>::to_f32(e[i]); s += x * x; }
    return s;
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
    constexpr int NT = L::NT, BV = L::BV, NB = L::NB;
    constexpr int NTG = NB * (NB + 1) / 2;            // lower-triangle 16x16 Gram tiles
    constexpr int SG = (NTG + NW - 1) / NW;
    constexpr int NDB = DK / 16;                      // 16-row blocks of the state
    constexpr int NTW = NDB * NB;                     // W^T tiles; also K^T blocks
    constexpr int SW = (NTW + NW - 1) / NW;
    constexpr int EPV = 16 / (int)sizeof(In);         // input elements per 16-byte load
    constexpr int VPRQ = DK / EPV;                    // 16-byte loads per q/k row
    constexpr int VPRV = BV / EPV;                    // 16-byte loads per v row of the tile
    constexpr int QV = C * VPRQ, QPT = (QV + NT - 1) / NT;
    constexpr int VV = C * VPRV, VPT = (VV + NT - 1) / NT;
    constexpr int TPL = C >= 64 ? C / 64 : 1;         // decay tokens per lane of wave 0
    constexpr bool LOADQ = !SUMMARY;
    constexpr int KS_D = DK / Op::KSTEP;              // k-steps over DK
    constexpr int KS_C = C / Op::KSTEP;               // k-steps over C

    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    E* Qh = reinterpret_cast<E*>(smem + L::O_QH);      // [C][LDD]  q^ rows
    E* Kh = reinterpret_cast<E*>(smem + L::O_KH);      // [C][LDD]  k^ rows
    E* Vr = reinterpret_cast<E*>(smem + L::O_VR);      // [C][LDV]  v rows of the tile
    E* Aoff = reinterpret_cast<E*>(smem + L::O_AOFF);
    E* Tt = reinterpret_cast<E*>(smem + L::O_TT);
    float* Adt = reinterpret_cast<float*>(smem + L::O_AD);
    E* Xd = reinterpret_cast<E*>(smem + L::O_XD);
    E* Wn = reinterpret_cast<E*>(smem);
    E* Afold = reinterpret_cast<E*>(smem);
    E* Kt = reinterpret_cast<E*>(smem + L::OFF_KT);
    E* Pm = reinterpret_cast<E*>(smem + L::OFF_P);
    E* Tm = reinterpret_cast<E*>(smem + L::OFF_T);
    E* T2m = reinterpret_cast<E*>(smem + L::OFF_T2);
    float* v_g2 = reinterpret_cast<float*>(smem + L::OFF_VEC);
    float* v_gam = v_g2 + C;
    float* v_eg = v_gam + C;
    float* v_beta = v_eg + C;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int lc = lane & 15;          // column (or row) within a 16-wide block
    const int lg = lane >> 4;          // lane group 0..3

    const int T = p.T, dv = p.dv;
    const int nseg = p.nseg;
    const int nsum = nseg - 1;
    // workgroup -> (bh, seg, column tile)
    int bh, seg, ctile, ncol;
    if constexpr (SUMMARY) {
        ncol = (DK + dv) / BV;
        ctile = block_x(p.rev_wg) % ncol;
        const int r = block_x(p.rev_wg) / ncol;
        seg = r % nsum;
        bh = r / nsum;
    } else {
        ncol = dv / BV;
        ctile = block_x(p.rev_wg) % ncol;
        const int r = block_x(p.rev_wg) / ncol;
        seg = r % nseg;
        bh = r / nseg;
    }
    bh = uniform(bh);
    seg = uniform(seg);
    ctile = uniform(ctile);
    const bool ident = SUMMARY && ctile < DK / BV;       // identity columns of A_s
    const int vcol0 = SUMMARY ? (ident ? 0 : (ctile - DK / BV) * BV) : ctile * BV;
    const int mycol = 16 * wave + lc;                    // this lane's column in the tile

    const int nchunks = (T + C - 1) / C;
    const int ch0 = seg * p.seg_chunks;
    const int ch1 = min(nchunks, ch0 + p.seg_chunks);

    // per-head bases; offsets inside a head fit in 32 bits
    const In* qg = reinterpret_cast<const In*>(p.q) + (size_t)bh * T * DK;
    const In* kg = reinterpret_cast<const In*>(p.k) + (size_t)bh * T * DK;
    const In* vg = reinterpret_cast<const In*>(p.v) + (size_t)bh * T * dv + vcol0;
    const In* ag = reinterpret_cast<const In*>(p.alpha) + (size_t)bh * T;
    const In* bg = reinterpret_cast<const In*>(p.beta) + (size_t)bh * T;
    E* summA_bh = reinterpret_cast<E*>(p.summA) + (size_t)bh * nsum * DK * DK;
    float* summB_bh = p.summB + (size_t)bh * nsum * DK * dv;
    constexpr unsigned SI = sizeof(In);
    // buffer resources of this head: rows past T read as zero, stores past T drop
    const rsrc_t rq_ = make_rsrc(qg, (unsigned)T * DK * SI);
    const rsrc_t rk_ = make_rsrc(kg, (unsigned)T * DK * SI);
    const rsrc_t rv_ = make_rsrc(reinterpret_cast<const In*>(p.v) + (size_t)bh * T * dv, (unsigned)T * dv * SI);
    const rsrc_t ra_ = make_rsrc(ag, (unsigned)T * SI);
    const rsrc_t rb_ = make_rsrc(bg, (unsigned)T * SI);
    const unsigned osz = p.out_bf16 ? 2u : 4u;
    const rsrc_t ro_ = make_rsrc(SUMMARY ? nullptr : (const char*)p.out + (size_t)bh * T * dv * osz,
                                 SUMMARY ? 0u : (unsigned)T * dv * osz);
    const bool gated = !SUMMARY && p.out_gate != nullptr;
    const TokMap tm = tok_map(T, p.reverse);             // walk position -> token
    const bool accum = !SUMMARY && p.accumulate;     // fp32 plane added before the store
    const rsrc_t rac_ = make_rsrc(accum ? p.acc_src + (size_t)bh * T * dv : nullptr,
                                  accum ? (unsigned)T * dv * 4u : 0u);
    const rsrc_t rg_ = make_rsrc(gated ? (const char*)p.out_gate + (size_t)bh * T * dv * SI : nullptr,
                                 gated ? (unsigned)T * dv * SI : 0u);

    // Structurally zero parts of the persistent matrices (upper blocks).
    for (int e = tid; e < C * C; e += NT) {
        const int r = e / C, s = e % C;
        if ((s >> 4) > (r >> 4)) {
            Pm[r * L::LDC + s] = (E)0.f;
            Tm[r * L::LDC + s] = (E)0.f;
            T2m[r * L::LDC + s] = (E)0.f;
        }
    }

    // ---------------- working scale of the tile (bf16 inputs) --------------
    // The rule is linear in (v, S): the walk runs on v / ws and S / ws and
    // multiplies outputs and the final state by ws (a power of two, exact),
    // so that the fp16 operands formed from v, S and U stay near magnitude 1
    // whatever the scale of the inputs.  Both passes of a segmented call take
    // the same ws from the same data: the largest |state_in| of the tile's
    // columns and the largest |v| of the sequence's first chunk in them
    // (identity columns keep 1; fp32 inputs, on fp32 products, keep 1).
    float ws = 1.f;
    if constexpr (sizeof(In) == 2) {
        __shared__ float wred[NW];
        float m = 0.f;
        if (!ident) {
            const float* src = SUMMARY ? p.state_in : (nseg > 1 ? (p.state_in ? p.snap : nullptr) : p.state_in);
            if (src) {
                const float* sp = src + (size_t)bh * DK * dv + vcol0 + mycol;
                for (int i = lg; i < DK; i += 4) m = fmaxf(m, fabsf(sp[(unsigned)(i * dv)]));
            }
            for (int e = tid; e < C * BV / 8; e += NT) {
                const int r = e / (BV / 8), part = e % (BV / 8);
                m = fmaxf(m, maxabs8_bf16(buf_load16(rv_, (unsigned)(tm(r) * dv + vcol0 + 8 * part) * 2u)));
            }
        }
        m = wave_max(m);
        if (lane == 0) wred[wave] = m;
        __syncthreads();
        float mm = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) mm = fmaxf(mm, wred[w2]);
        ws = uniform(ident ? 1.f : pow2_scale(mm));
    }
    const float wi = uniform(1.f / ws);

    // ---------------- incoming state: fp32 accumulator tiles --------------
    // Macc[ib] lane (lg, lc): rows 16 ib + 4 lg + i, column mycol
    f32x4 Macc[NDB];
#pragma unroll
    for (int ib = 0; ib < NDB; ++ib) Macc[ib] = zero4();
    if constexpr (SUMMARY) {
        if (ident) {
            const int cidx = ctile * BV + mycol;             // identity column index
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                for (int i = 0; i < 4; ++i) Macc[ib][i] = (16 * ib + 4 * lg + i == cidx) ? 1.f : 0.f;
        } else if (seg == 0 && p.snap && p.state_in) {
            // snapshot of the incoming state for the main pass (state_in may alias state_out)
            const float* sp = p.state_in + (size_t)bh * DK * dv + vcol0 + mycol;
            float* dp = p.snap + (size_t)bh * DK * dv + vcol0 + mycol;
            for (int i = lg; i < DK; i += 4) dp[i * dv] = sp[i * dv];
        }
    } else {
        const float* sinp = nseg > 1 ? (p.state_in ? p.snap : nullptr) : p.state_in;
        if (sinp) {
            const float* sp = sinp + (size_t)bh * DK * dv + vcol0;
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                for (int i = 0; i < 4; ++i) Macc[ib][i] = sp[(unsigned)((16 * ib + 4 * lg + i) * dv + mycol)] * wi;
        }
        // fold the maps of the preceding segments (in units of ws): M <- A_s M + B_s.  The next
        // map is loaded into registers while the current one is applied.
        constexpr int AV = DK * DK * (int)sizeof(E) / 16;      // 16-byte pieces of A_s
        constexpr int APT = (AV + NT - 1) / NT;
        uint4 apf[APT];
        f32x4 bpf[NDB];
        auto fold_load = [&](int s2) {
            const uint4* Ag = reinterpret_cast<const uint4*>(summA_bh + (size_t)s2 * DK * DK);
#pragma unroll
            for (int it = 0; it < APT; ++it) {
                const int idx = tid + NT * it;
                if (idx < AV) apf[it] = Ag[idx];
            }
            const float* Bg = summB_bh + (size_t)s2 * DK * dv + vcol0 + mycol;
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                for (int i = 0; i < 4; ++i) bpf[ib][i] = Bg[(unsigned)((16 * ib + 4 * lg + i) * dv)];
        };
        if (seg > 0) fold_load(0);
        for (int s2 = 0; s2 < seg; ++s2) {
            __syncthreads();                                  // Afold free
            constexpr int EPR = DK * (int)sizeof(E) / 16;     // pieces per row of A_s
#pragma unroll
            for (int it = 0; it < APT; ++it) {
                const int idx = tid + NT * it;
                if (idx < AV)
                    *reinterpret_cast<uint4*>(Afold + (idx / EPR) * L::LDD + (idx % EPR) * (16 / (int)sizeof(E))) = apf[it];
            }
            f32x4 bcur[NDB];
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib) bcur[ib] = bpf[ib];
            __syncthreads();
            if (s2 + 1 < seg) fold_load(s2 + 1);
            typename Op::frag mB[KS_D];
#pragma unroll
            for (int ks = 0; ks < KS_D; ++ks) mB[ks] = Op::b_acc(Macc, ks);
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib) {
                f32x4 acc = bcur[ib];
#pragma unroll
                for (int ks = 0; ks < KS_D; ++ks)
                    acc = Op::mma(Op::a_acc(Afold, L::LDD, 16 * ib, ks * Op::KSTEP, lane), mB[ks], acc);
                Macc[ib] = acc;
            }
        }
        if (seg > 0) __syncthreads();                         // Afold (region R1) dead
    }

    // ---------------- register prefetch of one chunk ----------------------
    // Buffer loads: rows past T come back as zero, so nothing is clamped and
    // nothing waits on the loads until the next chunk consumes them.
    uint4 pq[LOADQ ? QPT : 1], pk[QPT], pv[VPT];
    In pa[TPL], pb[TPL];
    auto prefetch = [&](int ch) {
        const int t0 = ch * C;
#pragma unroll
        for (int it = 0; it < QPT; ++it) {
            const int idx = tid + NT * it;
            const int r = idx / VPRQ, part = idx % VPRQ;
            const unsigned off = (unsigned)(tm(t0 + r) * DK + part * EPV) * SI;
            pk[it] = buf_load16(rk_, off);
            if constexpr (LOADQ) pq[it] = buf_load16(rq_, off);
        }
        if (!ident) {
#pragma unroll
            for (int it = 0; it < VPT; ++it) {
                const int idx = tid + NT * it;
                const int r = idx / VPRV, part = idx % VPRV;
                pv[it] = buf_load16(rv_, (unsigned)(tm(t0 + r) * dv + vcol0 + part * EPV) * SI);
            }
        }
        if (wave == 0) {
#pragma unroll
            for (int e = 0; e < TPL; ++e) {
                const unsigned off = (unsigned)tm(t0 + lane * TPL + e) * SI;
                if constexpr (sizeof(In) == 2) {
                    pa[e] = buf_load2(ra_, off);
                    pb[e] = buf_load2(rb_, off);
                } else {
                    pa[e] = __builtin_bit_cast(float, buf_load4(ra_, off));
                    pb[e] = __builtin_bit_cast(float, buf_load4(rb_, off));
                }
            }
        }
    };
    if (ch0 < ch1) prefetch(ch0);

    typename Op::frag mB[KS_D];                               // state as B operand
#pragma unroll
    for (int ks = 0; ks < KS_D; ++ks) mB[ks] = Op::b_acc(Macc, ks);

    for (int ch = ch0; ch < ch1; ++ch) {
        const int t0 = ch * C;
        const int n = min(C, T - t0);

        // ---- P1: q^, k^ (normalised) and v rows into LDS; decay scan --------
#pragma unroll
        for (int it = 0; it < QPT; ++it) {
            const int idx = tid + NT * it;
            if (idx < QV) {                           // whole waves in or out
                const int r = idx / VPRQ, part = idx % VPRQ;
                const uint4 kv = pk[it];                  // zero past the end
                const float sk = group_sum<VPRQ>(sumsq16<In>(kv));
                const float rk = p.qk_l2norm ? __builtin_amdgcn_rsqf(sk + p.eps) : 1.0f;
                put16<In>(Kh + r * L::LDD + part * EPV, kv, rk);
                if constexpr (LOADQ) {
                    const uint4 qv = pq[it];
                    const float sq = group_sum<VPRQ>(sumsq16<In>(qv));
                    const float rq = p.qk_l2norm ? p.scale * __builtin_amdgcn_rsqf(sq + p.eps) : p.scale;
                    put16<In>(Qh + r * L::LDD + part * EPV, qv, rq);
                }
            }
        }
        if (!ident) {
#pragma unroll
            for (int it = 0; it < VPT; ++it) {
                const int idx = tid + NT * it;
                if (idx < VV) {
                    const int r = idx / VPRV, part = idx % VPRV;
                    put16<In>(Vr + r * L::LDV + part * EPV, pv[it], wi);
                }
            }
        }
        if (wave == 0) {
            float la[TPL], bb[TPL];
            float run = 0.f;
#pragma unroll
            for (int e = 0; e < TPL; ++e) {
                const int r = lane * TPL + e;
                const bool ok = r < n;
                // padding rows: alpha = 1, beta = 0
                bb[e] = ok ? gate_beta(InTraits<In>::to_f32(pb[e]), p.gate_logits) : 0.f;
                run += ok ? gate_log2_alpha(InTraits<In>::to_f32(pa[e]), p.gate_logits) : 0.f;
                la[e] = run;
            }
            const float incl = wave_prefix_sum(run);
            const float excl = incl - run;
            const float gtot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, incl), 63));
#pragma unroll
            for (int e = 0; e < TPL; ++e) {
                const int r = lane * TPL + e;
                if (r < C) {
                    const float g = excl + la[e];
                    v_g2[r] = g;
                    v_gam[r] = exp2f(g);
                    v_eg[r] = exp2f(gtot - g);
                    v_beta[r] = bb[e];
                }
            }
        }
        __syncthreads();

        // ---- P2: Gram products (lower tiles) -> A (solve scratch), P -------
#pragma unroll
        for (int sl = 0; sl < SG; ++sl) {
            const int t = wave + NW * sl;
            if (t < NTG) {
                int I = 0;
                while ((I + 1) * (I + 2) / 2 <= t) ++I;
                const int J = t - I * (I + 1) / 2;        // J <= I
                typename Op::frag fa[KS_D], fk[KS_D], fq[LOADQ ? KS_D : 1];
#pragma unroll
                for (int ks = 0; ks < KS_D; ++ks) {
                    fa[ks] = frag_at<Op>(Kh, L::LDD, 16 * J, ks * Op::KSTEP, lane);
                    fk[ks] = frag_at<Op>(Kh, L::LDD, 16 * I, ks * Op::KSTEP, lane);
                    if constexpr (LOADQ) fq[ks] = frag_at<Op>(Qh, L::LDD, 16 * I, ks * Op::KSTEP, lane);
                }
                f32x4 kk = zero4(), kq = zero4();
#pragma unroll
                for (int ks = 0; ks < KS_D; ++ks) {
                    kk = Op::mma(fa[ks], fk[ks], kk);
                    if constexpr (LOADQ) kq = Op::mma(fa[ks], fq[ks], kq);
                }
                // element i: row s = 16J + 4 lg + i, column r = 16I + lc
                const int r = 16 * I + lc;
                const int s0 = 16 * J + 4 * lg;
                const float br = v_beta[r], gr = v_g2[r];
                const f32x4 gs = *reinterpret_cast<const f32x4*>(v_g2 + s0);
                float av[4], pv4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = s0 + i;
                    // G_rs = 2^(g_r - g_s) <= 1 for s <= r (clamped: rounding can make it > 0)
                    const float e = __builtin_amdgcn_exp2f(fminf(gr - gs[i], 0.f));
                    av[i] = (s < r) ? br * kk[i] * e : 0.f;
                    if constexpr (!SUMMARY) pv4[i] = (s <= r) ? kq[i] * e : 0.f;
                }
                if constexpr (!SUMMARY) st4(Pm + r * L::LDC + s0, pv4[0], pv4[1], pv4[2], pv4[3]);
                if (I == J) {
                    // diagonal block, stored transposed: Adt[I][s][r] = A[r][s]
#pragma unroll
                    for (int i = 0; i < 4; ++i) Adt[(16 * I + 4 * lg + i) * L::LDAD + lc] = av[i];
                } else {
                    st4(Aoff + r * L::LDC + s0, av[0], av[1], av[2], av[3]);
                }
            }
        }
        __syncthreads();

        // ---- P3a: wave 0 inverts the diagonal 16x16 blocks (T = X diag(beta))
        //      while every wave builds its V operand and O = gam .* (Q^ M0) and
        //      the waves share the K^T transposes --------------------------------
        if (tid < C) {
            // column elimination, one lane per column of a diagonal block
            const int b = tid >> 4, j = tid & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < 15; ++s) {
                // column s of the block: A[16b + r][16b + s], r = 0..15
                const f32x4* col = reinterpret_cast<const f32x4*>(Adt + (16 * b + s) * L::LDAD);
                const f32x4 c0 = col[0], c1 = col[1], c2 = col[2], c3 = col[3];
                const float cv[16] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3],
                                      c2[0], c2[1], c2[2], c2[3], c3[0], c3[1], c3[2], c3[3]};
                const float xs = x[s];
#pragma unroll
                for (int r = s + 1; r < 16; ++r) x[r] -= cv[r] * xs;
            }
            const int c = 16 * b + j;
            const float bc = v_beta[c], gc = v_gam[c];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float t = x[r] * bc;
                Tm[(16 * b + r) * L::LDC + c] = (E)t;
                T2m[(16 * b + r) * L::LDC + c] = (E)(t * gc);
                Xd[(16 * b + r) * L::LDX + j] = (E)x[r];
            }
#pragma unroll
            for (int r = 0; r < 16; r += 4)
                st4(Tt + c * L::LDC + 16 * b + r, x[r] * bc, x[r + 1] * bc, x[r + 2] * bc, x[r + 3] * bc);
        }
        // K^T blocks: Kt[16 ib + c][16 sb + 4 lg + i] = k^[16 sb + 4 lg + i][16 ib + c]
        // (shared by the waves that are not solving; wave 0 solves when C >= 64)
        {
            constexpr int NH = (C >= 64 && NW > 1) ? NW - 1 : NW;        // helper waves
            const int hw = (C >= 64 && NW > 1) ? wave - 1 : wave;
            if (hw >= 0) {
                for (int t = hw; t < NTW; t += NH) {
                    const int ib = t / NB, sb = t % NB;
                    const f32x4 x = transpose16<Op>(Kh + (16 * sb) * L::LDD + 16 * ib, L::LDD, lane);
                    st4(Kt + (16 * ib + lc) * L::LDC + 16 * sb + 4 * lg, x[0], x[1], x[2], x[3]);
                }
            }
        }
        // v rows of this wave's 16 columns in accumulator layout (rows = tokens)
        f32x4 Vacc[NB];
#pragma unroll
        for (int rb = 0; rb < NB; ++rb)
            Vacc[rb] = ident ? zero4() : transpose16<Op>(Vr + (16 * rb) * L::LDV + 16 * wave, L::LDV, lane);
        f32x4 Oacc[NB];
        if constexpr (!SUMMARY) {
            typename Op::frag fq[2][KS_D];
#pragma unroll
            for (int ks = 0; ks < KS_D; ++ks) fq[0][ks] = Op::a_acc(Qh, L::LDD, 0, ks * Op::KSTEP, lane);
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                if (rb + 1 < NB) {
#pragma unroll
                    for (int ks = 0; ks < KS_D; ++ks)
                        fq[(rb + 1) & 1][ks] = Op::a_acc(Qh, L::LDD, 16 * (rb + 1), ks * Op::KSTEP, lane);
                }
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < KS_D; ++ks) acc = Op::mma(fq[rb & 1][ks], mB[ks], acc);
                const f32x4 gm = *reinterpret_cast<const f32x4*>(v_gam + 16 * rb + 4 * lg);
#pragma unroll
                for (int i = 0; i < 4; ++i) Oacc[rb][i] = acc[i] * gm[i];
            }
        }
        __syncthreads();                                   // q^/k^/v rows dead (R1 free)
        // block rows below: T_ij = -X_ii sum_{k=j}^{i-1} A_ik T_kj
#pragma unroll
        for (int lev = 1; lev < NB; ++lev) {
            for (int j = wave; j < lev; j += NW) {
                f32x4 y = zero4();
                for (int k = j; k < lev; ++k)
                    y = mm_k16<Op>(Aoff + (16 * lev) * L::LDC + 16 * k, L::LDC,
                                   Tt + (16 * j) * L::LDC + 16 * k, L::LDC, y, lane);
                // Y (rows = k of the next product) feeds X_ii * Y from registers
                const f32x4 t = mm_k16_acc<Op>(Xd + (16 * lev) * L::LDX, L::LDX, y, zero4(), lane);
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
        {
            typename Op::frag fk[2][KS_C], ft[2][KS_C];
            auto loadw = [&](int buf, int t) {
                const int ib = t / NB, rb = t % NB;
#pragma unroll
                for (int ks = 0; ks < KS_C; ++ks) {
                    fk[buf][ks] = frag_at<Op>(Kt, L::LDC, 16 * ib, ks * Op::KSTEP, lane);
                    ft[buf][ks] = frag_at<Op>(T2m, L::LDC, 16 * rb, ks * Op::KSTEP, lane);
                }
            };
            if (wave < NTW) loadw(0, wave);
#pragma unroll
            for (int sl = 0; sl < SW; ++sl) {
                const int t = wave + NW * sl;
                if (t < NTW) {
                    if (t + NW < NTW) loadw((sl + 1) & 1, t + NW);
                    const int ib = t / NB, rb = t % NB;
                    f32x4 acc = zero4();
#pragma unroll
                    for (int ks = 0; ks < KS_C; ++ks) acc = Op::mma(fk[sl & 1][ks], ft[sl & 1][ks], acc);
                    st4(Wn + (16 * rb + lc) * L::LDD + 16 * ib + 4 * lg, -acc[0], -acc[1], -acc[2], -acc[3]);
                }
            }
        }
        f32x4 Uacc[NB];
        if (!ident) {
            typename Op::frag vB[KS_C];
#pragma unroll
            for (int ks = 0; ks < KS_C; ++ks) vB[ks] = Op::b_acc(Vacc, ks);
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < KS_C; ++ks)
                    acc = Op::mma(Op::a_acc(Tm, L::LDC, 16 * rb, ks * Op::KSTEP, lane), vB[ks], acc);
                Uacc[rb] = acc;
            }
        } else {
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) Uacc[rb] = zero4();
        }
        __syncthreads();                                   // W complete

        // ---- P5 (wave-local, registers): U = Ut - W M0; O += P U;
        //      M = gam_C M0 + K^T (eg .* U).  The next chunk's loads go out first.
        if (ch + 1 < ch1) prefetch(ch + 1);
        {
            typename Op::frag fw[2][KS_D];
#pragma unroll
            for (int ks = 0; ks < KS_D; ++ks) fw[0][ks] = Op::a_acc(Wn, L::LDD, 0, ks * Op::KSTEP, lane);
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                if (rb + 1 < NB) {
#pragma unroll
                    for (int ks = 0; ks < KS_D; ++ks)
                        fw[(rb + 1) & 1][ks] = Op::a_acc(Wn, L::LDD, 16 * (rb + 1), ks * Op::KSTEP, lane);
                }
#pragma unroll
                for (int ks = 0; ks < KS_D; ++ks) Uacc[rb] = Op::mma(fw[rb & 1][ks], mB[ks], Uacc[rb]);
            }
        }
        typename Op::frag uB[KS_C];
        if constexpr (!SUMMARY) {
#pragma unroll
            for (int ks = 0; ks < KS_C; ++ks) uB[ks] = Op::b_acc(Uacc, ks);
            typename Op::frag fp[NB][KS_C];
#pragma unroll
            for (int rb = 0; rb < NB; ++rb)
#pragma unroll
                for (int ks = 0; ks < KS_C; ++ks) fp[rb][ks] = Op::a_acc(Pm, L::LDC, 16 * rb, ks * Op::KSTEP, lane);
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
                for (int ks = 0; ks < KS_C; ++ks) Oacc[rb] = Op::mma(fp[rb][ks], uB[ks], Oacc[rb]);
#pragma unroll
                for (int i = 0; i < 4; ++i) Oacc[rb][i] *= ws;
                // rows past T fall outside the buffer and are dropped
                unsigned oe[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    oe[i] = (unsigned)(tm(t0 + 16 * rb + 4 * lg + i) * dv + vcol0 + mycol);
                if (gated) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) Oacc[rb][i] *= gate_at(rg_, oe[i], SI == 4);
                }
                if (accum) {
                    // accumulating: the fp32 plane is added, the sum rounded once
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Oacc[rb][i] += __builtin_bit_cast(float, buf_load4(rac_, oe[i] * 4u));
                }
                if (p.out_bf16) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        buf_store2(ro_, oe[i] * 2u, __builtin_bit_cast(uint16_t, (__bf16)Oacc[rb][i]));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) buf_store4(ro_, oe[i] * 4u, Oacc[rb][i]);
                }
            }
        }
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            const f32x4 eg = *reinterpret_cast<const f32x4*>(v_eg + 16 * rb + 4 * lg);
#pragma unroll
            for (int i = 0; i < 4; ++i) Uacc[rb][i] *= eg[i];
        }
#pragma unroll
        for (int ks = 0; ks < KS_C; ++ks) uB[ks] = Op::b_acc(Uacc, ks);
        const float gC = v_gam[C - 1];
        {
            typename Op::frag fk[2][KS_C];
#pragma unroll
            for (int ks = 0; ks < KS_C; ++ks) fk[0][ks] = Op::a_acc(Kt, L::LDC, 0, ks * Op::KSTEP, lane);
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib) {
                if (ib + 1 < NDB) {
#pragma unroll
                    for (int ks = 0; ks < KS_C; ++ks)
                        fk[(ib + 1) & 1][ks] = Op::a_acc(Kt, L::LDC, 16 * (ib + 1), ks * Op::KSTEP, lane);
                }
                f32x4 acc = Macc[ib] * gC;
#pragma unroll
                for (int ks = 0; ks < KS_C; ++ks) acc = Op::mma(fk[ib & 1][ks], uB[ks], acc);
                Macc[ib] = acc;
            }
        }
#pragma unroll
        for (int ks = 0; ks < KS_D; ++ks) mB[ks] = Op::b_acc(Macc, ks);
        __syncthreads();                                   // end of chunk: LDS reuse
    }

    // ---------------- results ---------------------------------------------
    if constexpr (SUMMARY) {
        if (ident) {
            // A_s in operand precision, row-major [DK][DK]
            E* dst = summA_bh + (size_t)seg * DK * DK + ctile * BV + mycol;
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(unsigned)((16 * ib + 4 * lg + i) * DK)] = (E)Macc[ib][i];
        } else {
            float* dst = summB_bh + (size_t)seg * DK * dv + vcol0 + mycol;
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(unsigned)((16 * ib + 4 * lg + i) * dv)] = Macc[ib][i];
        }
    } else {
        if (p.state_out && seg == nseg - 1) {
            float* sp = p.state_out + (size_t)bh * DK * dv + vcol0;
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                for (int i = 0; i < 4; ++i) sp[(unsigned)((16 * ib + 4 * lg + i) * dv + mycol)] = Macc[ib][i] * ws;
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
