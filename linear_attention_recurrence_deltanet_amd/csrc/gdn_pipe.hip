// gdn_pipe.hip -- pipelined chunk walker for bf16 inputs on gfx950 (MI355X).
//
// Same recurrence and chunk form as the segmented walker (SANA-Streaming,
// paperpeel page, section 2.1 with Gated DeltaNet [35]; state carried across
// streaming chunks, section 2.1 and appendix G.6).  With M = S^T [dk][dv],
// g_r = sum_{s<=r} log alpha_s, gam = exp(g), G_rs = exp(g_r - g_s) (r >= s):
//     A  = diag(beta) strict_tril(K^ K^T .* G),  T = (I + A)^-1 diag(beta)
//     U  = T (V - diag(gam) (K^ M0))   (= T V + (-T diag(gam)) (K^ M0))
//     O  = diag(gam) (Q^ M0) + tril(Q^ K^T .* G) U
//     M  = gam_C M0 + K^T diag(exp(g_C - g)) U
//
// Why a second walker.  With one wave per SIMD the segmented walker spends
// most of a chunk waiting: every phase is a short dependent chain.  Here a
// workgroup has eight waves, two per SIMD, with fixed roles:
//  * four "state" waves own 16 value columns each (CT tiles of 16 per wave)
//    and keep those columns of M in fp32 registers for the whole walk;
//  * four "key" waves prepare the state-independent products of the NEXT
//    chunk: norms, decay scan, Gram products, the triangular solve.
// The schedule is skewed so that nothing but a few decay vectors needs two
// LDS copies: the state waves finish chunk c (U, O, state update) while the
// key waves normalise chunk c+1; then the state waves already form
// K^ M and Q^ M of chunk c+1 (the only products that need the new state
// and the raw rows) while the key waves run the Gram products of chunk c+1;
// the triangular solve of c+1 follows, and T V is formed by the state waves
// from T at the start of the next step.  The two roles share each SIMD, so
// the matrix cores, the vector ALUs and LDS are kept busy by different waves.
//
// One step (chunk c done, chunk c+1 prepared), phases separated by barriers:
//   1  state: U = T Y, O, M update                        | key: normalise c+1
//   2  state: K^ M, Q^ M of c+1                           | key: K^ K^T of c+1
//   3  state: Y = V - diag(gam) K^ M of c+1, K^T blocks   | key: diagonal
//                                                           blocks of T
// (the segment walk at d_k = 128 keeps V and K^ M apart and forms
// U = T V + (-T diag gam)(K^ M) with a second triangular operand: there the
// extra phase-3 work of Y measured slower than the saved products)
//   4  state: P = tril(Q^ K^T .* G) of c+1               | key: off-diagonal
//                                                           block columns of T
// Operand precision as in the segmented walker: fp16 operands (11-bit
// significand), fp32 accumulation; the state and the solve stay in fp32.
#include <type_traits>

#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int pal16(int x) { return (x + 15) & ~15; }

// Cache policy of the segment walk's stores of Phi and the partial outputs,
// which the correction pass reads after the kernel boundary: sc0 sc1 (system
// scope) measured 2% faster on the 16-head streaming call than the default
// and neutral elsewhere; non-temporal was slower at d_k = 128.
constexpr int kStageStorePolicy = 1 | 16;
// The same for the outputs (walk and correction pass) and the segment maps:
// written through as produced, so the end of the kernel has little to write
// back before the next launch; measured on MI355X (same box, A/B) -1.6% per
// 16-head rollout call and -4% per streaming call, neutral on the prefill
// and the single-frame step.
constexpr int kOutPolicy = 1 | 16;

// Instantiations of the walker by the features a call uses (EXT).
constexpr int kExtGates = 1, kExtAll = 3;

// Compile-time LDS plan (bytes).
template <int DK, int C, int CT, bool SEG, int NCW_ = 4, int NPW_ = 4>
struct PPlan {
    static constexpr int NCW = NCW_, NPW = NPW_, NW = NCW + NPW, NT = 64 * NW, NPT = 64 * NPW;
    static constexpr int BV = 16 * NCW * CT;
    static constexpr int NB = C / 16, NDB = DK / 16;
    // fp16 row strides of 2 (mod 32) 32-bit words: the 8-byte operand reads
    // of 16 rows then fall into distinct LDS banks (measured on gfx950; the
    // strides of 16-byte-aligned rows conflict two-way or worse)
    static constexpr int LDD = DK + 4;        // rows of DK
    static constexpr int LDC = C + 4;         // rows of C
    static constexpr int LDV = BV + 4;        // rows of BV
    static constexpr int LDX = 20;            // rows of 16
    static constexpr int LDAD = 20;           // fp32 rows of 16 (+4)
    static constexpr int ADB = 16 * LDAD + 16;  // fp32 stride of one diagonal block
    static constexpr int O_QH = 0;                                  // q^   [C][LDD]
    static constexpr int O_KH = O_QH + pal16(C * LDD * 2);          // k^   [C][LDD]
    static constexpr int O_KT = O_KH + pal16(C * LDD * 2);          // k^T  [DK][LDC]
    static constexpr int O_PM = O_KT + pal16(DK * LDC * 2);         // P    [C][LDC]
    // one product U = T Y (YF), or T V + (-T diag(gam)) (K^ M) with the
    // second triangular operand stored too
    static constexpr bool YF = !(SEG && DK == 128);
    static constexpr int O_T2 = O_PM + pal16(C * LDC * 2);          // -T diag(gam) (not YF)
    static constexpr int O_TM = O_T2 + (YF ? 0 : pal16(C * LDC * 2));  // T    [C][LDC]
    static constexpr int O_TT = O_TM + pal16(C * LDC * 2);          // T^T  [C][LDC]
    static constexpr int O_AOFF = O_TT + pal16(C * LDC * 2);        // A off-diagonal
    static constexpr int O_AD = O_AOFF + pal16(C * LDC * 2);        // A diag^T fp32
    static constexpr int O_XD = O_AD + pal16(NB * ADB * 4);         // diag inverses
    static constexpr int O_VR = O_XD + pal16(C * LDX * 2);          // v rows [C][LDV]
    static constexpr int O_VEC = O_VR + pal16(C * LDV * 2);         // 2 x 4 x C fp32
    // segment walk epilogue: the tile's identity columns of the segment map,
    // staged row-major [DK][DK + 4] over the (then dead) start of the plan
    static constexpr int LDAS = DK + 4;
    static constexpr int SZ_AS = SEG ? DK * LDAS * 2 : 0;
    static constexpr int SZ_STEP = O_VEC + 2 * 4 * C * 4;
    static constexpr int TOTAL = SZ_STEP > SZ_AS ? SZ_STEP : SZ_AS;
};

template <int DK, int C, int CT, bool SEG, int NCW = 4, int NPW = 4>
constexpr bool pipe_fits() { return PPlan<DK, C, CT, SEG, NCW, NPW>::TOTAL <= 160 * 1024; }

// Four fp16 values, one 8-byte store (p 8-byte aligned at every call site).
__device__ __forceinline__ void st4h(_Float16* p, float a, float b, float c, float d) {
    *reinterpret_cast<f16x4*>(p) = f16x4{(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
}

// 8 bf16 -> 8 scaled fp16, two 8-byte stores (rows are 8-byte aligned).
__device__ __forceinline__ void put8(_Float16* dst, const uint4& raw, float scale) {
    const uint16_t* e = reinterpret_cast<const uint16_t*>(&raw);
    f16x4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = (_Float16)(bf16_to_f32(e[i]) * scale);
        hi[i] = (_Float16)(bf16_to_f32(e[4 + i]) * scale);
    }
    reinterpret_cast<f16x4*>(dst)[0] = lo;
    reinterpret_cast<f16x4*>(dst)[1] = hi;
}

// Broadcast lane `src` of each group of four lanes (src constant after unrolling).
__device__ __forceinline__ float quad_bcast(float v, int src) {
    switch (src) {
    case 0: return dpp<0x00>(v);
    case 1: return dpp<0x55>(v);
    case 2: return dpp<0xAA>(v);
    default: return dpp<0xFF>(v);
    }
}

// Fragment (row block rb, k-step ks) of a lower-triangular C x C operand in
// accumulator k order.  A k-step spans the column blocks 2ks and 2ks+1; when
// 2ks+1 > rb the second is above the diagonal: zero in registers, not read.
template <int LD>
__device__ __forceinline__ OpF16::frag a_lower(const _Float16* base, int rb, int ks, int lane) {
    if (2 * ks + 1 > rb) {
        const u16x4 lo = *reinterpret_cast<const u16x4*>(base + (16 * rb + (lane & 15)) * LD + 32 * ks + 4 * (lane >> 4));
        return OpF16::frag{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
    }
    return OpF16::a_acc(base, LD, 16 * rb, 32 * ks, lane);
}

// Tile t of P = tril(Q^ K^T .* G) (lower-triangle enumeration: t -> (I, J <= I)).
template <class L>
__device__ __forceinline__ void p_tile(const _Float16* Kh, const _Float16* Qh, _Float16* Pm,
                                       const float* v_g2, int t, int lane) {
    constexpr int KS_D = L::NDB * 16 / 32;
    int I = 0;
    while ((I + 1) * (I + 2) / 2 <= t) ++I;
    const int J = t - I * (I + 1) / 2;
    f32x4 kq = zero4();
#pragma unroll
    for (int ks = 0; ks < KS_D; ++ks)
        kq = OpF16::mma(OpF16::a_acc(Kh, L::LDD, 16 * J, ks * 32, lane),
                        OpF16::a_acc(Qh, L::LDD, 16 * I, ks * 32, lane), kq);
    // element i: row s = 16J + 4 lg + i (key), column r = 16I + lc (query)
    const int r = 16 * I + (lane & 15);
    const int s0 = 16 * J + 4 * (lane >> 4);
    const float gr = v_g2[r];
    const f32x4 gs = *reinterpret_cast<const f32x4*>(v_g2 + s0);
    float pv4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(fminf(gr - gs[i], 0.f));
        pv4[i] = (s0 + i <= r) ? kq[i] * e : 0.f;
    }
    st4h(Pm + r * L::LDC + s0, pv4[0], pv4[1], pv4[2], pv4[3]);
}

// Tile t of A = diag(beta) strict_tril(K^ K^T .* G) (t -> (I, J <= I)): the
// diagonal blocks fp32 and transposed into Adt, the others fp16 into Aoff.
template <class L>
__device__ __forceinline__ void g_tile(const _Float16* Kh, float* Adt, _Float16* Aoff,
                                       const float* v_beta, const float* v_g2, int t, int lane) {
    constexpr int KS_D = L::NDB * 16 / 32;
    typedef OpF16::frag F;
    const int lc = lane & 15, lg = lane >> 4;
    int I = 0;
    while ((I + 1) * (I + 2) / 2 <= t) ++I;
    const int J = t - I * (I + 1) / 2;
    F fa[KS_D], fk[KS_D];
#pragma unroll
    for (int ks = 0; ks < KS_D; ++ks) {
        // both operands in the same (accumulator) k order
        fa[ks] = OpF16::a_acc(Kh, L::LDD, 16 * J, ks * 32, lane);
        fk[ks] = OpF16::a_acc(Kh, L::LDD, 16 * I, ks * 32, lane);
    }
    f32x4 kk = zero4();
#pragma unroll
    for (int ks = 0; ks < KS_D; ++ks) kk = OpF16::mma(fa[ks], fk[ks], kk);
    // element i: row s = 16J + 4 lg + i, column r = 16I + lc
    const int r = 16 * I + lc;
    const int s0 = 16 * J + 4 * lg;
    const float br = v_beta[r], gr = v_g2[r];
    const f32x4 gs = *reinterpret_cast<const f32x4*>(v_g2 + s0);
    float av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int s_ = s0 + i;
        // G_rs = 2^(g_r - g_s) <= 1 for s <= r (clamped: rounding can make it > 0)
        const float e = __builtin_amdgcn_exp2f(fminf(gr - gs[i], 0.f));
        av[i] = (s_ < r) ? br * kk[i] * e : 0.f;
    }
    if (I == J) {
        // diagonal block, stored transposed: Adt[I][s][r] = A[r][s]
#pragma unroll
        for (int i = 0; i < 4; ++i) Adt[I * L::ADB + (4 * lg + i) * L::LDAD + lc] = av[i];
    } else {
        st4h(Aoff + r * L::LDC + s0, av[0], av[1], av[2], av[3]);
    }
}

// Sum of squares of 8 bf16 (bf16 products are exact in fp32).
__device__ __forceinline__ float sumsq8(const uint4& raw) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, raw.x), __builtin_bit_cast(bf2, raw.x), 0.f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, raw.y), __builtin_bit_cast(bf2, raw.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, raw.z), __builtin_bit_cast(bf2, raw.z), s, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, raw.w), __builtin_bit_cast(bf2, raw.w), s, false);
}

// 16x16 transpose of raw bf16 through the matrix core (A * I, exact): lane
// (g, c) receives a[4g+i][c], i < 4.
// `unit` is the bf16 bit pattern of the diagonal: a power of two s gives the
// transpose times s, still exactly (0x3F80 is 1).
__device__ __forceinline__ f32x4 transpose16_bf16(const uint16_t* a, int lda, int lane, short unit = 0x3F80) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    const int lc = lane & 15, lg = lane >> 4;
    const s4 fa = *reinterpret_cast<const s4*>(a + lc * lda + 4 * lg);
    s4 one;
#pragma unroll
    for (int j = 0; j < 4; ++j) one[j] = (4 * lg + j == lc) ? unit : (short)0;
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa, one, zero4(), 0, 0, 0);
}

}  // namespace

// SEG = false: one walk per (head, value tile) over the whole sequence,
//              from state_in; outputs and the final state.
// SEG = true : one walk per (head, segment, tile of [identity | value]
//              columns).  The walk is affine in the segment's incoming state
//              M_in, so it is run once on identity columns (the linear part)
//              and once on value columns from a zero state (the offset):
//                outputs  O = O_val + Phi M_in,   state  M_out = A_s M_in + B_s.
//              Value columns write O_val, identity columns write Phi (their
//              outputs, transposed) and both write the map (A_s, B_s); the
//              correction pass then folds the maps and adds Phi M_in.
// NCW: state waves (4, or 8 with one column tile each: three waves per SIMD
//      instead of two when one state wave would otherwise carry two tiles).
// NPW: key waves (4 or 8).
// EXT: 0 plain; kExtGates: gate logits and the output gate are honoured;
//      kExtAll: also the backward walk, accumulating outputs and the fused
//      bidirectional launch (separate instantiations, so that calls without
//      them run none of that code: the full variant costs 3-8% even unused).
template <int DK, int C, int CT, bool SEG, int NCW = 4, int NPW = 4, int EXT = 0>
__global__ __launch_bounds__(64 * (NCW + NPW)) void gdn_pipe_kernel(WalkArgs p) {
    typedef PPlan<DK, C, CT, SEG, NCW, NPW> L;
    constexpr bool XG = EXT != 0;                    // gates
    constexpr bool XR = EXT == kExtAll;              // reverse, accumulate, fused bidirectional
    typedef OpF16 Op;
    typedef _Float16 E;
    typedef Op::frag F;
    constexpr int NB = L::NB, NDB = L::NDB, BV = L::BV, NPT = L::NPT, NW = L::NW;
    constexpr int NTG = NB * (NB + 1) / 2;           // lower-triangle Gram tiles
    // P tiles: NTS on the state waves (a multiple of their count), the rest
    // (at most two) on the last key waves
    constexpr int NTS = NTG >= 2 * L::NCW ? L::NCW * (NTG / L::NCW) : NTG;
    static_assert(NTG - NTS <= 2 && (NTS % L::NCW == 0 || NTS == NTG), "P tile split");
    static_assert((NDB * NB) % NCW == 0, "K^T blocks per state wave");
    // Gram tiles on state waves: with eight state waves at d_k = 64 their
    // K^ M, Q^ M leave room in phase 2, and the key waves then take two
    // tiles each instead of three
    constexpr int NGS = (NCW == 8 && DK == 64) ? NTG % L::NPW : 0;
    // Block columns of the solve with their operands read ahead into
    // registers (measured faster), except where the registers are at the cap
    // of three waves per SIMD at d_k = 128 (the extra registers spill there).
    constexpr bool COL_AHEAD = !(NCW == 8 && DK == 128);
    constexpr int NTW = NDB * NB;                    // 16x16 blocks of K^T
    constexpr int VPRQ = DK / 8;                     // 16-byte pieces per q/k row
    constexpr int VPRV = BV / 8;                     // 16-byte pieces per v row of the tile
    constexpr int QV = C * VPRQ, QPT = QV / NPT;
    constexpr int VV = C * VPRV, VPT = VV / NPT;
    static_assert(QV % NPT == 0 && VV % NPT == 0, "whole key waves per row set");
    constexpr int TPL = C >= 64 ? C / 64 : 1;        // decay tokens per lane of the scan wave
    constexpr int SCANW = L::NPW - 1;                // key wave of the decay scan (no block column)
    constexpr int KS_D = DK / 32, KS_C = C / 32;     // k-steps over DK and over C

    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    E* Qh = reinterpret_cast<E*>(smem + L::O_QH);
    E* Kh = reinterpret_cast<E*>(smem + L::O_KH);
    E* Kt = reinterpret_cast<E*>(smem + L::O_KT);
    E* Pm = reinterpret_cast<E*>(smem + L::O_PM);
    E* T2n = reinterpret_cast<E*>(smem + L::O_T2);
    E* Tm = reinterpret_cast<E*>(smem + L::O_TM);
    constexpr bool YF = L::YF;
    E* Tt = reinterpret_cast<E*>(smem + L::O_TT);
    E* Aoff = reinterpret_cast<E*>(smem + L::O_AOFF);
    float* Adt = reinterpret_cast<float*>(smem + L::O_AD);
    E* Xd = reinterpret_cast<E*>(smem + L::O_XD);
    uint16_t* Vr = reinterpret_cast<uint16_t*>(smem + L::O_VR);   // raw bf16 v rows
    float* vecs = reinterpret_cast<float*>(smem + L::O_VEC);   // [2][g2 | gam | eg | beta][C]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lc = lane & 15, lg = lane >> 4;
    const bool is_state = wave < NCW;                 // wave-uniform role
    const int kw = wave - NCW;                        // key-wave index
    const int ktid = tid - 64 * NCW;                  // thread index among key waves

    const int T = p.T, dv = p.dv;
    const int nseg = p.nseg;
    // Workgroups are dealt to the 8 XCDs round-robin.  Remap so that
    // consecutive logical indices -- the column tiles and segments of one
    // head -- share an XCD and its L2: they read the same q/k rows at about
    // the same time.
    int wg = block_x(p.rev_wg);
    {
        const int w8 = (int)gridDim.x / 8 * 8;
        if (wg < w8) wg = (wg % 8) * (w8 / 8) + wg / 8;
    }
    // Segment 0 of a plain call walks its value columns from state_in (the
    // true incoming state), so its tiles of identity columns only are not
    // launched: per head, segment 0 has ncol - skip tiles, the others ncol.
    const bool direct = SEG && EXT == 0 && p.seg0_direct;
    int bh, seg, ctile, dir = 0;
    {
        const int ncol = SEG ? (DK + dv) / BV : dv / BV;
        const int skip = direct && DK != dv ? DK / BV : 0;
        const int per = ncol * nseg - skip;
        int i = wg % per;
        bh = wg / per;
        if (i < ncol - skip) {
            seg = 0;
            ctile = skip + i;
        } else {
            i -= ncol - skip;
            seg = 1 + i / ncol;
            ctile = i % ncol;
        }
        // a fused bidirectional launch: both directions of a head adjacent
        if constexpr (SEG && XR) {
            if (p.bidir) {
                dir = bh & 1;
                bh >>= 1;
            }
        }
    }
    bh = uniform(bh);
    seg = uniform(seg);
    ctile = uniform(ctile);
    // this walk is segment 0 of a plain call: outputs and final state direct
    const bool direct0 = direct && seg == 0;
    if constexpr (SEG && XR) dir = uniform(dir);
    // Tile-local columns [vlo, BV) are value columns, global v column =
    // vbase + local; local columns [0, vlo) are identity columns ibase + local.
    // A segment walk with d_k = d_v gives every tile half identity and half
    // value columns (tile t: identity and value columns t BV/2 .. t BV/2 +
    // BV/2 - 1), so that each SIMD pairs an identity wave with a value wave
    // and the tiles of a segment take the same time (pure tiles of 128
    // columns at d = 128 left the value tiles 1.3 us behind, measured on
    // MI355X); other shapes lay [identity | value] out in order.
    int vlo, vbase, ibase = 0;
    if constexpr (SEG) {
        if (DK == dv) {
            vlo = BV / 2;
            ibase = ctile * (BV / 2);
            vbase = ibase - BV / 2;
        } else {
            const int gc0 = ctile * BV;
            vlo = min(BV, max(0, DK - gc0));
            vbase = gc0 - DK;
            ibase = gc0;
        }
    } else {
        vlo = 0;
        vbase = ctile * BV;
    }
    vlo = uniform(vlo);
    ibase = uniform(ibase);

    const int nchunks = (T + C - 1) / C;
    const int ch0 = seg * p.seg_chunks;
    const int ch1 = min(nchunks, ch0 + p.seg_chunks);
    const int nch = max(0, ch1 - ch0);
    // First chunk in walk order.  Direction 1 of a fused bidirectional call
    // walks the padded sequence backward (walk chunk w is chunk
    // nchunks - 1 - w, rows reversed), so its segment `seg` covers the same
    // chunks ch0 .. ch1 - 1 as the forward one, last chunk first; it stores
    // its partial outputs and Phi in token order for the correction pass.
    const int wc0 = dir ? nchunks - ch1 : ch0;
    const float* state_in = dir ? nullptr : p.state_in;     // the backward scan starts at zero

    const uint16_t* qg = reinterpret_cast<const uint16_t*>(p.q) + (size_t)bh * T * DK;
    const uint16_t* kg = reinterpret_cast<const uint16_t*>(p.k) + (size_t)bh * T * DK;
    const uint16_t* vgp = reinterpret_cast<const uint16_t*>(p.v) + (size_t)bh * T * dv;
    const uint16_t* ag = reinterpret_cast<const uint16_t*>(p.alpha) + (size_t)bh * T;
    const uint16_t* bg = reinterpret_cast<const uint16_t*>(p.beta) + (size_t)bh * T;
    const rsrc_t rq_ = make_rsrc(qg, (unsigned)T * DK * 2u);
    const rsrc_t rk_ = make_rsrc(kg, (unsigned)T * DK * 2u);
    const rsrc_t rv_ = make_rsrc(vgp, (unsigned)T * dv * 2u);
    const rsrc_t ra_ = make_rsrc(ag, (unsigned)T * 2u);
    const rsrc_t rb_ = make_rsrc(bg, (unsigned)T * 2u);
    // outputs of the unsegmented walk; a segment walk stages fp16 partial
    // outputs that the correction pass completes
    const unsigned osz = p.out_bf16 ? 2u : 4u;
    const bool final_out = !SEG || direct0;
    const rsrc_t ro_ = make_rsrc(final_out ? (const char*)p.out + (size_t)bh * T * dv * osz : nullptr,
                                 final_out ? (unsigned)T * dv * osz : 0u);
    const bool gated = XG && !SEG && p.out_gate != nullptr;    // a segment walk leaves it to the correction
    const bool logits = XG && p.gate_logits;
    const bool accum = XR && !SEG && p.accumulate;
    // accumulating outputs add fp32 values from a separate plane before the store
    const rsrc_t rac_ = make_rsrc(accum ? p.acc_src + (size_t)bh * T * dv : nullptr,
                                  accum ? (unsigned)T * dv * 4u : 0u);
    // walk position -> token
    const TokMap tm = dir ? tok_map_padded(nchunks * C) : tok_map(T, XR && p.reverse);
    const rsrc_t rg_ = make_rsrc(gated ? (const char*)p.out_gate + (size_t)bh * T * dv * 2 : nullptr,
                                 gated ? (unsigned)T * dv * 2u : 0u);
    // Phi of this segment: [chunk][row block][k-step of 32 columns of d_k][lane] x 8 fp16,
    // an MFMA operand fragment in accumulator k order (16-column blocks 2 ks, 2 ks + 1);
    // partial outputs: [chunk][row block][16 value columns][lane] x 4 fp16
    const rsrc_t rphi_ = make_rsrc(SEG ? reinterpret_cast<E*>(dir ? p.bw.phi : p.phi) +
                                             ((size_t)bh * nseg + seg) * (size_t)p.seg_chunks * C * DK
                                       : nullptr,
                                   SEG ? (unsigned)(p.seg_chunks * C * DK * 2) : 0u);
    const rsrc_t rosg_ = make_rsrc(SEG ? reinterpret_cast<E*>(dir ? p.bw.ostage : p.ostage) +
                                             ((size_t)bh * nseg + seg) * (size_t)p.seg_chunks * C * dv
                                       : nullptr,
                                   SEG ? (unsigned)(p.seg_chunks * C * dv * 2) : 0u);

    // ---------------- state-wave registers ---------------------------------
    // Macc[ct][ib] lane (lg, lc): state rows 16 ib + 4 lg + i of column col0(ct) + lc
    f32x4 Macc[CT][NDB];
    F mB[CT][KS_D];                                   // state as B operand (fp16)
    // (Q^ M)^T = M^T Q^^T of the next chunk: lane (lg, lc) holds row 16 rb + lc,
    // columns col0 + 4 lg + i
    f32x4 QM[CT][NB];
    // Y = V - diag(gam) K^ M of the next chunk as B operand (fp16): one
    // product U = T Y instead of T V + (-T diag(gam)) (K^ M).  Phase 2 leaves
    // K^ M here (fp16), phase 3 replaces it by Y, formed in fp32 (YF), or
    // puts V beside it
    F yB[CT][KS_C];
    F vB[YF ? 1 : CT][KS_C];
    // Working scale of each column tile: the walk runs on M / wsc and v / wsc
    // (a power of two, so exact) and multiplies outputs and state by wsc
    // again; the fp16 operands formed from M, v and U then stay near
    // magnitude 1 whatever the scale of the inputs.  Every walk of a head's
    // 16 value columns (each segment, and the correction pass) takes the
    // same scale, from the same data: the largest |state_in| of the columns
    // and the largest |v| of the sequence's first chunk in them.  Identity
    // columns of a segment walk keep 1.
    float wsc[CT], winv[CT];
    short wunit[CT];                                  // bf16 bits of winv (exact: a power of two)
    // output gate of the next chunk's rows (this lane's row and 4 columns per
    // row block), loaded a step ahead of its use
    uint2 GV[XG && !SEG ? CT : 1][XG && !SEG ? NB : 1];
    uint4 AV[XR && !SEG ? CT : 1][XR && !SEG ? NB : 1];       // values to accumulate onto, likewise
    auto col0 = [&](int ct) { return 16 * (ct * NCW + wave); };
    auto ident = [&](int ct) { return SEG && col0(ct) < vlo; };

    // ---------------- key-wave prefetch registers ---------------------------
    uint4 pq[QPT], pk[QPT], pv[VPT];
    uint16_t pa[TPL], pb[TPL];
    auto prefetch = [&](int ch) {
        const int t0 = ch * C;
#pragma unroll
        for (int it = 0; it < QPT; ++it) {
            const int idx = ktid + NPT * it;
            const int r = idx / VPRQ, part = idx % VPRQ;
            const unsigned off = (unsigned)(tm(t0 + r) * DK + part * 8) * 2u;
            pk[it] = buf_load16(rk_, off);
            pq[it] = buf_load16(rq_, off);
        }
#pragma unroll
        for (int it = 0; it < VPT; ++it) {
            const int idx = ktid + NPT * it;
            const int r = idx / VPRV, part = idx % VPRV;
            // identity columns of a segment tile have no v (left as zero)
            pv[it] = (part * 8 >= vlo) ? buf_load16(rv_, (unsigned)(tm(t0 + r) * dv + vbase + part * 8) * 2u)
                                       : make_uint4(0u, 0u, 0u, 0u);
        }
        if (kw == SCANW) {
#pragma unroll
            for (int e = 0; e < TPL; ++e) {
                const unsigned off = (unsigned)tm(t0 + lane * TPL + e) * 2u;
                pa[e] = buf_load2(ra_, off);
                pb[e] = buf_load2(rb_, off);
            }
        }
    };
    // ---- incoming state of the walk (state waves): identity on identity
    // columns and zero on value columns of a segment walk, else state_in
    auto init_state = [&]() {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int gcol = ibase + col0(ct) + lc;           // identity column of a segment tile
            const int vcol = vbase + col0(ct) + lc;
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib) Macc[ct][ib] = zero4();
            if constexpr (SEG) {
                if (ident(ct)) {
#pragma unroll
                    for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            Macc[ct][ib][i] = (16 * ib + 4 * lg + i == gcol) ? 1.f : 0.f;
                }
            } else {
                if (state_in) {
                    const float* sp = state_in + (size_t)bh * DK * dv + vcol;
#pragma unroll
                    for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            Macc[ct][ib][i] = sp[(unsigned)((16 * ib + 4 * lg + i) * dv)];
                }
            }
        }
    };

    if (!is_state && nch > 0) prefetch(wc0);

    // The two roles run separate loops with the same barrier sequence, so the
    // compiler allocates registers per role (the branch is wave-uniform).
    if (is_state) {
        init_state();
        // The scale of a value tile, from the largest |state_in| of its columns
        // and the largest |v| of the sequence's first chunk in them (two
        // 16-byte pieces per row; rows past the sequence read zero).  A
        // segment walk's value columns start from zero: they read state_in
        // into the accumulators only for its maximum, and segment 0 leaves
        // the correction pass a copy of it at the working scale (state_in may
        // alias state_out, which that pass writes).
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            if constexpr (SEG) {
                if (!ident(ct) && state_in) {
                    const float* sp = state_in + (size_t)bh * DK * dv + vbase + col0(ct) + lc;
#pragma unroll
                    for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                        for (int i = 0; i < 4; ++i) Macc[ct][ib][i] = sp[(unsigned)((16 * ib + 4 * lg + i) * dv)];
                }
            }
            float m = 0.f;
            if (!ident(ct)) {
#pragma unroll
                for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(Macc[ct][ib][i]));
            }
#pragma unroll
            for (int j = 0; j < C / 32; ++j) {
                const int e = lane + 64 * j, r = e >> 1, part = e & 1;
                // the first chunk walked: the last C tokens for direction 1
                // (whose first walk chunk may be mostly padding)
                const int tr = dir ? T - 1 - r : tm(r);
                const uint4 x = buf_load16(rv_, (ident(ct) || tr < 0) ? kOffNone
                                                          : (unsigned)(tr * dv + vbase + col0(ct) + 8 * part) * 2u);
                m = fmaxf(m, maxabs8_bf16(x));
            }
            wsc[ct] = uniform(ident(ct) ? 1.f : pow2_scale(wave_max(m)));
            winv[ct] = uniform(1.f / wsc[ct]);
            wunit[ct] = (short)(__float_as_uint(winv[ct]) >> 16);
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                for (int i = 0; i < 4; ++i) Macc[ct][ib][i] *= winv[ct];
            if constexpr (SEG) {
                if (!ident(ct)) {
                    if (seg == 0) {
                        if (state_in && !direct0) {
                            float* sn = p.snap + (size_t)bh * DK * dv + vbase + col0(ct) + lc;
#pragma unroll
                            for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                                for (int i = 0; i < 4; ++i) sn[(unsigned)((16 * ib + 4 * lg + i) * dv)] = Macc[ct][ib][i];
                        }
                        if (lane == 0)
                            (dir ? p.bw.sscale : p.sscale)[(size_t)bh * (dv / 16) + (vbase + col0(ct)) / 16] = wsc[ct];
                    }
                    // a direct segment 0 keeps state_in (at the working scale)
                    if (!direct0) {
#pragma unroll
                        for (int ib = 0; ib < NDB; ++ib) Macc[ct][ib] = zero4();
                    }
                }
            }
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int ks = 0; ks < KS_D; ++ks) mB[ct][ks] = Op::b_acc(Macc[ct], ks);
        if constexpr (XG && !SEG) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    GV[ct][rb] = make_uint2(0u, 0u);
                    if constexpr (XR) AV[ct][rb] = make_uint4(0u, 0u, 0u, 0u);
                }
        }
        for (int s = 0; s <= nch; ++s) {
            const int pc = wc0 + s;
            const int vb = s & 1;
            if constexpr (XG && !SEG) {
                // the gate loaded last step arrives here on every path, so no
                // later reuse of its registers waits for the output stores
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int rb = 0; rb < NB; ++rb) {
                        asm volatile("" ::"v"(GV[ct][rb].x), "v"(GV[ct][rb].y));
                        if constexpr (XR)
                            asm volatile("" ::"v"(AV[ct][rb].x), "v"(AV[ct][rb].y), "v"(AV[ct][rb].z), "v"(AV[ct][rb].w));
                    }
            }
            // ---- phase 1: finish chunk pc - 1
            if (s > 0) {
                // finish chunk pc - 1 with the products prepared last step
                const int t0 = (pc - 1) * C;
                const float* vg = vecs + (vb ^ 1) * 4 * C;
                const float* v_gam = vg + C;
                const float* v_eg = vg + 2 * C;
                const float gC = v_gam[C - 1];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const bool idt = ident(ct);
                    f32x4 U[NB];
#pragma unroll
                    for (int rb = 0; rb < NB; ++rb) {
                        f32x4 acc = zero4();
                        // T and P are lower triangular: k-steps past row block rb are zero
#pragma unroll
                        for (int ks = 0; ks <= rb / 2; ++ks) {
                            if constexpr (YF) {
                                acc = Op::mma(a_lower<L::LDC>(Tm, rb, ks, lane), yB[ct][ks], acc);
                            } else {
                                if (!idt) acc = Op::mma(a_lower<L::LDC>(Tm, rb, ks, lane), vB[ct][ks], acc);
                                acc = Op::mma(a_lower<L::LDC>(T2n, rb, ks, lane), yB[ct][ks], acc);
                            }
                        }
                        U[rb] = acc;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    {
                        F uB[KS_C];
#pragma unroll
                        for (int ks = 0; ks < KS_C; ++ks) uB[ks] = Op::b_acc(U, ks);
                        // O^T = M^T Q^^T diag(gam) + U^T P^T, tiles of 16 columns x 16 rows;
                        // lane (lg, lc) holds row 16 rb + lc, columns col0 + 4 lg + i
                        // 16-column block: of d_k for identity columns, of d_v for value columns
                        const int cb = ((idt ? ibase : vbase) + col0(ct)) / 16;
                        // chunk within the segment, row block and lane of row lc, in
                        // token order (direction 1 mirrors all three)
                        const int lch = dir ? nch - s : s - 1;
                        const unsigned lrow = (unsigned)(lane ^ (dir ? 15 : 0));
#pragma unroll
                        for (int rb = 0; rb < NB; ++rb) {
                            const int rbs = dir ? NB - 1 - rb : rb;
                            const float gr = v_gam[16 * rb + lc];
                            f32x4 o;
#pragma unroll
                            for (int i = 0; i < 4; ++i) o[i] = QM[ct][rb][i] * gr;
#pragma unroll
                            for (int ks = 0; ks <= rb / 2; ++ks)
                                o = Op::mma(uB[ks], a_lower<L::LDC>(Pm, rb, ks, lane), o);
                            if constexpr (SEG) {
                              if (direct0) {
                                // segment 0 walked from state_in: the value columns'
                                // outputs are final (identity columns of a mixed tile
                                // store nothing); rows past T are dropped
                                if (!idt) {
#pragma unroll
                                    for (int i = 0; i < 4; ++i) o[i] *= wsc[ct];
                                    const unsigned e0 = (unsigned)(tm(t0 + 16 * rb + lc) * dv +
                                                                   vbase + col0(ct) + 4 * lg);
                                    if (p.out_bf16) {
                                        const uint2 w = make_uint2(
                                            (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[0]) |
                                                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[1]) << 16),
                                            (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[2]) |
                                                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[3]) << 16));
                                        buf_store8<kOutPolicy>(ro_, e0 * 2u, w);
                                    } else {
                                        buf_store16<kOutPolicy>(ro_, e0 * 4u, __builtin_bit_cast(uint4, o));
                                    }
                                }
                              } else {
                                const uint2 w = make_uint2(Op::pk2(o[0], o[1]), Op::pk2(o[2], o[3]));
                                // in range by construction: the wave-uniform part of the
                                // offset goes in the scalar operand
                                if (idt) {
                                    // identity columns: Phi, an operand fragment as stored
                                    buf_store8<kStageStorePolicy>(rphi_, lrow * 16u, w,
                                               uniform((lch * C * DK + (rbs * KS_D + cb / 2) * 512 + (cb & 1) * 4) * 2));
                                } else {
                                    // value columns: partial output (zero incoming state)
                                    buf_store8<kStageStorePolicy>(rosg_, lrow * 8u, w,
                                               uniform((lch * C * dv + (rbs * (dv / 16) + cb) * 256) * 2));
                                }
                              }
                            } else {
#pragma unroll
                                for (int i = 0; i < 4; ++i) o[i] *= wsc[ct];
                                // rows past T fall outside the buffer and are dropped
                                const unsigned e0 = (unsigned)(tm(t0 + 16 * rb + lc) * dv +
                                                               vbase + col0(ct) + 4 * lg);
                                if constexpr (XG && !SEG) {
                                    // consumed on every path (1 without a gate): a use under a
                                    // branch leaves the load pending on the other path, and the
                                    // next write of these registers then waits for every
                                    // outstanding store
                                    const uint2 w = GV[ct][rb];
                                    o[0] *= gated ? __builtin_bit_cast(float, w.x << 16) : 1.f;
                                    o[1] *= gated ? __builtin_bit_cast(float, w.x & 0xffff0000u) : 1.f;
                                    o[2] *= gated ? __builtin_bit_cast(float, w.y << 16) : 1.f;
                                    o[3] *= gated ? __builtin_bit_cast(float, w.y & 0xffff0000u) : 1.f;
                                    // accumulating: the plane is added (zeros otherwise), one rounding
                                    if constexpr (XR) add_f32x4(o, AV[ct][rb]);
                                }
                                if (p.out_bf16) {
                                    const uint2 w = make_uint2(
                                        (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[0]) |
                                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[1]) << 16),
                                        (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[2]) |
                                            ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[3]) << 16));
                                    buf_store8<kOutPolicy>(ro_, e0 * 2u, w);
                                } else {
                                    buf_store16<kOutPolicy>(ro_, e0 * 4u, __builtin_bit_cast(uint4, o));
                                }
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
#pragma unroll
                    for (int rb = 0; rb < NB; ++rb) {
                        const f32x4 eg = *reinterpret_cast<const f32x4*>(v_eg + 16 * rb + 4 * lg);
#pragma unroll
                        for (int i = 0; i < 4; ++i) U[rb][i] *= eg[i];
                    }
                    F euB[KS_C];
#pragma unroll
                    for (int ks = 0; ks < KS_C; ++ks) euB[ks] = Op::b_acc(U, ks);
#pragma unroll
                    for (int ib = 0; ib < NDB; ++ib) {
                        f32x4 acc = Macc[ct][ib] * gC;
#pragma unroll
                        for (int ks = 0; ks < KS_C; ++ks)
                            acc = Op::mma(Op::a_acc(Kt, L::LDC, 16 * ib, 32 * ks, lane), euB[ks], acc);
                        Macc[ct][ib] = acc;
                        if (ib % 4 == 3) __builtin_amdgcn_sched_barrier(0);
                    }
#pragma unroll
                    for (int ks = 0; ks < KS_D; ++ks) mB[ct][ks] = Op::b_acc(Macc[ct], ks);
                }
            }
            if (s == nch) break;
            __syncthreads();
            // ---- phase 2: K^ M, Q^ M of chunk pc
            if constexpr (XG && !SEG) {
                // output gate and values to accumulate onto of chunk pc, used
                // when it is finished next step (issued three phases ahead of
                // that, so the wait at the top of the step finds them loaded).
                // Issued whether or not a gate is given (the resource is empty
                // then), so that the wait before its use counts exactly and
                // does not drain the output stores issued in between
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int rb = 0; rb < NB; ++rb) {
                        const unsigned e = (unsigned)(tm(pc * C + 16 * rb + lc) * dv + vbase + col0(ct) + 4 * lg);
                        GV[ct][rb] = buf_load8(rg_, e * 2u);
                        if constexpr (XR) AV[ct][rb] = buf_load16(rac_, e * 4u);
                    }
            }

            // K^ M and Q^ M of chunk pc with the state after chunk pc - 1
            f32x4 KMlo[CT];
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                F fk[KS_D], fq[KS_D];
#pragma unroll
                for (int ks = 0; ks < KS_D; ++ks) {
                    fk[ks] = Op::a_acc(Kh, L::LDD, 16 * rb, 32 * ks, lane);
                    fq[ks] = Op::a_acc(Qh, L::LDD, 16 * rb, 32 * ks, lane);
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    f32x4 km = zero4();
#pragma unroll
                    for (int ks = 0; ks < KS_D; ++ks) km = Op::mma(fk[ks], mB[ct][ks], km);
                    // fp16, in the B operand order of phase 1 (row blocks 2j, 2j+1 -> k-step j)
                    if (rb % 2 == 0)
                        KMlo[ct] = km;
                    else
                        yB[ct][rb / 2] = Op::pack8(KMlo[ct][0], KMlo[ct][1], KMlo[ct][2], KMlo[ct][3],
                                                   km[0], km[1], km[2], km[3]);
                    f32x4 qm = zero4();
#pragma unroll
                    for (int ks = 0; ks < KS_D; ++ks) qm = Op::mma(mB[ct][ks], fq[ks], qm);
                    QM[ct][rb] = qm;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (NGS > 0) {
                if (wave < NGS) {
                    const float* vcur = vecs + vb * 4 * C;
                    g_tile<L>(Kh, Adt, Aoff, vcur + 3 * C, vcur, wave, lane);
                }
            }
            __syncthreads();
            // ---- phase 3: Y = V - diag(gam) K^ M of chunk pc (V tiles transposed on
            // the matrix cores; identity columns have no V): lane (lg, lc) holds
            // rows 16 rb + 4 lg + i of column lc in each
            if constexpr (!YF) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    if (!ident(ct)) {
                        f32x4 Vacc[NB];
#pragma unroll
                        for (int rb = 0; rb < NB; ++rb)
                            Vacc[rb] = transpose16_bf16(Vr + (16 * rb) * L::LDV + col0(ct), L::LDV, lane, wunit[ct]);
#pragma unroll
                        for (int ks = 0; ks < KS_C; ++ks) vB[ct][ks] = Op::b_acc(Vacc, ks);
                    }
                }
            } else {
                const float* v_gam_c = vecs + vb * 4 * C + C;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    f32x4 Y[NB];
#pragma unroll
                    for (int rb = 0; rb < NB; ++rb) {
                        const f32x4 vt = ident(ct) ? zero4()
                                                   : transpose16_bf16(Vr + (16 * rb) * L::LDV + col0(ct), L::LDV,
                                                                      lane, wunit[ct]);
                        const f32x4 gr = *reinterpret_cast<const f32x4*>(v_gam_c + 16 * rb + 4 * lg);
                        const f16x8 km = __builtin_bit_cast(f16x8, yB[ct][rb / 2]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) Y[rb][i] = vt[i] - gr[i] * (float)km[4 * (rb & 1) + i];
                    }
#pragma unroll
                    for (int ks = 0; ks < KS_C; ++ks) yB[ct][ks] = Op::b_acc(Y, ks);
                }
            }
            // The LDS addresses of the K^T blocks and of P derive from the lane
            // index read afresh here (volatile, so not hoisted): formed every
            // step instead of kept across the loop, where at d_k = 128 they
            // would be spilled, and every reload of a spill waits for all
            // outstanding memory operations, the output stores included.
            int lq;
            asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lq));
            // K^T blocks: Kt[16 ib + c][16 sb + 4 lg + i] = k^[16 sb + 4 lg + i][16 ib + c]
#pragma unroll
            for (int u = 0; u < NTW / NCW; ++u) {
                const int t = wave + NCW * u;
                const int ib = t / NB, sb = t % NB;
                const f32x4 x = transpose16<Op>(Kh + (16 * sb) * L::LDD + 16 * ib, L::LDD, lq);
                st4h(Kt + (16 * ib + (lq & 15)) * L::LDC + 16 * sb + 4 * (lq >> 4), x[0], x[1], x[2], x[3]);
            }
            __syncthreads();
            // ---- phase 4: P = tril(Q^ K^T .* G) of chunk pc, needed from the
            // next step on (the key waves solve for T meanwhile; the two key
            // waves with the shortest block columns take the last tiles)
            {
                const float* v_g2 = vecs + vb * 4 * C;
#pragma unroll
                for (int u = 0; u < (NTS + NCW - 1) / NCW; ++u)
                    if (wave + NCW * u < NTS) p_tile<L>(Kh, Qh, Pm, v_g2, wave + NCW * u, lq);
            }
            __syncthreads();
        }
    } else {
        for (int s = 0; s <= nch; ++s) {
            const int pc = wc0 + s;
            const int vb = s & 1;
            // ---- phase 1: normalise chunk pc, decay scan, prefetch pc + 1
            if (s == nch) break;
            // key waves: q^, k^ (normalised) and v rows of chunk pc; decay scan
#pragma unroll
            for (int it = 0; it < QPT; ++it) {
                const int idx = ktid + NPT * it;
                const int r = idx / VPRQ, part = idx % VPRQ;
                const float sk = group_sum<VPRQ>(sumsq8(pk[it]));
                const float rk = p.qk_l2norm ? __builtin_amdgcn_rsqf(sk + p.eps) : 1.0f;
                put8(Kh + r * L::LDD + part * 8, pk[it], rk);
                {
                    const float sq = group_sum<VPRQ>(sumsq8(pq[it]));
                    const float rq = p.qk_l2norm ? p.scale * __builtin_amdgcn_rsqf(sq + p.eps) : p.scale;
                    put8(Qh + r * L::LDD + part * 8, pq[it], rq);
                }
            }
#pragma unroll
            for (int it = 0; it < VPT; ++it) {
                const int idx = ktid + NPT * it;
                const int r = idx / VPRV, part = idx % VPRV;
                uint2* dst = reinterpret_cast<uint2*>(Vr + r * L::LDV + part * 8);
                dst[0] = make_uint2(pv[it].x, pv[it].y);
                dst[1] = make_uint2(pv[it].z, pv[it].w);
            }
            if (kw == SCANW) {
                float* vg = vecs + vb * 4 * C;
                float la[TPL], bb[TPL];
                float run = 0.f;
#pragma unroll
                for (int e = 0; e < TPL; ++e) {
                    const int r = lane * TPL + e;
                    const bool ok = r < C && tm(pc * C + r) < T;
                    // padding rows (past T, at either end of the walk) and lanes past
                    // the chunk: alpha = 1, beta = 0
                    bb[e] = ok ? gate_beta(bf16_to_f32(pb[e]), logits) : 0.f;
                    run += ok ? gate_log2_alpha(bf16_to_f32(pa[e]), logits) : 0.f;
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
                        vg[r] = g;
                        vg[C + r] = exp2f(g);
                        vg[2 * C + r] = exp2f(gtot - g);
                        vg[3 * C + r] = bb[e];
                    }
                }
            }
            if (s + 1 < nch) prefetch(pc + 1);
            __syncthreads();
            const float* vcur = vecs + vb * 4 * C;
            const float* v_g2 = vcur;
            const float* v_gam = vcur + C;
            const float* v_beta = vcur + 3 * C;
            // ---- phase 2: Gram tiles of chunk pc
            // Gram tiles (I, J <= I) of K^ K^T -> A (solve scratch); the first
            // NGS tiles are on state waves
            for (int t = NGS + kw; t < NTG; t += L::NPW) g_tile<L>(Kh, Adt, Aoff, v_beta, v_g2, t, lane);
            __syncthreads();
            // ---- phase 3: diagonal blocks, one per key wave.  X = (I + A_bb)^-1 by
            // elimination down the columns: lane 4 j + q holds rows 4q..4q+3 of
            // column j; the pivot row is broadcast inside the group of four.
            if (kw < NB) {
                const int b = kw;
                const int j = lane >> 2, q = lane & 3;
                f32x4 acol[15];                       // acol[s][i] = A[4q + i][s] (zero for 4q + i <= s)
#pragma unroll
                for (int s_ = 0; s_ < 15; ++s_)
                    acol[s_] = *reinterpret_cast<const f32x4*>(Adt + b * L::ADB + s_ * L::LDAD + 4 * q);
                float x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = (4 * q + i == j) ? 1.f : 0.f;
#pragma unroll
                for (int s_ = 0; s_ < 15; ++s_) {
                    const float xs = quad_bcast(x[s_ & 3], s_ >> 2);   // X[s][j], final
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] -= acol[s_][i] * xs;
                }
                const int c = 16 * b + j;
                const float bc = v_beta[c], gc = v_gam[c];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * b + 4 * q + i;
                    const float t = x[i] * bc;
                    Tm[r * L::LDC + c] = (E)t;
                    if constexpr (!YF) T2n[r * L::LDC + c] = (E)(-t * gc);
                    Xd[r * L::LDX + j] = (E)x[i];
                }
                st4h(Tt + c * L::LDC + 16 * b + 4 * q, x[0] * bc, x[1] * bc, x[2] * bc, x[3] * bc);
            }
            __syncthreads();
            // ---- phase 4: off-diagonal blocks, block column j on key wave j:
            // T_ij = -X_ii sum_{k=j}^{i-1} A_ik T_kj, the T_kj of the column kept
            // in registers, so the column needs no barrier
            if constexpr (COL_AHEAD) {
                // The column's operands (A_ik, X_ii, T_jj) are read before its
                // first store, so the stores do not hold back the reads.
                auto column = [&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    const int c = 16 * j + lc;
                    const float gc = v_gam[c];
                    auto frag16 = [&](const E* base, int ld) {
                        return Op::load16(base + lc * ld + lg * Op::KPER16);
                    };
                    Op::frag16 fA[NB][NB], fX[NB];
                    const Op::frag16 fT = frag16(Tt + (16 * j) * L::LDC + 16 * j, L::LDC);
    #pragma unroll
                    for (int i = j + 1; i < NB; ++i) {
    #pragma unroll
                        for (int k = j; k < i; ++k) fA[i][k] = frag16(Aoff + (16 * i) * L::LDC + 16 * k, L::LDC);
                        fX[i] = frag16(Xd + (16 * i) * L::LDX, L::LDX);
                    }
                    auto asB = [](const f32x4& v) {
                        u16x4 fb;
    #pragma unroll
                        for (int e = 0; e < 4; ++e) fb[e] = __builtin_bit_cast(uint16_t, (E)v[e]);
                        return fb;
                    };
                    Op::frag16 fTc[NB];
    #pragma unroll
                    for (int i = j + 1; i < NB; ++i) {
                        f32x4 y = Op::mma16(fA[i][j], fT, zero4());
    #pragma unroll
                        for (int k = j + 1; k < i; ++k) y = Op::mma16(fA[i][k], fTc[k], y);
                        const f32x4 t = Op::mma16(fX[i], asB(y), zero4());
                        f32x4 tn;
    #pragma unroll
                        for (int ii = 0; ii < 4; ++ii) tn[ii] = -t[ii];
                        fTc[i] = asB(tn);
    #pragma unroll
                        for (int ii = 0; ii < 4; ++ii) {
                            const int r = 16 * i + 4 * lg + ii;
                            Tm[r * L::LDC + c] = (E)tn[ii];
                            if constexpr (!YF) T2n[r * L::LDC + c] = (E)(t[ii] * gc);
                        }
                        st4h(Tt + c * L::LDC + 16 * i + 4 * lg, tn[0], tn[1], tn[2], tn[3]);
                    }
                };
                if constexpr (NB > 1) {
                    if (kw == 0) column(std::integral_constant<int, 0>{});
                }
                if constexpr (NB > 2) {
                    if (kw == 1) column(std::integral_constant<int, 1>{});
                }
                if constexpr (NB > 3) {
                    if (kw == 2) column(std::integral_constant<int, 2>{});
                }
                static_assert(NB <= 4, "block columns");
            } else {
                if (kw < NB - 1) {
                    const int j = kw;
                    const int c = 16 * j + lc;
                    const float gc = v_gam[c];
                    f32x4 Tc[NB];
    #pragma unroll
                    for (int i = 1; i < NB; ++i) {
                        if (i > j) {
                            f32x4 y = mm_k16<Op>(Aoff + (16 * i) * L::LDC + 16 * j, L::LDC,
                                                 Tt + (16 * j) * L::LDC + 16 * j, L::LDC, zero4(), lane);
    #pragma unroll
                            for (int k = 1; k < i; ++k)
                                if (k > j) y = mm_k16_acc<Op>(Aoff + (16 * i) * L::LDC + 16 * k, L::LDC, Tc[k], y, lane);
                            const f32x4 t = mm_k16_acc<Op>(Xd + (16 * i) * L::LDX, L::LDX, y, zero4(), lane);
    #pragma unroll
                            for (int ii = 0; ii < 4; ++ii) {
                                Tc[i][ii] = -t[ii];
                                const int r = 16 * i + 4 * lg + ii;
                                Tm[r * L::LDC + c] = (E)(-t[ii]);
                                if constexpr (!YF) T2n[r * L::LDC + c] = (E)(t[ii] * gc);
                            }
                            st4h(Tt + c * L::LDC + 16 * i + 4 * lg, -t[0], -t[1], -t[2], -t[3]);
                        }
                    }
                }
            }
            if constexpr (NTG > NTS) {
                if (kw >= L::NPW - (NTG - NTS)) p_tile<L>(Kh, Qh, Pm, v_g2, NTS + (L::NPW - 1 - kw), lane);
            }
            __syncthreads();
        }
    }

    // ---------------- results ----------------------------------------------
    if constexpr (SEG) {
        // Segment maps in the order the correction pass consumes them: A_s as
        // MFMA A-operand fragments [ib][ks][lane] x 16 bytes (fp16), B_s in
        // accumulator order [column block of 16][ib][lane] x f32x4.  Each
        // fold operand is then one coalesced 16-byte load per lane.
        E* summA_bh = reinterpret_cast<E*>(dir ? p.bw.summA : p.summA) + (size_t)bh * nseg * DK * DK;
        float* summB_bh = (dir ? p.bw.summB : p.summB) + (size_t)bh * nseg * DK * dv;
        __syncthreads();                                  // both role loops done: LDS free
        E* As = reinterpret_cast<E*>(smem);
        if (is_state) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                if (direct0) {
                    // segment 0 walked from state_in: its final state (at the
                    // working scale) is the state entering segment 1, from which
                    // the correction pass folds; it writes no map
                    if (!ident(ct)) {
                        float* sn = p.snap + (size_t)bh * DK * dv + vbase + col0(ct) + lc;
#pragma unroll
                        for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                            for (int i = 0; i < 4; ++i) sn[(unsigned)((16 * ib + 4 * lg + i) * dv)] = Macc[ct][ib][i];
                    }
                } else if (ident(ct)) {
                    const int c = ibase + col0(ct) + lc;          // identity column = k index
#pragma unroll
                    for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                        for (int i = 0; i < 4; ++i) As[(16 * ib + 4 * lg + i) * L::LDAS + c] = (E)Macc[ct][ib][i];
                } else {
                    // B_s in units of the working scale (written through)
                    const int c16 = (vbase + col0(ct)) / 16;
                    const rsrc_t rb_ = make_rsrc(summB_bh + (size_t)seg * DK * dv, (unsigned)(DK * dv * 4));
#pragma unroll
                    for (int ib = 0; ib < NDB; ++ib)
                        buf_store16<kOutPolicy>(rb_, (unsigned)(((c16 * NDB + ib) * 64 + lane) * 16),
                                                       __builtin_bit_cast(uint4, Macc[ct][ib]));
                }
            }
        }
        __syncthreads();
        const int k0 = ibase;                             // first identity column of the tile
        if (vlo > 0 && !direct0) {
            const int ks0 = k0 / 32, nks = vlo / 32;
            const rsrc_t ra_ = make_rsrc(summA_bh + (size_t)seg * DK * DK, (unsigned)(DK * DK * 2));
            for (int f = wave; f < NDB * nks; f += NW) {
                const int ib = f / nks, ks = ks0 + f % nks;
                const F fr = Op::a_acc(As, L::LDAS, 16 * ib, 32 * ks, lane);
                buf_store16<kOutPolicy>(ra_, (unsigned)(((ib * KS_D + ks) * 64 + lane) * 16),
                                               __builtin_bit_cast(uint4, fr));
            }
        }
    } else {
        // Kept in this shape on purpose: folding the role test into the store
        // condition changed the compiler's block layout and cost 16% on long
        // unsegmented walks (measured on MI355X, same box, A/B).
        if (is_state) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                if (p.state_out && seg == nseg - 1) {
                    float* sp = p.state_out + (size_t)bh * DK * dv + vbase + col0(ct) + lc;
#pragma unroll
                    for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                        for (int i = 0; i < 4; ++i) sp[(unsigned)((16 * ib + 4 * lg + i) * dv)] = Macc[ct][ib][i] * wsc[ct];
                }
            }
        }
    }
}

// Correction pass of a segmented call.  One workgroup of 16 waves per
// (head, segment, 64 value columns).  Wave (cg, rg) = (wave % 4, wave / 4)
// owns value columns 16 cg .. 16 cg + 15 of the tile and, of the state, the
// RB 16-row blocks of row group rg, in fp32 accumulators.  The state entering
// the segment is folded from the copy of state_in through the maps of the
// preceding segments, M <- A_s M + B_s: per map every wave forms its rows
// from A_s (staged once in LDS) and the whole of M, which the waves exchange
// as fp16 operand fragments through LDS -- one barrier and a few MFMAs per
// map.  The segment's outputs then get Phi M added, row block rg of each
// chunk on row group rg (fp32 out, or bf16); the last segment also applies
// its own map for state_out.
// BI (fused bidirectional call): the backward direction's state entering the
// segment is folded the same way, from zero through the maps of the segments
// after this one, last first; each output is the sum of both directions'
// corrected outputs, each in its own working scale, rounded once.
// PL: a plain call (no output gate, no accumulation), whose corrections load
// only Phi and the partial outputs: measured on MI355X (per-workgroup clock
// stamps, same box) the pass ends 1.3 us earlier on the 16-head d = 128
// rollout and 1.2 us on the d = 64 streaming chunk than with the gate and
// accumulation loads issued on empty ranges.  Two correction groups stay in
// flight: four, six and eight were each slower (their loads, issued before
// the fold, delay the map loads the fold waits on).
template <int DK, int C, bool BI, bool PL = false>
__global__ __launch_bounds__(1024) void gdn_pipe_fix_kernel(WalkArgs p) {
    typedef OpF16 Op;
    typedef Op::frag F;
    constexpr int NDB = DK / 16, KS_D = DK / 32, NB = C / 16;
    constexpr int RG = 4, RB = NDB / RG;                // row groups; state row blocks per wave
    constexpr int CPG = RG / NB;                        // chunks per correction group
    constexpr int APC = DK * DK * 2 / 16;               // 16-byte pieces of one A_s
    constexpr int APT = (APC + 1023) / 1024;            // ... per thread
    constexpr int PPG = RG * 16 * DK * 2 / 16;          // 16-byte pieces of Phi per correction group
    // maps in flight (d_k = 128; the column-owner fold at d_k = 64 stages its
    // own): two measured 1.3% faster per rollout call than three (same box),
    // and four would spill
    constexpr int D = DK == 64 ? 4 : 2;
    static_assert(NDB % RG == 0 && RG % NB == 0 && PPG <= 1024 && APC % 512 == 0, "fix layout");
    // d_k = 128: A_s of the map being folded (two copies); d_k = 64: rings of
    // FR maps (A_s and the tile's B_s) staged for the four column owners
    constexpr int FR = 2;                               // maps per staging group (d_k = 64)
    constexpr int BPC = DK * 64 / 4;                    // 16-byte pieces of a map's B_s for 64 columns
    __shared__ uint4 Ast[2][DK == 64 ? 1 : APC];
    __shared__ uint4 As2[2][DK == 64 ? FR * APC : 1];
    __shared__ uint4 Bs2[2][DK == 64 ? FR * BPC : 1];
    __shared__ uint4 Mf[2][KS_D][4][64];                // M as fp16 B fragments [k-step][column group][lane]
    __shared__ uint4 Phs[2][PPG];
    // the backward direction's Phi [2][PPG], staged over the fold buffers,
    // which are free once both folds are done
    static_assert((DK == 64 ? FR * APC : APC) >= 2 * PPG, "backward Phi staging");
    uint4* const Phb = DK == 64 ? &As2[0][0] : &Ast[0][0];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cg = wave & 3, rg = wave >> 2;
    const int lc = lane & 15, lg = lane >> 4;
    const int T = p.T, dv = p.dv, nseg = p.nseg;
    int wg = block_x(p.rev_wg);
    {
        // the segments of one head read the same maps: keep them on one XCD
        const int w8 = (int)gridDim.x / 8 * 8;
        if (wg < w8) wg = (wg % 8) * (w8 / 8) + wg / 8;
    }
    // Segments s0 .. nseg - 1 are corrected (s0 = 1 when segment 0 walked
    // from state_in and wrote its outputs itself); the last nsp of them, whose
    // folds are the longest, by two workgroups each, one per half of their
    // chunks, so that the deepest fold is not followed by a whole segment of
    // corrections.
    const int ntile = dv / 64;
    const int vt = uniform(wg % ntile);
    const int s0 = BI ? 0 : p.seg0_direct;
    const int nsp = BI ? 0 : p.fix_split;
    const int n1 = nseg - s0 - nsp;                     // segments of one workgroup
    const int per = n1 + 2 * nsp;
    int seg, part, nparts;
    {
        int i = (wg / ntile) % per;
        if (i < n1) {
            seg = s0 + i;
            part = 0;
            nparts = 1;
        } else {
            i -= n1;
            seg = s0 + n1 + i / 2;
            part = i % 2;
            nparts = 2;
        }
    }
    seg = uniform(seg);
    part = uniform(part);
    nparts = uniform(nparts);
    const int bh = uniform(wg / ntile / per);
    // state_out: applied by the last segment's workgroup with fewer chunks
    const bool last = seg == nseg - 1 && part == nparts - 1 && p.state_out != nullptr;
    // the state the fold starts from: segment 1's incoming state (written by a
    // direct segment 0), else the copy of state_in (zero without one)
    const bool from_snap = s0 > 0 || p.state_in != nullptr;

    const int col = vt * 64 + 16 * cg + lc;             // value column of this lane
    const int c16 = vt * 4 + cg;                        // its 16-column block
    const int nchunks = (T + C - 1) / C;
    const int ch0 = seg * p.seg_chunks;
    const int ch1 = min(nchunks, ch0 + p.seg_chunks);
    // the chunks this workgroup corrects: [cb, ce) of the segment's [ch0, ch1)
    const int half = (ch1 - ch0 + 1) / 2;
    const int cb = uniform(nparts == 2 && part == 1 ? ch0 + half : ch0);
    const int ce = uniform(nparts == 2 && part == 0 ? min(ch1, ch0 + half) : ch1);
    // segment data of one direction: maps of all segments, this segment's Phi
    // and partial outputs
    auto maps_a = [&](const void* base) {
        return make_rsrc(reinterpret_cast<const _Float16*>(base) + (size_t)bh * nseg * DK * DK,
                         (unsigned)(nseg * DK * DK * 2));
    };
    auto maps_b = [&](const float* base) {
        return make_rsrc(base + (size_t)bh * nseg * DK * dv, (unsigned)(nseg * DK * dv * 4));
    };
    auto seg_phi = [&](const void* base) {
        return make_rsrc(reinterpret_cast<const _Float16*>(base) +
                             ((size_t)bh * nseg + seg) * (size_t)p.seg_chunks * C * DK,
                         (unsigned)(p.seg_chunks * C * DK * 2));
    };
    auto seg_out = [&](const void* base) {
        return make_rsrc(reinterpret_cast<const _Float16*>(base) +
                             ((size_t)bh * nseg + seg) * (size_t)p.seg_chunks * C * dv,
                         (unsigned)(p.seg_chunks * C * dv * 2));
    };
    const rsrc_t rA = maps_a(p.summA), rB = maps_b(p.summB), rP = seg_phi(p.phi), rO = seg_out(p.ostage);
    const rsrc_t rAb = BI ? maps_a(p.bw.summA) : make_rsrc(nullptr, 0u);
    const rsrc_t rBb = BI ? maps_b(p.bw.summB) : make_rsrc(nullptr, 0u);
    const rsrc_t rPb = BI ? seg_phi(p.bw.phi) : make_rsrc(nullptr, 0u);
    const rsrc_t rOb = BI ? seg_out(p.bw.ostage) : make_rsrc(nullptr, 0u);
    const rsrc_t rW = make_rsrc((const char*)p.out + (size_t)bh * T * dv * (p.out_bf16 ? 2 : 4),
                                (unsigned)T * dv * (p.out_bf16 ? 2u : 4u));
    const bool gated = p.out_gate != nullptr;
    const rsrc_t rG = make_rsrc(gated ? (const char*)p.out_gate + (size_t)bh * T * dv * 2 : nullptr,
                                gated ? (unsigned)T * dv * 2u : 0u);
    const int col4 = vt * 64 + 16 * cg + 4 * lg;        // first of this lane's four output columns
    const TokMap tm = tok_map(T, p.reverse);            // walk position -> token
    // accumulating outputs add an fp32 plane before the store (empty range otherwise)
    const bool accum = !BI && p.accumulate;
    const rsrc_t rAc = make_rsrc(accum ? p.acc_src + (size_t)bh * T * dv : nullptr,
                                 accum ? (unsigned)T * dv * 4u : 0u);

    // Loads and stores below are unconditional (kOffNone where there is
    // nothing to move) so that the compiler counts the loads in flight
    // exactly and never drains them early.

    // ---- working scale of these 16 value columns, the one every walk of them
    // used: partial outputs, maps and the copy of state_in are in its units.
    // The pass folds and corrects on those units too and multiplies outputs
    // and state back (a uniform address: a scalar load).  Each direction of a
    // bidirectional call has its own.
    const float s_w = p.sscale[(size_t)bh * (dv / 16) + c16];
    const float s_b = BI ? p.bw.sscale[(size_t)bh * (dv / 16) + c16] : 0.f;

    // ---- correction operands of a group of CPG chunks (RG row blocks): one
    // 16-byte piece of Phi per thread, staged in LDS; the wave's own row block
    // of the partial outputs (fp16, 4 columns per lane); the same of the
    // backward direction (stored in token order by its walk)
    auto cload = [&](uint4& h, uint2& o, uint2& gt, uint4& av, uint4& hb, uint2& ob, int g) {
        const int c0 = cb + g * CPG;
        const int c = c0 + rg / NB, rb = rg % NB;
        const unsigned hoff = (c0 < ce && tid < PPG) ? (unsigned)((c0 - ch0) * C * DK * 2 + tid * 16) : kOffNone;
        const unsigned ooff = c < ce ? (unsigned)((((c - ch0) * NB + rb) * (dv / 16) + c16) * 64 + lane) * 8u
                                     : kOffNone;
        h = buf_load16(rP, hoff);
        o = buf_load8(rO, ooff);
        if constexpr (BI) {
            hb = buf_load16(rPb, hoff);
            ob = buf_load8(rOb, ooff);
        }
        if constexpr (!PL) {
            // output gate of the same four elements (the range is empty without one)
            const unsigned e = (unsigned)(tm(c * C + 16 * rb + lc) * dv + col4);
            gt = buf_load8(rG, c < ce ? e * 2u : kOffNone);
            // values to accumulate onto (the range is empty unless accumulating)
            if constexpr (!BI) av = buf_load16(rAc, c < ce ? e * 4u : kOffNone);
        }
    };
    // a ring of NPF correction groups in flight, the first issued before the fold
    constexpr int NPF = 2;
    static_assert(NPF % 2 == 0, "the staging copies alternate");
    uint4 ph[NPF], av2[NPF], phb[NPF];
    uint2 ov[NPF], gv2[NPF], ovb[NPF];
#pragma unroll
    for (int j = 0; j < NPF; ++j) cload(ph[j], ov[j], gv2[j], av2[j], phb[j], ovb[j], j);

    // ---- the state entering the segment, per direction, as fp16 B fragments
    // of the whole of M for every wave.  A direction folds nfold maps, map
    // indices base, base + step, ..., onto the copy of state_in (from_snap) or
    // zero; own: the map after them is this segment's own, applied to M_in for
    // state_out.
    F mI[KS_D];
    F mIb[BI ? KS_D : 1];
    if constexpr (DK == 64) {
    // ---- fold by column owners: waves 0..3 (column group cg = wave) keep all
    // d_k rows of their 16 columns in fp32, so the state needs no exchange
    // between waves (its operand fragments come from the owner's own
    // accumulators); all 16 waves stage the maps -- A_s and this tile's B_s --
    // into LDS, FR maps per barrier.  The own map is staged as one more map
    // and applied after M_in is published.
    const bool owner = wave < 4;
    constexpr int SA = FR * APC / 1024, SB = FR * BPC / 1024;   // pieces per thread per group
    static_assert(FR * APC % 1024 == 0 && FR * BPC % 1024 == 0, "staging split");
    auto fold = [&](const rsrc_t& rA_, const rsrc_t& rB_, int nfold, bool own, int base, int step,
                    bool from_snap, F (&mOut)[KS_D]) {
        const int nst = nfold + (own ? 1 : 0);
        const int ngrp = (nst + FR - 1) / FR;
        f32x4 Mw[NDB];
#pragma unroll
        for (int ib = 0; ib < NDB; ++ib) Mw[ib] = zero4();
        if (owner && from_snap) {
            const float* sp = p.snap + (size_t)bh * DK * dv + col;
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                for (int i = 0; i < 4; ++i) Mw[ib][i] = sp[(16 * ib + 4 * lg + i) * dv];
        }
        uint4 sa[SA], sb[SB];
        auto sload = [&](int g) {
#pragma unroll
            for (int j = 0; j < SA; ++j) {
                const int e = tid + 1024 * j, i = g * FR + e / APC;
                sa[j] = buf_load16(rA_, (g < ngrp && i < nst) ? (unsigned)(((base + step * i) * APC + e % APC) * 16)
                                                              : kOffNone);
            }
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int e = tid + 1024 * j, i = g * FR + e / BPC;
                sb[j] = buf_load16(rB_, (g < ngrp && i < nst)
                                            ? (unsigned)((base + step * i) * DK * dv * 4 + (vt * 4 * NDB * 64 + e % BPC) * 16)
                                            : kOffNone);
            }
        };
        auto sstore = [&](int slot) {
#pragma unroll
            for (int j = 0; j < SA; ++j) As2[slot][tid + 1024 * j] = sa[j];
#pragma unroll
            for (int j = 0; j < SB; ++j) Bs2[slot][tid + 1024 * j] = sb[j];
        };
        // M <- A M + B on an owner: operand fragments of the old M first
        auto oapply = [&](int slot, int r) {
            F mB[KS_D];
#pragma unroll
            for (int ks = 0; ks < KS_D; ++ks) mB[ks] = Op::b_acc(Mw, ks);
#pragma unroll
            for (int ib = 0; ib < NDB; ++ib) {
                f32x4 acc = __builtin_bit_cast(f32x4, Bs2[slot][r * BPC + (cg * NDB + ib) * 64 + lane]);
#pragma unroll
                for (int ks = 0; ks < KS_D; ++ks)
                    acc = Op::mma(__builtin_bit_cast(F, As2[slot][r * APC + (ib * KS_D + ks) * 64 + lane]), mB[ks], acc);
                Mw[ib] = acc;
            }
        };
        sload(0);
        sstore(0);
        sload(1);
        __syncthreads();
        for (int g = 0; g < ngrp; ++g) {
            if (owner) {
#pragma unroll
                for (int r = 0; r < FR; ++r)
                    if (g * FR + r < nfold) oapply(g & 1, r);
            }
            // copy (g + 1) & 1 was last read in group g - 1, before the previous barrier
            if (g + 1 < ngrp) sstore((g + 1) & 1);
            sload(g + 2);
            __syncthreads();
        }
        if (owner) {
#pragma unroll
            for (int ks = 0; ks < KS_D; ++ks) Mf[0][ks][cg][lane] = __builtin_bit_cast(uint4, Op::b_acc(Mw, ks));
            if (own) {
                // the own map sits in the last group's copy, which no later group overwrote
                oapply((ngrp - 1) & 1, nfold % FR);
                float* sp = p.state_out + (size_t)bh * DK * dv + col;
#pragma unroll
                for (int ib = 0; ib < NDB; ++ib)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sp[(16 * ib + 4 * lg + i) * dv] = Mw[ib][i] * s_w;
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < KS_D; ++ks) mOut[ks] = __builtin_bit_cast(F, Mf[0][ks][cg][lane]);
    };
    fold(rA, rB, seg - s0, last, s0, 1, from_snap, mI);
    if constexpr (BI) {
        __syncthreads();                  // every wave has read Mf and the staged maps
        fold(rAb, rBb, nseg - 1 - seg, false, nseg - 1, -1, false, mIb);
    }
    } else {
    // ---- fold: D maps in flight; the own map (state_out) is loaded from the start
    auto fold = [&](const rsrc_t& rA_, const rsrc_t& rB_, int nfold, bool own, int base, int step,
                    bool from_snap, F (&mOut)[KS_D]) {
        // rows 16 (rg RB + r) + 4 lg + i of M, column col
        f32x4 Macc[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) Macc[r] = zero4();
        if (from_snap) {
            const float* sp = p.snap + (size_t)bh * DK * dv + col;
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) Macc[r][i] = sp[(16 * (rg * RB + r) + 4 * lg + i) * dv];
        }
        uint4 ra[D][APT], ral[APT];
        f32x4 rb[D][RB], rbl[RB];
        // map index m (valid when ok)
        auto issue = [&](uint4 (&a)[APT], f32x4 (&b)[RB], int m, bool ok) {
#pragma unroll
            for (int j = 0; j < APT; ++j)
                a[j] = buf_load16(rA_, (ok && tid + 1024 * j < APC) ? (unsigned)(m * APC * 16 + (tid + 1024 * j) * 16)
                                                                    : kOffNone);
#pragma unroll
            for (int r = 0; r < RB; ++r)
                b[r] = __builtin_bit_cast(f32x4, buf_load16(rB_,
                            ok ? (unsigned)(m * DK * dv * 4 + ((c16 * NDB + rg * RB + r) * 64 + lane) * 16) : kOffNone));
        };
        // A_s into LDS copy buf (APC pieces over the first APC threads' slots)
        auto put_a = [&](const uint4 (&a)[APT], int buf) {
#pragma unroll
            for (int j = 0; j < APT; ++j)
                if (tid + 1024 * j < APC) Ast[buf][tid + 1024 * j] = a[j];
        };
        // this wave's rows of M as halves of fp16 B fragments (rows 32 ks + 16 h + ...)
        auto put_m = [&](int buf) {
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int ib = rg * RB + r;
                reinterpret_cast<uint2*>(&Mf[buf][ib / 2][cg][lane])[ib & 1] =
                    make_uint2(Op::pk2(Macc[r][0], Macc[r][1]), Op::pk2(Macc[r][2], Macc[r][3]));
            }
        };
        auto get_m = [&](F (&mF)[KS_D], int buf) {
#pragma unroll
            for (int ks = 0; ks < KS_D; ++ks) mF[ks] = __builtin_bit_cast(F, Mf[buf][ks][cg][lane]);
        };
        // this wave's rows of A M + B
        auto apply = [&](const F (&mF)[KS_D], int buf, const f32x4 (&b)[RB]) {
            F fa[RB][KS_D];
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int ks = 0; ks < KS_D; ++ks)
                    fa[r][ks] = __builtin_bit_cast(F, Ast[buf][((rg * RB + r) * KS_D + ks) * 64 + lane]);
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                f32x4 acc = b[r];
#pragma unroll
                for (int ks = 0; ks < KS_D; ++ks) acc = Op::mma(fa[r][ks], mF[ks], acc);
                Macc[r] = acc;
            }
        };
        issue(ral, rbl, base + step * nfold, own);
#pragma unroll
        for (int d = 0; d < D; ++d) issue(ra[d], rb[d], base + step * d, d < nfold);
        for (int i0 = 0; i0 < nfold; i0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int i = i0 + d;
                // copies i & 1 were last read two steps ago, before the previous barrier
                put_a(ra[d], i & 1);
                put_m(i & 1);
                __syncthreads();
                if (i < nfold) {
                    F mF[KS_D];
                    get_m(mF, i & 1);
                    apply(mF, i & 1, rb[d]);
                }
                issue(ra[d], rb[d], base + step * (i + D), i + D < nfold);
            }
        }
        // M_in of this segment as B fragments for every wave; the own map alongside
        put_m(nfold & 1);
        if (own) put_a(ral, nfold & 1);
        __syncthreads();
        get_m(mOut, nfold & 1);
        if (own) {
            apply(mOut, nfold & 1, rbl);
            float* sp = p.state_out + (size_t)bh * DK * dv + col;
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) sp[(16 * (rg * RB + r) + 4 * lg + i) * dv] = Macc[r][i] * s_w;
        }
    };
    fold(rA, rB, seg - s0, last, s0, 1, from_snap, mI);
    if constexpr (BI) {
        __syncthreads();                  // every wave has read Mf and the staged map
        fold(rAb, rBb, nseg - 1 - seg, false, nseg - 1, -1, false, mIb);
    }
    }

    // ---- outputs of the segment: O += Phi M_in, formed transposed
    // (O^T = M^T Phi^T): lane (lg, lc) holds row lc of the wave's row block
    // and four consecutive columns, one 16-byte access
    auto cfix = [&](const uint4& h, const uint2& o, const uint2& gt, const uint4& av, const uint4& hb,
                    const uint2& ob, int g, int buf) {
        const int c = cb + g * CPG + rg / NB, rb = rg % NB;
        if (tid < PPG) {
            Phs[buf][tid] = h;
            if constexpr (BI) Phb[buf * PPG + tid] = hb;
        }
        __syncthreads();                  // copy buf reused two groups later, after another barrier
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 ot = __builtin_bit_cast(h4, o);
        f32x4 acc = {(float)ot[0], (float)ot[1], (float)ot[2], (float)ot[3]};
#pragma unroll
        for (int ks = 0; ks < KS_D; ++ks)
            acc = Op::mma(mI[ks], __builtin_bit_cast(F, Phs[buf][(rg * KS_D + ks) * 64 + lane]), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= s_w;
        if constexpr (BI) {
            const h4 otb = __builtin_bit_cast(h4, ob);
            f32x4 accb = {(float)otb[0], (float)otb[1], (float)otb[2], (float)otb[3]};
#pragma unroll
            for (int ks = 0; ks < KS_D; ++ks)
                accb = Op::mma(mIb[ks], __builtin_bit_cast(F, Phb[buf * PPG + (rg * KS_D + ks) * 64 + lane]), accb);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += accb[i] * s_b;
        }
        // rows past T fall outside the buffer and are dropped
        const unsigned e0 = (unsigned)(tm(c * C + 16 * rb + lc) * dv + col4);
        if (!PL && gated) {
            acc[0] *= __builtin_bit_cast(float, gt.x << 16);
            acc[1] *= __builtin_bit_cast(float, gt.x & 0xffff0000u);
            acc[2] *= __builtin_bit_cast(float, gt.y << 16);
            acc[3] *= __builtin_bit_cast(float, gt.y & 0xffff0000u);
        }
        if constexpr (!BI && !PL) add_f32x4(acc, av);   // accumulating: one rounding of the sum
        if (p.out_bf16) {
            const uint2 w = make_uint2(
                (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[0]) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[1]) << 16),
                (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[2]) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[3]) << 16));
            buf_store8<kOutPolicy>(rW, c < ce ? e0 * 2u : kOffNone, w);
        } else {
            buf_store16<kOutPolicy>(rW, c < ce ? e0 * 4u : kOffNone, __builtin_bit_cast(uint4, acc));
        }
    };
    const int ngroups = (ce - cb + CPG - 1) / CPG;
    for (int g = 0; g < ngroups; g += NPF) {
#pragma unroll
        for (int j = 0; j < NPF; ++j) {
            cfix(ph[j], ov[j], gv2[j], av2[j], phb[j], ovb[j], g + j, j & 1);
            cload(ph[j], ov[j], gv2[j], av2[j], phb[j], ovb[j], g + j + NPF);
        }
    }
}

// ---------------------------------------------------------------------------
// Launch table
// ---------------------------------------------------------------------------
namespace {

template <int DK, int C, int CTS, int EXT>
hipError_t launch_pipe_g(const WalkArgs& a, hipStream_t s) {
    // a segment tile of 128 columns: eight state waves of one tile each
    // (three waves per SIMD; measured faster than four state waves of two
    // tiles, which spill at d_k = 128)
    constexpr int SNCW = CTS == 2 ? 8 : 4;
    constexpr int SCT = CTS * 4 / SNCW;
    constexpr int UNPW = C == 64 ? 8 : 4;                // key waves of the unsegmented walk
    static_assert(pipe_fits<DK, C, 1, false, 4, UNPW>() && pipe_fits<DK, C, SCT, true, SNCW>(), "LDS plan exceeds 160 KiB");
    const int bh = a.B * a.H;
    if (a.nseg > 1) {
        WalkArgs b = a;
        const int ncol = (DK + a.dv) / (64 * CTS);
        // plain calls: segment 0 walks from state_in and writes its outputs
        // itself, so its tiles of identity columns only are not launched
        b.seg0_direct = EXT == 0 ? 1 : 0;
        const int skip = b.seg0_direct && DK != a.dv ? DK / (64 * CTS) : 0;
        const int grid = bh * (a.nseg * ncol - skip);
        // a fused bidirectional call walks both directions in one launch
        const int walks = EXT == kExtAll && a.bidir ? 2 : 1;
        b.fix_split = 0;
        hipLaunchKernelGGL((gdn_pipe_kernel<DK, C, SCT, true, SNCW, 4, EXT>), dim3(grid * walks), dim3(64 * (SNCW + 4)),
                           0, s, b);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // correction: one workgroup per (head, corrected segment, 64 value
        // columns); the deepest segments take a second one while the launch
        // still fits one round on the 256 compute units
        const long long unit = (long long)bh * (a.dv / 64);
        if (walks == 2) {
            hipLaunchKernelGGL((gdn_pipe_fix_kernel<DK, C, true>), dim3(unit * a.nseg), dim3(1024), 0, s, b);
        } else {
            const int nfix = a.nseg - b.seg0_direct;
            const long long room = 256 / unit - nfix;
            b.fix_split = (int)(room <= 0 ? 0 : (room < nfix ? room : nfix));
            if (!a.out_gate && !a.accumulate)
                hipLaunchKernelGGL((gdn_pipe_fix_kernel<DK, C, false, true>), dim3(unit * (nfix + b.fix_split)),
                                   dim3(1024), 0, s, b);
            else
                hipLaunchKernelGGL((gdn_pipe_fix_kernel<DK, C, false>), dim3(unit * (nfix + b.fix_split)), dim3(1024),
                                   0, s, b);
        }
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gdn_pipe_kernel<DK, C, 1, false, 4, UNPW, EXT>), dim3(bh * (a.dv / 64)), dim3(64 * (4 + UNPW)), 0, s, a);
    return hipGetLastError();
}

template <int DK, int C, int CTS>
hipError_t launch_pipe_t(const WalkArgs& a, hipStream_t s) {
    if (a.reverse || a.accumulate || a.bidir) return launch_pipe_g<DK, C, CTS, kExtAll>(a, s);
    if (a.gate_logits || a.out_gate) return launch_pipe_g<DK, C, CTS, kExtGates>(a, s);
    return launch_pipe_g<DK, C, CTS, 0>(a, s);
}

template <int DK, int C>
hipError_t pipe_cts(const WalkArgs& a, int cts, hipStream_t s) {
    if (cts == 2) return launch_pipe_t<DK, C, 2>(a, s);
    return launch_pipe_t<DK, C, 1>(a, s);
}

template <int DK>
hipError_t pipe_c(const WalkArgs& a, int C, int cts, hipStream_t s) {
    switch (C) {
    case 32: return pipe_cts<DK, 32>(a, cts, s);
    case 64: return pipe_cts<DK, 64>(a, cts, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool pipe_supported(int in_f32, int dk, int dv, int chunk) {
    return !in_f32 && (dk == 64 || dk == 128) && dv % 64 == 0 && (chunk == 32 || chunk == 64);
}

int pipe_seg_tiles(int dk, int dv) {
    return (dk + dv) % 128 == 0 ? 2 : 1;
}

size_t pipe_workspace(int B, int H, int dk, int dv, int chunk, int nseg, int seg_chunks) {
    if (nseg <= 1) return 0;
    const size_t bh = (size_t)B * H, ns = (size_t)nseg, rows = (size_t)seg_chunks * chunk;
    return bh * ns * dk * dk * 2          // A_s (fp16)
         + bh * ns * dk * dv * 4          // B_s
         + bh * dk * dv * 4               // copy of state_in
         + bh * ns * rows * dk * 2        // Phi (fp16)
         + bh * ns * rows * dv * 2        // partial outputs (fp16)
         + bh * (dv / 16) * 4;            // working scale per 16 value columns
}

hipError_t launch_pipe(const WalkArgs& a, int chunk, hipStream_t s) {
    const int cts = pipe_seg_tiles(a.dk, a.dv);
    switch (a.dk) {
    case 64: return pipe_c<64>(a, chunk, cts, s);
    case 128: return pipe_c<128>(a, chunk, cts, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
