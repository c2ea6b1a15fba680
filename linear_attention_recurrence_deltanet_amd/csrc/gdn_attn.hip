// gdn_attn.hip -- softmax attention of a streaming chunk over a persistent
// sink chunk, a window of recent chunks and the chunk itself (SANA-Streaming,
// paperpeel page, section 2.1 "Softmax blocks for local window and sink
// refinement": the softmax blocks of the hybrid restrict each chunk's context
// to itself, a sink chunk shared across the stream and a short recent window),
// for gfx950.
//
//   O = softmax(scale * Q K^T) V,  K = [K_sink; K_win; K_cur], V likewise,
//   no mask (a chunk is denoised as a whole).
//
// One workgroup of four waves per (head, 128 queries); each wave owns 32
// queries (two blocks of 16).  The keys are walked in tiles of 64 across the
// three segments, staged in LDS (K row-major, V transposed) and double
// buffered: the next tile's loads are issued before the current tile's
// products and written to the other copy after them, one barrier per tile.
// Per tile and wave the products are formed transposed, so that the softmax
// statistics and the output rescale belong to lanes (lane (g, c) holds query
// c of each block):
//   S^T = K Q^T          keys x queries (K from LDS, Q^T kept in registers),
//                        bf16 operands as given
//   online softmax over the keys: running max m per query, exp2
//   O^T += V^T P^T       P^T taken as it stands from the S^T accumulators;
//                        one more block of V^T, a row of ones, gives the
//                        softmax denominators on the matrix cores;
//                        fp16 operands (11-bit significand: P in bf16 alone
//                        costs ~1e-3 relative on the output), V converted
//                        exactly while it is transposed into LDS
// The output is O = (O^T)^T / l: lane (g, c) writes four consecutive columns
// of query c, one 16-byte store in fp32.
// Few heads leave compute units idle and a lone wave per SIMD waiting on its
// own latencies; the key tiles are then split into up to four ranges, one
// workgroup each, which store their unnormalised output with the running max
// and sum of every query, and gdn_attn_combine_kernel merges the ranges with
// the weights exp2(m_s - max_s m_s) (the log-sum-exp identity).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gdn_common.h"
#include "gdn_kernels.h"

namespace gdn {

namespace {

constexpr int AQ = 128;   // queries per workgroup (4 waves x 32)
constexpr int AK = 64;    // keys per tile
constexpr float kLazy = 8.f;   // headroom of the softmax reference max (log2 units)
// outputs (and the parts of a split call) written through as produced (sc0
// sc1): measured 0.7-1.4% faster per call than the default policy
constexpr int kOutPolicy = 1 | 16;

template <int D>
struct APlan {
    // row strides of 2 (mod 32) 32-bit words beyond 16-byte multiples keep the
    // 8-byte operand reads of 16 rows in distinct banks
    static constexpr int LDK = D + 4;             // K rows: D bf16
    static constexpr int LDV = AK + 4;            // V^T rows: AK bf16
    static constexpr int KSZ = AK * LDK;          // elements of one K copy
    static constexpr int VSZ = D * LDV;           // elements of one V^T copy
    static constexpr int PPR = D / 8;             // 16-byte pieces per key row
    static constexpr int NPC = AK / 2 * PPR / 256; // (row pair, piece) items per thread per tile
};

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one query column of
// an accumulator tile): v_permlane32_swap / v_permlane16_swap exchange halves
// and rows of two registers on the VALU, no LDS round trip.  Written as asm
// with both registers in and out: through the compiler builtin, a swap of
// two equal inputs had its second result replaced by the first (checked on
// the hardware, whose results differ), losing the exchange.
__device__ __forceinline__ float xlane_max4(float x) {
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    float c = fmaxf(a, b), d = c;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(c), "+v"(d));
    return fmaxf(c, d);
}

// Operand fragment in accumulator k order (row lane % 16; k = kb + 4 g + i
// and kb + 16 + 4 g + i for lane group g), from 16-bit rows in LDS.
__device__ __forceinline__ u16x8 frag_rows(const uint16_t* base, int ld, int row0, int kb, int lane) {
    const uint16_t* p = base + (row0 + (lane & 15)) * ld + kb + 4 * (lane >> 4);
    const u16x4 lo = *reinterpret_cast<const u16x4*>(p);
    const u16x4 hi = *reinterpret_cast<const u16x4*>(p + 16);
    return u16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Eight fp32 -> fp16 (round to nearest even), packed in pairs.
__device__ __forceinline__ u16x8 pack8_f16(const f32x4& a, const f32x4& b) {
    return OpF16::pack8(a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]);
}

// Eight fp32 -> bf16 (round to nearest even), packed in pairs.
__device__ __forceinline__ u16x8 pack8_bf16(const f32x4& a, const f32x4& b) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a[0], a[1]}, bf2)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a[2], a[3]}, bf2)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{b[0], b[1]}, bf2)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{b[2], b[3]}, bf2))};
    return __builtin_bit_cast(u16x8, w);
}

template <int D>
__global__ __launch_bounds__(256, 2) void gdn_attn_kernel(AttnArgs p) {
    typedef APlan<D> L;
    typedef OpBF16 Op;
    constexpr int KSD = D / 32;                   // k-steps of the head dimension
    constexpr int NDB = D / 16;                   // 16-row blocks of O^T
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][L::KSZ];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][L::VSZ];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lc = lane & 15, lg = lane >> 4;
    const int Nq = p.Nq;
    const int nqb = (Nq + AQ - 1) / AQ;
    const int nsplit = p.nsplit;
    int wg = block_x(p.rev_wg);
    {
        // the query blocks of one head read the same keys: keep them on one XCD
        const int w8 = (int)gridDim.x / 8 * 8;
        if (wg < w8) wg = (wg % 8) * (w8 / 8) + wg / 8;
    }
    const int sp = uniform(wg % nsplit);               // key range of this workgroup
    const int qblk = uniform((wg / nsplit) % nqb);
    const int bh = uniform(wg / nsplit / nqb);
    const int q0 = qblk * AQ + 32 * wave;          // this wave's first query

    const rsrc_t rq = make_rsrc(reinterpret_cast<const uint16_t*>(p.q) + (size_t)bh * Nq * D,
                                (unsigned)Nq * D * 2u);
    const unsigned osz = p.out_bf16 ? 2u : 4u;
    const rsrc_t ro = make_rsrc(reinterpret_cast<const char*>(p.out) + (size_t)bh * Nq * D * osz,
                                (unsigned)Nq * D * osz);
    // tiles of each segment; tile t of the walk lies in segment seg at key base
    const int nt0 = (p.n[0] + AK - 1) / AK, nt1 = (p.n[1] + AK - 1) / AK, nt2 = (p.n[2] + AK - 1) / AK;
    const int ntiles = nt0 + nt1 + nt2;
    const int t_lo = ntiles * sp / nsplit, t_hi = ntiles * (sp + 1) / nsplit;
    auto locate = [&](int t, int& seg, int& base) {
        if (t < nt0) { seg = 0; base = t * AK; }
        else if (t < nt0 + nt1) { seg = 1; base = (t - nt0) * AK; }
        else { seg = 2; base = (t - nt0 - nt1) * AK; }
    };

    // ---- key/value tile staging: registers, then LDS.  A thread moves the
    // same 16-byte piece of two consecutive keys, so that V can be written
    // transposed as 4-byte (key pair) words
    uint4 kr[2 * L::NPC], vr[2 * L::NPC];
    auto load_tile = [&](int t) {
        int seg, base;
        locate(t, seg, base);
        const int n = seg == 0 ? p.n[0] : seg == 1 ? p.n[1] : p.n[2];
        const void* kp = seg == 0 ? p.k[0] : seg == 1 ? p.k[1] : p.k[2];
        const void* vp = seg == 0 ? p.v[0] : seg == 1 ? p.v[1] : p.v[2];
        // keys past the segment's end read as zero (and are masked below)
        const rsrc_t rk = make_rsrc(reinterpret_cast<const uint16_t*>(kp) + (size_t)bh * n * D, (unsigned)n * D * 2u);
        const rsrc_t rv = make_rsrc(reinterpret_cast<const uint16_t*>(vp) + (size_t)bh * n * D, (unsigned)n * D * 2u);
#pragma unroll
        for (int it = 0; it < L::NPC; ++it) {
            const int idx = tid + 256 * it;
            const int r = 2 * (idx / L::PPR), c = idx % L::PPR;
            const unsigned off = (unsigned)((base + r) * D + 8 * c) * 2u;
            kr[2 * it] = buf_load16(rk, off);
            kr[2 * it + 1] = buf_load16(rk, off + D * 2u);
            vr[2 * it] = buf_load16(rv, off);
            vr[2 * it + 1] = buf_load16(rv, off + D * 2u);
        }
    };
    auto store_tile = [&](int b) {
#pragma unroll
        for (int it = 0; it < L::NPC; ++it) {
            const int idx = tid + 256 * it;
            const int r = 2 * (idx / L::PPR), c = idx % L::PPR;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint2* kd = reinterpret_cast<uint2*>(&Ks[b][(r + h) * L::LDK + 8 * c]);
                kd[0] = make_uint2(kr[2 * it + h].x, kr[2 * it + h].y);
                kd[1] = make_uint2(kr[2 * it + h].z, kr[2 * it + h].w);
            }
            // bf16 -> fp16 (exact for |v| in [2^-14, 65504]; smaller values keep
            // an absolute error below 2^-25), transposed: word (key r, key r + 1)
            const uint32_t w0[4] = {vr[2 * it].x, vr[2 * it].y, vr[2 * it].z, vr[2 * it].w};
            const uint32_t w1[4] = {vr[2 * it + 1].x, vr[2 * it + 1].y, vr[2 * it + 1].z, vr[2 * it + 1].w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t a = (j & 1) ? (w0[j / 2] & 0xffff0000u) : (w0[j / 2] << 16);
                const uint32_t e = (j & 1) ? (w1[j / 2] & 0xffff0000u) : (w1[j / 2] << 16);
                typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                typedef float f2 __attribute__((ext_vector_type(2)));
                const h2 v2 = __builtin_convertvector(f2{__builtin_bit_cast(float, a), __builtin_bit_cast(float, e)}, h2);
                *reinterpret_cast<uint32_t*>(&Vt[b][(8 * c + j) * L::LDV + r]) = __builtin_bit_cast(uint32_t, v2);
            }
        }
    };

    // ---- this wave's queries as B fragments (Q^T), accumulator k order
    u16x8 qf[2][KSD];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            const unsigned off = (unsigned)((q0 + 16 * qb + lc) * D + 32 * ks + 4 * lg) * 2u;
            const uint2 lo = buf_load8(rq, off), hi = buf_load8(rq, off + 32u);
            qf[qb][ks] = __builtin_bit_cast(u16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }

    f32x4 O[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db) O[db][0] = O[db][1] = zero4();
    // the softmax denominators ride along with the output: one more 16-row
    // block of V^T whose first row is all ones (fp16 1.0 on lanes of row 0),
    // so that row 0 of Lacc accumulates sum_k P[k][query] on the matrix cores
    const uint32_t one2 = lc == 0 ? 0x3C003C00u : 0u;
    const u16x8 ones = __builtin_bit_cast(u16x8, make_uint4(one2, one2, one2, one2));
    f32x4 Lacc[2] = {zero4(), zero4()};
    // running max (exp2 domain) per query block; it starts finite so that
    // fully masked keys give exp2(-inf) = 0
    float m[2] = {-1e30f, -1e30f};
    const float cs = p.scale * 1.4426950408889634f;

    if (t_lo < t_hi) {
        load_tile(t_lo);
        store_tile(0);
    }
    __syncthreads();
    for (int t = t_lo; t < t_hi; ++t) {
        if (t + 1 < t_hi) load_tile(t + 1);
        const int b = (t - t_lo) & 1;
        int seg, base;
        locate(t, seg, base);
        const int kmax = min(AK, (seg == 0 ? p.n[0] : seg == 1 ? p.n[1] : p.n[2]) - base);

        // S^T = K Q^T: rows = keys 16 kb + 4 g + i, column = query c
        f32x4 S[4][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) S[kb][0] = S[kb][1] = zero4();
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const u16x8 a = frag_rows(Ks[b], L::LDK, 16 * kb, 32 * ks, lane);
                S[kb][0] = Op::mma(a, qf[0][ks], S[kb][0]);
                S[kb][1] = Op::mma(a, qf[1][ks], S[kb][1]);
            }

        // keys past a segment's end (its last tile only) get no weight
        if (kmax < AK) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * kb + 4 * lg + i >= kmax) S[kb][0][i] = S[kb][1][i] = -INFINITY;
        }
        // online softmax over the keys, per query (the four lanes of a column);
        // the scale enters once, in the exponent's fma (cs > 0)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[kb][qb][i]);
            // the reference max of a query moves only when the tile's max
            // exceeds it by more than kLazy (exp2 domain): the weights stay
            // below 2^kLazy (exact in fp16) and most tiles skip the rescale;
            // the result does not depend on it (numerator and denominator
            // share the reference)
            const float cand = xlane_max4(mx) * cs;
            const float mn = cand > m[qb] + kLazy ? cand : m[qb];
            const float corr = __builtin_amdgcn_exp2f(m[qb] - mn);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[kb][qb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][qb][i], cs, -mn));
            // the running output and denominators are rescaled only when some
            // query's max grew (corr is exactly 1 for the others)
            if (__builtin_amdgcn_ballot_w64(mn > m[qb]) != 0) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) O[db][qb] *= corr;
                Lacc[qb] *= corr;
            }
            m[qb] = mn;
        }

        // O^T += V^T P^T: P^T as B fragments straight from the accumulators
        u16x8 pf[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) pf[qb][k2] = pack8_f16(S[2 * k2][qb], S[2 * k2 + 1][qb]);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const u16x8 a = frag_rows(Vt[b], L::LDV, 16 * db, 32 * k2, lane);
                O[db][0] = OpF16::mma(a, pf[0][k2], O[db][0]);
                O[db][1] = OpF16::mma(a, pf[1][k2], O[db][1]);
            }
            Lacc[0] = OpF16::mma(ones, pf[0][k2], Lacc[0]);
            Lacc[1] = OpF16::mma(ones, pf[1][k2], Lacc[1]);
        }

        if (t + 1 < t_hi) store_tile(b ^ 1);     // copy b ^ 1 was last read before the previous barrier
        __syncthreads();
    }

    if (nsplit > 1) {
        // ---- one key range: unnormalised O and (m, l) per query, for the combine
        const size_t prow = ((size_t)sp * p.B * p.H + bh) * Nq;          // first row of this head's part
        const rsrc_t rpo = make_rsrc(p.part_o + prow * D, (unsigned)Nq * D * 4u);
        const rsrc_t rpm = make_rsrc(p.part_ml + prow * 2, (unsigned)Nq * 8u);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float ls = __shfl(Lacc[qb][0], lc);       // row 0 sits on lanes 0..15
            const int row = q0 + 16 * qb + lc;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                buf_store16<kOutPolicy>(rpo, (unsigned)(row * D + 16 * db + 4 * lg) * 4u, __builtin_bit_cast(uint4, O[db][qb]));
            if (lg == 0)
                buf_store8<kOutPolicy>(rpm, (unsigned)row * 8u, make_uint2(__builtin_bit_cast(uint32_t, m[qb]),
                                                               __builtin_bit_cast(uint32_t, ls)));
        }
        return;
    }
    // ---- O = (O^T)^T / l: lane (g, c) holds columns 16 db + 4 g + i of query c
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float inv = 1.f / __shfl(Lacc[qb][0], lc);   // row 0 sits on lanes 0..15
        const int row = q0 + 16 * qb + lc;                 // rows past Nq are dropped
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const f32x4 o = O[db][qb] * inv;
            const unsigned e = (unsigned)(row * D + 16 * db + 4 * lg);
            if (p.out_bf16) {
                const u16x8 w = pack8_bf16(o, o);
                const uint4 u = __builtin_bit_cast(uint4, w);
                buf_store8<kOutPolicy>(ro, e * 2u, make_uint2(u.x, u.y));
            } else {
                buf_store16<kOutPolicy>(ro, e * 4u, __builtin_bit_cast(uint4, o));
            }
        }
    }
}

// Merge of the key ranges: thread = (row, four columns).  With m_s the
// running max (exp2 domain) and l_s the sum of range s,
//   O = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s,   m = max_s m_s.
template <int D>
__global__ __launch_bounds__(256) void gdn_attn_combine_kernel(AttnArgs p) {
    const long long rows = (long long)p.B * p.H * p.Nq;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * (D / 4)) return;
    const long long row = idx / (D / 4);
    const int c = (int)(idx % (D / 4)) * 4;
    float mx = -INFINITY;
    for (int s = 0; s < p.nsplit; ++s) mx = fmaxf(mx, p.part_ml[((size_t)s * rows + row) * 2]);
    f32x4 acc = zero4();
    float L = 0.f;
    for (int s = 0; s < p.nsplit; ++s) {
        const float* ml = p.part_ml + ((size_t)s * rows + row) * 2;
        const float w = __builtin_amdgcn_exp2f(ml[0] - mx);
        L += w * ml[1];
        acc += w * *reinterpret_cast<const f32x4*>(p.part_o + ((size_t)s * rows + row) * D + c);
    }
    const f32x4 o = acc * (1.f / L);
    if (p.out_bf16) {
        const u16x8 w = pack8_bf16(o, o);
        const uint4 u = __builtin_bit_cast(uint4, w);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + row * D + c) = make_uint2(u.x, u.y);
    } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + row * D + c) = o;
    }
}

}  // namespace

bool attn_supported(int d) { return d == 64 || d == 128; }

int attn_splits(int B, int H, int Nq, const int n[3]) {
    const long long wgs = (long long)B * H * ((Nq + 127) / 128);
    const int ntiles = (n[0] + AK - 1) / AK + (n[1] + AK - 1) / AK + (n[2] + AK - 1) / AK;
    // about two resident workgroups per compute unit (512 in all), rounded to
    // the nearest count: measured best at 2 ranges for 336 query blocks and 3
    // for 168 (4 ranges there run 2.6 workgroups per unit, in uneven rounds)
    int ns = wgs > 0 ? (int)((512 + wgs / 2) / wgs) : 1;
    ns = ns > 4 ? 4 : ns;
    const int cap = ntiles / 8;                                  // at least 8 tiles per range
    if (ns > cap) ns = cap;
    return ns < 1 ? 1 : ns;
}

size_t attn_workspace(int B, int H, int Nq, int d, int nsplit) {
    return nsplit > 1 ? (size_t)nsplit * B * H * Nq * (d + 2) * 4 : 0;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
    const int nqb = (a.Nq + 127) / 128;
    const dim3 grid((unsigned)(a.B * a.H * nqb * a.nsplit)), block(256);
    if (a.d == 64)
        hipLaunchKernelGGL(gdn_attn_kernel<64>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(gdn_attn_kernel<128>, grid, block, 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit <= 1) return e;
    const long long threads = (long long)a.B * a.H * a.Nq * (a.d / 4);
    const dim3 cgrid((unsigned)((threads + 255) / 256));
    if (a.d == 64)
        hipLaunchKernelGGL(gdn_attn_combine_kernel<64>, cgrid, block, 0, s, a);
    else
        hipLaunchKernelGGL(gdn_attn_combine_kernel<128>, cgrid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace gdn
