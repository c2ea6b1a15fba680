// gdn_common.h -- device-side building blocks shared by the libgdn kernels:
// operand policies for the gfx950 matrix cores, LDS fragment loads and
// scalar conversions.  Internal header (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Matrix-core operand policies.  Each describes one MFMA shape producing a
// 16x16 fp32 tile whose lane l holds rows 4*(l/16)+i (i<4) of column l%16.
// Operand fragments: lane l supplies row (A) or column (B) l%16 and KPER
// consecutive k values starting at (l/16)*KPER within a KSTEP-wide k block.
// Both operands of a product are read with the same k order, so the
// hardware's k order inside one instruction cancels in the dot product.
// ---------------------------------------------------------------------------

// "acc-order" fragments.  A 16x16 accumulator tile holds rows 4g+i (g = lane/16,
// i < 4) in lane g's four registers.  Feeding accumulators of one product as
// the B operand of the next needs no data movement if the k order of that
// product follows the accumulator rows: for KSTEP = 32 lane g supplies k =
// 4g..4g+3 (tile 0) and 16+4g..16+4g+3 (tile 1); for KSTEP = 4, k-step s
// takes row 4g+s.  The A operand of such a product is then read from LDS in
// the same k order (a_acc below).

// fp16 operands (11-bit significand), fp32 accumulate: v_mfma_f32_16x16x32_f16
struct OpF16 {
    typedef _Float16 elem;
    typedef u16x8 frag;
    typedef u16x4 frag16;   // K = 16 variant (v_mfma_f32_16x16x16_f16)
    static constexpr int KSTEP = 32, KPER = 8, KPER16 = 4;
    __device__ static __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4 mma16(const frag16& a, const frag16& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ elem from_f32(float x) { return (_Float16)x; }
    __device__ static __forceinline__ frag load(const elem* p) {
        return *reinterpret_cast<const frag*>(p);
    }
    __device__ static __forceinline__ frag16 load16(const elem* p) {
        return *reinterpret_cast<const frag16*>(p);
    }
    // A fragment in acc order: row (lane & 15), k block at kb.
    __device__ static __forceinline__ frag a_acc(const elem* base, int ld, int row0, int kb, int lane) {
        const elem* p = base + (row0 + (lane & 15)) * ld + kb + 4 * (lane >> 4);
        const u16x4 lo = *reinterpret_cast<const u16x4*>(p);
        const u16x4 hi = *reinterpret_cast<const u16x4*>(p + 16);
        return frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    // B fragment of k-step ks from accumulator tiles t[2ks], t[2ks+1] (rows = k).
    __device__ static __forceinline__ frag b_acc(const f32x4* t, int ks) {
        const f32x4 a = t[2 * ks], b = t[2 * ks + 1];
        return pack8(a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]);
    }
    // eight fp32 -> eight fp16 (round to nearest even), packed in pairs
    __device__ static __forceinline__ frag pack8(float a0, float a1, float a2, float a3,
                                                  float a4, float a5, float a6, float a7) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        u32x4 w = {pk2(a0, a1), pk2(a2, a3), pk2(a4, a5), pk2(a6, a7)};
        return __builtin_bit_cast(frag, w);
    }
    __device__ static __forceinline__ uint32_t pk2(float a, float b) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        typedef float f2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, h2));
    }
};

// bf16 operands taken raw from the inputs: v_mfma_f32_16x16x32_bf16
struct OpBF16 {
    typedef uint16_t elem;
    typedef u16x8 frag;
    static constexpr int KSTEP = 32, KPER = 8;
    __device__ static __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ frag load(const elem* p) {
        return *reinterpret_cast<const frag*>(p);
    }
};

// fp32 operands: v_mfma_f32_16x16x4_f32
struct OpF32 {
    typedef float elem;
    typedef float frag;
    typedef float frag16;
    static constexpr int KSTEP = 4, KPER = 1, KPER16 = 1;
    __device__ static __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ elem from_f32(float x) { return x; }
    __device__ static __forceinline__ frag load(const elem* p) { return *p; }
    __device__ static __forceinline__ frag a_acc(const elem* base, int ld, int row0, int kb, int lane) {
        // k-step kb covers rows 16*(kb/16) + 4g + (kb/4)%4
        return base[(row0 + (lane & 15)) * ld + (kb & ~15) + 4 * (lane >> 4) + ((kb >> 2) & 3)];
    }
    __device__ static __forceinline__ frag b_acc(const f32x4* t, int ks) {
        return t[ks >> 2][ks & 3];
    }
};

// Fragment of a row-major LDS array (row stride `ld` elements): rows
// [row0, row0+16), k block starting at kb.
template <class Op>
__device__ __forceinline__ typename Op::frag frag_at(const typename Op::elem* base, int ld,
                                                     int row0, int kb, int lane) {
    return Op::load(base + (row0 + (lane & 15)) * ld + kb + (lane >> 4) * Op::KPER);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Block index along one grid dimension, taken in reverse order of dispatch
// when `rev` is set: a debug switch (the environment variable
// GDN_DEBUG_REVERSE_WORKGROUPS read by the API) under which every result must
// stay the same bit for bit, since no workgroup of a launch reads what another
// one writes and none waits for another.
__device__ __forceinline__ int block_x(int rev) { return rev ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x; }
__device__ __forceinline__ int block_y(int rev) { return rev ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y; }
__device__ __forceinline__ int block_z(int rev) { return rev ? (int)(gridDim.z - 1 - blockIdx.z) : (int)blockIdx.z; }

// Workgroup barrier for exchanges through LDS only.  __syncthreads() also
// orders global memory, which on this target waits for every load and store
// the wave has in flight (vmcnt(0)); loads issued ahead of their use would
// then complete at the barrier.  This one waits for the wave's LDS operations
// only; the memory clobber keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// Raw buffer access: a 128-bit resource (base, byte size) in scalar registers
// and a 32-bit per-lane byte offset.  Loads past `bytes` return zero and
// stores past it are dropped by the hardware range check.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // 32-bit data format, raw (untyped) access

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uniform(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}
template <class T>
__device__ __forceinline__ T* uniform(T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}
// Resource of a wave-uniform range (base and size are made scalar).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform(base)), (short)0,
                                             uniform((int)bytes), kRsrcWord3);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, unsigned off) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 buf_load8(rsrc_t r, unsigned off) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint16_t buf_load2(rsrc_t r, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
template <int AUX = 0>
__device__ __forceinline__ void buf_store4(rsrc_t r, unsigned off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, AUX);
}
__device__ __forceinline__ void buf_store2(rsrc_t r, unsigned off, uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}
// soff: a wave-uniform byte offset added in the scalar operand (not part of
// the range check: only for stores known to be in range)
// AUX: cache-policy bits of the store (0: default).
template <int AUX = 0>
__device__ __forceinline__ void buf_store8(rsrc_t r, unsigned off, uint2 v, unsigned soff = 0) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, off, (int)soff, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ void buf_store16(rsrc_t r, unsigned off, uint4 v) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, r, off, 0, AUX);
}
// Accumulating outputs (the second scan of a bidirectional call) add fp32
// values from a separate plane before their one rounding: four of them, as
// loaded, to a lane's four outputs.
template <class V4>
__device__ __forceinline__ void add_f32x4(V4& o, uint4 w) {
    o[0] += __builtin_bit_cast(float, w.x);
    o[1] += __builtin_bit_cast(float, w.y);
    o[2] += __builtin_bit_cast(float, w.z);
    o[3] += __builtin_bit_cast(float, w.w);
}

// Walk position -> token row.  A backward scan walks the tokens in reverse:
// position t < T is token T - 1 - t.  Positions at or past T (the padding of
// a partial last chunk) stay rows at or past T in both directions, so their
// offsets lie past the range as usual (loads read zero, stores are dropped)
// and no offset is ever negative.  tok_map_padded(P) reverses the padded
// length P (a whole number of chunks) instead: position t is row P - 1 - t,
// so the backward walk's chunks are the forward chunks in reverse and its
// padding rows (at or past T) come first.
struct TokMap {
    int last;    // reversed: position t < lim is row last - t
    int lim;
    bool rev;
    __device__ __forceinline__ int operator()(int t) const { return (rev && t < lim) ? last - t : t; }
};
__device__ __forceinline__ TokMap tok_map(int T, int reverse) { return TokMap{T - 1, T, reverse != 0}; }
__device__ __forceinline__ TokMap tok_map_padded(int P) { return TokMap{P - 1, P, true}; }

// Offset past every range a resource here covers (ranges stay below 2 GiB):
// a load from it returns zeros and a store to it is dropped, with no memory
// traffic.  Used to keep loads and stores unconditional.
constexpr unsigned kOffNone = 0x80000000u;

// ---------------------------------------------------------------------------
// Gate maps.  The decay and write gates arrive as values (alpha in (0, 1],
// beta) or as logits a, b with alpha = exp(-softplus(a)), beta = sigmoid(b).
// The scan needs log2 alpha; from a logit it is formed directly,
// -softplus(a) / ln 2 = -(max(a, 0) + log(1 + exp(-|a|))) / ln 2, which
// stays exact where alpha rounds to 1 in fp32.  log2(0) is clamped at -200
// (2^-200 is 0 in fp32, so the state resets as alpha = 0 asks).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float gate_log2_alpha(float x, bool logits) {
    constexpr float kLog2e = 1.4426950408889634f;
    if (!logits) return fmaxf(log2f(x), -200.f);
    const float t = exp2f(-fabsf(x) * kLog2e);                 // exp(-|a|) in (0, 1]
    return -(fmaxf(x, 0.f) * kLog2e + log2f(1.f + t));
}
__device__ __forceinline__ float gate_beta(float x, bool logits) {
    constexpr float kLog2e = 1.4426950408889634f;
    return logits ? 1.f / (1.f + exp2f(-x * kLog2e)) : x;
}

// Output gate (elementwise on out, input dtype): element e of a head's slice.
__device__ __forceinline__ float gate_at(rsrc_t r, unsigned e, bool f32) {
    return f32 ? __builtin_bit_cast(float, buf_load4(r, e * 4u)) : bf16_to_f32(buf_load2(r, e * 2u));
}

// ---------------------------------------------------------------------------
// Cross-lane helpers on DPP (no LDS traffic).
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 ROW_MASK, 0xF, BOUND_ZERO));
}

// Sum over aligned groups of W consecutive lanes (W = 2..64); every lane of
// the group gets the total.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (W >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (W >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (W >= 8) v += dpp<0x141>(v);   // row_half_mirror: other quad of the 8
    if constexpr (W >= 16) v += dpp<0x140>(v);  // row_mirror: other half of the 16
    if constexpr (W >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (W >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Maximum over the 64 lanes of a wave; every lane gets it.  NaN inputs are
// passed over (fmaxf returns the other operand).
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    return fmaxf(v, __shfl_xor(v, 32, 64));
}

// Largest magnitude among the eight bf16 values packed in a 16-byte piece.
__device__ __forceinline__ float maxabs8_bf16(const uint4& raw) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w[j] << 16)), fabsf(__uint_as_float(w[j] & 0xffff0000u))));
    return m;
}

// Working scale of a walk whose values and state reach magnitude m: the power
// of two 2^floor(log2 m), kept within [2^-100, 2^100]; 1 for m = 0, NaN or
// Inf.  The recurrence is linear in (v, S), so a walk may run on v / s and
// S / s and multiply its outputs and final state by s: exact in binary
// floating point, and it keeps the fp16 operands formed from the state and
// from v near magnitude 1 whatever the scale of the inputs.
__device__ __forceinline__ float pow2_scale(float m) {
    if (!(m > 0.f) || !(m <= 3.0e38f)) return 1.f;
    int e;
    (void)frexpf(m, &e);                 // m = f 2^e, f in [0.5, 1)
    e = min(100, max(-100, e - 1));
    return ldexpf(1.f, e);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_prefix_sum(float v) {
    v += dpp<0x111, 0xF, true>(v);   // row_shr:1
    v += dpp<0x112, 0xF, true>(v);   // row_shr:2
    v += dpp<0x114, 0xF, true>(v);   // row_shr:4
    v += dpp<0x118, 0xF, true>(v);   // row_shr:8
    v += dpp<0x142, 0xA>(v);         // row_bcast:15 into rows 1 and 3
    v += dpp<0x143, 0xC>(v);         // row_bcast:31 into rows 2 and 3
    return v;
}

// 16x16 block transpose through the matrix core: with B = I the product
// A * I returns A in accumulator layout, i.e. lane (g, c) receives
// a[4g+i][c] (i < 4) -- column c of the block, four consecutive rows.  The
// products are exact (one nonzero term per output).
template <class Op>
__device__ __forceinline__ f32x4 transpose16(const typename Op::elem* a, int lda, int lane) {
    const int lc = lane & 15, lg = lane >> 4;
    if constexpr (Op::KSTEP == 4) {
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = Op::mma(a[lc * lda + 4 * s + lg], (4 * s + lg == lc) ? 1.f : 0.f, acc);
        return acc;
    } else {
        auto fa = Op::load16(a + lc * lda + 4 * lg);
        u16x4 one;
#pragma unroll
        for (int j = 0; j < 4; ++j) one[j] = (4 * lg + j == lc) ? (uint16_t)0x3C00 : (uint16_t)0;
        return Op::mma16(fa, one, zero4());
    }
}

// 16x16 tile += A[16 x 16] * B, A row-major in LDS (k contiguous), B given
// as an accumulator tile (rows = k).  For K = 16 the x16 fp16 instruction's
// operand order already matches the accumulator rows.
template <class Op>
__device__ __forceinline__ f32x4 mm_k16_acc(const typename Op::elem* a, int lda, f32x4 b, f32x4 acc,
                                            int lane) {
    if constexpr (Op::KSTEP == 4) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = Op::mma(a[(lane & 15) * lda + 4 * (lane >> 4) + s], b[s], acc);
        return acc;
    } else {
        auto fa = Op::load16(a + (lane & 15) * lda + (lane >> 4) * Op::KPER16);
        u16x4 fb;
#pragma unroll
        for (int i = 0; i < 4; ++i) fb[i] = __builtin_bit_cast(uint16_t, (_Float16)b[i]);
        return Op::mma16(fa, fb, acc);
    }
}

// 16x16 tile += A[16 x 16] * B[16 x 16] with A row-major (k contiguous) and B
// stored column-major ([n][k], k contiguous), both in LDS.
template <class Op>
__device__ __forceinline__ f32x4 mm_k16(const typename Op::elem* a, int lda,
                                        const typename Op::elem* b, int ldb, f32x4 acc, int lane) {
    if constexpr (Op::KSTEP == 4) {
#pragma unroll
        for (int kb = 0; kb < 16; kb += 4)
            acc = Op::mma(a[(lane & 15) * lda + kb + (lane >> 4)], b[(lane & 15) * ldb + kb + (lane >> 4)], acc);
        return acc;
    } else {
        auto fa = Op::load16(a + (lane & 15) * lda + (lane >> 4) * Op::KPER16);
        auto fb = Op::load16(b + (lane & 15) * ldb + (lane >> 4) * Op::KPER16);
        return Op::mma16(fa, fb, acc);
    }
}

}  // namespace gdn
