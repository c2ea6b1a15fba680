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
};

// Fragment of a row-major LDS array (row stride `ld` elements): rows
// [row0, row0+16), k block starting at kb.
template <class Op>
__device__ __forceinline__ typename Op::frag frag_at(const typename Op::elem* base, int ld,
                                                     int row0, int kb, int lane) {
    return Op::load(base + (row0 + (lane & 15)) * ld + kb + (lane >> 4) * Op::KPER);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

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
