// device_common.h -- small device helpers shared by the libw4a16 HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

constexpr int kWave = 64;

// bf16 / fp16 bit patterns <-> fp32.  Widening is exact; narrowing rounds to nearest even
// (gfx950 v_cvt_pk_bf16_f32 and v_cvt_f16_f32, denormals kept).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// Two fp32 values -> one dword holding two bf16, `lo` in bits 0..15 (one v_cvt_pk_bf16_f32).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
}

// fp32 dot of two bf16 pairs plus an accumulator: v_dot2c_f32_bf16.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}
// fp32 dot of two fp16 pairs plus an accumulator: v_dot2c_f32_f16.
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

// DPP lane moves (GFX9 encodings).  Lanes that the row mask disables, or that read outside
// the row, receive `old` = 0.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask,
                                                                 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// Sum over the 16 lanes of each DPP row; every lane of the row gets the row's total.
// The order of additions is fixed, so the result is bitwise reproducible.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f32<kDppQuadXor1>(v);
    v += dpp_f32<kDppQuadXor2>(v);
    v += dpp_f32<kDppRowHalfMirror>(v);
    v += dpp_f32<kDppRowMirror>(v);
    return v;
}

// Sum over all 64 lanes, returned wave-uniform (read from lane 63).
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    v += dpp_f32<kDppRowBcast15, 0xA>(v);
    v += dpp_f32<kDppRowBcast31, 0xC>(v);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Orders one wave's own LDS accesses where its lanes exchange values through LDS: the writes
// before the barrier are complete and visible to every lane of the wave before the reads after
// it (and reads before it complete before later writes).  Wavefront scope: the hardware already
// runs one wave's LDS operations in order, so this only keeps the compiler from moving LDS
// accesses across it and costs no instruction.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace w4a16
