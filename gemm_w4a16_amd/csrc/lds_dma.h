// lds_dma.h -- direct-to-LDS copies and their waits, and the exact B-fragment dequant, shared by
// the kernels that stage operands in LDS (gfx950 only).
#pragma once

#include "device_common.h"

namespace w4a16 {

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Direct-to-LDS copies: lane l reads 16 (or 4) bytes at sbase + voff and the load unit writes
// them to LDS byte m0 + 16 l (or 4 l), with m0 = lds + kImm.  They are issued from inline
// assembly so that the compiler does not track them: it cannot tell LDS stages apart and would
// wait for every copy in flight before any LDS access.  The only waits for them are explicit
// wait_vm<n>() calls, placed by count.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int kImm = 0>
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds) {
    if constexpr (kImm == 0)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
                     : "memory", "m0");
    else
        asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds),
                     "n"(kImm)
                     : "memory", "m0", "scc");
}
template <int kImm = 0>
__device__ __forceinline__ void dma4(uint32_t voff, const void* sbase, uint32_t lds) {
    if constexpr (kImm == 0)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
                     : "memory", "m0");
    else
        asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds),
                     "n"(kImm)
                     : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(n): at most n of this wave's global loads and copies are still in flight (they
// complete in issue order as far as the counter is concerned).
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | 0x0F70 /* expcnt, lgkmcnt: no wait */);
}

// One dequantized word: 8 k of one column -> 16 bytes of bf16, w_hat = bf16_rne(fmaf(q, s, m)).
// Each byte of w & 0x0F0F0F0F (codes 0, 2, 4, 6) and of (w >> 4) & 0x0F0F0F0F (codes 1, 3, 5, 7)
// read as an OCP fp8 e4m3 value is exactly q * 2^-9 (codes 0..7 are the subnormals m * 2^-9,
// codes 8..15 the normals of exponent field 1, (8 + m) * 2^-9), so one scaled conversion, whose
// scale applies only its power of two, yields two exact fp32 codes.  The mask arrives as a
// kernel argument.
__device__ __forceinline__ uint4 dequant_word(uint32_t w, uint32_t mlo, float s, float m) {
    const uint32_t ev = w & mlo, od = (w >> 4) & mlo;
    const f32x2_t q02 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 512.0f, false);
    const f32x2_t q46 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ev, 512.0f, true);
    const f32x2_t q13 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(od, 512.0f, false);
    const f32x2_t q57 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(od, 512.0f, true);
    const float v0 = __builtin_fmaf(q02.x, s, m), v2 = __builtin_fmaf(q02.y, s, m);
    const float v4 = __builtin_fmaf(q46.x, s, m), v6 = __builtin_fmaf(q46.y, s, m);
    const float v1 = __builtin_fmaf(q13.x, s, m), v3 = __builtin_fmaf(q13.y, s, m);
    const float v5 = __builtin_fmaf(q57.x, s, m), v7 = __builtin_fmaf(q57.y, s, m);
    return make_uint4(pack2_bf16(v0, v1), pack2_bf16(v2, v3), pack2_bf16(v4, v5), pack2_bf16(v6, v7));
}

}  // namespace w4a16
