// ve_device.h -- device-side helpers shared by the kernel files: bf16 <->
// fp32 conversion, vector types, global-memory vector accesses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ve {

// bf16 halves of a dword, widened to fp32 (exact).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values to a bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x2 v = {a, b};
    bf16x2 h = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

// Buffers handed in through pointer tables are generic pointers; they live in
// device global memory, so address them as such (global_* instead of flat_*
// accesses).
#define VE_GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Vector accesses with an optional non-temporal (streaming) hint, used where
// a wave-wide access covers whole cache lines and every byte is touched once.
#ifndef VE_NONTEMPORAL
#define VE_NONTEMPORAL 1
#endif
template <bool NT, class V>
__device__ __forceinline__ V ldv(const VE_GLOBAL V* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT, class V>
__device__ __forceinline__ void stv(VE_GLOBAL V* p, V v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

}  // namespace ve
