// gd_device.h -- small device helpers shared by the library's kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gd {

// (byte B of w) & 0x3c as one v_and_b32 with an SDWA byte select: a 4-bit
// field held at bits 2..5 of a byte, already multiplied by 4 (a table offset
// in bytes for 4-byte entries).
template <int B>
__device__ __forceinline__ uint32_t grp(uint32_t w) {
    static_assert(B >= 0 && B < 4, "byte select");
    uint32_t r;
    const uint32_t mask = 0x3cu;
    if constexpr (B == 0)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0 src1_sel:DWORD"
            : "=v"(r) : "v"(w), "v"(mask));
    else if constexpr (B == 1)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
            : "=v"(r) : "v"(w), "v"(mask));
    else if constexpr (B == 2)
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 src1_sel:DWORD"
            : "=v"(r) : "v"(w), "v"(mask));
    else
        asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
            : "=v"(r) : "v"(w), "v"(mask));
    return r;
}

// A load of data read exactly once (weights), with the non-temporal hint:
// streamed past the caches that way, such data arrives measurably faster
// than through plain loads. Reused data (activations, tables) takes plain
// loads.
template <typename T>
__device__ __forceinline__ T ld_stream(const T __attribute__((address_space(1))) *p) {
    return __builtin_nontemporal_load(p);
}

}  // namespace gd
