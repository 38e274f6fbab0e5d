// Device helpers shared by the bit-plane decode paths (GEMV and MFMA tiles):
// the in-register bit transpose that turns b plane words into byte-wide codes,
// and raw buffer loads.
#pragma once

#include "common.hpp"

namespace apmoe {

// (x & m) | (y & ~m).  Written as the instruction itself: the compiler
// otherwise re-canonicalises chains of these merges into longer sequences.
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t x, uint32_t y) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(m), "v"(x), "v"(y));
    return r;
}

// One delta-swap stage of distance D over rows r and r + D (r with bit D
// clear): the bits of row r + D selected by m trade places with the bits of
// row r selected by m << D.  NZ marks the rows that may be non-zero, so rows
// known to be zero cost nothing (a lone non-zero row splits in two ops or
// three).
template <int D, int NZ>
__device__ __forceinline__ void swap_stage(uint32_t q[8], uint32_t m) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        if (r & D) continue;
        const bool za = !((NZ >> r) & 1), zb = !((NZ >> (r + D)) & 1);
        if (za && zb) continue;
        const uint32_t hi = m << D;
        if (zb) {
            q[r + D] = (q[r] >> D) & m;
            q[r] &= ~hi;
        } else if (za) {
            q[r] = (q[r + D] << D) & hi;
            q[r + D] &= m;
        } else {
            const uint32_t a = q[r], b = q[r + D];
            q[r] = bfi(hi, b << D, a);
            q[r + D] = bfi(m, a >> D, b);
        }
    }
}

// q[r] holds code bit r of 32 columns (bit i = column i), rows r >= B zero.
// Afterwards byte u of q[s] holds the code of column 8*u + s.  The three
// stages commute; distance 1 and 2 go first, while rows B..7 are still zero.
template <int B>
__device__ __forceinline__ void transpose_bytes(uint32_t q[8]) {
    constexpr int z0 = (1 << B) - 1;
    constexpr int z1 = z0 | ((z0 & 0x55) << 1) | ((z0 & 0xAA) >> 1);
    constexpr int z2 = z1 | ((z1 & 0x33) << 2) | ((z1 & 0xCC) >> 2);
    swap_stage<1, z0>(q, 0x55555555u);
    swap_stage<2, z1>(q, 0x33333333u);
    swap_stage<4, z2>(q, 0x0F0F0F0Fu);
}

// Raw buffer resources: 32-bit byte offsets from a uniform base, and loads
// past num_records bytes return zero.
constexpr int kBufFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kBufFlags);
}
__device__ __forceinline__ uint32_t buf_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, (int)soff, 0);
}
__device__ __forceinline__ half8_t buf_load_h8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(half8_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;   // any offset past num_records reads zeros

}  // namespace apmoe
