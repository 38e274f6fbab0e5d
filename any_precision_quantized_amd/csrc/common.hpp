// Internal helpers shared by the libapmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "apmoe.h"

namespace apmoe {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t uint32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
// Largest activation buffer or weight matrix the expert kernels accept: they
// address it with 32-bit byte offsets from raw buffer resources.
constexpr long long kMaxBufferBytes = 1ll << 31;
constexpr int kPlanes = 6;

__host__ __device__ inline bool valid_bits(int b) { return (b >= 3 && b <= 6) || b == 16; }

// Cross-lane moves inside a 16-lane row (DPP: VALU operations, no LDS round
// trip): swap lanes 2i and 2i + 1, swap pairs inside a quad, mirror each
// half row, mirror the row.  Applied in this order, each step combines a lane
// with one holding the rest of its group, so after the four steps every lane
// of a row holds the row's combination; lanes 0, 16, 32 and 48 are then read
// into scalars and combined in a fixed order.  Every lane gets the same
// result, independent of scheduling.
constexpr int kDppQuad1032 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppQuad2301 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int C>
__device__ inline uint32_t dpp32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, C, 0xF, 0xF, true);
}
template <int C>
__device__ inline double dpp64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t r = (uint64_t)dpp32<C>((uint32_t)u) | ((uint64_t)dpp32<C>((uint32_t)(u >> 32)) << 32);
    return __builtin_bit_cast(double, r);
}
template <int C>
__device__ inline float dpp_f(float v) {
    return __builtin_bit_cast(float, dpp32<C>(__builtin_bit_cast(uint32_t, v)));
}
__device__ inline uint32_t lane_u32(uint32_t v, int lane) { return (uint32_t)__builtin_amdgcn_readlane((int)v, lane); }
__device__ inline double lane_f64(double v, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    return __builtin_bit_cast(double, (uint64_t)lane_u32((uint32_t)u, lane) |
                                          ((uint64_t)lane_u32((uint32_t)(u >> 32), lane) << 32));
}

// Wave-wide sums in a fixed order (rows by DPP, then (r0 + r1) + (r2 + r3)).
__device__ inline float wave_sum(float v) {
    v += dpp_f<kDppQuad1032>(v);
    v += dpp_f<kDppQuad2301>(v);
    v += dpp_f<kDppRowHalfMirror>(v);
    v += dpp_f<kDppRowMirror>(v);
    const float r0 = __builtin_bit_cast(float, lane_u32(__builtin_bit_cast(uint32_t, v), 0));
    const float r1 = __builtin_bit_cast(float, lane_u32(__builtin_bit_cast(uint32_t, v), 16));
    const float r2 = __builtin_bit_cast(float, lane_u32(__builtin_bit_cast(uint32_t, v), 32));
    const float r3 = __builtin_bit_cast(float, lane_u32(__builtin_bit_cast(uint32_t, v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ inline double wave_sum(double v) {
    v += dpp64<kDppQuad1032>(v);
    v += dpp64<kDppQuad2301>(v);
    v += dpp64<kDppRowHalfMirror>(v);
    v += dpp64<kDppRowMirror>(v);
    return (lane_f64(v, 0) + lane_f64(v, 16)) + (lane_f64(v, 32) + lane_f64(v, 48));
}

// Inclusive prefix sum over the 64 lanes (Hillis-Steele inside each row by
// row shifts, then row 0's total into row 1, row 2's into row 3, and rows
// 0-1's into rows 2-3 by the row broadcasts).
__device__ inline int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return v;
}

__device__ inline float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// hipGetLastError reports the last error of any earlier HIP call on this
// host thread, not only ours: entry points clear it before their launches so
// that their status reflects those launches alone.
inline void clear_stale_error() { (void)hipGetLastError(); }

inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? APMOE_OK : APMOE_EHIP;
}

// b-bit code of column i (0..31) of a word from the top b plane words.
__device__ inline int code_of(const uint32_t* w, int b, int i) {
    int c = 0;
    for (int p = 0; p < b; ++p) c = (c << 1) | ((w[p] >> i) & 1u);
    return c;
}

// Pointers read out of the device-side descriptor table are generic; these
// global-address-space views let loads through them be global (not flat)
// loads, which count only against vmcnt and so never stall LDS waits.
typedef __attribute__((address_space(1))) const uint32_t gu32_t;
typedef __attribute__((address_space(1))) const half_t gh16_t;
typedef __attribute__((address_space(1))) const uint16_t gu16_t;

__device__ inline half8_t load_h8g(gh16_t* p) {
    return *reinterpret_cast<__attribute__((address_space(1))) const half8_t*>(p);
}

struct MatView {
    gu32_t* planes;   // plane p of row r, word w: planes[(p * rows + r) * W + w]
    gh16_t* lut;      // [rows][1 << b]
    gh16_t* w16;      // [rows][K]
};

// A pointer every lane holds the same value of, in scalar registers: buffer
// resources built from it then need no per-lane loop.
template <class P>
__device__ __forceinline__ P uniform_ptr(P p) {
    const uint64_t u = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return (P)(((uint64_t)hi << 32) | lo);
}

__device__ inline MatView mat_view(const apmoe_mat& m, int b) {
    MatView v;
    v.planes = (gu32_t*)m.planes;
    v.lut = (b >= 3 && b <= 6) ? (gh16_t*)m.lut[b - 3] : nullptr;
    v.w16 = (gh16_t*)m.w16;
    return v;
}

// Packed plane layout: inside each plane slab, the words of 16-row group rg
// are ordered [step][g][i] = canonical word 4*step + g of row 16*rg + i.
__host__ __device__ inline int packed_steps(int cols) { return (cols / 32 + 3) / 4; }
__host__ __device__ inline size_t packed_slab_words(int rows, int cols) {
    return (size_t)rows * 4 * packed_steps(cols);
}
__device__ inline size_t packed_index(int rows, int nsteps, int p, int row, int w) {
    return (size_t)p * rows * 4 * nsteps + ((size_t)(row >> 4) * nsteps + (w >> 2)) * 64 + (w & 3) * 16 + (row & 15);
}

// Internal launchers of the two expert-FFN paths (apmoe_bitplane_lut_gemm).
struct GemmArgs {
    int stage;
    const apmoe_expert* experts;
    const int8_t* bits;
    int E;
    const int32_t* offsets;
    const int32_t* sorted_slots;
    int k;
    const uint16_t* in;
    void* out;
    int T, H, I;
    int mfma_min_tokens;
};

int launch_gemv(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t s);
size_t route_workspace_bytes(int T, int E, int H);
size_t gemv_workspace_bytes(int T, int k, int E, int rows, int K, int nmat);
int launch_tile(const GemmArgs& a, hipStream_t s);

}  // namespace apmoe
