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
constexpr int kPlanes = 6;

__host__ __device__ inline bool valid_bits(int b) { return (b >= 3 && b <= 6) || b == 16; }

// Wave-wide sum in a fixed order (xor butterfly), so every lane gets the same
// bit-identical total regardless of scheduling.
__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ inline float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

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
