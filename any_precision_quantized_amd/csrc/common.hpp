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

int launch_gemv(const GemmArgs& a, hipStream_t s);
int launch_tile(const GemmArgs& a, hipStream_t s);

}  // namespace apmoe
