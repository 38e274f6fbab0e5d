// Router: top-k over the router logits, then a softmax over the k chosen.
//
// One wave per token.  Products fp16 x fp32 are exact in fp64 and the sums run
// in fp64 with a fixed butterfly order, so the expert choice only depends on
// logits that differ in the last bits of a double.  The logits sit in LDS while
// k rounds of a wave-wide argmax (ties to the lower expert) pick the top k.
#include "common.hpp"

namespace apmoe {

constexpr int kRouteWaves = 4;  // tokens per workgroup

__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kRouteWaves * kWave) void route_kernel(
    const half_t* __restrict__ x, int T, int H, const float* __restrict__ w_router,
    const float* __restrict__ bias, float scale, int E, int k, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w) {
    __shared__ double logits[kRouteWaves][APMOE_MAX_EXPERTS];
    __shared__ double chosen[kRouteWaves][APMOE_MAX_EXPERTS];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * kRouteWaves + wave;
    if (t >= T) return;  // wave-uniform; the block never synchronises
    const half_t* xt = x + (size_t)t * H;

    for (int e = 0; e < E; ++e) {
        const float* w = w_router + (size_t)e * H;
        double acc = 0.0;
        for (int h = lane; h < H; h += kWave) acc = fma((double)xt[h], (double)w[h], acc);
        acc = wave_sum(acc);
        if (lane == 0) logits[wave][e] = (double)scale * (acc + (bias ? (double)bias[e] : 0.0));
    }
    wave_lds_sync();

    for (int j = 0; j < k; ++j) {
        double best = -__builtin_inf();
        int best_e = E;
        for (int e = lane; e < E; e += kWave) {
            double v = logits[wave][e];
            if (v > best || (v == best && e < best_e)) { best = v; best_e = e; }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            double ov = __shfl_xor(best, o, kWave);
            int oe = __shfl_xor(best_e, o, kWave);
            if (ov > best || (ov == best && oe < best_e)) { best = ov; best_e = oe; }
        }
        if (lane == 0) {
            chosen[wave][j] = best;
            logits[wave][best_e] = -__builtin_inf();
            topk_ids[(size_t)t * k + j] = best_e;
        }
        wave_lds_sync();
    }
    if (lane == 0) {
        const double lmax = chosen[wave][0];
        double sum = 0.0;
        for (int j = 0; j < k; ++j) sum += exp(chosen[wave][j] - lmax);
        for (int j = 0; j < k; ++j)
            topk_w[(size_t)t * k + j] = (float)(exp(chosen[wave][j] - lmax) / sum);
    }
}

}  // namespace apmoe

using namespace apmoe;

extern "C" int apmoe_route(const uint16_t* x, int T, int H, const float* w_router, const float* bias,
                           float logit_scale, int E, int k, int32_t* topk_ids, float* topk_w,
                           void* stream) {
    if (T < 0 || H <= 0 || E < 1 || E > APMOE_MAX_EXPERTS || k < 1 || k > E) return APMOE_EINVAL;
    if (!(logit_scale > 0.0f)) return APMOE_EINVAL;
    if (T == 0) return APMOE_OK;
    if (!x || !w_router || !topk_ids || !topk_w) return APMOE_EINVAL;
    dim3 grid((T + kRouteWaves - 1) / kRouteWaves);
    hipLaunchKernelGGL(route_kernel, grid, dim3(kRouteWaves * kWave), 0, as_stream(stream),
                       reinterpret_cast<const half_t*>(x), T, H, w_router, bias, logit_scale, E, k,
                       topk_ids, topk_w);
    return launch_status();
}
