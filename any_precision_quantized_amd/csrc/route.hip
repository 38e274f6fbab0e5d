// Router: top-k over the router logits, then a softmax over the k chosen.
//
// One workgroup (4 waves) per token.  Lanes split the hidden dimension and the
// waves split the experts: wave w accumulates, for experts e = w, w+4, ...,
// the products of its lanes' slice in fp64 (fp16 x fp32 products are exact in
// fp64), up to 16 experts at once so their loads overlap.  Per-lane partials meet in
// LDS and one thread per expert adds the 64 lane partials in lane order, so
// the logit is a fixed-order fp64 sum.  Then one wave runs k rounds of a
// wave-wide argmax (ties to the lower expert) and the softmax over the k.
#include "common.hpp"

namespace apmoe {

constexpr int kRouteWaves = 4;
constexpr int kRouteChunk = 64;      // experts reduced per LDS round

__global__ __launch_bounds__(kRouteWaves * kWave) __attribute__((amdgpu_waves_per_eu(1, 2))) void route_kernel(
    const half_t* __restrict__ x, int T, int H, const float* __restrict__ w_router,
    const float* __restrict__ bias, float scale, int E, int k, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w) {
    __shared__ double red[kRouteChunk][kWave + 1];
    __shared__ double logits[APMOE_MAX_EXPERTS];
    __shared__ double chosen[APMOE_MAX_EXPERTS];
    const int t = blockIdx.x;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const half_t* xt = x + (size_t)t * H;

    // Experts in chunks of 64 (one LDS round each); wave w owns experts
    // c0 + w + 4 j, j < 16, and walks H eight columns per lane at a time with
    // every load of the chunk independent.
    const int uw = __builtin_amdgcn_readfirstlane(wave);
    for (int c0 = 0; c0 < E; c0 += kRouteChunk) {
        const int ce = min(kRouteChunk, E - c0);
        double acc[kRouteChunk / kRouteWaves];
#pragma unroll
        for (int j = 0; j < kRouteChunk / kRouteWaves; ++j) acc[j] = 0.0;
        for (int h0 = 0; h0 < H; h0 += 8 * kWave) {
            // columns past H: address clamped, activation zero (no branches,
            // so every load of the chunk is in flight at once)
            double xv[8];
            int hc[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int h = h0 + lane + kWave * u;
                hc[u] = min(h, H - 1);
                const double v = (double)xt[hc[u]];
                xv[u] = h < H ? v : 0.0;
            }
#pragma unroll
            for (int j = 0; j < kRouteChunk / kRouteWaves; ++j) {
                // experts past the chunk read a valid row; their sums are dropped below
                const int el = min(uw + kRouteWaves * j, ce - 1);
                const float* w = w_router + (size_t)(c0 + el) * H;
#pragma unroll
                for (int u = 0; u < 8; ++u) acc[j] = fma(xv[u], (double)w[hc[u]], acc[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < kRouteChunk / kRouteWaves; ++j) {
            const int el = uw + kRouteWaves * j;
            if (el < ce) red[el][lane] = acc[j];
        }
        __syncthreads();
        if (threadIdx.x < ce) {
            double s = 0.0;
            for (int l = 0; l < kWave; ++l) s += red[threadIdx.x][l];
            const int e = c0 + threadIdx.x;
            logits[e] = (double)scale * (s + (bias ? (double)bias[e] : 0.0));
        }
        __syncthreads();
    }
    if (wave != 0) return;   // no block barrier follows

    for (int j = 0; j < k; ++j) {
        double best = -__builtin_inf();
        int best_e = E;
        for (int e = lane; e < E; e += kWave) {
            const double v = logits[e];
            if (v > best || (v == best && e < best_e)) { best = v; best_e = e; }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const double ov = __shfl_xor(best, o, kWave);
            const int oe = __shfl_xor(best_e, o, kWave);
            if (ov > best || (ov == best && oe < best_e)) { best = ov; best_e = oe; }
        }
        if (lane == 0) {
            chosen[j] = best;
            logits[best_e] = -__builtin_inf();
            topk_ids[(size_t)t * k + j] = best_e;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (lane == 0) {
        const double lmax = chosen[0];
        double sum = 0.0;
        for (int j = 0; j < k; ++j) sum += exp(chosen[j] - lmax);
        for (int j = 0; j < k; ++j) topk_w[(size_t)t * k + j] = (float)(exp(chosen[j] - lmax) / sum);
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
    hipLaunchKernelGGL(route_kernel, dim3(T), dim3(kRouteWaves * kWave), 0, as_stream(stream),
                       reinterpret_cast<const half_t*>(x), T, H, w_router, bias, logit_scale, E, k,
                       topk_ids, topk_w);
    return launch_status();
}
