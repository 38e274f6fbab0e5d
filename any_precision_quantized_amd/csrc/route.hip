// Router: top-k over the router logits, then a softmax over the k chosen.
//
// A few tokens over a small router matrix run one kernel (route_kernel): a
// workgroup takes one token, computes its logits for every expert
// into LDS and selects from there, so no logit leaves the CU and the layer
// pays one launch.  Everything else runs two kernels.  The logits kernel tiles
// (TB tokens x 8 experts) per workgroup: wave w owns experts 2w, 2w+1 of the
// tile and its lanes split the hidden dimension (four columns each per 256),
// so one 16-byte router-weight load feeds TB tokens and the tile's weights and
// activations cross the CU once.  TB is 4 unless that leaves fewer than two
// workgroups per CU; then 2, or 1 (router load latency is hidden by more
// workgroups, not by longer tiles: at 64 tokens x 60 experts, 512 one-token
// tiles route in 12.2 us against 15.1 us for 128 four-token tiles; at 256
// tokens x 128 experts four-token tiles are the fastest).
// Products and sums are fp64 (an fp16 x fp32 product is exact in fp64); each
// lane's partial sums meet in a fixed reduction order, so a logit never depends
// on scheduling.  The logits go to the workspace; the select kernel then runs
// one wave per token: k rounds of a wave-wide argmax (ties to the lower
// expert), then the softmax over the k chosen logits in fp64.
#include "common.hpp"

namespace apmoe {
namespace {

constexpr int kEPW = 2;                 // experts per wave
constexpr int kRWaves = 4;
constexpr int kEB = kEPW * kRWaves;     // experts per logits tile

typedef float float4v_t __attribute__((ext_vector_type(4)));

template <int kTB>
__global__ __launch_bounds__(kRWaves * kWave) void logits_kernel(const half_t* __restrict__ x, int T, int H,
                                                                  const float* __restrict__ w_router,
                                                                  const float* __restrict__ bias, float scale,
                                                                  int E, double* __restrict__ L,
                                                                  float* __restrict__ norms) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int t0 = blockIdx.x * kTB;
    const int e0 = blockIdx.y * kEB + wave * kEPW;
    // rows past T or E read a valid row; their sums are never written
    const half_t* xr[kTB];
#pragma unroll
    for (int j = 0; j < kTB; ++j) xr[j] = x + (size_t)min(t0 + j, T - 1) * H;
    const float* wr[kEPW];
#pragma unroll
    for (int j = 0; j < kEPW; ++j) wr[j] = w_router + (size_t)min(e0 + j, E - 1) * H;

    double acc[kTB][kEPW];
    float sq[kTB];   // ||x_t||^2 on the first expert tile's first wave (the same order as norms_kernel)
    const bool do_norm = norms && blockIdx.y == 0 && wave == 0;
#pragma unroll
    for (int t = 0; t < kTB; ++t) {
        sq[t] = 0.f;
#pragma unroll
        for (int j = 0; j < kEPW; ++j) acc[t][j] = 0.0;
    }
#pragma unroll 2
    for (int h = 4 * lane; h < H; h += 4 * kWave) {   // H % 32 == 0: h + 3 < H
        float4v_t wv[kEPW];
#pragma unroll
        for (int j = 0; j < kEPW; ++j) wv[j] = *reinterpret_cast<const float4v_t*>(wr[j] + h);
#pragma unroll
        for (int t = 0; t < kTB; ++t) {
            const half4_t xv = *reinterpret_cast<const half4_t*>(xr[t] + h);
#pragma unroll
            for (int j = 0; j < kEPW; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[t][j] = fma((double)xv[c], (double)wv[j][c], acc[t][j]);
            if (do_norm)
#pragma unroll
                for (int c = 0; c < 4; ++c) sq[t] = fmaf((float)xv[c], (float)xv[c], sq[t]);
        }
    }
    if (do_norm)
#pragma unroll
        for (int t = 0; t < kTB; ++t) {
            const float n2 = wave_sum(sq[t]);
            if (lane == 0 && t0 + t < T) norms[t0 + t] = sqrtf(n2);
        }
#pragma unroll
    for (int t = 0; t < kTB; ++t)
#pragma unroll
        for (int j = 0; j < kEPW; ++j) {
            const double s = wave_sum(acc[t][j]);
            const int tt = t0 + t, e = e0 + j;
            if (lane == 0 && tt < T && e < E)
                L[(size_t)tt * E + e] = (double)scale * (s + (bias ? (double)bias[e] : 0.0));
        }
}

// k rounds of a wave-wide argmax over v (lane's experts lane + 64c), ties to
// the lower expert, then the softmax over the chosen logits in fp64: lane j
// takes the exponentials of chosen logits j, j + 64, ... and the wave adds
// them in a fixed order.  chosen: k doubles of LDS for this wave.
template <int kPer>
__device__ __forceinline__ void select_topk(double (&v)[kPer], int E, int k, int t, int lane, double* chosen,
                                            int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
    for (int j = 0; j < k; ++j) {
        double best = -__builtin_inf();
        int best_e = E;
#pragma unroll
        for (int c = 0; c < kPer; ++c) {   // ascending e within the lane: ties keep the lower
            const int e = lane + kWave * c;
            if (e < E && (v[c] > best || (v[c] == best && e < best_e))) { best = v[c]; best_e = e; }
        }
        wave_argmax(best, best_e);
        // every lane holds the same winner; its owner drops it from the race
#pragma unroll
        for (int c = 0; c < kPer; ++c)
            if (lane + kWave * c == best_e) v[c] = -__builtin_inf();
        if (lane == (j & (kWave - 1))) {
            chosen[j] = best;
            topk_ids[(size_t)t * k + j] = best_e;
        }
    }
    // chosen[] was written by other lanes of this wave: order the reads after it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const double lmax = chosen[0];
    double part = 0.0;
    for (int j = lane; j < k; j += kWave) part += exp(chosen[j] - lmax);
    const double sum = wave_sum(part);
    for (int j = lane; j < k; j += kWave) topk_w[(size_t)t * k + j] = (float)(exp(chosen[j] - lmax) / sum);
}

// Fused router: TB tokens per workgroup, all E logits in LDS, then select.
// Sixteen waves: wave w sums the hidden-dimension quarter w % 4 for the
// expert group w / 4 (experts in chunks of EC, chunk g, g + 4, ...), its lanes
// splitting the quarter as in the logits kernel; the four quarter sums of a
// logit then meet in a fixed order.  Dynamic LDS: P[4][TB][E] quarter sums
// (P[0] becomes the logits), then k chosen logits per wave.
constexpr int kFWaves = 16;
template <int TB>
__global__ __launch_bounds__(kFWaves * kWave) void route_kernel(const half_t* __restrict__ x, int T, int H,
                                                                 const float* __restrict__ w_router,
                                                                 const float* __restrict__ bias, float scale, int E,
                                                                 int k, int32_t* __restrict__ topk_ids,
                                                                 float* __restrict__ topk_w, float* __restrict__ norms) {
    constexpr int EC = 8;   // TB * EC <= 16 fp64 accumulators
    __shared__ float sqq[4][TB];   // ||x_t||^2 per hidden quarter
    extern __shared__ double dyn[];
    double* P = dyn;                                      // [4][TB][E]
    double* chosen = dyn + 4 * TB * E;                    // [kFWaves][k]
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int hq = wave & 3, eg = wave >> 2;
    const int Hq = H / 4;                                 // H % 32 == 0: a multiple of 8
    const int t0 = blockIdx.x * TB;
    const half_t* xr[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) xr[t] = x + (size_t)min(t0 + t, T - 1) * H;   // rows past T: a valid row, never used
    // the four quarter waves of expert group 0 also sum x^2 (token norms) over
    // the x values they load for their first expert chunk
    const bool do_norm = norms && eg == 0;
    for (int e0 = eg * EC; e0 < E; e0 += 4 * EC) {
        const bool nrm = do_norm && e0 == 0;
        float sq[TB];
#pragma unroll
        for (int t = 0; t < TB; ++t) sq[t] = 0.f;
        const float* wr[EC];
#pragma unroll
        for (int j = 0; j < EC; ++j) wr[j] = w_router + (size_t)min(e0 + j, E - 1) * H;
        double acc[TB][EC];
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int j = 0; j < EC; ++j) acc[t][j] = 0.0;
        for (int h = hq * Hq + 4 * lane; h < (hq + 1) * Hq; h += 4 * kWave) {
            float4v_t wv[EC];
#pragma unroll
            for (int j = 0; j < EC; ++j) wv[j] = *reinterpret_cast<const float4v_t*>(wr[j] + h);
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                const half4_t xv = *reinterpret_cast<const half4_t*>(xr[t] + h);
#pragma unroll
                for (int j = 0; j < EC; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[t][j] = fma((double)xv[c], (double)wv[j][c], acc[t][j]);
                if (nrm)
#pragma unroll
                    for (int c = 0; c < 4; ++c) sq[t] = fmaf((float)xv[c], (float)xv[c], sq[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int j = 0; j < EC; ++j) {
                const double sm = wave_sum(acc[t][j]);
                const int e = e0 + j;
                if (lane == 0 && e < E) P[(hq * TB + t) * E + e] = sm;
            }
        if (nrm)
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                const float s2 = wave_sum(sq[t]);
                if (lane == 0) sqq[hq][t] = s2;
            }
    }
    __syncthreads();
    if (norms && threadIdx.x < TB && t0 + (int)threadIdx.x < T) {
        const int t = threadIdx.x;
        norms[t0 + t] = sqrtf((sqq[0][t] + sqq[1][t]) + (sqq[2][t] + sqq[3][t]));
    }
    for (int i = threadIdx.x; i < TB * E; i += blockDim.x) {
        const int e = i % E;
        const double sm = (P[i] + P[TB * E + i]) + (P[2 * TB * E + i] + P[3 * TB * E + i]);
        P[i] = (double)scale * (sm + (bias ? (double)bias[e] : 0.0));
    }
    __syncthreads();
    constexpr int kPer = APMOE_MAX_EXPERTS / kWave;
    for (int t = wave; t < TB; t += kFWaves) {
        if (t0 + t >= T) break;   // uniform over the wave; no barrier follows
        double v[kPer];
#pragma unroll
        for (int c = 0; c < kPer; ++c) {
            const int e = lane + kWave * c;
            v[c] = e < E ? P[t * E + e] : -__builtin_inf();
        }
        select_topk<kPer>(v, E, k, t0 + t, lane, chosen + wave * k, topk_ids, topk_w);
    }
}

constexpr int kSelWaves = 1;   // one-wave workgroups spread the tokens over the most CUs

__global__ __launch_bounds__(kSelWaves * kWave) void select_kernel(const double* __restrict__ L, int T, int E, int k,
                                                                    int32_t* __restrict__ topk_ids,
                                                                    float* __restrict__ topk_w) {
    __shared__ double chosen[kSelWaves][APMOE_MAX_EXPERTS];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * kSelWaves + wave;
    if (t >= T) return;   // uniform over the wave; no block barrier follows
    constexpr int kPer = APMOE_MAX_EXPERTS / kWave;
    double v[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        const int e = lane + kWave * c;
        v[c] = e < E ? L[(size_t)t * E + e] : -__builtin_inf();
    }
    select_topk<kPer>(v, E, k, t, lane, chosen[wave], topk_ids, topk_w);
}

// Routing statistics (the planner's online inputs).  norms_kernel: one wave
// per token, ||x_t||_2 with the squares summed in fp32 and met in a fixed
// order.  stats_kernel: one 16-wave workgroup per expert scans the T*k
// slots (thread i takes slots i, i + 1024, ...) adding its gates and gate *
// norm in fp32; lanes meet in a fixed order and the 16 waves in index
// order, so the sums never depend on scheduling.
__global__ __launch_bounds__(4 * kWave) void norms_kernel(const half_t* __restrict__ x, int T, int H,
                                                          float* __restrict__ norms) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;   // uniform over the wave; no barrier follows
    const half_t* xr = x + (size_t)t * H;
    float acc = 0.f;
    for (int h = 4 * lane; h < H; h += 4 * kWave) {   // H % 32 == 0: h + 3 < H
        const half4_t v = *reinterpret_cast<const half4_t*>(xr + h);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = fmaf((float)v[c], (float)v[c], acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) norms[t] = sqrtf(acc);
}

constexpr int kStatWaves = 16;
constexpr int kStatThreads = kStatWaves * kWave;
constexpr int kStatUnroll = 4;

__global__ __launch_bounds__(kStatThreads) void stats_kernel(const int32_t* __restrict__ ids,
                                                             const float* __restrict__ w, int S, int k,
                                                             const float* __restrict__ norms,
                                                             float* __restrict__ mass, float* __restrict__ wnorm) {
    __shared__ float part[2][kStatWaves];
    const int e = blockIdx.x;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    float m = 0.f, n = 0.f;
    for (int s0 = threadIdx.x; s0 < S; s0 += kStatUnroll * kStatThreads) {
        int id[kStatUnroll];   // the unrolled id loads are independent, so they overlap
#pragma unroll
        for (int u = 0; u < kStatUnroll; ++u) {
            const int s = s0 + u * kStatThreads;
            id[u] = s < S ? ids[s] : -1;
        }
#pragma unroll
        for (int u = 0; u < kStatUnroll; ++u) {
            const int s = s0 + u * kStatThreads;
            if (id[u] == e) {
                const float g = w[s];
                m += g;
                n = fmaf(g, norms[s / k], n);
            }
        }
    }
    m = wave_sum(m);
    n = wave_sum(n);
    if (lane == 0) {
        part[0][wave] = m;
        part[1][wave] = n;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float sm = 0.f, sn = 0.f;
        for (int v = 0; v < kStatWaves; ++v) {
            sm += part[0][v];
            sn += part[1][v];
        }
        mass[e] = sm;
        wnorm[e] = sn;
    }
}

}  // namespace

// The fused kernel pays off for a few tokens and a small router matrix:
// every fused workgroup streams the whole matrix through its CU, and each
// (token, expert) sum costs four wave reductions, so with more tokens the
// reductions dominate.  It runs for T <= 32 when the matrix is at most
// 160 KB; otherwise the two-kernel path, whose workgroups split the experts,
// runs.  One token per workgroup: at 32 tokens over a 128 KB matrix, 32
// workgroups of one token route in 11.3 us where 16 of two took 15.2 us; at
// 64 tokens over a 480 KB matrix the fused kernel (16.2 us) no longer beats
// the two kernels (15 us).
int fused_tokens(int T, int E, int H) {
    if (T > 32) return 0;
    const int tb = 1;
    const double wbytes = (double)E * H * 4.0;
    const double lds = (4.0 * tb * E + (double)kFWaves * E) * sizeof(double);
    return (wbytes <= 160.0 * 1024 && lds <= 65536.0) ? tb : 0;
}

size_t route_workspace_bytes(int T, int E, int H) {
    if (T <= 0 || E <= 0 || H <= 0 || fused_tokens(T, E, H)) return 0;
    return (size_t)T * (size_t)E * sizeof(double);
}

}  // namespace apmoe

using namespace apmoe;

extern "C" int apmoe_route(const uint16_t* x, int T, int H, const float* w_router, const float* bias,
                           float logit_scale, int E, int k, int32_t* topk_ids, float* topk_w, float* x_norms,
                           void* ws, size_t ws_bytes, void* stream) {
    if (T < 0 || H <= 0 || H % 32 || E < 1 || E > APMOE_MAX_EXPERTS || k < 1 || k > E) return APMOE_EINVAL;
    if (!(logit_scale > 0.0f)) return APMOE_EINVAL;
    if (T == 0) return APMOE_OK;
    if (!x || !w_router || !topk_ids || !topk_w) return APMOE_EINVAL;
    hipStream_t s = as_stream(stream);
    const half_t* xh = reinterpret_cast<const half_t*>(x);
    switch (fused_tokens(T, E, H)) {
#define APMOE_ROUTE_FUSED(TB_)                                                                                \
    case TB_:                                                                                                 \
        hipLaunchKernelGGL(route_kernel<TB_>, dim3((T + TB_ - 1) / TB_), dim3(kFWaves * kWave),                \
                           (4 * TB_ * E + kFWaves * k) * sizeof(double), s, xh, T, H, w_router, bias, logit_scale, \
                           E, k, topk_ids, topk_w, x_norms);                                                  \
        return launch_status();
        APMOE_ROUTE_FUSED(1)
#undef APMOE_ROUTE_FUSED
        default: break;
    }
    if (!ws || ws_bytes < route_workspace_bytes(T, E, H)) return APMOE_ENOSPACE;
    double* L = reinterpret_cast<double*>(ws);
    const int etiles = (E + kEB - 1) / kEB;
    int ncu = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return APMOE_EHIP;
    auto tiles = [&](int tb) { return (long long)((T + tb - 1) / tb) * etiles; };
    const int tb = tiles(4) >= 2LL * ncu ? 4 : tiles(2) >= 2LL * ncu ? 2 : 1;
    const dim3 grid((T + tb - 1) / tb, etiles);
    if (tb == 4)
        hipLaunchKernelGGL(logits_kernel<4>, grid, dim3(kRWaves * kWave), 0, s, xh, T, H, w_router, bias, logit_scale,
                           E, L, x_norms);
    else if (tb == 2)
        hipLaunchKernelGGL(logits_kernel<2>, grid, dim3(kRWaves * kWave), 0, s, xh, T, H, w_router, bias, logit_scale,
                           E, L, x_norms);
    else
        hipLaunchKernelGGL(logits_kernel<1>, grid, dim3(kRWaves * kWave), 0, s, xh, T, H, w_router, bias, logit_scale,
                           E, L, x_norms);
    int rc = launch_status();
    if (rc != APMOE_OK) return rc;
    hipLaunchKernelGGL(select_kernel, dim3((T + kSelWaves - 1) / kSelWaves), dim3(kSelWaves * kWave), 0, s, L, T, E,
                       k, topk_ids, topk_w);
    return launch_status();
}

extern "C" int apmoe_route_stats(const uint16_t* x, int T, int H, const int32_t* topk_ids, const float* topk_w,
                                 int k, int E, float* mass, float* wnorm, void* ws, size_t ws_bytes,
                                 void* stream) {
    if (T < 0 || H <= 0 || H % 32 || E < 1 || E > APMOE_MAX_EXPERTS || k < 1 || k > E) return APMOE_EINVAL;
    if (!mass || !wnorm) return APMOE_EINVAL;
    if (T > 0 && (!x || !topk_ids || !topk_w)) return APMOE_EINVAL;
    if ((long long)T * k > (1ll << 30)) return APMOE_EINVAL;
    if (T > 0 && (!ws || ws_bytes < (size_t)T * sizeof(float))) return APMOE_ENOSPACE;
    hipStream_t s = as_stream(stream);
    float* norms = reinterpret_cast<float*>(ws);
    if (T > 0) {
        hipLaunchKernelGGL(norms_kernel, dim3((T + 3) / 4), dim3(4 * kWave), 0, s, reinterpret_cast<const half_t*>(x),
                           T, H, norms);
        const int rc = launch_status();
        if (rc != APMOE_OK) return rc;
    }
    hipLaunchKernelGGL(stats_kernel, dim3(E), dim3(kStatThreads), 0, s, topk_ids, topk_w, T * k, k, norms, mass,
                       wnorm);
    return launch_status();
}
