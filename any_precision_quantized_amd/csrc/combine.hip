// Weighted scatter-combine, the bitwidth-table commit and the small host entry points.
#include "common.hpp"

namespace apmoe {

// out[t][h] = sum_j w[t][j] * Y[pos[t*kk + nsh + j]][h]
//           + sum_{j < nsh} Y[pos[t*kk + j]][h] (+ y_shared[t][h]), kk = k + nsh,
// fp32 in that order (routed in ascending j, then the always-on parts), one
// rounding to fp16.  One thread per 4 consecutive h.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Y,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ w, int T, int k, int nsh,
                                                      int H, const float* __restrict__ ysh,
                                                      half_t* __restrict__ out) {
    const int t = blockIdx.y;
    const int h = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (t >= T || h >= H) return;
    const size_t kk = (size_t)(k + nsh);
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    // unrolled by 4 so a thread has four rows' loads in flight (the sums keep
    // their order): at 64 tokens x (4 + 4) rows x 2048 the launch, timed with
    // HIP events, went 7.3 -> 6.5 us
#pragma unroll 4
    for (int j = 0; j < k; ++j) {
        const float g = w[(size_t)t * k + j];
        const float4_t y = *reinterpret_cast<const float4_t*>(Y + (size_t)pos[t * kk + nsh + j] * H + h);
        acc = acc + g * y;
    }
#pragma unroll 4
    for (int j = 0; j < nsh; ++j) acc = acc + *reinterpret_cast<const float4_t*>(Y + (size_t)pos[t * kk + j] * H + h);
    if (ysh) acc = acc + *reinterpret_cast<const float4_t*>(ysh + (size_t)t * H + h);
    half4_t o = {(half_t)acc[0], (half_t)acc[1], (half_t)acc[2], (half_t)acc[3]};
    *reinterpret_cast<half4_t*>(out + (size_t)t * H + h) = o;
}

// Canonical [6][rows][W] planes -> packed layout (one output word per thread,
// so the writes are contiguous).
__global__ __launch_bounds__(256) void pack_planes_kernel(const uint32_t* __restrict__ src, int rows, int cols,
                                                          uint32_t* __restrict__ dst) {
    const int W = cols / 32;
    const int nsteps = packed_steps(cols);
    const size_t slab = packed_slab_words(rows, cols);
    const size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= 6 * slab) return;
    const int p = (int)(o / slab);
    const size_t rem = o % slab;
    const int rg = (int)(rem / ((size_t)nsteps * 64));
    const int r2 = (int)(rem % ((size_t)nsteps * 64));
    const int s = r2 / 64, l = r2 % 64;
    const int w = 4 * s + l / 16;
    const int row = 16 * rg + l % 16;
    dst[o] = w < W ? src[((size_t)p * rows + row) * W + w] : 0u;
}

struct BitsArg {
    int8_t v[APMOE_MAX_EXPERTS];
};

__global__ void commit_bits_kernel(BitsArg bits, int E, int8_t* __restrict__ dst) {
    const int e = threadIdx.x;
    if (e < E) dst[e] = bits.v[e];
}

}  // namespace apmoe

using namespace apmoe;

extern "C" int apmoe_combine(const float* Y, const int32_t* pos_of_slot, const float* topk_w, int T,
                             int k, int n_shared, int H, const float* y_shared, uint16_t* out, void* stream) {
    if (T < 0 || k < 1 || n_shared < 0 || H <= 0 || H % 32) return APMOE_EINVAL;
    if (T == 0) return APMOE_OK;
    if (!Y || !pos_of_slot || !topk_w || !out) return APMOE_EINVAL;
    dim3 grid((H / 4 + 255) / 256, T);
    clear_stale_error();
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, as_stream(stream), Y, pos_of_slot, topk_w,
                       T, k, n_shared, H, y_shared, reinterpret_cast<half_t*>(out));
    return launch_status();
}

extern "C" int apmoe_commit_bits(const int8_t* bits_host, int E, int8_t* bits_dev, void* stream) {
    if (E < 1 || E > APMOE_MAX_EXPERTS || !bits_host || !bits_dev) return APMOE_EINVAL;
    BitsArg a = {};
    for (int e = 0; e < E; ++e) {
        if (!valid_bits(bits_host[e])) return APMOE_EBITS;
        a.v[e] = bits_host[e];
    }
    clear_stale_error();
    hipLaunchKernelGGL(commit_bits_kernel, dim3(1), dim3(APMOE_MAX_EXPERTS), 0, as_stream(stream), a,
                       E, bits_dev);
    return launch_status();
}

extern "C" size_t apmoe_workspace_bytes(int T, int k, int E, int H, int I) {
    if (T <= 0 || k <= 0 || E <= 0 || H <= 0 || I <= 0) return 0;
    const size_t gu = gemv_workspace_bytes(T, k, E, I, H, 2);
    const size_t dn = gemv_workspace_bytes(T, k, E, H, I, 1);
    const size_t rt = route_workspace_bytes(T, E, H);
    const size_t m = gu > dn ? gu : dn;
    return m > rt ? m : rt;
}

extern "C" size_t apmoe_packed_plane_words(int rows, int cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return 6 * packed_slab_words(rows, cols);
}

extern "C" int apmoe_pack_planes(const uint32_t* src, int rows, int cols, uint32_t* dst, void* stream) {
    if (!src || !dst || rows <= 0 || cols <= 0 || rows % 16 || cols % 32) return APMOE_EINVAL;
    const size_t n = apmoe_packed_plane_words(rows, cols);
    const char* s0 = reinterpret_cast<const char*>(src);
    const char* d0 = reinterpret_cast<const char*>(dst);
    const size_t sb = (size_t)6 * rows * (cols / 32) * 4, db = n * 4;
    if (s0 < d0 + db && d0 < s0 + sb) return APMOE_EINVAL;   // overlapping buffers
    clear_stale_error();
    hipLaunchKernelGGL(pack_planes_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, as_stream(stream), src,
                       rows, cols, dst);
    return launch_status();
}

extern "C" const char* apmoe_strerror(int code) {
    switch (code) {
        case APMOE_OK: return "ok";
        case APMOE_EINVAL: return "invalid argument (shape, pointer or stage)";
        case APMOE_EBITS: return "bitwidth outside {3,4,5,6,16}";
        case APMOE_ENOSPACE: return "workspace too small or budget infeasible";
        case APMOE_EHIP: return "HIP runtime error at launch";
        default: return "unknown error";
    }
}
