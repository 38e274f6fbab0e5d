// Router: top-k over the router logits, then a softmax over the k chosen.
//
// Logits are sums of fp16 x fp32 products, each exact in fp64, summed in
// fp64.  Three launch shapes:
//  * A few tokens over a small router matrix (route_fused_kernel): a
//    workgroup takes one token, its 16 waves sum the logits of every expert
//    on the vector fp64 units into LDS and it selects from there, so no logit
//    leaves the CU and the layer pays one launch.  The matrix cores would pad
//    one token to sixteen.
//  * Otherwise the logits run on the fp64 matrix cores (logits_kernel):
//    v_mfma_f64_16x16x4 takes a 16-token x 16-expert tile four hidden columns
//    at a time.  A workgroup of 16 waves owns one (token tile, expert tile,
//    K chunk); the hidden dimension is cut into 32-column units dealt evenly
//    to the KC * 16 waves of a tile, and lane (r, g) = (lane % 16, lane / 16)
//    loads 8 columns of token row r (one 16-byte load) and of expert row r
//    (two) per unit, the lane groups g = 0..3 being the four K rows of the
//    eight matrix steps.  The 16 wave tiles meet in LDS in wave order.
//  * When one expert tile and one chunk cover a token tile, that workgroup
//    selects at once (wave w: token w); otherwise it stores its partial tile
//    and select_kernel (one wave per token) adds the KC partials in chunk
//    order, so a logit never depends on scheduling, and selects.  A second
//    launch is cheaper here than a last-arriving-workgroup finish: the
//    agent-scope fences that would make the partials visible across XCDs
//    cost more than the launch.
// Selection: k rounds of a wave-wide argmax (ties to the lower expert), then
// the softmax over the k chosen logits in fp64.  Token norms (fp32 squares in
// a fixed order) come from the x values already loaded: the waves of expert
// tile 0, or of expert group 0 in the one-token kernel.
#include "common.hpp"

namespace apmoe {
namespace {

constexpr int kRt = 16;        // tokens and experts per tile
constexpr int kRtWaves = 16;   // waves per workgroup
constexpr int kUnit = 32;      // hidden columns per unit (four lane groups x 8)

typedef double double4v_t __attribute__((ext_vector_type(4)));
typedef float float4v_t __attribute__((ext_vector_type(4)));

// Wave-wide argmax of (v, e), ties to the lower e, in two reductions: the
// maximum of v (DPP within rows, then the four row results), then the lowest e
// among the lanes that hold it.  Every lane ends with the winner.  (Given
// each lane's own best with its lowest e, the lowest e of the lanes holding
// the maximum is the lowest e of all the entries equal to it.)
__device__ __forceinline__ double wave_max_f64(double v) {
    v = fmax(v, dpp64<kDppQuad1032>(v));
    v = fmax(v, dpp64<kDppQuad2301>(v));
    v = fmax(v, dpp64<kDppRowHalfMirror>(v));
    v = fmax(v, dpp64<kDppRowMirror>(v));
    return fmax(fmax(lane_f64(v, 0), lane_f64(v, 16)), fmax(lane_f64(v, 32), lane_f64(v, 48)));
}
__device__ __forceinline__ int wave_min_i32(int e) {
    e = min(e, (int)dpp32<kDppQuad1032>((uint32_t)e));
    e = min(e, (int)dpp32<kDppQuad2301>((uint32_t)e));
    e = min(e, (int)dpp32<kDppRowHalfMirror>((uint32_t)e));
    e = min(e, (int)dpp32<kDppRowMirror>((uint32_t)e));
    return min(min((int)lane_u32((uint32_t)e, 0), (int)lane_u32((uint32_t)e, 16)),
               min((int)lane_u32((uint32_t)e, 32), (int)lane_u32((uint32_t)e, 48)));
}
__device__ __forceinline__ void wave_argmax(double& v, int& e) {
    const double m = wave_max_f64(v);
    e = wave_min_i32(v == m ? e : 0x7FFFFFFF);
    v = m;
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

// Grid: blockIdx.x = (tt * ET + et) * KC + kc.  part: [TT][KC][16][16 ET]
// fp64 partial logits and npart: [TT][KC][16] fp32 partial squares (both only
// when ET * KC > 1, for select_kernel).
__global__ __launch_bounds__(kRtWaves * kWave) void logits_kernel(
    const half_t* __restrict__ x, int T, int H, const float* __restrict__ w_router, const float* __restrict__ bias,
    float scale, int E, int k, int ET, int KC, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    float* __restrict__ norms, double* __restrict__ part, float* __restrict__ npart) {
    __shared__ double red[kRtWaves * kRt * kRt];   // the waves' tiles, then the token tile's logits [16][16]
    __shared__ float nred[kRtWaves][4][kRt];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int r = lane % kRt, g = lane / kRt;
    const int kc = blockIdx.x % KC;
    const int et = (blockIdx.x / KC) % ET;
    const int tt = blockIdx.x / KC / ET;
    const int t0 = tt * kRt, e0 = et * kRt;
    const int U = H / kUnit;
    const int slices = KC * kRtWaves, slice = kc * kRtWaves + wave;
    const int u0 = (int)((long long)slice * U / slices), u1 = (int)((long long)(slice + 1) * U / slices);
    const bool nrm = norms && et == 0;   // uniform over the workgroup
    // the biases the in-place selection adds (ET * KC == 1), loaded now so
    // that no load waits at the end (clamped index, no per-lane condition)
    constexpr int kPer = APMOE_MAX_EXPERTS / kWave;
    float bv[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) bv[c] = (bias && ET * KC == 1) ? bias[min(lane + kWave * c, E - 1)] : 0.f;
    // rows past T or E read a valid row; their sums are never used
    const half_t* xr = x + (size_t)min(t0 + r, T - 1) * H + 8 * g;
    const float* wr = w_router + (size_t)min(e0 + r, E - 1) * H + 8 * g;
    // one unit's loads in flight while the previous unit is multiplied (46
    // VGPRs: two 16-wave workgroups fit a CU); two accumulators halve the
    // dependent MFMA chain and meet in a fixed order
    half8_t xn = {};
    float4_t wan = {}, wbn = {};
    if (u0 < u1) {
        xn = *reinterpret_cast<const half8_t*>(xr + (size_t)kUnit * u0);
        wan = *reinterpret_cast<const float4_t*>(wr + (size_t)kUnit * u0);
        wbn = *reinterpret_cast<const float4_t*>(wr + (size_t)kUnit * u0 + 4);
    }
    double4v_t acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = acc0;
    float sq = 0.f;
    for (int u = u0; u < u1; ++u) {
        const half8_t xv = xn;
        const float4_t wa = wan, wb = wbn;
        if (u + 1 < u1) {
            xn = *reinterpret_cast<const half8_t*>(xr + (size_t)kUnit * (u + 1));
            wan = *reinterpret_cast<const float4_t*>(wr + (size_t)kUnit * (u + 1));
            wbn = *reinterpret_cast<const float4_t*>(wr + (size_t)kUnit * (u + 1) + 4);
        }
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[i], (double)(i < 4 ? wa[i] : wb[i - 4]), acc0,
                                                        0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[i + 1], (double)(i < 4 ? wa[i + 1] : wb[i - 3]),
                                                        acc1, 0, 0, 0);
        }
        if (nrm)
#pragma unroll
            for (int i = 0; i < 8; ++i) sq = fmaf((float)xv[i], (float)xv[i], sq);
    }
    const double4v_t acc = acc0 + acc1;
    // the fp64 16x16 result: lane (r, g) holds tokens g, g + 4, g + 8, g + 12 of
    // the tile for expert r (register v is token 4v + g)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave * kRt * kRt + (4 * v + g) * kRt + r] = acc[v];
    if (nrm) nred[wave][g][r] = sq;
    __syncthreads();
    const int i = threadIdx.x;   // element (token i / 16, expert i % 16) of the tile
    double tile = 0.0;
    float nq = 0.f;
    if (i < kRt * kRt)
#pragma unroll
        for (int w = 0; w < kRtWaves; ++w) tile += red[w * kRt * kRt + i];
    if (nrm && i < kRt)
#pragma unroll
        for (int w = 0; w < kRtWaves; ++w) nq += (nred[w][0][i] + nred[w][1][i]) + (nred[w][2][i] + nred[w][3][i]);
    if (ET * KC > 1) {   // uniform: select_kernel finishes
        double* pt = part + (size_t)(tt * KC + kc) * kRt * (ET * kRt);
        if (i < kRt * kRt) pt[(i / kRt) * (ET * kRt) + e0 + i % kRt] = tile;
        if (nrm && i < kRt) npart[(size_t)(tt * KC + kc) * kRt + i] = nq;
        return;
    }
    double* L = red;   // [16][16]
    __syncthreads();   // every wave has read red
    if (i < kRt * kRt) L[i] = tile;
    if (nrm && i < kRt && t0 + i < T) norms[t0 + i] = sqrtf(nq);
    constexpr int Ep = kRt;
    __syncthreads();
    const int t = t0 + wave;
    if (t >= T) return;   // uniform over the wave; no barrier follows
    double* row = L + wave * Ep;
    double v[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        const int e = lane + kWave * c;
        v[c] = e < E ? (double)scale * (row[e] + (double)bv[c]) : -__builtin_inf();
    }
    // the row is this wave's alone from here: its first k entries take the chosen logits
    select_topk<kPer>(v, E, k, t, lane, row, topk_ids, topk_w);
}

// Fused router: TB tokens per workgroup, all E logits in LDS, then select.
// Sixteen waves: wave w sums the hidden-dimension quarter w % 4 for the
// expert group w / 4 (experts in chunks of EC, chunk g, g + 4, ...), its lanes
// splitting the quarter as in the logits kernel; the four quarter sums of a
// logit then meet in a fixed order.  Dynamic LDS: P[4][TB][E] quarter sums
// (P[0] becomes the logits), then k chosen logits per wave.
constexpr int kFWaves = 16;
template <int TB>
__global__ __launch_bounds__(kFWaves * kWave) void route_fused_kernel(const half_t* __restrict__ x, int T, int H,
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

// One wave per token of the logits kernel's partial tiles: the KC partials
// of each logit added in chunk order, then the selection.
constexpr int kSelWaves = 1;   // one-wave workgroups spread the tokens over the most CUs

__global__ __launch_bounds__(kSelWaves * kWave) void select_kernel(const double* __restrict__ part,
                                                                    const float* __restrict__ npart, int T, int E,
                                                                    int k, int ET, int KC,
                                                                    const float* __restrict__ bias, float scale,
                                                                    int32_t* __restrict__ topk_ids,
                                                                    float* __restrict__ topk_w,
                                                                    float* __restrict__ norms) {
    __shared__ double chosen[kSelWaves][APMOE_MAX_EXPERTS];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * kSelWaves + wave;
    if (t >= T) return;   // uniform over the wave; no block barrier follows
    const int tt = t / kRt, tr = t % kRt, Ep = ET * kRt;
    const double* p0 = part + ((size_t)tt * KC * kRt + tr) * Ep;
    // the first 64 norm partials (lane q: chunk q) go out with the logits'
    // loads, so the norm adds no second memory round trip
    const float pv0 = (norms && lane < KC) ? npart[((size_t)tt * KC + lane) * kRt + tr] : 0.f;
    constexpr int kPer = APMOE_MAX_EXPERTS / kWave;
    // each logit adds its KC partials in chunk order; the loads carry no
    // condition (columns past Ep re-read column Ep - 1, never used), so the
    // compiler issues a whole unrolled group of them before the first add
    double v[kPer];
    int ec[kPer];
    float bv[kPer];   // biases, loaded with the partials (clamped index, no per-lane condition)
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        v[c] = 0.0;
        ec[c] = min(lane + kWave * c, Ep - 1);
        bv[c] = bias ? bias[min(lane + kWave * c, E - 1)] : 0.f;
    }
    constexpr int kQB = 4;   // chunks whose loads go out together
    for (int q0 = 0; q0 < KC; q0 += kQB) {
        double tq[kQB][kPer];
#pragma unroll
        for (int j = 0; j < kQB; ++j) {
            const double* pq = p0 + (size_t)min(q0 + j, KC - 1) * kRt * Ep;
#pragma unroll
            for (int c = 0; c < kPer; ++c) tq[j][c] = pq[ec[c]];
        }
#pragma unroll
        for (int j = 0; j < kQB; ++j)
            if (q0 + j < KC)   // uniform
#pragma unroll
                for (int c = 0; c < kPer; ++c) v[c] += tq[j][c];
    }
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
        const int e = lane + kWave * c;
        v[c] = e < E ? (double)scale * (v[c] + (double)bv[c]) : -__builtin_inf();
    }
    if (norms) {   // lane q loads chunk q's partial; the wave adds them in chunk order
        float sm = 0.f;
        for (int q0 = 0; q0 < KC; q0 += kWave) {
            const int q = q0 + lane;
            const float pv = q0 == 0 ? pv0 : (q < KC ? npart[((size_t)tt * KC + q) * kRt + tr] : 0.f);
            const int n = min(kWave, KC - q0);
            for (int j = 0; j < n; ++j)
                sm += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), j));
        }
        if (lane == 0) norms[t] = sqrtf(sm);
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

// Matrix-core shape: TT token tiles x ET expert tiles x KC chunks of the
// hidden dimension.  The fp64 MFMA work of a small router still needs many
// CUs (64 tokens x 60 experts x 2048 on 16 CUs take 3.4 us of MFMA time), so
// KC aims at about 256 workgroups, as far as every wave keeps a unit.
struct RoutePlan {
    int TT, ET, KC;
    size_t part_bytes;   // partial logits + partial squares (0: one launch)
};

RoutePlan route_plan(int T, int E, int H) {
    RoutePlan p{};
    p.TT = (T + kRt - 1) / kRt;
    p.ET = (E + kRt - 1) / kRt;
    const long long J = (long long)p.TT * p.ET;
    const int U = H / kUnit;
    p.KC = (int)std::min<long long>((256 + J - 1) / J, std::max(1, U / kRtWaves));
    if ((long long)p.ET * p.KC > 1) {
        const size_t logits = (size_t)p.TT * p.KC * kRt * p.ET * kRt * sizeof(double);
        const size_t sq = (size_t)p.TT * p.KC * kRt * sizeof(float);
        p.part_bytes = (logits + sq + 255) / 256 * 256;
    }
    return p;
}

// The most any router of up to E experts needs (the need is not monotone in
// E, and one workspace may serve a router over fewer experts than it was
// sized for).
size_t route_workspace_bytes(int T, int E, int H) {
    if (T <= 0 || E <= 0 || H <= 0) return 0;
    size_t m = 0;
    for (int e = 1; e <= E; ++e)
        if (!fused_tokens(T, e, H)) m = std::max(m, route_plan(T, e, H).part_bytes);
    return m;
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
    if ((uintptr_t)x % 16 || (uintptr_t)w_router % 16) return APMOE_EINVAL;
    if ((long long)T * k > (1ll << 30)) return APMOE_EINVAL;
    hipStream_t s = as_stream(stream);
    const half_t* xh = reinterpret_cast<const half_t*>(x);
    if (fused_tokens(T, E, H)) {
        clear_stale_error();
        hipLaunchKernelGGL(route_fused_kernel<1>, dim3(T), dim3(kFWaves * kWave), (4 * E + kFWaves * k) * sizeof(double),
                           s, xh, T, H, w_router, bias, logit_scale, E, k, topk_ids, topk_w, x_norms);
        return launch_status();
    }
    const RoutePlan p = route_plan(T, E, H);
    double* part = nullptr;
    float* npart = nullptr;
    if (p.part_bytes) {
        if (!ws || (uintptr_t)ws % 8 || ws_bytes < p.part_bytes) return APMOE_ENOSPACE;
        part = reinterpret_cast<double*>(ws);
        npart = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                         (size_t)p.TT * p.KC * kRt * p.ET * kRt * sizeof(double));
    }
    const long long blocks = (long long)p.TT * p.ET * p.KC;
    clear_stale_error();
    hipLaunchKernelGGL(logits_kernel, dim3((unsigned)blocks), dim3(kRtWaves * kWave), 0, s, xh, T, H, w_router, bias,
                       logit_scale, E, k, p.ET, p.KC, topk_ids, topk_w, x_norms, part, npart);
    int rc = launch_status();
    if (rc != APMOE_OK || !p.part_bytes) return rc;
    hipLaunchKernelGGL(select_kernel, dim3((T + kSelWaves - 1) / kSelWaves), dim3(kSelWaves * kWave), 0, s, part,
                       npart, T, E, k, p.ET, p.KC, bias, logit_scale, topk_ids, topk_w, x_norms);
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
        clear_stale_error();
        hipLaunchKernelGGL(norms_kernel, dim3((T + 3) / 4), dim3(4 * kWave), 0, s, reinterpret_cast<const half_t*>(x),
                           T, H, norms);
        const int rc = launch_status();
        if (rc != APMOE_OK) return rc;
    }
    clear_stale_error();
    hipLaunchKernelGGL(stats_kernel, dim3(E), dim3(kStatThreads), 0, s, topk_ids, topk_w, T * k, k, norms, mass,
                       wnorm);
    return launch_status();
}
