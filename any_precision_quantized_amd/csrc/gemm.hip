// Expert FFN stages over bit-plane + LUT weights: apmoe_bitplane_lut_gemm,
// and its dequantise-to-LDS + MFMA tile path (groups of >= mfma_min_tokens).
//
// Dispatch happens on the device: every workgroup reads its expert's slot
// count and bitwidth and leaves at once when the group is empty or belongs to
// the other path, so no count ever travels to the host.
#include "common.hpp"

namespace apmoe {

// ---------------------------------------------------------------------------
// Tile path (groups of at least mfma_min_tokens): the weight tile is decoded
// into LDS as exact fp16 and multiplied with v_mfma_f32_16x16x16_f16.
//   D[token][row] = sum_k X[token][k] * W[row][k]
// Workgroup tile 64 tokens x 64 rows, K step 32, 4 waves each 32 x 32.
// ---------------------------------------------------------------------------

constexpr int kBM = 64, kBN = 64, kBK = 32, kLdsPad = 8;

template <int NMAT>
__global__ __launch_bounds__(256) void tile_simple_kernel(GemmArgs a) {
    const int rows = NMAT == 2 ? a.I : a.H;
    const int K = NMAT == 2 ? a.H : a.I;
    const int W = K / 32;
    const int n0 = blockIdx.x * kBN;

    // Nothing to do unless some group reaches the threshold: one wave-wide
    // vote per 64 experts, before any LDS traffic (uniform over the workgroup).
    {
        const int lane = threadIdx.x % kWave;
        bool any = false;
        for (int c0 = 0; c0 < a.E && !any; c0 += kWave) {
            const int e = c0 + lane;
            const int c = e < a.E ? a.offsets[e + 1] - a.offsets[e] : 0;
            any = __ballot(c >= a.mfma_min_tokens) != 0;
        }
        if (!any) return;
    }
    // Map blockIdx.y to (expert, m-tile) over the groups that take this path
    // (slot counts staged in LDS once, then a scan from LDS).
    __shared__ int cnt[APMOE_MAX_EXPERTS + 1];
    for (int ee = threadIdx.x; ee <= a.E; ee += blockDim.x) cnt[ee] = a.offsets[ee];
    __syncthreads();
    for (int slot = blockIdx.y; slot < a.T * a.k / kBM + a.E; slot += gridDim.y) {
    int q = slot, e = -1, m0 = 0, off = 0, m = 0;
    for (int ee = 0; ee < a.E; ++ee) {
        const int o = cnt[ee], c = cnt[ee + 1] - o;
        if (c < a.mfma_min_tokens || c == 0) continue;
        const int tiles = (c + kBM - 1) / kBM;
        if (q < tiles) { e = ee; m0 = q * kBM; off = o; m = c; break; }
        q -= tiles;
    }
    if (e < 0) break;   // slots past the last tile: uniform over the workgroup
    const int b = a.bits[e];
    if (!valid_bits(b)) continue;
    MatView mv[NMAT];
    if (NMAT == 2) {
        mv[0] = mat_view(a.experts[e].gate, b);
        mv[NMAT - 1] = mat_view(a.experts[e].up, b);
    } else {
        mv[0] = mat_view(a.experts[e].down, b);
    }
    const half_t* in = reinterpret_cast<const half_t*>(a.in);

    __shared__ half_t xs[kBM][kBK + kLdsPad];
    __shared__ half_t ws[NMAT][kBN][kBK + kLdsPad];

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / 2, wn = wave % 2;  // 32 x 32 sub-tile of the wave
    float4_t acc[NMAT][2][2];
    for (int qq = 0; qq < NMAT; ++qq)
        for (int i = 0; i < 2; ++i)
            for (int j = 0; j < 2; ++j) acc[qq][i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

    // Loader roles: thread -> (row or token = tid / 4, eight columns at 8 * (tid % 4)).
    const int lr = tid / 4, lc = 8 * (tid % 4);
    const int tok = m0 + lr;
    const half_t* xsrc = nullptr;
    if (tok < m) {
        const int j = off + tok;
        xsrc = NMAT == 2 ? in + (size_t)(a.sorted_slots[j] / a.k) * K : in + (size_t)j * K;
    }
    const int wrow = n0 + lr;

    for (int kw = 0; kw < W; ++kw) {
        // activations
        half8_t xv = {0, 0, 0, 0, 0, 0, 0, 0};
        if (xsrc) xv = *reinterpret_cast<const half8_t*>(xsrc + 32 * kw + lc);
        // weights
        half8_t wv[NMAT];
        for (int qq = 0; qq < NMAT; ++qq) {
            half8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
            if (wrow < rows) {
                if (b == 16) {
                    v = load_h8g(mv[qq].w16 + (size_t)wrow * K + 32 * kw + lc);
                } else {
                    uint32_t pw[6];
                    for (int p = 0; p < b; ++p) pw[p] = mv[qq].planes[packed_index(rows, packed_steps(K), p, wrow, kw)];
                    gh16_t* lut = mv[qq].lut + (size_t)wrow * (1 << b);
                    for (int i = 0; i < 8; ++i) v[i] = lut[code_of(pw, b, lc + i)];
                }
            }
            wv[qq] = v;
        }
        __syncthreads();
        *reinterpret_cast<half8_t*>(&xs[lr][lc]) = xv;
        for (int qq = 0; qq < NMAT; ++qq) *reinterpret_cast<half8_t*>(&ws[qq][lr][lc]) = wv[qq];
        __syncthreads();
        for (int kk = 0; kk < kBK; kk += 16) {
            const int kq = kk + 4 * (lane / 16);
            half4_t av[2];
            for (int i = 0; i < 2; ++i)
                av[i] = *reinterpret_cast<const half4_t*>(&xs[wm * 32 + i * 16 + lane % 16][kq]);
            for (int qq = 0; qq < NMAT; ++qq) {
                for (int j = 0; j < 2; ++j) {
                    const half4_t bv = *reinterpret_cast<const half4_t*>(&ws[qq][wn * 32 + j * 16 + lane % 16][kq]);
                    for (int i = 0; i < 2; ++i)
                        acc[qq][i][j] = __builtin_amdgcn_mfma_f32_16x16x16f16(av[i], bv, acc[qq][i][j], 0, 0, 0);
                }
            }
        }
    }
    // D lane layout: token = 4 * (lane / 16) + r, row = lane % 16.
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j)
            for (int r = 0; r < 4; ++r) {
                const int t = m0 + wm * 32 + i * 16 + 4 * (lane / 16) + r;
                const int n = n0 + wn * 32 + j * 16 + lane % 16;
                if (t < m && n < rows) {
                    const size_t o = (size_t)(off + t) * rows + n;
                    if (NMAT == 2)
                        reinterpret_cast<half_t*>(a.out)[o] =
                            (half_t)(silu_f32(acc[0][i][j][r]) * acc[NMAT - 1][i][j][r]);
                    else
                        reinterpret_cast<float*>(a.out)[o] = acc[0][i][j][r];
                }
            }
    __syncthreads();
    }
}

int launch_tile(const GemmArgs& a, hipStream_t s) {
    const int S = a.T * a.k;
    if (S < a.mfma_min_tokens) return APMOE_OK;  // no group can reach the threshold
    const int rows = a.stage == APMOE_GATE_UP_SWIGLU ? a.I : a.H;
    const int mslots = (S + kBM - 1) / kBM + a.E;
    dim3 grid((rows + kBN - 1) / kBN, mslots < 16 ? mslots : 16);
    if (a.stage == APMOE_GATE_UP_SWIGLU)
        hipLaunchKernelGGL(tile_simple_kernel<2>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(tile_simple_kernel<1>, grid, dim3(256), 0, s, a);
    return launch_status();
}

}  // namespace apmoe

using namespace apmoe;

extern "C" int apmoe_bitplane_lut_gemm(int stage, const apmoe_expert* experts, const int8_t* bits,
                                       int E, const int32_t* offsets, const int32_t* sorted_slots,
                                       int k, const uint16_t* in, void* out, int T, int H, int I,
                                       int mfma_min_tokens, void* ws, size_t ws_bytes, void* stream) {
    const int paths = stage & (APMOE_ONLY_GEMV | APMOE_ONLY_TILE);
    stage &= ~(APMOE_ONLY_GEMV | APMOE_ONLY_TILE);
    if (stage != APMOE_GATE_UP_SWIGLU && stage != APMOE_DOWN) return APMOE_EINVAL;
    if (paths == (APMOE_ONLY_GEMV | APMOE_ONLY_TILE)) return APMOE_EINVAL;
    if (T < 0 || E < 1 || E > APMOE_MAX_EXPERTS || k < 1 || H <= 0 || I <= 0) return APMOE_EINVAL;
    if (H % 32 || I % 32 || mfma_min_tokens < 1) return APMOE_EINVAL;
    if ((long long)T * k > (1ll << 30)) return APMOE_EINVAL;
    if (T == 0) return APMOE_OK;
    if (!experts || !bits || !offsets || !in || !out) return APMOE_EINVAL;
    if (stage == APMOE_GATE_UP_SWIGLU && !sorted_slots) return APMOE_EINVAL;
    if (ws_bytes < apmoe_workspace_bytes(T, k, E, H, I)) return APMOE_ENOSPACE;
    GemmArgs a{stage, experts, bits, E, offsets, sorted_slots, k, in, out, T, H, I, mfma_min_tokens};
    hipStream_t s = as_stream(stream);
    if (paths != APMOE_ONLY_TILE) {
        const int rc = launch_gemv(a, ws, ws_bytes, s);
        if (rc != APMOE_OK) return rc;
    }
    if (paths != APMOE_ONLY_GEMV) return launch_tile(a, s);
    return APMOE_OK;
}
