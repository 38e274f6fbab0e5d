// Bit-plane + LUT GEMV path of apmoe_bitplane_lut_gemm: expert groups smaller
// than mfma_min_tokens (decode-sized groups).
//
// Layout of the work (gfx950, wave64, v_mfma_f32_16x16x32_f16):
//   D[row][token] = sum_k W[row][k] * X[token][k]
//   A operand (W): lane l holds row (l % 16) of a 16-row group and the eight
//                  consecutive columns 8*q + 0..7 of the 32-column word that
//                  lane group g = l / 16 owns in this step (q = 0..3 picks
//                  one of the four MFMAs a word feeds).
//   B operand (X): lane l holds token (l % 16) at the same eight columns; one
//                  16-byte load from the activation row.
//   D:             lane l holds rows 4*g + 0..3 for token l % 16.
// A decoded A operand is reused for up to four 16-token tiles.
//
// Decode of one lane's word (32 columns of one row, b planes):
//   * the plane words come from the packed layout: one 256-byte run per plane
//     and 16-row group per step, so every load uses whole cache lines;
//   * the b plane words are bit-transposed in registers with three delta-swap
//     stages, giving eight registers R_s whose byte u is the b-bit code of
//     column 8*u + s (one 8x8 bit transpose per byte lane);
//   * each wave stages the LUTs of its rows in its own 16 KB LDS region as
//     table[code][matrix][slot] dwords, slot = 16*(g % 2) + row, so the 32
//     lanes of a half-wave read 32 different banks whatever the codes;
//   * the region number rides in code bits 6-7 (two constant input words of
//     the transpose), so a lookup address is code' * 256 + 4 * (lane % 32),
//     built with one byte permute.
// Only the top b planes of a b-bit expert are read.
//
// Scheduling: a persistent grid walks a work list of items (expert, block of
// 16 or 32 rows, K split) built on the device from the slot counts.  Each wave
// owns whole items, so waves never wait for each other.  Loads are issued one
// K step ahead into two register buffers that trade roles.  When the host
// splits K (only when the work list would be too short to fill the GPU), each
// split writes fp32 partial sums to the workspace and a finalize kernel adds
// them in split order (and applies SwiGLU), so results never depend on
// scheduling.
#include "common.hpp"

namespace apmoe {
namespace {

constexpr int kWaves = 4;                   // waves per workgroup, one LDS region each
constexpr int kThreads = kWaves * kWave;
constexpr int kRegion = 16 * 1024;          // LUT bytes per wave: P * 2^b * 256 <= 16 KB
constexpr int kTargetWaves = 2048;          // 256 CUs x 8 resident waves

__device__ __forceinline__ void delta_swap(uint32_t& a, uint32_t& b, int d, uint32_t m) {
    const uint32_t t = ((a >> d) ^ b) & m;
    b ^= t;
    a ^= t << d;
}

// q[r] holds code bit r of 32 columns (bit i = column i).  Afterwards byte u of
// q[s] holds the code of column 8*u + s.
__device__ __forceinline__ void transpose_bytes(uint32_t q[8]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) delta_swap(q[r], q[r + 4], 4, 0x0F0F0F0Fu);
#pragma unroll
    for (int r = 0; r < 8; r += 4) {
        delta_swap(q[r], q[r + 2], 2, 0x33333333u);
        delta_swap(q[r + 1], q[r + 3], 2, 0x33333333u);
    }
#pragma unroll
    for (int r = 0; r < 8; r += 2) delta_swap(q[r], q[r + 1], 1, 0x55555555u);
}

__device__ __forceinline__ half8_t load_h8(const half_t* p) { return *reinterpret_cast<const half8_t*>(p); }

// Activations of eight columns, or zeros past the end of K (no branch).
__device__ __forceinline__ half8_t load_x8(const half_t* p, bool ok) {
    const half8_t v = load_h8(p);
    const half8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
    return ok ? v : z;
}

__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct Mats {
    gu32_t* planes[2];
    gh16_t* lut[2];
    gh16_t* w16[2];
};

struct Shape {
    int rows, K, Wd, nsteps, k, KS, S;
    const half_t* in;
    const int32_t* slots;
    float* partial;      // [KS][S][NMAT][rows] when KS > 1
};

struct Item {
    int e, off, m, b, P, row0, ks;
};

// Rows per item: two 16-row groups for single-tile groups whose tables fit.
__device__ __forceinline__ int rows_groups(int m, int b) { return (m <= 16 && (b <= 5 || b == 16)) ? 2 : 1; }

// Stage the LUTs of one item into this wave's region, at byte offset
//   r * 2^B * 256 + v * 256 + mat * 128 + 4 * slot,  slot = 16 * c + row, c = 0, 1.
template <int NMAT, int B, int P>
__device__ __forceinline__ void stage_luts(uint32_t* region, const Mats& mv, int row0, int lane) {
    constexpr int nent = 1 << B;
    constexpr int total = P * NMAT * nent * 16;
    for (int idx = lane; idx < total; idx += kWave) {
        const int v = idx % nent;                 // consecutive lanes: consecutive entries of one row
        const int i = (idx / nent) & 15;
        const int t = idx / (nent * 16);          // r * NMAT + mat
        const int r = t / NMAT, mat = t % NMAT;
        gh16_t* lut = (NMAT == 2 && mat) ? mv.lut[1] : mv.lut[0];
        const uint32_t val = ((gu16_t*)lut)[(size_t)(row0 + 16 * r + i) * nent + v];
        uint32_t* tab = region + (r * nent + v) * 64 + mat * 32 + i;
        tab[0] = val;
        tab[16] = val;
    }
}

// Plane words of one K step for every (row group, matrix) of the item, from
// the packed layout: one 256-byte run per plane and row group.
template <int NMAT, int B, int P>
__device__ __forceinline__ void load_planes(uint32_t (&w)[P][NMAT][B], const Mats& mv, const Shape& sh, int row0,
                                            int step, int lane) {
    const size_t slab = (size_t)sh.rows * 4 * sh.nsteps;
#pragma unroll
    for (int r = 0; r < P; ++r) {
        const size_t at = ((size_t)((row0 >> 4) + r) * sh.nsteps + step) * 64 + lane;
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
            for (int p = 0; p < B; ++p) w[r][mat][p] = mv.planes[mat][p * slab + at];
    }
}

// Activations of one K step (four MFMA column groups x TT tiles).
template <int TT>
__device__ __forceinline__ void load_x(half8_t (&bx)[4][TT], const half_t* const (&xr)[TT], int word, int Wd) {
    const bool ok = word < Wd;
    const int wc = min(word, Wd - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) bx[q][tt] = load_x8(xr[tt] + 32 * wc + 8 * q, ok);
}

// Decode one step's plane words and run its MFMAs.  hi6/hi7 hold code bits 6
// and 7 (the wave's LDS region) for every column: all ones or zero.
template <int NMAT, int B, int P, int TT>
__device__ __forceinline__ void lut_step(const uint32_t (&w)[P][NMAT][B], const half8_t (&bx)[4][TT],
                                         const char* lds, uint32_t lane_off, uint32_t hi6, uint32_t hi7,
                                         float4_t (&acc)[P][NMAT][TT]) {
    uint32_t qv[P][NMAT][8];
#pragma unroll
    for (int r = 0; r < P; ++r)
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat) {
#pragma unroll
            for (int rr = 0; rr < 6; ++rr) qv[r][mat][rr] = rr < B ? w[r][mat][B - 1 - rr] : 0u;  // bit rr <- plane B-1-rr
            qv[r][mat][6] = hi6;
            qv[r][mat][7] = hi7;
            transpose_bytes(qv[r][mat]);
        }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        // address = (region << 6 | code) * 256 + 4 * (lane % 32), code = byte q of R_s
        const uint32_t sel = 0x0C0C0000u | ((4u + q) << 8);
#pragma unroll
        for (int r = 0; r < P; ++r)
#pragma unroll
            for (int mat = 0; mat < NMAT; ++mat) {
                const char* tab = lds + r * (1 << B) * 256 + mat * 128;
                half8_t a;
#pragma unroll
                for (int s = 0; s < 8; ++s)
                    a[s] = *reinterpret_cast<const half_t*>(tab + __builtin_amdgcn_perm(qv[r][mat][s], lane_off, sel));
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
                    acc[r][mat][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bx[q][tt], acc[r][mat][tt], 0, 0, 0);
            }
    }
}

// K loop of one wave over steps [s0, s1): in each step lane group g owns word
// 4*step + g of every (row group, matrix) of the item.  Everything a step needs
// is issued one step ahead, before the loads of the step after it, so the
// in-order completion of loads never makes a step wait for its successor's
// data; two register buffers trade roles (unrolled by two) so no register is
// copied while its load is in flight.
template <int NMAT, int B, int P, int TT>
__device__ __forceinline__ void kloop(const Mats& mv, const char* lds, const Shape& sh, const Item& it, int t0,
                                      int s0, int s1, int lane, uint32_t hi6, uint32_t hi7,
                                      float4_t (&acc)[P][NMAT][TT]) {
    const int i = lane & 15, g = lane >> 4;
    const half_t* xr[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int n = min(t0 + 16 * tt + i, it.m - 1);
        xr[tt] = NMAT == 2 ? sh.in + (size_t)(sh.slots[it.off + n] / sh.k) * sh.K
                           : sh.in + (size_t)(it.off + n) * sh.K;
    }
    if (s0 >= s1) return;
    const int last = 4 * (s1 - 1) + g;   // past the last step: re-read it (from cache)
    half8_t xa[4][TT], xb[4][TT == 1 ? 1 : 1];
    if constexpr (B == 16) {
        half8_t wa[P][NMAT][4], wb[P][NMAT][4];
        auto load_w = [&](half8_t (&w)[P][NMAT][4], int word) {
            const int wc = min(word, sh.Wd - 1);
#pragma unroll
            for (int r = 0; r < P; ++r)
#pragma unroll
                for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        w[r][mat][q] = load_h8g(mv.w16[mat] + (size_t)(it.row0 + 16 * r + i) * sh.K + 32 * wc + 8 * q);
        };
        auto mma = [&](const half8_t (&w)[P][NMAT][4], const half8_t (&bx)[4][TT]) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < P; ++r)
#pragma unroll
                    for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                        for (int tt = 0; tt < TT; ++tt)
                            acc[r][mat][tt] =
                                __builtin_amdgcn_mfma_f32_16x16x32_f16(w[r][mat][q], bx[q][tt], acc[r][mat][tt], 0, 0, 0);
        };
        if constexpr (TT == 1) {
            load_x<TT>(xa, xr, 4 * s0 + g, sh.Wd);
            load_w(wa, 4 * s0 + g);
            for (int step = s0; step < s1; step += 2) {
                const int w1 = min(4 * (step + 1) + g, last), w2 = min(4 * (step + 2) + g, last);
                load_x<TT>(xb, xr, w1, sh.Wd);
                load_w(wb, w1);
                mma(wa, xa);
                load_x<TT>(xa, xr, w2, sh.Wd);
                load_w(wa, w2);
                if (step + 1 < s1) mma(wb, xb);
            }
        } else {
            // multi-tile activations take one buffer, loaded at the start of
            // each step ahead of the next step's weights
            load_w(wa, 4 * s0 + g);
            for (int step = s0; step < s1; step += 2) {
                const int w0 = 4 * step + g;
                const int w1 = min(4 * (step + 1) + g, last), w2 = min(4 * (step + 2) + g, last);
                load_x<TT>(xa, xr, w0, sh.Wd);
                load_w(wb, w1);
                mma(wa, xa);
                load_x<TT>(xa, xr, w1, sh.Wd);
                load_w(wa, w2);
                if (step + 1 < s1) mma(wb, xa);
            }
        }
    } else {
        const uint32_t lane_off = 4u * (lane & 31);
        uint32_t wa[P][NMAT][B], wb[P][NMAT][B];
        const int sl = s1 - 1;   // past the last step: re-read it (from cache)
        if constexpr (TT == 1) {
            load_x<TT>(xa, xr, 4 * s0 + g, sh.Wd);
            load_planes<NMAT, B, P>(wa, mv, sh, it.row0, s0, lane);
            for (int step = s0; step < s1; step += 2) {
                const int w1 = min(4 * (step + 1) + g, last), w2 = min(4 * (step + 2) + g, last);
                load_x<TT>(xb, xr, w1, sh.Wd);
                load_planes<NMAT, B, P>(wb, mv, sh, it.row0, min(step + 1, sl), lane);
                lut_step<NMAT, B, P, TT>(wa, xa, lds, lane_off, hi6, hi7, acc);
                load_x<TT>(xa, xr, w2, sh.Wd);
                load_planes<NMAT, B, P>(wa, mv, sh, it.row0, min(step + 2, sl), lane);
                if (step + 1 < s1) lut_step<NMAT, B, P, TT>(wb, xb, lds, lane_off, hi6, hi7, acc);
            }
        } else {
            load_planes<NMAT, B, P>(wa, mv, sh, it.row0, s0, lane);
            for (int step = s0; step < s1; step += 2) {
                const int w0 = 4 * step + g;
                const int w1 = min(4 * (step + 1) + g, last);
                load_x<TT>(xa, xr, w0, sh.Wd);
                load_planes<NMAT, B, P>(wb, mv, sh, it.row0, min(step + 1, sl), lane);
                lut_step<NMAT, B, P, TT>(wa, xa, lds, lane_off, hi6, hi7, acc);
                load_x<TT>(xa, xr, w1, sh.Wd);
                load_planes<NMAT, B, P>(wa, mv, sh, it.row0, min(step + 2, sl), lane);
                if (step + 1 < s1) lut_step<NMAT, B, P, TT>(wb, xa, lds, lane_off, hi6, hi7, acc);
            }
        }
    }
}

// Results of row group r, token tok in this lane (rows 4g..4g+3): the final
// value, or this K split's partial sums.
template <int NMAT>
__device__ __forceinline__ void store_result(const GemmArgs& a, const Shape& sh, const Item& it, int r, int tok,
                                             int g, const float4_t (&s)[NMAT]) {
    if (tok >= it.m) return;
    const int row = it.row0 + 16 * r + 4 * g;
    const int p = it.off + tok;
    if (sh.KS > 1) {
        float* dst = sh.partial + ((size_t)it.ks * sh.S + p) * NMAT * sh.rows + row;
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat) *reinterpret_cast<float4_t*>(dst + (size_t)mat * sh.rows) = s[mat];
        return;
    }
    const size_t o = (size_t)p * sh.rows + row;
    if (NMAT == 2) {
        half4_t h;
#pragma unroll
        for (int c = 0; c < 4; ++c) h[c] = (half_t)(silu_f32(s[0][c]) * s[NMAT - 1][c]);
        *reinterpret_cast<half4_t*>(reinterpret_cast<half_t*>(a.out) + o) = h;
    } else {
        *reinterpret_cast<float4_t*>(reinterpret_cast<float*>(a.out) + o) = s[0];
    }
}

// One item on one wave: stage its LUTs in the wave's region, then one pass
// over its K range per 16*TT tokens.
template <int NMAT, int B, int P, int TT>
__device__ __forceinline__ void run_item(const GemmArgs& a, const Mats& mv, const char* lds, char* region,
                                         const Shape& sh, const Item& it, int lane, uint32_t hi6, uint32_t hi7) {
    const int i = lane & 15, g = lane >> 4;
    const int per = (sh.nsteps + sh.KS - 1) / sh.KS;
    const int s0 = min(sh.nsteps, it.ks * per), s1 = min(sh.nsteps, s0 + per);
    if (B != 16) {
        wave_lds_fence();   // the previous item's lookups come before the tables change
        stage_luts<NMAT, B, P>(reinterpret_cast<uint32_t*>(region), mv, it.row0, lane);
        wave_lds_fence();
    }
    for (int t0 = 0; t0 < it.m; t0 += 16 * TT) {
        float4_t acc[P][NMAT][TT];
#pragma unroll
        for (int r = 0; r < P; ++r)
#pragma unroll
            for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) acc[r][mat][tt] = float4_t{0.f, 0.f, 0.f, 0.f};
        kloop<NMAT, B, P, TT>(mv, lds, sh, it, t0, s0, s1, lane, hi6, hi7, acc);
#pragma unroll
        for (int r = 0; r < P; ++r)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
                float4_t s[NMAT];
#pragma unroll
                for (int mat = 0; mat < NMAT; ++mat) s[mat] = acc[r][mat][tt];
                store_result<NMAT>(a, sh, it, r, t0 + 16 * tt + i, g, s);
            }
    }
}

template <int NMAT, int B>
__device__ __forceinline__ void run_item_b(const GemmArgs& a, const Mats& mv, const char* lds, char* region,
                                           const Shape& sh, const Item& it, int lane, uint32_t hi6, uint32_t hi7) {
    if (it.P == 2) {
        run_item<NMAT, B, 2, 1>(a, mv, lds, region, sh, it, lane, hi6, hi7);
    } else if (it.m <= 16) {
        run_item<NMAT, B, 1, 1>(a, mv, lds, region, sh, it, lane, hi6, hi7);
    } else if (it.m <= 32) {
        run_item<NMAT, B, 1, 2>(a, mv, lds, region, sh, it, lane, hi6, hi7);
    } else {
        run_item<NMAT, B, 1, 4>(a, mv, lds, region, sh, it, lane, hi6, hi7);
    }
}

// Row blocks of the experts on this path, in expert order (identical in every
// workgroup).
struct WorkList {
    int first[APMOE_MAX_EXPERTS + 1];
    int nrb[APMOE_MAX_EXPERTS];
    int cnt[APMOE_MAX_EXPERTS];
};

__device__ __forceinline__ void build_work_list(WorkList& wl, const GemmArgs& a, int rows) {
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
        const int m = a.offsets[e + 1] - a.offsets[e];
        const int b = a.bits[e];
        const bool on = m > 0 && m < a.mfma_min_tokens && valid_bits(b);
        wl.cnt[e] = m;
        wl.nrb[e] = on ? rows / (16 * rows_groups(m, b)) : 0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int e = 0; e < a.E; ++e) {
            wl.first[e] = run;
            run += wl.nrb[e];
        }
        wl.first[a.E] = run;
    }
    __syncthreads();
}

__device__ __forceinline__ int expert_of(const WorkList& wl, int E, int blk) {
    int lo = 0, hi = E - 1;   // last e with first[e] <= blk
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (wl.first[mid] <= blk) lo = mid; else hi = mid - 1;
    }
    return lo;
}

template <int NMAT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemv_kernel(GemmArgs a, int KS, float* partial) {
    __shared__ __attribute__((aligned(16))) char lds[kWaves * kRegion];
    __shared__ WorkList wl;

    Shape sh;
    sh.rows = NMAT == 2 ? a.I : a.H;
    sh.K = NMAT == 2 ? a.H : a.I;
    sh.Wd = sh.K / 32;
    sh.nsteps = (sh.Wd + 3) / 4;
    sh.k = a.k;
    sh.KS = KS;
    sh.S = a.T * a.k;
    sh.in = reinterpret_cast<const half_t*>(a.in);
    sh.slots = a.sorted_slots;
    sh.partial = partial;

    build_work_list(wl, a, sh.rows);
    const int total = wl.first[a.E] * KS;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    char* region = lds + wave * kRegion;                 // staging target of this wave
    const uint32_t hi6 = (wave & 1) ? 0xFFFFFFFFu : 0u;  // lookups reach the region
    const uint32_t hi7 = (wave & 2) ? 0xFFFFFFFFu : 0u;  // through code bits 6 and 7

    const int nwaves = gridDim.x * kWaves;
    for (int idx = blockIdx.x * kWaves + wave; idx < total; idx += nwaves) {
        const int blk = idx / KS;
        const int e = expert_of(wl, a.E, blk);
        Item it;
        it.e = e;
        it.off = a.offsets[e];
        it.m = wl.cnt[e];
        it.b = a.bits[e];
        it.P = rows_groups(it.m, it.b);
        it.row0 = (blk - wl.first[e]) * 16 * it.P;
        it.ks = idx % KS;

        Mats mv;
        const apmoe_mat& m0 = NMAT == 2 ? a.experts[e].gate : a.experts[e].down;
        const apmoe_mat& m1 = a.experts[e].up;
        const MatView v0 = mat_view(m0, it.b), v1 = mat_view(m1, it.b);
        mv.planes[0] = v0.planes;
        mv.lut[0] = v0.lut;
        mv.w16[0] = v0.w16;
        mv.planes[1] = v1.planes;
        mv.lut[1] = v1.lut;
        mv.w16[1] = v1.w16;

        switch (it.b) {
            case 3: run_item_b<NMAT, 3>(a, mv, lds, region, sh, it, lane, hi6, hi7); break;
            case 4: run_item_b<NMAT, 4>(a, mv, lds, region, sh, it, lane, hi6, hi7); break;
            case 5: run_item_b<NMAT, 5>(a, mv, lds, region, sh, it, lane, hi6, hi7); break;
            case 6: run_item_b<NMAT, 6>(a, mv, lds, region, sh, it, lane, hi6, hi7); break;
            default: run_item_b<NMAT, 16>(a, mv, lds, region, sh, it, lane, hi6, hi7); break;
        }
    }
}

// Sum the K-split partials in split order (SwiGLU for gate/up).  One thread
// per (position, 4 rows); positions of tile-path groups are left alone.
template <int NMAT>
__global__ __launch_bounds__(256) void gemv_finalize_kernel(GemmArgs a, int KS, const float* partial) {
    __shared__ int offs[APMOE_MAX_EXPERTS + 1];
    for (int e = threadIdx.x; e <= a.E; e += blockDim.x) offs[e] = a.offsets[e];
    __syncthreads();
    const int rows = NMAT == 2 ? a.I : a.H;
    const int S = a.T * a.k;
    const int q4 = rows / 4;
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long long)S * q4) return;
    const int p = (int)(idx / q4);
    const int row = (int)(idx % q4) * 4;
    int lo = 0, hi = a.E - 1;   // expert holding position p: last e with offs[e] <= p
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offs[mid] <= p) lo = mid; else hi = mid - 1;
    }
    const int m = offs[lo + 1] - offs[lo];
    if (m >= a.mfma_min_tokens || !valid_bits(a.bits[lo])) return;
    float4_t s[NMAT];
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat) {
        s[mat] = float4_t{0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < KS; ++ks)
            s[mat] = s[mat] + *reinterpret_cast<const float4_t*>(partial + ((size_t)ks * S + p) * NMAT * rows +
                                                                 (size_t)mat * rows + row);
    }
    const size_t o = (size_t)p * rows + row;
    if (NMAT == 2) {
        half4_t h;
#pragma unroll
        for (int c = 0; c < 4; ++c) h[c] = (half_t)(silu_f32(s[0][c]) * s[NMAT - 1][c]);
        *reinterpret_cast<half4_t*>(reinterpret_cast<half_t*>(a.out) + o) = h;
    } else {
        *reinterpret_cast<float4_t*>(reinterpret_cast<float*>(a.out) + o) = s[0];
    }
}

}  // namespace

// K splits, chosen from shapes alone: only when one item per row block of every
// expert that could be active would leave waves idle (at least 4 K steps each).
int gemv_splits(int T, int k, int E, int rows, int K) {
    const long long slots = (long long)T * k;
    const long long active = E < slots ? E : slots;
    const long long items = active * (rows / 16);
    const int nsteps = (K / 32 + 3) / 4;
    long long ks = items > 0 ? (kTargetWaves + items - 1) / items : 1;
    const int cap = nsteps / 4 > 1 ? nsteps / 4 : 1;
    if (ks > cap) ks = cap;
    return ks < 1 ? 1 : (int)ks;
}

size_t gemv_workspace_bytes(int T, int k, int E, int rows, int K, int nmat) {
    const int ks = gemv_splits(T, k, E, rows, K);
    if (ks <= 1) return 0;
    return (size_t)ks * T * k * nmat * rows * sizeof(float);
}

int launch_gemv(const GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
    const bool gu = a.stage == APMOE_GATE_UP_SWIGLU;
    const int rows = gu ? a.I : a.H;
    const int K = gu ? a.H : a.I;
    const int nmat = gu ? 2 : 1;
    const int KS = gemv_splits(a.T, a.k, a.E, rows, K);
    float* partial = nullptr;
    if (KS > 1) {
        if (!ws || ws_bytes < gemv_workspace_bytes(a.T, a.k, a.E, rows, K, nmat)) return APMOE_ENOSPACE;
        partial = reinterpret_cast<float*>(ws);
    }
    dim3 grid(kTargetWaves / kWaves), block(kThreads);
    if (gu)
        hipLaunchKernelGGL(gemv_kernel<2>, grid, block, 0, s, a, KS, partial);
    else
        hipLaunchKernelGGL(gemv_kernel<1>, grid, block, 0, s, a, KS, partial);
    int rc = launch_status();
    if (rc != APMOE_OK || KS == 1) return rc;
    const long long n = (long long)a.T * a.k * (rows / 4);
    dim3 fgrid((unsigned)((n + 255) / 256));
    if (gu)
        hipLaunchKernelGGL(gemv_finalize_kernel<2>, fgrid, dim3(256), 0, s, a, KS, partial);
    else
        hipLaunchKernelGGL(gemv_finalize_kernel<1>, fgrid, dim3(256), 0, s, a, KS, partial);
    return launch_status();
}

}  // namespace apmoe
