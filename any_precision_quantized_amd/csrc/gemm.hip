// Expert FFN stages over bit-plane + LUT weights: apmoe_bitplane_lut_gemm,
// and its dequantise-to-LDS + MFMA tile path (groups of >= mfma_min_tokens).
//
// Dispatch happens on the device: every workgroup reads its expert's slot
// count and bitwidth and leaves at once when the group is empty or belongs to
// the other path, so no count ever travels to the host.
#include <algorithm>
#include <climits>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "decode.hpp"

namespace apmoe {

// ---------------------------------------------------------------------------
// Tile path (groups of at least mfma_min_tokens): every K step the weight
// tile is decoded from the bit-planes into LDS as exact fp16 and multiplied
// with v_mfma_f32_32x32x16_f16 against an LDS tile of the group's tokens.
//   D[row][token] = sum_k W[row][k] * X[token][k]
// Workgroup tile: 256 weight rows x 256 tokens, K step 32 (one plane word
// per row).  For gate/up the 256 rows are 128 gate rows and the same 128 up
// rows, so the SwiGLU pairs meet in one lane.  Eight waves (two per SIMD)
// each own 128 rows x 64 tokens (4 x 2 MFMA tiles, 128 fp32 accumulators per
// lane).  Thread t < 256 (waves 0-3) decodes row t of the weight tile (its b
// plane words, the same byte transpose and LUT-in-LDS lookups as the GEMV
// path); thread 256 + t (waves 4-7) stages token t of the activation tile, so
// each SIMD runs one decoding and one staging wave and the hardware overlaps
// one wave's decode with the other's MFMAs.  Loads run three steps ahead in a
// register ring; three LDS stages rotate, one barrier per step.
// Items are (expert, row tile, token tile) with the token tile fastest, so
// the workgroups the dispatcher sends to one XCD share that XCD's L2 copy of
// a token tile while all XCDs walk the same weight rows.
// ---------------------------------------------------------------------------

namespace {

constexpr int kThreadsTile = 512;
constexpr int kTToks = 256;              // tokens per tile
constexpr int kRowB = 80;                // LDS bytes per tile row: 32 halves + 16 pad
constexpr int kTileB = 256 * kRowB;
// LDS map: LUT block 0 at 0, stage 0 (W0 | X0) at 16K, LUT block 1 at 64K,
// stage 1 at 80K (the lookup permute puts the LUT block into address byte 2).
// Two stages: step s uses stage s % 2, the same index as its register slot,
// so the loop unrolls by two with no branch in its body.
constexpr int kStageOff[2] = {16384, 81920};
constexpr int kTileLds = 81920 + 2 * kTileB;
static_assert(16384 + 2 * kTileB <= 65536, "stage 0 overlaps LUT block 1");
static_assert(kTileLds <= 160 * 1024, "tile LDS exceeds 160 KiB");

struct TileItem {
    int e, off, m, b, rt, tt;
};

// Item of workgroup idx over the groups on this path, each owning
// ceil(m / 256) x RT items in (row tile, token tile) order.
__device__ __forceinline__ bool find_tile_item(const GemmArgs& a, int RT, int idx, TileItem& it) {
    const int lane = threadIdx.x % kWave;
    int base = 0;
    for (int c0 = 0; c0 < a.E; c0 += kWave) {
        const int e = c0 + lane;
        int m = 0, b = 0;
        if (e < a.E) {
            m = a.offsets[e + 1] - a.offsets[e];
            b = a.bits[e];
        }
        const int nt = (m + kTToks - 1) / kTToks;
        const int n = (m > 0 && m >= a.mfma_min_tokens && valid_bits(b)) ? nt * RT : 0;
        const int inc = wave_incl_scan(n);
        const int first = base + inc - n;
        const unsigned long long hit = __ballot(n > 0 && idx >= first && idx < first + n);
        if (hit) {
            const int src = __ffsll((long long)hit) - 1;
            it.e = __builtin_amdgcn_readfirstlane(c0 + src);
            it.m = __builtin_amdgcn_readlane(m, src);
            it.b = __builtin_amdgcn_readlane(b, src);
            const int q = idx - __builtin_amdgcn_readlane(first, src);
            const int ntile = (it.m + kTToks - 1) / kTToks;
            it.rt = q / ntile;
            it.tt = q % ntile;
            it.off = a.offsets[it.e];
            return true;
        }
        base += __builtin_amdgcn_readlane(inc, kWave - 1);
    }
    return false;
}

template <int NMAT, int B>
__device__ __forceinline__ void tile_item(const GemmArgs& a, char* lds, const TileItem& it) {
    constexpr int kMatRows = NMAT == 2 ? 128 : 256;   // rows of one matrix in the tile
    const int rows = NMAT == 2 ? a.I : a.H;
    const int K = NMAT == 2 ? a.H : a.I;
    const int ns = K / 32;                    // K steps
    const int nsteps128 = (K / 32 + 3) / 4;   // steps of the packed plane layout
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int r0 = it.rt * kMatRows, t0 = it.tt * kTToks;
    const bool dec = wave < 4;   // role: decode weight row (waves 0-3) or stage token (4-7)
    const int tr = tid & 255;    // the role's tile row / token

    // decode role: tile row tr = matrix hsel, row r0 + (tr % kMatRows)
    const int hsel = NMAT == 2 ? (wave >> 1) & 1 : 0;   // gate/up: matrix (waves 2, 3: up); down: 0
    const int rowc = min(r0 + tr % kMatRows, rows - 1);
    const apmoe_mat& mt = NMAT == 2 ? (hsel ? a.experts[it.e].up : a.experts[it.e].gate) : a.experts[it.e].down;
    MatView mv = mat_view(mt, it.b);
    // the same matrix for the whole wave: scalar registers, so the buffer
    // resources need no per-lane loop
    mv.planes = uniform_ptr(mv.planes);
    mv.w16 = uniform_ptr(mv.w16);
    // the resource covers the b resident planes only (none at 16 bits)
    const uint32_t pbytes = (uint32_t)(it.b <= kPlanes ? it.b : 0) * (uint32_t)rows * 16u * (uint32_t)nsteps128;
    const uint32_t slab = (uint32_t)rows * 16u * (uint32_t)nsteps128;
    const uint32_t wbytes = (uint32_t)rows * (uint32_t)K * 2u;

    // activation role: token t0 + tr of the group
    const int tok = t0 + tr;
    const bool tok_ok = tok < it.m;
    const int tokc = it.off + min(tok, it.m - 1);
    const int xrow = NMAT == 2 ? a.sorted_slots[tokc] / a.k : tokc;
    const uint32_t xbytes = (uint32_t)((NMAT == 2 ? (size_t)a.T : (size_t)a.T * a.k) * K * 2);
    const uint32_t xbase = (uint32_t)xrow * (uint32_t)K * 2u;

    // LUTs of the tile's rows: entry (code v, row r < 128) at block r / 64,
    // v * 256 + 4 * (r % 64); low half gate (down: row r), high half up
    // (down: row r + 128)
    if constexpr (B != 16) {
        constexpr int nent = 1 << B;
        const gu16_t* l0;
        const gu16_t* l1;
        if (NMAT == 2) {
            l0 = (const gu16_t*)mat_view(a.experts[it.e].gate, it.b).lut;
            l1 = (const gu16_t*)mat_view(a.experts[it.e].up, it.b).lut;
        } else {
            l0 = l1 = (const gu16_t*)mv.lut;
        }
        for (int idx = tid; idx < 128 * nent; idx += kThreadsTile) {
            const int v = idx / 128, r = idx % 128;
            const int ra = min(r0 + r, rows - 1);
            const int rb = NMAT == 2 ? ra : min(r0 + 128 + r, rows - 1);
            const uint32_t val = (uint32_t)l0[(size_t)ra * nent + v] | ((uint32_t)l1[(size_t)rb * nent + v] << 16);
            *reinterpret_cast<uint32_t*>(lds + ((r >> 6) << 16) + v * 256 + 4 * (r & 63)) = val;
        }
    }
    // lookup address: byte 0 = slot (row % 64) * 4 + 2 * half, byte 1 = code,
    // byte 2 = LUT block (row / 64 % 2)
    const uint32_t lane_off = ((uint32_t)(wave & 1) << 16) |
                              (4u * (uint32_t)lane + 2u * (uint32_t)(NMAT == 2 ? hsel : (wave >> 1)));

    // one register ring for both roles: a step's 32 activations or its fp16
    // weights (16 dwords), or its b plane words.  The role is a compile-time
    // argument: each role runs its own copy of the step loop, so no branch
    // splits a step and its MFMAs and decode share one scheduling region.
    using DecRole = std::integral_constant<bool, true>;
    using XRole = std::integral_constant<bool, false>;
    uint32_t reg[2][16];
    auto load = [&](auto role, int r, int s) {   // steps past ns read zeros
        constexpr bool kDec = decltype(role)::value;
        const bool ok = s < ns;
        if constexpr (!kDec) {
            const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.in, ok ? xbytes : 0u);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32x4_t v = __builtin_bit_cast(
                    uint32x4_t, buf_load_h8(xr, tok_ok ? xbase + 64u * s + 16u * j : kOutOfRange));
#pragma unroll
                for (int c = 0; c < 4; ++c) reg[r][4 * j + c] = v[c];
            }
        } else if constexpr (B == 16) {
            const __amdgpu_buffer_rsrc_t wr = make_rsrc((const void*)mv.w16, ok ? wbytes : 0u);
            const uint32_t base = ((uint32_t)rowc * (uint32_t)K + 32u * s) * 2u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32x4_t v = __builtin_bit_cast(uint32x4_t, buf_load_h8(wr, base + 16u * j));
#pragma unroll
                for (int c = 0; c < 4; ++c) reg[r][4 * j + c] = v[c];
            }
        } else {
            const __amdgpu_buffer_rsrc_t pr = make_rsrc((const void*)mv.planes, ok ? pbytes : 0u);
            const int sc = min(s, ns - 1);
            const uint32_t at = ((uint32_t)(rowc >> 4) * (uint32_t)nsteps128 + (uint32_t)(sc >> 2)) * 256u +
                                64u * (uint32_t)(sc & 3) + 4u * (uint32_t)(rowc & 15);
#pragma unroll
            for (int p = 0; p < B; ++p) reg[r][p] = buf_load_u32(pr, at, p * slab);
        }
    };
    auto store = [&](auto role, int r, int st) {   // decode / stage into LDS stage st
        constexpr bool kDec = decltype(role)::value;
        char* wt = lds + kStageOff[st] + tr * kRowB;
        if constexpr (!kDec) {
            char* xt = wt + kTileB;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32x4_t v;
#pragma unroll
                for (int c = 0; c < 4; ++c) v[c] = reg[r][4 * j + c];
                *reinterpret_cast<uint32x4_t*>(xt + 16 * j) = v;
            }
        } else if constexpr (B == 16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32x4_t v;
#pragma unroll
                for (int c = 0; c < 4; ++c) v[c] = reg[r][4 * j + c];
                *reinterpret_cast<uint32x4_t*>(wt + 16 * j) = v;
            }
        } else {
            uint32_t q[8];
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) q[rr] = rr < B ? reg[r][B - 1 - rr] : 0u;   // bit rr <- plane B-1-rr
            transpose_bytes<B>(q);
            // byte u of q[j] is the code of column 8u + j.  All 32 lookups go
            // out before any store: a store between them would be ordered
            // before the later lookups (same LDS array), one round trip each.
            uint32x4_t v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t sel = 0x0C020400u | ((uint32_t)u << 8);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t lo = *reinterpret_cast<const uint16_t*>(lds + __builtin_amdgcn_perm(q[2 * c], lane_off, sel));
                    const uint32_t hi = *reinterpret_cast<const uint16_t*>(lds + __builtin_amdgcn_perm(q[2 * c + 1], lane_off, sel));
                    v[u][c] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) *reinterpret_cast<uint32x4_t*>(wt + 16 * u) = v[u];
        }
    };

    // MFMA role: wave (wr, wtk) owns tile rows {64wr + 32j, 128 + 64wr + 32j}
    // (gate/up) or 128wr + 32j (down), j < 2 / 4, and tokens 64wtk + 32i, i < 2
    const int wr = wave & 1, wtk = wave >> 1;
    int rbase[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        rbase[j] = NMAT == 2 ? (j < 2 ? 64 * wr + 32 * j : 128 + 64 * wr + 32 * (j - 2)) : 128 * wr + 32 * j;
    float16_t acc[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;
    const int l32 = lane & 31, lh = lane >> 5;
    // all twelve operand reads of the step go out before its first MFMA
    auto compute = [&](int st) {
        const char* wt = lds + kStageOff[st];
        const char* xt = wt + kTileB;
        half8_t av[2][4], bv[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                av[h][j] = *reinterpret_cast<const half8_t*>(wt + (rbase[j] + l32) * kRowB + 32 * h + 16 * lh);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                bv[h][i] = *reinterpret_cast<const half8_t*>(xt + (64 * wtk + 32 * i + l32) * kRowB + 32 * h + 16 * lh);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[h][j], bv[h][i], acc[j][i], 0, 0, 0);
    };

    // Step st: refill the register slot step st left with step st + 2,
    // multiply step st, decode / stage step st + 1 (loaded a step earlier)
    // into the other stage (read last at step st - 1, before the barrier).
    // No branch inside a step, and the operand reads precede the stage writes
    // in program order, so no assumed LDS alias holds the MFMAs behind the
    // decode; a step past ns (at most one in the last pair) reads zeros and
    // adds nothing.  Both roles meet at the same barriers.
    auto run = [&](auto role) {
        load(role, 0, 0);
        load(role, 1, 1);
        store(role, 0, 0);
        __syncthreads();
        for (int s = 0; s < ns; s += 2) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int st = s + u;
                load(role, u, st + 2);
                compute(u);
                store(role, 1 - u, 1 - u);
                __syncthreads();
            }
        }
    };
    __syncthreads();   // LUT tables complete
    if (dec)
        run(DecRole{});
    else
        run(XRole{});

    // D lane layout: row 8 * (r / 4) + 4 * (lane / 32) + r % 4, token lane % 32
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tk = t0 + 64 * wtk + 32 * i + l32;
        if (tk >= it.m) continue;
        const size_t p = (size_t)(it.off + tk);
#pragma unroll
        for (int j = 0; j < (NMAT == 2 ? 2 : 4); ++j)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int row = r0 + (NMAT == 2 ? 64 * wr + 32 * j : 128 * wr + 32 * j) + 8 * q4 + 4 * lh;
                if (row >= rows) continue;
                if (NMAT == 2) {
                    half4_t hv;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        hv[c] = (half_t)(silu_f32(acc[j][i][4 * q4 + c]) * acc[j + 2][i][4 * q4 + c]);
                    *reinterpret_cast<half4_t*>(reinterpret_cast<half_t*>(a.out) + p * rows + row) = hv;
                } else {
                    float4_t fv;
#pragma unroll
                    for (int c = 0; c < 4; ++c) fv[c] = acc[j][i][4 * q4 + c];
                    *reinterpret_cast<float4_t*>(reinterpret_cast<float*>(a.out) + p * rows + row) = fv;
                }
            }
    }
}

template <int NMAT>
__global__ __launch_bounds__(kThreadsTile) __attribute__((amdgpu_waves_per_eu(2, 2)))
void tile_kernel(GemmArgs a, int RT) {
    __shared__ __attribute__((aligned(16))) char lds[kTileLds];
    TileItem it;
    if (!find_tile_item(a, RT, blockIdx.x, it)) return;   // uniform
    switch (it.b) {
        case 3: tile_item<NMAT, 3>(a, lds, it); break;
        case 4: tile_item<NMAT, 4>(a, lds, it); break;
        case 5: tile_item<NMAT, 5>(a, lds, it); break;
        case 6: tile_item<NMAT, 6>(a, lds, it); break;
        default: tile_item<NMAT, 16>(a, lds, it); break;
    }
}

}  // namespace

int launch_tile(const GemmArgs& a, hipStream_t s) {
    const long long S = (long long)a.T * a.k;
    if (S < a.mfma_min_tokens || a.mfma_min_tokens == INT_MAX) return APMOE_OK;  // no group can reach it
    const bool gu = a.stage == APMOE_GATE_UP_SWIGLU;
    const int mat_rows = gu ? 128 : 256;
    const int RT = ((gu ? a.I : a.H) + mat_rows - 1) / mat_rows;
    // token tiles: at most ceil(S / 256) plus one partial tile per group
    const long long groups = std::min<long long>(a.E, S / a.mfma_min_tokens);
    const long long items = ((S + kTToks - 1) / kTToks + groups) * RT;
    if (items <= 0) return APMOE_OK;
    clear_stale_error();
    if (gu)
        hipLaunchKernelGGL(tile_kernel<2>, dim3((unsigned)items), dim3(kThreadsTile), 0, s, a, RT);
    else
        hipLaunchKernelGGL(tile_kernel<1>, dim3((unsigned)items), dim3(kThreadsTile), 0, s, a, RT);
    return launch_status();
}

}  // namespace apmoe

using namespace apmoe;

namespace apmoe {
namespace {

// Validation and dispatch shared by both entry points; ws may be NULL when the
// shapes never split K (apmoe_workspace_bytes says how much a call needs).
int gemm_call(int stage, const apmoe_expert* experts, const int8_t* bits, int E, const int32_t* offsets,
              const int32_t* sorted_slots, int k, const uint16_t* in, void* out, int T, int H, int I,
              int mfma_min_tokens, void* ws, size_t ws_bytes, size_t ws_need, void* stream) {
    const int paths = stage & (APMOE_ONLY_GEMV | APMOE_ONLY_TILE);
    stage &= ~(APMOE_ONLY_GEMV | APMOE_ONLY_TILE);
    if (stage != APMOE_GATE_UP_SWIGLU && stage != APMOE_DOWN) return APMOE_EINVAL;
    if (paths == (APMOE_ONLY_GEMV | APMOE_ONLY_TILE)) return APMOE_EINVAL;
    if (T < 0 || E < 1 || E > APMOE_MAX_EXPERTS || k < 1 || H <= 0 || I <= 0) return APMOE_EINVAL;
    if (H % 32 || I % 32 || mfma_min_tokens < 1) return APMOE_EINVAL;
    if ((long long)T * k > (1ll << 30)) return APMOE_EINVAL;
    // The kernels address the activation buffer and each weight matrix with
    // 32-bit byte offsets from raw buffer resources: both must stay below
    // 2 GiB (the fp16 copy, H * I * 2 bytes, is the largest form of a matrix).
    const long long in_bytes = stage == APMOE_GATE_UP_SWIGLU ? (long long)T * H * 2 : (long long)T * k * I * 2;
    if (in_bytes >= kMaxBufferBytes || (long long)H * I * 2 >= kMaxBufferBytes) return APMOE_EINVAL;
    if (T == 0) return APMOE_OK;
    if (!experts || !bits || !offsets || !in || !out) return APMOE_EINVAL;
    if (stage == APMOE_GATE_UP_SWIGLU && !sorted_slots) return APMOE_EINVAL;
    if (ws_bytes < ws_need) return APMOE_ENOSPACE;
    // A token holds at most one slot of each expert, so no group exceeds T
    // slots: below the threshold every group takes the GEMV path and the tile
    // launch is skipped (the effective threshold keeps that true for any
    // grouping the caller passes).
    const int eff_min = T < mfma_min_tokens ? INT_MAX : mfma_min_tokens;
    GemmArgs a{stage, experts, bits, E, offsets, sorted_slots, k, in, out, T, H, I, eff_min};
    hipStream_t s = as_stream(stream);
    if (paths != APMOE_ONLY_TILE) {
        const int rc = launch_gemv(a, ws, ws_bytes, s);
        if (rc != APMOE_OK) return rc;
    }
    if (paths != APMOE_ONLY_GEMV) return launch_tile(a, s);
    return APMOE_OK;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: the split-K partial sums live
// in this file-scope device array (one copy per GPU, held until the process
// ends).  Host code never passes the array's name to a kernel: on the host it
// is only a stand-in for the symbol.  Its device address is looked up once per
// device (hipGetSymbolAddress with that device current) and that address is
// what the kernels receive.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)APMOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch, or NULL on a HIP error.
void* scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

// Scratch bytes one stage needs (the split-K partial sums of its GEMV launch).
size_t noalloc_need(int stage, int T, int k, int E, int H, int I) {
    if (T <= 0 || k < 1 || E < 1 || H <= 0 || I <= 0) return 0;
    const bool gu = (stage & ~(APMOE_ONLY_GEMV | APMOE_ONLY_TILE)) == APMOE_GATE_UP_SWIGLU;
    return gu ? gemv_workspace_bytes(T, k, E, I, H, 2) : gemv_workspace_bytes(T, k, E, H, I, 1);
}

}  // namespace
}  // namespace apmoe

extern "C" int apmoe_bitplane_lut_gemm(int stage, const apmoe_expert* experts, const int8_t* bits,
                                       int E, const int32_t* offsets, const int32_t* sorted_slots,
                                       int k, const uint16_t* in, void* out, int T, int H, int I,
                                       int mfma_min_tokens, void* ws, size_t ws_bytes, void* stream) {
    const size_t need = (T > 0 && E >= 1 && k >= 1 && H > 0 && I > 0) ? apmoe_workspace_bytes(T, k, E, H, I) : 0;
    return gemm_call(stage, experts, bits, E, offsets, sorted_slots, k, in, out, T, H, I, mfma_min_tokens, ws,
                     ws_bytes, need, stream);
}

extern "C" int apmoe_bitplane_lut_gemm_noalloc(int stage, const apmoe_expert* experts, const int8_t* bits,
                                               int E, const int32_t* offsets, const int32_t* sorted_slots,
                                               int k, const uint16_t* in, void* out, int T, int H, int I,
                                               int mfma_min_tokens, void* stream) {
    const size_t need = noalloc_need(stage, T, k, E, H, I);
    if (need > kScratchBytes) return APMOE_ENOSPACE;   // beyond the fixed scratch: use apmoe_bitplane_lut_gemm
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_on_current_device();
        if (!ws) return APMOE_EHIP;
    }
    return gemm_call(stage, experts, bits, E, offsets, sorted_slots, k, in, out, T, H, I, mfma_min_tokens, ws,
                     need > 0 ? kScratchBytes : 0, need, stream);
}
