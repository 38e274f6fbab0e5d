// Bit-plane + LUT GEMV path of apmoe_bitplane_lut_gemm: expert groups smaller
// than mfma_min_tokens (decode-sized groups).
//
// Layout of the work (gfx950, wave64), D[row][token] = sum_k W[row][k] X[token][k]:
//
// Bit-plane experts with at most 32 tokens (the decode case), with
// v_mfma_f32_32x32x16_f16 on 32-row blocks:
//   A operand (W): lane l holds row l % 32 of its wave pair's block and eight
//                  consecutive columns of the plane word it decodes; waves
//                  2p and 2p + 1 share rows 32p..32p+31 and split each K step
//                  (128 columns = 4 words): wave parity h takes words 2h and
//                  2h + 1, lane l word 2h + l / 32.
//   B operand (X): lane l holds token l % 32 at the same eight columns.
//   D:             lane l holds rows 8*(r/4) + 4*(l/32) + r%4 (r = 0..15) of
//                  token l % 32; the pair adds its two halves at the end.
// Other groups (fp16 rows, or more than 32 tokens), with
// v_mfma_f32_16x16x32_f16 on 16-row blocks:
//   A operand (W): lane l holds row (l % 16) of the wave's 16-row block and
//                  the eight consecutive columns 8*q + 0..7 of the 32-column
//                  word that lane group g = l / 16 owns in this K step
//                  (q = 0..3 picks one of the four MFMAs a word feeds).
//   B operand (X): lane l holds token (l % 16) of a 16-token tile at the
//                  same eight columns.
//   D:             lane l holds rows 4*g + 0..3 for token l % 16.
//   One decoded A operand feeds up to four 16-token tiles.
//
// A workgroup is four waves on 64 consecutive rows of one expert (one item:
// expert, 64-row block, K split), so the four waves read the same
// activations: the workgroup stages each K step's activation tiles in LDS
// once (double-buffered, one barrier per step; 16-byte chunks XOR-swizzled by
// token row, so neither the stores nor the operand reads conflict) and every
// wave reads its B operands from there.  LDS holds 48 KB and the kernel 168
// VGPRs, so three workgroups share a CU.  The grid holds one workgroup per
// possible item and is not persistent: the hardware dispatcher hands items to
// free CUs, which balances items of very different cost (3..6-bit or fp16
// rows, 1..4 tiles).
//
// Decode of one lane's word (32 columns of one row, b planes):
//   * the plane words come from the packed layout: one 256-byte run per plane
//     and 16-row group per step, so every load uses whole cache lines, and
//     they are issued several steps ahead into a register ring;
//   * the b plane words are bit-transposed in registers with delta swaps,
//     giving eight registers R_s whose byte u is the b-bit code of column
//     8*u + s (an 8x8 bit transpose per byte lane; the swaps of distance 1
//     and 2 run first, while the planes past b are still zero words, so
//     they cost nothing);
//   * each wave stages the LUTs of its 16 rows in LDS: the entry of code c for
//     row r of wave w sits at c * 256 + 64 * w + 4 * r, gate in the low and up
//     in the high half of the dword.  A lookup address (code in byte 1, the
//     lane's row slot in byte 0) takes one byte permute.  On the 32-row path
//     the 32 lanes of a half-wave hold 32 different rows, so they hit 32
//     different banks whatever the codes;
//   * a second permute packs each pair of looked-up halves into an operand
//     dword, and every lookup of a step is issued before its first MFMA.
//   * 3-bit experts on the 32-row path instead keep, per row and matrix, a
//     table of the 64 code pairs (one fp16 pair = one operand dword), so one
//     32-bit lookup replaces two 16-bit lookups and the packing permute.
// Only the top b planes of a b-bit expert are read.  On the 32-row path the
// activations are loaded as far ahead as the plane words: vector loads retire
// in order, so a nearer activation load would make its wait also wait for
// the planes issued before it.
//
// When the host splits K (only while each split keeps enough K steps to repay
// an item's prologue and the launch stays within about four workgroups per
// CU), each split writes fp32 partial sums to the workspace and a finalize
// kernel adds them in split order (and applies SwiGLU), so results never
// depend on scheduling.
#include <algorithm>

#include "common.hpp"
#include "decode.hpp"

namespace apmoe {
namespace {

constexpr int kWaves = 4;                    // 16-row blocks per item
constexpr int kThreads = kWaves * kWave;
constexpr int kItemRows = 16 * kWaves;
constexpr int kMaxTiles = 4;                 // 16-token tiles per pass
constexpr int kXRow = 256;                   // bytes per token row of a tile (128 halves)
constexpr int kXTile = 16 * kXRow;
// LDS: the four waves' LUTs at 0 (2^6 codes x 4 waves x 16 rows x 4 bytes),
// then the double-buffered activation ring: 48 KB, three workgroups per CU.
constexpr int kLutBytes = 64 * 256;
constexpr int kXRing = kLutBytes;
constexpr int kLdsBytes = kXRing + 2 * kMaxTiles * kXTile;
static_assert(kLdsBytes <= 48 * 1024, "three workgroups per CU");
constexpr int kTargetGroups = 1024;          // workgroups a K split may grow a launch to (4 per CU)

// Weight sources of one item.  Buffer resources are rebuilt per load group
// with num_records = 0 when the group is not needed, so every load is issued
// unconditionally (static wait counts) and unneeded ones move no data.
struct Mats {
    gu32_t* lut[2];          // LUT_b as pairs of halves, [rows][2^b]
    const void* planes[2];   // packed plane slabs
    const void* w16[2];      // fp16 rows
    uint32_t pbytes, wbytes;
};

struct Shape {
    int rows, K, Wd, nsteps, k, KS, S;
    const void* in;       // activations
    uint32_t in_bytes;
    const int32_t* slots;
    float* partial;       // [KS][S][NMAT][rows] when KS > 1
};

struct Item {
    int e, off, m, b, rb, ks;
};

// Item of workgroup `idx`: experts on this path each own ceil(rows / 64) row
// blocks times KS splits, in expert order.  Every wave finds it on its own:
// the slot counts and bitwidths of all experts (up to four chunks of 64) are
// loaded at once and a wave-wide scan per chunk numbers the items; returns
// false past the last item.
//
// Item orders.  ORD == kRotated (gate/up): with one K split, at most 64
// experts and between 2 and 3 items per CU,
// ncu is the CU count: the dispatcher places workgroups b, b + ncu and
// b + 2 ncu on one CU, so the first N - 2 ncu block numbers land on the CUs
// that hold three items.  The items are then rotated so that those blocks
// take the last items (the least routed experts, the cheapest) and the head of
// the expert order (fp16 always-on experts, the most routed ones) lands on CUs
// that hold two.  ORD == kXcdRuns (down): the dispatcher sends workgroup j to
// XCD j % 8, each XCD with its own L2.  The items are cut into runs of kRun
// consecutive items (consecutive row blocks of one expert, which all read the
// same rows of A) dealt to the XCDs in turn: workgroup j = 8 s + x takes item
// r kRun + s % kRun of run r = (s / kRun) 8 + x.  An expert's A rows are then
// fetched by about nrb / kRun L2s instead of all eight, while every XCD still
// gets an even share of the runs.  The launch rounds its grid up to a multiple
// of 8 kRun.  Runs of 8 cut the down stage's counted HBM bytes from 1.15x to
// 1.07x the algorithmic bytes at the same launch time; runs of 16 (1.03x) and
// 32 (1.01x) were about 12% slower, also with the runs dealt to the XCDs in a
// rotating order, so it is not XCD imbalance: more CUs of one XCD then read
// the same A rows at the same moment.
constexpr int kMaxChunks = APMOE_MAX_EXPERTS / kWave;
enum ItemOrder { kRotated = 0, kXcdRuns = 1 };
constexpr int kXcds = 8;
constexpr int kRun = 8;

template <int ORD>
__device__ __forceinline__ bool find_item(const GemmArgs& a, int nrb, int KS, int idx, int ncu, Item& it) {
    const int lane = threadIdx.x % kWave;
    const int nch = (a.E + kWave - 1) / kWave;
    int o[kMaxChunks], m[kMaxChunks], b[kMaxChunks], n[kMaxChunks], inc[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        o[c] = 0;
        m[c] = 0;
        b[c] = 0;
        const int e = c * kWave + lane;
        if (c < nch && e < a.E) {
            o[c] = a.offsets[e];
            m[c] = a.offsets[e + 1] - o[c];
            b[c] = a.bits[e];
        }
    }
    int total = 0;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        n[c] = (m[c] > 0 && m[c] < a.mfma_min_tokens && valid_bits(b[c])) ? nrb : 0;
        inc[c] = 0;
        if (c < nch) {   // uniform
            inc[c] = wave_incl_scan(n[c]) + total;
            total = __builtin_amdgcn_readlane(inc[c], kWave - 1);
        }
    }
    if constexpr (ORD == kXcdRuns) {
        const int x = idx % kXcds, sl = idx / kXcds;
        idx = ((sl / kRun) * kXcds + x) * kRun + sl % kRun;
    }
    if (idx >= total * KS) return false;
    if constexpr (ORD == kRotated) {
        if (KS == 1 && a.E <= kWave) {
            const int three = total - 2 * ncu;   // CUs that hold a third item
            if (three > 0 && three <= ncu) idx = (idx - three + total) % total;
        }
    }
    const int blk = idx / KS;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        if (c >= nch) break;   // uniform
        const int first = inc[c] - n[c];
        const unsigned long long hit = __ballot(n[c] > 0 && blk >= first && blk < first + n[c]);
        if (hit) {
            const int src = __ffsll((long long)hit) - 1;
            it.e = __builtin_amdgcn_readfirstlane(c * kWave + src);
            it.m = __builtin_amdgcn_readlane(m[c], src);
            it.b = __builtin_amdgcn_readlane(b[c], src);
            it.rb = blk - __builtin_amdgcn_readlane(first, src);
            it.off = __builtin_amdgcn_readlane(o[c], src);   // no second, dependent load
            it.ks = idx % KS;
            return true;
        }
    }
    return false;
}

// Stage the LUTs of this wave's 16 rows: the entry of code v for row r sits
// at v * 256 + 64 * wave + 4 * r (tab points at 64 * wave), gate in the low
// and up in the high half of the dword.  Lane (r = lane % 16, p = lane / 16)
// writes codes v0 + 2p and v0 + 2p + 1.
template <int NMAT, int B>
__device__ __forceinline__ void stage_luts(char* tab, const Mats& mv, int rowc, int lane) {
    constexpr int nent = 1 << B;
    const int sl = lane & 15;
    const int row = rowc + sl;
#pragma unroll
    for (int v0 = 0; v0 < nent; v0 += 8) {
        const int v = v0 + 2 * (lane >> 4);
        const uint32_t g = mv.lut[0][(row * nent + v) >> 1];
        uint32_t e0 = g & 0xFFFFu, e1 = g >> 16;
        if (NMAT == 2) {
            const uint32_t u = mv.lut[1][(row * nent + v) >> 1];
            e0 = __builtin_amdgcn_perm(u, g, 0x05040100u);
            e1 = __builtin_amdgcn_perm(u, g, 0x07060302u);
        }
        *reinterpret_cast<uint32_t*>(tab + v * 256 + 4 * sl) = e0;
        *reinterpret_cast<uint32_t*>(tab + (v + 1) * 256 + 4 * sl) = e1;
    }
}

// 3-bit experts on the 32-row path look up two codes at once: per row and
// matrix, a table of the 64 code pairs (c0, c1) -> (lut[c0], lut[c1]) as one
// fp16 pair (the MFMA operand dword of two adjacent columns), gate at 0 and up
// at 16 KB, entry of pair p for row slot r at p * 256 + 4 * r.  Lane
// (r = lane % 16, g = lane / 16) of wave w writes the pairs with c0 = 2g,
// 2g + 1 of row slot 16 w + r.
constexpr int kPairTable = 64 * 256;
template <int NMAT>
__device__ __forceinline__ void stage_pair_luts(char* lds, const Mats& mv, int rowc, int wave, int lane) {
    const int sl = lane & 15, g = lane >> 4;
    const int row = rowc + sl;
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat) {
        const gu32_t* l = mv.lut[mat] + (size_t)row * 4;   // eight halves
        uint32_t h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = l[j];
        const uint32_t d = l[g];                           // halves c0 = 2g, 2g + 1
        char* tab = lds + mat * kPairTable + 64 * wave + 4 * sl + 2 * g * 256;
#pragma unroll
        for (int c1 = 0; c1 < 8; ++c1)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t sel = (j ? 0x0302u : 0x0100u) | ((c1 & 1) ? 0x07060000u : 0x05040000u);
                *reinterpret_cast<uint32_t*>(tab + (j + 8 * c1) * 256) = __builtin_amdgcn_perm(h[c1 >> 1], d, sel);
            }
    }
}

// Results of one 16-token tile in this lane (rows row..row+3, token tok): the
// final value, or this K split's partial sums.
template <int NMAT>
__device__ __forceinline__ void store_result(const GemmArgs& a, const Shape& sh, const Item& it, int row, int tok,
                                             const float4_t (&s)[NMAT]) {
    if (tok >= it.m) return;
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

// One pass of the workgroup over its K steps [s0, s1) for the tokens
// t0 .. t0 + 16*TT - 1 of the item.  Per step: issue the activation loads two
// steps ahead and the weight loads D steps ahead, run this step's MFMAs
// (B operands from the LDS tile), write the next step's activation tile
// (loaded a step earlier), barrier.
//
// W32 (bit-plane experts, at most 32 tokens): v_mfma_f32_32x32x16_f16 on
// 32-row blocks.  Waves 2p and 2p + 1 share rows 32p..32p+31 of the item and
// split every step's columns (wave parity h takes words 2h, 2h + 1; lane l
// holds row l % 32 and word 2h + l / 32), so the 32 lanes of a half-wave read
// 32 different rows' LUT slots: the lookups are free of bank conflicts with
// one table copy.  The pair adds its two halves at the end.
template <int NMAT, int B, int TT, bool W32 = false>
__device__ __forceinline__ void kpass(const GemmArgs& a, char* lds, const Shape& sh, const Item& it, const Mats& mv,
                                      int t0, int s0, int s1, int wave, int lane, bool live, int rowc) {
    // Steps of weights in flight, within the 168-register budget: deeper for
    // the small-tile variants, which hold the fewest accumulators and operand
    // registers (measured on the decode shapes).  NB (the unroll) stays even
    // so the two activation buffers alternate with u.
    constexpr int D = B == 16 ? (NMAT == 2 ? (TT == 1 ? 3 : 1) : 3)
                              : ((TT == 1 || W32) ? (NMAT == 2 ? 3 : 5) : (TT == 2 ? 3 : 1));
    static_assert(!W32 || (B != 16 && TT <= 2), "W32 covers bit-plane experts with up to 32 tokens");
    constexpr int NB = D + 1;
    static_assert(NB % 2 == 0, "the activation buffers alternate with u");
    const int tid = threadIdx.x;
    const int i = lane & 15, g = lane >> 4;

    // activation staging: thread -> token row xn of every tile, 16-byte chunk xc
    const int xc = tid & 15, xn = tid >> 4;
    uint32_t xrow[TT];
    bool xok[TT];
#pragma unroll
    for (int j = 0; j < TT; ++j) {
        const int n = t0 + 16 * j + xn;
        xok[j] = n < it.m;
        const int nn = min(n, it.m - 1);
        const int row = NMAT == 2 ? sh.slots[it.off + nn] / sh.k : it.off + nn;
        xrow[j] = (uint32_t)row * (uint32_t)sh.K * 2u;
    }
    // 3-bit experts on the 32-row path keep pair tables (one per matrix) in
    // the first 32 KB; the ring follows them
    constexpr bool kPair = W32 && B == 3;
    static_assert(!kPair || 2 * kPairTable + 2 * TT * kXTile <= kLdsBytes, "pair tables and ring fit");
    char* ring = lds + (kPair ? 2 * kPairTable : kXRing);
    // activations travel global -> registers (XD steps ahead) -> LDS ring
    // slot (one step ahead); xs[k] holds the step with (step - s0) % NXB == k.
    // Vector loads retire in order, so waiting for a step's activations also
    // waits for every load issued before them: on the W32 path they are
    // loaded as far ahead as the plane words (XD = D), so that wait never
    // cuts the planes' prefetch distance short.
    constexpr int XD = W32 ? D : 2;
    constexpr int NXB = W32 ? NB : 2;
    half8_t xs[NXB][TT];
    auto x_load = [&](half8_t (&x)[TT], int s) {   // steps past s1 read zeros
        const __amdgpu_buffer_rsrc_t r = make_rsrc(sh.in, s < s1 ? sh.in_bytes : 0u);
        const int col = 128 * s + 8 * xc;
#pragma unroll
        for (int j = 0; j < TT; ++j)
            x[j] = buf_load_h8(r, (xok[j] && col < sh.K) ? xrow[j] + 2u * (uint32_t)col : kOutOfRange);
    };
    auto x_store = [&](const half8_t (&x)[TT], int slot) {
        char* p = ring + slot * (TT * kXTile) + xn * kXRow + 16 * (xc ^ xn);   // chunk c of row n at c ^ n
#pragma unroll
        for (int j = 0; j < TT; ++j) *reinterpret_cast<half8_t*>(p + j * kXTile) = x[j];
    };

    float4_t acc[NMAT][TT];
    float16_t acc32[NMAT];
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[mat][tt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 16; ++r) acc32[mat][r] = 0.f;
    }
    // W32: row block of the wave pair, word half, token row of the B operand
    const int hp = wave & 1, rowc32 = rowc - 16 * hp;
    const int n32 = lane & 31, h32 = lane >> 5;
    const int nn = TT == 1 ? (n32 & 15) : n32;   // tokens past the staged tile read a staged row

    // B operands of column group q from a ring slot (lane group g holds the
    // columns 32g + 8q + 0..7 of the step: chunk 4g + q of row i)
    auto b_tiles = [&](int slot, int q, half8_t (&bx)[TT]) {
        const char* p = ring + slot * (TT * kXTile) + i * kXRow + 16 * ((4 * g + q) ^ i);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) bx[tt] = *reinterpret_cast<const half8_t*>(p + tt * kXTile);
    };

    if constexpr (B == 16) {
        half8_t wr[NB][NMAT][4];
        // fp16 rows: MFMA q takes the step's columns 32q + 8g + 0..7, so each
        // load instruction reads 64 contiguous bytes of every row
        auto w_load = [&](half8_t (&w)[NMAT][4], int s) {   // idle waves and steps past s1 read zeros
            const uint32_t n = (live && s < s1) ? mv.wbytes : 0u;
            const uint32_t base = ((uint32_t)(rowc + i) * (uint32_t)sh.K + 128u * s + 8u * g) * 2u;
#pragma unroll
            for (int mat = 0; mat < NMAT; ++mat) {
                const __amdgpu_buffer_rsrc_t r = make_rsrc(mv.w16[mat], n);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w[mat][q] = buf_load_h8(r, 4 * s + q < sh.Wd ? base + 64u * q : kOutOfRange);
            }
        };
        auto compute = [&](const half8_t (&w)[NMAT][4], int slot) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                half8_t bx[TT];
                const char* p = ring + slot * (TT * kXTile) + i * kXRow + 16 * ((4 * q + g) ^ i);
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) bx[tt] = *reinterpret_cast<const half8_t*>(p + tt * kXTile);
#pragma unroll
                for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt)
                        acc[mat][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w[mat][q], bx[tt], acc[mat][tt], 0, 0, 0);
            }
        };
        x_load(xs[0], s0);
        x_load(xs[1], s0 + 1);
#pragma unroll
        for (int u = 0; u < D; ++u) w_load(wr[u], s0 + u);
        x_store(xs[0], 0);
        __syncthreads();
        for (int s = s0; s < s1; s += NB) {
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int st = s + u;   // past s1 (the last group's tail): loads read zeros, no MFMAs
                x_load(xs[u % 2], st + 2);
                w_load(wr[(u + D) % NB], st + D);
                if (live && st < s1) compute(wr[u], (st - s0) & 1);
                x_store(xs[(u + 1) % 2], (st + 1 - s0) & 1);
                __syncthreads();
            }
        }
    } else {
        uint32_t pw[NB][NMAT][B];
        const uint32_t slab = (uint32_t)sh.rows * 16u * (uint32_t)sh.nsteps;   // bytes per plane
        // the lane's word of each plane: row group, word within the step's run
        const uint32_t rg = W32 ? (uint32_t)((rowc32 >> 4) + (n32 >> 4)) : (uint32_t)(rowc >> 4);
        const uint32_t lw = W32 ? 64u * (uint32_t)(2 * hp + h32) + 4u * (uint32_t)(n32 & 15) : 4u * (uint32_t)lane;
        auto p_load = [&](uint32_t (&w)[NMAT][B], int s) {   // idle waves and steps past s1 read zeros
            const uint32_t n = (live && s < s1) ? mv.pbytes : 0u;
            const uint32_t at = (rg * (uint32_t)sh.nsteps + (uint32_t)min(s, sh.nsteps - 1)) * 256u + lw;
#pragma unroll
            for (int mat = 0; mat < NMAT; ++mat) {
                const __amdgpu_buffer_rsrc_t r = make_rsrc(mv.planes[mat], n);
#pragma unroll
                for (int p = 0; p < B; ++p) w[mat][p] = buf_load_u32(r, at, p * slab);
            }
        };
        // lookup address: byte 0 = the lane's row slot, byte 1 = code (the
        // pair's 32 rows are the two waves' 16-row tables, side by side)
        const uint32_t lane_off = W32 ? (((uint32_t)(wave >> 1) << 7) | (4u * (uint32_t)n32))
                                      : (((uint32_t)wave << 6) | (4u * (lane & 15)));
        auto compute = [&](const uint32_t (&w)[NMAT][B], int slot) {
            uint32_t qv[NMAT][8];
#pragma unroll
            for (int mat = 0; mat < NMAT; ++mat) {
#pragma unroll
                for (int rr = 0; rr < 8; ++rr) qv[mat][rr] = rr < B ? w[mat][B - 1 - rr] : 0u;  // bit rr <- plane B-1-rr
                transpose_bytes<B>(qv[mat]);
            }
            // Every lookup of the step (four column groups, both matrices) is
            // issued before the first MFMA that needs one, so the step pays one
            // LDS round trip instead of one per column group; a permute packs
            // each pair of looked-up halves into one operand dword (3-bit
            // pair tables return the dword whole: byte u of pc[mat][c] is the
            // pair code of columns 8u + 2c, 8u + 2c + 1).
            {
                uint32x4_t w[4][NMAT];
                if constexpr (kPair) {
                    uint32_t pc[NMAT][4];
#pragma unroll
                    for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                        for (int c = 0; c < 4; ++c) pc[mat][c] = qv[mat][2 * c] | (qv[mat][2 * c + 1] << 3);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t sel = 0x0C0C0400u | ((uint32_t)q << 8);
#pragma unroll
                        for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                            for (int c = 0; c < 4; ++c)
                                w[q][mat][c] = *reinterpret_cast<const uint32_t*>(
                                    lds + mat * kPairTable + __builtin_amdgcn_perm(pc[mat][c], lane_off, sel));
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t sel = 0x0C0C0400u | ((uint32_t)q << 8);
#pragma unroll
                        for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                const uint32_t lo = *reinterpret_cast<const uint16_t*>(
                                    lds + 2 * mat + __builtin_amdgcn_perm(qv[mat][2 * c], lane_off, sel));
                                const uint32_t hi = *reinterpret_cast<const uint16_t*>(
                                    lds + 2 * mat + __builtin_amdgcn_perm(qv[mat][2 * c + 1], lane_off, sel));
                                w[q][mat][c] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                            }
                    }
                }
                if constexpr (W32) {
                    // B operand: token nn, columns 32 (2 hp + h32) + 8q + 0..7
                    const char* xb = ring + slot * (TT * kXTile) + (nn >> 4) * kXTile + (nn & 15) * kXRow;
                    const int cb = 4 * (2 * hp + h32);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const half8_t bx = *reinterpret_cast<const half8_t*>(xb + 16 * ((cb + q) ^ (nn & 15)));
#pragma unroll
                        for (int mat = 0; mat < NMAT; ++mat)
                            acc32[mat] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, w[q][mat]),
                                                                                bx, acc32[mat], 0, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        half8_t bx[TT];
                        b_tiles(slot, q, bx);
#pragma unroll
                        for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                            for (int tt = 0; tt < TT; ++tt)
                                acc[mat][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    __builtin_bit_cast(half8_t, w[q][mat]), bx[tt], acc[mat][tt], 0, 0, 0);
                    }
                }
            }
        };
#pragma unroll
        for (int u = 0; u < XD; ++u) x_load(xs[u], s0 + u);
#pragma unroll
        for (int u = 0; u < D; ++u) p_load(pw[u], s0 + u);
        x_store(xs[0], 0);
        __syncthreads();   // also publishes the LUT tables
        for (int s = s0; s < s1; s += NB) {
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int st = s + u;   // past s1 (the last group's tail): loads read zeros, no MFMAs
                x_load(xs[(u + XD) % NXB], st + XD);
                p_load(pw[(u + D) % NB], st + D);
                if (live && st < s1) compute(pw[u], (st - s0) & 1);
                x_store(xs[(u + 1) % NXB], (st + 1 - s0) & 1);
                __syncthreads();
            }
        }
    }

    if constexpr (W32) {
        // The odd wave of each pair hands its sums to the even one through
        // LDS ([pair][mat][element][lane]); the even wave adds them (its half
        // first) and stores rows 8 (r / 4) + 4 h32 + r % 4 for token n32.
        __syncthreads();   // the ring is free
        float* red = reinterpret_cast<float*>(ring) + (wave >> 1) * (NMAT * 16 * kWave);
        if (hp) {
#pragma unroll
            for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                for (int r = 0; r < 16; ++r) red[(mat * 16 + r) * kWave + lane] = acc32[mat][r];
        }
        __syncthreads();
        if (!hp && live) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                float4_t s[NMAT];
#pragma unroll
                for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        s[mat][c] = acc32[mat][4 * rr + c] + red[(mat * 16 + 4 * rr + c) * kWave + lane];
                store_result<NMAT>(a, sh, it, rowc32 + 8 * rr + 4 * h32, t0 + n32, s);
            }
        }
    } else if (live) {
        const int row = rowc + 4 * g;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            float4_t s[NMAT];
#pragma unroll
            for (int mat = 0; mat < NMAT; ++mat) s[mat] = acc[mat][tt];
            store_result<NMAT>(a, sh, it, row, t0 + 16 * tt + i, s);
        }
    }
}

template <int NMAT, int B>
__device__ __forceinline__ void run_item(const GemmArgs& a, char* lds, const Shape& sh, const Item& it, const Mats& mv,
                                         int wave, int lane) {
    const int row0 = it.rb * kItemRows + 16 * wave;
    const bool live = row0 < sh.rows;              // blocks past the last row idle but share the barriers
    const int rowc = live ? row0 : sh.rows - 16;
    const int per = (sh.nsteps + sh.KS - 1) / sh.KS;
    const int s0 = min(sh.nsteps, it.ks * per), s1 = min(sh.nsteps, s0 + per);
    if (s0 >= s1) return;   // uniform over the workgroup
    if constexpr (B != 16) {
        if (live) {
            if (B == 3 && it.m <= 32)
                stage_pair_luts<NMAT>(lds, mv, rowc, wave, lane);
            else
                stage_luts<NMAT, B>(lds + 64 * wave, mv, rowc, lane);
        }
    }
    if constexpr (B != 16) {
        if (it.m <= 32) {   // one pass of 32-row MFMA blocks
            if (it.m > 16)
                kpass<NMAT, B, 2, true>(a, lds, sh, it, mv, 0, s0, s1, wave, lane, live, rowc);
            else
                kpass<NMAT, B, 1, true>(a, lds, sh, it, mv, 0, s0, s1, wave, lane, live, rowc);
            return;
        }
    }
    for (int t0 = 0; t0 < it.m; t0 += 16 * kMaxTiles) {
        const int left = it.m - t0;
        if (left > 32)
            kpass<NMAT, B, 4>(a, lds, sh, it, mv, t0, s0, s1, wave, lane, live, rowc);
        else if (left > 16)
            kpass<NMAT, B, 2>(a, lds, sh, it, mv, t0, s0, s1, wave, lane, live, rowc);
        else
            kpass<NMAT, B, 1>(a, lds, sh, it, mv, t0, s0, s1, wave, lane, live, rowc);
        if (t0 + 16 * kMaxTiles < it.m) __syncthreads();   // the ring is reused by the next pass
    }
}

template <int NMAT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void gemv_kernel(GemmArgs a, int KS, float* partial, int ncu) {
    __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];

    Shape sh;
    sh.rows = NMAT == 2 ? a.I : a.H;
    sh.K = NMAT == 2 ? a.H : a.I;
    sh.Wd = sh.K / 32;
    sh.nsteps = (sh.Wd + 3) / 4;
    sh.k = a.k;
    sh.KS = KS;
    sh.S = a.T * a.k;
    sh.slots = a.sorted_slots;
    sh.partial = partial;
    sh.in = a.in;
    sh.in_bytes = (uint32_t)((NMAT == 2 ? (size_t)a.T : (size_t)sh.S) * sh.K * 2);

    Item it;
    constexpr int ORD = NMAT == 2 ? kRotated : kXcdRuns;
    if (!find_item<ORD>(a, (sh.rows + kItemRows - 1) / kItemRows, KS, blockIdx.x, ncu, it)) return;   // uniform

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;

    Mats mv;
    const apmoe_mat& m0 = NMAT == 2 ? a.experts[it.e].gate : a.experts[it.e].down;
    const apmoe_mat& m1 = a.experts[it.e].up;
    const MatView v0 = mat_view(m0, it.b), v1 = mat_view(m1, it.b);
    mv.lut[0] = (gu32_t*)v0.lut;
    mv.lut[1] = (gu32_t*)v1.lut;
    mv.planes[0] = (const void*)v0.planes;
    mv.planes[1] = (const void*)v1.planes;
    mv.w16[0] = (const void*)v0.w16;
    mv.w16[1] = (const void*)v1.w16;
    // the resource covers the b resident planes only (none at 16 bits)
    mv.pbytes = (uint32_t)(it.b <= kPlanes ? it.b : 0) * (uint32_t)sh.rows * 16u * (uint32_t)sh.nsteps;
    mv.wbytes = (uint32_t)sh.rows * (uint32_t)sh.K * 2u;

    switch (it.b) {
        case 3: run_item<NMAT, 3>(a, lds, sh, it, mv, wave, lane); break;
        case 4: run_item<NMAT, 4>(a, lds, sh, it, mv, wave, lane); break;
        case 5: run_item<NMAT, 5>(a, lds, sh, it, mv, wave, lane); break;
        case 6: run_item<NMAT, 6>(a, lds, sh, it, mv, wave, lane); break;
        default: run_item<NMAT, 16>(a, lds, sh, it, mv, wave, lane); break;
    }
}

// Rows row..row+3 of position p: the K-split partial sums added in split
// order, then SwiGLU (gate/up) or stored as they are (down).
template <int NMAT>
__device__ __forceinline__ void finalize_rows(const GemmArgs& a, int KS, const float* partial, int S, int rows, int p,
                                              int row) {
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

// Sum the K-split partials in split order (SwiGLU for gate/up).  Workgroup
// (x, y) takes positions [x * pb, (x + 1) * pb) and rows [1024 y, 1024 y +
// 1024), four rows per thread.  Positions are grouped by expert, so the
// workgroup finds the expert of its first position once and then walks expert
// ranges, skipping a whole range when that group took the tile path (or has
// no bit-plane or fp16 weights); a launch whose groups all took the tile path
// costs one lookup per workgroup.  pb is chosen on the host to keep the grid
// near a thousand workgroups.
constexpr int kFinRows = 4 * 256;
template <int NMAT>
__global__ __launch_bounds__(256) void gemv_finalize_kernel(GemmArgs a, int KS, const float* partial, int pb) {
    __shared__ int offs[APMOE_MAX_EXPERTS + 1];
    for (int e = threadIdx.x; e <= a.E; e += blockDim.x) offs[e] = a.offsets[e];
    __syncthreads();
    const int rows = NMAT == 2 ? a.I : a.H;
    const int S = a.T * a.k;
    const int row = blockIdx.y * kFinRows + 4 * threadIdx.x;
    int p = blockIdx.x * pb;
    const int pend = min(S, p + pb);
    if (p >= pend) return;   // uniform over the workgroup
    int lo = 0, hi = a.E - 1;   // expert holding position p: last e with offs[e] <= p
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offs[mid] <= p) lo = mid; else hi = mid - 1;
    }
    // offs[lo] <= p < offs[lo + 1]; offs[E] = S >= pend ends the walk at e = E - 1
    for (int e = lo; p < pend; ++e) {
        const int eend = min(pend, offs[e + 1]);
        const int m = offs[e + 1] - offs[e];
        if (m < a.mfma_min_tokens && valid_bits(a.bits[e]) && row < rows)
            for (; p < eend; ++p) finalize_rows<NMAT>(a, KS, partial, S, rows, p, row);
        p = eend;
    }
}

long long items_per_split(int T, int k, int E, int rows) {
    const long long slots = (long long)T * k;
    const long long active = E < slots ? E : slots;
    return active * ((rows + kItemRows - 1) / kItemRows);
}

}  // namespace

// K splits, chosen from shapes alone: as many as keep the workgroups of every
// expert that could be active within kTargetGroups, but at least kMinSplitSteps
// K steps per split, since each split pays an item's prologue (LUT staging and
// the first steps' loads, about five steps' worth) again.  Measured on the
// Mixtral-shaped decode layer: one token's gate/up (448 items, 32 steps) is
// fastest unsplit, its down (128 items, 112 steps) with four splits, and the
// down stage of 8 or 32 tokens (512 items) with two.
constexpr int kMinSplitSteps = 28;
int gemv_splits(int T, int k, int E, int rows, int K) {
    const long long items = items_per_split(T, k, E, rows);
    const int nsteps = (K / 32 + 3) / 4;
    long long ks = items > 0 ? kTargetGroups / items : 1;
    const int cap = nsteps / kMinSplitSteps;
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
    long long groups = items_per_split(a.T, a.k, a.E, rows) * KS;
    if (groups <= 0) return APMOE_OK;
    if (!gu) groups = (groups + kXcds * kRun - 1) / (kXcds * kRun) * (kXcds * kRun);   // whole rounds of runs
    dim3 grid((unsigned)groups), block(kThreads);
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return APMOE_EHIP;
    clear_stale_error();
    if (gu)
        hipLaunchKernelGGL(gemv_kernel<2>, grid, block, 0, s, a, KS, partial, ncu);
    else
        hipLaunchKernelGGL(gemv_kernel<1>, grid, block, 0, s, a, KS, partial, ncu);
    int rc = launch_status();
    if (rc != APMOE_OK || KS == 1) return rc;
    const long long S = (long long)a.T * a.k;
    const long long chunks = (rows + kFinRows - 1) / kFinRows;
    const long long pb = std::max<long long>(1, S * chunks / 1024);   // about a thousand workgroups
    dim3 fgrid((unsigned)((S + pb - 1) / pb), (unsigned)chunks);
    if (gu)
        hipLaunchKernelGGL(gemv_finalize_kernel<2>, fgrid, dim3(256), 0, s, a, KS, partial, (int)pb);
    else
        hipLaunchKernelGGL(gemv_finalize_kernel<1>, fgrid, dim3(256), 0, s, a, KS, partial, (int)pb);
    return launch_status();
}

}  // namespace apmoe
