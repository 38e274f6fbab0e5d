// Lossless exponent codec for fp16 weights: the GPU decoder.
//
// One wave per group of 64 blocks, lane l decoding block l: each step peeks
// 12 bits of the lane's stream, looks the symbol and its code length up in a
// 4096-entry table in LDS, and writes weight g * 9216 + 64 j + l = (symbol
// << 8) | its raw low byte, so every store of the wave covers 64 consecutive
// weights (128 bytes) and every low-byte load 64 consecutive bytes.  A lane
// keeps a 64-bit window of its stream and shifts in one 32-bit word whenever
// 32 bits are used up.  The steps go in chunks of 16 (at most 16 x 12 bits,
// so at most six words are shifted in per chunk).  The words a chunk shifts
// in come from LDS: at the start of chunk c the lane loads the 13 words from
// two past its current word (a superset of what chunk c + 1 can need, since
// chunk c moves it at most six words on) into registers, and after chunk c's
// steps, before its stores, it writes them to its slot of a two-slot LDS
// window for chunk c + 1.  A step's refill is then an LDS read, and the only
// waits on global loads fall at chunk ends, a whole chunk after the loads
// went out and never behind a store.  (Loading the
// next word from global memory at each refill made every refill wait for the
// previous one's load: the compiler cannot count loads across the
// data-dependent refill branch, so it waited for all of them.)  The stream is
// read through a buffer resource of nwords words: words past the end (and
// anything a malformed stream points at) read as zeros.
#include "common.hpp"
#include "decode.hpp"

namespace apmoe {
namespace {

constexpr int kDWaves = 4;
constexpr int kLmax = 12;
constexpr int kS = 144;   // symbols per block (the stream format's block length)
constexpr int kGroup = kWave * kS;
constexpr int kC = 16;        // steps per chunk
constexpr int kWin = 13;      // words staged per chunk
constexpr int kWinPad = 16;   // LDS words per lane and slot

// Up to kMaxStreams matrices per launch, passed by value: matrix m owns the
// workgroups [first[m], first[m + 1]).
constexpr int kMaxStreams = APMOE_EXP_MAX_BATCH;
struct DecodeBatch {
    const uint32_t* words[kMaxStreams];
    const uint32_t* block_off[kMaxStreams];
    const uint8_t* lo[kMaxStreams];
    const uint16_t* table[kMaxStreams];
    uint16_t* out[kMaxStreams];
    uint64_t n[kMaxStreams];
    uint32_t nwords[kMaxStreams];
    uint32_t first[kMaxStreams + 1];
    int count;
};

__global__ __launch_bounds__(kDWaves * kWave) void exp_decode_kernel(const DecodeBatch bt) {
    int m = 0;   // the matrix of this workgroup (uniform)
    while (m + 1 < bt.count && blockIdx.x >= bt.first[m + 1]) ++m;
    const uint32_t* __restrict__ words = bt.words[m];
    const uint32_t nwords = bt.nwords[m];
    const uint32_t* __restrict__ block_off = bt.block_off[m];
    const uint8_t* __restrict__ lo = bt.lo[m];
    const uint16_t* __restrict__ table = bt.table[m];
    const uint64_t n = bt.n[m];
    uint16_t* __restrict__ out = bt.out[m];
    const uint32_t wg = blockIdx.x - bt.first[m];
    __shared__ uint16_t tab[1 << kLmax];
    __shared__ uint32_t win[kDWaves][2][kWinPad][kWave];   // [wave][slot][word][lane]: lanes on distinct banks
    for (int i = threadIdx.x; i < (1 << kLmax); i += blockDim.x) tab[i] = table[i];
    __syncthreads();
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const uint64_t g = (uint64_t)wg * kDWaves + wave;
    const uint64_t base = g * kGroup;
    if (base >= n) return;   // uniform over the wave; no barrier follows
    const int sg = (int)min<uint64_t>(kS, (n - base) / kWave);
    const uint32_t k = block_off[g * kWave + lane];
    const __amdgpu_buffer_rsrc_t ws = make_rsrc(words, 4u * nwords);
    uint32_t wi = k >> 5, off = k & 31;
    uint64_t buf = ((uint64_t)buf_load_u32(ws, 4u * wi) << 32) | buf_load_u32(ws, 4u * (wi + 1));
    // the 13 words from wi + 2: what the first chunk shifts in
    uint32_t nx[kWin];
    auto load_win = [&](uint32_t from) {
#pragma unroll
        for (int a = 0; a < kWin; ++a) nx[a] = buf_load_u32(ws, 4u * (from + a));
    };
    auto stage_win = [&](int slot) {
#pragma unroll
        for (int a = 0; a < kWin; ++a) win[wave][slot][a][lane] = nx[a];
    };
    const uint8_t* lp = lo + base + lane;
    uint16_t* op = out + base + lane;
    uint32_t lv[kC];   // raw low bytes of the current chunk (indices past sg repeat the last)
    auto load_lo = [&](int j0) {
#pragma unroll
        for (int u = 0; u < kC; ++u) lv[u] = lp[(size_t)kWave * min(j0 + u, sg - 1)];
    };
    // software pipeline over chunks: chunk c decodes from LDS slot c % 2; at
    // its end the window for chunk c + 1 (loaded a chunk earlier) is staged
    // and chunk c's weights are formed, then the loads for chunk c + 1's low
    // bytes and chunk c + 2's window go out, and last chunk c's weights are
    // stored, so every wait is for operations issued a chunk earlier
    load_win(wi + 2);
    stage_win(0);
    uint32_t cbase = wi + 2;   // stream word at position 0 of the current slot
    load_win(wi + 2);          // chunk 1 moves at most six words on: this window covers it
    uint32_t nbase = wi + 2;
    load_lo(0);
    for (int j0 = 0, c = 0; j0 < sg; j0 += kC, c ^= 1) {
        uint32_t hv[kC];   // decoded high bytes
        // nw is the word a refill would shift in (stream word wi + 2), read
        // from LDS at the end of every step for the next one: that read and
        // the next step's table lookup go out together, so a step waits for
        // one LDS round trip, not two.  The read is volatile so that it is not
        // sunk into the refill branch.  At most six refills per chunk keep the
        // index below 12 for any code of at most 12 bits; the clamp bounds a
        // malformed table.
        typedef __attribute__((address_space(3))) const volatile uint32_t lds_vu32;
        lds_vu32* wv = (lds_vu32*)&win[wave][c][0][lane];
        uint32_t nw = wv[min(wi + 2 - cbase, (uint32_t)kWin - 1) * kWave];
#pragma unroll
        for (int u = 0; u < kC; ++u) {   // steps past sg decode what follows the block
            const uint32_t e = tab[(uint32_t)((buf << off) >> (64 - kLmax))];
            off += e >> 8;
            if (off >= 32) {
                off -= 32;
                buf = (buf << 32) | nw;
                ++wi;
            }
            nw = wv[min(wi + 2 - cbase, (uint32_t)kWin - 1) * kWave];
            hv[u] = (e & 0xFFu) << 8;
        }
        // nothing after the steps moves into them: every wait below is for
        // memory operations issued a chunk ago, and the new loads go out only
        // after those waits
        __builtin_amdgcn_sched_barrier(0);
        stage_win(c ^ 1);
        uint32_t w[kC];
#pragma unroll
        for (int u = 0; u < kC; ++u) w[u] = hv[u] | lv[u];
        __builtin_amdgcn_sched_barrier(0);
        cbase = nbase;
        nbase = wi + 2;
        load_win(nbase);
        load_lo(j0 + kC);
        if (j0 + kC <= sg) {   // uniform over the wave
#pragma unroll
            for (int u = 0; u < kC; ++u) op[(size_t)kWave * (j0 + u)] = (uint16_t)w[u];
        } else {
#pragma unroll
            for (int u = 0; u < kC; ++u)
                if (j0 + u < sg) op[(size_t)kWave * (j0 + u)] = (uint16_t)w[u];
        }
    }
}

}  // namespace
}  // namespace apmoe

using namespace apmoe;

namespace {
int check_stream(const uint32_t* words, uint64_t nwords, const uint32_t* block_off, const uint8_t* lo,
                 const uint16_t* table, uint64_t n, const uint16_t* out, uint64_t& wgs) {
    if (!words || !block_off || !lo || !table || !out) return APMOE_EINVAL;
    if (n == 0 || n % kWave || nwords < 2 || nwords >= (1ull << 30)) return APMOE_EINVAL;
    const uint64_t groups = (n + kGroup - 1) / kGroup;
    wgs = (groups + kDWaves - 1) / kDWaves;
    return APMOE_OK;
}
}  // namespace

extern "C" int apmoe_exp_decode_batch(int count, const uint32_t* const* words, const uint64_t* nwords,
                                      const uint32_t* const* block_off, const uint8_t* const* lo,
                                      const uint16_t* const* table, const uint64_t* n, uint16_t* const* out,
                                      void* stream) {
    if (count < 1 || count > kMaxStreams || !words || !nwords || !block_off || !lo || !table || !n || !out)
        return APMOE_EINVAL;
    DecodeBatch bt = {};
    bt.count = count;
    uint64_t total = 0;
    for (int m = 0; m < count; ++m) {
        uint64_t wgs = 0;
        const int rc = check_stream(words[m], nwords[m], block_off[m], lo[m], table[m], n[m], out[m], wgs);
        if (rc != APMOE_OK) return rc;
        bt.words[m] = words[m];
        bt.nwords[m] = (uint32_t)nwords[m];
        bt.block_off[m] = block_off[m];
        bt.lo[m] = lo[m];
        bt.table[m] = table[m];
        bt.n[m] = n[m];
        bt.out[m] = out[m];
        bt.first[m] = (uint32_t)total;
        total += wgs;
        if (total > 0x7FFFFFFFull) return APMOE_EINVAL;
    }
    bt.first[count] = (uint32_t)total;
    clear_stale_error();
    hipLaunchKernelGGL(exp_decode_kernel, dim3((unsigned)total), dim3(kDWaves * kWave), 0, as_stream(stream), bt);
    return launch_status();
}

extern "C" int apmoe_exp_decode(const uint32_t* words, uint64_t nwords, const uint32_t* block_off, const uint8_t* lo,
                                const uint16_t* table, uint64_t n, uint16_t* out, void* stream) {
    return apmoe_exp_decode_batch(1, &words, &nwords, &block_off, &lo, &table, &n, &out, stream);
}
