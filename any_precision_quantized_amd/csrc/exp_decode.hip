// Lossless exponent codec for fp16 weights: the GPU decoder.
//
// One wave per group of 64 blocks, lane l decoding block l: each step peeks
// 12 bits of the lane's stream, looks the symbol and its code length up in a
// 4096-entry table in LDS, and writes weight g * 16384 + 64 j + l = (symbol
// << 8) | its raw low byte, so every store of the wave covers 64 consecutive
// weights (128 bytes) and every low-byte load 64 consecutive bytes.  A lane
// keeps a 64-bit window of its stream and refills it one 32-bit word at a
// time from a word it loaded at the previous refill, and works in chunks of
// 16 steps whose raw low bytes it loads and whose weights it stores together.  The stream is
// read through a buffer resource of nwords words: words past the end (and
// anything a malformed stream points at) read as zeros.
#include "common.hpp"
#include "decode.hpp"

namespace apmoe {
namespace {

constexpr int kDWaves = 4;
constexpr int kLmax = 12;
constexpr int kS = 256;
constexpr int kGroup = kWave * kS;

__global__ __launch_bounds__(kDWaves * kWave) void exp_decode_kernel(const uint32_t* __restrict__ words,
                                                                     uint32_t nwords,
                                                                     const uint32_t* __restrict__ block_off,
                                                                     const uint8_t* __restrict__ lo,
                                                                     const uint16_t* __restrict__ table, uint64_t n,
                                                                     uint16_t* __restrict__ out) {
    __shared__ uint16_t tab[1 << kLmax];
    for (int i = threadIdx.x; i < (1 << kLmax); i += blockDim.x) tab[i] = table[i];
    __syncthreads();
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const uint64_t g = (uint64_t)blockIdx.x * kDWaves + wave;
    const uint64_t base = g * kGroup;
    if (base >= n) return;   // uniform over the wave; no barrier follows
    const int sg = (int)min<uint64_t>(kS, (n - base) / kWave);
    const uint32_t k = block_off[g * kWave + lane];
    const __amdgpu_buffer_rsrc_t ws = make_rsrc(words, 4u * nwords);
    uint32_t wi = k >> 5, off = k & 31;
    uint64_t buf = ((uint64_t)buf_load_u32(ws, 4u * wi) << 32) | buf_load_u32(ws, 4u * (wi + 1));
    uint32_t nxt = buf_load_u32(ws, 4u * (wi + 2));   // the next word, loaded one refill ahead
    const uint8_t* lp = lo + base + lane;
    uint16_t* op = out + base + lane;
    // one step: look the symbol up and advance, refilling the window from
    // the word loaded at the previous refill; the weights of a chunk of 16
    // steps are stored together at its end, so a wait for a stream word
    // covers at most the previous chunk's stores.
    constexpr int kC = 16;
    auto step = [&]() -> uint32_t {
        const uint32_t e = tab[(uint32_t)((buf << off) >> (64 - kLmax))];
        off += e >> 8;
        if (off >= 32) {
            off -= 32;
            ++wi;
            buf = (buf << 32) | nxt;
            nxt = buf_load_u32(ws, 4u * (wi + 2));
        }
        return (e & 0xFFu) << 8;
    };
    for (int j0 = 0; j0 < sg; j0 += kC) {
        uint32_t lv[kC], hv[kC];   // raw low bytes (indices past sg repeat the last), decoded high bytes
#pragma unroll
        for (int u = 0; u < kC; ++u) lv[u] = lp[(size_t)kWave * min(j0 + u, sg - 1)];
#pragma unroll
        for (int u = 0; u < kC; ++u) hv[u] = step();   // steps past sg decode what follows the block
        if (j0 + kC <= sg) {   // uniform over the wave
#pragma unroll
            for (int u = 0; u < kC; ++u) op[(size_t)kWave * (j0 + u)] = (uint16_t)(hv[u] | lv[u]);
        } else {
#pragma unroll
            for (int u = 0; u < kC; ++u)
                if (j0 + u < sg) op[(size_t)kWave * (j0 + u)] = (uint16_t)(hv[u] | lv[u]);
        }
    }
}

}  // namespace
}  // namespace apmoe

using namespace apmoe;

extern "C" int apmoe_exp_decode(const uint32_t* words, uint64_t nwords, const uint32_t* block_off, const uint8_t* lo,
                                const uint16_t* table, uint64_t n, uint16_t* out, void* stream) {
    if (!words || !block_off || !lo || !table || !out) return APMOE_EINVAL;
    if (n == 0 || n % kWave || nwords < 2 || nwords >= (1ull << 30)) return APMOE_EINVAL;
    const uint64_t groups = (n + kGroup - 1) / kGroup;
    const uint64_t wgs = (groups + kDWaves - 1) / kDWaves;
    if (wgs > 0x7FFFFFFFull) return APMOE_EINVAL;
    clear_stale_error();
    hipLaunchKernelGGL(exp_decode_kernel, dim3((unsigned)wgs), dim3(kDWaves * kWave), 0, as_stream(stream), words,
                       (uint32_t)nwords, block_off, lo, table, n, out);
    return launch_status();
}
