// Lossless exponent codec for fp16 weights: the host (offline) encoder.
//
// A weight's high byte (sign, the five exponent bits, the top two mantissa
// bits) is coded with a canonical Huffman code built from the matrix's own
// histogram; the low byte is kept raw.  Code lengths are limited to 12 bits so
// the GPU decodes a symbol with one lookup in a 4096-entry table.  Weights are
// taken in groups of 64 blocks of up to 144 symbols; block l of group g holds
// every 64th weight starting at g * 9216 + l, so 64 lanes decoding the 64
// blocks of a group write 64 consecutive weights per step.  The block length
// sets how many decoding waves a matrix gives the GPU (one per group): 144
// keeps a layer's few fp16 matrices to about one round of the waves the GPU
// holds at once while the per-block offsets stay 0.2 bits per weight.
#include <algorithm>
#include <cstring>
#include <queue>
#include <utility>
#include <vector>

#include "apmoe.h"

namespace {

constexpr int kSym = 256;
constexpr int kLmax = 12;
constexpr int kS = 144;      // symbols per block
constexpr int kLanes = 64;   // blocks per group

// Huffman code lengths with the fixed tie rule: a node's key is (weight, id),
// leaves have id = symbol, merged nodes 256, 257, ... in creation order; the
// two smallest keys merge first.  A lone symbol gets length 1.
void huffman_lengths(const std::vector<uint64_t>& counts, int* len) {
    for (int s = 0; s < kSym; ++s) len[s] = 0;
    typedef std::pair<uint64_t, int> Key;
    std::priority_queue<Key, std::vector<Key>, std::greater<Key>> heap;
    int live = 0;
    for (int s = 0; s < kSym; ++s)
        if (counts[s]) {
            heap.push(Key(counts[s], s));
            ++live;
        }
    if (live == 0) return;
    if (live == 1) {
        len[heap.top().second] = 1;
        return;
    }
    std::vector<int> parent(2 * kSym, -1);
    int next = kSym;
    while (heap.size() > 1) {
        const Key a = heap.top();
        heap.pop();
        const Key b = heap.top();
        heap.pop();
        parent[a.second] = next;
        parent[b.second] = next;
        heap.push(Key(a.first + b.first, next));
        ++next;
    }
    for (int s = 0; s < kSym; ++s) {
        if (!counts[s]) continue;
        int d = 0;
        for (int node = s; parent[node] >= 0; node = parent[node]) ++d;
        len[s] = d;
    }
}

// While the longest code exceeds 12 bits, raise every non-zero count to at
// least total >> (12 - r), r = 2, 3, ..., and rebuild.
void limited_lengths(const std::vector<uint64_t>& counts, int* len) {
    huffman_lengths(counts, len);
    uint64_t total = 0;
    for (uint64_t c : counts) total += c;
    for (int r = 2; *std::max_element(len, len + kSym) > kLmax; ++r) {
        const uint64_t floor = std::max<uint64_t>(1, total >> (kLmax - r));
        std::vector<uint64_t> raised(kSym);
        for (int s = 0; s < kSym; ++s) raised[s] = counts[s] ? std::max(counts[s], floor) : 0;
        huffman_lengths(raised, len);
    }
}

// Canonical codes: by (length, symbol), consecutive values.
void canonical(const int* len, uint32_t* code) {
    std::vector<std::pair<int, int>> order;
    for (int s = 0; s < kSym; ++s)
        if (len[s]) order.push_back(std::make_pair(len[s], s));
    std::sort(order.begin(), order.end());
    uint32_t c = 0;
    int prev = 0;
    for (const auto& o : order) {
        c <<= (o.first - prev);
        code[o.second] = c++;
        prev = o.first;
    }
}

uint64_t groups_of(uint64_t n) { return (n + (uint64_t)kLanes * kS - 1) / ((uint64_t)kLanes * kS); }

bool valid(const uint16_t* w, uint64_t n) {
    // n a multiple of 64; every bit offset fits 32 bits (12 bits a weight at most)
    return w && n > 0 && n % kLanes == 0 && n * (uint64_t)kLmax < (1ull << 32) - 64;
}

}  // namespace

extern "C" int apmoe_exp_plan(const uint16_t* w, uint64_t n, uint8_t* lengths, uint64_t* nwords,
                              uint64_t* nblocks) {
    if (!valid(w, n) || !lengths || !nwords || !nblocks) return APMOE_EINVAL;
    std::vector<uint64_t> counts(kSym, 0);
    for (uint64_t i = 0; i < n; ++i) ++counts[w[i] >> 8];
    int len[kSym];
    limited_lengths(counts, len);
    uint64_t bits = 0;
    for (int s = 0; s < kSym; ++s) {
        lengths[s] = (uint8_t)len[s];
        bits += counts[s] * (uint64_t)len[s];
    }
    *nwords = (bits + 31) / 32 + 2;
    *nblocks = groups_of(n) * kLanes;
    return APMOE_OK;
}

extern "C" int apmoe_exp_encode(const uint16_t* w, uint64_t n, const uint8_t* lengths, uint32_t* words,
                                uint64_t nwords, uint32_t* block_off, uint8_t* lo, uint16_t* table) {
    if (!valid(w, n) || !lengths || !words || !block_off || !lo || !table) return APMOE_EINVAL;
    int len[kSym];
    for (int s = 0; s < kSym; ++s) {
        len[s] = lengths[s];
        if (len[s] > kLmax) return APMOE_EINVAL;
    }
    for (uint64_t i = 0; i < n; ++i)
        if (!len[w[i] >> 8]) return APMOE_EINVAL;   // a symbol the lengths give no code
    uint32_t code[kSym] = {};
    canonical(len, code);
    std::memset(words, 0, nwords * sizeof(uint32_t));
    uint64_t k = 0;   // bit position
    const uint64_t ng = groups_of(n);
    for (uint64_t g = 0; g < ng; ++g) {
        const uint64_t base = g * kLanes * kS;
        const uint64_t sg = std::min<uint64_t>(kS, (n - base) / kLanes);
        for (int l = 0; l < kLanes; ++l) {
            block_off[g * kLanes + l] = (uint32_t)k;
            for (uint64_t j = 0; j < sg; ++j) {
                const int s = w[base + kLanes * j + l] >> 8;
                const int L = len[s];
                if ((k + L + 31) / 32 + 2 > nwords) return APMOE_ENOSPACE;
                for (int i = L - 1; i >= 0; --i, ++k)
                    if ((code[s] >> i) & 1u) words[k >> 5] |= 1u << (31 - (k & 31));
            }
        }
    }
    if ((k + 31) / 32 + 2 > nwords) return APMOE_ENOSPACE;
    for (uint64_t i = 0; i < n; ++i) lo[i] = (uint8_t)(w[i] & 0xFF);
    // decode table: entry p (12 peeked bits) = (length << 8) | symbol of the code prefixing p
    for (int p = 0; p < (1 << kLmax); ++p) table[p] = 0;
    for (int s = 0; s < kSym; ++s) {
        if (!len[s]) continue;
        const uint32_t first = code[s] << (kLmax - len[s]);
        const uint32_t count = 1u << (kLmax - len[s]);
        for (uint32_t p = first; p < first + count; ++p) table[p] = (uint16_t)((len[s] << 8) | s);
    }
    return APMOE_OK;
}
