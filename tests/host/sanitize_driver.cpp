// Host-side fuzz driver for the library's plain C++ parts, built with the
// address and undefined-behaviour sanitizers by tests/test_host_sanitize.py:
// the first-fit arena (C ABI), the plane-paging residency bookkeeping
// (claims, rollback, retirement) and the pager's copy plans, the greedy and online planners with their
// routing multipliers, and the exponent encoder (round trip through a CPU
// decode of the stream it writes).  Exits non-zero on a failed check; the
// sanitizers abort on a memory or undefined-behaviour error.
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <random>
#include <vector>

#include "apmoe.h"
#include "residency.hpp"

#define CHECK(c)                                                               \
    do {                                                                       \
        if (!(c)) {                                                            \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);    \
            return 1;                                                          \
        }                                                                      \
    } while (0)

using Rng = std::mt19937_64;

// the exponent stream format: groups of 64 blocks of up to kBlockSyms symbols
constexpr uint64_t kBlockSyms = 144;
constexpr uint64_t kGroupW = 64 * kBlockSyms;

static uint64_t uni(Rng& r, uint64_t lo, uint64_t hi) { return std::uniform_int_distribution<uint64_t>(lo, hi)(r); }

// Arena against a shadow map of 256-byte units.
static int arena_fuzz(Rng& rng) {
    for (int trial = 0; trial < 40; ++trial) {
        const uint64_t units = uni(rng, 1, 300);
        apmoe_arena* a = nullptr;
        CHECK(apmoe_arena_create(units * 256 + uni(rng, 0, 255), &a) == APMOE_OK && a);
        std::vector<char> used(units, 0);
        std::vector<std::pair<uint64_t, uint64_t>> live;
        for (int op = 0; op < 400; ++op) {
            const int kind = (int)uni(rng, 0, 2);
            if (kind == 0) {
                const uint64_t bytes = uni(rng, 1, 40 * 256);
                uint64_t off = 0;
                const int rc = apmoe_arena_alloc(a, bytes, &off);
                const uint64_t n = (bytes + 255) / 256;
                if (rc == APMOE_OK) {
                    CHECK(off % 256 == 0 && off / 256 + n <= units);
                    for (uint64_t u = off / 256; u < off / 256 + n; ++u) {
                        CHECK(!used[u]);
                        used[u] = 1;
                    }
                    live.push_back({off, bytes});
                } else {
                    CHECK(rc == APMOE_ENOSPACE);
                }
            } else if (kind == 1 && !live.empty()) {
                const size_t i = uni(rng, 0, live.size() - 1);
                CHECK(apmoe_arena_release(a, live[i].first, live[i].second) == APMOE_OK);
                for (uint64_t u = live[i].first / 256; u < live[i].first / 256 + (live[i].second + 255) / 256; ++u)
                    used[u] = 0;
                // releasing it again is refused (the range is free) and changes nothing
                CHECK(apmoe_arena_release(a, live[i].first, live[i].second) == APMOE_EINVAL);
                live.erase(live.begin() + i);
            } else {
                const uint64_t off = uni(rng, 0, units) * 256, bytes = uni(rng, 1, 8 * 256);
                const int rc = apmoe_arena_take(a, off, bytes);
                if (rc == APMOE_OK) {
                    for (uint64_t u = off / 256; u < off / 256 + (bytes + 255) / 256; ++u) {
                        CHECK(!used[u]);
                        used[u] = 1;
                    }
                    live.push_back({off, bytes});
                }
            }
            uint64_t fb = 0, largest = 0;
            int nr = 0;
            CHECK(apmoe_arena_stats(a, &fb, &largest, &nr) == APMOE_OK);
            uint64_t free_units = 0;
            for (char c : used) free_units += !c;
            CHECK(fb == free_units * 256 && largest <= fb);
        }
        // out-of-range and misaligned requests
        CHECK(apmoe_arena_release(a, units * 256, 256) == APMOE_EINVAL);
        CHECK(apmoe_arena_take(a, 3, 256) == APMOE_EINVAL);
        apmoe_arena_destroy(a);
    }
    return 0;
}

// Residency bookkeeping: random plans over E experts x 3 matrices; a claim
// either fits (then every resident block lies in the arena and no two
// overlap) or is rolled back with the arena exactly as before.
static int residency_fuzz(Rng& rng) {
    using namespace apmoe;
    for (int trial = 0; trial < 30; ++trial) {
        const int E = (int)uni(rng, 1, 12);
        std::vector<MatResidency> mats(3 * E);
        for (auto& m : mats) {
            m.slab = 256 * uni(rng, 1, 6);
            for (int b = 3; b <= 6; ++b) m.lut_bytes[b - 3] = 512ull << (b - 3);
        }
        const uint64_t size = 256 * uni(rng, 60, 900);
        apmoe_arena arena;
        arena.size = size;
        arena.free_[0] = size;
        std::vector<Block> pending;
        for (int step = 0; step < 60; ++step) {
            for (const Block& b : pending) CHECK(arena.release(b.off, b.len));
            pending.clear();
            uint64_t before = 0, largest = 0;
            arena.stats(&before, &largest, nullptr);
            for (int e = 0; e < E; ++e) {
                const int bits = (int)uni(rng, 2, 6);   // 2 stands for the fp16 fallback: no planes
                for (int j = 0; j < 3; ++j) mats[3 * e + j].want = bits == 2 ? 0 : bits;
            }
            if (!claim(arena, mats)) {
                unstage(arena, mats);
                uint64_t after = 0;
                arena.stats(&after, nullptr, nullptr);
                CHECK(after == before);
                continue;
            }
            pending = retired_blocks(mats);
            adopt(mats);
            std::vector<Block> held;
            for (const auto& m : mats) {
                CHECK(m.planes.len == (uint64_t)m.have * m.slab);
                if (m.planes.len) held.push_back(m.planes);
                if (m.lut.len) held.push_back(m.lut);
            }
            for (const Block& b : pending) held.push_back(b);
            std::sort(held.begin(), held.end(), [](const Block& x, const Block& y) { return x.off < y.off; });
            for (size_t i = 0; i < held.size(); ++i) {
                CHECK(held[i].off + held[i].len <= size);
                if (i) CHECK(held[i - 1].off + held[i - 1].len <= held[i].off);
            }
        }
    }
    return 0;
}

// Copy plans of the pager, staged and direct, run on a byte model of the
// arena: the device-side copies of one stage (one kernel, all concurrent)
// neither overlap one another's destinations nor read what another writes,
// the host-to-device bytes are exactly the new planes and LUTs, and after
// every commit each resident block holds the host copy's planes and LUT.
static bool overlap(uint64_t a, uint64_t an, uint64_t b, uint64_t bn) { return a < b + bn && b < a + an; }

static int copy_plan_fuzz(Rng& rng) {
    using namespace apmoe;
    uint64_t n_staged = 0, n_direct = 0, n_moves = 0, n_multi = 0, n_demote = 0, n_merged = 0;
    for (int trial = 0; trial < 40; ++trial) {
        const int E = (int)uni(rng, 1, 8);
        std::vector<MatResidency> mats(3 * E);
        for (auto& m : mats) {
            m.slab = 256 * uni(rng, 1, 4);
            const uint64_t l = 256 * uni(rng, 1, 3);
            for (int b = 3; b <= 6; ++b) m.lut_bytes[b - 3] = l << (b - 3);
        }
        const HostLayout L = host_layout(mats);
        std::vector<uint8_t> host(L.bytes);
        for (auto& c : host) c = (uint8_t)uni(rng, 0, 255);
        // every plane and LUT sits at its own bytes of the host copy
        std::vector<uint8_t> seen(L.bytes, 0);
        for (int e = 0; e < E; ++e)
            for (int j = 0; j < 3; ++j) {
                const MatResidency& m = mats[3 * e + j];
                for (int p = 0; p < 6; ++p) {
                    const uint64_t o = host_plane_off(mats, L, e, j, p);
                    CHECK(o + m.slab <= L.bytes);
                    for (uint64_t i = o; i < o + m.slab; ++i) CHECK(seen[i]++ == 0);
                }
                for (int b = 3; b <= 6; ++b) {
                    const uint64_t o = host_lut_off(mats, L, e, j, b);
                    CHECK(o + m.lut_bytes[b - 3] <= L.bytes);
                    for (uint64_t i = o; i < o + m.lut_bytes[b - 3]; ++i) CHECK(seen[i]++ == 0);
                }
            }
        for (uint8_t c : seen) CHECK(c == 1);
        const uint64_t size = 256 * uni(rng, 100, 1500);
        apmoe_arena arena;
        arena.size = size;
        arena.free_[0] = size;
        std::vector<uint8_t> mem(size, 0);
        std::vector<Block> pending;
        for (int step = 0; step < 40; ++step) {
            for (const Block& b : pending) CHECK(arena.release(b.off, b.len));
            pending.clear();
            const int levels[5] = {0, 3, 4, 5, 6};
            for (int e = 0; e < E; ++e) {
                const int w = levels[uni(rng, 0, 4)];
                for (int j = 0; j < 3; ++j) mats[3 * e + j].want = w;
            }
            if (!claim(arena, mats)) {
                unstage(arena, mats);
                continue;
            }
            CopyPlan plan = plan_copies(mats, L, true, 0);
            CHECK(plan.ok);
            Block staging;
            uint64_t soff = 0;
            const bool staged = uni(rng, 0, 3) != 0 && plan.staged_bytes && arena.alloc(plan.staged_bytes, &soff);
            const uint64_t cap = uni(rng, 0, 1) ? 256 * uni(rng, 1, 8) : 0;
            if (staged) {
                staging = Block{soff, align_up(plan.staged_bytes)};
                plan = plan_copies(mats, L, true, soff, cap);
            } else {
                plan = plan_copies(mats, L, false, 0, cap);
            }
            for (const Copy& c : plan.h2d) CHECK(c.bytes > 0 && (!cap || c.bytes <= cap));
            CHECK(plan.ok && plan.dev.size() <= (size_t)18 * E);
            ++(staged ? n_staged : n_direct);
            for (const MatResidency& m : mats) {
                n_moves += m.moved && m.have;
                n_multi += m.want > m.have + 1;
                n_demote += m.want && m.want < m.have;
            }
            uint64_t want_h2d = 0, got_h2d = 0;
            for (const MatResidency& m : mats) {
                if (m.want > m.have) want_h2d += (uint64_t)(m.want - m.have) * m.slab;
                if (m.new_lut) want_h2d += m.lut_bytes[m.want - 3];
            }
            for (const Copy& c : plan.h2d) {
                CHECK(c.src + c.bytes <= L.bytes && c.dst + c.bytes <= size);
                if (staged) CHECK(c.dst >= staging.off && c.dst + c.bytes <= staging.off + staging.len);
                got_h2d += c.bytes;
                std::copy(host.begin() + c.src, host.begin() + c.src + c.bytes, mem.begin() + c.dst);
            }
            CHECK(got_h2d == want_h2d);
            if (staged && !cap) {   // one range per run of adjacent step blocks: fewer than the blocks when any merged
                size_t blocks = 0;
                for (int e = 0; e < E; ++e) {
                    const MatResidency& m = mats[3 * e];
                    blocks += m.want > m.have ? m.want - std::max(m.have, 2) : m.new_lut;
                }
                CHECK(plan.h2d.size() <= blocks);
                n_merged += blocks - plan.h2d.size();
            }
            for (size_t a = 0; a < plan.dev.size(); ++a) {
                const Copy& x = plan.dev[a];
                CHECK(x.src % 16 == 0 && x.dst % 16 == 0 && x.bytes % 16 == 0);
                CHECK(x.src + x.bytes <= size && x.dst + x.bytes <= size);
                for (size_t b = 0; b < plan.dev.size(); ++b) {
                    const Copy& y = plan.dev[b];
                    CHECK(!overlap(x.dst, x.bytes, y.src, y.bytes));
                    if (a != b) CHECK(!overlap(x.dst, x.bytes, y.dst, y.bytes));
                }
            }
            const std::vector<uint8_t> snap = mem;   // the kernel's copies all read the state before it
            for (const Copy& c : plan.dev)
                std::copy(snap.begin() + c.src, snap.begin() + c.src + c.bytes, mem.begin() + c.dst);
            pending = retired_blocks(mats);
            if (staging.len) pending.push_back(staging);
            adopt(mats);
            for (int e = 0; e < E; ++e)
                for (int j = 0; j < 3; ++j) {
                    const MatResidency& m = mats[3 * e + j];
                    CHECK(m.planes.len == (uint64_t)m.have * m.slab);
                    for (int p = 0; p < m.have; ++p)
                        CHECK(std::equal(mem.begin() + m.planes.off + p * m.slab,
                                         mem.begin() + m.planes.off + (p + 1) * m.slab,
                                         host.begin() + host_plane_off(mats, L, e, j, p)));
                    if (m.have)
                        CHECK(std::equal(mem.begin() + m.lut.off, mem.begin() + m.lut.off + m.lut_bytes[m.have - 3],
                                         host.begin() + host_lut_off(mats, L, e, j, m.have)));
                }
        }
    }
    printf("copy plans: %llu staged (%llu step blocks merged into a neighbour's range), %llu direct; matrices moved "
           "%llu, raised by several steps %llu, demoted %llu\n",
           (unsigned long long)n_staged, (unsigned long long)n_merged, (unsigned long long)n_direct,
           (unsigned long long)n_moves, (unsigned long long)n_multi, (unsigned long long)n_demote);
    CHECK(n_staged && n_merged && n_direct && n_moves && n_multi && n_demote);
    return 0;
}

static int planner_fuzz(Rng& rng) {
    const int8_t all_levels[5] = {16, 6, 5, 4, 3};
    for (int trial = 0; trial < 200; ++trial) {
        const int E = (int)uni(rng, 1, 70);
        const int L = (int)uni(rng, 2, 5);
        const int8_t* levels = all_levels + (5 - L);
        std::vector<double> harm((size_t)E * L);
        std::vector<uint64_t> bytes((size_t)E * L);
        std::vector<int8_t> floors(E), out(E), now(E);
        std::vector<float> mass(E), wnorm(E);
        for (int e = 0; e < E; ++e) {
            double h = 0;
            uint64_t b = uni(rng, 5000, 1u << 24);
            for (int l = 0; l < L; ++l) {
                harm[(size_t)e * L + l] = h;
                h += std::uniform_real_distribution<double>(0, 1)(rng);
                bytes[(size_t)e * L + l] = b;
                b -= uni(rng, 1, b / 4);
            }
            floors[e] = levels[uni(rng, 1, L - 1)];
            now[e] = levels[0];
            mass[e] = uni(rng, 0, 3) ? std::uniform_real_distribution<float>(0, 2)(rng) : 0.f;
            wnorm[e] = mass[e] * std::uniform_real_distribution<float>(10, 60)(rng);
        }
        uint64_t hi = 0, lo = 0;
        for (int e = 0; e < E; ++e) {
            hi += bytes[(size_t)e * L];
            int f = 0;
            for (int l = 0; l < L; ++l)
                if (levels[l] == floors[e]) f = l;
            lo += bytes[(size_t)e * L + f];
        }
        const uint64_t budget = lo + uni(rng, 0, hi - lo + 10) - (trial % 7 == 0 ? 5 : 0);
        const int rc = apmoe_plan_bitwidths(E, L, levels, harm.data(), bytes.data(), floors.data(), budget, out.data());
        CHECK(rc == APMOE_OK || rc == APMOE_ENOSPACE);
        uint64_t total = 0;
        for (int e = 0; e < E; ++e) {
            int l = -1, f = -1;
            for (int q = 0; q < L; ++q) {
                if (levels[q] == out[e]) l = q;
                if (levels[q] == floors[e]) f = q;
            }
            CHECK(l >= 0 && l <= f);
            total += bytes[(size_t)e * L + l];
        }
        if (rc == APMOE_OK) CHECK(total <= budget);
        std::vector<double> mult(E);
        CHECK(apmoe_harm_multipliers(E, mass.data(), wnorm.data(), mult.data()) == APMOE_OK);
        for (double m : mult) CHECK(m >= 0.0);
        const int rr = apmoe_plan_routed(E, L, levels, harm.data(), bytes.data(), floors.data(), budget, mass.data(),
                                         wnorm.data(), out.data());
        CHECK(rr == APMOE_OK || rr == APMOE_ENOSPACE);
        int stage = 0;
        const int8_t stages[2] = {levels[1], levels[L - 1]};
        const int ro = apmoe_plan_online(E, L, levels, harm.data(), bytes.data(), floors.data(), 2, stages, hi,
                                         hi - budget, uni(rng, 0, 1000), now.data(), out.data(), &stage);
        CHECK(ro == APMOE_OK || ro == APMOE_ENOSPACE);
        CHECK(stage >= -1 && stage < 2);
    }
    return 0;
}

// Exponent codec: encode, then decode the stream on the CPU from the block
// offsets and the 12-bit prefix table the encoder wrote.
static int codec_fuzz(Rng& rng) {
    for (int trial = 0; trial < 24; ++trial) {
        const uint64_t n = 64 * uni(rng, 1, 900);
        std::vector<uint16_t> w(n);
        const int kind = trial % 4;
        std::geometric_distribution<int> geo(0.45);
        for (auto& v : w) {
            if (kind == 0) v = (uint16_t)uni(rng, 0, 65535);                         // every high byte
            else if (kind == 1) v = (uint16_t)((std::min(geo(rng), 255) << 8) | uni(rng, 0, 255));   // skewed: long codes
            else if (kind == 2) v = (uint16_t)(0x3C00 | uni(rng, 0, 255));           // one symbol
            else v = (uint16_t)(((uni(rng, 0, 3) + 0x30) << 8) | uni(rng, 0, 255));
        }
        uint8_t lengths[256];
        uint64_t nwords = 0, nblocks = 0;
        CHECK(apmoe_exp_plan(w.data(), n, lengths, &nwords, &nblocks) == APMOE_OK);
        std::vector<uint32_t> words(nwords), off(nblocks);
        std::vector<uint8_t> lo(n);
        std::vector<uint16_t> table(4096);
        CHECK(apmoe_exp_encode(w.data(), n, lengths, words.data(), nwords, off.data(), lo.data(), table.data()) ==
              APMOE_OK);
        // a short stream buffer is refused
        if (nwords > 2) {
            std::vector<uint32_t> shortw(nwords - 1);
            CHECK(apmoe_exp_encode(w.data(), n, lengths, shortw.data(), nwords - 1, off.data(), lo.data(),
                                   table.data()) == APMOE_ENOSPACE);
        }
        for (uint64_t blk = 0; blk < nblocks; ++blk) {
            const uint64_t g = blk / 64, l = blk % 64;
            uint64_t pos = off[blk];
            for (uint64_t j = 0; j < kBlockSyms; ++j) {
                const uint64_t i = g * kGroupW + 64 * j + l;
                if (64 * j >= std::min<uint64_t>(kGroupW, n - g * kGroupW)) break;
                CHECK(pos / 32 + 1 < nwords);
                const uint64_t pair = ((uint64_t)words[pos / 32] << 32) | words[pos / 32 + 1];
                const uint32_t peek = (uint32_t)((pair << (pos % 32)) >> 52);
                const uint16_t ent = table[peek];
                const int len = ent >> 8;
                CHECK(len >= 1 && len <= 12);
                CHECK(((ent & 0xFF) << 8 | lo[i]) == w[i]);
                pos += len;
            }
        }
    }
    return 0;
}

int main() {
    Rng rng(20261203);
    if (arena_fuzz(rng)) return 1;
    if (residency_fuzz(rng)) return 1;
    if (copy_plan_fuzz(rng)) return 1;
    if (planner_fuzz(rng)) return 1;
    if (codec_fuzz(rng)) return 1;
    printf("host sanitize: arena, residency, copy plans, planners, exponent codec clean\n");
    return 0;
}
