// Host-side residency bookkeeping of plane paging, plain C++ (no HIP): the
// first-fit arena over the device address range and the per-matrix claims a
// re-plan makes.  The pager (pager.hip) drives it and adds the copies and the
// stream-ordered commit; a host build with the address and undefined-behaviour
// sanitizers exercises it on the CPU.
//
// A matrix at b in {3..6} bits holds one block with planes 0..b-1 back to back
// at the packed slab stride (so the kernels' addressing is the same for paged
// and unpaged weights) and one block with its b-bit LUT.  Promotion grows the
// plane block in place when the bytes after it are free and otherwise moves
// it; demotion shortens it; the blocks a change retires return to the arena
// only after the commit has executed.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <iterator>
#include <map>
#include <vector>

namespace apmoe {

constexpr uint64_t kAlign = 256;

inline uint64_t align_up(uint64_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

}  // namespace apmoe

// Arena: free ranges of a [0, size) address range, kept coalesced.
struct apmoe_arena {
    uint64_t size = 0;
    std::map<uint64_t, uint64_t> free_;   // offset -> length, disjoint, never adjacent

    // First fit in offset order.
    bool alloc(uint64_t bytes, uint64_t* off) {
        bytes = apmoe::align_up(bytes);
        for (auto it = free_.begin(); it != free_.end(); ++it) {
            if (it->second < bytes) continue;
            *off = it->first;
            const uint64_t rest = it->second - bytes;
            const uint64_t at = it->first + bytes;
            free_.erase(it);
            if (rest) free_[at] = rest;
            return true;
        }
        return false;
    }

    // Claim exactly [off, off + bytes) if all of it is free.
    bool take(uint64_t off, uint64_t bytes) {
        bytes = apmoe::align_up(bytes);
        if (bytes == 0) return true;
        auto it = free_.upper_bound(off);
        if (it == free_.begin()) return false;
        --it;
        const uint64_t lo = it->first, hi = it->first + it->second;
        if (off < lo || off + bytes > hi) return false;
        free_.erase(it);
        if (off > lo) free_[lo] = off - lo;
        if (off + bytes < hi) free_[off + bytes] = hi - off - bytes;
        return true;
    }

    // Return [off, off + bytes); false (and no change) if any of it is
    // outside the arena or already free.
    bool release(uint64_t off, uint64_t bytes) {
        bytes = apmoe::align_up(bytes);
        if (bytes == 0) return true;
        if (off % apmoe::kAlign || off > size || bytes > size - off) return false;
        auto next = free_.lower_bound(off);
        if (next != free_.end() && next->first < off + bytes) return false;
        if (next != free_.begin()) {
            auto prev = std::prev(next);
            if (prev->first + prev->second > off) return false;
        }
        uint64_t lo = off, len = bytes;
        if (next != free_.begin()) {
            auto prev = std::prev(next);
            if (prev->first + prev->second == off) {
                lo = prev->first;
                len += prev->second;
                free_.erase(prev);
            }
        }
        next = free_.lower_bound(off);
        if (next != free_.end() && next->first == off + bytes) {
            len += next->second;
            free_.erase(next);
        }
        free_[lo] = len;
        return true;
    }

    void stats(uint64_t* free_bytes, uint64_t* largest, int* n) const {
        uint64_t f = 0, l = 0;
        for (const auto& r : free_) {
            f += r.second;
            l = std::max(l, r.second);
        }
        if (free_bytes) *free_bytes = f;
        if (largest) *largest = l;
        if (n) *n = (int)free_.size();
    }
};

namespace apmoe {

struct Block {
    uint64_t off = 0, len = 0;   // len 0: nothing held
};

// What residency bookkeeping needs of one paged matrix.
struct MatResidency {
    uint64_t slab = 0;            // bytes of one packed plane slab (a multiple of 256)
    uint64_t lut_bytes[4] = {};   // bytes of the b-bit LUT, b = 3..6
    Block planes, lut;            // resident now
    int have = 0, lut_b = 0;      // resident plane count; bitwidth of the resident LUT (0: none)
    Block planes_new, lut_new;    // after the staged change
    int want = 0;
    bool grown = false, moved = false, new_lut = false;   // what the staged change claimed
};

// Undo the claims of a stage that failed before any copy was enqueued.
template <class M>
void unstage(apmoe_arena& arena, std::vector<M>& mats) {
    for (MatResidency& m : mats) {
        if (m.moved) arena.release(m.planes_new.off, m.planes_new.len);
        if (m.grown) arena.release(m.planes.off + m.planes.len, m.planes_new.len - m.planes.len);
        if (m.new_lut) arena.release(m.lut_new.off, m.lut_new.len);
        m.planes_new = m.planes;
        m.lut_new = m.lut;
        m.want = m.have;
        m.grown = m.moved = m.new_lut = false;
    }
}

// Claim the blocks every matrix needs for its `want` planes; false when the
// arena cannot hold them (the claims made so far are flagged for unstage).
template <class M>
bool claim(apmoe_arena& arena, std::vector<M>& mats) {
    for (MatResidency& m : mats) {
        m.planes_new = m.planes;
        m.lut_new = m.lut;
        m.grown = m.moved = m.new_lut = false;
    }
    for (MatResidency& m : mats) {
        const uint64_t need = (uint64_t)m.want * m.slab;
        if (m.want > m.have) {
            // grow in place when the bytes after the block are free, else a new block
            if (m.have && arena.take(m.planes.off + m.planes.len, need - m.planes.len)) {
                m.planes_new = Block{m.planes.off, need};
                m.grown = true;
            } else {
                uint64_t off;
                if (!arena.alloc(need, &off)) return false;
                m.planes_new = Block{off, need};
                m.moved = true;
            }
        } else if (m.want < m.have) {
            m.planes_new = m.want ? Block{m.planes.off, need} : Block{};
        }
        if (m.want != m.lut_b) {
            m.lut_new = Block{};
            if (m.want) {
                uint64_t off;
                if (!arena.alloc(m.lut_bytes[m.want - 3], &off)) return false;
                m.lut_new = Block{off, align_up(m.lut_bytes[m.want - 3])};
                m.new_lut = true;
            }
        }
    }
    return true;
}

// The blocks a claimed change retires at its commit: the old plane block of a
// moved matrix, the tail of a shortened one, and every LUT that changes.
template <class M>
std::vector<Block> retired_blocks(const std::vector<M>& mats) {
    std::vector<Block> r;
    for (const MatResidency& m : mats) {
        if (m.want > m.have) {
            if (m.moved && m.planes.len) r.push_back(m.planes);
        } else if (m.want < m.have) {
            r.push_back(Block{m.planes.off + m.planes_new.len, m.planes.len - m.planes_new.len});
        }
        if (m.want != m.lut_b && m.lut.len) r.push_back(m.lut);
    }
    return r;
}

// The staged change becomes the resident state (at the commit).
template <class M>
void adopt(std::vector<M>& mats) {
    for (MatResidency& m : mats) {
        m.planes = m.planes_new;
        m.lut = m.lut_new;
        m.have = m.want;
        m.lut_b = m.want;
    }
}

}  // namespace apmoe
