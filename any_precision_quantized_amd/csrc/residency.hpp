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

// The pager's pinned host copy, by promotion step and then expert: the block
// of step s = 3..6 of an expert holds what going to s bits adds (for s = 3,
// from no planes): the new planes of gate, up and down (planes 0..2 for s = 3,
// plane s-1 otherwise; each matrix's planes back to back), then the s-bit
// LUTs of gate, up and down.  Raising an expert by one step is then one
// contiguous range, and raising experts with adjacent indices to the same
// step is one range too.
inline int step_first_plane(int s) { return s == 3 ? 0 : s - 1; }
inline int step_planes(int s) { return s == 3 ? 3 : 1; }

template <class M>
uint64_t step_plane_bytes(const M* m3, int s) {
    return (uint64_t)step_planes(s) * (m3[0].slab + m3[1].slab + m3[2].slab);
}

template <class M>
uint64_t step_lut_bytes(const M* m3, int s) {
    return m3[0].lut_bytes[s - 3] + m3[1].lut_bytes[s - 3] + m3[2].lut_bytes[s - 3];
}

struct HostLayout {
    std::vector<uint64_t> step_off;   // [E][4]: where step s = 3..6 of expert e starts
    uint64_t bytes = 0;
};

// mats: 3 per expert (gate, up, down), as the pager holds them.
template <class M>
HostLayout host_layout(const std::vector<M>& mats) {
    HostLayout L;
    const size_t E = mats.size() / 3;
    L.step_off.resize(4 * E);
    for (int s = 3; s <= 6; ++s)
        for (size_t e = 0; e < E; ++e) {
            L.step_off[4 * e + s - 3] = L.bytes;
            L.bytes += step_plane_bytes(&mats[3 * e], s) + step_lut_bytes(&mats[3 * e], s);
        }
    return L;
}

// Offset in the host copy of plane p of matrix j (0 gate, 1 up, 2 down) of
// expert e, and of its b-bit LUT.
template <class M>
uint64_t host_plane_off(const std::vector<M>& mats, const HostLayout& L, size_t e, int j, int p) {
    const int s = p < 3 ? 3 : p + 1;
    uint64_t o = L.step_off[4 * e + s - 3];
    for (int i = 0; i < j; ++i) o += (uint64_t)step_planes(s) * mats[3 * e + i].slab;
    return o + (uint64_t)(p - step_first_plane(s)) * mats[3 * e + j].slab;
}

template <class M>
uint64_t host_lut_off(const std::vector<M>& mats, const HostLayout& L, size_t e, int j, int b) {
    uint64_t o = L.step_off[4 * e + b - 3] + step_plane_bytes(&mats[3 * e], b);
    for (int i = 0; i < j; ++i) o += mats[3 * e + i].lut_bytes[b - 3];
    return o;
}

struct Copy {
    uint64_t dst, src, bytes;
};

// The copies that make a claimed change resident.  h2d: src is an offset
// into the host copy, dst an arena offset; dev: copies within the arena.
// Staged (host to a staging block at staging_off, one range per run of
// contiguous step blocks, then placed device side): every h2d dst lies in the
// staging block, whose size is staged_bytes.  Direct: each matrix's planes of one
// step and each LUT go straight to their block.  Both move a relocated
// block's resident planes device side and copy the same host bytes: the new
// planes and the new LUT of every matrix, nothing more.  ok is false if the
// three matrices of an expert disagree on their bitwidths (they never do in
// the pager).  max_copy > 0 (a multiple of 256) splits every host-to-device
// range into pieces of at most that many bytes.
struct CopyPlan {
    std::vector<Copy> h2d, dev;
    uint64_t staged_bytes = 0;
    bool ok = true;
};

template <class M>
CopyPlan plan_copies(const std::vector<M>& mats, const HostLayout& L, bool staged, uint64_t staging_off,
                     uint64_t max_copy = 0) {
    CopyPlan P;
    const size_t E = mats.size() / 3;
    uint64_t cur = staging_off;
    for (size_t e = 0; e < E; ++e) {
        const M* m3 = &mats[3 * e];
        for (int j = 1; j < 3; ++j)
            if (m3[j].have != m3[0].have || m3[j].want != m3[0].want || m3[j].new_lut != m3[0].new_lut)
                P.ok = false;
        if (!P.ok) return P;
        for (int j = 0; j < 3; ++j)
            if (m3[j].moved && m3[j].have)
                P.dev.push_back(Copy{m3[j].planes_new.off, m3[j].planes.off, (uint64_t)m3[j].have * m3[j].slab});
        if (staged) continue;
        const int have = m3[0].have, want = m3[0].want;
        for (int s = have ? have + 1 : 3; s <= want; ++s)
            for (int j = 0; j < 3; ++j)
                P.h2d.push_back(Copy{m3[j].planes_new.off + (uint64_t)step_first_plane(s) * m3[j].slab,
                                     host_plane_off(mats, L, e, j, step_first_plane(s)),
                                     (uint64_t)step_planes(s) * m3[j].slab});
        if (m3[0].new_lut)
            for (int j = 0; j < 3; ++j)
                P.h2d.push_back(Copy{m3[j].lut_new.off, host_lut_off(mats, L, e, j, want), m3[j].lut_bytes[want - 3]});
    }
    // staged, in host-copy order (step, then expert), so adjacent blocks merge
    // into one range: the new planes of every step an expert climbs, and the
    // LUTs of the step it lands on (a demotion: those LUTs alone)
    for (int s = 3; staged && s <= 6; ++s)
        for (size_t e = 0; e < E; ++e) {
            const M* m3 = &mats[3 * e];
            const int have = m3[0].have, want = m3[0].want;
            const bool planes = want > have && s >= (have ? have + 1 : 3) && s <= want;
            const bool luts = m3[0].new_lut && s == want;
            if (!planes && !luts) continue;
            const uint64_t pb = step_plane_bytes(m3, s), lb = step_lut_bytes(m3, s);
            const uint64_t src = L.step_off[4 * e + s - 3] + (planes ? 0 : pb);
            const uint64_t n = (planes ? pb : 0) + (luts ? lb : 0);
            if (!P.h2d.empty() && P.h2d.back().src + P.h2d.back().bytes == src &&
                P.h2d.back().dst + P.h2d.back().bytes == cur)
                P.h2d.back().bytes += n;
            else
                P.h2d.push_back(Copy{cur, src, n});
            uint64_t o = cur;
            for (int j = 0; planes && j < 3; ++j) {
                const uint64_t nb = (uint64_t)step_planes(s) * m3[j].slab;
                P.dev.push_back(Copy{m3[j].planes_new.off + (uint64_t)step_first_plane(s) * m3[j].slab, o, nb});
                o += nb;
            }
            for (int j = 0; luts && j < 3; ++j) {
                P.dev.push_back(Copy{m3[j].lut_new.off, o, m3[j].lut_bytes[s - 3]});
                o += m3[j].lut_bytes[s - 3];
            }
            cur += n;
        }
    P.staged_bytes = cur - staging_off;
    if (max_copy) {
        std::vector<Copy> split;
        for (const Copy& c : P.h2d)
            for (uint64_t o = 0; o < c.bytes; o += max_copy)
                split.push_back(Copy{c.dst + o, c.src + o, std::min(max_copy, c.bytes - o)});
        P.h2d.swap(split);
    }
    return P;
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
