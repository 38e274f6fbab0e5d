// Plane paging: bit-planes and LUTs as the unit of residency.
//
// A b-bit expert needs only the top b bit-planes of each matrix and that
// matrix's b-bit LUT.  Demoting it to b' < b stops the kernels from reading
// planes b'..b-1 (the bits table says so) and returns their memory; promoting
// it copies planes b..b'-1 back from a host copy.  The copies run on a copy
// stream while the layer keeps computing at the old bitwidths; the new plane
// pointers, LUT pointers and bits take effect together at a safe boundary in
// the compute stream (a commit between two layer calls), and memory a commit
// retires is reused only after every kernel enqueued before it has finished.
//
// The host-to-device copies of one re-plan run on the copy engines (one
// hipMemcpyAsync per range on the copy stream): a gather kernel that read the
// pinned host copy over the bus was measured, and its long-latency reads
// slowed the layer running beside it by about 40%.  Each copy costs about
// 9 us beyond its bytes, so the pager keeps its own pinned host copy laid out
// by promotion step and then expert (residency.hpp): raising an expert by one
// step is one range, and so is raising experts with adjacent indices to the
// same step; the ranges are copied into a staging block of the arena.  The commit
// then places every staged plane and LUT (and moves the relocated blocks)
// with one short kernel on the compute stream, ahead of the pointer patch.
// The copy stream carries copies only, and stage records no event on it:
// streams share the few hardware queues, and a kernel or an event queued
// behind copies waits for them in its queue, holding up every stream that
// shares that queue (the layer was measured to stop for the whole copy
// window).  The commit records the event the compute stream waits for; by
// then the copies have normally finished.
// When the arena has no room for the staging block, each matrix's planes and
// LUT are copied straight into place.
//
// Device memory is one caller-owned arena carved by a host-side first-fit
// allocator (apmoe_arena_*).  A matrix's resident planes are one block holding
// planes 0..b-1 back to back at the packed slab stride, so the kernels'
// addressing (plane p at planes + p * slab) is the same for paged and unpaged
// weights.  Promotion grows a block in place when the bytes after it are free
// and otherwise moves it: planes 0..b-1 are copied device to device into the
// new block and the old block is retired at the commit.
#include <algorithm>
#include <cstddef>
#include <cstring>
#include <map>
#include <new>
#include <vector>

#include "common.hpp"
#include "residency.hpp"

using namespace apmoe;

// ---------------------------------------------------------------------------
// Pager
// ---------------------------------------------------------------------------

namespace apmoe {
namespace {

struct PagedMat : MatResidency {
    const char* host_planes = nullptr;
    const char* host_lut[4] = {};
    uint64_t* desc = nullptr;     // device address of this matrix's apmoe_mat
};

struct Patch {
    uint64_t* dst;
    uint64_t val;
};

// Device-side copies of a stage (arena offsets; sizes and offsets are
// multiples of 256 bytes): the staged ranges into their blocks and the
// resident planes of relocated blocks.  The list is cut into 64 KB chunks
// (first[i] is the first chunk of entry i, first[n] the total); each
// workgroup takes chunks in turn, finds a chunk's entry by binary search and
// copies it with 16-byte loads and stores, 16 per thread.
constexpr uint64_t kChunk = 65536;

__global__ __launch_bounds__(256) void pager_place_kernel(char* __restrict__ base, const Copy* __restrict__ cp,
                                                          const uint32_t* __restrict__ first, int n) {
    const uint32_t total = first[n];
    for (uint32_t c = blockIdx.x; c < total; c += gridDim.x) {
        int lo = 0, hi = n - 1;   // the entry with first[lo] <= c < first[lo + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (first[mid] <= c) lo = mid;
            else hi = mid - 1;
        }
        const Copy e = cp[lo];
        const uint64_t off = (uint64_t)(c - first[lo]) * kChunk;
        const uint64_t units = (e.bytes - off < kChunk ? e.bytes - off : kChunk) / 16;
        const uint4* src = reinterpret_cast<const uint4*>(base + e.src + off);
        uint4* dst = reinterpret_cast<uint4*>(base + e.dst + off);
        uint4 v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const uint64_t u = threadIdx.x + 256 * k;
            if (u < units) v[k] = src[u];
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const uint64_t u = threadIdx.x + 256 * k;
            if (u < units) dst[u] = v[k];
        }
    }
}

constexpr int kPlaceBlocks = 2048;

// Largest host-to-device copy (0: none).  Limits of 256 KB to 16 MB were
// measured: they slow the copies (to 19 GB/s at 256 KB) without lowering what
// the layer loses per step while copies run, so the total loss grows.
constexpr uint64_t kMaxCopy = 0;

// One patch list and the staged bits, laid out as the commit kernel reads them.
struct PatchHeader {
    int n_patch;
    int E;
};

__global__ void pager_commit_kernel(const char* __restrict__ buf, int8_t* __restrict__ bits) {
    const PatchHeader h = *reinterpret_cast<const PatchHeader*>(buf);
    const Patch* p = reinterpret_cast<const Patch*>(buf + sizeof(PatchHeader));
    const int8_t* b = reinterpret_cast<const int8_t*>(p + h.n_patch);
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < h.n_patch; i += gridDim.x * blockDim.x)
        *p[i].dst = p[i].val;
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < h.E; e += gridDim.x * blockDim.x) bits[e] = b[e];
}

inline int bits_planes(int b) { return b == 16 ? 0 : b; }

}  // namespace
}  // namespace apmoe

struct apmoe_pager {
    int E = 0;
    apmoe_arena arena;
    char* base = nullptr;            // device arena
    int8_t* bits_dev = nullptr;
    std::vector<PagedMat> mats;      // 3 per expert: gate, up, down
    std::vector<int8_t> bits_now, bits_staged;
    bool staged = false;
    hipEvent_t copies_done = nullptr;
    hipStream_t copy_stream = nullptr;   // of the staged change
    hipEvent_t last_commit = nullptr;
    bool committed_once = false;
    char* host_buf = nullptr;        // pinned staging of the commit's patch list
    uint64_t n_copies = 0;           // host-to-device ranges the last stage copied
    uint64_t dev_buf = 0;            // its device copy, carved from the arena
    size_t buf_bytes = 0;
    HostLayout layout;               // of host_copy
    char* host_copy = nullptr;       // pinned planes and LUTs by promotion step, then expert
    char* place_host = nullptr;      // pinned staging of the device-side copy list and its chunk starts
    uint64_t place_dev = 0;          // its device copy, carved from the arena
    size_t max_place = 0;            // entries it holds
    int n_place = 0;                 // entries the staged change's commit runs
    Block staging;                   // the staged change's staging block (len 0: none)
    struct Pending {
        hipEvent_t ev;
        std::vector<Block> blocks;
    };
    std::vector<Pending> pending;     // retired blocks, released once their event completes
    std::vector<Block> retire_next;   // blocks the staged change retires at its commit
    uint64_t h2d_bytes = 0, d2d_bytes = 0;   // copies enqueued by the last stage

    void reap(bool wait) {
        size_t keep = 0;
        for (size_t i = 0; i < pending.size(); ++i) {
            Pending& p = pending[i];
            const bool done = wait ? hipEventSynchronize(p.ev) == hipSuccess : hipEventQuery(p.ev) == hipSuccess;
            if (done) {
                for (const Block& b : p.blocks) arena.release(b.off, b.len);
                (void)hipEventDestroy(p.ev);
            } else {
                pending[keep++] = p;
            }
        }
        pending.resize(keep);
    }
};

namespace apmoe {
namespace {

void unstage(apmoe_pager* pg) {
    unstage(pg->arena, pg->mats);
    if (pg->staging.len) pg->arena.release(pg->staging.off, pg->staging.len);
    pg->staging = Block{};
    pg->retire_next.clear();
}

bool claim(apmoe_pager* pg) { return claim(pg->arena, pg->mats); }

}  // namespace
}  // namespace apmoe

extern "C" int apmoe_pager_create(int E, int H, int I, const void* const* host_planes,
                                  const void* const* host_luts, void* arena, uint64_t arena_bytes,
                                  apmoe_expert* experts, int8_t* bits, apmoe_pager** out) {
    if (!out) return APMOE_EINVAL;
    *out = nullptr;
    if (E < 1 || E > APMOE_MAX_EXPERTS || H <= 0 || I <= 0 || H % 32 || I % 32) return APMOE_EINVAL;
    if (!host_planes || !host_luts || !arena || !experts || !bits) return APMOE_EINVAL;
    if (reinterpret_cast<uintptr_t>(arena) % kAlign) return APMOE_EINVAL;
    for (int i = 0; i < 3 * E; ++i) {
        if (!host_planes[i]) return APMOE_EINVAL;
        for (int j = 0; j < 4; ++j)
            if (!host_luts[4 * i + j]) return APMOE_EINVAL;
    }
    apmoe_pager* pg = new (std::nothrow) apmoe_pager();
    if (!pg) return APMOE_ENOSPACE;
    pg->E = E;
    pg->arena.size = arena_bytes / kAlign * kAlign;
    if (pg->arena.size) pg->arena.free_[0] = pg->arena.size;
    pg->base = reinterpret_cast<char*>(arena);
    pg->bits_dev = bits;
    pg->mats.resize(3 * E);
    for (int e = 0; e < E; ++e) {
        apmoe_mat* dm[3] = {&experts[e].gate, &experts[e].up, &experts[e].down};
        for (int j = 0; j < 3; ++j) {
            PagedMat& m = pg->mats[3 * e + j];
            const int rows = j < 2 ? I : H, cols = j < 2 ? H : I;
            m.slab = (uint64_t)apmoe_packed_plane_words(rows, cols) / kPlanes * 4;
            for (int b = 3; b <= 6; ++b) {
                m.lut_bytes[b - 3] = (uint64_t)rows * (1u << b) * 2;
                m.host_lut[b - 3] = reinterpret_cast<const char*>(host_luts[4 * (3 * e + j) + b - 3]);
            }
            m.host_planes = reinterpret_cast<const char*>(host_planes[3 * e + j]);
            m.desc = reinterpret_cast<uint64_t*>(dm[j]);
        }
    }
    pg->bits_now.assign(E, 0);
    pg->bits_staged.assign(E, 0);
    pg->buf_bytes = sizeof(PatchHeader) + (size_t)3 * E * 5 * sizeof(Patch) + E;
    // per expert: up to four steps of three plane copies, three LUT copies, three moves
    pg->max_place = (size_t)18 * E;
    const size_t place_bytes = pg->max_place * sizeof(Copy) + (pg->max_place + 1) * sizeof(uint32_t);
    pg->layout = host_layout(pg->mats);
    int rc = APMOE_OK;
    if (!pg->arena.alloc(pg->buf_bytes, &pg->dev_buf) ||
        !pg->arena.alloc(place_bytes, &pg->place_dev))
        rc = APMOE_ENOSPACE;
    if (rc == APMOE_OK && (hipHostMalloc(reinterpret_cast<void**>(&pg->host_buf), pg->buf_bytes, 0) != hipSuccess ||
                           hipHostMalloc(reinterpret_cast<void**>(&pg->place_host), place_bytes, 0) != hipSuccess ||
                           hipHostMalloc(reinterpret_cast<void**>(&pg->host_copy), pg->layout.bytes, 0) != hipSuccess))
        rc = APMOE_EHIP;
    if (rc == APMOE_OK && (hipEventCreateWithFlags(&pg->copies_done, hipEventDisableTiming) != hipSuccess ||
                           hipEventCreateWithFlags(&pg->last_commit, hipEventDisableTiming) != hipSuccess))
        rc = APMOE_EHIP;
    if (rc == APMOE_OK) {
        // the caller's planes and LUTs, rearranged by step and expert
        for (int e = 0; e < E; ++e)
            for (int j = 0; j < 3; ++j) {
                const PagedMat& m = pg->mats[3 * e + j];
                for (int p = 0; p < kPlanes; ++p)
                    std::memcpy(pg->host_copy + host_plane_off(pg->mats, pg->layout, e, j, p),
                                m.host_planes + (uint64_t)p * m.slab, m.slab);
                for (int b = 3; b <= 6; ++b)
                    std::memcpy(pg->host_copy + host_lut_off(pg->mats, pg->layout, e, j, b), m.host_lut[b - 3],
                                m.lut_bytes[b - 3]);
            }
    }
    if (rc != APMOE_OK) {
        if (pg->host_buf) (void)hipHostFree(pg->host_buf);
        if (pg->place_host) (void)hipHostFree(pg->place_host);
        if (pg->host_copy) (void)hipHostFree(pg->host_copy);
        if (pg->copies_done) (void)hipEventDestroy(pg->copies_done);
        if (pg->last_commit) (void)hipEventDestroy(pg->last_commit);
        delete pg;
        return rc;
    }
    *out = pg;
    return APMOE_OK;
}

extern "C" int apmoe_pager_stage(apmoe_pager* pg, const int8_t* bits_new, void* copy_stream) {
    if (!pg || !bits_new) return APMOE_EINVAL;
    if (pg->staged) return APMOE_EINVAL;
    for (int e = 0; e < pg->E; ++e)
        if (!valid_bits(bits_new[e])) return APMOE_EBITS;
    // the patch and copy-list staging are read by copies the previous commit
    // waited for: wait for that commit
    if (pg->committed_once && hipEventSynchronize(pg->last_commit) != hipSuccess) return APMOE_EHIP;
    pg->reap(false);
    pg->staging = Block{};
    for (int e = 0; e < pg->E; ++e)
        for (int j = 0; j < 3; ++j) pg->mats[3 * e + j].want = bits_planes(bits_new[e]);
    if (!claim(pg)) {
        unstage(pg);
        pg->reap(true);   // retired blocks come back once their kernels have finished
        for (int e = 0; e < pg->E; ++e)
            for (int j = 0; j < 3; ++j) pg->mats[3 * e + j].want = bits_planes(bits_new[e]);
        if (!claim(pg)) {
            unstage(pg);
            return APMOE_ENOSPACE;
        }
    }
    // the copies: staged through one arena block when it fits, else straight
    // into place; record what the commit retires
    CopyPlan plan = plan_copies(pg->mats, pg->layout, true, 0);
    uint64_t soff = 0;
    if (plan.ok && plan.staged_bytes && pg->arena.alloc(plan.staged_bytes, &soff)) {
        pg->staging = Block{soff, align_up(plan.staged_bytes)};
        plan = plan_copies(pg->mats, pg->layout, true, soff, kMaxCopy);
    } else if (plan.ok) {
        plan = plan_copies(pg->mats, pg->layout, false, 0, kMaxCopy);
    }
    bool ok = plan.ok && plan.dev.size() <= pg->max_place;
    for (const Copy& c : plan.h2d)
        ok = ok && c.src <= pg->layout.bytes && c.bytes <= pg->layout.bytes - c.src && c.dst <= pg->arena.size &&
             c.bytes <= pg->arena.size - c.dst;
    for (const Copy& c : plan.dev)
        ok = ok && c.src % 16 == 0 && c.dst % 16 == 0 && c.bytes % 16 == 0 && c.src <= pg->arena.size &&
             c.bytes <= pg->arena.size - c.src && c.dst <= pg->arena.size && c.bytes <= pg->arena.size - c.dst;
    if (!ok) {   // a bookkeeping fault: nothing was enqueued
        unstage(pg);
        return APMOE_EINVAL;
    }
    hipStream_t cs = as_stream(copy_stream);
    pg->h2d_bytes = pg->d2d_bytes = 0;
    pg->n_copies = plan.h2d.size();
    pg->retire_next.clear();
    for (const Copy& c : plan.h2d) {
        ok = ok && hipMemcpyAsync(pg->base + c.dst, pg->host_copy + c.src, c.bytes, hipMemcpyHostToDevice, cs) ==
                       hipSuccess;
        pg->h2d_bytes += c.bytes;
    }
    for (const PagedMat& m : pg->mats)
        if (m.moved && m.have) pg->d2d_bytes += (uint64_t)m.have * m.slab;
    pg->n_place = (int)plan.dev.size();
    if (ok && pg->n_place) {   // the device-side copies and their chunk starts, run by the commit
        const size_t n = plan.dev.size();
        std::copy(plan.dev.begin(), plan.dev.end(), reinterpret_cast<Copy*>(pg->place_host));
        uint32_t* first = reinterpret_cast<uint32_t*>(pg->place_host + pg->max_place * sizeof(Copy));
        uint64_t chunks = 0;
        for (size_t i = 0; i < n; ++i) {
            first[i] = (uint32_t)chunks;
            chunks += (plan.dev[i].bytes + kChunk - 1) / kChunk;
        }
        first[n] = (uint32_t)chunks;
        ok = chunks < (1ull << 31) &&
             hipMemcpyAsync(pg->base + pg->place_dev, pg->place_host,
                            pg->max_place * sizeof(Copy) + (n + 1) * sizeof(uint32_t), hipMemcpyHostToDevice,
                            cs) == hipSuccess;
    }
    // the patch list (every matrix's plane pointer and four LUT pointers, then
    // the bits), copied behind the planes for the commit kernel
    PatchHeader* h = reinterpret_cast<PatchHeader*>(pg->host_buf);
    Patch* p = reinterpret_cast<Patch*>(pg->host_buf + sizeof(PatchHeader));
    int np = 0;
    for (PagedMat& m : pg->mats) {
        p[np++] = Patch{m.desc + offsetof(apmoe_mat, planes) / 8,
                        m.want ? reinterpret_cast<uint64_t>(pg->base + m.planes_new.off) : 0};
        for (int b = 3; b <= 6; ++b)
            p[np++] = Patch{m.desc + offsetof(apmoe_mat, lut) / 8 + (b - 3),
                            m.want == b ? reinterpret_cast<uint64_t>(pg->base + m.lut_new.off) : 0};
    }
    h->n_patch = np;
    h->E = pg->E;
    int8_t* hb = reinterpret_cast<int8_t*>(p + np);
    for (int e = 0; e < pg->E; ++e) hb[e] = bits_new[e];
    if (ok)
        ok = hipMemcpyAsync(pg->base + pg->dev_buf, pg->host_buf, sizeof(PatchHeader) + np * sizeof(Patch) + pg->E,
                            hipMemcpyHostToDevice, cs) == hipSuccess;
    pg->retire_next = retired_blocks(pg->mats);
    if (pg->staging.len) pg->retire_next.push_back(pg->staging);
    pg->copy_stream = cs;
    if (!ok) {
        (void)hipStreamSynchronize(cs);   // no copy may still land in a block unstage returns
        unstage(pg);
        return APMOE_EHIP;
    }
    for (int e = 0; e < pg->E; ++e) pg->bits_staged[e] = bits_new[e];
    pg->staged = true;
    return APMOE_OK;
}

extern "C" int apmoe_pager_commit(apmoe_pager* pg, void* stream) {
    if (!pg || !pg->staged) return APMOE_EINVAL;
    hipStream_t s = as_stream(stream);
    if (hipEventRecord(pg->copies_done, pg->copy_stream) != hipSuccess ||
        hipStreamWaitEvent(s, pg->copies_done, 0) != hipSuccess)
        return APMOE_EHIP;
    char* dbuf = pg->base + pg->dev_buf;
    clear_stale_error();
    if (pg->n_place) {
        const char* list = pg->base + pg->place_dev;
        hipLaunchKernelGGL(pager_place_kernel, dim3(kPlaceBlocks), dim3(256), 0, s, pg->base,
                           reinterpret_cast<const Copy*>(list),
                           reinterpret_cast<const uint32_t*>(list + pg->max_place * sizeof(Copy)), pg->n_place);
        const int rc = launch_status();
        if (rc != APMOE_OK) return rc;
    }
    hipLaunchKernelGGL(pager_commit_kernel, dim3(16), dim3(256), 0, s, dbuf, pg->bits_dev);
    int rc = launch_status();
    if (rc != APMOE_OK) return rc;
    if (hipEventRecord(pg->last_commit, s) != hipSuccess) return APMOE_EHIP;
    pg->committed_once = true;
    if (!pg->retire_next.empty()) {
        apmoe_pager::Pending p;
        if (hipEventCreateWithFlags(&p.ev, hipEventDisableTiming) != hipSuccess) return APMOE_EHIP;
        if (hipEventRecord(p.ev, s) != hipSuccess) return APMOE_EHIP;
        p.blocks.swap(pg->retire_next);
        pg->pending.push_back(std::move(p));
    }
    adopt(pg->mats);
    pg->staging = Block{};   // retired with the blocks above
    pg->bits_now = pg->bits_staged;
    pg->staged = false;
    return APMOE_OK;
}

extern "C" int apmoe_pager_stats(apmoe_pager* pg, uint64_t* resident_bytes, uint64_t* free_bytes,
                                 uint64_t* largest_free, uint64_t* h2d_bytes, uint64_t* d2d_bytes,
                                 uint64_t* copy_ranges) {
    if (!pg) return APMOE_EINVAL;
    pg->reap(false);
    uint64_t r = 0;
    for (const PagedMat& m : pg->mats) r += (uint64_t)m.have * m.slab + (m.lut_b ? m.lut_bytes[m.lut_b - 3] : 0);
    if (resident_bytes) *resident_bytes = r;
    pg->arena.stats(free_bytes, largest_free, nullptr);
    if (h2d_bytes) *h2d_bytes = pg->h2d_bytes;
    if (d2d_bytes) *d2d_bytes = pg->d2d_bytes;
    if (copy_ranges) *copy_ranges = pg->n_copies;
    return APMOE_OK;
}

extern "C" int apmoe_pager_destroy(apmoe_pager* pg) {
    if (!pg) return APMOE_OK;
    int rc = APMOE_OK;
    if (pg->staged && hipStreamSynchronize(pg->copy_stream) != hipSuccess) rc = APMOE_EHIP;
    if (pg->committed_once && hipEventSynchronize(pg->last_commit) != hipSuccess) rc = APMOE_EHIP;
    pg->reap(true);
    (void)hipEventDestroy(pg->copies_done);
    (void)hipEventDestroy(pg->last_commit);
    (void)hipHostFree(pg->host_buf);
    (void)hipHostFree(pg->place_host);
    (void)hipHostFree(pg->host_copy);
    delete pg;
    return rc;
}
