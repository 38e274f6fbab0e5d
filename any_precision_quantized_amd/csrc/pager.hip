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
// The copies of one re-plan run on the copy engines (one hipMemcpyAsync per
// range on the copy stream), so no compute unit takes part: a gather kernel
// that read the pinned host copy over the bus was measured, and its
// long-latency reads slowed the layer running beside it by about 40%.
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
    hipEvent_t last_commit = nullptr;
    bool committed_once = false;
    char* host_buf = nullptr;        // pinned staging of the commit's patch list
    uint64_t n_copies = 0;           // ranges the last stage copied
    uint64_t dev_buf = 0;            // its device copy, carved from the arena
    size_t buf_bytes = 0;
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
    int rc = APMOE_OK;
    if (!pg->arena.alloc(pg->buf_bytes, &pg->dev_buf)) rc = APMOE_ENOSPACE;
    if (rc == APMOE_OK && hipHostMalloc(reinterpret_cast<void**>(&pg->host_buf), pg->buf_bytes, 0) != hipSuccess)
        rc = APMOE_EHIP;
    if (rc == APMOE_OK && (hipEventCreateWithFlags(&pg->copies_done, hipEventDisableTiming) != hipSuccess ||
                           hipEventCreateWithFlags(&pg->last_commit, hipEventDisableTiming) != hipSuccess))
        rc = APMOE_EHIP;
    if (rc != APMOE_OK) {
        if (pg->host_buf) (void)hipHostFree(pg->host_buf);
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
    // the patch staging is read by the previous commit's copy: wait for it
    if (pg->committed_once && hipEventSynchronize(pg->last_commit) != hipSuccess) return APMOE_EHIP;
    pg->reap(false);
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
    // enqueue the copies (device-to-device moves of blocks that cannot grow in
    // place, host-to-device planes and LUTs); record what the commit retires
    hipStream_t cs = as_stream(copy_stream);
    pg->h2d_bytes = pg->d2d_bytes = 0;
    pg->n_copies = 0;
    pg->retire_next.clear();
    bool ok = true;
    auto copy = [&](char* d, const char* s_, uint64_t n, hipMemcpyKind kind) {
        ok = ok && hipMemcpyAsync(d, s_, n, kind, cs) == hipSuccess;
        (kind == hipMemcpyHostToDevice ? pg->h2d_bytes : pg->d2d_bytes) += n;
        ++pg->n_copies;
    };
    for (PagedMat& m : pg->mats) {
        if (m.want > m.have) {
            char* d = pg->base + m.planes_new.off;
            if (m.moved && m.have) copy(d, pg->base + m.planes.off, (uint64_t)m.have * m.slab, hipMemcpyDeviceToDevice);
            const uint64_t o = (uint64_t)m.have * m.slab;
            copy(d + o, m.host_planes + o, (uint64_t)(m.want - m.have) * m.slab, hipMemcpyHostToDevice);
        }
        if (m.want != m.lut_b && m.new_lut)
            copy(pg->base + m.lut_new.off, m.host_lut[m.want - 3], m.lut_bytes[m.want - 3], hipMemcpyHostToDevice);
    }
    pg->retire_next = retired_blocks(pg->mats);
    if (ok) ok = hipEventRecord(pg->copies_done, cs) == hipSuccess;
    if (!ok) {
        (void)hipStreamSynchronize(cs);   // no copy may still land in a block unstage returns
        unstage(pg);
        return APMOE_EHIP;
    }
    // the patch list: every matrix's plane pointer and four LUT pointers, then the bits
    PatchHeader* h = reinterpret_cast<PatchHeader*>(pg->host_buf);
    Patch* p = reinterpret_cast<Patch*>(pg->host_buf + sizeof(PatchHeader));
    int n = 0;
    for (PagedMat& m : pg->mats) {
        p[n++] = Patch{m.desc + offsetof(apmoe_mat, planes) / 8,
                       m.want ? reinterpret_cast<uint64_t>(pg->base + m.planes_new.off) : 0};
        for (int b = 3; b <= 6; ++b)
            p[n++] = Patch{m.desc + offsetof(apmoe_mat, lut) / 8 + (b - 3),
                           m.want == b ? reinterpret_cast<uint64_t>(pg->base + m.lut_new.off) : 0};
    }
    h->n_patch = n;
    h->E = pg->E;
    int8_t* hb = reinterpret_cast<int8_t*>(p + n);
    for (int e = 0; e < pg->E; ++e) {
        hb[e] = bits_new[e];
        pg->bits_staged[e] = bits_new[e];
    }
    pg->staged = true;
    return APMOE_OK;
}

extern "C" int apmoe_pager_commit(apmoe_pager* pg, void* stream) {
    if (!pg || !pg->staged) return APMOE_EINVAL;
    hipStream_t s = as_stream(stream);
    if (hipStreamWaitEvent(s, pg->copies_done, 0) != hipSuccess) return APMOE_EHIP;
    const size_t n = sizeof(PatchHeader) +
                     (size_t)reinterpret_cast<PatchHeader*>(pg->host_buf)->n_patch * sizeof(Patch) + pg->E;
    char* dbuf = pg->base + pg->dev_buf;
    if (hipMemcpyAsync(dbuf, pg->host_buf, n, hipMemcpyHostToDevice, s) != hipSuccess) return APMOE_EHIP;
    clear_stale_error();
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
    if (pg->staged && hipEventSynchronize(pg->copies_done) != hipSuccess) rc = APMOE_EHIP;
    if (pg->committed_once && hipEventSynchronize(pg->last_commit) != hipSuccess) rc = APMOE_EHIP;
    pg->reap(true);
    (void)hipEventDestroy(pg->copies_done);
    (void)hipEventDestroy(pg->last_commit);
    (void)hipHostFree(pg->host_buf);
    delete pg;
    return rc;
}
