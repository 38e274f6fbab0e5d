// apmoe_arena_*: the host-side first-fit allocator of plane paging (C ABI).
#include <new>

#include "apmoe.h"
#include "residency.hpp"

using namespace apmoe;

extern "C" int apmoe_arena_create(uint64_t bytes, apmoe_arena** out) {
    if (!out) return APMOE_EINVAL;
    *out = nullptr;
    apmoe_arena* a = new (std::nothrow) apmoe_arena();
    if (!a) return APMOE_ENOSPACE;
    a->size = bytes / kAlign * kAlign;
    if (a->size) a->free_[0] = a->size;
    *out = a;
    return APMOE_OK;
}

extern "C" void apmoe_arena_destroy(apmoe_arena* a) { delete a; }

extern "C" int apmoe_arena_alloc(apmoe_arena* a, uint64_t bytes, uint64_t* off) {
    if (!a || !off || bytes == 0) return APMOE_EINVAL;
    return a->alloc(bytes, off) ? APMOE_OK : APMOE_ENOSPACE;
}

extern "C" int apmoe_arena_take(apmoe_arena* a, uint64_t off, uint64_t bytes) {
    if (!a || off % kAlign) return APMOE_EINVAL;
    return a->take(off, bytes) ? APMOE_OK : APMOE_ENOSPACE;
}

extern "C" int apmoe_arena_release(apmoe_arena* a, uint64_t off, uint64_t bytes) {
    if (!a) return APMOE_EINVAL;
    return a->release(off, bytes) ? APMOE_OK : APMOE_EINVAL;
}

extern "C" int apmoe_arena_stats(const apmoe_arena* a, uint64_t* free_bytes, uint64_t* largest, int* n_ranges) {
    if (!a) return APMOE_EINVAL;
    a->stats(free_bytes, largest, n_ranges);
    return APMOE_OK;
}
