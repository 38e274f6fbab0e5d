// Greedy bitwidth planner (host only).
//
// Demotion sequence: start every expert at the highest level and, while the
// plan exceeds the budget, lower by one level the expert (not yet at its
// floor) whose next step costs the least harm per byte saved; ties go to the
// larger saving, then to the lower expert index.  This keeps key experts at
// full precision and demotes the least sensitive first, never below a floor,
// escalating only as far as the budget requires ("内存的饥饿游戏", zhichai.net,
// sections "核心洞察：权重也能分页" and "安全边界与异步搬运"); it is the greedy
// approximation of the budgeted selection problem max sum I_i Q_i subject to
// sum S(Q_i) <= M_w ("动态量化优化MoE模型服务", time-frame.cloud, section
// "方法与技术路线").  The order of demotions does not depend on the budget, so
// plans for smaller budgets only ever lower bitwidths further.
#include <stdint.h>

#include <vector>

#include "apmoe.h"

namespace {

bool valid_level(int b) { return (b >= 3 && b <= 6) || b == 16; }

}  // namespace

extern "C" int apmoe_plan_bitwidths(int E, int L, const int8_t* levels, const double* harm,
                                    const uint64_t* bytes, const int8_t* floor_bits, uint64_t budget,
                                    int8_t* bits_out) {
    if (E < 1 || E > APMOE_MAX_EXPERTS || L < 1 || L > 5) return APMOE_EINVAL;
    if (!levels || !harm || !bytes || !floor_bits || !bits_out) return APMOE_EINVAL;
    for (int l = 0; l < L; ++l) {
        if (!valid_level(levels[l])) return APMOE_EBITS;
        if (l > 0 && !(levels[l] < levels[l - 1])) return APMOE_EINVAL;
    }
    std::vector<int> floor_lvl(E), lvl(E, 0);
    for (int e = 0; e < E; ++e) {
        int f = -1;
        for (int l = 0; l < L; ++l)
            if (levels[l] == floor_bits[e]) f = l;
        if (f < 0) return APMOE_EINVAL;
        floor_lvl[e] = f;
        for (int l = 0; l + 1 < L; ++l)
            if (!(bytes[(size_t)e * L + l] > bytes[(size_t)e * L + l + 1])) return APMOE_EINVAL;
    }
    // 128-bit headroom is not needed: E * bytes fits in uint64 for any real model,
    // but guard the sum anyway.
    uint64_t total = 0;
    for (int e = 0; e < E; ++e) {
        uint64_t b = bytes[(size_t)e * L];
        if (total + b < total) return APMOE_EINVAL;
        total += b;
    }
    while (total > budget) {
        int best = -1;
        double best_cost = 0.0;
        uint64_t best_saved = 0;
        for (int e = 0; e < E; ++e) {
            const int l = lvl[e];
            if (l >= floor_lvl[e]) continue;
            const uint64_t saved = bytes[(size_t)e * L + l] - bytes[(size_t)e * L + l + 1];
            const double cost =
                (harm[(size_t)e * L + l + 1] - harm[(size_t)e * L + l]) / (double)saved;
            if (best < 0 || cost < best_cost || (cost == best_cost && saved > best_saved)) {
                best = e;
                best_cost = cost;
                best_saved = saved;
            }
        }
        if (best < 0) {
            for (int e = 0; e < E; ++e) bits_out[e] = levels[floor_lvl[e]];
            return APMOE_ENOSPACE;
        }
        total -= best_saved;
        lvl[best] += 1;
    }
    for (int e = 0; e < E; ++e) bits_out[e] = levels[lvl[e]];
    return APMOE_OK;
}
