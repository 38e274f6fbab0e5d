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

// One step of the online planner under the KV budget.  The weight budget is
// M_w = M_total - M_kv ("动态量化优化MoE模型服务", time-frame.cloud, section
// "方法与技术路线"); the search walks bitwidth stages from the safest to the most
// aggressive and stops at the first that fits, never below an expert's floor
// ("内存的饥饿游戏", zhichai.net, section "安全边界与异步搬运").  Stage s lets no
// expert below stage_bits[s] (nor below its own floor).  The current plan is
// kept while it fits M_w with less than `hysteresis` bytes to spare;
// otherwise the plan is recomputed for M_w - hysteresis, then for M_w.
extern "C" int apmoe_plan_online(int E, int L, const int8_t* levels, const double* harm, const uint64_t* bytes,
                                 const int8_t* floor_bits, int n_stages, const int8_t* stage_bits,
                                 uint64_t m_total, uint64_t m_kv, uint64_t hysteresis, const int8_t* bits_now,
                                 int8_t* bits_out, int* stage_out) {
    if (E < 1 || E > APMOE_MAX_EXPERTS || L < 1 || L > 5 || n_stages < 1 || n_stages > 5) return APMOE_EINVAL;
    if (!levels || !harm || !bytes || !floor_bits || !stage_bits || !bits_now || !bits_out || !stage_out)
        return APMOE_EINVAL;
    auto level_of = [&](int b) {
        for (int l = 0; l < L; ++l)
            if (levels[l] == b) return l;
        return -1;
    };
    for (int l = 0; l < L; ++l)
        if (!valid_level(levels[l])) return APMOE_EBITS;
    for (int s = 0; s < n_stages; ++s)
        if (level_of(stage_bits[s]) < 0) return APMOE_EINVAL;
    const uint64_t m_w = m_total > m_kv ? m_total - m_kv : 0;
    uint64_t used = 0;
    for (int e = 0; e < E; ++e) {
        const int l = level_of(bits_now[e]);
        if (l < 0) return APMOE_EINVAL;
        used += bytes[(size_t)e * L + l];
    }
    if (used <= m_w && m_w - used < hysteresis) {
        for (int e = 0; e < E; ++e) bits_out[e] = bits_now[e];
        *stage_out = -1;
        return APMOE_OK;
    }
    std::vector<int8_t> floors(E);
    auto stage_floors = [&](int s) {
        for (int e = 0; e < E; ++e) floors[e] = floor_bits[e] > stage_bits[s] ? floor_bits[e] : stage_bits[s];
    };
    const uint64_t target = m_w > hysteresis ? m_w - hysteresis : 0;
    for (uint64_t budget : {target, m_w}) {
        for (int s = 0; s < n_stages; ++s) {
            stage_floors(s);
            const int rc = apmoe_plan_bitwidths(E, L, levels, harm, bytes, floors.data(), budget, bits_out);
            if (rc == APMOE_OK) {
                *stage_out = s;
                return APMOE_OK;
            }
            if (rc != APMOE_ENOSPACE) return rc;
        }
    }
    stage_floors(n_stages - 1);
    for (int e = 0; e < E; ++e) bits_out[e] = floors[e];
    *stage_out = n_stages - 1;
    return APMOE_ENOSPACE;
}

// Harm multipliers from one router call's routing statistics.  The planner
// page ("内存的饥饿游戏", zhichai.net, section "三层感知：离线 + 路由 + 提示词")
// protects experts that receive more routing and corrects the offline
// sensitivity table with a residual from routing-weighted input norms; it
// gives no formula.  Read plainly: load = mass / mean(mass), residual = the
// mean input norm of the expert's slots against the mean over all slots (1 for
// an expert with no routing mass), multiplier = load * residual; 1 everywhere
// when nothing was routed.  Sums run in index order in double precision.
extern "C" int apmoe_harm_multipliers(int E, const float* mass, const float* wnorm, double* mult) {
    if (E < 1 || E > APMOE_MAX_EXPERTS || !mass || !wnorm || !mult) return APMOE_EINVAL;
    double tot_m = 0.0, tot_n = 0.0;
    for (int e = 0; e < E; ++e) {
        if (!(mass[e] >= 0.0f) || !(wnorm[e] >= 0.0f)) return APMOE_EINVAL;   // also rejects NaN
        tot_m += (double)mass[e];
        tot_n += (double)wnorm[e];
    }
    if (!(tot_m > 0.0 && tot_n > 0.0)) {
        for (int e = 0; e < E; ++e) mult[e] = 1.0;
        return APMOE_OK;
    }
    const double mean_m = tot_m / E, mean_norm = tot_n / tot_m;
    for (int e = 0; e < E; ++e) {
        const double m = (double)mass[e];
        const double load = m / mean_m;
        const double resid = m > 0.0 ? ((double)wnorm[e] / m) / mean_norm : 1.0;
        mult[e] = load * resid;
    }
    return APMOE_OK;
}

// The greedy plan over the offline harm table scaled per expert by the
// routing multipliers: harm'[e][l] = harm[e][l] * mult[e].
extern "C" int apmoe_plan_routed(int E, int L, const int8_t* levels, const double* harm, const uint64_t* bytes,
                                 const int8_t* floor_bits, uint64_t budget, const float* mass, const float* wnorm,
                                 int8_t* bits_out) {
    if (E < 1 || E > APMOE_MAX_EXPERTS || L < 1 || L > 5 || !harm) return APMOE_EINVAL;
    std::vector<double> mult(E), scaled((size_t)E * L);
    const int rc = apmoe_harm_multipliers(E, mass, wnorm, mult.data());
    if (rc != APMOE_OK) return rc;
    for (int e = 0; e < E; ++e)
        for (int l = 0; l < L; ++l) scaled[(size_t)e * L + l] = harm[(size_t)e * L + l] * mult[e];
    return apmoe_plan_bitwidths(E, L, levels, scaled.data(), bytes, floor_bits, budget, bits_out);
}
