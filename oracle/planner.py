"""Oracle of the host bitwidth planner.

The quality-aware planner lowers the precision of the least sensitive experts
first, keeps key experts at full precision, never goes below an expert's
bitwidth floor, and only moves to more aggressive plans as memory pressure
rises ("内存的饥饿游戏", zhichai.net, sections "核心洞察：权重也能分页" and
"安全边界与异步搬运").  The second summary states the budget M_w = M_total -
M_kv, the integer program max sum_i I_i Q_i s.t. sum_i S(Q_i) <= M_w, and a
greedy approximation that keeps important experts at high precision until the
memory runs out ("动态量化优化MoE模型服务", time-frame.cloud, section
"方法与技术路线").

Reading taken here, which satisfies both descriptions: a demotion sequence.
Start every expert at its highest level; while the plan is over budget, lower
by one level the expert (not yet at its floor) whose next step costs the least
harm per byte saved, ties to the larger saving, then the lower index.  The
sequence does not depend on the budget, so plans are nested across budgets.
"""
from __future__ import annotations

import itertools

import numpy as np

OK = 0
ENOSPACE = -3
EINVAL = -1


def plan_bitwidths(levels, harm, nbytes, floor_bits, budget):
    """Return (status, bits[E]) for the demotion-sequence greedy.

    levels      bitwidths from high to low, e.g. [16, 6, 5, 4, 3]
    harm        [E][L] quality loss of running expert e at level l (>= 0)
    nbytes      [E][L] bytes of expert e at level l (strictly decreasing in l)
    floor_bits  [E] lowest bitwidth allowed per expert (must be one of levels)
    budget      bytes available to expert weights
    """
    levels = [int(v) for v in levels]
    E = len(floor_bits)
    L = len(levels)
    harm = [[float(harm[e][l]) for l in range(L)] for e in range(E)]
    nb = [[int(nbytes[e][l]) for l in range(L)] for e in range(E)]
    floor_lvl = []
    for e in range(E):
        if int(floor_bits[e]) not in levels:
            return EINVAL, None
        floor_lvl.append(levels.index(int(floor_bits[e])))
    for e in range(E):
        for l in range(L - 1):
            if not nb[e][l] > nb[e][l + 1]:
                return EINVAL, None

    lvl = [0] * E
    total = sum(nb[e][0] for e in range(E))
    while total > budget:
        best = None
        for e in range(E):
            l = lvl[e]
            if l >= floor_lvl[e]:
                continue
            saved = nb[e][l] - nb[e][l + 1]
            cost = (harm[e][l + 1] - harm[e][l]) / float(saved)
            key = (cost, -saved, e)
            if best is None or key < best[0]:
                best = (key, e)
        if best is None:
            return ENOSPACE, np.array([levels[floor_lvl[e]] for e in range(E)], dtype=np.int8)
        e = best[1]
        total -= nb[e][lvl[e]] - nb[e][lvl[e] + 1]
        lvl[e] += 1
    return OK, np.array([levels[lvl[e]] for e in range(E)], dtype=np.int8)


def plan_total(levels, nbytes, bits):
    levels = [int(v) for v in levels]
    return sum(int(nbytes[e][levels.index(int(b))]) for e, b in enumerate(bits))


def plan_harm(levels, harm, bits):
    levels = [int(v) for v in levels]
    return sum(float(harm[e][levels.index(int(b))]) for e, b in enumerate(bits))


def brute_force(levels, harm, nbytes, floor_bits, budget):
    """Exact minimum-harm plan within the budget by enumeration (tiny E only)."""
    levels = [int(v) for v in levels]
    E = len(floor_bits)
    choices = [range(0, levels.index(int(floor_bits[e])) + 1) for e in range(E)]
    best = None
    for assign in itertools.product(*choices):
        tot = sum(int(nbytes[e][l]) for e, l in enumerate(assign))
        if tot > budget:
            continue
        h = sum(float(harm[e][l]) for e, l in enumerate(assign))
        if best is None or h < best[0]:
            best = (h, assign)
    if best is None:
        return None, None
    return best[0], np.array([levels[l] for l in best[1]], dtype=np.int8)


def online_step(levels, harm, nbytes, floor_bits, stage_bits, m_total, m_kv, hysteresis, bits_now):
    """One step of the online planner under the KV budget.

    The planner page searches several bitwidth stages, starting from the
    safest demotion plan and moving to more aggressive ones only when pressure
    demands it, never below an expert's floor ("内存的饥饿游戏", zhichai.net,
    section "安全边界与异步搬运"); the second summary recomputes the weight
    budget M_w = M_total - M_kv as the KV cache grows ("动态量化优化MoE模型服务",
    time-frame.cloud, section "方法与技术路线").  Reading taken here:

    * stage_bits[s] (high to low) is the lowest bitwidth stage s may use: an
      expert's floor in stage s is the higher of its own floor and
      stage_bits[s]; the stage's plan for a budget is the demotion-sequence
      greedy under those floors;
    * the current plan is kept while it fits M_w with less than `hysteresis`
      bytes to spare; otherwise (over M_w, or hysteresis or more to spare) the
      plan is recomputed for M_w - hysteresis: the first stage whose plan fits
      that; if none does, the first stage whose plan fits M_w; if none does,
      every expert at its last-stage floor with status ENOSPACE.

    Returns (status, bits[E], stage, changed); stage is -1 when the plan is kept.
    """
    levels = [int(v) for v in levels]
    E = len(floor_bits)
    m_w = max(0, int(m_total) - int(m_kv))
    now = [int(b) for b in bits_now]
    used = plan_total(levels, nbytes, now)
    h = int(hysteresis)
    if used <= m_w and m_w - used < h:
        return OK, np.array(now, dtype=np.int8), -1, False
    target = max(0, m_w - h)

    def stage_floors(s):
        return np.array([max(int(floor_bits[e]), int(stage_bits[s])) for e in range(E)], dtype=np.int8)

    for budget in (target, m_w):
        for s in range(len(stage_bits)):
            st, bits = plan_bitwidths(levels, harm, nbytes, stage_floors(s), budget)
            if st == EINVAL:
                return EINVAL, None, -1, False
            if st == OK:
                return OK, bits, s, bits.tolist() != now
    last = stage_floors(len(stage_bits) - 1)
    return ENOSPACE, last, len(stage_bits) - 1, last.tolist() != now


def harm_multipliers(mass, wnorm):
    """Per-expert multipliers of the offline harm table from one router call's
    routing statistics, float64.

    The planner page ("内存的饥饿游戏…", zhichai.net, section "三层感知：离线 +
    路由 + 提示词") protects experts that receive more routing and corrects the
    offline sensitivity table with a residual taken from routing-weighted input
    norms; it gives no formula.  Read plainly:
        load[e]  = mass[e] / mean over experts of mass
        resid[e] = (wnorm[e] / mass[e]) / (sum of wnorm / sum of mass)
                   (1 for an expert with no routing mass)
        mult[e]  = load[e] * resid[e]
    and mult = 1 everywhere when nothing was routed.  Returns (mult, load, resid).
    """
    mass = [float(v) for v in mass]
    wnorm = [float(v) for v in wnorm]
    E = len(mass)
    tot_m = sum(mass)
    tot_n = sum(wnorm)
    if not (tot_m > 0 and tot_n > 0):
        return np.ones(E), np.ones(E), np.ones(E)
    mean_m = tot_m / E
    mean_norm = tot_n / tot_m
    load = np.array([m / mean_m for m in mass])
    resid = np.array([(n / m) / mean_norm if m > 0 else 1.0 for m, n in zip(mass, wnorm)])
    return load * resid, load, resid


def plan_routed(levels, harm, nbytes, floor_bits, budget, mass, wnorm):
    """The greedy plan over the offline harm table scaled per expert by the
    routing multipliers (harm'[e][l] = harm[e][l] * mult[e])."""
    mult, _, _ = harm_multipliers(mass, wnorm)
    scaled = np.asarray(harm, dtype=np.float64) * mult[:, None]
    return plan_bitwidths(levels, scaled, nbytes, floor_bits, budget)

