"""Pins of the planner oracle: brute-force optimum of the budgeted selection
problem (time-frame.cloud page, section "方法与技术路线"), floors, nesting of
plans across budgets, and the Zipf-skewed 60-expert plan."""
import numpy as np
import pytest

import synth
from oracle import planner


def _instance(rng, E, levels):
    L = len(levels)
    nb = np.zeros((E, L), dtype=np.uint64)
    harm = np.zeros((E, L))
    for e in range(E):
        size = rng.integers(1000, 5000)
        nb[e] = [int(size * b / 16) + 17 for b in levels]
        inc = np.sort(rng.random(L))
        harm[e] = np.cumsum(inc) * rng.random()
        harm[e] -= harm[e][0]
    return harm, nb


@pytest.mark.parametrize("seed", range(12))
def test_greedy_feasible_and_never_beats_optimum(seed):
    rng = np.random.default_rng(seed)
    levels = [16, 6, 5, 4, 3] if seed % 2 else [6, 5, 4, 3]
    E = 4 + seed % 3
    harm, nb = _instance(rng, E, levels)
    floors = np.array([rng.choice(levels[1:]) for _ in range(E)], dtype=np.int8)
    lo = planner.plan_total(levels, nb, floors)
    hi = planner.plan_total(levels, nb, [levels[0]] * E)
    for budget in np.linspace(lo, hi, 7).astype(int):
        st, bits = planner.plan_bitwidths(levels, harm, nb, floors, budget)
        assert st == planner.OK
        assert planner.plan_total(levels, nb, bits) <= budget
        assert all(int(b) >= int(f) for b, f in zip(bits, floors))
        opt, _ = planner.brute_force(levels, harm, nb, floors, budget)
        h = planner.plan_harm(levels, harm, bits)
        assert h >= opt - 1e-12          # greedy is not claimed optimal; gap reported below
        print(f"seed {seed} budget {budget}: greedy harm {h:.6g} optimum {opt:.6g}")


def test_plans_nested_across_budgets():
    rng = np.random.default_rng(99)
    levels = [16, 6, 5, 4, 3]
    harm, nb = _instance(rng, 9, levels)
    floors = np.full(9, 3, dtype=np.int8)
    prev = None
    for budget in range(int(planner.plan_total(levels, nb, [16] * 9)), int(planner.plan_total(levels, nb, [3] * 9)) - 1, -997):
        st, bits = planner.plan_bitwidths(levels, harm, nb, floors, budget)
        assert st == planner.OK
        if prev is not None:
            assert np.all(bits <= prev)
        prev = bits


def test_infeasible_budget_returns_floors():
    levels = [6, 5, 4, 3]
    nb = np.array([[600, 500, 400, 300]] * 3, dtype=np.uint64)
    harm = np.array([[0, 1, 2, 3]] * 3, dtype=float)
    floors = np.array([4, 3, 5], dtype=np.int8)
    st, bits = planner.plan_bitwidths(levels, harm, nb, floors, 100)
    assert st == planner.ENOSPACE
    assert bits.tolist() == [4, 3, 5]


def test_tie_breaks():
    levels = [6, 5, 4, 3]
    # expert 1 saves more bytes per step at the same cost per byte -> demoted first
    nb = np.array([[60, 50, 40, 30], [120, 100, 80, 60], [60, 50, 40, 30]], dtype=np.uint64)
    harm = np.array([[0, 1, 2, 3], [0, 2, 4, 6], [0, 1, 2, 3]], dtype=float)
    floors = np.full(3, 3, dtype=np.int8)
    st, bits = planner.plan_bitwidths(levels, harm, nb, floors, 240 - 20)
    assert bits.tolist() == [6, 5, 6]
    st, bits = planner.plan_bitwidths(levels, harm, nb, floors, 240 - 30)
    assert bits.tolist() == [6, 4, 6]    # still the larger saving
    floors = np.array([3, 5, 3], dtype=np.int8)
    st, bits = planner.plan_bitwidths(levels, harm, nb, floors, 240 - 30)
    assert bits.tolist() == [5, 5, 6]    # expert 1 at its floor: lower index among equal keys


def test_invalid_inputs():
    levels = [6, 5, 4, 3]
    nb = np.array([[600, 600, 400, 300]], dtype=np.uint64)   # not strictly decreasing
    st, _ = planner.plan_bitwidths(levels, np.zeros((1, 4)), nb, np.array([3], np.int8), 10**6)
    assert st == planner.EINVAL
    nb = np.array([[600, 500, 400, 300]], dtype=np.uint64)
    st, _ = planner.plan_bitwidths(levels, np.zeros((1, 4)), nb, np.array([7], np.int8), 10**6)
    assert st == planner.EINVAL


def test_zipf_plan_keeps_hot_experts_high():
    cfg = synth.get("qwen_decode")
    p = synth.gen.zipf_prior(cfg.E, cfg.zipf_s)
    plan = synth.planner_inputs(cfg, p)
    st, bits = planner.plan_bitwidths(plan["levels"], plan["harm"], plan["bytes"], plan["floors"], plan["budget"])
    assert st == planner.OK
    assert planner.plan_total(plan["levels"], plan["bytes"], bits) <= plan["budget"]
    assert bits[0] == 6 and bits[-1] == 3
    assert np.all(np.diff(bits.astype(int)) <= 0)        # hotter experts never get fewer bits
    hist = {b: int((bits == b).sum()) for b in (6, 5, 4, 3)}
    print("qwen plan histogram", hist, "mean bits", bits.mean())
    assert all(v > 0 for v in hist.values())


# ---------------------------------------------------------------------------
# Routing statistics -> planner multipliers (host logic of the layer)
# ---------------------------------------------------------------------------

def test_harm_multipliers_hand_values():
    # equal input norms (2): the residual is 1 everywhere and the multiplier is
    # the expert's share of routing against an even 3/4 per expert
    mult, load, resid = planner.harm_multipliers([0.8, 0.8, 1.4, 0.0], [1.6, 1.6, 2.8, 0.0])
    np.testing.assert_allclose(load, [16 / 15, 16 / 15, 28 / 15, 0.0], rtol=1e-15)
    np.testing.assert_allclose(resid, [1.0, 1.0, 1.0, 1.0], rtol=1e-15)
    np.testing.assert_allclose(mult, load, rtol=1e-15)
    # equal routing, inputs of norm 1 and 3: residuals 1/2 and 3/2 of the mean 2
    mult, load, resid = planner.harm_multipliers([1.0, 1.0], [1.0, 3.0])
    assert load.tolist() == [1.0, 1.0] and resid.tolist() == [0.5, 1.5] and mult.tolist() == [0.5, 1.5]
    # nothing routed: the offline table stands
    mult, _, _ = planner.harm_multipliers([0.0, 0.0, 0.0], [0.0, 0.0, 0.0])
    assert mult.tolist() == [1.0, 1.0, 1.0]


def test_native_harm_multipliers_match_oracle():
    """apmoe_harm_multipliers through the C ABI: the hand values exactly, and the
    oracle bit for bit on routing statistics of random routings (same formula,
    sums in the same index order, float64)."""
    from any_precision_quantized_amd import _lib
    assert _lib.harm_multipliers([1.0, 1.0], [1.0, 3.0]).tolist() == [0.5, 1.5]
    assert _lib.harm_multipliers([0.0, 0.0, 0.0], [0.0, 0.0, 0.0]).tolist() == [1.0, 1.0, 1.0]
    # inputs rounded to fp32 as the device hands them over (0.8 is not exact)
    np.testing.assert_allclose(_lib.harm_multipliers([0.8, 0.8, 1.4, 0.0], [1.6, 1.6, 2.8, 0.0]),
                               [16 / 15, 16 / 15, 28 / 15, 0.0], rtol=1e-7)
    from oracle import moe
    rng = np.random.default_rng(7)
    for trial in range(10):
        T, E, k, H = int(rng.integers(1, 40)), int(rng.integers(2, 70)), 2, 64
        x = rng.normal(size=(T, H)).astype(np.float16)
        w = rng.normal(0, 0.02, size=(E, H)).astype(np.float32)
        ids, gates, _ = moe.route(x, w, None, 1.0, k)
        mass, wnorm = moe.route_stats(x, ids, gates, E)
        mass, wnorm = mass.astype(np.float32), wnorm.astype(np.float32)   # what the device hands over
        ref, _, _ = planner.harm_multipliers(mass, wnorm)
        assert np.array_equal(_lib.harm_multipliers(mass, wnorm), ref)
    for bad in (([1.0, -1.0], [1.0, 1.0]), ([1.0, float("nan")], [1.0, 1.0])):
        with pytest.raises(_lib.ApmoeError):
            _lib.harm_multipliers(*bad)


def test_routed_plan_demotes_idle_experts_first():
    """The routed plan (offline harm scaled by the routing multipliers): with
    the same offline table for every expert, the expert nobody routes to goes
    first, to its floor; native and oracle agree."""
    from any_precision_quantized_amd import _lib
    levels = np.array([6, 5, 4, 3], np.int8)
    E = 4
    harm = np.tile(np.array([0.0, 2.0 ** -5, 2.0 ** -4, 2.0 ** -3]), (E, 1))   # the same offline table
    nbytes = np.tile(np.array([600, 500, 400, 300], np.uint64), (E, 1))
    floors = np.full(E, 3, np.int8)
    mass, wnorm = [1.5, 0.0, 1.0, 1.5], [3.0, 0.0, 2.0, 3.0]
    budget = 4 * 600 - 300          # room for one expert at 3 bits
    st, bits = _lib.plan_routed(levels, harm, nbytes, floors, budget, mass, wnorm)
    assert st == _lib.OK
    assert bits.tolist() == [6, 3, 6, 6]
    st, ref = planner.plan_routed(levels, harm, nbytes, floors, budget, mass, wnorm)
    assert st == planner.OK and ref.tolist() == bits.tolist()


def test_native_routed_plan_matches_oracle():
    from any_precision_quantized_amd import _lib
    rng = np.random.default_rng(11)
    levels = [6, 5, 4, 3]
    for trial in range(20):
        E = int(rng.integers(1, 60))
        size = rng.integers(1000, 10**7, size=E)
        nb = np.array([[int(sz * b / 16) + 31 for b in levels] for sz in size], dtype=np.uint64)
        harm = np.cumsum(rng.random((E, 4)), axis=1)
        harm -= harm[:, :1]
        floors = np.full(E, 3, np.int8)
        mass = (rng.random(E) * (rng.random(E) > 0.3)).astype(np.float32)
        wnorm = (mass * rng.uniform(20, 60, size=E)).astype(np.float32)
        lo = planner.plan_total(levels, nb, floors)
        hi = planner.plan_total(levels, nb, [6] * E)
        for budget in np.linspace(lo, hi, 5).astype(np.int64):
            st_ref, ref = planner.plan_routed(levels, harm, nb, floors, int(budget), mass, wnorm)
            st, bits = _lib.plan_routed(levels, harm, nb, floors, int(budget), mass, wnorm)
            assert st == st_ref and np.array_equal(bits, ref)


# ---------------------------------------------------------------------------
# Online planner under the KV budget (oracle pins)
# ---------------------------------------------------------------------------

def _online_case():
    levels = [6, 5, 4, 3]
    harm = np.array([[0.0, 1.0, 3.0, 7.0],       # expert 0: sensitive
                     [0.0, 0.1, 0.3, 0.7],       # expert 1: tolerant
                     [0.0, 0.5, 1.5, 3.5]])
    nbytes = np.array([[600, 500, 400, 300]] * 3, dtype=np.uint64)
    floors = np.array([4, 3, 3], np.int8)
    stages = [5, 4, 3]
    return levels, harm, nbytes, floors, stages


def test_online_ample_budget_keeps_full_precision():
    levels, harm, nbytes, floors, stages = _online_case()
    st, bits, stage, changed = planner.online_step(levels, harm, nbytes, floors, stages, 10_000, 0, 100,
                                                   [3, 3, 3])
    assert st == planner.OK and bits.tolist() == [6, 6, 6] and stage == 0 and changed


def test_online_stages_escalate_only_under_pressure():
    levels, harm, nbytes, floors, stages = _online_case()
    # 1500 of 1800 bytes: three 100-byte demotions; stage 0 (nobody below 5)
    # allows exactly one per expert
    st, bits, stage, _ = planner.online_step(levels, harm, nbytes, floors, stages, 1500, 0, 0, [6, 6, 6])
    assert st == planner.OK and stage == 0 and bits.tolist() == [5, 5, 5]
    # 1600 bytes: two demotions, the tolerant expert then the middle one
    st, bits, stage, _ = planner.online_step(levels, harm, nbytes, floors, stages, 1600, 0, 0, [6, 6, 6])
    assert st == planner.OK and stage == 0 and bits.tolist() == [6, 5, 5]
    # 1300 bytes: stage 0 bottoms out at 1500, stage 1 (down to 4 bits) fits
    st, bits, stage, _ = planner.online_step(levels, harm, nbytes, floors, stages, 1300, 0, 0, [5, 5, 5])
    assert st == planner.OK and stage == 1
    assert planner.plan_total(levels, nbytes, bits) <= 1300 and min(bits) >= 4
    # 1000 bytes: only stage 2 fits; the sensitive expert keeps its own floor of 4
    st, bits, stage, _ = planner.online_step(levels, harm, nbytes, floors, stages, 1000, 0, 0, [6, 6, 6])
    assert st == planner.OK and stage == 2 and bits[0] >= 4
    assert planner.plan_total(levels, nbytes, bits) <= 1000
    # below every floor: floors of the last stage, ENOSPACE
    st, bits, stage, _ = planner.online_step(levels, harm, nbytes, floors, stages, 900, 0, 0, [6, 6, 6])
    assert st == planner.ENOSPACE and bits.tolist() == [4, 3, 3] and stage == 2


def test_online_budget_is_total_minus_kv_and_hysteresis_band_keeps_the_plan():
    levels, harm, nbytes, floors, stages = _online_case()
    # M_w = 2000 - 400 = 1600 with hysteresis 100: replanned for 1500
    st, bits, stage, changed = planner.online_step(levels, harm, nbytes, floors, stages, 2000, 400, 100,
                                                   [6, 6, 6])
    assert st == planner.OK and changed and planner.plan_total(levels, nbytes, bits) <= 1500
    # KV grows by 50: the plan (1500 bytes) still fits 1550 with less than 100 spare -> kept
    st2, bits2, stage2, changed2 = planner.online_step(levels, harm, nbytes, floors, stages, 2000, 450, 100, bits)
    assert st2 == planner.OK and stage2 == -1 and not changed2 and bits2.tolist() == bits.tolist()
    # KV shrinks back to 300: 200 spare >= 100 -> replanned for 1600, a promotion
    st3, bits3, stage3, changed3 = planner.online_step(levels, harm, nbytes, floors, stages, 2000, 300, 100, bits)
    assert st3 == planner.OK and changed3 and planner.plan_total(levels, nbytes, bits3) <= 1600
    assert planner.plan_total(levels, nbytes, bits3) > planner.plan_total(levels, nbytes, bits)
    assert all(int(a) >= int(b) for a, b in zip(bits3, bits))


def test_online_first_feasible_stage_is_chosen():
    rng = np.random.default_rng(5)
    levels = [6, 5, 4, 3]
    stages = [5, 4, 3]
    for _ in range(50):
        E = int(rng.integers(2, 6))
        harm = np.cumsum(rng.uniform(0, 1, size=(E, 4)), axis=1) - rng.uniform(0, 1, size=(E, 1))
        harm[:, 0] = 0.0
        harm = np.maximum.accumulate(np.abs(harm), axis=1)
        nbytes = np.array([[600, 500, 400, 300]] * E, dtype=np.uint64)
        floors = rng.choice([3, 4], size=E).astype(np.int8)
        budget = int(rng.integers(300 * E, 600 * E + 1))
        st, bits, stage, _ = planner.online_step(levels, harm, nbytes, floors, stages, budget, 0, 0, [6] * E)
        fits = []
        for s, sb in enumerate(stages):
            f = np.maximum(floors, sb).astype(np.int8)
            fits.append(planner.plan_bitwidths(levels, harm, nbytes, f, budget)[0] == planner.OK)
        if any(fits):
            assert st == planner.OK and stage == fits.index(True)
            assert planner.plan_total(levels, nbytes, bits) <= budget
        else:
            assert st == planner.ENOSPACE


def test_native_online_step_matches_oracle():
    """apmoe_plan_online against the oracle step, bit-exact, over random
    scenarios including a KV budget that grows and shrinks across steps."""
    from any_precision_quantized_amd import _lib
    rng = np.random.default_rng(21)
    levels = np.array([6, 5, 4, 3], np.int8)
    for trial in range(40):
        E = int(rng.integers(1, 9))
        harm = np.sort(rng.uniform(0, 1, size=(E, 4)), axis=1)
        harm[:, 0] = 0.0
        nbytes = np.sort(rng.integers(100, 1000, size=(E, 4)), axis=1)[:, ::-1].astype(np.uint64)
        nbytes[:, 1:] = np.minimum(nbytes[:, 1:], nbytes[:, :-1] - 1)
        floors = rng.choice([3, 4, 5], size=E).astype(np.int8)
        stages = np.array([5, 4, 3], np.int8) if trial % 2 else np.array([4, 3], np.int8)
        m_total = int(nbytes[:, 0].sum())
        hyst = int(rng.integers(0, 200))
        now = np.full(E, 6, np.int8)
        for m_kv in np.concatenate([np.linspace(0, m_total, 7), np.linspace(m_total, 0, 7)]).astype(np.int64):
            st, bits, stage = _lib.plan_online(levels, harm, nbytes, floors, stages, m_total, int(m_kv), hyst, now)
            rst, rbits, rstage, _ = planner.online_step(levels, harm, nbytes, floors, stages, m_total, int(m_kv),
                                                       hyst, now)
            assert st == rst and stage == rstage, (trial, m_kv)
            assert bits.tolist() == rbits.tolist(), (trial, m_kv)
            now = bits
