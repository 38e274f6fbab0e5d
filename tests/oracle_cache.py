"""Memoised oracle results for the full-size parity tests.

Values are computed only by ``oracle`` on inputs from ``synth``; the cache
key hashes the source of both packages, the configuration, seed, bitwidths
and token subset, so any change to the oracle or the generator recomputes.
The cache lives in ``_cache/oracle`` (not committed).

    python -m tests.oracle_cache           # fill the cache for every workload
"""
from __future__ import annotations

import glob
import hashlib
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import moe, planner  # noqa: E402

CACHE = os.path.join(ROOT, "_cache", "oracle")
KEEP = ("ids", "gates", "logits", "counts", "offsets", "sorted_slots", "pos_of_slot", "out", "mag", "tokens")


def _src_hash() -> str:
    h = hashlib.sha1()
    for pat in ("oracle/*.py", "synth/*.py"):
        for f in sorted(glob.glob(os.path.join(ROOT, pat))):
            h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def resolve_bits(inp):
    """Bitwidths of a generated layer; planner-chosen ones come from the planner oracle."""
    if inp.bits is not None:
        return np.asarray(inp.bits, dtype=np.int8)
    pl = inp.plan
    st, bits = planner.plan_bitwidths(pl["levels"], pl["harm"], pl["bytes"], pl["floors"], pl["budget"])
    assert st == planner.OK
    return bits


def layer_ref(inp, bits, tokens=None):
    key_src = repr((_src_hash(), inp.cfg, inp.seed, np.asarray(bits).tolist(),
                    None if tokens is None else sorted(int(t) for t in tokens)))
    key = hashlib.sha1(key_src.encode()).hexdigest()[:20]
    path = os.path.join(CACHE, f"{inp.cfg.name}_{key}.npz")
    if os.path.exists(path):
        with np.load(path, allow_pickle=False) as z:
            return {k: z[k] for k in z.files}
    ref = moe.layer(inp, bits=bits, tokens=tokens)
    out = {k: np.asarray(ref[k]) for k in KEEP}
    os.makedirs(CACHE, exist_ok=True)
    tmp = path + ".tmp.npz"
    np.savez_compressed(tmp, **out)
    os.replace(tmp, path)
    return out


def fill_all():
    import time
    for name in synth.CONFIG_ORDER:
        cfg = synth.get(name)
        t = time.time()
        inp = synth.make_inputs(cfg, seed=0)
        bits = resolve_bits(inp)
        layer_ref(inp, bits)
        print(f"{name}: {time.time() - t:.1f}s", flush=True)


if __name__ == "__main__":
    fill_all()
