"""GPU decode of the lossless exponent codec (apmoe_exp_decode): the decoded
fp16 weights equal the originals bit for bit, for the library's encoder and
for streams the oracle encoded, at small sizes with a partial last group and
at the full size of the Qwen-shaped shared expert and the Mixtral-shaped fp16
expert."""
import numpy as np
import pytest

import synth
from any_precision_quantized_amd import _lib
from oracle import expcodec as X

from . import gpu_helpers as G

pytestmark = pytest.mark.gpu


def _device(enc):
    import torch
    d = {k: torch.from_numpy(np.ascontiguousarray(enc[k]).view(v)).cuda()
         for k, v in (("words", np.int32), ("block_off", np.int32), ("lo", np.uint8), ("table", np.int16))}
    return d


def _decode(enc, n):
    import torch
    d = _device(enc)
    out = torch.full((n,), -1, dtype=torch.int16, device="cuda")
    _lib.exp_decode(d["words"], d["block_off"], d["lo"], d["table"], out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("n", [64, 64 * X.S, 64 * X.S * 3 + 64 * 17])
def test_decode_native_stream(n):
    G.say(f"exp decode n={n}")
    rng = np.random.default_rng(n + 1)
    w = rng.normal(0.0, 0.02, n).astype(np.float16).view(np.uint16)
    out = _decode(_lib.exp_encode(w), n)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w)


def test_decode_oracle_stream():
    n = 64 * X.S + 64 * 3
    rng = np.random.default_rng(3)
    w = rng.normal(0.0, 1.0, n).astype(np.float16).view(np.uint16)
    lengths, words, offs, lo = X.encode(w)
    enc = {"words": words, "block_off": offs, "lo": lo, "table": _lib.exp_encode(w)["table"]}
    out = _decode(enc, n)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w)


@pytest.mark.parametrize("name,which", [("qwen_decode", "shared"), ("mixtral_decode_t1", "expert0")])
def test_decode_full_size_fp16_weights(name, which):
    import torch
    cfg = synth.get(name)
    G.say(f"exp decode full size {name} {which}")
    inp = G.inputs(cfg)
    mats = inp.shared if which == "shared" else inp.experts[0]
    for mname in ("gate", "up", "down"):
        w = np.ascontiguousarray(mats[mname].w16).view(np.uint16).reshape(-1)
        enc = _lib.exp_encode(w)
        out = _decode(enc, w.size)
        ref = torch.from_numpy(w.view(np.int16)).cuda()
        assert torch.equal(out, ref), mname
        G.say(f"  {mname}: {w.size} weights, {enc['words'].size * 4 + w.size + enc['block_off'].size * 4} "
              f"bytes coded of {2 * w.size}")


def test_decode_batch_matches_each_matrix():
    """One launch over several coded matrices of different sizes, each with its
    own table (ragged last groups included), equals the weights bit for bit;
    the workgroups of one matrix never write another's output."""
    import torch
    G.say("exp decode batch")
    rng = np.random.default_rng(11)
    sizes = [64, 64 * X.S * 5 + 64 * 3, 64 * X.S, 64 * 77]
    ws, streams = [], []
    for i, n in enumerate(sizes):
        w = rng.normal(0.0, 0.02 * (i + 1), n).astype(np.float16).view(np.uint16)
        d = _device(_lib.exp_encode(w))
        d["out"] = torch.full((n,), -1, dtype=torch.int16, device="cuda")
        ws.append(w)
        streams.append(d)
    _lib.exp_decode_batch(streams)
    torch.cuda.synchronize()
    for w, d in zip(ws, streams):
        assert np.array_equal(d["out"].cpu().numpy().view(np.uint16), w)
