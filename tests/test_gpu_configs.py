"""The decode workloads at their own full-size inputs, in the benchmark's
launch configuration: every stored slot against the oracle's encoding of the
same rows (store bar: FP8 keys, scale and zero bit-exact; codes bit-exact
except next to a decision boundary, at most 1e-5 of the codes), then the
decode of whole sequences (every query head) against the oracle's exact
attention over the same cache bytes (5e-3 per row).

Workloads: tiny (4bit_nc, 256 tokens), llama8b (k8v4, 32 x 4096), qwen32b
(3bit_nc, 64 ragged sequences), longctx (k3v4_nc, 4 x 131072, 32 splits).
Each workload is generated and stored on the GPU once per module (the
largest holds ~2 GB of inputs); tests are split by sequence range so that
each finishes in well under a minute of host time.
"""

import numpy as np
import pytest

import gpu_case as G
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

SPLITS = {"tiny": 4, "llama8b": 8, "qwen32b": 8, "longctx": 32}
_STATE = {}


def _case(name):
    """(DecodeCase, device cache, host copy of the cache) of a workload,
    stored by the GPU; only the most recent workload is kept."""
    if name not in _STATE:
        import torch

        _STATE.clear()
        torch.cuda.empty_cache()
        w = W.WORKLOADS[name]
        G.log(f"[{name}] generating inputs")
        c = G.DecodeCase(w, need_oracle_cache=False)
        G.log(f"[{name}] GPU store of {int(c.lens.sum())} tokens x {w.num_kv_heads} heads")
        cache = c.gpu_store_all()
        torch.cuda.synchronize()
        _STATE[name] = (c, cache, cache.cpu().numpy())
    return _STATE[name]


def _chunks(name, n):
    B = W.WORKLOADS[name].batch
    step = -(-B // n)
    return [(name, i, min(i + step, B)) for i in range(0, B, step)]


def _store(name, b0, b1):
    """Every slot of sequences [b0, b1) (all KV heads) against the oracle's
    encoding of the same input rows."""
    c, _, got = _case(name)
    w = c.w
    bs = w.block_size
    R = O.rotation(c.signs.astype(np.float64)) if O.needs_rotation(c.lay) else None
    gots, wants, keys, vals = [], [], [], []
    for b in range(b0, b1):
        L = int(c.lens[b])
        if L == 0:
            continue
        slots = W.slot_mapping_for_sequence(w, b, c.table, c.lens)
        for hk in range(w.num_kv_heads):
            k = O.widen(c.K[b][:, hk], w.dtype)
            v = O.widen(c.V[b][:, hk], w.dtype)
            gots.append(got[slots // bs, slots % bs, hk])
            wants.append(O.encode_slots(c.lay, k, v, R, c.c32, c.b32))
            keys.append(k)
            vals.append(v)
    G.log(f"[{name}] sequences {b0}..{b1 - 1}: comparing {sum(len(x) for x in gots)} slots")
    n = G.compare_slots(c.lay, np.concatenate(gots), np.concatenate(wants), np.concatenate(keys), c.signs, c.c32,
                        c.b32, np.concatenate(vals))
    G.log(f"[{name}] sequences {b0}..{b1 - 1}: {n} codes differ at decision boundaries")


def _decode(name, b):
    """Every query head of sequence b, decoded by the GPU in the benchmark's
    launch configuration, against the oracle's attention over the same
    (GPU-stored) cache bytes."""
    c, cache, got = _case(name)
    S = SPLITS[name]
    key = ("decode", name, S)
    if key not in _STATE:
        G.log(f"[{name}] GPU decode, {S} splits")
        _STATE[key] = c.gpu_decode(cache, S)
    out, lse = _STATE[key]
    assert np.all(np.isfinite(out))
    rows = [(b, h) for h in range(c.w.num_q_heads)]
    G.log(f"[{name}] oracle decode of sequence {b} ({int(c.lens[b])} tokens, {len(rows)} query heads)")
    ref, rlse = c.oracle_decode(rows=rows, cache=got)
    worst = G.check_decode(out, lse, ref, rlse, rows)
    G.log(f"[{name}] sequence {b}: worst row error {worst:.2e}")


def _decode_seqs(name):
    w = W.WORKLOADS[name]
    lens = W.seq_lens(w)
    if name == "llama8b":
        return [0, w.batch - 1]
    if name == "qwen32b":
        return [int(np.argmax(lens)), int(np.argmin(lens))]
    return list(range(w.batch))


# per workload: its store chunks, then its whole-sequence decodes (one
# generation and GPU store per workload)
CASES = []
for _name, _n in (("tiny", 1), ("llama8b", 4), ("qwen32b", 8), ("longctx", 4)):
    CASES += [("store",) + ch for ch in _chunks(_name, _n)]
    CASES += [("decode", _name, b, b + 1) for b in _decode_seqs(_name)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,name,b0,b1", CASES)
def test_config_parity(kind, name, b0, b1):
    if kind == "store":
        _store(name, b0, b1)
    else:
        _decode(name, b0)
