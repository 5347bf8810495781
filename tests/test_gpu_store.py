"""tq_store on the GPU against the oracle: FP8 keys, value scale and zero
bit-exact; Lloyd-Max key codes and uniform value codes bit-exact except next
to a decision boundary (|u - b| < 1e-6 for keys, |(v - z)/s - (k + 1/2)| <
1e-6 * (2^b - 1) for values; at most 1e-5 of the coordinates); stored key
norms within 1e-3 relative; bytes outside the addressed slots untouched."""

import numpy as np
import pytest

import gpu_case as G
import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


def _run_store(preset, N, Hk, bs, dtype, seed, skip_every=0, sentinel=0xA5, head_dim=128, block_layout="aos"):
    import torch
    import quantized_decode_attention_tq_amd as tq

    G.log(f"store preset={preset} N={N} Hk={Hk} bs={bs} dtype={dtype} seed={seed} D={head_dim} {block_layout}")
    K, V, slots, nb = W.store_inputs(num_tokens=N, num_kv_heads=Hk, block_size=bs, seed=seed, dtype=dtype,
                                     head_dim=head_dim)
    nb += 2  # spare blocks stay untouched
    if skip_every:
        slots[::skip_every] = -1
    lay = O.layout(preset, head_dim)
    lay_c = tq.layout_init(preset, head_dim, block_layout)
    signs = W.signs(seed, head_dim)
    c32, b32 = G.oracle_tables(lay)
    tab = G.gpu_tables(lay_c, signs)
    shape = (nb, bs, Hk, lay.slot_size_aligned)
    cache = torch.full(shape, sentinel, dtype=torch.uint8, device="cuda")
    tq.store(lay_c, G.dev16(K, dtype), G.dev16(V, dtype), torch.from_numpy(slots).cuda(), cache, tab.signs,
             tab.centroids, tab.boundaries)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    return lay, K, V, slots, got, signs, c32, b32, shape, sentinel


def check_store_parity(preset, dtype, N, Hk, bs, seed, skip_every, head_dim=128):
    """Store N tokens on the GPU and compare every slot with the oracle's."""
    lay, K, V, slots, got, signs, c32, b32, shape, sentinel = _run_store(preset, N, Hk, bs, dtype, seed,
                                                                         skip_every=skip_every, head_dim=head_dim)
    want = np.full(shape, sentinel, np.uint8)
    O.store_rows(lay, O.widen(K, dtype), O.widen(V, dtype), slots, want, signs, c32, b32)
    # untouched slots: identical sentinel bytes
    written = np.zeros(shape[:3], bool)
    keep = slots >= 0
    written[slots[keep] // shape[1], slots[keep] % shape[1]] = True
    np.testing.assert_array_equal(got[~written], want[~written])
    # written slots
    N, Hk = K.shape[:2]
    rows_got = got[slots[keep] // shape[1], slots[keep] % shape[1]].reshape(-1, lay.slot_size_aligned)
    rows_want = want[slots[keep] // shape[1], slots[keep] % shape[1]].reshape(-1, lay.slot_size_aligned)
    G.compare_slots(lay, rows_got, rows_want, O.widen(K[keep], dtype).reshape(-1, lay.head_dim), signs, c32, b32,
                    O.widen(V[keep], dtype).reshape(-1, lay.head_dim))


@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_store_parity_small(preset, dtype):
    check_store_parity(preset, dtype, 1237, 3, 16, 11, 13)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("preset", O.PRESETS)
def test_store_parity_full_sweep(preset):
    """The store sweep at full size (65536 tokens x 8 KV heads, bs 32, random
    slot mapping), as the benchmark launches it: every slot against the
    oracle's encoding of the same rows."""
    s = W.STORE_WORKLOAD
    lay, K, V, slots, got, signs, c32, b32, shape, _ = _run_store(preset, s["num_tokens"], s["num_kv_heads"],
                                                                 s["block_size"], s["dtype"], s["seed"])
    R = O.rotation(signs.astype(np.float64)) if O.needs_rotation(lay) else None
    rows = got[slots // shape[1], slots % shape[1]].reshape(-1, lay.slot_size_aligned)
    Kr = O.widen(K, s["dtype"]).reshape(-1, G.D)
    Vr = O.widen(V, s["dtype"]).reshape(-1, G.D)
    chunk = 65536
    want = np.concatenate([O.encode_slots(lay, Kr[i : i + chunk], Vr[i : i + chunk], R, c32, b32)
                           for i in range(0, Kr.shape[0], chunk)])
    n = G.compare_slots(lay, rows, want, Kr, signs, c32, b32, Vr)
    G.log(f"store sweep {preset}: {rows.shape[0]} slots, {n} codes differ at decision boundaries")


def test_store_edge_cases():
    import torch
    import quantized_decode_attention_tq_amd as tq

    lay_c = tq.layout_init("turboquant_3bit_nc")
    tab = G.gpu_tables(lay_c, W.signs(3))
    cache = torch.full((4, 16, 2, 102), 7, dtype=torch.uint8, device="cuda")
    k = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    G.log("store N=0")
    tq.store(lay_c, k, k, torch.zeros(0, dtype=torch.int64, device="cuda"), cache, tab.signs, tab.centroids,
             tab.boundaries)  # no-op
    G.log("store all slots negative")
    k = torch.randn((5, 2, 128), device="cuda").to(torch.bfloat16)
    tq.store(lay_c, k, k, torch.full((5,), -1, dtype=torch.int64, device="cuda"), cache, tab.signs, tab.centroids,
             tab.boundaries)
    torch.cuda.synchronize()
    assert torch.all(cache == 7)
    # zero key and constant value rows, fused-QKV style token stride
    qkv = torch.zeros((6, 8 * 128), dtype=torch.bfloat16, device="cuda")
    qkv[:, 2 * 128 : 4 * 128] = torch.randn((6, 256), device="cuda").to(torch.bfloat16)
    qkv[1, 2 * 128 : 3 * 128] = 0.0
    qkv[:, 4 * 128 : 6 * 128] = 2.5
    keys = qkv[:, 2 * 128 : 4 * 128]
    vals = qkv[:, 4 * 128 : 6 * 128]
    slots = torch.tensor([0, 5, 17, 33, 40, 63], dtype=torch.int64, device="cuda")
    G.log("store strided rows")
    tq.store(lay_c, keys, vals, slots, cache, tab.signs, tab.centroids, tab.boundaries)
    torch.cuda.synchronize()
    lay = O.layout("turboquant_3bit_nc", 128)
    c32, b32 = G.oracle_tables(lay)
    want = np.full((4, 16, 2, 102), 7, np.uint8)
    kb = keys.float().cpu().numpy().reshape(6, 2, 128).astype(np.float64)
    vb = vals.float().cpu().numpy().reshape(6, 2, 128).astype(np.float64)
    sl = slots.cpu().numpy()
    O.store_rows(lay, kb, vb, sl, want, W.signs(3), c32, b32)
    got = cache.cpu().numpy()
    written = np.zeros((4, 16, 2), bool)
    written[sl // 16, sl % 16] = True
    np.testing.assert_array_equal(got[~written], want[~written])
    G.compare_slots(lay, got[sl // 16, sl % 16].reshape(-1, 102), want[sl // 16, sl % 16].reshape(-1, 102),
                    kb.reshape(-1, 128), W.signs(3), c32, b32, vb.reshape(-1, 128))
