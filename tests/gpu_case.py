"""Shared set-up of the GPU parity tests: seeded inputs from workloads.py,
the oracle's result on them, and the HIP library's result on the same
bytes, plus the comparison rules (spec tolerances)."""

from __future__ import annotations

import math
import sys

import numpy as np

import oracle as O
import workloads as W

D = 128
DECODE_RTOL = 5e-3  # max_i |o - o_ref| / max_i |o_ref| per (sequence, query head)
LSE_ATOL = 5e-3
GAMMA_RTOL = 1e-3
BOUNDARY_EPS = 1e-6
MISMATCH_FRAC = 1e-5


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch():
    import torch as t

    return t


def dev16(bits: np.ndarray, dtype: str):
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return x.view(t.bfloat16 if dtype == "bf16" else t.float16)


def oracle_tables(lay):
    if lay.key_fp8:
        return None, None
    return O.codebook_tables(lay.head_dim, lay.key_bits)


def gpu_tables(lay_c, signs):
    import quantized_decode_attention_tq_amd as tq

    return tq.Tables(lay_c, signs)


# ------------------------------------------------------------------ store


def _compare_codes(lay, bits, got, want, rows, R, cent, bound, nc, min_allowed=0, n_total=None):
    """got/want: (rows, code bytes + 2) = packed Lloyd-Max codes then the
    fp16 norm of the same rows; rows: (rows, D) float64 inputs.  A code may
    differ only next to a bucket boundary (|u - b| < 1e-6, by one), at most
    1e-5 of the codes (or min_allowed of them, for samples too small for that
    rate); the norm within 1e-3, re-derived from the GPU's codes where they
    differ.  Returns the number of differing codes."""
    nb = got.shape[1] - 2
    cg = O.unpack_lsb(got[:, :nb], bits, lay.head_dim)
    cw = O.unpack_lsb(want[:, :nb], bits, lay.head_dim)
    bad = np.argwhere(cg != cw)
    if len(bad):
        U = O.key_units(lay, rows[np.unique(bad[:, 0])], R)
        row_idx = {r: i for i, r in enumerate(np.unique(bad[:, 0]))}
        u = np.array([U[row_idx[r], j] for r, j in bad])
        dist = np.min(np.abs(u[:, None] - np.asarray(bound, np.float64)[None, :]), axis=1)
        assert np.all(dist < BOUNDARY_EPS), f"code mismatch away from a boundary: {dist.max()}"
        assert np.all(np.abs(cg[bad[:, 0], bad[:, 1]] - cw[bad[:, 0], bad[:, 1]]) == 1)
    n_total = cg.size if n_total is None else n_total
    assert len(bad) <= max(MISMATCH_FRAC * n_total, min_allowed), f"{len(bad)} code mismatches of {n_total}"
    gg = got[:, nb : nb + 2].copy().view(np.float16).astype(np.float64)[:, 0]
    gw = want[:, nb : nb + 2].copy().view(np.float16).astype(np.float64)[:, 0]
    for r in np.unique(bad[:, 0]) if len(bad) else []:
        nu = np.sqrt(np.sum(rows[r] ** 2))
        chat = np.asarray(cent, np.float64)[cg[r]]
        gw[r] = float(np.float16(nu / np.sqrt(np.sum(chat ** 2)))) if nc else nu
    np.testing.assert_allclose(gg, gw, rtol=GAMMA_RTOL, atol=0)
    return len(bad)


def _compare_value_codes(lay, got, want, values, min_allowed=0, n_total=None):
    """got/want: (rows, value data + 4) = packed uniform value codes, fp16
    scale, fp16 zero of the same rows; values: (rows, D) float64 inputs.
    Scale and zero are bit-exact.  A code may differ from the oracle's exact
    floor((v - z) / s + 1/2) only by one, where that quotient is within
    1e-6 * (2^b - 1) of a half-integer (the kernel decides in fp32), at most
    1e-5 of the codes (or min_allowed).  Returns the number of differing
    codes."""
    vd, vb = lay.value_data_bytes, lay.value_bits
    np.testing.assert_array_equal(got[:, vd:], want[:, vd:])
    cg = O.unpack_lsb(got[:, :vd], vb, lay.head_dim)
    cw = O.unpack_lsb(want[:, :vd], vb, lay.head_dim)
    bad = np.argwhere(cg != cw)
    if len(bad):
        s = want[:, vd : vd + 2].copy().view(np.float16).astype(np.float64)[:, 0]
        z = want[:, vd + 2 : vd + 4].copy().view(np.float16).astype(np.float64)[:, 0]
        r, c = bad[:, 0], bad[:, 1]
        x = (values[r, c] - z[r]) / s[r]
        dist = np.abs(x - (np.floor(x) + 0.5))
        assert np.all(dist < BOUNDARY_EPS * ((1 << vb) - 1)), f"value code mismatch away from a tie: {dist.max()}"
        assert np.all(np.abs(cg[r, c] - cw[r, c]) == 1)
    n_total = cg.size if n_total is None else n_total
    assert len(bad) <= max(MISMATCH_FRAC * n_total, min_allowed), f"{len(bad)} value code mismatches of {n_total}"
    return len(bad)


def compare_slots(lay, got: np.ndarray, want: np.ndarray, keys, signs, c32, b32, values, min_allowed=0):
    """got/want: (rows, slot) bytes of the same rows; keys / values: (rows, D)
    float64 inputs of those rows.  Lloyd-Max codes (MSE keys, Lloyd-Max
    values) follow _compare_codes, uniform value codes _compare_value_codes;
    FP8 keys, value scale and zero and padding are bit-exact.  Only rows
    whose bytes differ are decoded; the mismatch cap counts all rows' codes.
    Returns the number of code mismatches."""
    assert got.shape == want.shape
    diff = np.nonzero(np.any(got != want, axis=1))[0]
    if len(diff) == 0:
        return 0
    n_total = got.shape[0] * lay.head_dim
    got, want, keys, values = got[diff], want[diff], keys[diff], values[diff]
    R = O.rotation(np.asarray(signs, np.float64)) if O.needs_rotation(lay) else None
    kd, vo, vd = lay.key_data_bytes, lay.key_packed_size, lay.value_data_bytes
    n = 0
    if lay.key_fp8:
        np.testing.assert_array_equal(got[:, :kd], want[:, :kd])
    else:
        n += _compare_codes(lay, lay.key_bits, got[:, : kd + 2], want[:, : kd + 2], keys, R, c32, b32,
                            lay.norm_correction, min_allowed, n_total)
    if lay.value_lm:
        vc32, vb32 = O.value_tables(lay)
        n += _compare_codes(lay, lay.value_bits, got[:, vo : vo + vd + 2], want[:, vo : vo + vd + 2], values, R,
                            vc32, vb32, True, min_allowed, n_total)
        np.testing.assert_array_equal(got[:, vo + vd + 2 :], want[:, vo + vd + 2 :])
    else:
        n += _compare_value_codes(lay, got[:, vo : vo + vd + 4], want[:, vo : vo + vd + 4], values, min_allowed,
                                  n_total)
        np.testing.assert_array_equal(got[:, vo + vd + 4 :], want[:, vo + vd + 4 :])
    return n


# ------------------------------------------------------------------ decode


class DecodeCase:
    """Inputs of one decode workload, the oracle cache, and device copies.
    block_layout "soa": the library calls use the SoA convention; the oracle
    cache stays in combined slots (``oracle_cache_bytes`` converts it)."""

    def __init__(self, w: W.Workload, need_oracle_cache: bool = True, block_layout: str = "aos"):
        t = torch()
        import quantized_decode_attention_tq_amd as tq

        self.w = w
        self.D = w.head_dim
        self.soa = block_layout == "soa"
        self.lay = O.layout(w.preset, self.D)
        self.lay_c = tq.layout_init(w.preset, self.D, block_layout)
        self.lens = W.seq_lens(w)
        self.table = W.block_table(w)
        self.nb = W.num_blocks(w)
        self.signs = W.signs(w)
        self.K, self.V = W.kv_all(w)
        self.qbits = W.queries(w)
        self.c32, self.b32 = oracle_tables(self.lay)
        self.tab = gpu_tables(self.lay_c, self.signs)
        self.shape = (self.nb, w.block_size, w.num_kv_heads, self.lay.slot_size_aligned)
        self.cache_o = None
        if need_oracle_cache:
            self.cache_o = np.zeros(self.shape, np.uint8)
            for b in range(w.batch):
                O.store_rows(self.lay, O.widen(self.K[b], w.dtype), O.widen(self.V[b], w.dtype),
                             W.slot_mapping_for_sequence(w, b, self.table, self.lens), self.cache_o, self.signs,
                             self.c32, self.b32)
        self.q = dev16(self.qbits, w.dtype)
        self.bt = t.from_numpy(self.table).cuda()
        self.sl = t.from_numpy(self.lens).cuda()
        self.scale = 1.0 / math.sqrt(self.D)

    def oracle_cache_bytes(self):
        """The oracle's cache in this case's block convention."""
        return O.soa_from_aos(self.lay, self.cache_o) if self.soa else self.cache_o

    def as_oracle_cache(self, cache_np):
        """Cache bytes of this case's convention -> combined slots."""
        return O.aos_from_soa(self.lay, cache_np) if self.soa else cache_np

    def gpu_store_all(self):
        """Fresh device cache filled by tq_store, one call per sequence."""
        t = torch()
        import quantized_decode_attention_tq_amd as tq

        cache = t.zeros(self.shape, dtype=t.uint8, device="cuda")
        for b in range(self.w.batch):
            if self.lens[b] == 0:
                continue
            slots = t.from_numpy(W.slot_mapping_for_sequence(self.w, b, self.table, self.lens)).cuda()
            tq.store(self.lay_c, dev16(self.K[b], self.w.dtype), dev16(self.V[b], self.w.dtype), slots, cache,
                     self.tab.signs, self.tab.centroids, self.tab.boundaries)
        return cache

    def gpu_decode(self, cache, num_kv_splits, out_dtype=None, sliding_window=0, sinks=None, value_gate=0.0):
        import quantized_decode_attention_tq_amd as tq

        t = torch()
        sk = None if sinks is None else t.from_numpy(np.asarray(sinks, np.float32)).cuda()
        out, lse = tq.decode(self.lay_c, self.q, cache, self.bt, self.sl, self.tab.signs, self.tab.centroids,
                             self.scale, num_kv_splits, out_dtype=out_dtype or t.float32,
                             sliding_window=sliding_window, sinks=sk, value_gate=value_gate)
        t.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)

    def gpu_decode_two_stage(self, cache, num_kv_splits, workspace_fill=None, sliding_window=0, sinks=None):
        """tq_decode_stage1 then tq_decode_stage2 (the split entry points)."""
        import quantized_decode_attention_tq_amd as tq

        t = torch()
        B, Hq = self.q.shape[:2]
        ws = t.empty(tq.decode_workspace_bytes(B, Hq, self.D, num_kv_splits), dtype=t.uint8, device="cuda")
        if workspace_fill is not None:
            ws.fill_(workspace_fill)
        tq.decode_stage1(self.lay_c, self.q, cache, self.bt, self.sl, self.tab.signs, self.tab.centroids, self.scale,
                         num_kv_splits, ws, sliding_window=sliding_window)
        out = t.empty((B, Hq, self.D), dtype=t.float32, device="cuda")
        lse = t.empty((B, Hq), dtype=t.float32, device="cuda")
        sk = None if sinks is None else t.from_numpy(np.asarray(sinks, np.float32)).cuda()
        tq.decode_stage2(B, Hq, self.D, num_kv_splits, ws, out, lse, sinks=sk)
        t.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)

    def oracle_decode(self, rows=None, cache=None, sliding_window=0, sinks=None):
        q = O.widen(self.qbits, self.w.dtype)
        sk = None if sinks is None else np.asarray(sinks, np.float32).astype(np.float64)
        return O.decode(self.lay, q, self.cache_o if cache is None else cache, self.table, self.lens, self.signs,
                        self.c32, self.scale, rows=rows, sliding_window=sliding_window, sinks=sk)

    def oracle_decode_rows_from_inputs(self, rows, sliding_window=0, sinks=None):
        """Oracle result for (b, hq) rows, storing only the needed sequence /
        KV head from the raw inputs (full-size workloads)."""
        w = self.w
        g = w.num_q_heads // w.num_kv_heads
        q = O.widen(self.qbits, w.dtype)
        R = O.rotation(self.signs.astype(np.float64)) if O.needs_rotation(self.lay) else None
        res = {}
        for b, hq in rows:
            hk = hq // g
            L = int(self.lens[b])
            slots = O.encode_slots(self.lay, O.widen(self.K[b][:, hk], w.dtype), O.widen(self.V[b][:, hk], w.dtype),
                                   R, self.c32, self.b32)
            Kd, Vd = O.decode_slots(self.lay, slots, self.c32, R)
            qq = q[b, hq] if self.lay.key_fp8 else R @ q[b, hq]
            f = O.window_start(L, sliding_window)
            sink = -math.inf if sinks is None else float(np.float32(sinks[hq]))
            res[(b, hq)] = O.attend(qq, Kd[f:L], Vd[f:L], self.scale, sink)
        return res


def check_decode(out, lse, ref_out, ref_lse, rows):
    worst = 0.0
    for b, hq in rows:
        ro, rl = ref_out[b, hq], ref_lse[b, hq]
        if rl == -math.inf:
            assert np.all(out[b, hq] == 0) and lse[b, hq] == -math.inf, (b, hq)
            continue
        err = np.max(np.abs(out[b, hq] - ro)) / max(np.max(np.abs(ro)), 1e-30)
        worst = max(worst, err)
        assert err <= DECODE_RTOL, (b, hq, err)
        assert abs(lse[b, hq] - rl) <= LSE_ATOL * max(1.0, abs(rl)), (b, hq, lse[b, hq], rl)
    return worst
