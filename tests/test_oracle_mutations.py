"""Planted mistakes in the oracle (CPU only): each plausible slip must make at
least one pin fail.  This guards the pins themselves."""

import math

import numpy as np
import pytest

import oracle as O
from oracle import tq_oracle as T
import test_oracle_pins as P


def _patch(monkeypatch, name, fn):
    """Replace a function in the oracle module and in the package namespace."""
    monkeypatch.setattr(T, name, fn)
    monkeypatch.setattr(O, name, fn)


def _fails(pin, *args):
    with pytest.raises(AssertionError):
        pin(*args)


def test_transposed_rotation_is_caught(monkeypatch):
    real = T.rotation
    _patch(monkeypatch, "rotation", lambda s: real(s).T)
    _fails(P.test_rotation_properties, 128)


def test_signs_on_wrong_side_are_caught(monkeypatch):
    _patch(monkeypatch, "rotation", lambda s: T.hadamard(s.shape[0]) * s[:, None] / math.sqrt(s.shape[0]))
    _fails(P.test_rotation_properties, 128)


def test_unrotated_query_is_caught(monkeypatch):
    real_decode = T.decode

    def bad_decode(lay, query, *a, **k):
        if lay.key_fp8:
            return real_decode(lay, query, *a, **k)
        # score the raw query against rotated-domain keys
        s = a[3]
        Rinv = T.rotation(np.asarray(s, dtype=np.float64)).T
        return real_decode(lay, np.einsum("ij,bhj->bhi", Rinv, query), *a, **k)

    _patch(monkeypatch, "decode", bad_decode)
    _fails(P.test_decode_close_to_unquantized_attention)


def test_dropped_norm_correction_is_caught(monkeypatch):
    real = T.quantize_key_mse
    _patch(monkeypatch, "quantize_key_mse", lambda x, R, c, b, nc: real(x, R, c, b, False))
    _fails(P.test_mse_key_reconstruction_statistics, 3, 0.03455, 128)


def test_inclusive_bucketize_is_caught(monkeypatch):
    def bad(u, b):
        u = np.asarray(u, dtype=np.float64)
        return (np.asarray(b, np.float64)[None, :] <= u.reshape(-1, 1)).sum(axis=1).reshape(u.shape)

    _patch(monkeypatch, "bucketize", bad)
    _fails(P.test_bucketize_ties_and_ends)


def test_msb_first_packing_is_caught(monkeypatch):
    real = T.pack_lsb

    def bad(codes, bits):
        codes = np.asarray(codes)
        rev = np.zeros_like(codes)
        for k in range(bits):
            rev |= ((codes >> k) & 1) << (bits - 1 - k)
        return real(rev, bits)

    _patch(monkeypatch, "pack_lsb", bad)
    _fails(P.test_pack_hand_examples)


def test_swapped_scale_zero_is_caught(monkeypatch):
    real = T.quantize_values
    _patch(monkeypatch, "quantize_values", lambda v, bits: (lambda c, s, z: (c, z, s))(*real(v, bits)))
    _fails(P.test_value_codec_properties)


def test_off_by_one_gather_is_caught(monkeypatch):
    real = T.gather_sequence

    def bad(lay, cache, row, L, hk, c, R=None):
        K, V = real(lay, cache, row, L + 1 if L > 0 else L, hk, c, R)
        return K[1:], V[1:]

    _patch(monkeypatch, "gather_sequence", bad)
    _fails(P.test_decode_close_to_unquantized_attention)


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    real = T.decode

    def bad(lay, query, cache, *a, **k):
        # interleaved instead of contiguous query-head groups
        B, Hq, D = query.shape
        Hk = cache.shape[2]
        g = Hq // Hk
        perm = np.array([(h % Hk) * g + h // Hk for h in range(Hq)])
        out, lse = real(lay, query[:, perm], cache, *a, **k)
        inv = np.argsort(perm)
        return out[:, inv], lse[:, inv]

    _patch(monkeypatch, "decode", bad)
    _fails(P.test_decode_close_to_unquantized_attention)


def test_head_major_soa_rows_are_caught(monkeypatch):
    real = T.soa_from_aos

    def bad(lay, c):
        c = np.asarray(c, np.uint8)
        return real(lay, c.transpose(0, 2, 1, 3).copy().reshape(c.shape))  # rows h * bs + t

    _patch(monkeypatch, "soa_from_aos", bad)
    _fails(P.test_soa_field_positions_of_one_slot, "turboquant_k3v4_nc")


def test_swapped_soa_scale_and_zero_are_caught(monkeypatch):
    real = T._slot_fields
    monkeypatch.setattr(T, "_slot_fields", lambda lay: real(lay)[:-2] + real(lay)[-2:][::-1])
    _fails(P.test_soa_field_positions_of_one_slot, "turboquant_k8v4")


def test_soa_meta_offset_counting_the_norm_is_caught(monkeypatch):
    real = T.soa_geometry

    def bad(lay, bs, Hk):  # the key norm counted as data
        data, meta, nf = real(lay, bs, Hk)
        return data, bs * Hk * (lay.key_packed_size + lay.value_data_bytes), nf

    _patch(monkeypatch, "soa_geometry", bad)
    _fails(P.test_soa_geometry_matches_the_pages_constants, "turboquant_k3v4_nc", 16, 8)


def test_sink_left_out_of_the_lse_is_caught(monkeypatch):
    real = T.attend

    def bad(q, K, V, scale, sink=-math.inf):
        o, l = real(q, K, V, scale, sink)
        return o, real(q, K, V, scale)[1]

    _patch(monkeypatch, "attend", bad)
    _fails(P.test_sink_closed_form_against_no_sink)


def test_sink_in_the_numerator_is_caught(monkeypatch):
    real = T.attend

    def bad(q, K, V, scale, sink=-math.inf):  # the sink weight spread over the values
        o, l = real(q, K, V, scale)
        if sink == -math.inf or K.shape[0] == 0:
            return real(q, K, V, scale, sink)
        return o, np.logaddexp(l, sink)

    _patch(monkeypatch, "attend", bad)
    _fails(P.test_sink_closed_form_against_no_sink)


def test_window_off_by_one_is_caught(monkeypatch):
    real = T.window_start
    _patch(monkeypatch, "window_start", lambda L, W: max(0, real(L, W) - 1) if W else 0)
    _fails(P.test_sliding_window_closed_forms)


def test_lloyd_max_values_left_rotated_are_caught(monkeypatch):
    """Decoding Lloyd-Max values without the inverse rotation leaves them in
    the rotated space: their error is about 2x the signal, not the codebook
    distortion."""
    real = T.decode_slots

    def bad(lay, slots, c32, R=None):
        K, V = real(lay, slots, c32, R)
        return K, (V @ R.T) if lay.value_lm else V

    _patch(monkeypatch, "decode_slots", bad)
    _fails(P.test_dequant_original_space_error_matches_lloyd_max_distortion, "turboquant_3bit_lm", 128)


def test_sparse_v_gate_renormalized_over_kept_tokens_is_caught(monkeypatch):
    """The gate skips only the value side: dividing by the kept tokens'
    weights alone (dropping the gated ones from the denominator) moves o."""
    def bad(q, K, V, scale, gate, sink=-math.inf):
        o, lse = T.attend(q, K, V, scale, sink)
        s = scale * (K @ q)
        f = np.exp(s - s.max())
        keep = f >= gate
        return (f[keep] @ V[keep]) / (f[keep].sum() + math.exp(sink - s.max())), lse, np.zeros(V.shape[1])

    _patch(monkeypatch, "attend_sparse_v", bad)
    _fails(P.test_sparse_v_gate_closed_form)


def _pages_trapz_variant(intervals=200, start=3.5, keep_post=False):
    """A copy of the pages' solver with one planted change."""

    def solver(d, bits, max_iter=200, tol=1e-10, info=None):
        L = 1 << bits
        s2 = 1.0 / d
        sigma = math.sqrt(s2)
        pdf = lambda x: math.exp(-x * x / (2.0 * s2)) / math.sqrt(2.0 * math.pi * s2)
        trap = lambda f, a, b: T._trapz(f, a, b, intervals)
        lo, hi = -start * sigma, start * sigma
        c = [lo + (hi - lo) * (i + 0.5) / L for i in range(L)]
        rounds, conv = 0, False
        for _ in range(max_iter):
            rounds += 1
            mids = [(c[i] + c[i + 1]) / 2.0 for i in range(L - 1)]
            edges = [-10.5 * sigma] + mids + [10.5 * sigma]
            new = [trap(lambda x: x * pdf(x), edges[i], edges[i + 1]) / trap(pdf, edges[i], edges[i + 1])
                   for i in range(L)]
            if max(abs(new[i] - c[i]) for i in range(L)) < tol:
                conv = True
                if keep_post:
                    c = new
                break
            c = new
        if info is not None:
            info.update(rounds=rounds, converged=conv)
        c = np.array(c)
        return c, (c[:-1] + c[1:]) / 2.0

    return solver


def test_pages_trapz_unchanged_copy_passes(monkeypatch):
    _patch(monkeypatch, "lloyd_max_pages_trapz", _pages_trapz_variant())
    for bits in (2, 3, 4):
        P.test_pages_trapz_against_numpy_trapezoid(bits)


@pytest.mark.parametrize("change", [{"intervals": 100}, {"start": 3.0}, {"keep_post": True}])
def test_pages_trapz_planted_changes_are_caught(monkeypatch, change):
    _patch(monkeypatch, "lloyd_max_pages_trapz", _pages_trapz_variant(**change))
    failed = 0
    for bits in (2, 3, 4):
        try:
            P.test_pages_trapz_against_numpy_trapezoid(bits)
        except AssertionError:
            failed += 1
    assert failed > 0, change


def test_value_codes_half_to_even_is_caught(monkeypatch):
    def bad(v, z, s, bits):
        with np.errstate(all="ignore"):
            x = (np.asarray(v, np.float64) - np.asarray(z, np.float64)[:, None]) / np.asarray(s, np.float64)[:, None]
        return np.clip(np.nan_to_num(np.round(x)), 0, (1 << bits) - 1).astype(np.int64)

    _patch(monkeypatch, "value_codes", bad)
    _fails(P.test_value_codes_exact_definition, 4)
