"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and its host-side functions (layout, codebook solvers, signs,
workspace size, argument validation) agree with the oracle.  No GPU work is
launched here."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import quantized_decode_attention_tq_amd as tq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_symbols():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(tq_\w+)\s*\(", src, flags=re.M))


def test_library_exports_every_declared_symbol():
    declared = _header_symbols()
    assert declared == set(tq.ABI_SYMBOLS), declared ^ set(tq.ABI_SYMBOLS)
    lib = ctypes.CDLL(tq.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert "gfx950" in tq.version()


@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("D", [64, 128, 256])
def test_layout_matches_oracle(preset, D):
    got = tq.layout_init(preset, D).as_dict()
    want = O.layout(preset, D)
    for k in ("key_data_bytes", "key_packed_size", "value_data_bytes", "value_packed_size", "slot_size",
              "slot_size_aligned", "key_bits", "value_bits"):
        assert got[k] == getattr(want, k), k
    assert got["key_fp8"] == int(want.key_fp8) and got["norm_correction"] == int(want.norm_correction)
    assert got["n_centroids"] == want.n_centroids
    assert got["preset"] == list(O.PRESETS).index(preset)


@pytest.mark.parametrize("preset", O.PRESETS)
@pytest.mark.parametrize("D", [64, 128, 256])
def test_soa_layout_matches_oracle(preset, D):
    """The SoA layout keeps every slot field of the combined one and adds the
    oracle's SoA geometry (data bytes per row, metadata fields per row)."""
    aos = tq.layout_init(preset, D).as_dict()
    soa = tq.layout_init(preset, D, "soa").as_dict()
    data, meta, nf = O.soa_geometry(O.layout(preset, D), 16, 1)
    assert aos["block_layout"] == tq.LAYOUT_AOS and aos["soa_data_bytes"] == 0 and aos["soa_meta_fields"] == 0
    assert soa["block_layout"] == tq.LAYOUT_SOA and soa["soa_data_bytes"] == data and soa["soa_meta_fields"] == nf
    for k, v in aos.items():
        if k not in ("block_layout", "soa_data_bytes", "soa_meta_fields"):
            assert soa[k] == v, k
    for bs in O.BLOCK_SIZES:
        assert tq.kv_cache_shape(tq.layout_init(preset, D, "soa"), 5, bs, 3) == tq.kv_cache_shape(
            tq.layout_init(preset, D), 5, bs, 3)


def test_soa_layout_codes():
    L = tq.Layout()
    assert tq._lib.tq_layout_init_ex(0, 128, 2, ctypes.byref(L)) == tq.TQ_EINVAL
    assert tq._lib.tq_layout_init_ex(0, 128, -1, ctypes.byref(L)) == tq.TQ_EINVAL
    bad = tq.layout_init("turboquant_k3v4_nc", 128, "soa")
    bad.soa_meta_fields = 2  # not what tq_layout_init_ex produces
    assert _store_validate(bad) == tq.TQ_EINVAL
    mixed = tq.layout_init("turboquant_k3v4_nc")
    mixed.block_layout = tq.LAYOUT_SOA  # AoS sizes with the SoA flag
    assert _store_validate(mixed) == tq.TQ_EINVAL
    S = tq.layout_init("turboquant_k3v4_nc", 128, "soa")
    # decode over SoA: all heads in one workgroup (<= 8) or groups of 8
    for Hk, want in ((1, tq.TQ_OK), (3, tq.TQ_OK), (8, tq.TQ_OK), (16, tq.TQ_OK), (12, tq.TQ_EUNSUPPORTED),
                     (10, tq.TQ_EUNSUPPORTED)):
        assert _decode_validate(S, Hk=Hk, Hq=Hk * 4, wsb=tq.decode_workspace_bytes(4, Hk * 4, 128, 8)) == want, Hk
    assert _dequant_validate(S) == tq.TQ_OK
    assert _store_validate(S) == tq.TQ_OK


def test_kv_cache_shape_and_presets():
    for p in O.PRESETS:
        L = tq.layout_init(p)
        for bs in O.BLOCK_SIZES:
            assert tq.kv_cache_shape(L, 37, bs, 8) == O.kv_cache_shape(O.layout(p, 128), 37, bs, 8)
        with pytest.raises(tq.TQError) as e:
            tq.kv_cache_shape(L, 37, 24, 8)
        assert e.value.status == tq.TQ_EBLOCK
    with pytest.raises(tq.TQError) as e:
        tq.preset_from_name("turboquant_5bit")
    assert e.value.status == tq.TQ_EPRESET
    with pytest.raises(tq.TQError) as e:
        tq.layout_init(len(O.PRESETS))
    assert e.value.status == tq.TQ_EPRESET


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_lloyd_max_exact_matches_oracle(bits, d):
    c, b = tq.lloyd_max(d, bits, 0)
    oc, ob = O.codebook_tables(d, bits, "exact")
    np.testing.assert_array_equal(c, oc)
    np.testing.assert_array_equal(b, ob)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_max_pages_trapz_matches_oracle(bits):
    c, b = tq.lloyd_max(128, bits, 1)
    oc, ob = O.codebook_tables(128, bits, "pages-trapz")
    np.testing.assert_array_equal(c, oc)
    np.testing.assert_array_equal(b, ob)


@pytest.mark.parametrize("seed", [0, 1, 42, 1337, 2 ** 63 + 5])
def test_wht_signs_match_oracle_splitmix64(seed):
    np.testing.assert_array_equal(tq.wht_signs(256, seed), O.wht_signs(256, seed).astype(np.float32))


def test_workspace_bytes():
    """At least the pages' (B, Hq, S, D+1) partial buffer; the library's own
    layout is a (first unit, unit count) table per sequence, then 16-byte
    partial rows (D outputs + LSE + pad) for up to S_max = S * max(1,
    ceil(512 / (B * S))) units per sequence."""
    for B, Hq, S in ((1, 2, 1), (32, 32, 16), (4, 40, 32), (64, 64, 8), (32, 32, 8), (3, 6, 5)):
        n = tq.decode_workspace_bytes(B, Hq, 128, S)
        assert n >= O.workspace_bytes(B, Hq, 128, S) and n % 256 == 0
        s_max = S * max(1, -(-512 // (B * S)))
        want = -(-8 * B // 256) * 256 + B * Hq * s_max * (128 + 4) * 4
        assert n == -(-want // 256) * 256, (B, Hq, S)


# ------------------------------------------------------------ validation
# The *_validate entry points check arguments on the host and touch no
# memory, so fake (aligned, non-null) addresses are fine here.

A = 0x10000  # a 16-byte aligned fake address


def _store_validate(L, **kw):
    args = dict(key=A, value=A, in_dtype=tq.TQ_BF16, N=4, Hk=8, ks=1024, vs=1024, slots=A, cache=A, nb=10, bs=16,
                signs=A, cent=A, bnd=A)
    args.update(kw)
    return tq._lib.tq_store_validate(ctypes.byref(L), args["key"], args["value"], args["in_dtype"], args["N"],
                                     args["Hk"], args["ks"], args["vs"], args["slots"], args["cache"], args["nb"],
                                     args["bs"], args["signs"], args["cent"], args["bnd"])


def test_store_validation_codes():
    L = tq.layout_init("turboquant_3bit_nc")
    assert _store_validate(L) == tq.TQ_OK
    assert _store_validate(L, N=0, key=None, value=None, slots=None, cache=None) == tq.TQ_OK  # N = 0: no-op
    assert _store_validate(L, bs=24) == tq.TQ_EBLOCK
    assert _store_validate(L, in_dtype=tq.TQ_F32) == tq.TQ_EDTYPE
    assert _store_validate(L, key=None) == tq.TQ_EINVAL
    assert _store_validate(L, key=A + 2) == tq.TQ_EINVAL  # misaligned
    assert _store_validate(L, ks=1020) == tq.TQ_EINVAL  # stride below Hk*D
    assert _store_validate(L, signs=None) == tq.TQ_EINVAL
    assert _store_validate(L, N=-1) == tq.TQ_EINVAL
    assert _store_validate(tq.layout_init("turboquant_k8v4"), signs=None, cent=None, bnd=None) == tq.TQ_OK
    assert _store_validate(tq.layout_init("turboquant_3bit_nc", 64)) == tq.TQ_EHEADDIM
    assert _store_validate(tq.layout_init("turboquant_3bit_nc", 256), ks=2048, vs=2048) == tq.TQ_OK
    assert _store_validate(tq.layout_init("turboquant_3bit_nc", 256)) == tq.TQ_EINVAL  # stride below Hk * 256
    bad = tq.layout_init("turboquant_3bit_nc")
    bad.slot_size_aligned = 104  # layout not produced by tq_layout_init
    assert _store_validate(bad) == tq.TQ_EINVAL


def _decode_validate(L, **kw):
    args = dict(q=A, qd=tq.TQ_BF16, B=4, Hq=32, Hk=8, cache=A, nb=100, bs=16, bt=A, bts=64, sl=A, signs=A, cent=A,
                S=8, win=0, gate=0.0, ws=A, wsb=tq.decode_workspace_bytes(4, 32, 128, 8), out=A, od=tq.TQ_F32)
    args.update(kw)
    return tq._lib.tq_decode_validate(ctypes.byref(L), args["q"], args["qd"], args["B"], args["Hq"], args["Hk"],
                                      args["cache"], args["nb"], args["bs"], args["bt"], args["bts"], args["sl"],
                                      args["signs"], args["cent"], args["S"], args["win"], args["gate"], args["ws"],
                                      args["wsb"],
                                      args["out"], args["od"])


def test_decode_validation_codes():
    L = tq.layout_init("turboquant_k3v4_nc")
    assert _decode_validate(L) == tq.TQ_OK
    assert _decode_validate(L, Hq=33) == tq.TQ_EGQA
    assert _decode_validate(L, Hk=0) == tq.TQ_EGQA
    assert _decode_validate(L, bs=8) == tq.TQ_EBLOCK
    assert _decode_validate(L, wsb=1024) == tq.TQ_EWORKSPACE
    assert _decode_validate(L, qd=tq.TQ_F32) == tq.TQ_EDTYPE
    assert _decode_validate(L, od=7) == tq.TQ_EDTYPE
    assert _decode_validate(L, S=0) == tq.TQ_EINVAL
    assert _decode_validate(L, win=-1) == tq.TQ_EINVAL
    assert _decode_validate(L, win=4096) == tq.TQ_OK
    assert _decode_validate(L, gate=1e-3) == tq.TQ_OK  # the opt-in sparse-V gate
    for bad in (-1e-3, 1.0, float("nan"), float("inf")):
        assert _decode_validate(L, gate=bad) == tq.TQ_EINVAL, bad
    assert _decode_validate(L, sl=None) == tq.TQ_EINVAL
    assert _decode_validate(L, ws=A + 8) == tq.TQ_EINVAL
    assert _decode_validate(L, signs=None) == tq.TQ_EINVAL
    assert _decode_validate(tq.layout_init("turboquant_k8v4"), signs=None, cent=None) == tq.TQ_OK
    assert _decode_validate(L, B=0, q=None, sl=None, bt=None, ws=None, out=None) == tq.TQ_OK


def test_one_hip_runtime_in_the_process():
    """libtq.so binds to the HIP runtime torch already loaded: a second copy
    would not see torch's streams or graph captures."""
    import torch  # noqa: F401

    maps = open("/proc/self/maps").read().split("\n")
    paths = {l.split()[-1] for l in maps if "libamdhip64" in l and "/" in l}
    assert len({os.path.realpath(p) for p in paths}) == 1, paths


def _dequant_validate(L, **kw):
    args = dict(cache=A, nb=10, bs=16, Hk=8, bt=A, n=100, signs=A, cent=A, ko=A, vo=A, od=tq.TQ_F16, stride=1024)
    args.update(kw)
    return tq._lib.tq_dequant_validate(ctypes.byref(L), args["cache"], args["nb"], args["bs"], args["Hk"], args["bt"],
                                       args["n"], args["signs"], args["cent"], args["ko"], args["vo"], args["od"],
                                       args["stride"])


def test_dequant_validation_codes():
    L = tq.layout_init("turboquant_k3v4_nc")
    assert _dequant_validate(L) == tq.TQ_OK
    assert _dequant_validate(L, n=0, cache=None, bt=None, ko=None, vo=None) == tq.TQ_OK  # empty prefix: no-op
    assert _dequant_validate(L, bs=8) == tq.TQ_EBLOCK
    assert _dequant_validate(L, od=7) == tq.TQ_EDTYPE
    assert _dequant_validate(L, od=tq.TQ_F32) == tq.TQ_OK
    assert _dequant_validate(L, n=-1) == tq.TQ_EINVAL
    assert _dequant_validate(L, Hk=0) == tq.TQ_EINVAL
    assert _dequant_validate(L, ko=A + 8) == tq.TQ_EINVAL  # misaligned output
    assert _dequant_validate(L, stride=1020) == tq.TQ_EINVAL  # token stride below Hk * D
    assert _dequant_validate(L, stride=1028) == tq.TQ_EINVAL  # not a multiple of 8 elements
    assert _dequant_validate(L, stride=2048) == tq.TQ_OK  # rows inside a larger buffer
    assert _dequant_validate(L, n=161) == tq.TQ_EINVAL  # needs 11 blocks, 10 exist
    assert _dequant_validate(L, signs=None) == tq.TQ_EINVAL
    assert _dequant_validate(tq.layout_init("turboquant_k8v4"), signs=None, cent=None) == tq.TQ_OK
    assert _dequant_validate(tq.layout_init("turboquant_k3v4_nc", 64)) == tq.TQ_EHEADDIM
    assert _dequant_validate(tq.layout_init("turboquant_k3v4_nc", 256), stride=2048) == tq.TQ_OK
    assert _dequant_validate(L, n=1 << 28, nb=1 << 30) == tq.TQ_EINVAL  # rows beyond 2^31


def _noalloc(L, **kw):
    args = dict(q=A, qd=tq.TQ_BF16, B=4, Hq=32, Hk=8, cache=A, nb=100, bs=16, bt=A, bts=64, sl=A, signs=A, cent=A,
                S=8, win=0, gate=0.0, sinks=None, out=A, od=tq.TQ_F32, lse=None)
    args.update(kw)
    return tq._lib.tq_decode_attention_noalloc(ctypes.byref(L), args["q"], args["qd"], args["B"], args["Hq"],
                                               args["Hk"], args["cache"], args["nb"], args["bs"], args["bt"],
                                               args["bts"], args["sl"], args["signs"], args["cent"], 1.0, args["S"],
                                               args["win"], args["gate"], args["sinks"], args["out"], args["od"],
                                               args["lse"], None)


def test_noalloc_scratch_limit_and_argument_errors():
    """tq_decode_attention_noalloc checks every argument, and the workspace
    its launch needs against the scratch it holds (TQ_NOALLOC_SCRATCH_BYTES),
    on the host before any HIP call: these calls return before touching a
    device (fake addresses)."""
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    m = re.search(r"#define TQ_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == tq.NOALLOC_SCRATCH_BYTES
    L = tq.layout_init("turboquant_k3v4_nc")
    # the largest case that fits and the smallest that does not, for 64 query heads and 8 splits
    assert tq.decode_workspace_bytes(64, 64, 128, 8) <= tq.NOALLOC_SCRATCH_BYTES
    assert tq.decode_workspace_bytes(128, 64, 128, 8) > tq.NOALLOC_SCRATCH_BYTES
    assert _noalloc(L, B=128, Hq=64) == tq.TQ_EWORKSPACE
    assert _noalloc(L, B=4, Hq=40, S=1024) == tq.TQ_EWORKSPACE
    assert _noalloc(L, Hq=33) == tq.TQ_EGQA
    assert _noalloc(L, bs=8) == tq.TQ_EBLOCK
    assert _noalloc(L, od=7) == tq.TQ_EDTYPE
    assert _noalloc(L, out=None) == tq.TQ_EINVAL
    assert _noalloc(L, gate=1.0) == tq.TQ_EINVAL
    assert _noalloc(L, B=0, q=None, sl=None, bt=None, out=None) == tq.TQ_OK  # nothing to do
