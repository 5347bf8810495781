"""Plain, slow CPU oracle for the TurboQuant KV-cache store and decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this module imports nothing from the product path.

Everything here is NumPy in float64.  Where a floating-point comparison decides
an integer (a Lloyd-Max bucket, a value code) the oracle takes the decision on
the exact value of the defining expression; the kernels take it in fp32, so
their codes may differ next to a decision boundary, which the parity tests
allow for (at most one step, within 1e-6 of the boundary, on at most 1e-5 of
the coordinates).

Sources (cited by page title and section; the pages are the only authority):

* [TRACK]  vLLM issue #40069 "[Tracking issue]: TurboQuant/HIGGS Attention
           follow-ups".
* [PR]     prhub summary of vLLM PR #38479 (TurboQuant attention backend):
           sections "功能与动机" (motivation), "实现拆解" (implementation
           breakdown), "关键源码片段" (source excerpts of turboquant_attn.py,
           centroids.py and attention.py::_init_turboquant_buffers),
           "评论区精华" (review highlights).
* [API]    vLLM API docs page "vllm.v1.attention.backends.turboquant_attn":
           TurboQuantAttentionBackend, TurboQuantAttentionImpl.__init__,
           _ensure_on_device, do_kv_cache_update, _store_kv,
           _continuation_prefill, _decode_attention.
* [TQ+]    Atlas docs "TurboQuant+ — KV-cache compression beyond the Google
           baseline": sections "Background", "What landed (file-by-file)".

Where the pages leave a point open, the function that depends on it
states the reading it takes.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (and guarded by the planted-mistake tests in
``tests/test_oracle_mutations.py``).  One property is "parity unpinned":
byte-for-byte compatibility of a slot with the pages' own (vLLM) kernels --
the pages print no worked slot, so the slot byte order is pinned only by
self-consistency and the hand-derived packing examples.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# --------------------------------------------------------------------------
# Presets and slot layout
# --------------------------------------------------------------------------

#: preset name -> (key_fp8, key_bits, value_bits, norm_correction, value_lloyd_max)
#: [PR] "实现拆解" item 1 (four named presets, each fixing key bits, value bits
#: and norm correction); [PR] "评论区精华" (k8v4 = FP8 keys + 4-bit values);
#: [API] TurboQuantAttentionBackend.supported_kv_cache_dtypes.
PRESETS = {
    "turboquant_k8v4": (True, 8, 4, False, False),
    "turboquant_4bit_nc": (False, 4, 4, True, False),
    "turboquant_k3v4_nc": (False, 3, 4, True, False),
    "turboquant_3bit_nc": (False, 3, 3, True, False),
    # More codecs, from the Atlas page ([TQ+] "What landed": the 2-bit
    # Lloyd-Max codebook "Turbo2", 4 codes per byte; asymmetric K/V pairs
    # with FP8 keys or 4-bit keys over 3-bit values).  Reading: the pairs
    # take this module's key codecs and its uniform value codec at the
    # stated bit widths (the Atlas value codebook is not modelled); the
    # 2-bit preset quantizes keys with the 2-bit Lloyd-Max codebook and
    # values with the 2-bit uniform codec, norm-corrected like the others.
    "turboquant_k8v3": (True, 8, 3, False, False),
    "turboquant_k4v3_nc": (False, 4, 3, True, False),
    "turboquant_2bit_nc": (False, 2, 2, True, False),
    # The Atlas value codec ([TQ+] "What landed": values take the same
    # rotation ("WHT bookend") and Lloyd-Max codebook as keys, with the
    # matched-norm correction; [TQ+] asymmetric pairs such as FP8 K + 3-bit
    # V, and the symmetric 3-bit codec).  The value region is [codes | fp16
    # norm]; the value codebook is the Lloyd-Max codebook of the value bit
    # width for N(0, 1/D), as for keys.
    "turboquant_k8v3lm": (True, 8, 3, False, True),
    "turboquant_3bit_lm": (False, 3, 3, True, True),
    # The same value codec at the other widths of the Atlas page's
    # turbo2/3/4 family ([TQ+] "What landed": 2-, 3- and 4-bit Lloyd-Max
    # codebooks, asymmetric pairs with FP8 keys): FP8 K + 4-bit V, and the
    # symmetric 4- and 2-bit codecs.
    "turboquant_k8v4lm": (True, 8, 4, False, True),
    "turboquant_4bit_lm": (False, 4, 4, True, True),
    "turboquant_2bit_lm": (False, 2, 2, True, True),
}

#: kernel block sizes the backend accepts ([PR] turboquant_attn.py excerpt,
#: get_supported_kernel_block_sizes; [API] same method).
BLOCK_SIZES = (16, 32, 64, 128)


@dataclass(frozen=True)
class Layout:
    """Byte layout of one combined K+V slot (one token, one KV head).

    [API] TurboQuantAttentionImpl.__init__ (mse bytes = ceil(D*bits/8), or D
    for FP8 keys; value data bytes = ceil(D*value_bits/8)); [API]
    _continuation_prefill (key packed size differs from the MSE bytes: the
    norm follows the codes; scale and zero are 16-bit fields); [PR]
    turboquant_attn.py excerpt get_kv_cache_shape (slot rounded up to even).
    """

    preset: str
    head_dim: int
    key_fp8: bool
    key_bits: int
    value_bits: int
    norm_correction: bool
    key_data_bytes: int  # packed key codes, or D fp8 bytes
    key_packed_size: int  # key region: codes + fp16 norm (MSE), or D (fp8)
    value_data_bytes: int  # packed value codes
    value_packed_size: int  # value region: codes + fp16 scale + fp16 zero (Lloyd-Max values: + fp16 norm)
    slot_size: int
    slot_size_aligned: int
    value_lm: bool = False  # values: rotated Lloyd-Max codes with a norm (else uniform min/max codes)

    @property
    def n_centroids(self) -> int:
        return 0 if self.key_fp8 else (1 << self.key_bits)


def layout(preset: str, head_dim: int) -> Layout:
    key_fp8, kb, vb, nc, vlm = PRESETS[preset]
    D = head_dim
    if key_fp8:
        kdata = D
        kps = D  # FP8 keys carry no norm field
    else:
        kdata = math.ceil(D * kb / 8)
        kps = kdata + 2  # fp16 norm after the codes
    vdata = math.ceil(D * vb / 8)
    vps = vdata + (2 if vlm else 4)  # fp16 norm, or fp16 scale + fp16 zero
    slot = kps + vps
    aligned = ((slot + 1) // 2) * 2
    return Layout(preset, D, key_fp8, kb, vb, nc, kdata, kps, vdata, vps, slot, aligned, vlm)


def needs_rotation(lay: Layout) -> bool:
    """Whether the slots of this layout hold rotated coordinates (MSE keys
    or Lloyd-Max values)."""
    return (not lay.key_fp8) or lay.value_lm


def value_tables(lay: Layout):
    """The value codebook and boundaries (fp32) of a Lloyd-Max value layout."""
    return codebook_tables(lay.head_dim, lay.value_bits)


def kv_cache_shape(lay: Layout, num_blocks: int, block_size: int, num_kv_heads: int):
    """Combined cache shape, no leading K/V dimension ([PR] get_kv_cache_shape)."""
    return (num_blocks, block_size, num_kv_heads, lay.slot_size_aligned)


# --------------------------------------------------------------------------
# Lloyd-Max codebook for the coordinate marginal N(0, 1/d)
# --------------------------------------------------------------------------


def _phi(x: float) -> float:
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _cell_mean_std_normal(a: float, b: float) -> float:
    """E[Z | a < Z < b] for Z ~ N(0,1), closed form (phi(a)-phi(b))/(Phi(b)-Phi(a)).

    The probability mass uses erfc on the side that keeps it accurate in the
    tails.  a may be -inf and b may be +inf.
    """
    pa = 0.0 if math.isinf(a) else _phi(a)
    pb = 0.0 if math.isinf(b) else _phi(b)
    if a >= 0.0:
        mass = 0.5 * (math.erfc(a / math.sqrt(2.0)) - (0.0 if math.isinf(b) else math.erfc(b / math.sqrt(2.0))))
    elif b <= 0.0:
        mass = 0.5 * (math.erfc(-b / math.sqrt(2.0)) - (0.0 if math.isinf(a) else math.erfc(-a / math.sqrt(2.0))))
    else:
        lo = 0.0 if math.isinf(a) else 0.5 * math.erfc(-a / math.sqrt(2.0))
        hi = 1.0 if math.isinf(b) else 1.0 - 0.5 * math.erfc(b / math.sqrt(2.0))
        mass = hi - lo
    return (pa - pb) / mass


def lloyd_max_exact(d: int, bits: int, tol: float = 1e-15, max_iter: int = 200000):
    """Exact Lloyd-Max quantizer for N(0, 1/d), float64.

    [PR] "关键源码片段", centroids.py: after a random rotation each coordinate
    of a unit vector is approximately N(0, 1/d); the codebook solves the
    Lloyd-Max conditions (boundaries at midpoints of adjacent centroids, each
    centroid the conditional mean of its cell).  The pages integrate the cell
    moments with a trapezoid rule (see ``lloyd_max_pages_trapz``); this is the
    exact solution (reading R3): the conditional means are the closed form
    for the Gaussian, iterated to a fixed point in float64.

    The density is symmetric, so the unique optimum is antisymmetric; it is
    solved on the positive half-line and mirrored, which makes
    c[L-1-j] == -c[j] exactly.  Returns (centroids, boundaries) in float64,
    sorted ascending, boundaries = midpoints.
    """
    L = 1 << bits
    sigma = 1.0 / math.sqrt(d)
    half = L // 2
    # positive half: centroids p[0] < ... < p[half-1]; cells [0,t1), [t1,t2), ..., [t_{h-1}, inf)
    p = [(k + 0.5) * 3.0 / half for k in range(half)]  # in units of sigma
    for _ in range(max_iter):
        t = [0.0] + [(p[k] + p[k + 1]) / 2.0 for k in range(half - 1)] + [math.inf]
        new = [_cell_mean_std_normal(t[k], t[k + 1]) for k in range(half)]
        delta = max(abs(new[k] - p[k]) for k in range(half))
        p = new
        if delta < tol:
            break
    pos = np.array(p, dtype=np.float64) * sigma
    cents = np.concatenate([-pos[::-1], pos])
    bounds = (cents[:-1] + cents[1:]) / 2.0
    return cents, bounds


def _trapz(f, a: float, b: float, n: int = 200) -> float:
    h = (b - a) / n
    s = 0.5 * (f(a) + f(b))
    for i in range(1, n):
        s += f(a + i * h)
    return s * h


def lloyd_max_pages_trapz(d: int, bits: int, max_iter: int = 200, tol: float = 1e-10, info=None):
    """The pages' own solver ([PR] "关键源码片段", centroids.py), transcribed
    step for step so that its output can be reproduced exactly (reading R3).

    Start from 2^bits centroids spread uniformly over +-3.5 sigma; each round
    takes boundaries at midpoints, closes the outer cells at +-10.5 sigma,
    and sets each centroid to the trapezoid-rule (200 intervals) ratio of the
    first to the zeroth moment of the N(0, 1/d) density over its cell.  It
    stops after ``max_iter`` rounds or as soon as no centroid moves by
    ``tol`` -- and in that case keeps the centroids from before the last
    update.  Returns float64 (centroids, boundaries) before the fp32 cast the
    pages apply.  ``info`` (a dict, optional) receives the number of rounds
    run and whether the tolerance stopped it.
    """
    L = 1 << bits
    s2 = 1.0 / d
    sigma = math.sqrt(s2)

    def pdf(x):
        return math.exp(-x * x / (2.0 * s2)) / math.sqrt(2.0 * math.pi * s2)

    lo, hi = -3.5 * sigma, 3.5 * sigma
    c = [lo + (hi - lo) * (i + 0.5) / L for i in range(L)]
    rounds, converged = 0, False
    for _ in range(max_iter):
        rounds += 1
        mids = [(c[i] + c[i + 1]) / 2.0 for i in range(L - 1)]
        edges = [3.0 * lo] + mids + [3.0 * hi]
        new = []
        for i in range(L):
            a, b = edges[i], edges[i + 1]
            num = _trapz(lambda x: x * pdf(x), a, b)
            den = _trapz(pdf, a, b)
            new.append(num / den if den > 1e-15 else c[i])
        if max(abs(new[i] - c[i]) for i in range(L)) < tol:
            converged = True
            break
        c = new
    if info is not None:
        info.update(rounds=rounds, converged=converged)
    c = np.array(c, dtype=np.float64)
    return c, (c[:-1] + c[1:]) / 2.0


def codebook_tables(d: int, bits: int, mode: str = "exact"):
    """fp32 (centroids, boundaries) as the kernels consume them.

    Centroids are cast to fp32; boundaries are the fp32 midpoints of the
    sorted fp32 centroids ([API] _ensure_on_device derives the midpoints from
    the fp32 centroids; reading R4).  Halving is exact in binary, so the fp32
    midpoint equals fl32(a + b) / 2.
    """
    if mode == "exact":
        c, _ = lloyd_max_exact(d, bits)
    elif mode == "pages-trapz":
        c, _ = lloyd_max_pages_trapz(d, bits)
    else:
        raise ValueError(mode)
    c32 = np.sort(c.astype(np.float32))
    b32 = ((c32[:-1] + c32[1:]) / np.float32(2.0)).astype(np.float32)
    return c32, b32


# --------------------------------------------------------------------------
# Rademacher signs (counter-based generator, from its published definition)
# --------------------------------------------------------------------------

_M64 = (1 << 64) - 1


def splitmix64(seed: int, n: int):
    """n outputs of SplitMix64 (Steele, Lea, Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014; the 64-bit finalizer of
    Stafford's Mix13): state += 0x9E3779B97F4A7C15, then two xor-shift-
    multiply rounds and a final xor-shift."""
    out = []
    x = seed & _M64
    for _ in range(n):
        x = (x + 0x9E3779B97F4A7C15) & _M64
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        z = z ^ (z >> 31)
        out.append(z)
    return out


def wht_signs(d: int, seed: int) -> np.ndarray:
    """Rademacher signs for the rotation: s_i = -1 when the top bit of the
    i-th SplitMix64 draw is set (reading R15; the pages generate the signs
    from a per-layer seed, [PR] attention.py excerpt, but do not print the
    generator)."""
    return np.array([-1.0 if (z >> 63) else 1.0 for z in splitmix64(seed, d)], dtype=np.float64)


# --------------------------------------------------------------------------
# Randomized Hadamard rotation
# --------------------------------------------------------------------------


def hadamard(d: int) -> np.ndarray:
    """Sylvester-ordered Walsh-Hadamard matrix: H[i][j] = (-1)^popcount(i & j)."""
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def rotation(signs: np.ndarray) -> np.ndarray:
    """R = H_D . diag(s) / sqrt(D): signs first, then the Walsh-Hadamard
    transform ([TQ+] "Background": the randomized Hadamard transform applies
    a random sign vector before the WHT; [PR] "功能与动机": the WHT rotation
    makes the coordinates nearly independent).  Orthonormal."""
    D = signs.shape[0]
    return hadamard(D) * signs[None, :] / math.sqrt(D)


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit input patterns -> float64 values (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        if dtype == "bf16":
            return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        if dtype == "f16":
            return bits.view(np.float16).astype(np.float64)
    raise ValueError(dtype)


def fp16_bits(x) -> np.ndarray:
    """IEEE binary16, round to nearest even (NumPy's cast), as uint16 bits."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def fp8_e4m3fn_decode(codes) -> np.ndarray:
    """OCP FP8 E4M3 ("fn": no infinities, S.1111.111 is NaN), exponent bias 7."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7.0))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


_E4M3_POS = fp8_e4m3fn_decode(np.arange(0x7F))  # finite non-negative values, codes 0..0x7E, ascending


def fp8_e4m3fn_encode(x) -> np.ndarray:
    """Round to the nearest finite E4M3 value, ties to even code, saturating at
    +-448 (reading R13: OCP E4M3 on gfx950, no per-tensor scale, [API]
    TurboQuantAttentionBackend.supports_per_head_quant_scales is False).
    NaN maps to 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.where(np.isnan(x), 0.0, np.abs(x))
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = np.abs(_E4M3_POS[hi] - a)
    d_lo = np.abs(a - _E4M3_POS[lo])
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = pick.astype(np.int64) | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# Code packing
# --------------------------------------------------------------------------


def pack_lsb(codes, bits: int) -> np.ndarray:
    """Pack b-bit codes as one little-endian bit stream: code j occupies bits
    [b*j, b*j+b).  At 3 bits this puts 8 codes in every 3 bytes ([TQ+]
    "Background": Turbo3 stores 8 values per 3 bytes); at 4 bits the even
    index is the low nibble (reading R10)."""
    codes = np.asarray(codes, dtype=np.int64)
    n = codes.shape[-1]
    nbytes = math.ceil(n * bits / 8)
    out = np.zeros(codes.shape[:-1] + (nbytes,), dtype=np.int64)
    for j in range(n):
        for k in range(bits):
            pos = bits * j + k
            out[..., pos // 8] |= ((codes[..., j] >> k) & 1) << (pos % 8)
    return out.astype(np.uint8)


def unpack_lsb(data, bits: int, n: int) -> np.ndarray:
    data = np.asarray(data, dtype=np.int64)
    out = np.zeros(data.shape[:-1] + (n,), dtype=np.int64)
    for j in range(n):
        for k in range(bits):
            pos = bits * j + k
            out[..., j] |= ((data[..., pos // 8] >> (pos % 8)) & 1) << k
    return out


def _u16_le(bits16) -> np.ndarray:
    b = np.asarray(bits16, dtype=np.uint16)
    return np.stack([(b & 0xFF).astype(np.uint8), (b >> 8).astype(np.uint8)], axis=-1)


def _from_u16_le(two_bytes) -> np.ndarray:
    t = np.asarray(two_bytes, dtype=np.uint16)
    return (t[..., 0] | (t[..., 1] << 8)).astype(np.uint16)


# --------------------------------------------------------------------------
# Quantizers
# --------------------------------------------------------------------------


def bucketize(u, boundaries) -> np.ndarray:
    """Code = number of boundaries strictly below the value (reading R5: ties
    go to the lower bucket).  [PR] "评论区精华" item 3: bucketing is a search
    over the sorted boundaries, not a scan that stops early."""
    u = np.asarray(u, dtype=np.float64)
    b = np.asarray(boundaries, dtype=np.float64)
    return (b[None, :] < u.reshape(-1, 1)).sum(axis=1).reshape(u.shape)


def quantize_key_mse(x, R, centroids32, boundaries32, norm_correction: bool):
    """One key vector -> (codes, norm field value).

    ν = ||x||, u = R x / ν, code_i = bucketize(u_i); with norm correction the
    stored norm is γ = ν / ||c[code]||, so that γ·c[code] has the input's
    norm ([TQ+] "Background": the L2-minimising scale is ||original|| /
    ||reconstructed||, not max/amax; [TQ+] "What landed": matched-norm L2
    correction in the turbo write paths).  ν = 0 gives u = 0 and γ = 0.
    """
    x = np.asarray(x, dtype=np.float64)
    nu = math.sqrt(float(np.dot(x, x)))
    u = (R @ x) / nu if nu > 0.0 else np.zeros_like(x)
    codes = bucketize(u, boundaries32)
    chat = np.asarray(centroids32, dtype=np.float64)[codes]
    if nu == 0.0:
        gamma = 0.0
    elif norm_correction:
        gamma = nu / math.sqrt(float(np.dot(chat, chat)))
    else:
        gamma = nu
    return codes, gamma


def _value_scale_zero(vmin, vmax, bits: int):
    """fp16 (scale, zero) of rows with extremes vmin, vmax (float64 arrays):
    zero = fp16(min v), scale = fp16((max v - min v) / (2^b - 1)), each
    rounded to nearest even once from the float64 value ([API]
    _continuation_prefill: the value region ends with 16-bit scale and zero
    fields).  For 16-bit inputs the difference is exact in float64 and the
    quotient's one float64 rounding does not change its fp16 rounding."""
    levels = (1 << bits) - 1
    with np.errstate(all="ignore"):
        s16 = ((vmax - vmin) / float(levels)).astype(np.float16)
    z16 = np.asarray(vmin, dtype=np.float64).astype(np.float16)
    return s16, z16


def value_codes(v, z, s, bits: int) -> np.ndarray:
    """code = clamp(floor((v - z) / s + 1/2), 0, 2^b - 1) against the stored
    fp16 scale s and zero z (reading R12: round half up, clamp; scale 0
    gives all-zero codes; a NaN quotient gives 0).  v: (rows, D) float64;
    z, s: (rows,) float64.  The decision is exact: the float64 quotient
    settles every code whose quotient is not within 1e-9 of a half-integer,
    and those few are recomputed in rational arithmetic from the exact
    binary values of v, z and s."""
    from fractions import Fraction

    levels = (1 << bits) - 1
    v = np.asarray(v, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)[:, None]
    s = np.asarray(s, dtype=np.float64)[:, None]
    with np.errstate(all="ignore"):
        x = (v - z) / s
        fl = np.floor(x + 0.5)
    fl = np.where(np.isnan(fl), 0.0, fl)
    frac = x - np.floor(x)
    near = np.isfinite(x) & np.isfinite(v) & np.isfinite(z) & np.isfinite(s) & (s != 0) & \
        (np.abs(frac - 0.5) < 1e-9 * np.maximum(1.0, np.abs(x)))
    for r, c in zip(*np.nonzero(near)):
        q = (Fraction(float(v[r, c])) - Fraction(float(z[r, 0]))) / Fraction(float(s[r, 0])) + Fraction(1, 2)
        fl[r, c] = float(q.numerator // q.denominator)
    codes = np.clip(fl, 0, levels).astype(np.int64)
    codes[np.broadcast_to(s == 0, codes.shape)] = 0
    return codes


def quantize_values(v, bits: int):
    """One value vector -> (codes, fp16 scale bits, fp16 zero bits).

    Uniform asymmetric codes in the unrotated space with a per-slot fp16
    scale and zero ([API] _continuation_prefill: the value region holds the
    codes then two 16-bit fields, scale and zero; values are not rotated),
    the codes formed against the stored fp16 scale and zero (reading R12):
    see ``_value_scale_zero`` and ``value_codes``.
    """
    v = np.asarray(v, dtype=np.float64).reshape(1, -1)
    s16, z16 = _value_scale_zero(v.min(axis=1), v.max(axis=1), bits)
    codes = value_codes(v, z16.astype(np.float64), s16.astype(np.float64), bits)[0]
    return codes, np.array(s16[0]).view(np.uint16), np.array(z16[0]).view(np.uint16)


def encode_slot(lay: Layout, k, v, R, centroids32, boundaries32) -> np.ndarray:
    """One (token, KV head) -> slot bytes (length slot_size_aligned).

    AoS slot: [key codes | fp16 γ][value codes | fp16 scale | fp16 zero][pad]
    for MSE keys, or [D x fp8 key][value region][pad] for FP8 keys (reading
    R9; [API] _continuation_prefill for the region sizes).
    """
    out = np.zeros(lay.slot_size_aligned, dtype=np.uint8)
    if lay.key_fp8:
        out[: lay.head_dim] = fp8_e4m3fn_encode(k)
    else:
        codes, gamma = quantize_key_mse(k, R, centroids32, boundaries32, lay.norm_correction)
        out[: lay.key_data_bytes] = pack_lsb(codes, lay.key_bits)
        out[lay.key_data_bytes : lay.key_data_bytes + 2] = _u16_le(fp16_bits(gamma))
    o = lay.key_packed_size
    if lay.value_lm:
        vcent, vbound = value_tables(lay)
        vc, gv = quantize_key_mse(v, R, vcent, vbound, True)
        out[o : o + lay.value_data_bytes] = pack_lsb(vc, lay.value_bits)
        o += lay.value_data_bytes
        out[o : o + 2] = _u16_le(fp16_bits(gv))
        return out
    vc, s16, z16 = quantize_values(v, lay.value_bits)
    out[o : o + lay.value_data_bytes] = pack_lsb(vc, lay.value_bits)
    o += lay.value_data_bytes
    out[o : o + 2] = _u16_le(s16)
    out[o + 2 : o + 4] = _u16_le(z16)
    return out


def encode_slots(lay: Layout, K, V, R, centroids32, boundaries32) -> np.ndarray:
    """``encode_slot`` applied to every row of K, V (R rows x D), the same
    steps written over arrays of rows.  Returns (rows, slot_size_aligned)."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    rows, D = K.shape
    out = np.zeros((rows, lay.slot_size_aligned), dtype=np.uint8)
    if lay.key_fp8:
        out[:, :D] = fp8_e4m3fn_encode(K)
    else:
        nu = np.sqrt(np.sum(K * K, axis=1))
        with np.errstate(invalid="ignore", divide="ignore"):
            U = np.where(nu[:, None] > 0, (K @ R.T) / nu[:, None], 0.0)
        codes = (np.asarray(boundaries32, np.float64)[None, None, :] < U[:, :, None]).sum(axis=2)
        chat = np.asarray(centroids32, dtype=np.float64)[codes]
        r = np.sqrt(np.sum(chat * chat, axis=1))
        with np.errstate(invalid="ignore", divide="ignore"):
            gamma = np.where(nu > 0, nu / r if lay.norm_correction else nu, 0.0)
        out[:, : lay.key_data_bytes] = pack_lsb(codes, lay.key_bits)
        out[:, lay.key_data_bytes : lay.key_data_bytes + 2] = _u16_le(fp16_bits(gamma))
    if lay.value_lm:  # the steps of quantize_key_mse on the value rows
        vcent, vbound = value_tables(lay)
        nu = np.sqrt(np.sum(V * V, axis=1))
        with np.errstate(invalid="ignore", divide="ignore"):
            U = np.where(nu[:, None] > 0, (V @ R.T) / nu[:, None], 0.0)
        vc = (np.asarray(vbound, np.float64)[None, None, :] < U[:, :, None]).sum(axis=2)
        chat = np.asarray(vcent, dtype=np.float64)[vc]
        with np.errstate(invalid="ignore", divide="ignore"):
            gv = np.where(nu > 0, nu / np.sqrt(np.sum(chat * chat, axis=1)), 0.0)
        o = lay.key_packed_size
        out[:, o : o + lay.value_data_bytes] = pack_lsb(vc, lay.value_bits)
        o += lay.value_data_bytes
        out[:, o : o + 2] = _u16_le(fp16_bits(gv))
        return out
    # values: the steps of quantize_values, per row
    s16, z16 = _value_scale_zero(V.min(axis=1), V.max(axis=1), lay.value_bits)
    vc = value_codes(V, z16.astype(np.float64), s16.astype(np.float64), lay.value_bits)
    o = lay.key_packed_size
    out[:, o : o + lay.value_data_bytes] = pack_lsb(vc, lay.value_bits)
    o += lay.value_data_bytes
    out[:, o : o + 2] = _u16_le(s16.view(np.uint16))
    out[:, o + 2 : o + 4] = _u16_le(z16.view(np.uint16))
    return out


def key_units(lay: Layout, K, R):
    """The rotated, normalized key coordinates u = R k / ||k|| of every row
    (float64), the quantity each key code is decided on."""
    K = np.asarray(K, dtype=np.float64)
    nu = np.sqrt(np.sum(K * K, axis=1))
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(nu[:, None] > 0, (K @ R.T) / nu[:, None], 0.0)


def store_rows(lay: Layout, key, value, slot_mapping, kv_cache, signs, centroids32, boundaries32):
    """``store`` with the rows encoded by ``encode_slots``."""
    key = np.asarray(key, dtype=np.float64)
    value = np.asarray(value, dtype=np.float64)
    N, Hk, D = key.shape
    bs = kv_cache.shape[1]
    R = rotation(np.asarray(signs, dtype=np.float64)) if needs_rotation(lay) else None
    if N == 0:
        return kv_cache
    slots = encode_slots(lay, key.reshape(N * Hk, D), value.reshape(N * Hk, D), R, centroids32,
                         boundaries32).reshape(N, Hk, lay.slot_size_aligned)
    m = np.asarray(slot_mapping, dtype=np.int64)
    keep = m >= 0
    kv_cache[m[keep] // bs, m[keep] % bs] = slots[keep]
    return kv_cache


def store(lay: Layout, key, value, slot_mapping, kv_cache, signs, centroids32, boundaries32):
    """Quantize N tokens x Hk heads and write their slots into the paged cache.

    key, value: (N, Hk, D) float64; slot_mapping: (N,) int, negative = skip
    (reading R19); kv_cache: (num_blocks, block_size, Hk, slot_aligned) uint8,
    modified in place.  Slot m lives at cache[m // bs, m % bs, h]
    ([API] do_kv_cache_update; [PR] turboquant_attn.py excerpt, cache layout).
    Returns kv_cache.
    """
    key = np.asarray(key, dtype=np.float64)
    value = np.asarray(value, dtype=np.float64)
    N, Hk, D = key.shape
    bs = kv_cache.shape[1]
    R = rotation(np.asarray(signs, dtype=np.float64)) if needs_rotation(lay) else None
    for n in range(N):
        m = int(slot_mapping[n])
        if m < 0:
            continue
        for h in range(Hk):
            kv_cache[m // bs, m % bs, h, :] = encode_slot(lay, key[n, h], value[n, h], R, centroids32, boundaries32)
    return kv_cache


# --------------------------------------------------------------------------
# SoA block layout
# --------------------------------------------------------------------------
#
# The pages' gfx950 path writes the cache in a second byte convention with
# the same tensor shape ([API] _store_kv: data region and metadata region
# separated per block, shape identical to the combined-slot store; [API]
# forward: a cache written that way must be read by the matching decode, the
# combined-slot reader takes norm, scale and zero from the wrong offsets;
# [API] _continuation_prefill: the reader's constants -- data bytes per slot
# = key data + value data, metadata region offset = block_size * Hk * data
# bytes per slot, 3 fields for MSE keys (norm 0, scale 1, zero 2) and 2 for
# FP8 keys (scale 0, zero 1)).
#
# Readings (the pages give only those constants): rows inside each region
# keep the combined cache's token-major order, row r = t * Hk + h; data row r
# is [key data | value data] at r * data_bytes; field f of row r is the
# little-endian u16 at meta_offset + 2 * (r * fields + f).


def soa_geometry(lay: Layout, block_size: int, num_kv_heads: int):
    """(data bytes per row, metadata region offset, u16 fields per row).
    Lloyd-Max values carry one field (their norm) where uniform values carry
    two (scale, zero); this extends the pages' field list to that codec."""
    data = lay.key_data_bytes + lay.value_data_bytes
    fields = (0 if lay.key_fp8 else 1) + (1 if lay.value_lm else 2)
    return data, block_size * num_kv_heads * data, fields


def _slot_fields(lay: Layout):
    """Byte offsets, inside a combined slot, of the u16 metadata fields in
    SoA field order."""
    vfields = lay.key_packed_size + lay.value_data_bytes
    keyn = [] if lay.key_fp8 else [lay.key_data_bytes]
    return keyn + ([vfields] if lay.value_lm else [vfields, vfields + 2])


def soa_from_aos(lay: Layout, kv_cache):
    """Combined-slot cache (num_blocks, bs, Hk, slot) -> the same cache in
    the SoA convention (new array of the same shape and dtype uint8)."""
    c = np.asarray(kv_cache, dtype=np.uint8)
    nb, bs, Hk, slot = c.shape
    data, meta, nf = soa_geometry(lay, bs, Hk)
    rows = c.reshape(nb, bs * Hk, slot)  # row r = t * Hk + h
    out = np.zeros((nb, bs * Hk * slot), np.uint8)
    kd, vd, kps = lay.key_data_bytes, lay.value_data_bytes, lay.key_packed_size
    for r in range(bs * Hk):
        out[:, r * data : r * data + kd] = rows[:, r, :kd]
        out[:, r * data + kd : (r + 1) * data] = rows[:, r, kps : kps + vd]
        for f, o in enumerate(_slot_fields(lay)):
            a = meta + 2 * (r * nf + f)
            out[:, a : a + 2] = rows[:, r, o : o + 2]
    return out.reshape(nb, bs, Hk, slot)


def aos_from_soa(lay: Layout, kv_cache):
    """Inverse of ``soa_from_aos`` (slot padding bytes, if any, read 0)."""
    c = np.asarray(kv_cache, dtype=np.uint8)
    nb, bs, Hk, slot = c.shape
    data, meta, nf = soa_geometry(lay, bs, Hk)
    flat = c.reshape(nb, bs * Hk * slot)
    out = np.zeros((nb, bs * Hk, slot), np.uint8)
    kd, vd, kps = lay.key_data_bytes, lay.value_data_bytes, lay.key_packed_size
    for r in range(bs * Hk):
        out[:, r, :kd] = flat[:, r * data : r * data + kd]
        out[:, r, kps : kps + vd] = flat[:, r * data + kd : (r + 1) * data]
        for f, o in enumerate(_slot_fields(lay)):
            a = meta + 2 * (r * nf + f)
            out[:, r, o : o + 2] = flat[:, a : a + 2]
    return out.reshape(nb, bs, Hk, slot)


def store_soa(lay: Layout, key, value, slot_mapping, kv_cache, signs, centroids32, boundaries32):
    """``store`` into a cache held in the SoA convention (in place)."""
    aos = aos_from_soa(lay, kv_cache)
    store_rows(lay, key, value, slot_mapping, aos, signs, centroids32, boundaries32)
    kv_cache[...] = soa_from_aos(lay, aos)
    return kv_cache


# --------------------------------------------------------------------------
# Dequantization and decode attention
# --------------------------------------------------------------------------


def decode_slot(lay: Layout, slot, centroids32, R=None):
    """Slot bytes -> (key, value) in float64.

    MSE keys are returned in the rotated domain, k' = γ·c[code]; FP8 keys as
    decoded.  Values are v = zero + scale·code from the stored fp16 fields;
    Lloyd-Max values are v = R^T (γ_v c_v[code]) in the original space (R
    is then required).
    """
    slot = np.asarray(slot, dtype=np.uint8)
    D = lay.head_dim
    if lay.key_fp8:
        k = fp8_e4m3fn_decode(slot[:D])
    else:
        codes = unpack_lsb(slot[: lay.key_data_bytes], lay.key_bits, D)
        gamma = float(np.uint16(_from_u16_le(slot[lay.key_data_bytes : lay.key_data_bytes + 2])).view(np.float16))
        k = gamma * np.asarray(centroids32, dtype=np.float64)[codes]
    o = lay.key_packed_size
    vc = unpack_lsb(slot[o : o + lay.value_data_bytes], lay.value_bits, D)
    o += lay.value_data_bytes
    if lay.value_lm:
        gv = float(np.uint16(_from_u16_le(slot[o : o + 2])).view(np.float16))
        return k, (gv * np.asarray(value_tables(lay)[0], dtype=np.float64)[vc]) @ R
    s = float(np.uint16(_from_u16_le(slot[o : o + 2])).view(np.float16))
    z = float(np.uint16(_from_u16_le(slot[o + 2 : o + 4])).view(np.float16))
    return k, z + s * vc.astype(np.float64)


def decode_slots(lay: Layout, slots, centroids32, R=None):
    """``decode_slot`` applied to every row of slots (rows, slot bytes)."""
    slots = np.asarray(slots, dtype=np.uint8)
    D = lay.head_dim
    if lay.key_fp8:
        K = fp8_e4m3fn_decode(slots[:, :D])
    else:
        codes = unpack_lsb(slots[:, : lay.key_data_bytes], lay.key_bits, D)
        gamma = _from_u16_le(slots[:, lay.key_data_bytes : lay.key_data_bytes + 2]).view(np.float16).astype(np.float64)
        K = gamma[:, None] * np.asarray(centroids32, dtype=np.float64)[codes]
    o = lay.key_packed_size
    vc = unpack_lsb(slots[:, o : o + lay.value_data_bytes], lay.value_bits, D)
    o += lay.value_data_bytes
    if lay.value_lm:
        gv = _from_u16_le(slots[:, o : o + 2]).view(np.float16).astype(np.float64)
        return K, (gv[:, None] * np.asarray(value_tables(lay)[0], dtype=np.float64)[vc]) @ R
    s = _from_u16_le(slots[:, o : o + 2]).view(np.float16).astype(np.float64)
    z = _from_u16_le(slots[:, o + 2 : o + 4]).view(np.float16).astype(np.float64)
    return K, z[:, None] + s[:, None] * vc.astype(np.float64)


def gather_sequence(lay: Layout, kv_cache, block_table_row, seq_len: int, hk: int, centroids32, R=None):
    """Dequantize tokens [0, seq_len) of one sequence and KV head.  Token t is
    in block block_table_row[t // bs] at offset t % bs; entries past
    ceil(seq_len / bs) are never read ([TRACK]: decode index-out-of-bounds
    fix)."""
    bs = kv_cache.shape[1]
    t = np.arange(seq_len)
    blk = np.asarray(block_table_row, dtype=np.int64)[t // bs]
    if seq_len == 0:
        return np.zeros((0, lay.head_dim)), np.zeros((0, lay.head_dim))
    return decode_slots(lay, kv_cache[blk, t % bs, hk], centroids32, R)


def attend(q, K, V, scale: float, sink: float = -math.inf):
    """Textbook softmax attention of one query over (K, V), float64.
    Returns (o, lse) with lse = log sum exp(scores); empty K gives (0, -inf).

    sink: an attention-sink logit ([API] TurboQuantAttentionImpl.__init__
    and _decode_attention pass per-head ``sinks`` to the decode kernel).
    Reading: the sink is one more logit in the softmax denominator, in the
    units of the scaled scores, with no value: o = sum_t e^{s_t} v_t /
    (sum_t e^{s_t} + e^{sink}), lse = log(sum_t e^{s_t} + e^{sink});
    -inf is no sink."""
    s = scale * (K @ q) if K.shape[0] else np.zeros(0)
    m = max(s.max() if len(s) else -math.inf, sink)
    if m == -math.inf:
        return np.zeros(V.shape[1]), -math.inf
    p = np.exp(s - m)
    l = p.sum() + math.exp(sink - m)
    return (p @ V) / l if len(s) else np.zeros(V.shape[1]), m + math.log(l)


def attend_sparse_v(q, K, V, scale: float, gate: float, sink: float = -math.inf):
    """Attention with the sparse-V gate of [TQ+] "nvfp4 dec_after_8K cliff
    explained": a token whose softmax factor exp(s_t - max) is below the gate
    adds no value; its weight stays in the denominator (only the value side
    is skipped), so the lse is the exact one.  Here max is the maximum over
    all of the query's scores (the sink excluded, as it has no value row).
    Returns (o, lse, bound): bound[d] = sum over gated tokens of
    e^{s_t - max} |V[t, d]| / L, L the exact denominator, bounds how far any
    result that drops only gated tokens' values can be from exact attention
    in dim d -- in particular one gated against a running maximum, which
    never exceeds this max, so it drops a subset of these tokens."""
    o, lse = attend(q, K, V, scale, sink)
    D = V.shape[1]
    if K.shape[0] == 0 or lse == -math.inf:
        return o, lse, np.zeros(D)
    s = scale * (K @ q)
    M = s.max()
    f = np.exp(s - M)
    L = math.exp(lse - M)  # the exact denominator in units of e^M, sink included
    drop = f < gate
    o_gated = (f[~drop] @ V[~drop]) / L
    bound = (f[drop] @ np.abs(V[drop])) / L
    return o_gated, lse, bound


def window_start(seq_len: int, sliding_window: int) -> int:
    """First token a decode query attends to ([API] TurboQuantAttentionImpl.__init__
    takes ``sliding_window``; _decode_attention passes it to the decode
    kernel).  Reading: the query (the sequence's last token) sees the last
    ``sliding_window`` tokens, itself included; 0 or None means no window."""
    if not sliding_window or sliding_window <= 0:
        return 0
    return max(0, seq_len - sliding_window)


def decode(lay: Layout, query, kv_cache, block_table, seq_lens, signs, centroids32, scale: float, rows=None,
           sliding_window: int = 0, sinks=None):
    """Decode attention of one query per sequence over the compressed cache.

    query: (B, Hq, D) float64.  GQA: query head hq reads KV head hq // g with
    g = Hq / Hk ([API] TurboQuantAttentionImpl.__init__, num_kv_groups).
    MSE keys: the query is rotated by the same R and scored in the rotated
    domain, s_t = scale·(R q)·(γ_t c[code_t]); FP8 keys: s_t = scale·q·k_t
    ([API] _decode_attention passes the rotation to the decode kernel; [API]
    _continuation_prefill: only MSE keys are ever inverse-rotated).  Output
    = exact softmax attention over the dequantized cache (the split-KV +
    log-sum-exp merge of the kernels is a faster route to the same value).
    ``rows``: optional iterable of (b, hq) to compute; others stay NaN.
    ``sliding_window`` / ``sinks`` (Hq logits): see ``window_start`` and
    ``attend``.
    Returns (out (B,Hq,D), lse (B,Hq)).
    """
    query = np.asarray(query, dtype=np.float64)
    B, Hq, D = query.shape
    Hk = kv_cache.shape[2]
    g = Hq // Hk
    R = rotation(np.asarray(signs, dtype=np.float64)) if needs_rotation(lay) else None
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    want = {(b, h) for b in range(B) for h in range(Hq)} if rows is None else set(rows)
    cache = {}
    for b, hq in sorted(want):
        hk = hq // g
        if (b, hk) not in cache:
            cache = {(b, hk): gather_sequence(lay, kv_cache, block_table[b], int(seq_lens[b]), hk, centroids32, R)}
        K, V = cache[(b, hk)]
        f = window_start(int(seq_lens[b]), sliding_window)
        q = query[b, hq] if lay.key_fp8 else R @ query[b, hq]
        sink = -math.inf if sinks is None else float(sinks[hq])
        out[b, hq], lse[b, hq] = attend(q, K[f:], V[f:], scale, sink)
    return out, lse


def split_ranges(seq_len: int, num_splits: int, block_size: int):
    """Token ranges of the S splits: chunk = ceil(ceil(L / S) / bs) * bs
    (reading R16; splits after the end are empty)."""
    per = -(-seq_len // num_splits) if seq_len > 0 else 0
    chunk = -(-per // block_size) * block_size
    return [(min(s * chunk, seq_len), min((s + 1) * chunk, seq_len)) for s in range(num_splits)]


def merge_partials(parts, sink: float = -math.inf):
    """Log-sum-exp merge of (o_s, lse_s) partials, o_s normalized within its
    split: M = max lse_s, w_s = exp(lse_s - M), o = sum w_s o_s / sum w_s,
    lse = M + log sum w_s; empty partials (lse = -inf) drop out ([PR]
    "实现拆解" item 4: stage 2 performs the log-sum-exp reduction).  A sink
    logit joins the merge as one more weight with a zero output."""
    live = [(o, l) for o, l in parts if l != -math.inf]
    if sink != -math.inf:
        live.append((np.zeros_like(parts[0][0]), sink))
    if not live:
        return np.zeros_like(parts[0][0]), -math.inf
    M = max(l for _, l in live)
    w = np.array([math.exp(l - M) for _, l in live])
    o = sum(wi * oi for wi, (oi, _) in zip(w, live)) / w.sum()
    return o, M + math.log(w.sum())


def decode_split(q_rot, K, V, scale: float, num_splits: int, block_size: int, sink: float = -math.inf):
    """Stage 1 per split then stage 2, for one query over one sequence/head."""
    parts = [attend(q_rot, K[a:b], V[a:b], scale) for a, b in split_ranges(K.shape[0], num_splits, block_size)]
    return merge_partials(parts, sink)


def dequant_original_space(lay: Layout, kv_cache, block_table_row, seq_len: int, hk: int, signs, centroids32):
    """Cached prefix back to the original space: K = R^T (γ c[code]) for MSE
    keys, FP8 keys as decoded; V = zero + scale·code ([API]
    _continuation_prefill: dequantize the prefix, inverse-rotate MSE keys
    only)."""
    R = rotation(np.asarray(signs, dtype=np.float64)) if needs_rotation(lay) else None
    K, V = gather_sequence(lay, kv_cache, block_table_row, seq_len, hk, centroids32, R)
    if not lay.key_fp8:
        K = K @ R
    return K, V


def workspace_bytes(batch: int, num_q_heads: int, head_dim: int, num_kv_splits: int) -> int:
    """Bytes of the pages' stage-1 scratch: (B, Hq, S, D+1) fp32, the
    split's partial output and its LSE ([PR] attention.py excerpt, the mid_o
    buffer; [API] _decode_attention).  A decode workspace must hold at least
    this much partial state."""
    return batch * num_q_heads * num_kv_splits * (head_dim + 1) * 4
