"""Python binding of libtq, the TurboQuant KV-cache store / decode-attention
library for AMD MI355X (gfx950).

Argument marshalling only: every step of the store and of decode attention
runs in the library's HIP kernels.  PyTorch supplies device memory and the
current stream.  The binding raises ``ImportError`` when libtq.so has not
been built (``python quantized_decode_attention_tq_amd/build.py``) and
``TQError`` when the library rejects a call; there is no fallback path.

The functions carry the names of the C ABI (include/tq.h) without the
``tq_`` prefix.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK, TQ_EINVAL, TQ_EPRESET, TQ_EHEADDIM, TQ_EBLOCK, TQ_EGQA, TQ_EWORKSPACE, TQ_EDTYPE, TQ_EHIP, TQ_EUNSUPPORTED = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9)
TQ_F16, TQ_BF16, TQ_F32 = 0, 1, 2
#: every preset of include/tq.h, in preset-id order
PRESETS = ("turboquant_k8v4", "turboquant_4bit_nc", "turboquant_k3v4_nc", "turboquant_3bit_nc", "turboquant_k8v3",
           "turboquant_k4v3_nc", "turboquant_2bit_nc", "turboquant_k8v3lm", "turboquant_3bit_lm",
           "turboquant_k8v4lm", "turboquant_4bit_lm", "turboquant_2bit_lm")

#: every symbol include/tq.h declares
ABI_SYMBOLS = ("tq_version", "tq_status_str", "tq_last_hip_error", "tq_preset_from_name", "tq_layout_init",
               "tq_layout_init_ex", "tq_kv_cache_shape",
               "tq_lloyd_max", "tq_wht_signs", "tq_decode_workspace_bytes", "tq_store", "tq_store_validate",
               "tq_decode_attention", "tq_decode_validate", "tq_decode_stage1", "tq_decode_stage2",
               "tq_decode_attention_noalloc", "tq_dequant_kv", "tq_dequant_validate")


class TQError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: {_lib.tq_status_str(status).decode()} (status {status})"
        if status == TQ_EHIP:
            msg += f": {_lib.tq_last_hip_error().decode()}"
        super().__init__(msg)
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "preset", "head_dim", "key_fp8", "key_bits", "value_bits", "norm_correction", "n_centroids",
        "key_data_bytes", "key_packed_size", "value_data_bytes", "value_packed_size", "slot_size",
        "slot_size_aligned", "block_layout", "soa_data_bytes", "soa_meta_fields", "value_lloyd_max")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with: python quantized_decode_attention_tq_amd/build.py")
    # PyTorch ships its own HIP runtime under the same soname as ROCm's
    # (libamdhip64.so.7).  Importing torch first makes libtq.so bind to that
    # already-loaded runtime, so the process has one HIP runtime: torch's
    # streams, events and graph capture then see libtq's launches.  Loaded
    # the other way round, the process would hold two runtimes.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, u64, sz, vp, fp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p,
                                 ctypes.c_float)
    L = ctypes.POINTER(Layout)
    sig = {
        "tq_version": (ctypes.c_char_p, []),
        "tq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "tq_last_hip_error": (ctypes.c_char_p, []),
        "tq_preset_from_name": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(i32)]),
        "tq_layout_init": (ctypes.c_int, [i32, i32, L]),
        "tq_layout_init_ex": (ctypes.c_int, [i32, i32, i32, L]),
        "tq_kv_cache_shape": (ctypes.c_int, [L, i64, i32, i32, ctypes.POINTER(i64)]),
        "tq_lloyd_max": (ctypes.c_int, [i32, i32, i32, vp, vp]),
        "tq_wht_signs": (ctypes.c_int, [i32, u64, vp]),
        "tq_decode_workspace_bytes": (ctypes.c_int, [i32, i32, i32, i32, ctypes.POINTER(sz)]),
        "tq_store": (ctypes.c_int, [L, vp, vp, i32, i64, i32, i64, i64, vp, vp, i64, i32, vp, vp, vp, vp]),
        "tq_store_validate": (ctypes.c_int, [L, vp, vp, i32, i64, i32, i64, i64, vp, vp, i64, i32, vp, vp, vp]),
        "tq_decode_attention": (ctypes.c_int, [L, vp, i32, i32, i32, i32, vp, i64, i32, vp, i32, vp, vp, vp, fp, i32,
                                               i32, fp, vp, vp, sz, vp, i32, vp, vp]),
        "tq_decode_validate": (ctypes.c_int, [L, vp, i32, i32, i32, i32, vp, i64, i32, vp, i32, vp, vp, vp, i32, i32,
                                              fp, vp, sz, vp, i32]),
        "tq_decode_stage1": (ctypes.c_int, [L, vp, i32, i32, i32, i32, vp, i64, i32, vp, i32, vp, vp, vp, fp, i32, i32,
                                            fp, vp, sz, vp]),
        "tq_decode_stage2": (ctypes.c_int, [i32, i32, i32, i32, vp, vp, sz, vp, i32, vp, vp]),
        "tq_decode_attention_noalloc": (ctypes.c_int, [L, vp, i32, i32, i32, i32, vp, i64, i32, vp, i32, vp, vp, vp,
                                                       fp, i32, i32, fp, vp, vp, i32, vp, vp]),
        "tq_dequant_kv": (ctypes.c_int, [L, vp, i64, i32, i32, vp, i32, vp, vp, vp, vp, i32, i64, vp]),
        "tq_dequant_validate": (ctypes.c_int, [L, vp, i64, i32, i32, vp, i32, vp, vp, vp, vp, i32, i64]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def _check(status: int, where: str) -> None:
    if status != TQ_OK:
        raise TQError(status, where)


# --------------------------------------------------------------------- host


def version() -> str:
    return _lib.tq_version().decode()


def status_str(status: int) -> str:
    return _lib.tq_status_str(status).decode()


def preset_from_name(name: str) -> int:
    p = ctypes.c_int32()
    _check(_lib.tq_preset_from_name(name.encode(), ctypes.byref(p)), "tq_preset_from_name")
    return p.value


LAYOUT_AOS, LAYOUT_SOA = 0, 1


def layout_init(preset, head_dim: int = 128, block_layout="aos") -> Layout:
    """tq_layout_init_ex; block_layout "aos" (combined slots) or "soa" (data
    region + metadata region per block), or the tq_block_layout id."""
    if isinstance(preset, str):
        preset = preset_from_name(preset)
    if isinstance(block_layout, str):
        block_layout = {"aos": LAYOUT_AOS, "soa": LAYOUT_SOA}[block_layout]
    lay = Layout()
    _check(_lib.tq_layout_init_ex(preset, head_dim, block_layout, ctypes.byref(lay)), "tq_layout_init_ex")
    return lay


def kv_cache_shape(layout: Layout, num_blocks: int, block_size: int, num_kv_heads: int):
    out = (ctypes.c_int64 * 4)()
    _check(_lib.tq_kv_cache_shape(ctypes.byref(layout), num_blocks, block_size, num_kv_heads, out), "tq_kv_cache_shape")
    return tuple(out)


def lloyd_max(d: int, bits: int, mode: int = 0):
    """(centroids, boundaries) fp32 numpy arrays; mode 0 exact, 1 pages' trapezoid."""
    c = np.zeros(1 << bits, np.float32)
    b = np.zeros((1 << bits) - 1, np.float32)
    _check(_lib.tq_lloyd_max(d, bits, mode, c.ctypes.data, b.ctypes.data), "tq_lloyd_max")
    return c, b


def wht_signs(d: int, seed: int) -> np.ndarray:
    s = np.zeros(d, np.float32)
    _check(_lib.tq_wht_signs(d, seed & 0xFFFFFFFFFFFFFFFF, s.ctypes.data), "tq_wht_signs")
    return s


def decode_workspace_bytes(batch: int, num_q_heads: int, head_dim: int, num_kv_splits: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.tq_decode_workspace_bytes(batch, num_q_heads, head_dim, num_kv_splits, ctypes.byref(n)),
           "tq_decode_workspace_bytes")
    return n.value


# --------------------------------------------------------------------- device


def _torch():
    import torch

    return torch


def _dt(t) -> int:
    torch = _torch()
    m = {torch.float16: TQ_F16, torch.bfloat16: TQ_BF16, torch.float32: TQ_F32}
    if t.dtype not in m:
        raise TQError(TQ_EDTYPE, f"dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def store(layout: Layout, key, value, slot_mapping, kv_cache, signs=None, centroids=None, boundaries=None,
          stream=None) -> None:
    """Quantize key/value rows (N, Hk, D) or (N, Hk*D) and write their slots.

    key/value: fp16 or bf16 CUDA tensors whose last dim is contiguous and
    whose heads are contiguous within a token; slot_mapping: int64 (N,);
    kv_cache: uint8 (num_blocks, block_size, Hk, slot_size_aligned)."""
    N = slot_mapping.shape[0]
    Hk = kv_cache.shape[2]
    D = layout.head_dim
    for t in (key, value):
        if t.stride(-1) != 1 or (t.dim() == 3 and t.stride(1) != D):
            raise TQError(TQ_EINVAL, "store: heads must be contiguous within a token")
    if key.dtype != value.dtype:
        raise TQError(TQ_EDTYPE, "store: key and value dtypes differ")
    _check(_lib.tq_store(ctypes.byref(layout), key.data_ptr(), value.data_ptr(), _dt(key), N, Hk, key.stride(0),
                         value.stride(0), slot_mapping.data_ptr(), kv_cache.data_ptr(), kv_cache.shape[0],
                         kv_cache.shape[1], _ptr(signs), _ptr(centroids), _ptr(boundaries),
                         _stream(stream, kv_cache.device)), "tq_store")


def _decode_common(query, kv_cache, block_table):
    B, Hq, D = query.shape
    return B, Hq, kv_cache.shape[2], block_table.stride(0) if block_table.dim() == 2 else 0


def decode(layout: Layout, query, kv_cache, block_table, seq_lens, signs, centroids, scale: float,
           num_kv_splits: int, workspace=None, out=None, out_dtype=None, lse=None, stream=None,
           sliding_window: int = 0, sinks=None, value_gate: float = 0.0):
    """Decode attention; returns (out, lse).  query (B, Hq, D) fp16/bf16;
    block_table int32 (B, max_blocks); seq_lens int32 (B,); sinks fp32 (Hq,)
    or None; value_gate 0 (exact) or the opt-in sparse-V gate in (0, 1).
    Allocates the workspace, out and lse with torch when they are not
    given."""
    torch = _torch()
    B, Hq, Hk, bt_stride = _decode_common(query, kv_cache, block_table)
    D = layout.head_dim
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(B, Hq, D, num_kv_splits), dtype=torch.uint8,
                                device=query.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or query.dtype, device=query.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=query.device)
    _check(_lib.tq_decode_attention(ctypes.byref(layout), query.data_ptr(), _dt(query), B, Hq, Hk,
                                    kv_cache.data_ptr(), kv_cache.shape[0], kv_cache.shape[1], block_table.data_ptr(),
                                    bt_stride, seq_lens.data_ptr(), _ptr(signs), _ptr(centroids), float(scale),
                                    num_kv_splits, int(sliding_window), float(value_gate), _ptr(sinks),
                                    workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), out.data_ptr(), _dt(out), _ptr(lse),
                                    _stream(stream, query.device)),
           "tq_decode_attention")
    return out, lse


#: bytes of the device scratch tq_decode_attention_noalloc uses (TQ_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_noalloc(layout: Layout, query, kv_cache, block_table, seq_lens, signs, centroids, scale: float,
                   num_kv_splits: int, out, lse=None, stream=None, sliding_window: int = 0, sinks=None,
                   value_gate: float = 0.0):
    """tq_decode_attention_noalloc: decode attention into the caller's `out`
    (and `lse`, optional) with the library's own device scratch; nothing is
    allocated.  Same arguments as decode otherwise."""
    B, Hq, Hk, bt_stride = _decode_common(query, kv_cache, block_table)
    _check(_lib.tq_decode_attention_noalloc(ctypes.byref(layout), query.data_ptr(), _dt(query), B, Hq, Hk,
                                            kv_cache.data_ptr(), kv_cache.shape[0], kv_cache.shape[1],
                                            block_table.data_ptr(), bt_stride, seq_lens.data_ptr(), _ptr(signs),
                                            _ptr(centroids), float(scale), num_kv_splits, int(sliding_window),
                                            float(value_gate), _ptr(sinks), out.data_ptr(), _dt(out), _ptr(lse),
                                            _stream(stream, query.device)),
           "tq_decode_attention_noalloc")
    return out, lse


def decode_stage1(layout: Layout, query, kv_cache, block_table, seq_lens, signs, centroids, scale: float,
                  num_kv_splits: int, workspace, stream=None, sliding_window: int = 0,
                  value_gate: float = 0.0) -> None:
    B, Hq, Hk, bt_stride = _decode_common(query, kv_cache, block_table)
    _check(_lib.tq_decode_stage1(ctypes.byref(layout), query.data_ptr(), _dt(query), B, Hq, Hk, kv_cache.data_ptr(),
                                 kv_cache.shape[0], kv_cache.shape[1], block_table.data_ptr(), bt_stride,
                                 seq_lens.data_ptr(), _ptr(signs), _ptr(centroids), float(scale), num_kv_splits,
                                 int(sliding_window), float(value_gate), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream(stream, query.device)),
           "tq_decode_stage1")


def decode_stage2(batch: int, num_q_heads: int, head_dim: int, num_kv_splits: int, workspace, out, lse=None,
                  stream=None, sinks=None) -> None:
    _check(_lib.tq_decode_stage2(batch, num_q_heads, head_dim, num_kv_splits, _ptr(sinks), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), out.data_ptr(), _dt(out), _ptr(lse),
                                 _stream(stream, out.device)), "tq_decode_stage2")


def dequant_kv(layout: Layout, kv_cache, block_table, num_tokens: int, signs=None, centroids=None, key_out=None,
               value_out=None, out_dtype=None, stream=None):
    """Cached prefix of one sequence back to dense (num_tokens, Hk, D) K and V
    in the original space; returns (key_out, value_out).  block_table: int32
    (ceil(num_tokens / block_size),) block ids of the sequence.  The outputs
    may be row slices of larger (tokens, Hk, D) buffers (same token stride,
    last two dims contiguous); they are allocated with torch when not given."""
    torch = _torch()
    Hk = kv_cache.shape[2]
    D = layout.head_dim
    dt = out_dtype or torch.float16
    if key_out is None:
        key_out = torch.empty((num_tokens, Hk, D), dtype=dt, device=kv_cache.device)
    if value_out is None:
        value_out = torch.empty((num_tokens, Hk, D), dtype=dt, device=kv_cache.device)
    for t in (key_out, value_out):
        if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != D or t.shape[0] < num_tokens:
            raise TQError(TQ_EINVAL, "dequant_kv: outputs must be (tokens, Hk, D) with contiguous heads")
    if key_out.stride(0) != value_out.stride(0) or key_out.dtype != value_out.dtype:
        raise TQError(TQ_EINVAL, "dequant_kv: key_out and value_out must share dtype and token stride")
    _check(_lib.tq_dequant_kv(ctypes.byref(layout), kv_cache.data_ptr(), kv_cache.shape[0], kv_cache.shape[1], Hk,
                              block_table.data_ptr(), int(num_tokens), _ptr(signs), _ptr(centroids),
                              key_out.data_ptr(), value_out.data_ptr(), _dt(key_out), key_out.stride(0),
                              _stream(stream, kv_cache.device)), "tq_dequant_kv")
    return key_out, value_out


class Tables:
    """Per-layer tables on the device: signs (D,), centroids, boundaries (fp32),
    for a preset.  FP8-key presets carry none."""

    def __init__(self, layout: Layout, signs: np.ndarray, device="cuda", mode: int = 0):
        torch = _torch()
        self.layout = layout
        # the key codebook (MSE keys), then the value codebook (Lloyd-Max values)
        books = ([layout.key_bits] if not layout.key_fp8 else []) + ([layout.value_bits] if layout.value_lloyd_max else [])
        if not books:
            self.signs = self.centroids = self.boundaries = None
            return
        cb = [lloyd_max(layout.head_dim, bits, mode) for bits in books]
        self.signs = torch.from_numpy(np.ascontiguousarray(signs, dtype=np.float32)).to(device)
        self.centroids = torch.from_numpy(np.concatenate([c for c, _ in cb])).to(device)
        self.boundaries = torch.from_numpy(np.concatenate([b for _, b in cb])).to(device)
