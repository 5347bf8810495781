"""ctypes access to libtq_probe.so (test-only kernels and the host model of
the kernels' bit helpers)."""

import ctypes
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = os.path.join(ROOT, "quantized_decode_attention_tq_amd", "libtq_probe.so")

N_IN, N_OUT = 12, 8
OPS = {"perm": 0, "alignbyte": 1, "key3_selectors": 2, "lut8": 3, "lut16": 4, "val4_pairs": 5, "val3_pairs": 6,
       "f32_to_e4m3": 7, "val2_pairs": 8, "key2_selectors": 9, "lm_value_selectors": 10,
       "key3_pair_fields": 11, "key3_pair_entries": 12,
       "key3_pair_windows": 13, "lm4_value_selectors": 14, "lm2_value_selectors": 15}


def lib():
    if not os.path.exists(PATH):
        raise ImportError(f"{PATH} missing; build with python quantized_decode_attention_tq_amd/build.py")
    import torch  # noqa: F401  (load torch's HIP runtime first, so the probe library shares it)

    L = ctypes.CDLL(PATH)
    vp = ctypes.c_void_p
    for name, args in (("tq_probe_bits_host", [ctypes.c_int, vp, vp, ctypes.c_int]),
                       ("tq_probe_bits_device", [ctypes.c_int, vp, vp, ctypes.c_int]),
                       ("tq_probe_mfma_16x16x32_f16", [vp, vp, vp]),
                       ("tq_probe_mfma_16x16x16_f16", [vp, vp, vp]),
                       ("tq_probe_cvt_fp8_f16", [vp, vp, ctypes.c_int]),
                       ("tq_probe_permlane_swap", [vp, vp]),
                       ("tq_probe_wave_ops", [vp, vp, ctypes.c_int]),
                       ("tq_probe_fp8_encode", [vp, vp, ctypes.c_int]),
                       ("tq_probe_stream_read", [vp, ctypes.c_int64, ctypes.c_int64, vp, vp]),
                       ("tq_probe_copy", [vp, vp, ctypes.c_int64, ctypes.c_int, vp]),
                       ("tq_probe_gather_read", [vp, vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int64, ctypes.c_int, vp, vp])):
        f = getattr(L, name)
        f.restype = ctypes.c_int
        f.argtypes = args
    return L


def bits_host(op: str, inputs: np.ndarray) -> np.ndarray:
    """inputs: (n, <=12) uint32 -> (n, 8) uint32 from the host model."""
    n = inputs.shape[0]
    inp = np.zeros((n, N_IN), np.uint32)
    inp[:, : inputs.shape[1]] = inputs
    out = np.zeros((n, N_OUT), np.uint32)
    assert lib().tq_probe_bits_host(OPS[op], inp.ctypes.data, out.ctypes.data, n) == 0
    return out


def bits_device(op: str, inputs: np.ndarray) -> np.ndarray:
    import torch

    n = inputs.shape[0]
    inp = np.zeros((n, N_IN), np.uint32)
    inp[:, : inputs.shape[1]] = inputs
    din = torch.from_numpy(inp.view(np.int32)).cuda()
    dout = torch.zeros((n, N_OUT), dtype=torch.int32, device="cuda")
    assert lib().tq_probe_bits_device(OPS[op], din.data_ptr(), dout.data_ptr(), n) == 0
    return dout.cpu().numpy().view(np.uint32)
