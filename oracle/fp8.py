"""FP8 E4M3 ("fn" variant) decoding table, written from the format definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The decode API page ("FlashInfer attention kernels", flashinfer.decode ›
BatchDecodeWithPagedKVCacheWrapper › run(), parameters k_scale / v_scale) says
fp8 key/value inputs carry a calibration scale; the XQA entry on the same page
names torch.float8_e4m3fn as the fp8 KV dtype. The format is the OCP 8-bit
floating point E4M3 encoding:

* bit 7 is the sign, bits 6..3 the biased exponent (bias 7), bits 2..0 the
  mantissa;
* exponent field 0 encodes subnormals: value = mantissa * 2**-9;
* exponent field 1..15 encodes normals: value = (1 + mantissa/8) * 2**(e-7);
* the single pattern with exponent 15 and mantissa 7 (0x7F / 0xFF) is NaN;
  there is no infinity, so the largest finite magnitude is 448 (0x7E).

The real value of a stored code c is ``scale * value(c)``; the scale is applied
by the caller (oracle.widen).

Parity pin: tests/test_oracle.py compares all 256 entries with the library
routine ``torch.float8_e4m3fn -> float32`` and checks spot values of the format.
"""
import numpy as np


def _decode_code(c: int) -> float:
    sign = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_decode_code(c) for c in range(256)], dtype=np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact fp64 values of an array of uint8 E4M3 codes (unscaled)."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("E4M3 codes must be uint8")
    return E4M3_TABLE[codes]
