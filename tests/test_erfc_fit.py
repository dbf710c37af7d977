"""The bf16 epilogues' erfc fit against scipy, on the CPU.

The fit erfc(z) = t e^{-z^2} S(t), t = 1 / (1 + p z), with S of degree 6, is
read from the device source (its constants as written there) and evaluated in
fp64; its relative error must stay below the bound the source states, for
every z up to where erfc leaves the fp64 range.  A wrong or mistyped
coefficient moves the error far above it."""
import math
import pathlib
import re

import numpy as np
import pytest
from scipy.special import erfc

SRC = pathlib.Path(__file__).resolve().parents[1] / "megatron_tensor_transformer_fwd_amd" / "csrc" / "common.hpp"


def _fit_constants():
    text = SRC.read_text()
    body = text[text.index("PhiTail phi_tail_bf16(float x)"):]
    body = body[:body.index("return PhiTail")]
    a = re.search(r"fmaf\(fabsf\(x\),\s*([0-9.]+)f\s*\*\s*([0-9.]+)f,\s*1\.0f\)", body)
    p = float(a.group(1)) * float(a.group(2))          # t = 1 / (1 + p' |x|), p' = p / sqrt 2
    c1 = float(re.search(r"x \* ([0-9.]+)f;", body).group(1))
    s0 = float(re.search(r"float s = (-?[0-9.]+)f;", body).group(1))
    rest = [float(v) for v in re.findall(r"s = fmaf\(s, t, (-?[0-9.]+)f\);", body)]
    return p, c1, [s0] + rest                          # S / 2, highest order first


def test_constants_found():
    p, c1, coef = _fit_constants()
    assert len(coef) == 7
    assert p == pytest.approx(0.395 / math.sqrt(2), rel=1e-6)
    assert c1 == pytest.approx(math.sqrt(math.log2(math.e) / 2), rel=1e-9)


def test_half_erfc_relative_error():
    p, c1, coef = _fit_constants()
    x = np.concatenate([np.linspace(0.0, 8.0, 200001), np.linspace(8.0, 37.0, 20001)])
    t = 1.0 / (1.0 + p * x)
    e = np.exp2(-(x * c1) ** 2)                        # e^{-x^2/2}
    s = np.zeros_like(x)
    for c in coef:
        s = s * t + c
    h = t * e * s
    ref = 0.5 * erfc(x / math.sqrt(2.0))
    rel = np.abs(h / ref - 1.0)
    assert rel.max() < 3.5e-6, (rel.max(), x[np.argmax(rel)])
