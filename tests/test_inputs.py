"""CPU checks of the seeded input generator's dtype and decay options and of
the binding's copy of the C descriptor layout."""
import ctypes
import os
import subprocess

import numpy as np

from linear_recurrent_lm_amd import synth
from linear_recurrent_lm_amd import wkv7 as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_log_decay_stream_is_the_log_of_the_recipe_decay():
    """Same seed, same draws: exp of the log-form w equals the multiplicative w
    of the recipe (w = exp(-exp(x))) up to fp32 rounding; everything else is equal."""
    m = synth.make_inputs(2, 9, 3, 64, seed=5, dtype="f32", with_dy=True)
    g = synth.make_inputs(2, 9, 3, 64, seed=5, dtype="f32", with_dy=True, decay="log")
    assert g.decay == "log" and m.decay == "mult"
    assert np.all(g.w < 0)
    np.testing.assert_allclose(np.exp(g.w.astype(np.float64)), m.w, rtol=3e-7)
    for n in ("r", "k", "v", "a", "b", "dy"):
        assert np.array_equal(getattr(g, n), getattr(m, n)), n


def test_f16_streams_are_exact_fp16_values():
    x = synth.make_inputs(1, 40, 2, 64, seed=6, dtype="f16", with_dy=True)
    for s in (*x.streams(), x.dy):
        assert np.array_equal(s.astype(np.float16).astype(np.float32), s)
    f = synth.make_inputs(1, 40, 2, 64, seed=6, dtype="f32", with_dy=True)
    # rounding only: within half an fp16 ulp of the fp32 draw
    for a, b in zip(x.streams(), f.streams()):
        assert np.all(np.abs(a - b) <= np.abs(b) * 2.0 ** -11 + 2.0 ** -25)
    # ties go to even
    t = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11], dtype=np.float32)
    assert list(synth.round_f16(t)) == [1.0, 1 + 4 * 2.0 ** -11]


def test_descriptor_layout_matches_header(tmp_path):
    """sizeof / offsetof of wkv7_desc from the C compiler equal the ctypes copy."""
    src = tmp_path / "layout.c"
    fields = [f for f, _ in W.Desc._fields_]
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "wkv7.h"\nint main(void) {\n'
                   '  printf("%zu", sizeof(wkv7_desc));\n'
                   + "".join(f'  printf(" %zu", offsetof(wkv7_desc, {f}));\n' for f in fields)
                   + '  return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert out[0] == ctypes.sizeof(W.Desc)
    assert out[1:] == [getattr(W.Desc, f).offset for f in fields]
