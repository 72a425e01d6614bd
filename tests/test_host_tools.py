"""Host-side checks of the profile bookkeeping (mla_latent_kv_30_amd/traffic.py):
a counter summary is tied to the code of the sources its kernel is built
from, so an edit to comments leaves it valid and an edit to code does not."""

import os

from mla_latent_kv_30_amd import traffic as T


def test_code_text_drops_comments_and_whitespace_only():
    a = "int f(int x) {  // the input\n  return x + 1; /* one\n more */ }\n"
    b = "int f(int x)\n{\n\treturn x + 1;\n}"
    assert T.code_text(a) == T.code_text(b)
    assert T.code_text("return x + 1;") != T.code_text("return x - 1;")
    assert T.code_text("a /* x */ b") != T.code_text("ab")


def _write(d, name, text):
    with open(os.path.join(d, "csrc", name), "w") as f:
        f.write(text)


def test_source_digest_follows_the_kernels_own_sources(tmp_path, monkeypatch):
    d = str(tmp_path)
    os.makedirs(os.path.join(d, "csrc"))
    monkeypatch.setattr(T, "HERE", d)
    for name in ("decode.hip", "decode_common.h", "common.h", "kernels.h", "linear.hip"):
        _write(d, name, f"// {name}\nint v_{name.split('.')[0]} = 1;\n")
    dec, lin = T.source_digest("decode_mfma_kernel"), T.source_digest("linear_kernel")
    # a comment edit changes neither
    _write(d, "decode.hip", "// reworded\nint v_decode  =  1;  // same code\n")
    assert T.source_digest("decode_mfma_kernel") == dec
    # a code edit in decode.hip changes the decode digest only
    _write(d, "decode.hip", "int v_decode = 2;\n")
    assert T.source_digest("decode_mfma_kernel") != dec
    assert T.source_digest("linear_kernel") == lin
    # a shared header changes both
    _write(d, "common.h", "int v_common = 3;\n")
    assert T.source_digest("linear_kernel") != lin
