"""Rules on the library's sources that no GPU run would reliably catch.

* One matrix-core shape per accumulation chain.  A 16x16x16 bf16 product whose result
  was read as the accumulator of a 16x16x32 product one wait state later gave stale
  rows 2-3 on gfx950 -- only when two wavefronts competed for the matrix pipe, so a
  parity run can pass with it.  Every product in the kernels therefore goes through the
  wrappers of csrc/mfma_tile.h, which issue v_mfma_f32_16x16x32_bf16 only (a k=16
  product is a zero-padded k=32 one); no other MFMA builtin and no MFMA written in
  inline assembly may appear anywhere in csrc/.
* Packed fp32 arithmetic stays out of the generated code: the build disables the
  feature, and no source spells the packed add / multiply / FMA instructions by hand.
* The product path never imports, links or executes the oracle.
"""
import ast
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sliding_window_attention_amd")
CSRC = os.path.join(PKG, "csrc")


def _sources():
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h", ".cpp", ".hpp")):
            with open(os.path.join(CSRC, f)) as fh:
                yield f, fh.read()


def _strip_comments(text):
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.sub(r"//[^\n]*", "", text)


def test_every_mfma_is_the_16x16x32_bf16_wrapper():
    allowed = "__builtin_amdgcn_mfma_f32_16x16x32_bf16"
    seen = 0
    for name, text in _sources():
        code = _strip_comments(text)
        for m in re.finditer(r"__builtin_amdgcn_(?:mfma|smfmac)\w*", code):
            assert m.group(0) == allowed, f"{name}: {m.group(0)} (only {allowed} is allowed)"
            assert name == "mfma_tile.h", f"{name}: call the mfma_tile.h wrappers, not the builtin"
            seen += 1
        assert not re.search(r"\bv_s?mfmac?_", code), f"{name}: MFMA in inline assembly"
    assert seen >= 1


def test_no_hand_written_packed_fp32_ops():
    for name, text in _sources():
        code = _strip_comments(text)
        assert not re.search(r"v_pk_(?:add|mul|fma)_f32", code), name
    with open(os.path.join(PKG, "build.py")) as fh:
        build = fh.read()
    assert '"-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"' in build


def _imports(path):
    with open(path) as fh:
        tree = ast.parse(fh.read(), path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


def test_product_never_imports_the_oracle():
    for f in sorted(os.listdir(PKG)):
        if f.endswith(".py"):
            mods = list(_imports(os.path.join(PKG, f)))
            assert not any(m == "oracle" or m.startswith("oracle.") or m.startswith("tests") for m in mods), f
    for name, text in _sources():
        assert "oracle" not in _strip_comments(text), name
