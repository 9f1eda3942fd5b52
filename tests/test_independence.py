"""The oracle and the HIP path share no code: neither imports the other, and
the product package never reaches into oracle/ (CPU only, static check)."""
import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _imports(path):
    tree = ast.parse(open(path).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            names.add(node.module.split(".")[0])
    return names


def _py_files(d):
    for dp, _, fs in os.walk(os.path.join(ROOT, d)):
        for f in fs:
            if f.endswith(".py"):
                yield os.path.join(dp, f)


def test_oracle_does_not_import_the_library():
    for p in _py_files("oracle"):
        assert "outlier_aware_bit_amd" not in _imports(p), p


def test_library_does_not_import_or_read_the_oracle():
    for p in _py_files("outlier_aware_bit_amd"):
        assert "oracle" not in _imports(p), p
        assert "oracle/" not in open(p).read(), p
    for dp, _, fs in os.walk(os.path.join(ROOT, "outlier_aware_bit_amd", "csrc")):
        for f in fs:
            assert "oracle" not in open(os.path.join(dp, f)).read().lower(), f


def test_input_generator_is_independent():
    imps = _imports(os.path.join(ROOT, "synth.py"))
    assert "oracle" not in imps and "outlier_aware_bit_amd" not in imps
