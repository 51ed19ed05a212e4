"""The oracle and the HIP path share no code: no module of the product package imports the oracle,
and the oracle imports nothing but numpy (weights and token ids are handed to it). Checked on the
source text, so it runs on the host."""
import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def imported_modules(path):
    tree = ast.parse(open(path).read(), path)
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.level == 0 and node.module:
            mods.add(node.module.split(".")[0])
    return mods


def python_files(folder):
    for name in sorted(os.listdir(os.path.join(ROOT, folder))):
        if name.endswith(".py"):
            yield os.path.join(ROOT, folder, name)


def test_product_package_never_imports_the_oracle():
    for path in python_files("looped_ngpt_language_amd"):
        assert "oracle" not in imported_modules(path), path


def test_oracle_imports_only_numpy_and_the_standard_library():
    for path in python_files("oracle"):
        mods = imported_modules(path) - {"__future__", "math", "dataclasses", "typing", "collections"}
        assert mods <= {"numpy"}, (path, mods)


def test_native_sources_do_not_reference_the_oracle():
    csrc = os.path.join(ROOT, "looped_ngpt_language_amd", "csrc")
    for name in os.listdir(csrc):
        text = open(os.path.join(csrc, name)).read()
        assert "oracle" not in text.lower(), name


def test_missing_library_fails_loudly(tmp_path):
    """With the HIP library absent the binding raises instead of computing anything another way
    (run in a child process so the library this test session loaded stays as it is)."""
    import subprocess
    import sys
    code = ("import looped_ngpt_language_amd.dory as d\n"
            f"d.LIB_PATH = {str(tmp_path / 'absent' / 'libdory.so')!r}\n"
            "try:\n"
            "    d.lib()\n"
            "except ImportError as e:\n"
            "    print('raised', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0 and r.stdout.startswith("raised"), (r.stdout, r.stderr)
