"""Runs the C-ABI CPU tests (test_abi_cpu.py) against a sanitized host-only build of the library.

Invoked by test_sanitizers.py in a child process whose environment preloads the sanitizer runtime:
  python tests/sanitized_abi_driver.py <path of the sanitized library>
The package's ctypes module is loaded from its file alone (the package itself imports torch, which
the sanitizer runtime need not see), its library handle is replaced by the sanitized build, and
pytest runs the ABI tests, which only validate arguments and compute sizes on the host."""
import ctypes
import importlib.util
import os
import sys
import types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def main(lib_path: str) -> int:
    pkg_dir = os.path.join(ROOT, "long_context_decode_gqa_amd")
    pkg = types.ModuleType("long_context_decode_gqa_amd")
    pkg.__path__ = [pkg_dir]
    sys.modules["long_context_decode_gqa_amd"] = pkg
    spec = importlib.util.spec_from_file_location("long_context_decode_gqa_amd._lib", os.path.join(pkg_dir, "_lib.py"))
    lib_mod = importlib.util.module_from_spec(spec)
    sys.modules["long_context_decode_gqa_amd._lib"] = lib_mod
    spec.loader.exec_module(lib_mod)
    pkg._lib = lib_mod
    L = ctypes.CDLL(lib_path)
    for name, (argtypes, restype) in lib_mod.SIGNATURES.items():
        fn = getattr(L, name)
        fn.argtypes = argtypes
        fn.restype = restype
    lib_mod._lib = L
    lib_mod.LIB_PATH = lib_path
    import pytest
    return pytest.main([os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu"])


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
