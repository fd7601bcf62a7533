"""pytest plugin for the sanitizer run: swaps in the libraries built with
-fsanitize=address,undefined (paths from SAN_FA_LIB and SAN_ORACLE_LIB)
before any test loads the regular ones."""
import os


def pytest_configure(config):
    from exact_attention_32_amd import _lib
    from oracle import oracle as oracle_impl

    _lib._lib = None
    _lib.load_library(os.environ["SAN_FA_LIB"])
    oracle_impl._default = oracle_impl.Oracle(os.environ["SAN_ORACLE_LIB"])
    print(f"sanitizer builds: {_lib._lib._name}, {oracle_impl._default.libpath}", flush=True)
