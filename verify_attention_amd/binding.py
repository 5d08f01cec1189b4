"""ctypes binding of libspecattn.so (filled in with the C ABI)."""
import os

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path():
    return os.path.join(_HERE, "libspecattn.so")


def load():
    raise RuntimeError("libspecattn.so binding not built yet")
