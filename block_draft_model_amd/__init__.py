"""MI355X-native Kolibri-1 block-drafter round (libkdraft) and its Python binding."""
from . import kdraft  # noqa: F401  (the library itself loads on first use)

__all__ = ["kdraft"]
