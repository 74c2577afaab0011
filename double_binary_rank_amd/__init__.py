"""MI355X (gfx950) double-binary-factorised product behind a C ABI.

Importing this package loads the in-tree HIP library ``libdbf.so``; it raises
if the library has not been built (there is no CPU fallback).
"""
from ._lib import DbfError, EXPORTS, LIB_PATH  # noqa: F401
from .api import *  # noqa: F401,F403
from .api import __all__ as _api_all

__all__ = ["DbfError", "EXPORTS", "LIB_PATH", *_api_all]
