"""Helpers for tests of libhcr.so: build on demand, header parsing."""

import os
import re

from bf16_hyper_connection_amd import hcr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hcr.h")


def ensure_built():
    if not os.path.exists(hcr.LIB_PATH):
        from bf16_hyper_connection_amd import build
        build.build()
    return hcr.lib()


def declared_functions():
    """Names of the functions include/hcr.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hcr_[a-z_]+)\s*\(", text)))
