"""Hash of the library's sources, embedded in liblorapool.so at build time and checked at import.

The build passes it to the compiler; lora_version() returns it; importing the package recomputes it
from the sources beside the library and refuses a library built from other sources.
"""
from __future__ import annotations

import glob
import hashlib
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)


def source_files() -> list:
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")) + glob.glob(os.path.join(PKG, "csrc", "*.h")))
    files.append(os.path.join(ROOT, "include", "lorapool.h"))
    return files


def source_hash() -> str | None:
    """16 hex digits over the names and contents of the sources; None if they are not all here."""
    h = hashlib.sha256()
    for f in source_files():
        if not os.path.exists(f):
            return None
        h.update(os.path.relpath(f, ROOT).encode())
        h.update(b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()[:16]
