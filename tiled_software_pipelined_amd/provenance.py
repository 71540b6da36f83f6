"""Identity of the compiled kernels, for matching measurements to code.

A counter measurement (HBM bytes per launch) is only valid for the kernel
source it was taken on; ``source_hash()`` fingerprints every file under
``csrc/`` so that a stored measurement can be recognised as stale.
"""
from __future__ import annotations

import glob
import hashlib
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")

_TAG = re.compile(r"<!-- tgemm-profile (.*?) -->")


def source_hash() -> str:
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if path.endswith((".hip", ".hpp", ".h", ".cpp")):
            h.update(os.path.basename(path).encode())
            h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def profile_tag(**fields) -> str:
    return "<!-- tgemm-profile %s -->" % " ".join("%s=%s" % kv for kv in fields.items())


def find_profile(kernel: str, workload: str, directory: str = PROFILES):
    """Fields of a committed profile summary taken on the current sources
    for this kernel and workload, or None."""
    src = source_hash()
    for path in sorted(glob.glob(os.path.join(directory, "*.md"))):
        m = _TAG.search(open(path).read())
        if not m:
            continue
        fields = dict(kv.split("=", 1) for kv in m.group(1).split())
        if fields.get("kernel") == kernel and fields.get("workload") == workload and \
                fields.get("source") == src:
            fields["path"] = os.path.relpath(path, ROOT)
            return fields
    return None
