"""Profiling helpers: collecting rocprofv3 kernel statistics and HBM byte
counters for bench.py workloads (collect.sh) and turning them into the short
text summaries kept under profiles/ (summarize.py)."""
import hashlib
import os

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "csrc")


def source_digest() -> str:
    """Digest of the kernel sources: counter figures taken on other sources
    no longer describe the kernels."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]
