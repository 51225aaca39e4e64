"""Content hash of the HIP kernel sources (prefill, decode, backward and the
headers they include), used to tie stored hardware-counter figures (HBM
traffic, matrix-core cycles of those kernels) to the exact code they were
measured on. The C ABI glue does not enter it: it does not change the code of
the kernels the figures describe."""
import hashlib
from pathlib import Path

CSRC = Path(__file__).resolve().parent / "csrc"
KERNEL_SOURCES = ("kda_common.hpp", "kda_launch.hpp", "kda_decode.hip", "kda_prefill.hip", "kda_backward.hip")


def csrc_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        p = CSRC / name
        h.update(p.name.encode())
        h.update(p.read_bytes())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    print(csrc_hash())
