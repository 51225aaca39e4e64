"""Content hash of the HIP sources, used to tie stored hardware-counter figures
to the exact kernels they were measured on."""
import hashlib
from pathlib import Path

CSRC = Path(__file__).resolve().parent / "csrc"


def csrc_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(CSRC.glob("*")):
        if p.suffix in (".hip", ".hpp", ".h"):
            h.update(p.name.encode())
            h.update(p.read_bytes())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    print(csrc_hash())
