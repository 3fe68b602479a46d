"""Plain device copy of a known size, for calibrating HBM byte counters.

``python -m non_cartesian_mri_fhd_amd.copycal [--mib 1024] [--reps 3]``
copies a float32 buffer of the given size on cuda:0 ``reps`` times with
torch's copy kernel. Each dispatch reads and writes exactly ``mib`` MiB, so
the FETCH_SIZE and WRITE_SIZE counters of these dispatches give the factor
between the counters' KiB and algorithmic bytes.
"""
from __future__ import annotations

import argparse
import json
import sys


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args(sys.argv[1:] if argv is None else argv)
    import torch
    n = args.mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_dispatch": n * 4,
                      "copy_bytes_written_per_dispatch": n * 4, "reps": args.reps}))
    return 0


if __name__ == "__main__":
    sys.exit(main())
