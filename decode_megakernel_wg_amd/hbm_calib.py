"""Calibration workload for HBM byte counters: a plain device-to-device copy of a known size.

python -m decode_megakernel_wg_amd.hbm_calib [--mib 1024] [--reps 3]

Each repetition launches one elementwise kernel (torch's `neg` from one contiguous
fp32 tensor into another: a copy with the sign flipped) that reads exactly N bytes
and writes exactly N bytes.  Run under
`rocprofv3 --pmc FETCH_SIZE` and then `--pmc WRITE_SIZE`: the counter value per
dispatch divided by N KiB gives the factor that turns the same counters read
on the megakernel into bytes.
"""
from __future__ import annotations

import argparse
import json
import sys


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    import torch

    if not torch.cuda.is_available():
        print("hbm_calib needs a GPU", file=sys.stderr)
        sys.exit(2)
    n = args.mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda")
    dst = torch.empty(n, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ms = []
    for _ in range(args.reps):
        ev[0].record()
        torch.neg(src, out=dst)
        ev[1].record()
        torch.cuda.synchronize()
        ms.append(ev[0].elapsed_time(ev[1]))
    assert torch.equal(dst, -src)
    nbytes = n * 4
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": args.reps,
                      "ms": [round(m, 4) for m in ms], "GB_per_s_read_plus_write": round(2 * nbytes / (min(ms) * 1e-3) / 1e9, 1)}),
          flush=True)


if __name__ == "__main__":
    main()
