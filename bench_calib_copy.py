"""A plain device copy of known size, for calibrating HBM byte counters.

    python bench_calib_copy.py [MiB]

Copies a MiB-sized fp32 buffer into another three times with torch's copy
kernel: each launch reads MiB and writes MiB.  Profiled with
``rocprofv3 --pmc FETCH_SIZE`` (then ``WRITE_SIZE``), the counters' reading
per launch against these known bytes gives the factor that turns the
counters of another kernel into bytes.
"""
import sys

import torch


def main():
    mib = int(sys.argv[1]) if len(sys.argv) > 1 else 256
    a = torch.ones(mib * 1024 * 1024 // 4, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copy kernel: {mib} MiB read + {mib} MiB written per launch, 3 launches", flush=True)


if __name__ == "__main__":
    main()
