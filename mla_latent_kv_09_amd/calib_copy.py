"""Plain device-to-device copy of a known size, used to calibrate the HBM byte
counters (FETCH_SIZE / WRITE_SIZE) that rocprofv3 reports for the MLA kernels.

    python -m mla_latent_kv_09_amd.calib_copy [--mib 1024] [--reps 3]

Each repetition copies `mib` MiB from one fresh buffer to another with torch's
copy kernel, so one dispatch reads and writes exactly that many bytes.
"""
import argparse

import torch


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    n = args.mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {args.mib} MiB x {args.reps}")


if __name__ == "__main__":
    main()
