"""A plain library bf16 GEMM on random data: the sustained matrix-core rate of this
chip, for comparison with the MLA kernels' MFMA rate.

    python -m mla_latent_kv_09_amd.calib_gemm [--n 8192] [--reps 20]

C = A B with A, B [n x n] bf16 drawn from N(0, 1) (torch.matmul, which calls the vendor
GEMM library), 2 n^3 flops per dispatch.  Prints the event-timed rate; run under
rocprofv3 with GRBM_GUI_ACTIVE to see the clock the chip holds during it.
"""
import argparse

import torch


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--n", type=int, default=8192)
    ap.add_argument("--reps", type=int, default=20)
    args = ap.parse_args()
    n = args.n
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(n, n, device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
    c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.reps
    print(f"bf16 GEMM n={n}: {ms * 1e3:.1f} us per dispatch, "
          f"{2.0 * n ** 3 / (ms * 1e-3) / 1e12:.0f} TFLOP/s (random N(0,1) operands)")
    del c


if __name__ == "__main__":
    main()
