"""HBM bandwidth probe: repeated device-to-device copies with libbdstep's streaming copy
kernel (bd_hbm_copy).

It gives the achievable copy bandwidth beside the 8 TB/s specification, and it is the
calibration run for the HBM traffic counters: a copy of B bytes moves exactly B bytes in
and B bytes out, so FETCH_SIZE and WRITE_SIZE read on it give the counters' scale.

Usage: python -m block_diffusion_lm_router_amd.hbm_probe [--mib 1024] [--iters 20]
"""

import argparse
import json


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024, help="bytes copied per launch, in MiB")
    ap.add_argument("--iters", type=int, default=20)
    args = ap.parse_args()
    import torch
    from . import _binding as bd
    n = args.mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        bd.hbm_copy(src, dst)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.iters):
        bd.hbm_copy(src, dst)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.iters
    ok = bool(torch.equal(src, dst))
    print(json.dumps({"probe": "bd_hbm_copy", "bytes_per_launch": n, "read_bytes": n,
                      "write_bytes": n, "avg_ms": round(ms, 4),
                      "copy_gbs": round(2 * n / (ms * 1e-3) / 1e9, 1), "verified": ok}))


if __name__ == "__main__":
    main()
