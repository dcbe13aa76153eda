"""HBM bandwidth probe: repeated device-to-device copies with libbdstep's streaming copy
kernel (bd_hbm_copy), or with --read repeated streaming reads (bd_hbm_read).

The copy gives the achievable copy bandwidth beside the 8 TB/s specification, and it is the
calibration run for the HBM traffic counters: a copy of B bytes moves exactly B bytes in
and B bytes out, so FETCH_SIZE and WRITE_SIZE read on it give the counters' scale.  The read
gives the achievable read-only bandwidth, the ceiling for the weight streams of the GEMMs.
Launches alternate between two buffers of --mib each so that the 256 MB last-level cache
cannot serve a repeat.

Usage: python -m block_diffusion_lm_router_amd.hbm_probe [--mib 1024] [--iters 20] [--read]
"""

import argparse
import json


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024, help="bytes copied per launch, in MiB")
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--read", action="store_true", help="streaming reads instead of copies")
    args = ap.parse_args()
    import torch
    from . import _binding as bd
    n = args.mib << 20
    if args.read:
        return read_probe(n, args.iters)
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


def read_probe(n, iters):
    print(json.dumps(read_rate(n, iters)))


def read_rate(n, iters, verify=True):
    """Average streaming-read rate over iters launches, alternating between two buffers of n
    bytes; with verify, the XOR checksums are checked on the host.  Returns the record."""
    import numpy as np
    import torch
    from . import _binding as bd
    bufs = [torch.randint(-2 ** 31, 2 ** 31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
            for _ in range(2)]
    W = 2112                      # >= bd.HBM_READ_WORDS, a multiple of 64 words
    sums = torch.zeros(2 * W, dtype=torch.int32, device="cuda")
    for i in range(4):
        bd.hbm_read(bufs[i % 2], sums[W * (i % 2):W * (i % 2 + 1)])
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(iters):
        bd.hbm_read(bufs[i % 2], sums[W * (i % 2):W * (i % 2 + 1)])
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / iters
    ok = None
    if verify:
        got = sums.cpu().numpy()[[0, W]].view(np.uint32)
        want = [np.bitwise_xor.reduce(b.cpu().numpy().view(np.uint32)) for b in bufs]
        ok = bool(got[0] == want[0] and got[1] == want[1])
    return {"probe": "bd_hbm_read", "bytes_per_launch": n, "read_bytes": n,
            "avg_ms": round(ms, 4), "read_gbs": round(n / (ms * 1e-3) / 1e9, 1), "verified": ok}


if __name__ == "__main__":
    main()
