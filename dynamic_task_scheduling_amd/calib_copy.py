"""Plain device-to-device copy of a known size, used to calibrate hardware
memory-traffic counters (FETCH_SIZE / WRITE_SIZE) against true bytes."""
import json
import sys

import torch


def main(mib: int = 1024, reps: int = 3) -> None:
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_dispatch": n, "reps": reps}))


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 1024)
