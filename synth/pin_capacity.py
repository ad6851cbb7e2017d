"""How much pinned, device-mapped host memory this machine gives one process.

The offload workloads keep half of their facts in pinned host memory, so
their size depends on this figure.  The probe takes mapped pinned memory
with hipHostMalloc in 4 GiB pieces until a piece is refused or a cap is
reached (default: the smaller of 192 GiB and MemAvailable - 32 GiB), prints
what it got, and frees everything.

    python synth/pin_capacity.py [cap_gib]
"""
from __future__ import annotations

import ctypes
import os
import resource
import sys

PIECE = 4 << 30
HIP_HOST_MALLOC_MAPPED = 0x2


def meminfo() -> dict:
    out = {}
    with open("/proc/meminfo") as f:
        for line in f:
            k, v = line.split(":", 1)
            out[k] = int(v.split()[0]) << 10
    return out


def main() -> int:
    mi = meminfo()
    cap = min(192 << 30, mi["MemAvailable"] - (32 << 30))
    if len(sys.argv) > 1:
        cap = min(cap, int(float(sys.argv[1]) * (1 << 30)))
    soft, hard = resource.getrlimit(resource.RLIMIT_MEMLOCK)
    print(f"MemTotal {mi['MemTotal'] / 2**30:.1f} GiB, MemAvailable "
          f"{mi['MemAvailable'] / 2**30:.1f} GiB, RLIMIT_MEMLOCK soft {soft} hard {hard}, "
          f"cap {cap / 2**30:.0f} GiB", flush=True)
    hip = ctypes.CDLL(os.path.join("/opt/rocm/lib", "libamdhip64.so"))
    hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t,
                                  ctypes.c_uint]
    hip.hipHostFree.argtypes = [ctypes.c_void_p]
    got = []
    rc = 0
    while (len(got) + 1) * PIECE <= cap:
        p = ctypes.c_void_p()
        rc = hip.hipHostMalloc(ctypes.byref(p), PIECE, HIP_HOST_MALLOC_MAPPED)
        if rc != 0:
            break
        got.append(p.value)
        print(f"pinned {len(got) * 4} GiB", flush=True)
    total = len(got) * PIECE
    for p in got:
        hip.hipHostFree(p)
    why = f"refused (hipError {rc})" if rc != 0 else "reached the cap"
    print(f"pinned and mapped {total / 2**30:.0f} GiB in 4 GiB pieces; the next piece {why}",
          flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
