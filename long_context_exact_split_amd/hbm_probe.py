"""HBM reference measurements for the roofline (read stream and copy).

python -m long_context_exact_split_amd.hbm_probe [--gib 4] [--blocks 0] [--reps 20]

Prints one JSON line with the read-stream and copy bandwidths (HIP events on
the launch stream).  The copy kernel of known size is the calibration run for
the FETCH_SIZE / WRITE_SIZE counters.
"""
import argparse
import ctypes
import json
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(PKG, "libhbm_probe.so")


def load():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built")
    lib = ctypes.CDLL(LIB)
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.hbm_copy_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_void_p]
    lib.hbm_read_share_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_void_p]
    lib.attn_probe_wg_stamps.argtypes = [ctypes.c_void_p, ctypes.c_int]
    return lib


def main():
    import torch
    ap = argparse.ArgumentParser()
    ap.add_argument("--gib", type=float, default=4.0)
    ap.add_argument("--blocks", type=int, default=0, help="0: sweep 1,2,4,8,16 blocks per CU")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--copy-only", action="store_true")
    args = ap.parse_args()
    lib = load()
    nbytes = int(args.gib * (1 << 30)) // 16 * 16
    src = torch.randint(0, 1 << 30, (nbytes // 4,), dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(cus * 64, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    out = {"bytes": nbytes, "cu_count": cus}

    def timed(fn):
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.reps)]
        for a, b in ev:
            a.record(s)
            fn()
            b.record(s)
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in ev)

    if not args.copy_only:
        sweep = [args.blocks] if args.blocks else [cus * k for k in (1, 2, 4, 8, 16)]
        reads = {}
        for nt in (0, 1):
            for blocks in sweep:
                ms = timed(lambda: lib.hbm_read_probe(src.data_ptr(), nbytes, sink.data_ptr(),
                                                      blocks, nt, s.cuda_stream))
                reads[f"{'nt' if nt else 'plain'}_{blocks}"] = nbytes / (ms * 1e-3) / 1e9
        out["read_gbps"] = reads
        out["read_gbps_best"] = max(reads.values())
    half = nbytes // 2 // 16 * 16
    dst = torch.empty(half // 4, dtype=torch.int32, device="cuda")
    ms = timed(lambda: lib.hbm_copy_probe(dst.data_ptr(), src.data_ptr(), half, cus * 8,
                                          s.cuda_stream))
    out["copy_bytes_each_way"] = half
    out["copy_ms"] = ms
    out["copy_gbps_read_plus_write"] = 2 * half / (ms * 1e-3) / 1e9
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
