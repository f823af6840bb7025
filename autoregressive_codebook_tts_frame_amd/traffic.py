"""HBM traffic of the persistent frame kernel from two rocprofv3 counter runs.

    python -m autoregressive_codebook_tts_frame_amd.traffic FETCH_DIR WRITE_DIR \
        [--workload bf16_b1] [--steps 2] [--copy-mib 1024] [--out profiles/frame_kernel_bf16_b1_traffic.json]

Each directory holds the output of one `rocprofv3 --pmc FETCH_SIZE` (or
WRITE_SIZE) run of `bench.py --steps S --warmup 1 --copy-calibration MIB`.
The counters read KiB per dispatch.  Each is scaled by what it reads for the
run's three plain device copies of MIB MiB (each reads and writes MIB MiB), so
bytes = counter * 1024 * (copy bytes / copy counter bytes).  The frame kernel's
figure is the mean over the S timed launches (the last S frame_kernel
dispatches).  The result records the sha256 of the kernel sources it was taken
on; bench.py reports it only while they are unchanged."""
import argparse
import glob
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _values(d: str, counter: str):
    db = glob.glob(os.path.join(d, "**", "*.db"), recursive=True)[0]
    c = sqlite3.connect(db)
    rows = c.execute("select name, counter_value from pmc_events where counter_name = ? order by dispatch_id",
                     (counter,)).fetchall()
    frame = [v for n, v in rows if "frame_kernel" in n]
    copies = [v for n, v in rows if "copyBuffer" in n]
    return frame, copies


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_dir")
    ap.add_argument("write_dir")
    ap.add_argument("--workload", default="bf16_b1")
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles", "frame_kernel_bf16_b1_traffic.json"))
    a = ap.parse_args()
    sys.path.insert(0, ROOT)
    import bench
    from autoregressive_codebook_tts_frame_amd import synth

    wl = synth.WORKLOADS[a.workload]
    fr_f, cp_f = _values(a.fetch_dir, "FETCH_SIZE")
    fr_w, cp_w = _values(a.write_dir, "WRITE_SIZE")
    fr_f, fr_w, cp_f, cp_w = fr_f[-a.steps:], fr_w[-a.steps:], cp_f[-3:], cp_w[-3:]
    kib = a.copy_mib * 1024.0
    fetch_scale = kib / (sum(cp_f) / len(cp_f))
    write_scale = kib / (sum(cp_w) / len(cp_w))
    fetch_b = sum(fr_f) / len(fr_f) * 1024 * fetch_scale
    write_b = sum(fr_w) / len(fr_w) * 1024 * write_scale
    mean_len = wl.prompt + (wl.frames + 1) / 2.0  # valid talker keys, mean over the step's frames
    algo = bench.frame_bytes(wl.model, wl.batch, mean_len) * wl.frames
    res = {"workload": wl.name, "frames_per_step": wl.frames, "kernel_sha256": bench.kernel_source_hash(),
           "bytes_per_launch": fetch_b + write_b, "fetch_bytes_per_launch": fetch_b,
           "write_bytes_per_launch": write_b, "fetch_scale": fetch_scale, "write_scale": write_scale,
           "fetch_kib_raw": fr_f, "write_kib_raw": fr_w, "copy_fetch_kib_raw": cp_f, "copy_write_kib_raw": cp_w,
           "algorithmic_bytes_per_launch": algo}
    with open(a.out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))
    print(f"measured / algorithmic = {(fetch_b + write_b) / algo:.4f}")


if __name__ == "__main__":
    main()
