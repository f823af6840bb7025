"""Per-kernel summaries of a rocprofv3 kernel trace.

    python -m autoregressive_codebook_tts_frame_amd.trace_summary DIR          one replay of the per-op graph
    python -m autoregressive_codebook_tts_frame_amd.trace_summary --stats DIR  every kernel of the trace
    python -m autoregressive_codebook_tts_frame_amd.trace_summary --prefill DIR  the last prompt prefill

The replay summary takes the last replay before the last advance_kernel and
splits it into predictor and talker stages; --stats lists calls, total and
average duration and share per kernel over the whole trace."""
import collections
import glob
import sqlite3
import sys


def main(d: str) -> None:
    db = glob.glob(d + "/**/*.db", recursive=True)[0]
    c = sqlite3.connect(db)
    rows = c.execute("select name, start, end, grid_x, workgroup_x, grid_y, grid_z from kernels order by start").fetchall()
    adv = [i for i, r in enumerate(rows) if "advance_kernel" in r[0]]
    seg = rows[adv[-2] + 1:adv[-1] + 1]
    frames = sum(1 for r in seg if "gather_kernel" in r[0])
    stage, agg = "pred", collections.defaultdict(lambda: [0, 0.0])
    for r in seg:
        n = r[0]
        if "pred_input" in n:
            stage = "predictor"
        if "gather_kernel" in n:
            stage = "talker"
        key = (stage, n.split("(")[0].replace("void ", ""), "%dx%dx%d" % (r[3] // r[4], r[5], r[6]))
        agg[key][0] += 1
        agg[key][1] += (r[2] - r[1]) / 1e3
    print("| stage | kernel | grid | calls per frame-step | avg us | us per frame-step |")
    print("|---|---|---|---:|---:|---:|")
    tot = 0.0
    for k, (n, t) in sorted(agg.items(), key=lambda x: -x[1][1]):
        tot += t
        print("| %s | `%s` | %s | %g | %.2f | %.1f |" % (k[0], k[1], k[2], n / frames, t / n, t / frames))
    span = (seg[-1][2] - seg[0][1]) / 1e3
    print("\nKernels per replay: %d over %d frame-steps; kernel time %.1f us and span %.1f us per frame-step."
          % (len(seg), frames, tot / frames, span / frames))


def stats(d: str) -> None:
    db = glob.glob(d + "/**/*.db", recursive=True)[0]
    c = sqlite3.connect(db)
    agg = collections.defaultdict(lambda: [0, 0.0])
    for name, start, end in c.execute("select name, start, end from kernels"):
        agg[name][0] += 1
        agg[name][1] += (end - start) / 1e3
    tot = sum(t for _, t in agg.values())
    print("| kernel | calls | total (us) | average (us) | % |")
    print("|---|---:|---:|---:|---:|")
    for k, (n, t) in sorted(agg.items(), key=lambda x: -x[1][1]):
        print("| `%s` | %d | %.1f | %.1f | %.2f |" % (k[:110], n, t, t / n, 100 * t / tot))


def prefill(d: str) -> None:
    db = glob.glob(d + "/**/*.db", recursive=True)[0]
    c = sqlite3.connect(db)
    rows = c.execute("select name, start, end, grid_x, workgroup_x, grid_y, grid_z from kernels order by start").fetchall()
    fk = [i for i, r in enumerate(rows) if "frame_kernel" in r[0]]
    seg = rows[fk[-2] + 1:fk[-1]]
    agg = collections.defaultdict(lambda: [0, 0.0])
    for r in seg:
        key = (r[0].split("(")[0].replace("void ", ""), "%dx%dx%d" % (r[3] // r[4], r[5], r[6]))
        agg[key][0] += 1
        agg[key][1] += (r[2] - r[1]) / 1e3
    tot = sum(t for _, t in agg.values())
    print("| kernel | grid | calls | average (us) | total (us) | % |")
    print("|---|---|---:|---:|---:|---:|")
    for k, (n, t) in sorted(agg.items(), key=lambda x: -x[1][1]):
        print("| `%s` | %s | %d | %.2f | %.1f | %.1f |" % (k[0], k[1], n, t / n, t, 100 * t / tot))
    span = (seg[-1][2] - seg[0][1]) / 1e3
    print("\nKernels in the prefill: %d; kernel time %.1f us, span %.1f us; the frame kernel that follows: %.1f us."
          % (len(seg), tot, span, (rows[fk[-1]][2] - rows[fk[-1]][1]) / 1e3))


if __name__ == "__main__":
    if sys.argv[1] == "--stats":
        stats(sys.argv[2])
    elif sys.argv[1] == "--prefill":
        prefill(sys.argv[2])
    else:
        main(sys.argv[1])
