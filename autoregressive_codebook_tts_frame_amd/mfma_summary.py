"""MFMA use and HBM traffic of the per-op path's kernels from rocprofv3
counter runs of `bench.py --workload W --frames F --steps 1 --warmup 1
--copy-calibration MIB`.

    python -m autoregressive_codebook_tts_frame_amd.mfma_summary MFMA_DIR FETCH_DIR WRITE_DIR [--copy-mib 1024]

MFMA_DIR: a run with SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES,
SQ_BUSY_CYCLES and GRBM_GUI_ACTIVE; FETCH_DIR, WRITE_DIR: FETCH_SIZE and
WRITE_SIZE runs.  Only the timed step's replays count: the dispatches between
the second and the last advance_kernel (the warmup step ends at the second).
Per kernel: MFMA FLOP (MOPS x 512) per dispatch and per second of dispatch
time, MFMA busy cycles over GPU-active cycles x SIMDs (1,024 on MI355X), and
HBM bytes per dispatch scaled by the plain 1 GiB copies at the end of each
run (counter bytes x copy bytes / the copy's counter bytes)."""
import argparse
import collections
import glob
import os
import sqlite3

SIMDS = 1024


def _rows(d):
    db = glob.glob(os.path.join(d, "**", "*.db"), recursive=True)[0]
    c = sqlite3.connect(db)
    return c.execute("select dispatch_id, name, start, end, counter_name, counter_value from pmc_events "
                     "order by dispatch_id").fetchall()


def _window(rows):
    """{dispatch: (name, duration ns, {counter: value})} of the timed step, and the copies."""
    disp = collections.OrderedDict()
    for did, name, start, end, cn, cv in rows:
        e = disp.setdefault(did, [name, end - start, {}])
        e[2][cn] = e[2].get(cn, 0.0) + cv
    ids = list(disp)
    adv = [i for i in ids if "advance_kernel" in disp[i][0]]
    lo, hi = adv[1], adv[-1]
    timed = {i: disp[i] for i in ids if lo < i <= hi}
    copies = [disp[i] for i in ids if "copyBuffer" in disp[i][0]][-3:]
    return timed, copies


def _short(name):
    return name.split("(")[0].replace("void ", "").replace("qtk::", "")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("mfma_dir")
    ap.add_argument("fetch_dir")
    ap.add_argument("write_dir")
    ap.add_argument("--copy-mib", type=int, default=1024)
    a = ap.parse_args()
    m_timed, _ = _window(_rows(a.mfma_dir))
    f_timed, f_cp = _window(_rows(a.fetch_dir))
    w_timed, w_cp = _window(_rows(a.write_dir))
    kib = a.copy_mib * 1024.0
    fscale = kib / (sum(c[2]["FETCH_SIZE"] for c in f_cp) / len(f_cp))
    wscale = kib / (sum(c[2]["WRITE_SIZE"] for c in w_cp) / len(w_cp))
    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    for t, key in ((m_timed, "m"), (f_timed, "f"), (w_timed, "w")):
        for name, dur, cv in t.values():
            g = agg[_short(name)]
            g[key + "n"] += 1
            g[key + "dur"] += dur
            for cn, v in cv.items():
                g[cn] += v
    print("fetch scale %.4f, write scale %.4f (1 GiB copies)" % (fscale, wscale))
    print("| kernel | dispatches | MFMA GFLOP per dispatch | MFMA TFLOP/s over its dispatch time | MFMA busy | "
          "HBM MB per dispatch (read + write) | GPU-active cycles per ns of dispatch |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for k, g in sorted(agg.items(), key=lambda x: -x[1]["mdur"]):
        n = g["mn"] or 1
        flop = g["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        busy = g["SQ_VALU_MFMA_BUSY_CYCLES"] / (g["GRBM_GUI_ACTIVE"] * SIMDS) if g["GRBM_GUI_ACTIVE"] else 0.0
        hbm = (g["FETCH_SIZE"] * 1024 * fscale / (g["fn"] or 1) + g["WRITE_SIZE"] * 1024 * wscale / (g["wn"] or 1))
        print("| `%s` | %d | %.3f | %.1f | %.2f%% | %.2f | %.2f |" % (
            k, g["mn"], flop / n / 1e9, flop / g["mdur"] / 1e3 if g["mdur"] else 0.0, 100 * busy, hbm / 1e6,
            g["GRBM_GUI_ACTIVE"] / g["mdur"] if g["mdur"] else 0.0))


if __name__ == "__main__":
    main()
