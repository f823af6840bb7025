"""Per-phase timing of the persistent frame kernel from its own stamps.

    python -m autoregressive_codebook_tts_frame_amd.phase_trace [--workload bf16_b1] [--calls 3]

Decodes `calls` calls of the workload's frames with QT_F_TRACE (the first
GEMV workgroup stamps every phase of the first frame of a call with the
100 MHz wall clock; attention workgroup 0 stamps its events) and prints, per
stack and phase type, the mean time from the phase's start to: its first
wave's inputs in (poll), the barrier with every wave and the weight slice
(barrier), the normalised operand built (norm), the GEMV and its publish done
(gemv), the phase's stamps written (end), and the next phase's start (gap);
the total; and when the phase's weight slice had landed, measured from the
phase's start (negative: before it).  The stamps are taken on one workgroup:
they show where its time goes, not the slowest workgroup's.
"""
from __future__ import annotations

import argparse
import collections
import os
import sys

import numpy as np

NAMES = {0: "QKV", 1: "ATTN", 2: "COMB", 3: "O", 4: "GU", 5: "D", 6: "HEAD"}


def summarise(tr: np.ndarray) -> str:
    rows = []
    for i in range(768):
        if int(tr[i, 0]) == 255:
            break
        rows.append(tr[i].astype(np.int64))
    agg = collections.defaultdict(list)
    for i, r in enumerate(rows):
        typ, stack = int(r[0]) & 0xFF, (int(r[0]) >> 8) & 0xFF
        nxt = rows[i + 1][1] if i + 1 < len(rows) else r[3]
        # stamps: 1 start, 2 barrier passed, 3 end, 4 norm done, 5 GEMV done,
        # 6 first wave's inputs in, 7 weight slice landed
        agg[(stack, NAMES.get(typ, str(typ)))].append(
            [r[6] - r[1], r[2] - r[6], r[4] - r[2], r[5] - r[4], r[3] - r[5], nxt - r[3], nxt - r[1], r[7] - r[1]])
    out = ["| stack | phase | n | poll | barrier | norm | gemv | end | gap | total | slice landed |",
           "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    total = 0.0
    for k in sorted(agg):
        a = np.array(agg[k], np.float64) / 100.0  # 100 MHz ticks -> us
        total += a[:, 6].sum()
        mu = a.mean(0)
        out.append(f"| {'talker' if k[0] else 'predictor'} | {k[1]} | {len(a)} | " +
                   " | ".join(f"{v:.2f}" for v in mu) + " |")
    out.append("")
    out.append(f"Phases stamped: {len(rows)}; sum of phase totals {total:.1f} us (one frame).")
    ev = []
    for i in range(768, 1024):
        if int(tr[i, 0]) == 255:
            break
        ev.append(tr[i].astype(np.int64))
    kinds = collections.defaultdict(list)
    for r in ev:
        kinds[(int(r[0]) >> 8) & 0xFF].append([r[2] - r[1], r[3] - r[2], r[3] - r[1]])
    for k, v in sorted(kinds.items()):
        a = np.array(v, np.float64) / 100.0
        out.append(f"Attention workgroup 0, {'talker' if k else 'predictor'}: {len(a)} events, "
                   f"waiting for inputs {a[:, 0].mean():.2f} us, computing {a[:, 1].mean():.2f} us per event.")
    return "\n".join(out)


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="bf16_b1")
    ap.add_argument("--calls", type=int, default=3)
    args = ap.parse_args()
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from autoregressive_codebook_tts_frame_amd import qt, synth

    wl = synth.WORKLOADS[args.workload]
    m = wl.model
    w = synth.make_weights(m)
    d = qt.Decoder(m, w, 1, max_frames_per_call=wl.frames, flags=qt.QT_F_TRACE)
    assert d.path == qt.QT_PATH_FRAME, "the trace is the persistent kernel's"
    codes, text = synth.make_prompt(wl, 0)
    d.prefill(0, codes, text)
    st = d.get_state(0)
    ov = synth.make_overlays(wl, wl.frames)
    for _ in range(args.calls):  # the last call's first frame is reported
        d.set_state(0, *st)
        d.decode(wl.frames, ov)
    print(f"Workload {wl.name}: stamps of the first frame of call {args.calls} "
          f"({wl.frames} frames per call), microseconds.\n")
    print(summarise(d.dump(qt.QT_DUMP_TRACE)))
    d.close()


if __name__ == "__main__":
    main()
