"""Run the exchange-latency probe (exchange_probe.hip, built by build.py).

    python -m autoregressive_codebook_tts_frame_amd.exchange_probe

Prints a markdown table: for each mode and word count, microseconds per
round of exchanges among one workgroup per compute unit (the modes are
described at the top of exchange_probe.hip)."""
import os
import subprocess
import sys

from autoregressive_codebook_tts_frame_amd.build import PROBE


def main() -> int:
    if not os.path.exists(PROBE):
        print(f"{PROBE} is not built: run __graft_entry__.build() first", file=sys.stderr)
        return 1
    return subprocess.run([PROBE], timeout=300).returncode


if __name__ == "__main__":
    sys.exit(main())
