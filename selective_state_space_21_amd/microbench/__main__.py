"""Build (hipcc, gfx950, packed fp32 off) and run the issue-rate probes in
issue_rates.hip; the binary is written next to the source."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def main() -> int:
    src = os.path.join(HERE, "issue_rates.hip")
    exe = os.path.join(HERE, "issue_rates")
    if not os.path.exists(exe) or os.path.getmtime(exe) < os.path.getmtime(src):
        subprocess.run(["/opt/rocm/bin/hipcc", "-O3", "--offload-arch=gfx950", "-Xclang",
                        "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", exe],
                       check=True)
    if "--build-only" in sys.argv:
        return 0
    return subprocess.run([exe]).returncode


if __name__ == "__main__":
    sys.exit(main())
