"""Per-kernel resource usage of libdh's gfx950 build, from clang's resource-usage remarks.

    python few_row_vocab_amd/resource_usage.py [--markdown]

Compiles the device side of every csrc/*.hip with the library's flags and
-Rpass-analysis=kernel-resource-usage, and prints one line per kernel instance: VGPRs,
AGPRs, SGPRs, scratch bytes a lane (non-zero: the kernel spills), LDS bytes a workgroup
(static; the GEMV and the rescore add dynamic LDS at launch) and the occupancy the compiler
reports (waves a SIMD).  Scratch without VGPR spills is a stack object.
"""
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import build as lb  # noqa: E402

FIELDS = [("VGPRs", "VGPRs"), ("AGPRs", "AGPRs"), ("TotalSGPRs", "SGPRs"),
          ("VGPRs Spill", "VGPR spill"), ("ScratchSize [bytes/lane]", "scratch B/lane"),
          ("LDS Size [bytes/block]", "LDS B"), ("Occupancy [waves/SIMD]", "waves/SIMD")]


def demangle(names):
    out = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True,
                         check=True).stdout.splitlines()
    short = []
    for d in out:
        d = d.replace("void ", "", 1).replace("dh::(anonymous namespace)::", "")
        d = re.sub(r"\(.*\)$", "", d)
        short.append(d)
    return short


def usage(src):
    cmd = [lb.HIPCC, *lb.FLAGS, "--cuda-device-only", "-c", src, "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark: (.+?): (\S+)\s*(\[.*\])?\s*$", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = m.group(2)
    names = list(kernels)
    return [(os.path.basename(src), d, kernels[n]) for d, n in zip(demangle(names), names)]


def main():
    md = "--markdown" in sys.argv
    rows = [row for src in lb.sources() for row in usage(src)]
    if md:
        print("| file | kernel instance | " + " | ".join(h for _, h in FIELDS) + " |")
        print("|---|---|" + "---|" * len(FIELDS))
    for f, k, v in rows:
        vals = [v.get(key, "?") for key, _ in FIELDS]
        if md:
            print(f"| {f} | `{k}` | " + " | ".join(vals) + " |")
        else:
            print(f"{f:12s} {k:60s} " + " ".join(f"{x:>5s}" for x in vals))
    spills = [(f, k) for f, k, v in rows if v.get("ScratchSize [bytes/lane]", "0") != "0"]
    print(f"\n{len(rows)} kernel instances; {len(spills)} with scratch (spills)")


if __name__ == "__main__":
    main()
