"""Compile the HIP sources in csrc/ into libtca.so for gfx950 (in-tree).

Every call recompiles. Flags:
  --offload-arch=gfx950          CDNA4 only
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                 no packed fp32 VALU instructions are generated
  -munsafe-fp-atomics            float atomics map to hardware float adds
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtca.so")
# the benchmark report's probes (not the attention library): the matrix-core
# throughput loop and the per-block instruction-mix ceilings
MEASURE_SRCS = sorted(glob.glob(os.path.join(HERE, "measure", "*.hip")))
MEASURE_LIB = os.path.join(HERE, "libtca_measure.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(srcs, out: str, extra=(), verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    os.replace(tmp, out)
    return out


def build(out: str = LIB, extra=(), verbose: bool = False) -> str:
    """The attention library (and, for the default output, the measurement probe)."""
    _compile(sources(), out, extra, verbose)
    if out == LIB:
        _compile(MEASURE_SRCS, MEASURE_LIB, extra, verbose)
    return out


def resource_usage() -> list:
    """Per-kernel registers, LDS and occupancy as the compiler reports them
    (hipcc -Rpass-analysis=kernel-resource-usage on the device code)."""
    import re
    from concurrent.futures import ThreadPoolExecutor

    def report(src):   # one compile per source file, run side by side
        cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")], "-c", src,
               "--offload-device-only", "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr[-2000:]}")
        return res.stderr

    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as pool:
        texts = list(pool.map(report, srcs))
    rows, cur = [], None
    for src, text in zip(srcs, texts):
        for line in text.splitlines():
            m = re.search(r"remark:\s+(.*?)\s+\[-Rpass", line)
            if not m:
                continue
            key, _, val = m.group(1).partition(":")
            if key.strip() == "Function Name":
                cur = {"kernel": val.strip(), "source": os.path.basename(src)}
                rows.append(cur)
            elif cur is not None:
                cur[key.strip()] = val.strip()
    return rows


def resource_usage_markdown() -> str:
    import re

    def short(n):   # tca::<name><template arguments> from the mangled kernel name
        m = re.match(r"_ZN3tca(\d+)", n)
        if not m:
            return n
        ln = int(m.group(1))
        name, rest = n[m.end():m.end() + ln], n[m.end() + ln:]
        if not rest.startswith("I"):
            return name
        args, i = [], 1
        names = {"f": "float", "t": "bf16", "DF16_": "half"}
        while i < len(rest) and rest[i] != "E":
            lit = re.match(r"Li(\d+)E", rest[i:])
            if lit:
                args.append(lit.group(1))
                i += lit.end()
                continue
            flag = re.match(r"Lb([01])E", rest[i:])
            if flag:
                args.append("true" if flag.group(1) == "1" else "false")
                i += flag.end()
                continue
            for code, ty in names.items():
                if rest.startswith(code, i):
                    args.append(ty)
                    i += len(code)
                    break
            else:
                return name
        return f"{name}<{', '.join(args)}>"

    out = ["| Kernel | Source | VGPRs | AGPRs | VGPR spills | LDS bytes per workgroup | Waves per SIMD |",
           "|---|---|---|---|---|---|---|"]
    for r in resource_usage():
        out.append(f"| `{short(r['kernel'])}` | {r['source']} | {r.get('VGPRs')} | {r.get('AGPRs')} | "
                   f"{r.get('VGPRs Spill')} | {r.get('LDS Size [bytes/block]')} | {r.get('Occupancy [waves/SIMD]')} |")
    return "\n".join(out)


if __name__ == "__main__":
    if "--resource-usage" in sys.argv:
        print(resource_usage_markdown())
    else:
        print(build(verbose=True))
