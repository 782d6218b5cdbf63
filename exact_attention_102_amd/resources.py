"""Per-kernel register, spill, LDS and occupancy table of the built kernels (host tool).

    python -m exact_attention_102_amd.resources [--out profiles/resources_gfx950.md]

Compiles the kernel sources for gfx950 with the compiler's kernel-resource-usage
remarks (-Rpass-analysis=kernel-resource-usage, the same flags as the library
build) and turns them into one row per kernel instantiation: VGPRs, AGPRs, spilled
VGPRs, scratch bytes per lane, LDS bytes per workgroup and the waves per CU that
registers and LDS allow.  "Potential algorithmic improvements for backward pass"
(flash-attention issue 1172) frames the block-shape choice as a search over what is
held in registers, what spills, and what fits on chip; this table is that record
for every configuration the sweep (sweep.py) times.
"""
from __future__ import annotations

import argparse
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["fa_fwd.hip", "fa_bwd.hip"]
LDS_PER_CU = 160 * 1024
SIMDS_PER_CU = 4
REGS_PER_SIMD_LANE = 512   # unified VGPR + AGPR file per lane of a SIMD

# template parameter names per kernel, in order
PARAMS = {
    "fwd_kernel": ["D", "DV", "BC", "NW", "OCC", "CAUSAL", "DROP", "OPT"],
    "dkdv_kernel": ["D", "DV", "BQ", "NW", "CAUSAL", "ATOMIC", "KVL", "DEFER", "DROP"],
    "dkdv_wide_kernel": ["D", "DV", "BQ", "NW", "CAUSAL", "ATOMIC"],
    "dkdv_split_kernel": ["D", "DV", "WIN", "BQ", "NW", "CAUSAL", "ATOMIC"],
    "dq_kernel": ["D", "DV", "BC", "NW", "OCC", "CAUSAL", "DROP"],
    "preprocess_kernel": ["D"],
}


def demangle(name: str):
    """(kernel, {param: value}) from an Itanium-mangled fa:: kernel name, or (name, {})."""
    m = re.match(r"_ZN2fa\d+(\w+?_kernel)I(.*)EEvNS_\d+\w+E$", name)
    if not m:
        return name, {}
    kind, args = m.group(1), m.group(2)
    vals = [int(v) if t == "i" else bool(int(v)) for t, v in re.findall(r"L([ib])(\d+)E", args)]
    return kind, dict(zip(PARAMS.get(kind, []), vals))


def describe(kind: str, p: dict) -> str:
    """The configuration a kernel serves, in the style of the library's configuration names."""
    if not p:
        return kind
    tiles = "" if p.get("DV", p["D"]) == p["D"] else " (tiles %d)" % p["D"]
    d = p.get("DV", p["D"])
    if kind == "fwd_kernel":
        s = "fwd d%d%s Br32x%d Bc%d occ%d" % (d, tiles, p["NW"], p["BC"], p["OCC"])
        return s + (" opt" if p["OPT"] else "") + (" +dropout" if p["DROP"] else "")
    if kind == "dq_kernel":
        return "dq d%d%s Bq32x%d Bc%d occ%d" % (d, tiles, p["NW"], p["BC"], p["OCC"]) + (
            " +dropout" if p["DROP"] else "")
    if kind == "dkdv_wide_kernel":
        return "dkdv%s d%d%s Bk64x%d Bq%d wide" % ("+atomic-dq" if p["ATOMIC"] else "", d, tiles, p["NW"], p["BQ"])
    if kind == "dkdv_split_kernel":
        return "dkdv%s d%d%s Bk32x%d Bq%d kv_regs split%d" % ("+atomic-dq" if p["ATOMIC"] else "", d, tiles, p["NW"],
                                                              p["BQ"], p["WIN"])
    if kind == "dkdv_kernel":
        kvl = {0: "kv_regs", 1: "kv_lds", 2: "k_lds"}[p["KVL"]]
        return "dkdv%s d%d%s Bk32x%d Bq%d %s%s%s" % ("+atomic-dq" if p["ATOMIC"] else "", d, tiles, p["NW"], p["BQ"],
                                                    kvl, " deferred" if p["DEFER"] else "",
                                                    " +dropout" if p["DROP"] else "")
    if kind == "preprocess_kernel":
        return "preprocess d%d" % p["D"]
    return kind


def remarks(src: str) -> list:
    """[(mangled name, {field: value})] from one source's resource-usage remarks."""
    from exact_attention_102_amd.build import FLAGS, hipcc
    cmd = [hipcc()] + FLAGS + ["--cuda-device-only", "-c", "-x", "hip", os.path.join(CSRC, src), "-o", os.devnull,
                               "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s" % (src, r.stderr))
    out, cur = [], None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: +(.*?) \[-Rpass-analysis", line)
        if not m:
            continue
        text = m.group(1).strip()
        if text.startswith("Function Name:"):
            cur = (text.split(":", 1)[1].strip(), {})
            out.append(cur)
        elif cur is not None and ":" in text:
            k, v = text.rsplit(":", 1)
            cur[1][k.strip()] = v.strip()
    return out


def waves_per_cu(vgprs: int, agprs: int, lds: int, nw: int) -> int:
    """Resident waves per CU that the register file (4 SIMDs) and the LDS allow, in whole workgroups."""
    regs = ((vgprs + 3) // 4) * 4 + agprs if agprs else vgprs
    regs = max(8, ((regs + 7) // 8) * 8)
    by_regs = min(8, REGS_PER_SIMD_LANE // regs) * SIMDS_PER_CU     # waves per CU
    wgs = by_regs // nw
    if lds:
        wgs = min(wgs, LDS_PER_CU // lds)
    return wgs * nw


def table() -> list:
    rows = []
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        for src, rem in zip(SOURCES, ex.map(remarks, SOURCES)):
            for name, f in rem:
                kind, p = demangle(name)
                if kind not in PARAMS:
                    continue
                v, a = int(f.get("VGPRs", 0)), int(f.get("AGPRs", 0))
                lds = int(f.get("LDS Size [bytes/block]", 0))
                nw = p.get("NW", 4)
                rows.append({"kernel": describe(kind, p), "mask": "causal" if p.get("CAUSAL") else "full",
                             "vgprs": v, "agprs": a, "vgpr_spill": int(f.get("VGPRs Spill", 0)),
                             "scratch": int(f.get("ScratchSize [bytes/lane]", 0)), "lds": lds,
                             "waves_per_cu": waves_per_cu(v, a, lds, nw), "source": src, "mangled": name})
    return rows


def markdown(rows: list) -> str:
    out = ["| configuration | mask | VGPRs | AGPRs | spilled VGPRs | scratch B/lane | LDS B/workgroup | waves/CU |",
           "|---|---|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: (r["source"], r["kernel"], r["mask"])):
        out.append("| %s | %s | %d | %d | %d | %d | %d | %d |" % (r["kernel"], r["mask"], r["vgprs"], r["agprs"],
                                                                  r["vgpr_spill"], r["scratch"], r["lds"],
                                                                  r["waves_per_cu"]))
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    rows = table()
    body = markdown(rows)
    spills = [r for r in rows if r["vgpr_spill"] or r["scratch"]]
    text = ("# Register, spill, LDS and occupancy per kernel (gfx950)\n\n"
            "Command (from the repository root): `python -m exact_attention_102_amd.resources --out %s`\n\n"
            "From the compiler's kernel-resource-usage remarks for every instantiation in fa_fwd.hip and "
            "fa_bwd.hip, built with the library's flags.  waves/CU = resident waves in whole workgroups that the 512-entry "
            "unified register file of each of the 4 SIMDs and the 160 KB of LDS per CU allow.  Kernels with spills or scratch: %d.\n\n"
            % (a.out or "<file>", len(spills))) + body + "\n"
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text)
    print(text)


if __name__ == "__main__":
    main()
