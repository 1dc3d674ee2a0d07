"""Runs the gfx950 throughput probes of libbra_micro.so and prints a summary.

    python -m vision_transformer_sparse_amd.micro.run [--out FILE]

Unit probes run `blocks` = CUs x w workgroups of four waves (w waves per
SIMD), each wave stepping a loop whose step issues a fixed number of
independent v_exp_f32 / v_fma_f32 / v_mfma_f32_16x16x32_bf16 instructions.
Reported per probe: the shader clock measured inside the kernel (s_memtime
against s_memrealtime), cycles per step per SIMD, and the rate per clock per
CU of each instruction kind (lanes for exp and fma, flops for the matrix
cores). A mixed probe whose cycles per step equal the larger of its parts'
ran them side by side; equal to their sum, one after the other.
LDS probes: the operand-read patterns of the attention kernels (see
probes.hip), in cycles per 64-lane instruction per CU and bytes per clock
per CU, taking 2.4 GHz.
HBM probes: read, write and copy of 2 GiB, best of five, in GB/s (1e9 B/s).
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libbra_micro.so")

# probe id -> (name, exps, fmas, mfmas per step)
UNIT = {
    0: ("exp", 8, 0, 0),
    1: ("fma", 0, 8, 0),
    2: ("mfma", 0, 0, 4),
    3: ("exp+fma", 8, 8, 0),
    4: ("mfma+exp4", 4, 0, 4),
    5: ("mfma+exp8", 8, 0, 4),
    6: ("mfma+exp8+fma8", 8, 8, 4),
    7: ("mfma+fma8", 0, 8, 4),
    8: ("mfma32", 0, 0, 2),
    9: ("mfma32+exp8", 8, 0, 2),
    18: ("mfma32+exp8+fma8", 8, 8, 2),
    19: ("mfma32x4+exp16", 16, 0, 4),
}
MFMA32 = {8, 9, 18, 19}  # v_mfma_f32_32x32x16_bf16: 32768 flops an instruction
MFMA_FLOPS = 16 * 16 * 32 * 2
# LDS probes: id -> (name, bytes each lane reads per instruction); eight
# instructions a step
LDS = {
    10: ("lds_b128_linear", 16),
    11: ("lds_b128_K_swizzled", 16),
    12: ("lds_b128_K_plain", 16),
    13: ("lds_b128_K_pitch80", 16),
    14: ("lds_tr_b64_V_swizzled", 8),
    15: ("lds_tr_b64_V_plain", 8),
    16: ("lds_tr_b64_V_pitch80", 8),
    17: ("lds_tr_b64_contiguous", 8),
}


def load():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: build with `python -m vision_transformer_sparse_amd.build`")
    lib = ctypes.CDLL(LIB)
    d = ctypes.POINTER(ctypes.c_double)
    lib.micro_unit.argtypes = [ctypes.c_int] * 4 + [d, d, d]
    lib.micro_unit.restype = ctypes.c_int
    lib.micro_hbm.argtypes = [ctypes.c_int, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, d]
    lib.micro_hbm.restype = ctypes.c_int
    lib.micro_error.restype = ctypes.c_char_p
    lib.micro_cu_count.restype = ctypes.c_int
    return lib


def unit(lib, probe, w, cus, iters):
    ms, clk, span = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    rc = lib.micro_unit(probe, cus * w, iters, 3, ctypes.byref(ms), ctypes.byref(clk), ctypes.byref(span))
    if rc:
        raise RuntimeError(lib.micro_error().decode())
    name, ne, nf, nm = UNIT[probe]
    t = ms.value * 1e-3
    steps_per_simd = w * iters * 4
    cyc = t * clk.value * 1e6 / steps_per_simd
    row = {"probe": name, "w": w, "ms": ms.value, "clk_mhz": clk.value, "span": span.value,
           "cycles_per_step": cyc}
    waves = cus * w * 4
    for kind, n, per in (("exp", ne, 64), ("fma", nf, 64),
                         ("mfma", nm, MFMA_FLOPS * (2 if probe in MFMA32 else 1))):
        if n:
            total = waves * iters * 4 * n * per
            row[f"{kind}_per_clk_cu"] = total / t / (cus * clk.value * 1e6)
    return row


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None, help="also write the summary to this file")
    ap.add_argument("--iters", type=int, default=4000)
    a = ap.parse_args(argv)
    lib = load()
    cus = lib.micro_cu_count()
    lines = [f"# gfx950 throughput probes (libbra_micro.so), {cus} CUs",
             f"# command: python -m vision_transformer_sparse_amd.micro.run"
             + (f" --out {a.out}" if a.out else ""),
             "# probe, waves/SIMD, kernel ms, clock MHz (in-kernel), cycles/step/SIMD, rates per clock per CU"]
    for probe in UNIT:
        for w in (1, 2, 4, 8):
            r = unit(lib, probe, w, cus, a.iters)
            rates = " ".join(f"{k}={v:.2f}" for k, v in r.items() if k.endswith("_per_clk_cu"))
            s = (f"{r['probe']:16s} w={w} ms={r['ms']:.3f} clk={r['clk_mhz']:.0f} "
                 f"cyc/step={r['cycles_per_step']:.2f} {rates}")
            print(s, flush=True)
            lines.append(s)
    for probe, (name, nb) in LDS.items():
        for w in (2, 4):
            ms, clk, span = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
            rc = lib.micro_unit(probe, cus * w, a.iters, 3, ctypes.byref(ms), ctypes.byref(clk), ctypes.byref(span))
            if rc:
                raise RuntimeError(lib.micro_error().decode())
            t = ms.value * 1e-3
            instrs_per_cu = w * 4 * a.iters * 8  # waves per CU x steps x reads
            byts = instrs_per_cu * 64 * nb
            s = (f"{name:24s} w={w} ms={ms.value:.3f} cycles/instr/CU={t * 2.4e9 / instrs_per_cu:.2f} "
                 f"B/clk/CU={byts / (t * 2.4e9):.1f} (at 2.4 GHz)")
            print(s, flush=True)
            lines.append(s)
    for kind, name in ((0, "read"), (1, "write"), (2, "copy")):
        ms = ctypes.c_double()
        nbytes = 2 << 30
        rc = lib.micro_hbm(kind, nbytes, cus * 16, 5, ctypes.byref(ms))
        if rc:
            raise RuntimeError(lib.micro_error().decode())
        moved = nbytes * (2 if kind == 2 else 1)
        s = f"hbm_{name:5s} bytes={moved} ms={ms.value:.3f} GB/s={moved / (ms.value * 1e-3) / 1e9:.1f}"
        print(s, flush=True)
        lines.append(s)
    if a.out:
        with open(a.out, "w") as f:
            f.write("\n".join(lines) + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
