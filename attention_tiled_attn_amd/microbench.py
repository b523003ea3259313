"""Microbenchmarks of the gfx950 units the attention kernels lean on.

    python -m attention_tiled_attn_amd.microbench [--json]

Runs the kernels of csrc/microbench.hip (libflexattn_mb.so, built beside the
attention library) on cuda:0 and reports, per unit:

* bf16 matrix cores: v_mfma_f32_32x32x16_bf16 cycles per instruction per SIMD
  with one and with two waves on a SIMD, the shader clock under that load and
  the TFLOP/s it sustains (32768 FLOP per instruction);
* exponential (v_exp_f32) and plain vector FMA (v_fma_f32): results per clock
  per CU and cycles per instruction of one wave, alone and two per SIMD, and
  one wave issuing both;
* interference: a wave multiplying while the other wave of its SIMD issues
  FMAs or exponentials; the extra matrix cycles per instruction of the other
  wave, and the other way round, the vector wave's cycles per instruction
  while every one of its instructions has a multiplying partner;
* LDS: bytes per clock per CU read with ds_read_b128 (conflict-free rows) and
  with the transposing ds_read_b64_tr_b16;
* HBM: read and copy bandwidth over 1 GiB.

The figures describe the hardware, not the attention kernels: they are the
context for the kernels' counter summaries (what the matrix cores sustain at
the clock the chip actually runs, what the vector side costs them). The
roofline fractions themselves use the published peaks. Measurement tooling,
not part of the attention library's C ABI.
"""
from __future__ import annotations

import ctypes
import json
import os
import statistics as st
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
MB_PATH = os.path.join(HERE, "libflexattn_mb.so")
REALTIME_HZ = 100e6      # s_memrealtime counts at a constant 100 MHz
MFMA_FLOP = 32 * 32 * 16 * 2
CUS = 256

MFMA, EXP, FMA, MIX_FMA, MIX_EXP, LDS, LDS_TR, EXP_FMA = range(8)


def _lib():
    if not os.path.exists(MB_PATH):
        raise RuntimeError(f"{MB_PATH} is missing: build it with python -m attention_tiled_attn_amd.build")
    lib = ctypes.CDLL(MB_PATH)
    lib.flexattn_mb_units.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.flexattn_mb_read.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p]
    lib.flexattn_mb_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_int,
                                     ctypes.c_void_p]
    for f in (lib.flexattn_mb_units, lib.flexattn_mb_read, lib.flexattn_mb_copy):
        f.restype = ctypes.c_int
    return lib


def _units(lib, torch, kind, wps, iters, iters_vec=1, wgs=CUS):
    """Per-wave (cycles, real-time ticks, operations) of one launch, and its
    event time in seconds."""
    waves = wgs * 4 * wps
    rec = torch.zeros(waves * 3, dtype=torch.int64, device="cuda")
    sink = torch.zeros(wgs, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(2):   # the first launch warms the clock and the code
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = lib.flexattn_mb_units(kind, wps, iters, iters_vec, wgs, rec.data_ptr(), sink.data_ptr(), stream)
        e1.record()
        if rc != 0:
            raise RuntimeError(f"flexattn_mb_units({kind}, {wps}) returned {rc}")
        torch.cuda.synchronize()
    r = rec.view(waves, 3).cpu().tolist()
    return r, e0.elapsed_time(e1) * 1e-3


def _wave_rows(r, wps, which):
    """Rows of the waves in the given half (0: waves 0-3, 1: waves 4-7 of
    each workgroup), or all."""
    per = 4 * wps
    return [row for i, row in enumerate(r) if which is None or (i % per) // 4 == which]


def run() -> dict:
    import torch
    torch.cuda.init()
    lib = _lib()
    out = {"gpu": torch.cuda.get_device_name(0)}

    # matrix cores. Cycles per MFMA per SIMD over the launch (event time x
    # clock): the two waves of a SIMD need not run over the same interval, so
    # one wave's own span says nothing about the SIMD's rate then
    for wps in (1, 2):
        r, t = _units(lib, torch, MFMA, wps, 4000)
        cyc = st.median(c for c, _, _ in r)
        ops = r[0][2]
        clk = st.median(c / (w / REALTIME_HZ) for c, w, _ in r) / 1e9
        total = sum(o for _, _, o in r)
        out[f"mfma_{wps}w"] = {
            "cycles_per_mfma_per_simd": t * clk * 1e9 / (ops * wps),
            "wave_cycles_per_own_mfma": cyc / ops,
            "clock_ghz": clk,
            "tflops": total * MFMA_FLOP / t / 1e12,
            # the longest wave by the real-time counter against the launch's
            # event time: checks the counter's assumed 100 MHz
            "realtime_over_events": max(w for _, w, _ in r) / REALTIME_HZ / t,
        }
    # exponential and FMA
    for kind, name in ((EXP, "exp"), (FMA, "fma")):
        for wps in (1, 2):
            r, _ = _units(lib, torch, kind, wps, 20000)
            cyc = st.median(c for c, _, _ in r)
            ops = r[0][2]
            out[f"{name}_{wps}w"] = {
                "cycles_per_instr_per_wave": cyc / ops,
                "results_per_clock_per_cu": 4 * wps * ops * 64 / cyc,
            }
    # one wave issuing 16 exponentials and 32 FMAs per step: against the sum
    # and the larger of the two alone
    r, _ = _units(lib, torch, EXP_FMA, 1, 10000)
    cyc = st.median(c for c, _, _ in r) / 10000
    e1, f1 = out["exp_1w"]["cycles_per_instr_per_wave"], out["fma_1w"]["cycles_per_instr_per_wave"]
    out["exp_and_fma_1w"] = {"cycles_per_step": cyc, "exp_alone": 16 * e1, "fma_alone": 32 * f1,
                             "sum_alone": 16 * e1 + 32 * f1}
    # interference: MFMA waves 0-3, vector waves 4-7; the vector waves run
    # longer than the MFMA waves, so every MFMA has a busy partner. The cost
    # per partner instruction takes the partner's issue interval from its
    # one-wave run (an estimate: its interval while the MFMA wave runs is not
    # observed on its own).
    base = out["mfma_1w"]["wave_cycles_per_own_mfma"]
    for kind, name, viters in ((MIX_FMA, "fma", 60000), (MIX_EXP, "exp", 30000)):
        r, _ = _units(lib, torch, kind, 2, 4000, viters)
        m_rows, v_rows = _wave_rows(r, 2, 0), _wave_rows(r, 2, 1)
        mc = st.median(c for c, _, _ in m_rows)
        mops = m_rows[0][2]
        cpm = mc / mops
        solo = out[f"{name}_1w"]["cycles_per_instr_per_wave"]
        out[f"mfma_beside_{name}"] = {
            "cycles_per_mfma": cpm,
            "partner_instr_per_mfma": cpm / solo,
            "extra_mfma_cycles_per_partner_instr": (cpm - base) / (cpm / solo),
            "partner_outlasted_mfma_waves": st.median(c for c, _, _ in v_rows) >= mc,
        }
        # the vector wave's own rate beside the products: a vector loop a
        # third as long as the MFMA loop (by the one-wave rates), so that it
        # ends while its partner is still multiplying
        short = max(1, int(mc / 3 / (solo * 16)))
        r, _ = _units(lib, torch, kind, 2, 4000, short)
        m_rows, v_rows = _wave_rows(r, 2, 0), _wave_rows(r, 2, 1)
        vc = st.median(c for c, _, _ in v_rows)
        out[f"{name}_beside_mfma"] = {
            "cycles_per_instr": vc / v_rows[0][2],
            "alone_cycles_per_instr": solo,
            "slowdown": vc / v_rows[0][2] / solo,
            "ended_before_mfma_waves": vc < st.median(c for c, _, _ in m_rows),
        }
    # LDS
    for wps in (1, 2):
        r, _ = _units(lib, torch, LDS, wps, 20000)
        cyc = st.median(c for c, _, _ in r)
        ops = r[0][2]
        out[f"lds_{wps}w"] = {"bytes_per_clock_per_cu": 4 * wps * ops * 1024 / cyc,
                              "cycles_per_read_per_wave": cyc / ops}
        r, _ = _units(lib, torch, LDS_TR, wps, 10000)
        cyc = st.median(c for c, _, _ in r)
        ops = r[0][2]
        out[f"lds_tr_{wps}w"] = {"bytes_per_clock_per_cu": 4 * wps * ops * 512 / cyc,
                                 "cycles_per_read_per_wave": cyc / ops}
    # HBM
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(CUS * 8 * 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for name, call, moved in (
            ("hbm_read", lambda: lib.flexattn_mb_read(src.data_ptr(), n, sink.data_ptr(), CUS * 8, stream), n),
            ("hbm_copy", lambda: lib.flexattn_mb_copy(src.data_ptr(), dst.data_ptr(), n, CUS * 8, stream), 2 * n)):
        times = []
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = call()
            e1.record()
            if rc != 0:
                raise RuntimeError(f"{name} returned {rc}")
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        t = st.median(times[1:])
        out[name] = {"gb_per_s": moved / t / 1e9, "bytes": moved}
    return out


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    res = run()
    if "--json" in argv:
        print(json.dumps(res))
        return 0
    print(f"gpu: {res['gpu']}")
    for k, v in res.items():
        if k == "gpu":
            continue
        print(f"{k:24s} " + ", ".join(f"{a} = {b:.4g}" if isinstance(b, float) else f"{a} = {b}"
                                       for a, b in v.items()))
    return 0


if __name__ == "__main__":
    sys.exit(main())
