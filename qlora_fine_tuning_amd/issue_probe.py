"""What other instructions between the MFMAs cost the matrix core, measured on the GPU.

Runs `lora_probe_mfma_issue` in each of its modes (one wave per SIMD on every CU, 128 x iters
bf16 16x16x32 MFMAs per wave) and prints shader cycles per MFMA, averaged over the waves, with
the shader clock each run saw.  The MFMAs alone run at about 16 cycles; the modes add s_nop
blocks of 2, 4 and 6 per MFMA, 20 VALU operations in one block or spread over 8 MFMAs, LDS
operand reads, and LDS DMA copies.

    python -m qlora_fine_tuning_amd.issue_probe [--iters N]
"""
from __future__ import annotations

import argparse

MODES = {
    0: "MFMAs only",
    1: "2 s_nop after every MFMA",
    2: "4 s_nop after every MFMA",
    3: "6 s_nop after every MFMA",
    4: "20 VALU after one MFMA in 8",
    5: "20 VALU spread over 8 MFMAs (2-3 each)",
    6: "operands from LDS: 2 reads per 8 MFMAs",
    7: "1 LDS DMA (16 B/lane) per 8 MFMAs",
}


def measure(mode: int, iters: int = 1000, blocks: int | None = None) -> tuple[float, float]:
    """(shader cycles per MFMA, shader clock in MHz) of one run of `mode`, after a warm-up run."""
    import torch

    from . import lora

    if blocks is None:
        blocks = torch.cuda.get_device_properties(0).multi_processor_count
    for _ in range(2):
        out = lora.lora_probe_mfma_issue(mode, blocks, iters)
        torch.cuda.synchronize()
    o = out.cpu().double()
    cycles, ticks = o[:, 0].mean().item(), o[:, 1].mean().item()
    return cycles / (128.0 * iters), cycles / (ticks / 100.0)


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--iters", type=int, default=1000)
    args = ap.parse_args()
    base = None
    print("| mode | between the MFMAs | cycles per MFMA | added | shader clock (MHz) |")
    print("|---|---|---|---|---|")
    for mode, what in MODES.items():
        cpm, mhz = measure(mode, args.iters)
        base = cpm if base is None else base
        print(f"| {mode} | {what} | {cpm:.2f} | {cpm - base:+.2f} | {mhz:.0f} |", flush=True)


if __name__ == "__main__":
    main()
