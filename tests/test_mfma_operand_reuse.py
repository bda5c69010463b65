"""Register reuse behind MFMA instructions, checked in the compiled gfx950 code.

A scorer design that was built and measured on this chip (kept-query
operands in registers, keys staged through LDS) produced wrong products
whenever the compiler placed a VALU instruction that overwrote an MFMA's
B-operand registers within a few instructions of the MFMA: its scores
differed from the current scorer's on about a fifth of the keys, a little
differently from run to run, and matched bit for bit once those registers
were kept live until the products had been consumed. None of the kernels here
contains that pattern; this test compiles every source that issues MFMAs to
assembly and checks that no instruction other than an MFMA, a memory access
or a scalar instruction writes a B-operand register in the WINDOW
instructions after the MFMA that reads it, so that a compiler or source
change that introduces it is caught before it reaches the chip. (A-operand
registers are overwritten right behind an MFMA in the attention and the
scorer, whose results match the oracle: the pattern is only known to matter
for B.)

CPU only: it runs hipcc -S (device code only) and reads the text.
"""
import concurrent.futures
import os
import re
import subprocess

import pytest

from chunked_prefill_kv_amd import build

WINDOW = 6
SOURCES = ["scorer.hip", "attention.hip", "topb.hip"]


def _assembly(src: str) -> str:
    cmd = [build.hipcc(), *build.compile_flags(), *build.FILE_FLAGS.get(src, []),
           "--offload-device-only", "-S", os.path.join(build.CSRC, src), "-o", "-"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc -S {src} failed:\n{p.stderr[-2000:]}")
    return p.stdout


def _kernels(asm: str):
    """{kernel symbol: [instruction lines]} of an assembly listing."""
    out, name, body = {}, None, []
    for raw in asm.splitlines():
        line = raw.strip()
        m = re.match(r"^(_Z\w+):", line)
        if m:
            if name:
                out[name] = body
            name, body = m.group(1), []
            continue
        if name and line and not line.startswith((";", ".")):
            body.append(line)
    if name:
        out[name] = body
    return out


def _regs(tok: str):
    m = re.match(r"[va]\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"[va](\d+)$", tok)
    return {int(m.group(1))} if m else set()


def b_operand_overwrites(lines, window=WINDOW):
    """(mfma, writer) pairs: a non-MFMA vector instruction whose destination
    overlaps the B operand of an MFMA issued at most `window` lines earlier."""
    hits = []
    for i, line in enumerate(lines):
        if not line.startswith("v_mfma"):
            continue
        ops = [t.strip() for t in line.split(None, 1)[1].split(",")]
        b = _regs(ops[2])
        for nxt in lines[i + 1:i + 1 + window]:
            if nxt.startswith(("v_mfma", "s_", "buffer_", "global_", "ds_")):
                continue
            parts = nxt.split(None, 1)
            if len(parts) == 2 and _regs(parts[1].split(",")[0].strip()) & b:
                hits.append((line, nxt))
                break
    return hits


def test_scanner_finds_the_pattern():
    # a hand-written listing with one offending and one harmless reuse
    lines = [
        "v_mfma_f32_16x16x32_bf16 v[76:79], v[8:11], v[68:71], v[76:79]",
        "v_add_u32_e32 v68, v148, v126",
        "v_mfma_f32_16x16x32_bf16 v[80:83], v[8:11], v[72:75], v[80:83]",
        "s_nop 7",
        "v_add_u32_e32 v8, v1, v2",
    ]
    hits = b_operand_overwrites(lines)
    assert len(hits) == 1 and hits[0][1].startswith("v_add_u32_e32 v68")


@pytest.fixture(scope="module")
def listings():
    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        return dict(zip(SOURCES, ex.map(_assembly, SOURCES)))


@pytest.mark.parametrize("src", SOURCES)
def test_no_b_operand_overwrite_behind_mfma(listings, src):
    kernels = _kernels(listings[src])
    mfma_kernels = {k: v for k, v in kernels.items() if any(l.startswith("v_mfma") for l in v)}
    assert mfma_kernels, f"no MFMA kernel found in {src}"
    bad = {k: b_operand_overwrites(v) for k, v in mfma_kernels.items()}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, "\n".join(f"{k}: {v[0][0]}  ->  {v[0][1]} ({len(v)} places)"
                              for k, v in bad.items())
