"""Static check of the gfx950 assembly the kernels compile to (CPU only: hipcc cross-compiles).

An MFMA whose accumulator input (SrcC) was produced by one of the previous
two MFMAs waits in the matrix pipeline after issue and reads its A/B source
registers late. A VALU op or an LDS / global load that rewrites one of those
registers soon after can land first and silently corrupt the product (seen
on MI355X as missing key blocks in P V). The kernels pin their MFMA order so
this never happens; this test fails if a compiler change or a kernel edit
brings the pattern back.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "swin3d_window_attention_amd", "csrc")
SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))

NEAR_MFMAS = 3      # a SrcC produced this many MFMAs back or fewer counts as "in flight"
WINDOW_INSTRS = 40  # instructions after such an MFMA in which its A/B must not be rewritten


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _kernels(asm_text):
    """Map kernel symbol -> list of instruction lines."""
    out, cur = {}, None
    for line in asm_text.splitlines():
        s = line.strip()
        m = re.match(r"^(_Z\S+):\s*(;.*)?$", s)
        if m and not s.startswith("."):
            cur = m.group(1)
            out[cur] = []
            continue
        if cur is None or not s or s.startswith((";", ".")) or s.endswith(":"):
            if s.startswith("s_endpgm"):
                cur = None
            continue
        out[cur].append(s)
        if s.startswith("s_endpgm"):
            cur = None
    return out


def stalled_mfma_war(instrs):
    """(hits, MFMA count). An MFMA counts as stalled when a register of its SrcC still holds the
    result of one of the previous NEAR_MFMAS MFMAs; a register that a load or a VALU op has
    rewritten since (an accumulator started from a value in LDS, say) no longer does."""
    hits, mfmas, risky = [], [], []
    for i, line in enumerate(instrs):
        parts = re.split(r"[\s,]+", line)
        op = parts[0]
        risky = [r for r in risky if i - r[0] <= WINDOW_INSTRS]
        if op.startswith("v_mfma"):
            dst, a, b, c = (_regs(p) for p in parts[1:5])
            stalled = bool(c) and any(c & d for _, d in mfmas[-NEAR_MFMAS:])
            mfmas.append((i, set(dst)))
            if stalled:
                risky.append((i, a | b, line))
            continue
        if op.startswith(("v_", "ds_read", "global_load", "buffer_load")) and len(parts) > 1:
            dst = _regs(parts[1])
            for j, srcs, text in risky:
                if dst & srcs:
                    hits.append((j, i, text, line))
            for _, d in mfmas[-NEAR_MFMAS:]:
                d -= dst
    return hits, len(mfmas)


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    """gfx950 assembly of every kernel source, concatenated."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    tmp = tmp_path_factory.mktemp("isa")
    text = []
    for src in SOURCES:
        out = tmp / (os.path.basename(src) + ".s")
        cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", str(out)]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout
        text.append(out.read_text())
    return "\n".join(text)


def test_scanner_flags_the_pattern():
    """The scanner itself: a dependent MFMA followed by an LDS load into its A operand is flagged."""
    bad = ["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
           "v_mfma_f32_16x16x32_bf16 v[0:3], v[12:15], v[8:11], v[0:3]",
           "ds_read2_b64 v[12:15], v20 offset1:4"]
    hits, _ = stalled_mfma_war(bad)
    assert len(hits) == 1
    ok = ["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
          "v_mfma_f32_16x16x32_bf16 v[16:19], v[4:7], v[8:11], 0",
          "v_mfma_f32_16x16x32_bf16 v[20:23], v[4:7], v[8:11], 0",
          "v_mfma_f32_16x16x32_bf16 v[24:27], v[4:7], v[8:11], 0",
          "v_mfma_f32_16x16x32_bf16 v[0:3], v[12:15], v[8:11], v[0:3]",
          "ds_read2_b64 v[12:15], v20 offset1:4"]
    assert stalled_mfma_war(ok)[0] == []
    # an accumulator reloaded from LDS after the MFMA that last wrote it is not in flight
    reloaded = ["v_mfma_f32_16x16x4_f32 v[0:3], v4, v8, v[0:3]",
                "ds_read_b128 v[0:3], v20",
                "v_mfma_f32_16x16x4_f32 v[0:3], v5, v8, v[0:3]",
                "ds_read_b128 v[4:7], v20 offset:16"]
    assert stalled_mfma_war(reloaded)[0] == []
    # ... but a partial reload leaves the rest of the accumulator in flight
    partial = ["v_mfma_f32_16x16x4_f32 v[0:3], v4, v8, v[0:3]",
               "v_mov_b32_e32 v0, 0",
               "v_mfma_f32_16x16x4_f32 v[0:3], v5, v8, v[0:3]",
               "ds_read_b128 v[4:7], v20 offset:16"]
    assert len(stalled_mfma_war(partial)[0]) == 1


def test_no_stalled_mfma_operand_overwrite(asm):
    kernels = _kernels(asm)
    assert any("wattn_bf16" in k for k in kernels), list(kernels)
    total = 0
    for name, instrs in kernels.items():
        hits, n = stalled_mfma_war(instrs)
        total += n
        assert not hits, f"{name}: {len(hits)} risky overwrites, first: {hits[0]}"
    assert total > 0  # the matrix-core kernel was scanned


def test_no_register_spills(asm):
    """Every kernel keeps its registers: a spill to scratch makes the gather wait for all of its
    loads before it can park them, which costs the bf16 kernel about a tenth of its speed."""
    sizes = re.findall(r"\.amdhsa_kernel\s+(\S+).*?\.amdhsa_private_segment_fixed_size\s+(\d+)", asm, re.S)
    assert sizes and any("wattn_bf16" in k for k, _ in sizes)
    assert all(int(n) == 0 for _, n in sizes), sizes


def test_bf16_kernel_occupancy(asm):
    """Four workgroups of the matrix-core kernel share a CU (four waves per SIMD)."""
    m = re.search(r"wattn_bf16_item\w*:.*?; Occupancy: (\d+)", asm, re.S)
    assert m and int(m.group(1)) >= 4


def _reg_range(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return int(m.group(1)), int(m.group(2))
    m = re.match(r"v(\d+)$", tok)
    return (int(m.group(1)), int(m.group(1))) if m else None


def _kernels_with_labels(asm_text):
    """Map kernel symbol -> instruction lines, with '<label>' marking basic-block starts."""
    out, cur = {}, None
    for line in asm_text.splitlines():
        s = line.strip()
        m = re.match(r"^(_Z\S+):\s*(;.*)?$", s)
        if m:
            cur = m.group(1)
            out[cur] = []
            continue
        if cur is None or not s or s.startswith(";") or (s.startswith(".") and not s.endswith(":")):
            continue
        out[cur].append("<label>" if s.endswith(":") else s)
        if s.startswith("s_endpgm"):
            cur = None
    return out


def dead_load_words(instrs):
    """16-byte global loads one of whose destination words is overwritten, inside the same basic
    block, before anything reads it. That is either wasted bandwidth or a miscompile: the compiler
    once built a bf16 split element by element and took every element from word 0 of the load."""
    hits = []
    for i, line in enumerate(instrs):
        m = re.match(r"global_load_dwordx4 v\[(\d+):(\d+)\]", line)
        if not m:
            continue
        for r in range(int(m.group(1)), int(m.group(2)) + 1):
            for later in instrs[i + 1:]:
                if later == "<label>" or later.startswith(("s_cbranch", "s_branch", "s_setpc")):
                    break
                parts = re.split(r"[\s,]+", later)
                # multiply-accumulate forms (v_fmac, v_mac, ...) read their destination too
                first_src = 1 if "mac" in parts[0] else 2
                srcs = [_reg_range(p) for p in parts[first_src:]]
                if any(s and s[0] <= r <= s[1] for s in srcs) or parts[0].startswith(("ds_write", "global_store")) \
                        and any(s and s[0] <= r <= s[1] for s in [_reg_range(p) for p in parts[1:]]):
                    break
                dst = _reg_range(parts[1]) if len(parts) > 1 else None
                if dst and dst[0] <= r <= dst[1] and not parts[0].startswith(("s_", "ds_write", "global_store")):
                    hits.append((i, r, line, later))
                    break
    return hits


def test_every_loaded_word_is_used(asm):
    kernels = _kernels_with_labels(asm)
    for name, instrs in kernels.items():
        hits = dead_load_words(instrs)
        assert not hits, f"{name}: {len(hits)} loaded words overwritten unread, first: {hits[0]}"


def test_dead_word_scanner_flags_the_pattern():
    bad = ["global_load_dwordx4 v[0:3], v6, s[0:1] nt",
           "v_cvt_pk_bf16_f32 v1, v0, s0",
           "global_store_dwordx4 v6, v[1:4], s[2:3]"]
    assert dead_load_words(bad)
    ok = ["global_load_dwordx4 v[0:3], v6, s[0:1] nt",
          "ds_write_b128 v7, v[0:3]",
          "v_mov_b32_e32 v1, 0"]
    assert not dead_load_words(ok)
