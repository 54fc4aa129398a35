"""Properties of the gfx950 code the kernels compile to (CPU only: hipcc cross-compiles).

Every HIP source is compiled to assembly with the library's own flags, and the listing is
checked for rules the design relies on:

* m0 is written only by the direct global-to-LDS load sequences (`s_add_u32 m0, ...`,
  then one `s_nop 0`, then `buffer_load_dwordx4 ... lds`): on this GFX9-family target a
  scalar-ALU write of m0 needs one wait state before an LDS-DMA load reads it, and the
  compiler's hazard recogniser cannot see inside the inline assembly that issues them, so
  the sequence must carry the wait itself;
* the cross-lane operations the sequential kernel issues as inline assembly
  (`v_permlane16_swap_b32`, the in-place `v_mov_b32_dpp ... row_bcast:15`) each carry the
  two wait states (`s_nop 1`) they need after a vector-ALU write of their operands, since
  the compiler's hazard recogniser cannot see inside the assembly either;
* no packed FP32 vector instruction (`v_pk_add_f32`, `v_pk_mul_f32`, `v_pk_fma_f32`)
  appears: the build disables them;
* no scalar memory store or scalar atomic appears: every store goes through the vector
  memory path;
* the fused scan kernel has no scratch (register spill) traffic where it works: no basic
  block that runs matrix products or touches the LDS accesses scratch, so the state and
  the operands stay in registers; at most a few scratch accesses sit outside those blocks
  (a pointer the compiler parks across the chunk loop, stored before it, loaded after it).
"""
import os
import re
import shutil
import subprocess

import pytest

from linear_attention_recurrence_gated_amd import build

HIPCC = build.HIPCC


def _device_asm(src):
    out = os.path.join(build.BUILD_DIR, os.path.basename(src) + ".s")
    os.makedirs(build.BUILD_DIR, exist_ok=True)
    flags = [f for f in build.FLAGS if f not in ("-fPIC",)]
    r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", out],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return f.read()


def _instructions(text):
    """(function, mnemonic, line) of every instruction of the listing."""
    fn = None
    for line in text.splitlines():
        m = re.match(r"^([A-Za-z_.$][\w.$]*):", line)
        if m and not m.group(1).startswith(".L"):
            fn = m.group(1)
            continue
        s = line.strip()
        if not s or s.startswith((";", ".", "//")) or s.endswith(":"):
            continue
        yield fn, s.split()[0], s


@pytest.fixture(scope="module")
def listings():
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    srcs = sorted(os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC)
                  if f.endswith(".hip"))
    return {os.path.basename(s): list(_instructions(_device_asm(s))) for s in srcs}


def test_m0_only_addressed_by_direct_loads(listings):
    seen = 0
    for name, ins in listings.items():
        for i, (fn, op, line) in enumerate(ins):
            if re.search(r"\bm0\b", line):
                assert op == "s_add_u32" and line.split()[1] == "m0,", (name, fn, line)
                # one wait state between the scalar write of m0 and the load that reads it
                assert ins[i + 1][1] == "s_nop" and ins[i + 1][2].split()[1] == "0", \
                    (name, line, ins[i + 1][2])
                nxt = ins[i + 2][2]
                assert nxt.startswith("buffer_load_dwordx4") and nxt.endswith(" lds"), (name, line, nxt)
                seen += 1
    assert seen > 0  # the direct loads are there


def test_every_direct_load_follows_its_m0_write_with_a_wait_state(listings):
    """Each LDS-DMA load is preceded by `s_nop 0` and, before that, the m0 write."""
    seen = 0
    for name, ins in listings.items():
        for i, (fn, op, line) in enumerate(ins):
            if op.startswith("buffer_load") and line.endswith(" lds"):
                assert ins[i - 1][1] == "s_nop", (name, fn, ins[i - 1][2], line)
                assert ins[i - 2][1] == "s_add_u32" and ins[i - 2][2].split()[1] == "m0,", \
                    (name, fn, ins[i - 2][2], line)
                seen += 1
    assert seen > 0


def test_inline_cross_lane_operations_carry_their_wait_states(listings):
    ins = listings["gdn_seq.hip"]
    seen = {"v_permlane16_swap_b32": 0, "row_bcast": 0}
    for i, (fn, op, line) in enumerate(ins):
        kind = ("v_permlane16_swap_b32" if op == "v_permlane16_swap_b32" else
                "row_bcast" if op == "v_mov_b32_dpp" and "row_bcast:15" in line else None)
        if kind is None:
            continue
        prev = ins[i - 1][2].split()
        assert prev[0] == "s_nop" and int(prev[1]) >= 1, (fn, line, ins[i - 1][2])
        seen[kind] += 1
    assert all(n > 0 for n in seen.values()), seen


def test_no_packed_fp32_vector_instructions(listings):
    for name, ins in listings.items():
        bad = [line for _, op, line in ins if op in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32")]
        assert not bad, (name, bad[:3])


def test_no_scalar_memory_writes(listings):
    for name, ins in listings.items():
        bad = [line for _, op, line in ins
               if op.startswith(("s_store", "s_buffer_store", "s_scratch_store", "s_atomic",
                                 "s_buffer_atomic", "s_dcache_wb"))]
        assert not bad, (name, bad[:3])


def _blocks(text, kernel):
    """Basic blocks (lists of instruction lines) of the function whose name contains
    `kernel`: a block ends at a label or after a branch."""
    blocks, cur, inside = [], [], False
    for line in text.splitlines():
        m = re.match(r"^([A-Za-z_.$][\w.$]*):", line)
        if m and not m.group(1).startswith(".L"):
            inside = kernel in m.group(1)
            continue
        if not inside:
            continue
        s = line.strip()
        if m or s.startswith("; %bb."):
            blocks.append(cur)
            cur = []
            continue
        if not s or s.startswith((";", ".", "//")) or s.endswith(":"):
            continue
        cur.append(s)
        if s.startswith(("s_cbranch", "s_branch", "s_endpgm")):
            blocks.append(cur)
            cur = []
    blocks.append(cur)
    return [b for b in blocks if b]


def test_fused_kernel_keeps_its_work_in_registers(listings):
    text = _device_asm(os.path.join(build.CSRC, "gdn_chunk.hip"))
    blocks = _blocks(text, "chunk_fused_kernel")
    assert sum(any(i.startswith("v_mfma") for i in b) for b in blocks) > 0
    scratch = [i for b in blocks for i in b if i.startswith("scratch_")]
    assert len(scratch) <= 4, scratch
    for b in blocks:
        works = any(i.startswith(("v_mfma", "ds_read", "ds_write", "buffer_load")) for i in b)
        bad = [i for i in b if i.startswith("scratch_")]
        assert not (works and bad), (bad, b[:8])
