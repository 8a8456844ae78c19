"""Code-generation invariants of the decode kernel (host only: hipcc
cross-compiles gfx950 here).  Each guards a regression that once cost tens
of percent while every numeric test still passed:

* no scratch (register spills) in the instances the library launches;
* no agent-scope L2 writeback / invalidate (each one flushes an XCD's L2)
  except the in-kernel merge's release increment and last-split acquire;
* the main loop keeps the next granule's loads in flight: its first waits
  on vector memory leave at least 8 loads outstanding (a wait for zero there
  means the loop drains every load each granule -- seen when a pending load
  of uncertain provenance reached the loop, and when block-table reads
  turned into vector loads);
* head-group instances of the packed formats (e2m3, e3m2, e2m1) keep their
  waves together with one workgroup barrier in the main loop, and no wait on
  memory precedes it (a wait there would drain the granule loads in flight);
  nvfp4 instances have none;
* no scaled MFMA has its E8M0 scale register rewritten within the next 24
  instructions: the instruction still reads it after issue and the compiler
  does not wait for that (a register-only probe whose scale register was
  reused two instructions later got wrong products in 15 of 16 rows).
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "paged_fp8_decode_amd", "csrc", "mj_decode_mfma.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# the instances the default dispatch launches: (operand format, rows per block,
# row blocks, KV cache policy, prefetch, waves per SIMD, waves per workgroup,
# KV heads per workgroup)
DEFAULT = [
           "Li0ELi4ELi1ELi2ELi1ELi2ELi4ELi1E", "Li0ELi8ELi1ELi2ELi1ELi2ELi4ELi1E", "Li0ELi16ELi1ELi2ELi1ELi2ELi4ELi1E",
           "Li0ELi16ELi2ELi2ELi1ELi2ELi4ELi1E", "Li0ELi16ELi2ELi2ELi1ELi2ELi8ELi1E", "Li1ELi4ELi1ELi2ELi1ELi2ELi4ELi1E",
           "Li1ELi8ELi1ELi2ELi1ELi2ELi4ELi1E", "Li1ELi16ELi1ELi2ELi1ELi2ELi4ELi1E", "Li1ELi16ELi2ELi2ELi1ELi1ELi4ELi1E",
           "Li2ELi4ELi1ELi2ELi1ELi2ELi4ELi1E", "Li2ELi8ELi1ELi2ELi1ELi2ELi4ELi1E", "Li2ELi16ELi1ELi2ELi1ELi2ELi4ELi1E",
           "Li2ELi16ELi2ELi2ELi1ELi1ELi4ELi1E", "Li3ELi4ELi1ELi2ELi1ELi2ELi4ELi1E", "Li3ELi8ELi1ELi2ELi1ELi2ELi4ELi1E",
           "Li3ELi16ELi1ELi2ELi1ELi2ELi4ELi1E", "Li3ELi16ELi2ELi2ELi1ELi1ELi4ELi1E", "Li4ELi4ELi1ELi2ELi1ELi2ELi4ELi1E",
           "Li4ELi8ELi1ELi2ELi1ELi2ELi4ELi1E", "Li4ELi16ELi1ELi2ELi1ELi2ELi4ELi1E", "Li4ELi16ELi2ELi2ELi1ELi2ELi4ELi1E",
           "Li4ELi16ELi2ELi2ELi1ELi2ELi8ELi1E", "Li5ELi4ELi1ELi2ELi1ELi2ELi4ELi1E", "Li5ELi8ELi1ELi2ELi1ELi2ELi4ELi1E",
           "Li5ELi16ELi1ELi2ELi1ELi2ELi4ELi1E", "Li5ELi16ELi2ELi2ELi1ELi1ELi4ELi1E", "Li6ELi4ELi1ELi2ELi1ELi2ELi4ELi1E",
           "Li6ELi8ELi1ELi2ELi1ELi2ELi4ELi1E", "Li6ELi16ELi1ELi2ELi1ELi2ELi4ELi1E", "Li6ELi16ELi2ELi2ELi1ELi1ELi4ELi1E",
           "Li1ELi4ELi1ELi0ELi1ELi2ELi4ELi4E", "Li1ELi8ELi1ELi0ELi1ELi2ELi4ELi4E", "Li1ELi16ELi1ELi0ELi1ELi2ELi4ELi4E",
           "Li3ELi4ELi1ELi0ELi1ELi2ELi4ELi4E", "Li3ELi8ELi1ELi0ELi1ELi2ELi4ELi4E", "Li3ELi16ELi1ELi0ELi1ELi2ELi4ELi4E",
           "Li4ELi4ELi1ELi0ELi1ELi2ELi4ELi4E", "Li4ELi8ELi1ELi0ELi1ELi2ELi4ELi4E", "Li4ELi16ELi1ELi0ELi1ELi2ELi4ELi4E",
           "Li5ELi4ELi1ELi0ELi1ELi2ELi4ELi4E", "Li5ELi8ELi1ELi0ELi1ELi2ELi4ELi4E", "Li5ELi16ELi1ELi0ELi1ELi2ELi4ELi4E",
           "Li6ELi4ELi1ELi0ELi1ELi2ELi4ELi4E", "Li6ELi8ELi1ELi0ELi1ELi2ELi4ELi4E", "Li6ELi16ELi1ELi0ELi1ELi2ELi4ELi4E",
           "Li4ELi4ELi1ELi0ELi1ELi2ELi8ELi8E", "Li4ELi8ELi1ELi0ELi1ELi2ELi8ELi8E", "Li4ELi16ELi1ELi0ELi1ELi2ELi8ELi8E"]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "mfma.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fhip-fp32-correctly-rounded-divide-sqrt",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics", "--cuda-device-only",
           "-S", "-o", str(out), SRC]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return out.read_text().splitlines()


def _body(lines, inst):
    name = f"_ZN2mj12_GLOBAL__N_118decode_mfma_kernelI{inst}EEvNS_12DecodeParamsE:"
    i = next(j for j, l in enumerate(lines) if l.startswith(name))
    e = next(j for j in range(i, len(lines)) if "s_endpgm" in lines[j])
    meta = next(j for j in range(e, len(lines)) if lines[j].strip().startswith(".private_segment_fixed_size") or
                ".private_segment_fixed_size" in lines[j])
    return lines[i:e], lines[e:meta + 1]


@pytest.mark.parametrize("inst", DEFAULT)
def test_no_scratch_and_no_l2_flush(asm, inst):
    body, meta = _body(asm, inst)
    scratch = [l for l in meta if ".private_segment_fixed_size" in l]
    assert scratch and int(scratch[-1].split()[-1]) == 0, scratch
    text = "\n".join(body)
    # the only L2 writeback / invalidate: the in-kernel merge's arrival (one
    # agent-scope release increment by one thread per workgroup, then the
    # last split's acquire; both run only when the launch merges its own
    # partials); instances of several KV heads per workgroup have no
    # in-kernel merge, hence none
    wb = [j for j, l in enumerate(body) if "buffer_wbl2" in l]
    inv = [j for j, l in enumerate(body) if "buffer_inv" in l]
    heads_per_wg = int(re.findall(r"Li(\d+)E", inst)[-1])
    if heads_per_wg > 1:
        assert not wb and not inv, (wb, inv)
    else:
        assert len(wb) == 1 and len(inv) == 1, (wb, inv)
        assert "global_atomic_add" in "\n".join(body[wb[0]:inv[0]]) and 0 < inv[0] - wb[0] <= 40
    assert "scratch_" not in text


@pytest.mark.parametrize("inst", DEFAULT)
def test_main_loop_keeps_loads_in_flight(asm, inst):
    body, _ = _body(asm, inst)
    heads = [j for j, l in enumerate(body) if "Loop Header" in l]
    loop = next(j for j in heads if any("v_mfma" in x for x in body[j:j + 300]) and
                any("buffer_load" in x for x in body[j:j + 300]))
    waits = [int(re.search(r"vmcnt\((\d+)\)", x).group(1)) for x in body[loop:loop + 1500] if "vmcnt(" in x][:4]
    assert len(waits) == 4 and min(waits) >= 8, waits


@pytest.mark.parametrize("inst", [i for i in DEFAULT if not i.endswith("Li1E")])
def test_head_group_lockstep_barrier(asm, inst):
    body, _ = _body(asm, inst)
    code = [l.strip() for l in body if l.strip() and not l.strip().startswith((";", ".")) and
            not l.strip().endswith(":")]
    bars = [j for j, l in enumerate(code) if l.startswith("s_barrier")]
    # the other barriers (Q quantization, epilogue) follow their LDS writes'
    # lgkmcnt wait
    free = [j for j in bars if not any(x.startswith("s_waitcnt") for x in code[j - 4:j])]
    fmt = int(re.findall(r"Li(\d+)E", inst)[0])
    assert len(free) == (0 if fmt in (5, 6) else 1), [code[j - 4:j + 1] for j in bars]


def _writes(line, reg):
    t = line.strip().split(None, 1)
    if len(t) < 2 or not t[0].startswith("v_"):
        return False
    dst = t[1].split(",")[0].strip()
    m = re.match(r"v\[(\d+):(\d+)\]", dst)
    if m:
        return int(m.group(1)) <= int(reg[1:]) <= int(m.group(2))
    return dst == reg


def test_scale_registers_not_rewritten_after_scaled_mfma(asm):
    n = 0
    for i, line in enumerate(asm):
        if "v_mfma_scale" not in line:
            continue
        ops = [x.strip() for x in line.split(None, 1)[1].split(",")]
        regs = {ops[4].split()[0], ops[5].split()[0]}
        n += 1
        for later in asm[i + 1:i + 24]:
            assert not any(_writes(later, r) for r in regs), (line.strip(), later.strip())
    assert n > 0
