"""The prefill kernel issues some global loads as inline asm that the
compiler does not track (the Q fragments, the per-wave block-id vector and
the K/V LDS DMA) and waits for them explicitly.  The compiler believes an asm
load's result is ready when the asm ends, so the contract is checked on the
gfx950 assembly of every prefill instantiation:

1. no other instruction reads or writes the destination VGPRs of an
   untracked load before an explicit `s_waitcnt vmcnt(N)` that covers it
   (loads complete in issue order: a wait with N no larger than the number
   of untracked loads issued after it covers it);
2. every LDS DMA follows its M0 write by at least one wait state (the GFX9
   hazard of an LDS DMA reading M0 right after an SALU write of M0);
3. no kernel of the library writes through the scalar data cache (scalar
   stores or atomics, its write-back or discard): stores and atomics
   (including the decode work counter) are vector-memory instructions.

CPU only: it compiles the kernel sources with hipcc and the library build's
flags, all at once (skipped if hipcc is missing)."""
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_attention_29_amd", "csrc")


def _build_flags(src):
    """The library build's compile flags for one source (its build script,
    loaded by path: importing the package would load the library)."""
    spec = importlib.util.spec_from_file_location(
        "pa_build", os.path.join(ROOT, "paged_kv_attention_29_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return [*mod.FLAGS, *mod.EXTRA.get(src, [])]


SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


@pytest.fixture(scope="module")
def all_asm(tmp_path_factory):
    """gfx950 assembly of every kernel source, compiled concurrently (one
    hipcc per source) with the library build's flags."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("isa")
    procs = {}
    for src in SOURCES:
        cmd = [hipcc, *_build_flags(src), "--cuda-device-only", "-S",
               os.path.join(CSRC, src), "-o", str(d / (src + ".s"))]
        procs[src] = subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE)
    texts = {}
    for src, proc in procs.items():
        _, err = proc.communicate()
        assert proc.returncode == 0, f"{src}: {err.decode()[-2000:]}"
        texts[src] = (d / (src + ".s")).read_text()
    return texts


@pytest.fixture(scope="module")
def prefill_asm(all_asm):
    text = all_asm["prefill.hip"]
    funcs = {}
    for name in re.findall(r"^(_Z\S*prefill_kernel\S*):", text, flags=re.M):
        start = text.index(name + ":")
        end = text.index(".Lfunc_end", start)
        funcs[name] = [l.strip() for l in text[start:end].split("\n")]
    assert funcs, "no prefill kernel found in the assembly"
    return funcs


def _vregs(operands):
    regs = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", operands):
        if m.group(3):
            regs.add(int(m.group(3)))
        else:
            regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return regs


def test_untracked_load_results_are_not_touched_before_their_wait(prefill_asm):
    checked = 0
    for name, lines in prefill_asm.items():
        in_asm = False
        pending = []  # [issue order, destination VGPRs]
        order = 0
        for l in lines:
            if l.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if l.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if not l or l.startswith((".", ";")):
                continue
            op = l.split()[0]
            m = re.match(r"s_waitcnt\s+vmcnt\((\d+)\)", l)
            if m:
                n = int(m.group(1))
                pending = [(o, d) for (o, d) in pending
                           if sum(1 for (o2, _) in pending if o2 > o) < n]
                continue
            if in_asm and op in ("global_load_dwordx4", "global_load_dwordx2", "global_load_dword"):
                pending.append((order, _vregs(l.split()[1].rstrip(","))))
                order += 1
                checked += 1
                continue
            touched = _vregs(" ".join(l.split()[1:]))
            for (_, dest) in pending:
                assert not (touched & dest), f"{name}: '{l}' touches an untracked load's result"
    assert checked > 0


def test_lds_dma_waits_after_m0_write(prefill_asm):
    n_dma = 0
    for name, lines in prefill_asm.items():
        body = [l for l in lines if l and not l.startswith((".", ";"))]
        for i, l in enumerate(body):
            if l.startswith("global_load_lds"):
                n_dma += 1
                j = i - 1
                while j >= 0 and not body[j].startswith("s_mov_b32 m0"):
                    assert j > i - 4, f"{name}: no M0 write right before an LDS DMA"
                    j -= 1
                between = body[j + 1:i]
                assert any(x.startswith("s_nop") for x in between), \
                    f"{name}: LDS DMA issued right after its M0 write"
    assert n_dma > 0


@pytest.mark.parametrize("src", SOURCES)
def test_no_scalar_cache_writes(src, all_asm):
    bad = [l.strip() for l in all_asm[src].split("\n")
           if re.match(r"\s*(s_atomic|s_store|s_buffer_store|s_scratch_store|s_dcache_wb|"
                       r"s_dcache_discard)", l)]
    assert not bad, f"{src}: {bad[:3]}"
