"""Checks on the machine code built here for the attention kernels (CPU only:
the object is disassembled, nothing runs on a GPU).

The fp8 attention kernel issues its loads into LDS from inline asm, which sets
m0 (the LDS address of such loads) and declares it clobbered.  That is sound
only while no compiler-generated code in the same object keeps anything in m0:
every write of m0 there must be the asm's own `s_add_u32 m0, ...`, directly
followed by its `buffer_load_dwordx4 ... lds`.

That `s_add_u32` also writes the scalar condition code (SCC, its carry).  The
asm declares SCC clobbered; without that, the compiler kept a comparison's
result in SCC across the asm and branched on the carry instead (the causal
mask of the diagonal block was then applied to the first block).  So after
each such asm, no instruction may read SCC before code of the compiler's own
has written it again."""

from __future__ import annotations

import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# the attention kernels without and with the online skip
OBJS = [os.path.join(ROOT, "block_sparse_attention_24_amd", "_build", f) for f in ("bsa.o", "bsa_skip.o")]
LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")


def _disassemble(obj: str) -> list[str]:
    with tempfile.TemporaryDirectory() as d:
        fat, dev = os.path.join(d, "fat.bin"), os.path.join(d, "dev.o")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", f".hip_fatbin={fat}", obj,
                        os.path.join(d, "host.o")], check=True, capture_output=True)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o", f"--input={fat}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={dev}"], check=True,
                       capture_output=True)
        out = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--no-show-raw-insn", dev],
                             check=True, capture_output=True, text=True).stdout
    # instruction lines only, without the trailing address/encoding comments
    return [ln.split("//")[0].strip() for ln in out.splitlines() if ln.startswith("\t")]


@pytest.mark.parametrize("obj", OBJS, ids=os.path.basename)
def test_m0_written_only_by_the_lds_loads(obj):
    if not os.path.exists(obj):
        pytest.skip("attention object not built (python -m block_sparse_attention_24_amd.build)")
    if not all(os.path.exists(os.path.join(LLVM, t)) for t in ("llvm-objcopy", "clang-offload-bundler",
                                                                  "llvm-objdump")):
        pytest.skip("LLVM tools not found")
    ins = _disassemble(obj)
    assert ins, "empty disassembly"
    ours = re.compile(r"^s_add_u32 m0, s\d+, (0x[0-9a-f]+|\d+)$")
    writes = 0
    for i, text in enumerate(ins):
        fields = text.replace(",", " ").split()
        if "m0" not in fields:
            continue
        assert ours.match(text), f"m0 used by compiler-generated code: {text!r}"
        nxt = ins[i + 1] if i + 1 < len(ins) else ""
        assert nxt.startswith("buffer_load_dwordx4") and nxt.endswith("offen lds"), (text, nxt)
        writes += 1
    assert writes > 0, "the loads into LDS were not found"


# SALU instructions that write SCC, and the ones that read it
_SCC_WRITE = re.compile(r"^s_(add_|sub_|addc_|subb_|and_|or_|xor_|andn2_|orn2_|nand_|nor_|xnor_|lshl|lshr_|ashr_|bfe_|"
                        r"min_|max_|abs_|absdiff_|not_|bcnt|cmp|bitcmp|quadmask|wqm)")
_SCC_READ = re.compile(r"^s_(cbranch_scc|cselect_|addc_|subb_|cmov)")


@pytest.mark.parametrize("obj", OBJS, ids=os.path.basename)
def test_no_branch_on_the_condition_code_the_lds_loads_write(obj):
    if not os.path.exists(obj):
        pytest.skip("attention object not built (python -m block_sparse_attention_24_amd.build)")
    if not all(os.path.exists(os.path.join(LLVM, t)) for t in ("llvm-objcopy", "clang-offload-bundler",
                                                                  "llvm-objdump")):
        pytest.skip("LLVM tools not found")
    ins = _disassemble(obj)
    ours = re.compile(r"^s_add_u32 m0, s\d+, (0x[0-9a-f]+|\d+)$")
    after_asm = False
    bad = []
    for i, text in enumerate(ins):
        op = text.split()[0] if text else ""
        if ours.match(text):
            after_asm = True
            continue
        if _SCC_READ.match(op) and after_asm:
            bad.append((i, text))
        if _SCC_WRITE.match(op) or op.startswith("s_endpgm"):
            after_asm = False
    assert not bad, f"SCC read after an LDS load's s_add_u32 m0 with no write in between: {bad[:5]}"
