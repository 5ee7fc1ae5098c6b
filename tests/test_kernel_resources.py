"""Register and scratch budgets of the hot kernels (CPU: hipcc's device assembly).

The schedules are built around these budgets: the d 64 prefill keeps three waves
per SIMD (at most 168 VGPRs of the 512 per SIMD lane), the d 128 prefill and the
decode kernels two (at most 256), top-K stage 1 four workgroups of four waves
per CU (at most 128); the only scratch use is a few values kept across the d 64
prefill and d 128 decode scans. A change that pushes a kernel past its budget
halves its occupancy or moves values to scratch memory, which the GPU tests
would not flag; this test does, from the compiler's own kernel descriptors.

The K/V copies of the attention kernels write M0 inside inline assembly. The
compiler treats M0 as a reserved register and does not promise to keep a value
of its own there across such a statement, so the attention kernels' device code
must not use M0 anywhere else; the last test checks that too.
"""
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_bga_packed_amd", "csrc")

# kernel name prefix (mangled) -> (source, max VGPRs, max scratch bytes per lane)
BUDGETS = {
    "_ZN3bga21packed_prefill_kernelILi64ELi4E": ("prefill.hip", 168, 16),
    "_ZN3bga21packed_prefill_kernelILi128ELi4E": ("prefill.hip", 256, 0),
    "_ZN3bga27shared_prefix_decode_kernelILi64E": ("decode.hip", 256, 0),
    "_ZN3bga27shared_prefix_decode_kernelILi128E": ("decode.hip", 256, 20),
    "_ZN3bga18topk_stage1_kernelILb1E": ("topk.hip", 128, 0),
    "_ZN3bga18topk_stage2_kernel": ("topk.hip", 256, 0),
    "_ZN3bga21suffix_reorder_kernel": ("reorder.hip", 256, 0),
}


def _build_module():
    spec = importlib.util.spec_from_file_location("bga_build", os.path.join(ROOT, "attention_bga_packed_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def descriptors(tmp_path_factory):
    hipcc = shutil.which(os.environ.get("HIPCC", "hipcc"))
    if hipcc is None:
        pytest.skip("hipcc not available")
    b = _build_module()
    out = tmp_path_factory.mktemp("asm")
    procs = []
    for src in sorted({v[0] for v in BUDGETS.values()}):
        dst = os.path.join(out, src + ".s")
        cmd = [hipcc, *b.HIPCC_FLAGS, *b.PER_FILE_FLAGS.get(src, []), "--cuda-device-only", "-S",
               os.path.join(CSRC, src), "-o", dst]
        procs.append((src, dst, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    desc, asm = {}, {}
    for src, dst, p in procs:
        log, _ = p.communicate()
        assert p.returncode == 0, f"{src}: {log[-2000:]}"
        text = open(dst).read()
        asm[src] = text
        # the code-object metadata lists every kernel with its resource counts
        for blk in re.split(r"\n  - \.", text.split("amdhsa.kernels:", 1)[1]):
            name = re.search(r"\.name:\s+(\S+)", blk)
            vgpr = re.search(r"\.vgpr_count:\s+(\d+)", blk)
            scratch = re.search(r"\.private_segment_fixed_size:\s+(\d+)", blk)
            if name and vgpr and scratch:
                desc[name.group(1)] = (int(vgpr.group(1)), int(scratch.group(1)))
    return desc, asm


@pytest.mark.parametrize("prefix", sorted(BUDGETS))
def test_kernel_stays_within_its_budget(descriptors, prefix):
    found = {n: v for n, v in descriptors[0].items() if n.startswith(prefix)}
    assert found, f"no kernel named {prefix}* in the device code"
    _, max_vgpr, max_scratch = BUDGETS[prefix]
    for name, (vgpr, scratch) in found.items():
        assert vgpr <= max_vgpr, f"{name}: {vgpr} VGPRs > {max_vgpr}"
        assert scratch <= max_scratch, f"{name}: {scratch} bytes of scratch per lane > {max_scratch}"


@pytest.mark.parametrize("src", ["prefill.hip", "decode.hip"])
def test_m0_is_written_only_by_the_copy_statements(descriptors, src):
    inside, uses = False, []
    for line in descriptors[1][src].splitlines():
        if ";;#ASMSTART" in line:
            inside = True
        elif ";;#ASMEND" in line:
            inside = False
        elif not inside and not line.lstrip().startswith((";", ".")) and re.search(r"\bm0\b", line):
            uses.append(line.strip())
    assert uses == [], f"{src}: the compiler uses M0 outside the copy statements: {uses[:3]}"


# scalar instructions that write SCC; none may sit inside inline assembly (see
# tests/test_inline_asm.py for why), checked here on the compiler's output too
_SCC_WRITER = re.compile(r"^\s*s_(cmp\w*|add_[iu]32|sub_[iu]32|addc_u32|subb_u32|addk_i32|and_\w+|or_\w+|xor_\w+|"
                         r"andn2_\w+|orn2_\w+|nand_\w+|nor_\w+|xnor_\w+|lshl\w*|lshr\w*|ashr\w*|bfe_\w+|min_\w+|"
                         r"max_\w+|abs\w*|not_\w+|bitcmp\w*|bcnt\w*|absdiff_\w+)\b")


@pytest.mark.parametrize("src", sorted({v[0] for v in BUDGETS.values()}))
def test_compiled_inline_asm_writes_no_scc(descriptors, src):
    inside, bad = False, []
    for line in descriptors[1][src].splitlines():
        if ";;#ASMSTART" in line:
            inside = True
        elif ";;#ASMEND" in line:
            inside = False
        elif inside and _SCC_WRITER.match(line):
            bad.append(line.strip())
    assert bad == [], f"{src}: inline assembly writes SCC: {bad[:3]}"
