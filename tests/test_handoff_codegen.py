"""The cross-block hand-offs compile to device-coherent memory accesses (CPU test on the library built here).

Blocks of one launch pass data to the block that draws a sequence's last ticket (tree build: per-slice candidates;
verification: per-slice argmax keys and sums) through relaxed agent-scope atomic stores and loads, and the writer
waits for its stores to complete before it takes the ticket. Their correctness rests on how gfx950 code implements
agent-scope atomics: a store or load carrying the sc1 cache-coherence bit goes through to the device coherence point
rather than stopping in one XCD's L2, and a store is complete once the wave's vmcnt reaches zero. This test unbundles
the gfx950 code object of each translation unit from libspectree.so, disassembles it and checks that the build and
verification units still contain sc1 loads, sc1 stores and ticket atomics, so that a toolchain change to these forms
fails here instead of surfacing as a rare wrong answer.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tree_attention_verification_03_amd", "libspectree.so")
LLVM = "/opt/rocm/llvm/bin"
TOOLS = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]


@pytest.fixture(scope="module")
def units(tmp_path_factory):
    if not os.path.exists(LIB):
        pytest.skip("libspectree.so is not built")
    if not all(os.path.exists(t) for t in TOOLS):
        pytest.skip("ROCm LLVM tools not found")
    d = tmp_path_factory.mktemp("codeobj")
    fat = d / "fat.bin"
    subprocess.run([TOOLS[0], f"--dump-section=.hip_fatbin={fat}", LIB, str(d / "stripped.so")], check=True,
                   capture_output=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(b"__CLANG_OFFLOAD_BUNDLE__"), data)]
    out = []
    for i, s in enumerate(starts):
        part = d / f"b{i}.bin"
        part.write_bytes(data[s:starts[i + 1] if i + 1 < len(starts) else len(data)])
        co = d / f"b{i}.co"
        subprocess.run([TOOLS[1], "--unbundle", "--type=o", f"--input={part}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"], check=True, capture_output=True)
        out.append(subprocess.run([TOOLS[2], "-d", str(co)], check=True, capture_output=True, text=True).stdout)
    shutil.rmtree(d, ignore_errors=True)
    return out


def _unit(units, kernel):
    found = [u for u in units if kernel in u]
    assert found, f"no code object holds {kernel}"
    return found[0]


@pytest.mark.parametrize("kernel", ["build_step_kernel", "verify_rows_kernel"])
def test_handoffs_use_device_coherent_accesses(units, kernel):
    text = _unit(units, kernel)
    stores = re.findall(r"\bglobal_store_\w+[^\n]*\bsc1\b", text)
    loads = re.findall(r"\bglobal_load_\w+[^\n]*\bsc1\b", text)
    assert stores and loads, f"{kernel}: agent-scope atomic stores / loads no longer carry sc1"
    assert re.search(r"\bglobal_atomic_add\w*", text), f"{kernel}: no ticket atomics"
    assert re.search(r"\bs_waitcnt vmcnt\(0\)", text), f"{kernel}: no store-completion waits"
