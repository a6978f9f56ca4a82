"""Resource check of the built decode kernels (no GPU needed).

The decode kernel keeps its K/V prefetch ring and its accumulators in
registers; if the compiler moves them to per-lane scratch memory the kernel
still computes the right answer but its time multiplies (a run-enabled build
once did: 224-240 bytes of scratch per lane, and the 8 x 32K-token decode
took 500 us instead of 180).
This test reads each kernel's private segment size from the gfx950 code
objects of the in-tree build (_build/*.o, written by
paged_kv_cache_387_amd.build) with the ROCm LLVM tools and requires:
  * no scratch in any fp16 / int8 / E4M3 decode kernel, nor in the merge;
  * at most 32 bytes per lane in the fp32-cache kernels of head_dim 128, whose
    register budget is full (a few spilled scalars, not the ring);
  * no scratch in any build of the pipelined fp16 multi-query pass (its
    accumulators, q and the scores of two steps fill both register files; a
    spill there reloads q from scratch at every MFMA);
  * no scratch in the int8 / E4M3 multi-query pass and the fp32-cache one
    (with their MFMA results in VGPRs they fit; built with AGPR results the
    head-dim-128 ones spilled 140-200 bytes per lane).
Skipped when the build objects or the tools are absent.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJ_DIR = os.path.join(ROOT, "paged_kv_cache_387_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
# decode_kernel<KV, D, OUT, SRC, BS, RUNS>: KV 0 = fp32, 1 = fp16, 3 = int8, 4 = E4M3
DECODE = re.compile(r"decode_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(n?\d+)ELi(\d+)ELb([01])E")


def _kernel_scratch(obj, tmp_path):
    tools = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
    if not all(os.path.exists(t) for t in tools) or not os.path.exists(obj):
        pytest.skip("build objects or ROCm LLVM tools not present")
    objcopy, bundler, readelf = tools
    fatbin = str(tmp_path / (os.path.basename(obj) + ".fatbin"))
    code = str(tmp_path / (os.path.basename(obj) + ".gfx950.o"))
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fatbin}", obj], check=True,
                   capture_output=True)
    subprocess.run([bundler, "--type=o", f"--targets={TARGET}", f"--input={fatbin}",
                    f"--output={code}", "--unbundle"], check=True, capture_output=True)
    notes = subprocess.run([readelf, "--notes", code], check=True, capture_output=True,
                           text=True).stdout
    out, name = {}, None
    for line in notes.splitlines():
        line = line.strip()
        if line.startswith(".name:"):
            name = line.split(":", 1)[1].strip()
        elif line.startswith(".private_segment_fixed_size:") and name is not None:
            out[name] = int(line.split(":", 1)[1])
            name = None
    return out


@pytest.mark.parametrize("src", ["decode.hip", "decode_runs.hip"])
def test_decode_kernels_keep_their_state_in_registers(src, tmp_path):
    scratch = _kernel_scratch(os.path.join(OBJ_DIR, src + ".o"), tmp_path)
    decode = {k: v for k, v in scratch.items() if "decode_kernel" in k}
    assert len(decode) == 96, f"{src}: expected 96 decode kernels, found {len(decode)}"
    for name, nbytes in scratch.items():
        m = DECODE.search(name)
        if m:
            kv, d = int(m.group(1)), int(m.group(2))
            limit = 32 if (kv == 0 and d == 128) else 0
            assert nbytes <= limit, f"{src}: {name} uses {nbytes} bytes of scratch per lane"
        elif "merge_kernel" in name:
            assert nbytes == 0, f"{src}: {name} uses {nbytes} bytes of scratch per lane"


def test_multi_query_pass_keeps_its_state_in_registers(tmp_path):
    scratch = _kernel_scratch(os.path.join(OBJ_DIR, "prefix_pipe.hip.o"), tmp_path)
    pipe = {k: v for k, v in scratch.items() if "pipe32_kernel" in k}
    # 2 head sizes x 3 block sizes x (shared prefix, token groups 1 and 2 +
    # prefill, fp32 and fp16 output, token groups 1 and 2)
    assert len(pipe) == 36, f"expected 36 pipelined-pass kernels, found {len(pipe)}"
    spilled = {k: v for k, v in pipe.items() if v}
    assert not spilled, f"scratch per lane: {spilled}"


def test_quantized_multi_query_pass_keeps_its_state_in_registers(tmp_path):
    scratch = _kernel_scratch(os.path.join(OBJ_DIR, "prefix.hip.o"), tmp_path)
    passes = {k: v for k, v in scratch.items() if "prefix32_kernel" in k or "prefix_kernel" in k}
    # prefix32_kernel: 2 cache dtypes x 2 head sizes x 3 block sizes x (shared
    # prefix, prefill); prefill once per output dtype; prefix_kernel: fp32 caches
    assert len(passes) == 42, f"expected 42 multi-query kernels, found {len(passes)}"
    spilled = {k: v for k, v in passes.items() if v}
    assert not spilled, f"scratch per lane: {spilled}"
