"""Host-side check of a code-generation assumption of the tiled GEMM kernels
(no GPU needed, hipcc required).

The tiled kernels issue their direct-to-LDS loads from inline assembly that
writes M0 (the LDS destination) itself; the compiler is told M0 is clobbered
but may not save a live M0 value around it.  This test compiles tiled.hip and
tiled8.hip for gfx950 and checks that in every tiled kernel M0 is written only
by those sequences (s_mov_b32 m0, s_nop 0, a direct-to-LDS load) and read only by the
direct-to-LDS load that follows each write."""
import os
import re
import shutil
import subprocess

import pytest

from expert_ffn_layer_gemm_amd import build

HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
@pytest.mark.parametrize("src,pattern,n_min", [("tiled.hip", r"_ZN3moe8k_tiled3\w+", 2),
                                               ("tiled8.hip", r"_ZN3moe8k_tiled8\w+", 6)])
def test_tiled_kernels_use_m0_only_for_their_direct_to_lds_loads(tmp_path, src, pattern, n_min):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, *build.HIPCC_FLAGS, "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    kernels = re.findall(r"^(" + pattern + r"):", asm, flags=re.M)
    assert len(kernels) >= n_min
    for name in kernels:
        body = asm[asm.index(name + ":"):]
        body = body[:body.index(".Lfunc_end")]
        ins = [l.split(";")[0].strip() for l in body.splitlines()]
        ins = [l for l in ins if l and not l.startswith(".") and not l.endswith(":")]
        writes = 0
        for i, l in enumerate(ins):
            if not re.search(r"\bm0\b", l):
                continue
            assert re.match(r"s_mov_b32 m0, s\d+$", l), f"{name}: unexpected use of m0: {l}"
            assert ins[i + 1] == "s_nop 0", f"{name}: {l} not followed by s_nop 0"
            assert ins[i + 2].startswith("global_load_lds_dword"), f"{name}: {ins[i + 2]}"
            writes += 1
        assert writes > 0, name
        # every direct-to-LDS load is preceded by its own M0 write
        for i, l in enumerate(ins):
            if l.startswith("global_load_lds_dword"):
                assert ins[i - 2].startswith("s_mov_b32 m0,"), f"{name}: load without its M0 write"
