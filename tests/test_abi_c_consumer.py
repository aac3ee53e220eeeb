"""The boundary from C: tests/abi_c_consumer.c includes include/sage_attn.h as strict C99
(-pedantic, warnings as errors), links the in-tree library and makes host-only calls (no device
work, so it runs on the CPU)."""
import os
import subprocess

import bit_quantized_attention_smooth_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_and_library_from_plain_c(tmp_path):
    S.lib()   # the in-tree library exists (built by build())
    libdir = os.path.join(ROOT, "bit_quantized_attention_smooth_amd")
    exe = str(tmp_path / "abi_c_consumer")
    subprocess.check_call(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_c_consumer.c"),
                           "-o", exe, "-L", libdir, "-lsage_attn", "-Wl,-rpath," + libdir])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi c consumer ok" in r.stdout
