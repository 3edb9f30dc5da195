"""Host code of the C ABI (plan.hip's argument validation, plan geometry, error paths)
built with AddressSanitizer and UndefinedBehaviorSanitizer for the host side only, linked
against the library's other (uninstrumented) objects, and run on the CPU: the driver
tests/sanitize/abi_host_checks.cpp calls every entry point on invalid arguments and NULL
plans and checks the documented statuses; any memory or undefined-behaviour finding
aborts it. Needs hipcc and the objects that `efficient_transformer_attention_segment_amd.build`
leaves under _build/ (built first if missing); no GPU."""
import os
import shlex
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "efficient_transformer_attention_segment_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
OTHER = ["segmeans", "context", "output", "proj", "backward", "backward_general", "flash"]
# host-only instrumentation: each sanitizer flag follows -Xarch_host
SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined " \
      "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer"
COMMON = ("--offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -Xclang -target-feature -Xclang "
          "-packed-fp32-ops -mllvm -amdgpu-mfma-vgpr-form=1 -Wno-unused-command-line-argument")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    if not all(os.path.exists(os.path.join(BUILD, f + ".o")) for f in OTHER):
        from efficient_transformer_attention_segment_amd import build
        build.build(verbose=False)
    inc = f"-I {os.path.join(ROOT, 'include')} -I {CSRC}"
    plan_o = tmp_path / "plan_san.o"
    main_o = tmp_path / "abi_host_checks.o"
    exe = tmp_path / "abi_host_checks"
    main_src = os.path.join(ROOT, "tests", "sanitize", "abi_host_checks.cpp")
    cmds = [
        f"{HIPCC} {COMMON} {SAN} {inc} -c {os.path.join(CSRC, 'plan.hip')} -o {plan_o}",
        f"{HIPCC} {COMMON} {SAN} {inc} -c {main_src} -o {main_o}",
        f"{HIPCC} --offload-arch=gfx950 {SAN} {main_o} {plan_o} "
        + " ".join(os.path.join(BUILD, f + ".o") for f in OTHER) + f" -o {exe}",
    ]
    for c in cmds:
        r = subprocess.run(shlex.split(c), capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "0 failure(s)" in r.stdout
