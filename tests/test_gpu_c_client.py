"""The path driven from C with no Python in between (tests/c_gpu_client.c, built by
__graft_entry__.build()): the allocator's block table over FP16, INT8, INT4 and INT2 pools,
chunked kv_quant_write prefill, kv_decode_step (or kv_decode_step_noalloc), kv_decode_attn at a
second split plan and kv_canary_kl, on hipMalloc'd memory, in either storage format, checked
against the oracle's C functions -- pool bytes and the ring bit for bit, attention rows within
2e-3, canary KL within 1e-4."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_bin", "c_gpu_client")


@pytest.mark.parametrize("mode", [[], ["asym"], ["noalloc"], ["asym", "noalloc"]],
                         ids=["symmetric", "asymmetric", "symmetric-noalloc", "asymmetric-noalloc"])
def test_c_program_runs_the_path_and_matches_the_oracle(mode):
    assert os.path.exists(EXE), "tests/_bin/c_gpu_client missing: run __graft_entry__.build()"
    print(f"\n[case] c_gpu_client {' '.join(mode)}: 3 ragged sequences, FP16/INT8/INT4/INT2 pages, "
          f"3-token step", flush=True)
    r = subprocess.run([EXE] + mode, capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("0 failures"), r.stdout + r.stderr
