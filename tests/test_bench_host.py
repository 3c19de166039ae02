"""Host-side logic of bench.py (no GPU): the algorithmic byte model behind the
roofline figures, the mapping from rocprofv3 kernel names onto it, the source
hashes that mark a stored HBM-traffic figure stale, and the refusal of more
than one GPU."""

import importlib.util
import os
import subprocess
import sys

import pytest

from selective_state_space_amd import inputs as gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def workload(name):
    return next(w for w in gen.WORKLOADS if w.name == name)


def test_forward_bytes_written_out_by_hand():
    """The 2.7B layer (batch 8, 4096 tokens, 80 heads of 64, N = 128, one
    group, chunks of 256, bf16 in, fp32 y, an initial state): every term
    counted once, from the shapes alone."""
    alg = bench.algorithmic(workload("mamba2_2p7b"), 2)
    Bt, T, H, P, N, L = 8, 4096, 80, 64, 128, 256
    nc = T // L
    x = Bt * T * H * P * 2
    y = Bt * T * H * P * 4
    b_or_c = Bt * T * N * 2
    h_prev = Bt * H * nc * P * N * 2
    g_dt = 2 * Bt * H * nc * L * 4
    state = Bt * H * P * N * 4
    assert alg["chunk_scan"]["bytes"] == x + y + 2 * b_or_c + h_prev + g_dt == 1212153856
    assert alg["state_fwd_kernel"]["bytes"] == x + b_or_c + g_dt + h_prev + 2 * state
    assert alg["chunk_cumsum"]["bytes"] == Bt * T * H * 4 + g_dt
    assert alg["b_fragments"]["bytes"] == 2 * b_or_c
    assert alg["cumsum_bfrag"]["bytes"] == (alg["chunk_cumsum"]["bytes"]
                                            + alg["b_fragments"]["bytes"])


@pytest.mark.parametrize("name,kind", [
    ("chunk_scan_bf16_kernel<256, 128, false>", "chunk_scan"),
    ("chunk_scan_bf16_kernel<256, 128, true>", None),          # the gated variant
    ("state_fwd_kernel<256, 128, 4, 0>", "state_fwd_kernel"),
    ("state_fwd_kernel<256, 128, 4, 1>", None),                # backward h_prev recompute
    ("state_fwd_kernel<256, 128, 4, 2>", None),                # backward adjoint scan
    ("chunk_cumsum_kernel<256>", "chunk_cumsum"),
    ("b_fragments_kernel<256, 128>", "b_fragments"),
    ("cumsum_bfrag_kernel<256, 128>", "cumsum_bfrag"),
    ("void ssd::(anonymous namespace)::cumsum_bfrag_kernel<256, 128>(float const*)", "cumsum_bfrag"),
    ("decode_step_kernel<128, bf16, false>", None),
])
def test_profile_kind(name, kind):
    assert bench.profile_kind(name) == kind


def test_source_hashes():
    kinds = ("chunk_scan", "state_fwd", "chunk_cumsum", "b_fragments", "cumsum_bfrag")
    sha = {k: bench.kernel_source_sha(k) for k in kinds}
    assert all(len(v) == 16 for v in sha.values())
    assert sha == {k: bench.kernel_source_sha(k) for k in kinds}   # deterministic
    # the combined launch also depends on the fragment layout's header
    assert sha["cumsum_bfrag"] != sha["chunk_cumsum"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
