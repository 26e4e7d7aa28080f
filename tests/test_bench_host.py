"""Host-side checks of the benchmark: the one-GPU guard, the algorithmic byte
counts behind the roofline, and the committed counter summaries it reads.
No GPU is used."""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


# Compulsory bytes of each op (every input read once, every output written
# once), worked out from the workload shapes: activations 2 B per element,
# states 3 BF16 slots per (row, channel), the filter [D,4], the bias [D],
# dW [D,4] and dB [D] in FP32.
@pytest.mark.parametrize("name,got,want", [
    # B=1 D=64 T=128, bias, final states returned
    ("tiny fwd", lambda: bench.fwd_bytes(1, 64, 128, 1, False, True, 2, True),
     2 * 64 * 128 * 2 + 64 * 6 + 64 * 4 * 2 + 64 * 2),
    # B=4 D=4096 T=2048, bias, initial and final states
    ("dense fwd", lambda: bench.fwd_bytes(4, 4096, 2048, 4, True, True, 2, True), 134455296),
    ("dense bwd", lambda: bench.bwd_bytes(4, 4096, 2048, 4, True, False, 2, True), 201646080),
    # 16 sequences, 33,280 tokens, D=5120, FP32 filter, no bias, states
    ("packed fwd", lambda: bench.fwd_bytes(1, 5120, 33280, 16, True, True, 4, False), 682639360),
    ("packed bwd", lambda: bench.bwd_bytes(1, 5120, 33280, 16, True, False, 4, False),
     1023508480),
    # B=256 D=8192 single-token update, bias
    ("decode update", lambda: bench.update_bytes(256, 8192, 2, True), 33636352),
    # B=8 D=8192 T=8192, no bias, no states
    ("large fwd", lambda: bench.fwd_bytes(8, 8192, 8192, 8, False, False, 2, False), 2147549184),
    ("large bwd", lambda: bench.bwd_bytes(8, 8192, 8192, 8, False, False, 2, False), 3221422080),
    # the dense shape with a width-2 filter: one state slot, [D,2] filter and dW
    ("dense_w2 fwd", lambda: bench.WORKLOAD_BYTES["dense_w2"]["fwd"],
     2 * 4 * 4096 * 2048 * 2 + 2 * 4 * 4096 * 2 + 4096 * 2 * 2 + 4096 * 2),
    ("dense_w2 bwd", lambda: bench.WORKLOAD_BYTES["dense_w2"]["bwd"],
     3 * 4 * 4096 * 2048 * 2 + 2 * 4 * 4096 * 2 + 4096 * 2 * 2 + 4096 * 2 * 4 + 4096 * (2 + 4)),
    # FP32 filter and FP32 bias
    ("dense_f32bias fwd", lambda: bench.WORKLOAD_BYTES["dense_f32bias"]["fwd"],
     2 * 4 * 4096 * 2048 * 2 + 2 * 4 * 4096 * 6 + 4096 * 4 * 4 + 4096 * 4),
    ("dense_f32bias bwd", lambda: bench.WORKLOAD_BYTES["dense_f32bias"]["bwd"],
     3 * 4 * 4096 * 2048 * 2 + 2 * 4 * 4096 * 6 + 4096 * 4 * 4 + 4096 * 4 * 4 + 4096 * (4 + 4)),
    # 8 tokens per call: the state read and written once, 8 tokens in, 8 out
    ("decode_tokens update", lambda: bench.WORKLOAD_BYTES["decode_tokens"]["update"],
     256 * 8192 * (6 + 6 + 8 * 2 + 8 * 2) + 8192 * 4 * 2 + 8192 * 2),
])
def test_algorithmic_bytes(name, got, want):
    assert got() == want, name


def test_rotation_leaves_the_memory_side_cache():
    """Between two uses of one operand copy, the other copies move at least
    three times the 256 MB memory-side cache (or the copy count is capped)."""
    class W:
        def __init__(self, b):
            self.b = b

        def step_bytes(self):
            return self.b

    for step in (303104, 33636352 * 64, 336404480, 1706147840, 5368971264):
        r = bench.rotation_count(W(step))
        assert 2 <= r <= 16
        assert (r - 1) * step >= 3 * bench.MALL_BYTES or r == 16


def test_committed_profiles_carry_a_traffic_record():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "k_*.md")))
    assert paths
    seen = 0
    for p in paths:
        text = open(p).read()
        recs = [l for l in text.splitlines() if l.startswith("<!-- traffic ")]
        if not recs:
            continue
        seen += 1
        rec = json.loads(recs[0][len("<!-- traffic "):].rsplit("-->", 1)[0])
        for key in ("kernel", "workload", "hbm_bytes_per_launch", "algorithmic_bytes",
                    "avg_kernel_us", "source_hash"):
            assert key in rec, (p, key)
        assert os.path.basename(p) == "%s_%s.md" % (rec["kernel"], rec["workload"])
        # counters read every compulsory byte, and little beyond it
        assert 1.0 <= rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes"] < 1.2, p
        assert "rocprofv3" in text and "bench.py" in text, p
    assert seen >= 7


@pytest.mark.parametrize("name,kernel,want", [
    ("k_fwd_tcp<4, true, 2>", "k_fwd_tcp", True),
    ("k_fwd_tcp_fix<4, true, 2>", "k_fwd_tcp", False),
    ("k_fwd_tcp_fix<4, true, 2>", "k_fwd_tcp_fix", True),
    ("k_fwd_tc<4, true, 1>", "k_fwd_tcp", False),
    ("k_fwd_tc<4, true, 1>", "k_fwd_tc", True),
    ("ccv::(anonymous namespace)::k_validate(int const*, long, long, unsigned int*, int)",
     "k_validate", True),
    ("void ccv::(anonymous namespace)::k_dw_reduce<4>(float const*, long)", "k_dw_reduce", True),
    ("k_update_staged<4, true, false, true, 2>", "k_update", False),
    ("__amd_rocclr_copyBuffer", "k_update", False),
])
def test_trace_names_match_whole_kernel_names(name, kernel, want):
    """Counter and trace rows are matched to a kernel by its whole name (a
    kernel whose name extends another's is another kernel)."""
    assert bench._is_kernel(name, kernel) is want


def test_every_workload_maps_its_ops_to_a_kernel_family():
    for wl in bench.WORKLOADS:
        ks = bench.op_kernels(wl)
        assert set(ks) == {"fwd", "bwd", "update"}, wl
    assert bench.op_kernels("packed_tc")["bwd"] == "k_bwd_tcp"
    assert bench.op_kernels("seqidx_tc")["fwd"] == "k_fwd_tcs"
    assert bench.op_kernels("dense_tc")["fwd"] == "k_fwd_tc"
    assert bench.op_kernels("packed")["fwd"] == "k_fwd_chan"
    assert "k_update_staged" in bench.UPDATE_KERNELS
