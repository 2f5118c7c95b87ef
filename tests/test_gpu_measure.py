"""GPU check of the measurement aid the benchmark reports beside the
attention call: the read-stream ceiling kernel (tsw_read_stream)."""
import pytest
import torch

import tree_verification_attention_tsw_amd as tsw
from tree_verification_attention_tsw_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsw.lib()
    return torch.device("cuda:0")


def _case(n_prefix=20000):
    w = wl.Workload("measure", Hq=32, Hkv=8, d=128, n_prefix=n_prefix, n_nodes=40, dtype=wl.BF16, seed=77)
    q, k, v = wl.make_qkv(w, device="cuda")
    return w, q, k, v


def test_read_stream_runs_and_is_faster_than_the_call():
    w, q, k, v = _case(60000)
    sink = torch.zeros(64, dtype=torch.uint8, device="cuda")
    tsw.read_stream(q, k, v, w.n_prefix, sink)
    tsw.tree_attn_verify(q, k, v, w.parent(), w.n_prefix)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(s)
    for _ in range(5):
        tsw.read_stream(q, k, v, w.n_prefix, sink)
    e[1].record(s)
    for _ in range(5):
        tsw.tree_attn_verify(q, k, v, w.parent(), w.n_prefix)
    e[2].record(s)
    torch.cuda.synchronize()
    t_read, t_call = e[0].elapsed_time(e[1]) / 5, e[1].elapsed_time(e[2]) / 5
    print("read stream %.2f us, verify %.2f us" % (t_read * 1e3, t_call * 1e3), flush=True)
    assert 0.0 < t_read <= t_call
    assert int(sink.sum()) == 0


def test_launch_floor_runs_and_is_faster_than_the_call():
    """The empty split-grid kernel runs and takes less time than the call."""
    w, q, k, v = _case(60000)
    fl = tsw.prepare_launch_floor(q, k, w.n_prefix)
    tsw.tree_attn_verify(q, k, v, w.parent(), w.n_prefix)
    fl()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(s)
    for _ in range(5):
        fl()
    e[1].record(s)
    for _ in range(5):
        tsw.tree_attn_verify(q, k, v, w.parent(), w.n_prefix)
    e[2].record(s)
    torch.cuda.synchronize()
    t_floor, t_call = e[0].elapsed_time(e[1]) / 5, e[1].elapsed_time(e[2]) / 5
    print("launch floor %.2f us, verify %.2f us" % (t_floor * 1e3, t_call * 1e3), flush=True)
    assert 0.0 < t_floor < t_call
