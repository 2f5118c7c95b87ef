"""The allocation-free verification entry point (tsw_tree_attn_verify_noalloc)
against tsw_tree_attn_verify, through the C ABI: the same kernels and split
plan, so the outputs must be identical.  Two calls in a row on the library's
shared partials array, the second with a smaller problem, then a problem too
large for the array (rejected before anything is launched)."""
import ctypes

import numpy as np
import pytest
import torch

import tree_verification_attention_tsw_amd as tsw
from tree_verification_attention_tsw_amd import workloads as wl

pytestmark = pytest.mark.gpu
ENOSPACE = -5


@pytest.fixture(scope="module", autouse=True)
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsw.lib()
    return torch.device("cuda:0")


def _case(name, Hq, Hkv, n_prefix, T, seed):
    w = wl.Workload(name, Hq=Hq, Hkv=Hkv, d=128, n_prefix=n_prefix, n_nodes=T, dtype=wl.BF16, seed=seed)
    q, k, v = wl.make_qkv(w, device="cuda")
    return w, q, k, v


def _noalloc(w, q, k, v):
    o = torch.full((w.n_nodes, w.Hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((w.n_nodes, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
    return tsw.tree_attn_verify_noalloc(q, k, v, w.parent(), w.n_prefix, o, lse)


def test_noalloc_matches_verify_twice_then_smaller():
    assert tsw.noalloc_scratch_bytes() == 32 << 20
    cases = [_case("big", 32, 8, 102400, 40, 11), _case("small", 8, 2, 3000, 13, 12)]
    for w, q, k, v in cases:
        print("noalloc case %s: T=%d Hq=%d Hkv=%d n_prefix=%d" % (w.name, w.n_nodes, w.Hq, w.Hkv, w.n_prefix),
              flush=True)
        o_ref, l_ref = tsw.tree_attn_verify(q, k, v, w.parent(), w.n_prefix)
        o, lse = _noalloc(w, q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), w.name



def test_noalloc_random_shapes_in_a_row():
    """Twelve seeded random problems one after another on the shared array
    (sizes going up and down; tree, head grouping, precision, head dim and
    length drawn), each identical to tsw_tree_attn_verify."""
    rng = np.random.default_rng(9800)
    for case in range(12):
        T = int(rng.integers(1, 65))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * int(rng.integers(1, 9))
        dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
        d = 128 if (dtype == torch.bfloat16 and rng.random() < 0.8) else int(rng.choice([64, 128]))
        n_prefix = int(rng.integers(0, 50001))
        parent = wl.random_tree_parent(T, 9800 + case)
        g = torch.Generator(device="cuda")
        g.manual_seed(9800 + case)
        q = torch.randn((T, Hq, d), generator=g, device="cuda").to(dtype)
        k = torch.randn((Hkv, n_prefix + T, d), generator=g, device="cuda").to(dtype)
        v = torch.randn((Hkv, n_prefix + T, d), generator=g, device="cuda").to(dtype)
        need = tsw.workspace_size(q, k, n_prefix)
        print("noalloc random case %d: T=%d Hq=%d Hkv=%d d=%d %s n_prefix=%d partials %d bytes" % (
            case, T, Hq, Hkv, d, "bf16" if dtype == torch.bfloat16 else "f32", n_prefix, need), flush=True)
        if need > tsw.noalloc_scratch_bytes():
            continue
        o_ref, l_ref = tsw.tree_attn_verify(q, k, v, parent, n_prefix)
        o = torch.full((T, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((T, Hq), float("nan"), dtype=torch.float32, device="cuda")
        o, lse = tsw.tree_attn_verify_noalloc(q, k, v, parent, n_prefix, o, lse)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), case


def test_noalloc_rejects_too_large():
    # 384 query rows on one kv head over a long cache (long enough that the
    # planner's floor of 3 x 384 keys per split still allows one split per
    # CU): 256 splits x 64 nodes x 6 heads x 129 floats need more than 32 MiB
    T, Hq, n_prefix = 64, 6, 300000
    q = torch.zeros((T, Hq, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, n_prefix + T, 128), dtype=torch.bfloat16, device="cuda")
    need = tsw.workspace_size(q, k, n_prefix)
    print("too-large case needs %d bytes of partials" % need, flush=True)
    if need <= tsw.noalloc_scratch_bytes():
        pytest.skip("this device plans fewer splits; the case fits")
    desc = tsw.make_desc(q, k, n_prefix)
    o = torch.full((T, Hq, 128), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((T, Hq), 7.0, dtype=torch.float32, device="cuda")
    p = np.ascontiguousarray(wl.kary_tree_parent(T, 3), dtype=np.int32)
    rc = tsw.lib().tsw_tree_attn_verify_noalloc(ctypes.byref(desc), ctypes.c_void_p(q.data_ptr()),
                                                 ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                                 p.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(o.data_ptr()),
                                                 ctypes.c_void_p(lse.data_ptr()), None)
    torch.cuda.synchronize()
    assert rc == ENOSPACE
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
