"""moe_permute_noalloc (the permute that allocates nothing: its rank table is
the library's static per-GPU scratch) against moe_permute, both called
through the C ABI with the same inputs: every output bit-exactly, on two
calls in a row, the second smaller than the first, so the second reuses the
scratch the first left behind."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _ids(rng, T, k, E):
    """Router-like ids: k distinct experts per token (hot experts first),
    plus a few "no route" (-1) and invalid ids."""
    w = 1.0 / np.arange(1, E + 1) ** 1.1
    ids = np.stack([rng.choice(E, size=k, replace=False, p=w / w.sum()) for _ in range(T)]).astype(np.int32)
    ids[rng.integers(0, T, size=3), 0] = -1
    ids[rng.integers(0, T, size=2), -1] = E + 5
    return ids


def _call(lib, name, x, ids, E, cap, ws=None):
    T, k = ids.shape
    R = T * k
    dev = x.device
    out = dict(x_perm=torch.zeros((R, x.shape[1]), dtype=x.dtype, device=dev),
               src=torch.full((R,), 7, dtype=torch.int32, device=dev),
               inv=torch.full((R,), 7, dtype=torch.int32, device=dev),
               sel=torch.zeros(E, dtype=torch.int32, device=dev),
               counts=torch.zeros(E, dtype=torch.int32, device=dev),
               offsets=torch.zeros(E + 1, dtype=torch.int32, device=dev),
               dropped=torch.zeros(1, dtype=torch.int32, device=dev),
               flags=torch.zeros(1, dtype=torch.int32, device=dev))
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    gi = torch.from_numpy(ids).to(dev)
    args = [p(x), 1, T, x.shape[1], p(gi), k, E, cap, p(out["x_perm"]), p(out["src"]), p(out["inv"]),
            p(out["sel"]), p(out["counts"]), p(out["offsets"]), p(out["dropped"])]
    if name == "moe_permute":
        args += [p(ws), ws.numel()]
    args += [p(out["flags"]), stream]
    st = getattr(lib, name)(*args)
    assert st == 0, (name, st)
    torch.cuda.synchronize()
    return {k_: v.cpu() for k_, v in out.items()}


def test_noalloc_permute_matches_permute():
    import grouped_expert_amd.binding as B
    lib = B.lib
    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(3)
    for i, (T, k, E, d, cap) in enumerate([(4096, 8, 384, 3072, -1), (700, 8, 384, 512, 20), (300, 2, 8, 128, 50)]):
        print(f"no-alloc permute call {i}: T={T} k={k} E={E} d={d} capacity={cap}", flush=True)
        assert lib.moe_permute_workspace(T, k, E) <= B.PERMUTE_NOALLOC_SCRATCH_BYTES
        ids = _ids(rng, T, k, E)
        x = torch.from_numpy(rng.integers(0, 1 << 16, size=(T, d), dtype=np.uint16).view(np.int16)).to(dev)
        x = x.view(torch.bfloat16)
        ws = torch.empty(lib.moe_permute_workspace(T, k, E), dtype=torch.uint8, device=dev)
        want = _call(lib, "moe_permute", x, ids, E, cap, ws)
        got = _call(lib, "moe_permute_noalloc", x, ids, E, cap)
        A = int(want["offsets"][E])
        assert A > 0 and int(want["flags"][0]) == int(got["flags"][0]) == B.FLAG_BAD_EXPERT
        for key in ("src", "inv", "sel", "counts", "offsets", "dropped"):
            assert torch.equal(got[key], want[key]), (i, key)
        assert torch.equal(got["x_perm"][:A].view(torch.int16), want["x_perm"][:A].view(torch.int16)), i
