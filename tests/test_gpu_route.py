"""GPU parity of the routing metadata: the HIP kernel behind moe_route must
match the oracle bit for bit (group sizes, offsets, padded offsets, stable
scatter, block map), on the workload recipes and on random shapes with
invalid ids."""
import numpy as np
import pytest

from skew_aware_grouped_amd import moe, workloads as W

pytestmark = pytest.mark.gpu


def _gpu_route(ids, T, k, E):
    import torch
    dev = "cuda:0"
    n_pad_cap, tile_cap = moe.moe_route_caps(T, k, E)
    N = T * k
    bufs = {
        "counts": torch.full((E,), -7, dtype=torch.int32, device=dev),
        "offsets": torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
        "padded_offsets": torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
        "pos": torch.full((max(N, 1),), -7, dtype=torch.int32, device=dev),
        "sorted_p": torch.full((max(N, 1),), -7, dtype=torch.int32, device=dev),
        "ppos": torch.full((max(N, 1),), -7, dtype=torch.int32, device=dev),
        "row_src": torch.full((max(n_pad_cap, 1),), -7, dtype=torch.int32, device=dev),
        "tile_expert": torch.full((max(tile_cap, 1),), -7, dtype=torch.int32, device=dev),
        "tile_row0": torch.full((max(tile_cap, 1),), -7, dtype=torch.int32, device=dev),
        "stats": torch.full((4,), -7, dtype=torch.int32, device=dev),
    }
    d_ids = torch.from_numpy(np.ascontiguousarray(ids.reshape(-1), dtype=np.int32)).to(dev)
    out = moe.moe_route_out(**{k_: v.data_ptr() for k_, v in bufs.items()})
    rc = moe.moe_route(T, k, E, d_ids.data_ptr() if N else None, out, moe._stream_ptr())
    assert rc == 0, moe.moe_error_string(rc)
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in bufs.items()}, n_pad_cap, tile_cap


def _compare(ids, T, k, E, oracle):
    g, n_pad_cap, tile_cap = _gpu_route(ids, T, k, E)
    r = oracle.route(ids.reshape(-1), E, moe.moe_block_m())
    N = T * k
    for name in ("counts", "offsets", "padded_offsets"):
        assert np.array_equal(g[name], r[name]), name
    for name in ("pos", "sorted_p", "ppos"):
        assert np.array_equal(g[name][:N], r[name][:N]), name
    assert np.array_equal(g["row_src"][:n_pad_cap], r["row_src"][:n_pad_cap])
    assert np.array_equal(g["tile_expert"][:tile_cap], r["tile_expert"][:tile_cap])
    assert np.array_equal(g["tile_row0"][:tile_cap], r["tile_row0"][:tile_cap])
    assert g["stats"][0] == r["dropped"] and g["stats"][1] == r["ntiles"] and g["stats"][2] == r["n_pad"]


@pytest.mark.parametrize("name", ["tiny", "qwen_bf16", "qwen_fp8", "ds_fp8_128", "ds_fp8_1024", "ds_fp8_8192"])
def test_route_matches_oracle_on_workloads(oracle, name):
    c = dict(W.CONFIGS[name])
    ids = W.make_routing(c["index"], c["T"], c["E"], c["k"], c["routing"])
    print(f"route parity {name} T={c['T']} E={c['E']} k={c['k']}", flush=True)
    _compare(ids, c["T"], c["k"], c["E"], oracle)


def _fuzz_cases():
    rng = np.random.default_rng(77)
    cases = []
    for i in range(40):
        T = int(rng.integers(0, 4097))
        k = int(rng.integers(1, 9))
        E = int(rng.integers(1, 257))
        kind = i % 4
        if kind == 0:
            ids = rng.integers(0, E, size=(T, k))
        elif kind == 1:  # invalid ids on both sides
            ids = rng.integers(-5, E + 5, size=(T, k))
        elif kind == 2:  # extreme skew: most rows on one or two experts
            ids = np.where(rng.random((T, k)) < 0.8, rng.integers(0, min(E, 2), size=(T, k)),
                           rng.integers(0, E, size=(T, k)))
        else:  # everything on the last expert
            ids = np.full((T, k), E - 1)
        cases.append((ids.astype(np.int32), T, k, E))
    cases.append((np.zeros((0, 2), np.int32), 0, 2, 8))
    cases.append((np.full((3, 2), -1, np.int32), 3, 2, 8))
    cases.append((np.arange(512, dtype=np.int32).reshape(256, 2) % 256, 256, 2, 256))
    cases.append((np.zeros((8192, 2), np.int32), 8192, 2, 1))
    return cases


@pytest.mark.parametrize("case", range(44))
def test_route_matches_oracle_fuzz(oracle, case):
    ids, T, k, E = _fuzz_cases()[case]
    print(f"route fuzz case {case}: T={T} k={k} E={E}", flush=True)
    _compare(ids, T, k, E, oracle)
