"""Steps captured in a HIP graph (torch.cuda.graph) and replayed: scatter +
split decode, the appending decode, and scatter + chunked prefill.  Every replay, with eager
work and synchronisation between replays, must give the eager result bit
for bit, and leave the pools as the eager step left them."""
import numpy as np
import pytest
import torch

import paged_kv_cache_92_amd as pkv
from paged_kv_cache_92_amd import workloads as W
from tests.gpu_run import DeviceWorkload, bits_of, new_cache

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                        # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _replays_match(g, out, want, cache, pools):
    for i in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_of(out), want), f"replay {i}"
        for name, dev, ref in (("K", cache.k_pool, pools[0]), ("V", cache.v_pool, pools[1])):
            assert np.array_equal(bits_of(dev).view(np.uint8), ref.view(np.uint8)), f"{name} pool, replay {i}"
        _ = (out.float() * 2).sum().item()          # eager work between replays


@pytest.mark.parametrize("part", [512, -1], ids=["p512", "auto"])
@pytest.mark.parametrize("G", [1, 4])
def test_decode_step_graph_replays(part, G):
    wl = W.make_decode(f"graph_{G}_{part}", 31 + G, lambda rng: [1, 17, 300, 1500, 2048], Hq=4 * G,
                       Hkv=4, d=128, B=16, dtype=W.BF16, max_context_len=2048, partition_size=part)
    dw = DeviceWorkload(wl)
    cache = new_cache(wl)
    dw.fill(cache)
    need = pkv.decode_workspace_bytes(cache, wl.S, wl.num_q_heads, wl.max_context_len, part)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty(dw.q.shape, dtype=torch.float32, device="cuda")

    def step():
        dw.apply(cache, dw.step)
        dw.attend(cache, out=out, workspace=ws, out_dtype=torch.float32)
    step()
    torch.cuda.synchronize()
    want = bits_of(out).copy()
    pools = (bits_of(cache.k_pool).copy(), bits_of(cache.v_pool).copy())
    _replays_match(_capture(step), out, want, cache, pools)


@pytest.mark.parametrize("G", [1, 4])
def test_appending_decode_graph_replays(G):
    wl = W.make_decode(f"graph_app_{G}", 41 + G, lambda rng: [2, 16, 33, 700, 2048], Hq=4 * G, Hkv=4,
                       d=128, B=16, dtype=W.F16, max_context_len=2048, partition_size=-1)
    dw = DeviceWorkload(wl)
    cache = new_cache(wl)
    dw.fill(cache)
    need = pkv.decode_workspace_bytes(cache, wl.S, wl.num_q_heads, wl.max_context_len, -1)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty(dw.q.shape, dtype=torch.float32, device="cuda")

    def step():
        dw.append_attend(cache, out=out, workspace=ws, out_dtype=torch.float32)
    step()
    torch.cuda.synchronize()
    want = bits_of(out).copy()
    pools = (bits_of(cache.k_pool).copy(), bits_of(cache.v_pool).copy())
    _replays_match(_capture(step), out, want, cache, pools)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefill_step_graph_replays(kv):
    # The chunk scatter + causal prefill: the workgroups rank their work items
    # on the device and may redo a walk on the exact route; a replay must
    # still give the eager result bit for bit.
    wl = W.chunked_prefill_bf16(S=4, chunk=300, shared_prefix=20, Hq=8, Hkv=4, max_context_len=1024,
                                hist_fn=lambda rng: np.array([30, 41, 600, 150]))
    if kv == "fp8":
        wl.kv_dtype, wl.k_scale, wl.v_scale = W.FP8, float(np.float32(0.02)), float(np.float32(0.03))
    dw = DeviceWorkload(wl)
    cache = new_cache(wl)
    dw.fill(cache)
    out = torch.empty(dw.q.shape, dtype=torch.float32, device="cuda")

    def step():
        dw.apply(cache, dw.step)
        dw.attend(cache, out=out, out_dtype=torch.float32)
    step()
    torch.cuda.synchronize()
    want = bits_of(out).copy()
    pools = (bits_of(cache.k_pool).copy(), bits_of(cache.v_pool).copy())
    _replays_match(_capture(step), out, want, cache, pools)
