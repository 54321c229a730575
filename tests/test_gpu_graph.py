"""Multi-layer quantise + decode steps captured in a HIP graph replay to the eager results.

The step of a multi-layer workload (every layer quantised, then every layer decoded) is captured
once; each replay, with unrelated eager work and synchronisations between replays, must reproduce
the eager pages and outputs bit for bit.  The kernels record no memset: the decode's arrival
counters return to zero by themselves at the end of every call.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from kv_cache_quantization_kvarn_amd import kvarn
    return kvarn


@pytest.mark.parametrize("name", ["kvarn_k4v2_g128", "kvarn_k8v4_g64"])
def test_graph_replays_match_eager(K, name):
    cfg = K.kvarn_config_parse(name)
    layers, batch, hq, hkv, nblk = 3, 4, 12, 2, 6
    say("case: %s, %d-layer step (quantise %d blocks x %d heads, decode %d sequences) captured, replayed 4 times"
        % (name, layers, batch * nblk, hkv, batch))
    g = torch.Generator().manual_seed(515)
    L = []
    for _ in range(layers):
        k = torch.randn(batch * nblk * 128, hkv, 128, generator=g).half().cuda()
        v = torch.randn(batch * nblk * 128, hkv, 128, generator=g).half().cuda()
        kp, vp = K.alloc_pools(cfg, batch * nblk, hkv)
        q = torch.randn(batch, hq, 128, generator=g).half().cuda()
        out = torch.zeros(batch, hq, 128, device="cuda")
        L.append(dict(k=k, v=v, kp=kp, vp=vp, q=q, out=out))
    pages = torch.arange(batch * nblk, dtype=torch.int32, device="cuda")
    bt = pages.view(batch, nblk).contiguous()
    sl = torch.full((batch,), nblk * 128, dtype=torch.int32, device="cuda")
    sl[1] = 3 * 128
    ws = K.alloc_workspace(cfg, batch, hq, hkv, nblk)
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")

    def step():
        for x in L:
            K.kvarn_quantize_blocks(cfg, x["k"], x["v"], pages, x["kp"], x["vp"], fl)
        for x in L:
            K.kvarn_decode_attention(cfg, x["q"], x["kp"], x["vp"], bt, sl, hkv, x["out"], ws, dev_flags=fl)

    step()
    torch.cuda.synchronize()
    eager = [(x["kp"].clone(), x["vp"].clone(), x["out"].clone()) for x in L]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    junk = torch.randn(512, 512, device="cuda")
    for rep in range(4):
        for x in L:
            x["kp"].fill_(0x5A)
            x["vp"].fill_(0x5A)
            x["out"].fill_(float("nan"))
        junk = junk @ junk.T / 512.0  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, (kp, vp, out) in zip(L, eager):
            assert torch.equal(x["kp"], kp) and torch.equal(x["vp"], vp)
            assert torch.equal(x["out"], out), "replay %d differs from the eager decode" % rep
    assert K.kvarn_read_flags(fl) == 0
    say("  4 replays bit-identical to the eager step")
