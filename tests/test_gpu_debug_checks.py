"""Debug checks of the quantise call (kvarn_set_debug_checks): with them on, destination pages that
repeat are refused with KVARN_ERR_SHAPE before anything is written; distinct pages give the same
bytes as without the checks; a page id outside [0, num_pages) is still left to the kernels (flag)."""
import pytest
import torch

from kv_cache_quantization_kvarn_amd import kvarn as K
from kv_cache_quantization_kvarn_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_on():
    K.kvarn_set_debug_checks(True)
    try:
        yield
    finally:
        K.kvarn_set_debug_checks(False)


@pytest.mark.parametrize("head_dim", [128, 64])
def test_repeated_pages_are_refused(debug_on, head_dim):
    print("debug checks: repeated pages, head_dim", head_dim, flush=True)
    cfg = K.kvarn_config_parse("kvarn_k4v2_g128", head_dim)
    w = synth.WORKLOADS["tiny_1x1024"] if head_dim == 128 else synth.HEAD_DIM_WORKLOADS["tiny_d%d_1x1024" % head_dim]
    n_blocks, hkv, num_pages = 8, w.hkv, 12
    k, v = synth.layer_kv(w, 0, n_blocks * 128, "cuda")
    kp, vp = K.alloc_pools(cfg, num_pages, hkv)
    kp.fill_(0xA5)
    vp.fill_(0x5A)
    dst = torch.tensor([3, 7, 1, 0, 9, 7, 2, 5], dtype=torch.int32, device="cuda")  # 7 twice
    with pytest.raises(K.KvarnError) as e:
        K.kvarn_quantize_blocks(cfg, k, v, dst, kp, vp)
    assert e.value.status == K.KVARN_ERR_SHAPE
    assert "distinct" in str(e.value)
    torch.cuda.synchronize()
    assert bool((kp == 0xA5).all()) and bool((vp == 0x5A).all()), "a refused call wrote pages"


def test_distinct_pages_match_the_unchecked_call(debug_on):
    print("debug checks: distinct pages", flush=True)
    cfg = K.kvarn_config_parse("kvarn_k4v2_g128")
    w = synth.WORKLOADS["tiny_1x1024"]
    n_blocks, hkv, num_pages = 8, w.hkv, 300
    k, v = synth.layer_kv(w, 0, n_blocks * 128, "cuda")
    # distinct pages spread over several bitmap words, one id out of range
    dst = torch.tensor([299, 31, 32, 0, 64, 250, -1, 33], dtype=torch.int32, device="cuda")
    pools = []
    for on in (True, False):
        K.kvarn_set_debug_checks(on)
        kp, vp = K.alloc_pools(cfg, num_pages, hkv)
        kp.zero_()
        vp.zero_()
        flags = torch.zeros(1, dtype=torch.int32, device="cuda")
        K.kvarn_quantize_blocks(cfg, k, v, dst, kp, vp, flags)
        assert K.kvarn_read_flags(flags) == K.FLAG_BAD_PAGE
        pools.append((kp, vp))
    torch.cuda.synchronize()
    assert torch.equal(pools[0][0], pools[1][0]) and torch.equal(pools[0][1], pools[1][1])
