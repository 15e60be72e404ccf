"""kvrq_paged_read, the page-gather read that measures the decode's same-pattern ceiling:
every pattern and grid size runs through the C ABI on ragged page lists (shorter than the
grid's waves, not a multiple of a unit group, ids outside the pool), writes nothing into the
cache, and leaves the sink alone (the folded words never equal the magic value for these
contents)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import int4_kv_cache_rotquant_amd as K
    K.lib()
    return K


@pytest.mark.parametrize("Hkv,P,num_pages", [(8, 16, 300), (2, 64, 40), (8, 64, 33)])
def test_paged_read_runs_and_writes_nothing(K, Hkv, P, num_pages):
    import torch
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(20260421 + P)
    cache = K.PagedInt4Cache(num_pages, Hkv, P, 128, 0, device=dev, fill=0)
    for t in (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params):
        u8 = t.view(torch.uint8)
        u8.copy_(torch.from_numpy(rng.integers(0, 256, u8.shape, dtype=np.uint8)).to(dev))
    before = [t.clone() for t in (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params)]
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for n in (1, 3, 7, 65, 1000):
        ids = rng.integers(0, num_pages, n).astype(np.int32)
        ids[::5] = -1                      # outside the pool: page 0 is read instead
        if n > 2:
            ids[1] = num_pages + 7
        pages = torch.from_numpy(ids).to(dev)
        for pattern in (0, 1, 2, 3):
            if pattern == 0 and (Hkv * P) % 128:
                continue
            for wg in (1, 2, 3, 4):
                K.kvrq_paged_read(cache, pages, sink, wgs_per_cu=wg, pattern=pattern)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    for b, t in zip(before, (cache.k_codes, cache.v_codes, cache.k_params, cache.v_params)):
        assert torch.equal(b, t)


def test_paged_read_rejects_bad_arguments(K):
    import torch
    dev = torch.device("cuda:0")
    cache = K.PagedInt4Cache(8, 8, 8, 0, 0, device=dev)        # 8 heads x 8 tokens: pattern 0 unsupported
    pages = torch.zeros(4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(K.KvrqError) as e:
        K.kvrq_paged_read(cache, pages, sink, pattern=0)
    assert e.value.status == K.KVRQ_EUNSUPPORTED
    with pytest.raises(K.KvrqError) as e:
        K.kvrq_paged_read(cache, pages, sink, pattern=1)     # 8-token pages: no 16-token blocks
    assert e.value.status == K.KVRQ_EUNSUPPORTED
    with pytest.raises(ValueError):
        K.kvrq_paged_read(cache, pages.to(torch.int64), sink)
