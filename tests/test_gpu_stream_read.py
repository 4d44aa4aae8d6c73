"""GPU check of the read-bandwidth probe: the XOR of the words it writes
equals the XOR of every 32-bit word of the blocks a decode call over the same
sequences reads (computed with numpy from the pool bytes), for any number of
wavefronts, zero-length and ragged sequences included."""
import numpy as np
import pytest
import torch

import nvfp4_quantized_kv_amd as kv

pytestmark = pytest.mark.gpu


def _expected(pool_bytes, num_pages, layers, hkv, layer, table, lens):
    blocks = pool_bytes.reshape(layers, num_pages, hkv, 9216)
    acc = np.uint32(0)
    for s, n in enumerate(lens):
        for kvh in range(hkv):
            for j in range((n + 63) // 64):
                words = blocks[layer, table[s, j], kvh].view(np.uint32)
                acc ^= np.bitwise_xor.reduce(words)
    return int(acc)


@pytest.mark.parametrize("n_waves", [1, 7, 64, 3000])
def test_stream_read_xor(n_waves):
    pages, layers, hkv = 90, 2, 3
    pool = kv.Pool.allocate(pages, layers, hkv, 32, 1, "cuda")
    g = torch.Generator(device="cuda").manual_seed(5)
    pool.data.copy_(torch.randint(0, 256, pool.data.shape, generator=g, dtype=torch.uint8, device="cuda"))
    lens = [1000, 0, 65, 64, 1, 1700]
    rng = np.random.default_rng(11)
    stride = 30
    table = rng.integers(0, pages, (len(lens), stride)).astype(np.int32)
    words = kv.nvfp4kv_stream_read(pool, 1, torch.from_numpy(table).cuda(),
                                   torch.tensor(lens, dtype=torch.int32, device="cuda"), n_waves)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(words.cpu().numpy().view(np.uint32)))
    ref = _expected(pool.data.cpu().numpy(), pages, layers, hkv, 1, table, lens)
    assert got == ref
