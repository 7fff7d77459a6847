"""The read-bandwidth probe of the measurement library reads every byte it is given: its per-wave XORs
equal those computed on the host from the same bytes with the same
assignment of 16-byte vectors to workgroups, waves and loads."""
import numpy as np
import pytest
import torch

from draft_token_verification_spec_amd import measure

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP device")]


def host_sink(words32: np.ndarray) -> np.ndarray:
    vecs = words32.reshape(-1, 4)
    n16 = vecs.shape[0]
    per = 256 * 8  # vectors per workgroup
    groups = (n16 + per - 1) // per
    out = np.zeros(groups * 4, dtype=np.uint32)
    x = np.bitwise_xor.reduce(vecs, axis=1)  # one word per vector
    for i in range(n16):
        g, r = divmod(i, per)
        t = r % 256  # load k = r // 256 of thread t
        out[g * 4 + t // 64] ^= x[i]
    return out


@pytest.mark.parametrize("nbytes", [16, 32768, 3 * 32768 + 4096 + 16, 100000 * 16])
def test_probe_reads_every_byte(nbytes):
    g = np.random.default_rng(nbytes)
    words = g.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    print(f"case probe bytes={nbytes}", flush=True)
    data = torch.from_numpy(words.view(np.int32)).cuda()
    sink = measure.read_probe(data)
    torch.cuda.synchronize()
    want = host_sink(words)
    got = sink.cpu().numpy().view(np.uint32)[:want.size]
    np.testing.assert_array_equal(got, want)
