"""GPU check of the read-ceiling diagnostic: sv_read_probe must read every 16-byte word of its
buffer exactly once, so the xor of its per-workgroup folds equals the xor of all input words.
Needs an MI355X and the built library."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_block_verification_sv_amd as pkg

    pkg.lib()


# word counts: fewer words than workgroups, a ragged count, several rounds per workgroup
@pytest.mark.parametrize("n_words", [1, 7, 1000, 65537, 1 << 20])
def test_read_probe_reads_every_word_once(n_words):
    import draft_block_verification_sv_amd as pkg

    rng = np.random.default_rng(n_words)
    host = rng.integers(-(2**31), 2**31 - 1, size=4 * n_words, dtype=np.int64).astype(np.int32)
    dev = torch.from_numpy(host).to("cuda:0")
    out = pkg.read_probe(dev)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert got == want
