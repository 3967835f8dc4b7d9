"""gdla_decode_noalloc (the decode entry point that allocates nothing: its
split partials live in the library's per-GPU scratch array) against
gdla_decode with a caller workspace, through the C ABI.

Two calls in a row on the same scratch, the second with a smaller input
(fewer sequences, shorter caches, a different split count): each must equal
gdla_decode's output bit for bit (same kernels, same splits) and the oracle
to the parity bar."""
import numpy as np
import pytest
import torch

import workload as W
from gdla_testutil import compare, log, oracle_decode, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    import attention_gdla_prefill_amd._lib as L
    L.load()
    yield


def case(lengths, n_kv, seed):
    w = W.Workload("noalloc", "decode", B=len(lengths), n_kv=n_kv)
    return to_dev(W.decode_inputs(w, seed=seed, lengths=torch.tensor(lengths), q_std=1.0, k_std=1.0))


def run_both(d, max_len, window):
    import attention_gdla_prefill_amd as gdla
    B, n_sig = d["q_signal"].shape[:2]
    args = (d["q_signal"], d["q_noise"], d["k_cache"], d["v_cache"], d["cu_seqlens"], max_len, d["lam"], d["gate"])
    want = gdla.decode(*args, window=window,
                       out=torch.full((B, n_sig, 128), float("nan"), dtype=torch.bfloat16, device="cuda"))
    got = torch.full((B, n_sig, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    gdla.decode_noalloc(*args, window=window, out=got)
    torch.cuda.synchronize()
    return got, want


@pytest.mark.parametrize("window", [0, 128])
def test_decode_noalloc_matches_decode_twice(window):
    import attention_gdla_prefill_amd as gdla
    first = [9000, 4097, 300, 1, 2049, 7000]
    second = [3000, 40, 2500]
    for lengths, n_kv, seed in ((first, 3, 21), (second, 2, 22)):
        log("decode_noalloc lengths=%s n_kv=%d W=%d (scratch %d bytes, %d needed)"
            % (lengths, n_kv, window, gdla.decode_noalloc_max_scratch(),
               gdla.decode_workspace_size(len(lengths), n_kv, max(lengths), window)))
        d = case(lengths, n_kv, seed)
        got, want = run_both(d, max(lengths), window)
        assert torch.equal(got, want), "decode_noalloc differs from decode"
        compare(got, oracle_decode(d, window), "decode_noalloc W%d B%d" % (window, len(lengths)))


def test_decode_noalloc_rejects_beyond_scratch():
    """A call whose partials exceed the scratch is refused before any launch
    and leaves the output untouched."""
    import attention_gdla_prefill_amd as gdla
    d = case([1] * 64, 16, 23)
    out = torch.full((64, 64, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    huge = 1 << 30          # a max_seqlen_k that sizes far more splits than the scratch holds
    assert gdla.decode_workspace_size(64, 16, huge) > gdla.decode_noalloc_max_scratch()
    with pytest.raises(gdla.GdlaError) as e:
        gdla.decode_noalloc(d["q_signal"], d["q_noise"], d["k_cache"], d["v_cache"], d["cu_seqlens"], huge,
                            d["lam"], d["gate"], out=out)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
