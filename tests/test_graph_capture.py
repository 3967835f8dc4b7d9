"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

An entry point given its output and workspace only enqueues kernels on the
caller's stream -- it allocates nothing, synchronises nothing and records no
memset -- so a serving or training loop can capture a prefill or decode step
once and replay it.  Each replay below runs after new values were written into
the captured input buffers and after eager work on the same device; it must
equal the eager call on the same inputs bit for bit (the kernels are
deterministic: every output element is summed in one fixed order)."""
import pytest
import torch

import workload as W
from gdla_testutil import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    import attention_gdla_prefill_amd._lib as L
    L.load()
    yield


def capture(fn):
    """One warm call on a side stream (default priority), then the capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_matches(g, bufs, out, new_inputs, eager, what):
    for rep, nd in enumerate(new_inputs):
        for k, t in bufs.items():
            t.copy_(nd[k])
        want = eager(nd)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(out, want)
        log("%s replay %d: bitwise equal to the eager call: %s" % (what, rep, same))
        assert same, "%s: replay %d differs from the eager call" % (what, rep)


@pytest.mark.parametrize("window", [0, 128])
def test_prefill_graph_replays(window):
    import attention_gdla_prefill_amd as gdla
    w = W.Workload("graph", "prefill", B=2, T=333, n_kv=2, window=window)
    keys = ("q_signal", "q_noise", "k", "v", "lam", "gate")
    x = to_dev(W.prefill_inputs(w, seed=1))
    bufs = {k: x[k] for k in keys}
    out = torch.empty(x["gate"].shape, dtype=torch.bfloat16, device="cuda")
    g = capture(lambda: gdla.prefill(*(bufs[k] for k in keys), window=window, out=out))
    new = [to_dev(W.prefill_inputs(w, seed=10 + i, q_std=1.0 if i else None)) for i in range(3)]
    replay_matches(g, bufs, out, new, lambda nd: gdla.prefill(*(nd[k] for k in keys), window=window),
                   "prefill W%d" % window)


DEC_KEYS = ("q_signal", "q_noise", "k_cache", "v_cache", "cu_seqlens", "lam", "gate")


def decode_case(lengths, seed, **kw):
    w = W.Workload("graph", "decode", B=len(lengths), n_kv=2)
    return to_dev(W.decode_inputs(w, seed=seed, lengths=torch.tensor(lengths), **kw))


def dec_args(d, max_len):
    return (d["q_signal"], d["q_noise"], d["k_cache"], d["v_cache"], d["cu_seqlens"], max_len, d["lam"], d["gate"])


@pytest.mark.parametrize("window", [0, 128])
def test_decode_graph_replays(window):
    """Full causal with several splits (the split and combine kernels), and the
    one-launch window kernel."""
    import attention_gdla_prefill_amd as gdla
    lengths = [1, 33, 600, 2500, 5000, 128]
    max_len = max(lengths)
    d = decode_case(lengths, 1)
    bufs = {k: d[k] for k in DEC_KEYS}
    B, n_sig = d["q_signal"].shape[:2]
    n_kv = d["q_noise"].shape[1]
    ws = torch.empty(max(16, gdla.decode_workspace_size(B, n_kv, max_len, window)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((B, n_sig, 128), dtype=torch.bfloat16, device="cuda")
    g = capture(lambda: gdla.decode(*dec_args(bufs, max_len), window=window, out=out, workspace=ws))
    new = [decode_case(lengths, 20 + i, q_std=1.0, k_std=1.0) for i in range(3)]
    replay_matches(g, bufs, out, new, lambda nd: gdla.decode(*dec_args(nd, max_len), window=window),
                   "decode W%d" % window)


def test_decode_noalloc_graph_replays():
    """The entry point that allocates nothing, its partials in the library's
    per-GPU scratch, captured and replayed likewise."""
    import attention_gdla_prefill_amd as gdla
    lengths = [7, 4100, 300, 2049]
    max_len = max(lengths)
    d = decode_case(lengths, 2)
    bufs = {k: d[k] for k in DEC_KEYS}
    B, n_sig = d["q_signal"].shape[:2]
    out = torch.empty((B, n_sig, 128), dtype=torch.bfloat16, device="cuda")
    g = capture(lambda: gdla.decode_noalloc(*dec_args(bufs, max_len), out=out))
    new = [decode_case(lengths, 30 + i, q_std=1.0, k_std=1.0) for i in range(3)]
    replay_matches(g, bufs, out, new, lambda nd: gdla.decode(*dec_args(nd, max_len)), "decode_noalloc")


LAT_KEYS = ("q_signal", "q_noise", "latent", "cu_seqlens", "w_uk", "w_uv", "lam", "gate")


@pytest.mark.parametrize("window", [0, 128])
def test_decode_latent_graph_replays(window):
    """The latent decode: four launches (absorb, split, redo, combine) with
    several splits, or the one-launch window kernel."""
    import attention_gdla_prefill_amd as gdla
    lengths = [9000, 130, 4097, 12]
    max_len = max(lengths)
    w = W.Workload("graph", "decode_latent", B=len(lengths), n_kv=2, window=window)
    case = lambda seed: to_dev(W.latent_decode_inputs(w, seed=seed, lengths=torch.tensor(lengths), q_std=1.0))
    d = case(1)
    bufs = {k: d[k] for k in LAT_KEYS}
    B, n_sig = d["q_signal"].shape[:2]
    ws = torch.empty(max(256, gdla.decode_latent_workspace_size(B, 2, max_len, window)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((B, n_sig, 128), dtype=torch.bfloat16, device="cuda")
    args = lambda t: (t["q_signal"], t["q_noise"], t["latent"], t["cu_seqlens"], max_len, t["w_uk"], t["w_uv"],
                      t["lam"], t["gate"])
    g = capture(lambda: gdla.decode_latent(*args(bufs), window=window, out=out, workspace=ws))
    new = [case(40 + i) for i in range(3)]
    replay_matches(g, bufs, out, new, lambda nd: gdla.decode_latent(*args(nd), window=window),
                   "latent decode W%d" % window)


def test_prep_graph_replays():
    """The step ahead of the core rotates its inputs in place: each replay
    starts from new unrotated values written into the captured buffers, and
    the rotated buffers, lambda and the gate must equal an eager call on a
    copy of the same values.  9,000 tokens: lambda's 64-token form."""
    import attention_gdla_prefill_amd as gdla
    w = W.Workload("graph", "prefill", B=1, T=9000, n_kv=2)
    keys = ("q_signal", "q_noise", "k_rope", "k", "x", "w_lambda", "gate_pre")
    d = to_dev(W.prep_inputs(w, seed=1, d_model=256))
    bufs = {k: d[k] for k in keys}
    lam = torch.empty((1, 9000, 8), dtype=torch.bfloat16, device="cuda")
    gate = torch.empty_like(d["gate_pre"])
    call = lambda t, lo, go: gdla.prep(t["q_signal"], t["q_noise"], t["k_rope"], t["k"], t["x"], t["w_lambda"],
                                       t["gate_pre"], pos0=5, lam_out=lo, gate_out=go)
    g = capture(lambda: call(bufs, lam, gate))
    for rep in range(3):
        nd = to_dev(W.prep_inputs(w, seed=50 + rep, d_model=256))
        for k in keys:
            bufs[k].copy_(nd[k])
        want_lam, want_gate = call(nd, None, None)       # rotates nd's buffers in place
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in ((lam, want_lam), (gate, want_gate), (bufs["q_signal"], nd["q_signal"]),
                                                  (bufs["q_noise"], nd["q_noise"]), (bufs["k"], nd["k"])))
        log("prep replay %d: bitwise equal to the eager call: %s" % (rep, same))
        assert same, "prep: replay %d differs from the eager call" % rep


def test_backward_graph_replays():
    """The backward: the saving forward, the element-wise kernel and both
    gradient kernels in one graph; its six gradients live in the graph's own
    memory and are read after each replay."""
    import attention_gdla_prefill_amd as gdla
    w = W.Workload("graph", "prefill", B=1, T=200, n_kv=2, window=64)
    keys = ("q_signal", "q_noise", "k", "v", "lam", "gate")
    case = lambda seed: to_dev(W.prefill_inputs(w, seed=seed, q_std=1.0))
    d = case(1)
    gen = torch.Generator().manual_seed(7)
    dout = torch.randn(d["gate"].shape, generator=gen).to(torch.bfloat16).cuda()
    bufs = dict({k: d[k] for k in keys}, d_out=dout)
    ws = torch.empty(max(256, gdla.prefill_backward_workspace_size(1, 200, 2)), dtype=torch.uint8, device="cuda")
    run = lambda t, wsp: gdla.prefill_backward(*(t[k] for k in keys), t["d_out"], window=64, workspace=wsp)
    grads = {}
    g = capture(lambda: grads.update(run(bufs, ws)))
    for rep in range(3):
        nd = case(60 + rep)
        nd["d_out"] = torch.randn(d["gate"].shape, generator=gen).to(torch.bfloat16).cuda()
        for k, t in bufs.items():
            t.copy_(nd[k])
        want = run(nd, None)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(grads[k], want[k]) for k in want)
        log("backward replay %d: bitwise equal to the eager call: %s" % (rep, same))
        assert same, "backward: replay %d differs from the eager call" % rep
