"""The entry points under HIP graph capture: one graph holding the streaming,
short-sequence, split-key (caller workspace and library scratch) and masked
forwards is replayed several times, with other GPU work and host
synchronisation between the replays, and every replay must equal the eager
launches bit for bit (the kernels are deterministic and allocate nothing)."""
import numpy as np
import pytest
import torch

import attn_inputs as ai
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _problems():
    # (name, case, causal, kind, n_splits)
    return [
        ("streaming", ai.random_case(2, 4, 1000, 128, ai.F16, seed=70_001, key_len=[1000, 613]),
         True, "fwd", 0),
        ("short", ai.random_case(3, 2, 200, 32, ai.BF16, seed=70_002, key_len=[200, 17, 0]),
         False, "fwd", 0),
        ("split", ai.random_case_general(2, 8, 2, 1, 3000, 64, ai.BF16, seed=70_003,
                                         key_len=[3000, 1234]), True, "split", 4),
        ("static", ai.random_case_general(2, 16, 4, 1, 2000, 128, ai.F16, seed=70_004,
                                          key_len=[2000, 77]), True, "static", 3),
        ("masked", ai.random_case_general(1, 4, 2, 300, 500, 64, ai.F16, seed=70_005), False,
         "masked", 0),
    ]


def _launch(attn, kind, q, k, v, o, lse, kl, scale, causal, n_splits, ws, mask):
    if kind == "fwd":
        attn.attn_fwd(q, k, v, o, lse, scale=scale, causal=causal, key_len=kl)
    elif kind == "split":
        attn.attn_fwd_gqa_splitkv(q, k, v, o, lse, workspace=ws, n_splits=n_splits, scale=scale,
                                  causal=causal, key_len=kl)
    elif kind == "static":
        attn.attn_fwd_gqa_splitkv_static(q, k, v, o, lse, n_splits=n_splits, scale=scale,
                                         causal=causal, key_len=kl)
    else:
        attn.attn_fwd_masked(q, k, v, o, lse, mask=mask, scale=scale, causal=causal, key_len=kl)


def test_graph_replays_equal_eager_launches():
    import exact_self_attention_amd as attn
    dev = gu.device()
    runs = []
    for name, case, causal, kind, n_splits in _problems():
        q, k, v, kl = gu.dev_inputs(case)
        ws = None
        if kind == "split":
            nbytes = attn.attn_fwd_splitkv_workspace_bytes(q.shape[0], q.shape[1], q.shape[2],
                                                           q.shape[3], n_splits)
            ws = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
        mask = None
        if kind == "masked":
            rng = np.random.Generator(np.random.PCG64(70_100))
            m = rng.normal(0.0, 1.0, (q.shape[2], k.shape[2])).astype(np.float32)
            m[rng.random(m.shape) < 0.2] = -np.inf
            mask = torch.from_numpy(m).to(dev)
        o_eager = torch.empty_like(q)
        lse_eager = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        o_graph = torch.empty_like(q)
        lse_graph = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        runs.append(dict(name=name, kind=kind, causal=causal, n_splits=n_splits, q=q, k=k, v=v,
                         kl=kl, ws=ws, mask=mask, scale=float(case["scale"]), o_eager=o_eager,
                         lse_eager=lse_eager, o_graph=o_graph, lse_graph=lse_graph))

    def launch(r, o, lse):
        _launch(attn, r["kind"], r["q"], r["k"], r["v"], o, lse, r["kl"], r["scale"], r["causal"],
                r["n_splits"], r["ws"], r["mask"])

    # eager results (the first call of the static form also looks up its
    # scratch address, outside the capture)
    for r in runs:
        gu.log(f"graph test: eager {r['name']}")
        launch(r, r["o_eager"], r["lse_eager"])
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in runs:
            launch(r, r["o_graph"], r["lse_graph"])
    torch.cuda.synchronize()

    other = runs[0]
    scratch_o = torch.empty_like(other["q"])
    for rep in range(3):
        for r in runs:
            r["o_graph"].fill_(float("nan"))
            r["lse_graph"].fill_(float("nan"))
        # eager work of the program between replays, then a host wait
        launch(other, scratch_o, None)
        torch.cuda.synchronize()
        gu.log(f"graph test: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for r in runs:
            assert torch.equal(r["o_graph"].view(torch.int16), r["o_eager"].view(torch.int16)), \
                (r["name"], rep)
            # (-inf for rows that see no key compares equal; NaN would not)
            assert torch.equal(r["lse_graph"], r["lse_eager"]), (r["name"], rep)


def test_concurrent_host_threads_and_streams_equal_sequential():
    # two host threads, each launching its problems repeatedly on its own
    # stream (default priority) while the other does the same: the C entry
    # points run concurrently (ctypes releases the GIL), and every output
    # equals the one a single sequential launch gives
    import threading
    import exact_self_attention_amd as attn
    dev = gu.device()
    probs = _problems()
    runs = []
    for name, case, causal, kind, n_splits in probs:
        if kind == "static":  # one library scratch per device: calls on two streams race
            continue
        q, k, v, kl = gu.dev_inputs(case)
        ws = None
        if kind == "split":
            nbytes = attn.attn_fwd_splitkv_workspace_bytes(q.shape[0], q.shape[1], q.shape[2],
                                                           q.shape[3], n_splits)
            ws = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
        mask = None
        if kind == "masked":
            rng = np.random.Generator(np.random.PCG64(70_200))
            mask = torch.from_numpy(rng.normal(0.0, 1.0, (q.shape[2], k.shape[2])).astype(np.float32)).to(dev)
        ref = torch.empty_like(q)
        _launch(attn, kind, q, k, v, ref, None, kl, float(case["scale"]), causal, n_splits, ws, mask)
        runs.append((name, kind, causal, n_splits, q, k, v, kl, ws, mask, float(case["scale"]), ref))
    torch.cuda.synchronize()

    # split the problems between the threads; each thread owns its outputs
    # and workspaces, so nothing is shared but the inputs
    halves = [runs[0::2], runs[1::2]]
    outs = [[torch.empty_like(r[4]) for r in h] for h in halves]
    wss = [[None if r[8] is None else torch.empty_like(r[8]) for r in h] for h in halves]
    errors = []

    def worker(t):
        try:
            s = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(s):
                for _ in range(10):
                    for i, r in enumerate(halves[t]):
                        name, kind, causal, n_splits, q, k, v, kl, _, mask, scale, _ = r
                        _launch(attn, kind, q, k, v, outs[t][i], None, kl, scale, causal, n_splits,
                                wss[t][i], mask)
            s.synchronize()
        except Exception as e:  # reported on the main thread
            errors.append(e)

    gu.log("concurrent streams: two host threads")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(2):
        for i, r in enumerate(halves[t]):
            assert torch.equal(outs[t][i].view(torch.int16), r[11].view(torch.int16)), r[0]
