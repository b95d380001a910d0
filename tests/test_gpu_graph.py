"""The decode step (append of every sequence's newest row, then the decode with fixed
partitions) captured once into a HIP graph and replayed: the library allocates nothing, clears
nothing with memset and never waits on the host, so the captured launches are the whole step.
The xInfer page replays its decode step as a captured graph (section "What actually sits
between the request and the tokens"). Every replay, with eager work and synchronisations in
between, must reproduce the eager step bit for bit, and every replay's output is also checked
against the oracle at the parity bar (2e-3 max-abs)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import fill, make_cache, to_dev, upload_tables

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _oracle_outs(W, q_bits, kv):
    """The oracle's decode of every sequence (its rows after the step's append)."""
    return [oracle.decode_sequence(W.dtype, q_bits[b], kv[b][0], kv[b][1], W.softmax_scale)[0]
            for b in range(W.batch)]


def _check_oracle(W, out, wants, what):
    got = out.cpu().numpy().astype(np.float64)
    for b, want in enumerate(wants):
        err = np.max(np.abs(got[b] - want))
        assert err <= TOL, f"{what}: seq {b} (L={W.seq_len(b)}): {err:.3e} from the oracle"


@pytest.mark.parametrize("dtype,hq", [(4, 16), (8, 32), (3, 40)])
def test_step_replays_from_a_captured_graph(dtype, hq):
    print("CASE graph", dtype, hq, flush=True)
    lens = [300, 45, 700, 1, 1029, 64]
    W = workloads.make(f"graph-{dtype}", 900 + dtype, dtype, lens, hq, 8, 16)
    cache = make_cache(W)
    bt, cl = upload_tables(W)
    kv = {b: W.kv_bits(b) for b in range(W.batch)}
    fill(cache, W, bt, kv=kv)
    qb = W.q_bits()
    q = to_dev(qb)
    # the step's new rows: each sequence's last position again (same data, so every replay
    # leaves the cache as it was)
    k_new = to_dev(np.stack([kv[b][0][-1] for b in range(W.batch)]))
    v_new = to_dev(np.stack([kv[b][1][-1] for b in range(W.batch)]))
    seq = to_dev(np.arange(W.batch, dtype=np.int32))
    pos = to_dev(np.array([L - 1 for L in lens], np.int32))
    hint, max_ctx = -256, W.max_context_len
    out = torch.empty((W.batch, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty((max(16, cache.workspace_bytes(W.batch, hq, max_ctx, hint)),), dtype=torch.uint8,
                     device="cuda")

    def step():
        cache.append(k_new, v_new, seq, pos, bt)
        cache.decode(q, bt, cl, max_ctx, W.softmax_scale, hint, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    want = out.clone()

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
    wants = _oracle_outs(W, qb, kv)
    for r in range(4):
        out.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda").sum()     # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r} differs from the eager step"
        assert bool(torch.isfinite(scratch))
        _check_oracle(W, out, wants, f"replay {r}")
    del graph


def test_layer_steps_replay_from_one_graph():
    """Several fused append + decode steps, one per layer cache, captured into ONE graph (as a
    model's decode graph holds a step per layer) and replayed: every layer's output must equal
    its eager step bit for bit on every replay, and the oracle's decode within the parity bar."""
    print("CASE graph layers", flush=True)
    lens = [300, 45, 700, 1, 1029, 64, 513, 128, 2000, 17, 900, 31, 256, 640, 77, 1500]
    hq, layers, refs = 16, [], []
    for layer in range(3):
        W = workloads.make(f"graph-layer-{layer}", 950 + layer, 4, lens, hq, 8, 16)
        cache = make_cache(W)
        bt, cl = upload_tables(W)
        kv = {b: W.kv_bits(b) for b in range(W.batch)}
        fill(cache, W, bt, kv=kv)
        k_new = to_dev(np.stack([kv[b][0][-1] for b in range(W.batch)]))
        v_new = to_dev(np.stack([kv[b][1][-1] for b in range(W.batch)]))
        max_ctx = W.max_context_len
        ws = torch.empty((max(16, cache.workspace_bytes(W.batch, hq, max_ctx, 0)),), dtype=torch.uint8,
                         device="cuda")
        order = cache.plan([int(x) for x in W.context_lens], hq, max_ctx, 0)
        out = torch.empty((W.batch, hq, 128), dtype=torch.float32, device="cuda")
        layers.append((W, cache, bt, cl, to_dev(W.q_bits()), k_new, v_new, ws, order, out))
        refs.append(_oracle_outs(W, W.q_bits(), kv))

    def step(layer):
        W, cache, bt, cl, q, k_new, v_new, ws, order, out = layer
        cache.append_decode(k_new, v_new, q, bt, cl, W.max_context_len, W.softmax_scale, 0, out=out,
                            workspace=ws, seq_order=order)

    want = []
    for layer in layers:
        step(layer)
        torch.cuda.synchronize()
        want.append(layer[-1].clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for layer in layers:
            step(layer)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for layer in layers:
            step(layer)
    torch.cuda.synchronize()
    for r in range(3):
        for layer in layers:
            layer[-1].fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda").sum()     # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, layer in enumerate(layers):
            assert torch.equal(layer[-1], want[i]), f"replay {r}, layer {i} differs from its eager step"
            _check_oracle(layer[0], layer[-1], refs[i], f"replay {r}, layer {i}")
        assert bool(torch.isfinite(scratch))
    del graph


@pytest.mark.parametrize("dtype,splits", [(4, 0), (3, 3), (8, 2)])
def test_prefill_replays_from_a_captured_graph(dtype, splits):
    """A prefill chunk (the tile kernel, and with several partitions its combine) captured into a
    graph and replayed: every replay equals the eager call bit for bit and the oracle's prefill
    within the parity bar (the infero page's chunked prefill, section "Beyond plain text
    decode", item "Continuous batching")."""
    print("CASE graph prefill", dtype, splits, flush=True)
    start, chunk, hq, hkv = 600, 70, 32, 8
    W = workloads.make(f"graph-prefill-{dtype}", 970 + dtype, dtype, [start + chunk], hq, hkv, 16)
    cache = make_cache(W)
    bt, _ = upload_tables(W)
    k, v = W.kv_bits(0)
    fill(cache, W, bt, kv={0: (k, v)})
    r = np.random.default_rng(dtype)
    qb = workloads.round_to_bf16_bits(r.standard_normal((chunk, hq, 128)).astype(np.float32))
    q = to_dev(qb)
    import bit_quantized_paged_turbo_amd as xq
    need = xq.xq_prefill_workspace_bytes(cache.layout, chunk, hq, start, splits)
    ws = torch.empty((max(16, need),), dtype=torch.uint8, device="cuda")
    out = torch.empty((chunk, hq, 128), dtype=torch.float32, device="cuda")

    def call():
        cache.prefill(q, bt[0], start, W.softmax_scale, splits, out=out, workspace=ws)

    call()
    torch.cuda.synchronize()
    want = out.clone()
    ref = oracle.prefill_sequence(dtype, qb, k, v, start, W.softmax_scale)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda").sum()     # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep} differs from the eager call"
        err = np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref))
        assert err <= TOL, f"replay {rep}: {err:.3e} from the oracle"
        assert bool(torch.isfinite(scratch))
    del graph
