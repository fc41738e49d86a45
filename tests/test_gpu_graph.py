"""The decode step captured once in a HIP graph and replayed, as the benchmark
times it: every replay writes exactly the bytes that the same step issued
eagerly writes (outputs, top-k sets, updated pages, staging rows and fold
states).  Before each replay the outputs are overwritten with garbage, so a
replay that skipped a write would show; between replays the test runs eager
work of its own and synchronizes, and every replay is checked, not only the
last.
"""

import math

import numpy as np
import pytest
import torch

import bench
import synth
from synth import gen
from tests import helpers as H

pytestmark = pytest.mark.gpu

hca = pytest.importorskip("decode_attention_compressed_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hca.lib()


def _workload():
    # one c4a layer (fp4 indexer keys, 8-token windows, top-256) and one c128a
    # layer, three sequences of drawn lengths with partial last blocks
    c4a = synth.LayerKind("c4a", 4, 256, "fp4", 128, 16, overlap=4)
    return synth.Workload(103, "graph-replay", 3, None, 512, 64, 128, "fp8", [c4a, synth.LayerKind("c128a", 128, None)],
                          L_range=(3000, 20000))


def _state(layers):
    """Every tensor a layer holds (inputs included, which must not change), and its pools' bytes."""
    snap = {}
    for li, lay in enumerate(layers):
        for name, v in sorted(vars(lay).items()):
            if isinstance(v, torch.Tensor):
                snap[f"{li}:{name}"] = v.detach().clone()
            elif isinstance(v, hca.PagedCache):
                snap[f"{li}:{name}.codes"] = v.codes.detach().clone()
                if v.scales is not None:
                    snap[f"{li}:{name}.scales"] = v.scales.detach().clone()
    return snap


def _poison(layers):
    """Overwrite the step's outputs with garbage (eager fills, not graph work)."""
    for lay in layers:
        lay.out8.fill_(0x5A)
        lay.out8s.fill_(-3.0)
        lay.lse.fill_(float("nan"))
        if getattr(lay, "sel", None) is not None:
            lay.sel.fill_(-7)
            lay.sel_n.fill_(-7)


def _same(a, b):
    return a.shape == b.shape and torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_graph_replays_write_the_eager_bytes():
    H.flush("graph replay: c4a + c128a step")
    w = _workload()
    layers, shared, _ = bench.build_state(w, len(w.layers), torch, hca, gen, lambda s: None)
    Lmax = shared["Lmax"]
    ws_idx = hca.workspace(hca.indexer_topk_workspace(w.B, Lmax, 4, 256))
    ws_att = {k: hca.workspace(hca.paged_hybrid_decode_workspace(w.B, w.H, w.d, Lmax, m, w.window, tk))
              for k, m, tk in (("c4a", 4, 256), ("c128a", 128, 0))}
    step = lambda: bench.decode_step(w, layers, shared, ws_idx, ws_att, hca)

    # the eager step, twice: the update is idempotent, so the second pass
    # (the state every replay starts from) must equal the first
    step()
    torch.cuda.synchronize()
    first = _state(layers)
    _poison(layers)
    step()
    torch.cuda.synchronize()
    eager = _state(layers)
    assert [k for k in first if not _same(first[k], eager[k])] == []
    assert any(int(t.numel()) > 0 for t in eager.values())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    noise = torch.empty(1 << 20, device="cuda")
    for rep in range(3):
        _poison(layers)
        noise.normal_()  # eager work of the program's own between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _state(layers)
        bad = [k for k in eager if not _same(eager[k], got[k])]
        assert bad == [], (rep, bad)
    # the outputs are the attention of the step: finite, one lse per (b, h)
    for lay in layers:
        assert torch.isfinite(lay.lse).all()
        assert math.isfinite(float(lay.out8s.float().max()))
    del g
    torch.cuda.synchronize()
