"""Decode-step benchmark of the hybrid compressed-KV decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4]

Workload (default): the 1M-token long-context stack -- batch 4, context 2^20,
61 layers (30 c4a: m=4, 262,144 entries, indexer top-2048 over fp4 E2M1 keys
with per-32 E4M3 scales; 31 c128a: m=128, 8,192 entries, all attended), shared
K=V dim 512 in fp8 E4M3 pages with a per-page fp32 scale, 64 query heads, a
128-token raw window.  The caches are filled by a prefill pass on the GPU
(kv_compress + kv_quantize_page over all 2^20 tokens of every layer), timed
and reported on its own.

A step is one decode step of the whole stack for the batch: per layer the
decode update (the open group's entry -- c4a: re-folded over its 8-token
window at stride 4; c128a: the newest token folded into the group's running
fold state -- with its RMSNorm and RoPE, and its page, the window insert of the new token and its page, the open indexer page:
one kv_compress_insert_jobs launch), then indexer_topk (c4a) and
paged_hybrid_decode, whose output is delivered as fp8 rows with a per-row
scale; layers stay in order.  The step is captured once in a HIP graph and replayed; `value` is
decode tokens/s = B / step time.

Also reported: the roofline of the dominant kernel (the indexer scoring
kernel: it streams the fp4 keys, ~77% of a step's bytes), measured with HIP
events around each of its launches; and the CPU oracle timed on a bounded
sample of the same workload.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s

# HBM bytes per launch of the fp4 score kernel on this workload, from
# rocprofv3 FETCH_SIZE and WRITE_SIZE passes over `bench.py --layers 2`, each
# scaled by what the same counter reads for the 1 GiB device copy in
# copy_bandwidth() (the summary with the commands is in profiles/).  They hold
# only for the kernel source they were taken on, identified by the SHA-256 of
# the indexer source and the headers it includes; otherwise traffic is null.
SCORE_TRAFFIC = {"source_sha256": "27475ce318c5781463f87d33311f670bd7d76570ff0046bf4fc387a5a086d253",
                 "fetch_bytes": 72065010, "write_bytes": 4671982}
SCORE_SOURCES = ("decode_attention_compressed_amd/csrc/indexer.hip", "decode_attention_compressed_amd/csrc/hca_common.h",
                 "decode_attention_compressed_amd/csrc/indexer_internal.h",
                 "decode_attention_compressed_amd/csrc/indexer_score.h")


def score_source_sha256():
    import hashlib

    h = hashlib.sha256()
    for f in SCORE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_of(kind):
    t = SCORE_TRAFFIC
    if t["source_sha256"] is None or kind.idx_dtype != "fp4" or score_source_sha256() != t["source_sha256"]:
        return None
    return int(t["fetch_bytes"] + t["write_bytes"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=0, help="debug only: first N layers (result is not the workload)")
    ap.add_argument("--replicas", type=int, default=0,
                    help="copies of a single-layer workload's caches, one per timed step in turn, so that one "
                         "step's pages are not still in the Infinity Cache from the step before (0: 4 for a "
                         "single-layer workload, 1 otherwise)")
    return ap.parse_args()


# ----------------------------------------------------------------- algorithmic bytes


def layer_bytes(kind, B, L, d, H, W, d_idx=128, h_idx=16):
    """Algorithmic HBM bytes of one decode step of one layer for the batch: each
    stored row read once (codes + its share of scales), queries, outputs, block
    table entries read; intermediate scores and indices are not counted."""
    m = kind.m
    N = -(-L // m)
    epp = 256 // m
    win = min(W, L)
    q = H * d * 2
    out = H * d + H * 4 + H * 4  # fp8 output row, its scale, the lse
    win_rows = win * d + 4 * (-(-win // 256) + 1)
    if kind.topk is not None:
        kk = min(kind.topk, N)
        idx_row = d_idx // 2 + d_idx // 32 if kind.idx_dtype == "fp4" else d_idx + 4.0 / epp
        idx = N * idx_row + h_idx * d_idx * 2 + h_idx * 4 + 4 * (-(-N // epp))
        rows = kk * (d + 4)  # each selected row and its page scale
        per_seq = idx + rows + win_rows + q + out + 4 * kk
    else:
        rows = N * d + 4 * (-(-N // epp))
        per_seq = rows + win_rows + q + out + 4 * (-(-N // epp))
    return B * per_seq


def score_bytes(kind, B, L, d_idx=128, h_idx=16):
    m = kind.m
    N = -(-L // m)
    epp = 256 // m
    idx_row = d_idx // 2 + d_idx // 32 if kind.idx_dtype == "fp4" else d_idx + 4.0 / epp
    return B * (N * idx_row + h_idx * d_idx * 2 + h_idx * 4 + 4 * (-(-N // epp)))


def update_bytes(kind, B, d, d_idx=128):
    """Bytes moved by the decode update of one layer while page scales hold
    (open group, open page, window page, open indexer page)."""
    m, epp, s = kind.m, 256 // kind.m, kind.slots
    if m > 16:  # the newest token + logit, the running fold state read and written, entry write
        b = d * 2 + 4 + 2 * (4 + d) * 4 + d * 4
    else:  # the window's ring tokens + logits, entry write
        b = s * d * 2 + s * 4 + d * 4
    b += 16 + d + 8  # open page: its header (amax of the closed rows), the row's codes, scale
    b += d * 2 + 4 + d * 4 + d + 8  # window token + logit, its staging row, its codes, scale
    if kind.topk is not None:
        b += d_idx * 4 + d_idx // 2 + d_idx // 32  # open indexer row: staging, codes, scales
    return B * b


# ----------------------------------------------------------------- GPU state


class Layer:
    pass


def build_state(w, n_layers, torch, hca, gen, log, replicas=1):
    """Fill every layer's pools with a GPU prefill pass; keep the decode-update
    state.  With replicas > 1 every layer is built that many times over (own
    pools and inputs: layer index li takes the kind of layer li % n_layers).
    Returns (layers, prefill stats)."""
    B, L, d, H, W = w.B, w.L, w.d, w.H, w.window
    lens_np = np.full((B,), L, np.int32)
    table_np, P, wtable_np, PW = gen.block_tables(w, lens_np)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    table, wtable, lens = dev(table_np), dev(wtable_np), dev(lens_np)
    zeros_b = dev(np.zeros(B, np.int32))
    layers = []
    pre_ms, pre_bytes = 0.0, 0.0
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for li in range(n_layers * replicas):
        kind = w.layers[li % n_layers]
        m, epp = kind.m, 256 // kind.m
        N = -(-L // m)
        lay = Layer()
        lay.kind, lay.N, lay.epp = kind, N, epp
        # raw tokens and logits of the whole context (seeded device draws)
        x = torch.empty((B, L, d), dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            x[b] = gen.device_normal((L, d), 1.0, (0, w.cid, li, gen.S_TOK, b), dtype=torch.bfloat16)
        z = gen.device_normal((B, L), 1.0, (0, w.cid, li, gen.S_LOGIT))
        o = kind.overlap
        beta = dev(gen.slot_bias(w, li, kind.slots))
        lay.gamma = dev(gen.norm_gain(w, li, d))
        ent = torch.empty((B, N, d), dtype=torch.float32, device="cuda")
        lay.kv = hca.PagedCache.empty(P, epp, d, w.kv_dtype)
        xi = x.view(torch.int16)
        torch.cuda.synchronize()
        ev0.record()
        hca.kv_compress(xi, z, beta, zeros_b, lens, m, w.theta, ent, L, norm_gamma=lay.gamma, overlap=o)
        hca.kv_quantize_page(ent, zeros_b, dev(np.full(B, N, np.int32)), N, table, lay.kv)
        ev1.record()
        torch.cuda.synchronize()
        pre_ms += ev0.elapsed_time(ev1)
        pre_bytes += B * (L * d * 2 + L * 4 + 2 * N * d * 4 + N * d + 4 * (-(-N // epp)))
        # decode-update state: the ring of the open group's window (the overlap's
        # tokens of the group before, then the open group), open page staging
        g_open = (L - 1) // m
        nt_open = L - g_open * m
        p_lo = max(0, g_open * m - o)
        lay.ring_x = torch.zeros((B, o + m, d), dtype=torch.int16, device="cuda")
        lay.ring_x[:, o - (g_open * m - p_lo): o + nt_open] = xi[:, p_lo: L]
        lay.ring_z = torch.zeros((B, o + m), dtype=torch.float32, device="cuda")
        lay.ring_z[:, o - (g_open * m - p_lo): o + nt_open] = z[:, p_lo: L]
        lay.x_open, lay.z_open = lay.ring_x[:, o:], lay.ring_z[:, o:]  # rows -o .. -1: the overlap
        lay.beta = beta
        e_open0 = (g_open // epp) * epp
        lay.stage = torch.zeros((B, epp, d), dtype=torch.float32, device="cuda")
        lay.stage[:, : N - e_open0] = ent[:, e_open0: N]
        lay.slot = g_open - e_open0
        lay.pos0 = dev(np.full(B, g_open * m, np.int32))
        lay.ntok = dev(np.full(B, L - g_open * m, np.int32))
        lay.e0 = dev(np.full(B, e_open0, np.int32))
        # the entries' update state: the open page's header (the amax of its
        # closed rows) and, for groups of more than 16 tokens, a running fold
        # state, so an update folds only the newest token; that one is brought
        # to the state after the open group's tokens but the newest (what the
        # previous step left) by an update call with one token fewer
        lay.fstate = torch.zeros((B, 4 + (2 * (4 + d) if m > 16 else 0)), dtype=torch.float32, device="cuda")
        if m > 16:
            if L - g_open * m >= 2:
                hca.kv_compress_insert(lay.ring_x[:, o:], lay.ring_z[:, o:], beta, lay.pos0,
                                       dev(np.full(B, L - g_open * m - 1, np.int32)), m, w.theta, lay.stage, lay.e0,
                                       table, lay.kv, append=False, norm_gamma=lay.gamma, overlap=o,
                                       fold_state=lay.fstate)
        lay.ne = dev(np.full(B, N - e_open0, np.int32))
        del ent
        # window pages: rows of the blocks that overlap [L-W, L)
        t0 = (max(0, L - W) // 256) * 256
        nw = L - t0
        wrows = torch.empty((B, nw, d), dtype=torch.float32, device="cuda")
        hca.kv_compress(xi[:, t0:], z[:, t0:], dev(np.zeros(1, np.float32)), dev(np.full(B, t0, np.int32)),
                        dev(np.full(B, nw, np.int32)), 1, w.theta, wrows, nw)
        lay.win = hca.PagedCache.empty(PW, 256, d, w.kv_dtype)
        hca.kv_quantize_page(wrows, dev(np.full(B, t0, np.int32)), dev(np.full(B, nw, np.int32)), nw, wtable, lay.win)
        tw0 = ((L - 1) // 256) * 256
        lay.wstage = torch.zeros((B, 256, d), dtype=torch.float32, device="cuda")
        lay.wstage[:, : L - tw0] = wrows[:, tw0 - t0:]
        lay.wslot = (L - 1) - tw0
        lay.x_last = xi[:, L - 1: L].contiguous()
        lay.z_last = z[:, L - 1: L].contiguous()
        lay.wpos0 = dev(np.full(B, L - 1, np.int32))
        lay.one = dev(np.full(B, 1, np.int32))
        lay.we0 = dev(np.full(B, tw0, np.int32))
        lay.wne = dev(np.full(B, L - tw0, np.int32))
        lay.zero1 = dev(np.zeros(1, np.float32))
        del x, z, wrows
        # queries
        lay.q = dev(gen.queries(w, li).view(np.int16))
        if kind.topk is not None:
            keys = gen.device_normal((B, N, kind.d_idx), 1.0, (0, w.cid, li, gen.S_IDXK))
            lay.idx = hca.PagedCache.empty(P, epp, kind.d_idx, kind.idx_dtype)
            hca.kv_quantize_page(keys, zeros_b, dev(np.full(B, N, np.int32)), N, table, lay.idx)
            lay.istage = torch.zeros((B, epp, kind.d_idx), dtype=torch.float32, device="cuda")
            lay.istage[:, : N - e_open0] = keys[:, e_open0: N]
            del keys
            lay.qi = dev(gen.index_queries(w, li, kind.h_idx, kind.d_idx).view(np.int16))
            lay.wi = dev(gen.index_weights(w, li, kind.h_idx))
            lay.sel = torch.zeros((B, kind.topk), dtype=torch.int32, device="cuda")
            lay.sel_n = torch.zeros((B,), dtype=torch.int32, device="cuda")
        # the attention output in the fp8 form the next projection takes
        lay.out8 = torch.zeros((B, H, d), dtype=torch.uint8, device="cuda")
        lay.out8s = torch.zeros((B, H), dtype=torch.float32, device="cuda")
        lay.lse = torch.zeros((B, H), dtype=torch.float32, device="cuda")
        layers.append(lay)
        torch.cuda.synchronize()
        if li % 10 == 0 or li == n_layers - 1:
            log(f"prefilled layer {li + 1}/{n_layers} ({kind.name})")
    shared = dict(table=table, wtable=wtable, lens=lens)
    return layers, shared, dict(ms=pre_ms, bytes=pre_bytes)


def decode_step(w, layers, shared, ws_idx, ws_att, hca, update=True, attend=True):
    """One decode step of the stack.  Per layer: the update (the window insert
    with its page, the open group's re-fold with its page and, for c4a, the
    open indexer page), the indexer (c4a) and the attention, which the next
    layer's update waits for.  c128a: the update is one launch.  c4a: the
    update runs inside the indexer call (indexer_topk_with_updates): the open
    indexer row by the score pass, the window insert and the open entry as
    extra blocks of the select's last launch.
    The attend-only and update-only variants make the calls separately."""
    import torch
    L, W = w.L, w.window
    table, wtable, lens = shared["table"], shared["wtable"], shared["lens"]
    scale = 1.0 / math.sqrt(w.d)
    for lay in layers:
        kind = lay.kind
        m = kind.m
        jobs = [hca.insert_job(lay.wstage, lay.wpos0, lay.we0, wtable, lay.win, 1, x=lay.x_last,
                               gate_logit=lay.z_last, pos_bias=lay.zero1, ntok=lay.one, rope_theta=w.theta,
                               append=True),
                hca.insert_job(lay.stage, lay.pos0, lay.e0, table, lay.kv, m, x=lay.x_open, gate_logit=lay.z_open,
                               pos_bias=lay.beta, ntok=lay.ntok, rope_theta=w.theta, append=True,
                               norm_gamma=lay.gamma, overlap=kind.overlap, fold_state=lay.fstate)]
        idx_job = (hca.insert_job(lay.istage, lay.pos0, lay.e0, table, lay.idx, m, append=True)
                   if kind.topk is not None else None)
        if update and attend and kind.topk is not None:
            # the indexer with the updates: the open indexer row written by the
            # score pass, the window insert and the open entry's update beside
            # the select's compaction
            hca.indexer_topk_with_updates(lay.qi, lay.wi, lay.idx, table, lens, L, m, kind.topk, lay.sel, lay.sel_n,
                                          ws_idx, jobs + [idx_job])
        else:
            if update:
                hca.kv_compress_insert_jobs(jobs + ([idx_job] if idx_job is not None else []), w.B)
            if attend and kind.topk is not None:
                hca.indexer_topk(lay.qi, lay.wi, lay.idx, table, lens, L, m, kind.topk, lay.sel, lay.sel_n, ws_idx)
        if attend:
            if kind.topk is not None:
                hca.paged_hybrid_decode(lay.q, lay.kv, table, lay.win, wtable, lens, L, m, W, lay.sel, lay.sel_n,
                                        scale, w.theta, None, lay.lse, ws_att[kind.name], out_fp8=lay.out8,
                                        out_scale=lay.out8s)
            else:
                hca.paged_hybrid_decode(lay.q, lay.kv, table, lay.win, wtable, lens, L, m, W, None, None, scale,
                                        w.theta, None, lay.lse, ws_att[kind.name], out_fp8=lay.out8,
                                        out_scale=lay.out8s)


def time_graph(torch, fn, steps, warmup):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall, g


def time_dominant(torch, hca, w, layers, shared, reps=4):
    """Average duration of the indexer scoring kernel on the stream it runs on:
    a GPU sleep lets every launch queue first, then one event pair brackets
    reps x (c4a layers) back-to-back launches (one per layer's own keys, so
    consecutive launches do not re-read each other's bytes)."""
    c4a = [l for l in layers if l.kind.topk is not None]
    if not c4a:
        return None
    kind = c4a[0].kind
    ws = hca.workspace(hca.indexer_topk_workspace(w.B, w.L, kind.m, kind.topk))
    stream = torch.cuda.current_stream()
    res = []
    for _ in range(3):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(100_000_000)
        e0.record(stream)
        for _ in range(reps):
            for lay in c4a:
                hca.indexer_score(lay.qi, lay.wi, lay.idx, shared["table"], shared["lens"], w.L, kind.m, kind.topk, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / (reps * len(c4a)))
    return float(np.mean(res)), float(np.median(res)), reps * len(c4a) * len(res)


def copy_bandwidth(torch, nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of nbytes (read + write), timed with events:
    the measured ceiling beside the 8 TB/s datasheet figure, and, under
    rocprofv3 counters, the known-size launch that calibrates FETCH_SIZE and
    WRITE_SIZE."""
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        y.copy_(x)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del x, y
    return 2 * nbytes / (best * 1e-3) / 1e9


# ----------------------------------------------------------------- CPU baseline


def cpu_baseline(w, budget_s=20.0):
    """The oracle's decode step (indexer scores + top-k + gather/decode + attention
    + fp8 output)
    for ONE sequence of one c4a and one c128a layer, on page contents of the
    workload's shape (random codes: the oracle's time does not depend on the
    values); repeated while within budget; scaled to the 61-layer stack."""
    from oracle import attention, indexer, paging
    from oracle.rope import rope  # noqa: F401  (the attention path uses it)

    rng = np.random.default_rng(0)
    L, d, H, W = w.L, w.d, w.H, w.window
    out = {}
    kinds = {}
    for k in w.layers:
        kinds.setdefault(k.name, k)
    t_layer = {}
    reps = {}
    t_start = time.perf_counter()
    for name, kind in kinds.items():
        m, epp = kind.m, 256 // kind.m
        N = -(-L // m)
        P = -(-L // 256)
        table = rng.permutation(P)
        kv = paging.Pool("fp8", P, epp, d)
        kv.codes[:] = rng.integers(0, 0x7E, kv.codes.shape, dtype=np.uint8)
        kv.scales[:] = rng.uniform(1e-3, 1e-2, P).astype(np.float32)
        win = paging.Pool("fp8", 1, 256, d)
        win.codes[:] = rng.integers(0, 0x7E, win.codes.shape, dtype=np.uint8)
        wtable = np.full(P, -1)
        wtable[(L - 1) // 256] = 0
        q = rng.standard_normal((H, d))
        if kind.topk is not None:
            idx = paging.Pool(kind.idx_dtype, P, epp, kind.d_idx)
            idx.codes[:] = rng.integers(0, 256, idx.codes.shape, dtype=np.uint8)
            idx.scales[:] = rng.integers(0x20, 0x40, idx.scales.shape, dtype=np.uint8)
            qi, wi = rng.standard_normal((kind.h_idx, kind.d_idx)), rng.standard_normal(kind.h_idx)
        times = []
        while True:
            t0 = time.perf_counter()
            if kind.topk is not None:
                keys = paging.decode_rows(idx, table, np.arange(N))
                s = indexer.scores(qi, wi, keys)
                sel = indexer.topk(s, kind.topk)
            else:
                sel = np.arange(N)
            rows = paging.decode_rows(kv, table, sel)
            rows = np.concatenate([rows, paging.decode_rows(win, wtable, attention.window_positions(L, W))])
            o, _, _ = attention.attend(q, rows, L, 1.0 / math.sqrt(d), w.theta)
            attention.quantize_out_fp8(o)
            times.append(time.perf_counter() - t0)
            if sum(times) > budget_s / len(kinds) or len(times) >= 200:
                break
        t_layer[name] = float(np.median(times))
        reps[name] = len(times)
    n_kind = {name: sum(1 for k in w.layers if k.name == name) for name in kinds}
    t_seq_step = sum(t_layer[nm] * n_kind[nm] for nm in kinds)
    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    out = {
        "value": 1.0 / t_seq_step,
        "unit": "tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle decode step (indexer scores + top-k + row gather/decode + attention + fp8 output) of one "
                   f"sequence at L={L} for one c4a layer ({reps.get('c4a', 0)} runs, median "
                   f"{t_layer.get('c4a', 0):.2f} s) and one c128a layer ({reps.get('c128a', 0)} runs, median "
                   f"{t_layer.get('c128a', 0):.2f} s), scaled by the stack's {n_kind} layers; the batch's "
                   f"sequences are independent so batch tokens/s equals per-sequence tokens/s; "
                   f"wall {time.perf_counter() - t_start:.1f} s"),
    }
    return out


# ----------------------------------------------------------------- page-pool packing


def pool_packing(w, hca):
    """The stack's KV kinds packed into size buckets of one arena (host
    bookkeeping only): buckets, arena bytes, and the host time to give every
    sequence of every layer its pages (one allocation per layer, kind and
    sequence, the shared-prefix pages found by key), then release them."""
    kinds, count = [], []
    nb = -(-w.L // 256)
    for k in w.layers:
        main = (k.m, w.d, w.kv_dtype)
        if main not in kinds:
            kinds.append(main)
            count.append(0)
        count[kinds.index(main)] += nb
        if k.topk is not None:
            ik = (k.m, k.d_idx, k.idx_dtype)
            if ik not in kinds:
                kinds.append(ik)
                count.append(0)
            count[kinds.index(ik)] += nb
    win = (1, w.d, w.kv_dtype)
    kinds.append(win)
    count.append(2 * len(w.layers))  # the blocks that overlap the window
    probe = hca.PagePool(kinds, [1] * len(kinds))
    cap = [0] * probe.n_buckets
    for i, c in enumerate(count):
        cap[probe.bucket_of(i)] += c * w.B
    pool = hca.PagePool(kinds, cap)
    t0 = time.perf_counter()
    held = []
    for _ in range(w.B):
        for i, c in enumerate(count):
            b = pool.bucket_of(i)
            held.append((b, pool.alloc(b, c)))
    t1 = time.perf_counter()
    for b, pages in held:
        pool.release(b, pages)
    t2 = time.perf_counter()
    pages = sum(len(p) for _, p in held)
    return {"kinds": [f"m={m} d={d} {t}" for m, d, t in kinds], "buckets": probe.n_buckets,
            "arena_GiB": round(pool.arena_bytes / 2 ** 30, 3),
            "arena_GiB_per_sequence": round(pool.arena_bytes / 2 ** 30 / w.B, 3),
            "pages": pages, "alloc_ms": round((t1 - t0) * 1e3, 3), "release_ms": round((t2 - t1) * 1e3, 3)}


# ----------------------------------------------------------------- main


METRIC_WORKLOAD = {4: "1M-token 61-layer stack", 2: "128K-token c4a layer, batch 16",
                   1: "64K-token c128a layer, batch 8", 0: "4K-token c4a layer, batch 1"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_attention_compressed_amd as hca
    import synth
    from synth import gen

    log = lambda s: print(f"[bench] {s}", file=sys.stderr, flush=True)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    hca.lib()
    w = synth.workload(args.config)
    if w.L is None:
        print("bench.py times fixed-length workloads (configs 0, 1, 2, 4)", file=sys.stderr)
        sys.exit(2)
    n_layers = len(w.layers) if args.layers <= 0 else min(args.layers, len(w.layers))
    R = args.replicas if args.replicas > 0 else (4 if n_layers == 1 else 1)
    log(f"workload {w.name}: B={w.B} L={w.L} layers={n_layers} replicas={R}")
    layers, shared, pre = build_state(w, n_layers, torch, hca, gen, log, replicas=R)
    # workspaces (one per kind; the indexer one must start zeroed and is left zeroed)
    kinds = {l.kind.name: l.kind for l in layers}
    ws_idx = None
    ws_att = {}
    for name, kind in kinds.items():
        if kind.topk is not None:
            ws_idx = hca.workspace(hca.indexer_topk_workspace(w.B, w.L, kind.m, kind.topk))
        ws_att[name] = hca.workspace(hca.paged_hybrid_decode_workspace(w.B, w.H, w.d, w.L, kind.m, w.window,
                                                                       kind.topk or 0))
    torch.cuda.synchronize()
    log("capturing decode step")
    t_step, wall, _g = time_graph(torch, lambda: decode_step(w, layers, shared, ws_idx, ws_att, hca), args.steps,
                                  args.warmup)
    t_step /= R
    log(f"step {t_step:.3f} ms")
    t_attn, _, _g2 = time_graph(torch, lambda: decode_step(w, layers, shared, ws_idx, ws_att, hca, update=False),
                                args.steps, args.warmup)
    t_upd, _, _g3 = time_graph(torch, lambda: decode_step(w, layers, shared, ws_idx, ws_att, hca, attend=False),
                               args.steps, args.warmup)
    t_attn /= R
    t_upd /= R
    dom = time_dominant(torch, hca, w, layers, shared)
    copy_gbs = copy_bandwidth(torch)
    alg = sum(layer_bytes(l.kind, w.B, w.L, w.d, w.H, w.window) for l in layers) / R
    upd = sum(update_bytes(l.kind, w.B, w.d) for l in layers) / R
    roofline = None
    if dom is not None:
        kind = [l.kind for l in layers if l.kind.topk is not None][0]
        sb = score_bytes(kind, w.B, w.L)
        achieved = sb / (dom[0] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_of(kind),
                    "frac_of_measured_copy": round(achieved / copy_gbs, 4), "measured_copy_GBps": round(copy_gbs, 1),
                    "kernel": f"score_kernel<{kind.idx_dtype},128> (indexer scoring)", "bytes_per_launch": int(sb),
                    "avg_launch_ms": round(dom[0], 5), "median_of_batches_ms": round(dom[1], 5), "launches": dom[2]}
    cpu = None
    if not args.no_cpu_baseline and n_layers == len(w.layers):
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w)
    value = w.B / (t_step * 1e-3)
    res = {
        "metric": f"decode-attn tokens/sec per GPU ({METRIC_WORKLOAD.get(args.config, w.name)})",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"{w.kv_dtype} KV" + "".join(sorted({f" / {l.kind.idx_dtype} idx" for l in layers if l.kind.idx_dtype}))
                  + ", f16+bf16 MFMA, fp32 acc"),
        "data": ("synthetic (seeded N(0,1) tokens, logits, queries, indexer keys; U(0.5, 1.5) RMSNorm gains; "
                 "random page permutation)"),
        "config": {"workload": w.name, "batch": w.B, "context": w.L, "layers": n_layers,
                   "c4a_layers": sum(1 for l in layers if l.kind.name == "c4a") // R,
                   "c128a_layers": sum(1 for l in layers if l.kind.name == "c128a") // R, "d": w.d, "heads": w.H,
                   "window": w.window, "topk": max([l.kind.topk or 0 for l in layers]) or None,
                   "cache_replicas": R, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "step_breakdown": {
            "algorithmic_bytes_per_step": int(alg),
            "update_bytes_per_step": int(upd),
            "step_GBps_incl_update": round((alg + upd) / (t_step * 1e-3) / 1e9, 1),
            "attn_only_ms": round(t_attn, 4),
            "attn_only_tokens_per_s": round(w.B / (t_attn * 1e-3), 2),
            "attn_only_GBps": round(alg / (t_attn * 1e-3) / 1e9, 1),
            "attn_only_frac_of_peak": round(alg / (t_attn * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "update_only_ms": round(t_upd, 4),
            "wall_s_timed_region": round(wall, 4),
        },
        "prefill": {"ms_all_layers": round(pre["ms"] / R, 3), "bytes": int(pre["bytes"] / R),
                    "GBps": round(pre["bytes"] / (pre["ms"] * 1e-3) / 1e9, 1) if pre["ms"] > 0 else None,
                    "what": "kv_compress + kv_quantize_page over the whole context of every layer"},
        "page_pool": pool_packing(w, hca),
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
