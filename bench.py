"""Decode-step benchmark of the hybrid compressed-KV decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4]

Workload (default): the 1M-token long-context stack -- batch 4, context 2^20,
61 layers (30 c4a: m=4, 262,144 entries, indexer top-2048 over fp4 E2M1 keys
with per-32 E4M3 scales; 31 c128a: m=128, 8,192 entries, all attended), shared
K=V dim 512 in fp8 E4M3 pages with a per-page fp32 scale, 64 query heads, a
128-token raw window.  The caches are filled by a prefill pass on the GPU
(kv_compress + kv_quantize_page over all 2^20 tokens of every layer), timed
and reported on its own.  The default run also times the 128K c4a layer
(batch 16, fp8 indexer keys) and reports it under "at_128k", so that both
context lengths of the metric are in one record.  `--config 3` is the mixed
paged batch (64 sequences of log-uniform lengths, a shared 8-block prefix
aliased in the block tables, one c4a and one c128a layer).

A step is one decode step of the whole stack for the batch: per layer the
decode update (the open group's entry -- c4a: re-folded over its 8-token
window at stride 4; c128a: the newest token folded into the group's running
fold state -- with its RMSNorm and RoPE, and its page, the window insert of the new token and its page, the open indexer page:
one kv_compress_insert_jobs launch), then indexer_topk (c4a) and
paged_hybrid_decode, whose output is delivered as fp8 rows with a per-row
scale; layers stay in order.  The step is captured once in a HIP graph and replayed; `value` is
decode tokens/s = B / step time.

Also reported: each kernel's average duration, measured with HIP events
around batches of back-to-back launches on the stream they run on, with its
algorithmic bytes and the fraction of the 8 TB/s HBM peak; `roofline` is the
kernel with the largest time per step; and the CPU oracle timed on a bounded
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

# HBM bytes per launch of a kernel on the stack's layer shape, from rocprofv3
# FETCH_SIZE and WRITE_SIZE passes, each scaled by what the same counter reads
# for the 1 GiB device copy in copy_bandwidth() (the summaries with the
# commands are in profiles/).  They hold only for the kernel source they were
# taken on, identified by the SHA-256 of the source files; otherwise traffic
# is null.
TRAFFIC = {
    # (workload, layer kind, kernel): sources, their SHA-256, bytes read and written per launch (rocprofv3 FETCH_SIZE and
    # WRITE_SIZE per dispatch, scaled by what the same counters read for the bench's 1 GiB device copy)
    ("stack-1m-b4-61layers", "c4a", "score"): {"sources": ("decode_attention_compressed_amd/csrc/indexer.hip",
                                   "decode_attention_compressed_amd/csrc/hca_common.h",
                                   "decode_attention_compressed_amd/csrc/indexer_internal.h",
                                   "decode_attention_compressed_amd/csrc/indexer_score.h"),
                       "source_sha256": "e15c22d671761d4d76830afa22ad947fd58b595f722bb1a7f0b76f65dd1d4706",
                       "fetch_bytes": 72060575, "write_bytes": 4662247},
    ("stack-1m-b4-61layers", "c128a", "attn_split"): {"sources": ("decode_attention_compressed_amd/csrc/attention.hip",
                                          "decode_attention_compressed_amd/csrc/hca_common.h",
                                          "decode_attention_compressed_amd/csrc/hca_internal.h"),
                              "source_sha256": "89a7dfe9ecfad1bc075885b4bf6d7c36ae379fd66cbc2287bd5114f4f1a922a9",
                              "fetch_bytes": 20030315, "write_bytes": 4259840},
    ("stack-1m-b4-61layers", "c4a", "attn_split"): {"sources": ("decode_attention_compressed_amd/csrc/attention.hip",
                                        "decode_attention_compressed_amd/csrc/hca_common.h",
                                        "decode_attention_compressed_amd/csrc/hca_internal.h"),
                            "source_sha256": "89a7dfe9ecfad1bc075885b4bf6d7c36ae379fd66cbc2287bd5114f4f1a922a9",
                            "fetch_bytes": 7384423, "write_bytes": 3727360},
}


def source_sha256(files):
    import hashlib

    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_of(workload, kind_name, kname):
    """Counted HBM bytes per launch of a kernel, for the workload and layer kind the counters were taken on
    (None for any other shape, or once the kernel's sources have changed)."""
    t = TRAFFIC.get((workload, kind_name, kname))
    if t is None or t["source_sha256"] is None or source_sha256(t["sources"]) != t["source_sha256"]:
        return None
    return int(t["fetch_bytes"] + t["write_bytes"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the 128K point the default run adds")
    ap.add_argument("--layers", type=int, default=0, help="debug only: first N layers (result is not the workload)")
    ap.add_argument("--layer-sample", type=int, default=0,
                    help="profiling only: the first N layers of each kind (result is not the workload)")
    ap.add_argument("--replicas", type=int, default=0,
                    help="copies of a workload's caches, one per timed step in turn, so that one step's pages "
                         "are not still in the Infinity Cache from the step before (0: 4 for workloads of one or "
                         "two layers, 1 otherwise)")
    return ap.parse_args()


# ----------------------------------------------------------------- algorithmic bytes


def _idx_row_bytes(kind, epp, d_idx):
    return d_idx // 2 + d_idx // 32 if kind.idx_dtype == "fp4" else d_idx + 4.0 / epp


def seq_bytes(kind, L, d, H, W, d_idx=128, h_idx=16):
    """Algorithmic HBM bytes of one decode step of one layer for one sequence
    of length L: each stored row read once (codes + its share of scales), the
    queries, outputs and block table entries; intermediate scores, indices and
    partial outputs are not counted."""
    m = kind.m
    N = -(-L // m)
    epp = 256 // m
    win = min(W, L)
    q = H * d * 2
    out = H * d + H * 4 + H * 4  # fp8 output row, its scale, the lse
    win_rows = win * d + 4 * (-(-win // 256) + 1)
    if kind.topk is not None:
        kk = min(kind.topk, N)
        idx = N * _idx_row_bytes(kind, epp, d_idx) + h_idx * d_idx * 2 + h_idx * 4 + 4 * (-(-N // epp))
        rows = kk * (d + 4)  # each selected row and its page scale
        return idx + rows + win_rows + q + out + 4 * kk
    rows = N * d + 4 * (-(-N // epp))
    return rows + win_rows + q + out + 4 * (-(-N // epp))


def layer_bytes(kind, lens, d, H, W):
    return float(sum(seq_bytes(kind, int(L), d, H, W) for L in lens))


def score_bytes(kind, lens, d_idx=128, h_idx=16):
    """What the indexer's score kernel reads: every entry's key (codes + its
    share of scales), the queries, head weights and the page list."""
    tot = 0.0
    for L in lens:
        N = -(-int(L) // kind.m)
        epp = 256 // kind.m
        tot += N * _idx_row_bytes(kind, epp, d_idx) + h_idx * d_idx * 2 + h_idx * 4 + 4 * (-(-N // epp))
    return tot


def attn_bytes(kind, lens, d, H, W):
    """What the attention's split kernel reads: the attended rows (codes + page
    scale), the window rows, the queries, the selection and block table
    entries."""
    tot = 0.0
    for L in lens:
        L = int(L)
        N = -(-L // kind.m)
        epp = 256 // kind.m
        win = min(W, L)
        rows = min(kind.topk, N) if kind.topk is not None else N
        tot += rows * (d + 4) + win * d + 4 * (-(-win // 256) + 1) + H * d * 2 + 4 * rows
    return tot


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


def prefill_bytes(kind, lens, d, d_idx=128):
    """Algorithmic bytes of one layer's prefill pass: the raw bf16 tokens and
    their logits read, the fp8 pages and scales written (the indexer keys'
    pages are a separate input, not counted)."""
    tot = 0.0
    for L in lens:
        L = int(L)
        N = -(-L // kind.m)
        epp = 256 // kind.m
        tot += L * d * 2 + L * 4 + N * d + 4 * (-(-N // epp))
    return tot


# ----------------------------------------------------------------- GPU state


class Layer:
    pass


def build_state(w, n_layers, torch, hca, gen, log, replicas=1):
    """Fill every layer's pools with a GPU prefill pass; keep the decode-update
    state.  Sequences may have different lengths and share prefix pages (the
    mixed batch): the shared blocks are written once, by the first sequence
    that holds them.  With replicas > 1 every layer is built that many times
    over (own pools and inputs: layer index li takes the kind of layer li %
    n_layers).  Returns (layers, shared tensors, prefill stats)."""
    B, d, H, W = w.B, w.d, w.H, w.window
    lens_np = gen.lengths(w)
    Lmax = int(lens_np.max())
    members = [int(b) for b in gen.shared_members(w, lens_np)]
    npre_tok = w.shared_prefix_blocks * 256 if members else 0
    table_np, P, wtable_np, PW = gen.block_tables(w, lens_np)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    table, wtable, lens = dev(table_np), dev(wtable_np), dev(lens_np)
    zeros_b = dev(np.zeros(B, np.int32))
    # sequences whose prefix pages another sequence writes
    rest = members[1:]
    layers = []
    pre_ms, pre_bytes = 0.0, 0.0
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0_np = (np.maximum(0, lens_np - W) // 256) * 256
    nw_np = lens_np - t0_np
    nwmax = int(nw_np.max())
    for li in range(n_layers * replicas):
        kind = w.layers[li % n_layers]
        m, epp = kind.m, 256 // kind.m
        N_np = -(-lens_np // m)
        Nmax = int(N_np.max())
        lay = Layer()
        lay.kind, lay.N, lay.epp = kind, N_np, epp
        # raw tokens and logits of the whole context (seeded device draws); a
        # shared prefix holds the same tokens in every sequence that shares it
        x = torch.empty((B, Lmax, d), dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            x[b] = gen.device_normal((Lmax, d), 1.0, (0, w.cid, li, gen.S_TOK, b), dtype=torch.bfloat16)
        z = gen.device_normal((B, Lmax), 1.0, (0, w.cid, li, gen.S_LOGIT))
        for b in rest:
            x[b, :npre_tok] = x[members[0], :npre_tok]
            z[b, :npre_tok] = z[members[0], :npre_tok]
        o = kind.overlap
        beta = dev(gen.slot_bias(w, li, kind.slots))
        lay.gamma = dev(gen.norm_gain(w, li, d))
        lay.kv = hca.PagedCache.empty(P, epp, d, w.kv_dtype)
        xi = x.view(torch.int16)
        npre_e = npre_tok // m
        # the fused prefill: fold, RMSNorm, RoPE and page write in one launch,
        # no fp32 entries in HBM; the shared prefix's pages are written once,
        # by the first sequence that holds them (the others' runs start after it)
        nt_own = lens_np.copy()
        nt_own[rest] = 0
        nt_rest = np.zeros(B, np.int32)
        nt_rest[rest] = lens_np[rest] - npre_tok
        nt_own_d, nt_rest_d, pre_d = dev(nt_own.astype(np.int32)), dev(nt_rest), dev(np.full(B, npre_tok, np.int32))
        torch.cuda.synchronize()
        ev0.record()
        hca.kv_prefill_pages(xi, z, beta, zeros_b, nt_own_d, m, w.theta, Lmax, table, lay.kv, norm_gamma=lay.gamma,
                             overlap=o)
        if rest:
            hca.kv_prefill_pages(xi[:, npre_tok:], z[:, npre_tok:], beta, pre_d, nt_rest_d, m, w.theta,
                                 Lmax - npre_tok, table, lay.kv, norm_gamma=lay.gamma, overlap=o)
        ev1.record()
        torch.cuda.synchronize()
        pre_ms += ev0.elapsed_time(ev1)
        pre_bytes += prefill_bytes(kind, lens_np, d)
        # decode-update state, per sequence: the ring of the open group's
        # window (the overlap's tokens of the group before, then the open
        # group), the open page's staging (its entries folded again from its
        # tokens, with the overlap's tokens before them)
        g_open = (lens_np - 1) // m
        nt_open = lens_np - g_open * m
        e_open0 = (g_open // epp) * epp
        lay.ring_x = torch.zeros((B, o + m, d), dtype=torch.int16, device="cuda")
        lay.ring_z = torch.zeros((B, o + m), dtype=torch.float32, device="cuda")
        xs = torch.zeros((B, o + 256, d), dtype=torch.int16, device="cuda")
        zs = torch.zeros((B, o + 256), dtype=torch.float32, device="cuda")
        for b in range(B):
            L = int(lens_np[b])
            p_lo = max(0, int(g_open[b]) * m - o)
            r0 = o - (int(g_open[b]) * m - p_lo)
            lay.ring_x[b, r0: o + int(nt_open[b])] = xi[b, p_lo: L]
            lay.ring_z[b, r0: o + int(nt_open[b])] = z[b, p_lo: L]
            t_lo = int(e_open0[b]) * m
            s_lo = max(0, t_lo - o)
            xs[b, o - (t_lo - s_lo): o + L - t_lo] = xi[b, s_lo: L]
            zs[b, o - (t_lo - s_lo): o + L - t_lo] = z[b, s_lo: L]
        lay.stage = torch.zeros((B, epp, d), dtype=torch.float32, device="cuda")
        hca.kv_compress(xs[:, o:], zs[:, o:], beta, dev((e_open0 * m).astype(np.int32)),
                        dev((lens_np - e_open0 * m).astype(np.int32)), m, w.theta, lay.stage, 256,
                        norm_gamma=lay.gamma, overlap=o)
        del xs, zs
        lay.x_open, lay.z_open = lay.ring_x[:, o:], lay.ring_z[:, o:]  # rows -o .. -1: the overlap
        lay.beta = beta
        lay.pos0 = dev((g_open * m).astype(np.int32))
        lay.ntok = dev(nt_open.astype(np.int32))
        lay.e0 = dev(e_open0.astype(np.int32))
        # the entries' update state: the open page's header (the amax of its
        # closed rows) and, for groups of more than 16 tokens, a running fold
        # state, so an update folds only the newest token; that one is brought
        # to the state after the open group's tokens but the newest (what the
        # previous step left) by an update call with one token fewer
        lay.fstate = torch.zeros((B, 4 + (2 * (4 + d) if m > 16 else 0)), dtype=torch.float32, device="cuda")
        if m > 16:
            hca.kv_compress_insert(lay.ring_x[:, o:], lay.ring_z[:, o:], beta, lay.pos0,
                                   dev((nt_open - 1).astype(np.int32)), m, w.theta, lay.stage, lay.e0, table, lay.kv,
                                   append=False, norm_gamma=lay.gamma, overlap=o, fold_state=lay.fstate)
        # window pages: every token of the blocks that overlap [L-W, L)
        xw = torch.zeros((B, nwmax, d), dtype=torch.int16, device="cuda")
        zw = torch.zeros((B, nwmax), dtype=torch.float32, device="cuda")
        for b in range(B):
            xw[b, : int(nw_np[b])] = xi[b, int(t0_np[b]): int(lens_np[b])]
            zw[b, : int(nw_np[b])] = z[b, int(t0_np[b]): int(lens_np[b])]
        wrows = torch.empty((B, nwmax, d), dtype=torch.float32, device="cuda")
        t0_d, nw_d = dev(t0_np.astype(np.int32)), dev(nw_np.astype(np.int32))
        hca.kv_compress(xw, zw, dev(np.zeros(1, np.float32)), t0_d, nw_d, 1, w.theta, wrows, nwmax)
        lay.win = hca.PagedCache.empty(max(1, PW), 256, d, w.kv_dtype)
        hca.kv_quantize_page(wrows, t0_d, nw_d, nwmax, wtable, lay.win)
        tw0 = ((lens_np - 1) // 256) * 256
        lay.wstage = torch.zeros((B, 256, d), dtype=torch.float32, device="cuda")
        lay.x_last = torch.empty((B, 1, d), dtype=torch.int16, device="cuda")
        lay.z_last = torch.empty((B, 1), dtype=torch.float32, device="cuda")
        for b in range(B):
            L = int(lens_np[b])
            lay.wstage[b, : L - int(tw0[b])] = wrows[b, int(tw0[b] - t0_np[b]): int(nw_np[b])]
            lay.x_last[b, 0] = xi[b, L - 1]
            lay.z_last[b, 0] = z[b, L - 1]
        lay.wpos0 = dev((lens_np - 1).astype(np.int32))
        lay.one = dev(np.full(B, 1, np.int32))
        lay.we0 = dev(tw0.astype(np.int32))
        lay.zero1 = dev(np.zeros(1, np.float32))
        del x, z, wrows, xw, zw
        # queries
        lay.q = dev(gen.queries(w, li).view(np.int16))
        if kind.topk is not None:
            keys = gen.device_normal((B, Nmax, kind.d_idx), 1.0, (0, w.cid, li, gen.S_IDXK))
            for b in rest:
                keys[b, :npre_e] = keys[members[0], :npre_e]
            lay.idx = hca.PagedCache.empty(P, epp, kind.d_idx, kind.idx_dtype)
            ne_own = N_np.copy()
            ne_own[rest] = 0
            hca.kv_quantize_page(keys, zeros_b, dev(ne_own.astype(np.int32)), Nmax, table, lay.idx)
            if rest:
                ne_rest = np.zeros(B, np.int32)
                ne_rest[rest] = N_np[rest] - npre_e
                hca.kv_quantize_page(keys[:, npre_e:], dev(np.full(B, npre_e, np.int32)), dev(ne_rest),
                                     Nmax - npre_e, table, lay.idx)
            lay.istage = torch.zeros((B, epp, kind.d_idx), dtype=torch.float32, device="cuda")
            for b in range(B):
                lay.istage[b, : int(N_np[b] - e_open0[b])] = keys[b, int(e_open0[b]): int(N_np[b])]
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
        if li % 10 == 0 or li == n_layers * replicas - 1:
            log(f"prefilled layer {li + 1}/{n_layers * replicas} ({kind.name})")
    shared = dict(table=table, wtable=wtable, lens=lens, lens_np=lens_np, Lmax=Lmax)
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
    W = w.window
    L = shared["Lmax"]
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
            sel, sel_n = (lay.sel, lay.sel_n) if kind.topk is not None else (None, None)
            hca.paged_hybrid_decode(lay.q, lay.kv, table, lay.win, wtable, lens, L, m, W, sel, sel_n, scale, w.theta,
                                    None, lay.lse, ws_att[kind.name], out_fp8=lay.out8, out_scale=lay.out8s)


def time_graph(torch, fn, steps, warmup, per_step=False):
    """Median-free mean over `steps` replays of the captured step (one event
    pair around them all); with per_step, also each replay's own duration
    (an event pair per replay) for percentiles."""
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
    each = None
    if per_step:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in evs:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        each = [a.elapsed_time(b) for a, b in evs]
    return e0.elapsed_time(e1) / steps, wall, g, each


def time_eager(torch, fn, steps):
    """The step without a graph: launches issued from Python as they come."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_launches(torch, launch, items, reps=4, rounds=3):
    """Average duration of one launch of a kernel on the stream it runs on: a
    GPU sleep lets every launch queue first, then one event pair brackets
    reps x len(items) back-to-back launches (one per layer's own data, so
    consecutive launches do not re-read each other's bytes).  Returns
    (mean over rounds, median over rounds, launches timed)."""
    if not items:
        return None
    stream = torch.cuda.current_stream()
    res = []
    for _ in range(rounds):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(50_000_000)
        e0.record(stream)
        for _ in range(reps):
            for it in items:
                launch(it)
        e1.record(stream)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / (reps * len(items)))
    return float(np.mean(res)), float(np.median(res)), reps * len(items) * rounds


def kernel_table(torch, hca, w, layers, shared, ws_att, R):
    """Per-kernel durations of a step's launches, per layer kind: the indexer's
    score kernel, the whole indexer call (score + select), the attention's
    split kernel and the whole attention call (split + combine).  Each entry:
    average us per launch, launches per step, us per step, algorithmic bytes
    per launch, GB/s and the fraction of the HBM peak."""
    lens_np, L = shared["lens_np"], shared["Lmax"]
    table, wtable, lens = shared["table"], shared["wtable"], shared["lens"]
    scale = 1.0 / math.sqrt(w.d)
    out = {}
    kinds = {}
    for lay in layers:
        kinds.setdefault(lay.kind.name, []).append(lay)
    for name, lays in kinds.items():
        kind = lays[0].kind
        n_step = len(lays) / R  # launches of this kind per step
        ws_split = hca.workspace(hca.paged_hybrid_decode_workspace(w.B, w.H, w.d, L, kind.m, w.window, kind.topk or 0))

        def split(lay, ws=ws_split):
            sel, sel_n = (lay.sel, lay.sel_n) if kind.topk is not None else (None, None)
            hca.attention_split(lay.q, lay.kv, table, lay.win, wtable, lens, L, kind.m, w.window, sel, sel_n, scale,
                                w.theta, ws)

        def attn(lay):
            sel, sel_n = (lay.sel, lay.sel_n) if kind.topk is not None else (None, None)
            hca.paged_hybrid_decode(lay.q, lay.kv, table, lay.win, wtable, lens, L, kind.m, w.window, sel, sel_n,
                                    scale, w.theta, None, lay.lse, ws_att[name], out_fp8=lay.out8,
                                    out_scale=lay.out8s)

        entries = [("attn_split", split, attn_bytes(kind, lens_np, w.d, w.H, w.window)),
                   ("attention (split + combine)", attn, layer_bytes(kind, lens_np, w.d, w.H, w.window)
                    - (score_bytes(kind, lens_np) if kind.topk is not None else 0.0))]
        if kind.topk is not None:
            ws_s = hca.workspace(hca.indexer_topk_workspace(w.B, L, kind.m, kind.topk))
            ws_i = hca.workspace(hca.indexer_topk_workspace(w.B, L, kind.m, kind.topk))

            def score(lay, ws=ws_s):
                hca.indexer_score(lay.qi, lay.wi, lay.idx, table, lens, L, kind.m, kind.topk, ws)

            def topk(lay, ws=ws_i):
                hca.indexer_topk(lay.qi, lay.wi, lay.idx, table, lens, L, kind.m, kind.topk, lay.sel, lay.sel_n, ws)

            entries = [("score", score, score_bytes(kind, lens_np)),
                       ("indexer (score + select)", topk, score_bytes(kind, lens_np))] + entries
        for kname, fn, nbytes in entries:
            t = time_launches(torch, fn, lays)
            avg_ms = t[0]
            gbs = nbytes / (avg_ms * 1e-3) / 1e9
            out[f"{name}:{kname}"] = {"avg_us": round(avg_ms * 1e3, 2), "median_of_rounds_us": round(t[1] * 1e3, 2),
                                      "launches_timed": t[2], "per_step": n_step,
                                      "us_per_step": round(avg_ms * 1e3 * n_step, 1),
                                      "bytes_per_launch": int(nbytes), "GBps": round(gbs, 1),
                                      "frac": round(gbs / HBM_PEAK_GBS, 4)}
        if kind.topk is not None:
            sc, ix = out[f"{name}:score"], out[f"{name}:indexer (score + select)"]
            out[f"{name}:select (indexer - score)"] = {"us_per_launch": round(ix["avg_us"] - sc["avg_us"], 2),
                                                       "per_step": n_step}
        sp, at = out[f"{name}:attn_split"], out[f"{name}:attention (split + combine)"]
        out[f"{name}:combine (attention - split)"] = {"us_per_launch": round(at["avg_us"] - sp["avg_us"], 2),
                                                      "per_step": n_step}
    return out


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
    + fp8 output) for one sequence of each layer kind, on page contents of the
    workload's shape (random codes: the oracle's time does not depend on the
    values); repeated while within budget; scaled to the workload's layers.
    For a batch of mixed lengths, a fixed sample of its sequences is timed per
    kind and their mean scaled to the batch."""
    from oracle import attention, indexer, paging
    from synth import gen

    rng = np.random.default_rng(0)
    d, H, W = w.d, w.H, w.window
    lens = gen.lengths(w)
    sample = sorted(set(np.linspace(0, w.B - 1, min(4, w.B)).astype(int).tolist())) if w.L is None else [0]
    kinds = {}
    for k in w.layers:
        kinds.setdefault(k.name, k)
    t_layer = {}
    reps = {}
    t_start = time.perf_counter()
    for name, kind in kinds.items():
        m, epp = kind.m, 256 // kind.m
        per_seq = []
        for b in sample:
            L = int(lens[b])
            N = -(-L // m)
            P = -(-L // 256)
            table = rng.permutation(P)
            kv = paging.Pool("fp8", P, epp, d)
            kv.codes[:] = rng.integers(0, 0x7E, kv.codes.shape, dtype=np.uint8)
            kv.scales[:] = rng.uniform(1e-3, 1e-2, P).astype(np.float32)
            win = paging.Pool("fp8", 2, 256, d)
            win.codes[:] = rng.integers(0, 0x7E, win.codes.shape, dtype=np.uint8)
            wtable = np.full(P, -1)
            wtable[(L - 1) // 256] = 0
            if L > W and (L - W) // 256 != (L - 1) // 256:
                wtable[(L - W) // 256] = 1
            q = rng.standard_normal((H, d))
            if kind.topk is not None:
                idx = paging.Pool(kind.idx_dtype, P, epp, kind.d_idx)
                idx.codes[:] = rng.integers(0, 256, idx.codes.shape, dtype=np.uint8)
                if kind.idx_dtype == "fp4":
                    idx.scales[:] = rng.integers(0x20, 0x40, idx.scales.shape, dtype=np.uint8)
                qi, wi = rng.standard_normal((kind.h_idx, kind.d_idx)), rng.standard_normal(kind.h_idx)
            times = []
            while True:
                t0 = time.perf_counter()
                if kind.topk is not None:
                    keys = paging.decode_rows(idx, table, np.arange(N))
                    sc = indexer.scores(qi, wi, keys)
                    sel = indexer.topk(sc, kind.topk)
                else:
                    sel = np.arange(N)
                rows = paging.decode_rows(kv, table, sel)
                rows = np.concatenate([rows, paging.decode_rows(win, wtable, attention.window_positions(L, W))])
                o, _, _ = attention.attend(q, rows, L, 1.0 / math.sqrt(d), w.theta)
                attention.quantize_out_fp8(o)
                times.append(time.perf_counter() - t0)
                if sum(times) > budget_s / len(kinds) / len(sample) or len(times) >= 200:
                    break
            per_seq.append(float(np.median(times)))
            reps[name] = reps.get(name, 0) + len(times)
        t_layer[name] = float(np.mean(per_seq))
    n_kind = {name: sum(1 for k in w.layers if k.name == name) for name in kinds}
    t_seq_step = sum(t_layer[nm] * n_kind[nm] for nm in kinds)  # one sequence through every layer
    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    what = (f"one sequence at L={w.L}" if w.L is not None else
            f"sequences {sample} of the batch (L = {[int(lens[b]) for b in sample]}), their mean scaled to the batch")
    return {
        "value": 1.0 / t_seq_step,  # sequences are independent: batch tokens/s = per-sequence tokens/s
        "unit": "tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle decode step (indexer scores + top-k + row gather/decode + attention + fp8 "
                   f"output) of {what}, per layer kind "
                   + ", ".join(f"{nm}: {reps[nm]} runs, {t_layer[nm]:.3f} s" for nm in kinds)
                   + f"; scaled by the workload's {n_kind} layers; wall {time.perf_counter() - t_start:.1f} s"),
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


# ----------------------------------------------------------------- page-pool packing


def pool_packing(w, hca):
    """The workload's KV kinds packed into size buckets of one arena (host
    bookkeeping only): buckets, arena bytes, and the host time to give every
    sequence of every layer its pages (one allocation per layer, kind and
    sequence), then release them."""
    from synth import gen

    lens = gen.lengths(w)
    kinds, count = [], []
    for k in w.layers:
        main = (k.m, w.d, w.kv_dtype)
        if main not in kinds:
            kinds.append(main)
            count.append([0] * w.B)
        if k.topk is not None:
            ik = (k.m, k.d_idx, k.idx_dtype)
            if ik not in kinds:
                kinds.append(ik)
                count.append([0] * w.B)
        for b in range(w.B):
            nb = -(-int(lens[b]) // 256)
            count[kinds.index(main)][b] += nb
            if k.topk is not None:
                count[kinds.index(ik)][b] += nb
    kinds.append((1, w.d, w.kv_dtype))
    count.append([2 * len(w.layers)] * w.B)  # the blocks that overlap the window
    probe = hca.PagePool(kinds, [1] * len(kinds))
    cap = [0] * probe.n_buckets
    for i, c in enumerate(count):
        cap[probe.bucket_of(i)] += sum(c)
    pool = hca.PagePool(kinds, cap)
    t0 = time.perf_counter()
    held = []
    for b in range(w.B):
        for i, c in enumerate(count):
            bk = pool.bucket_of(i)
            held.append((bk, pool.alloc(bk, c[b])))
    t1 = time.perf_counter()
    for bk, pages in held:
        pool.release(bk, pages)
    t2 = time.perf_counter()
    pages = sum(len(p) for _, p in held)
    return {"kinds": [f"m={m} d={d} {t}" for m, d, t in kinds], "buckets": probe.n_buckets,
            "arena_GiB": round(pool.arena_bytes / 2 ** 30, 3),
            "arena_GiB_per_sequence": round(pool.arena_bytes / 2 ** 30 / w.B, 3),
            "pages": pages, "alloc_ms": round((t1 - t0) * 1e3, 3), "release_ms": round((t2 - t1) * 1e3, 3)}


# ----------------------------------------------------------------- main


METRIC_WORKLOAD = {4: "1M-token 61-layer stack", 2: "128K-token c4a layer, batch 16",
                   1: "64K-token c128a layer, batch 8", 0: "4K-token c4a layer, batch 1",
                   3: "mixed paged batch of 64, c4a + c128a"}


def run_workload(args, cid, torch, hca, synth, gen, log, n_layers_arg=0, steps=None, per_kernel=True,
                 layer_sample=0):
    """Build one workload's caches, time its decode step (graph, per replay,
    eager, attend-only, update-only) and its kernels; returns a dict."""
    w = synth.workload(cid)
    if layer_sample > 0:
        import dataclasses

        picked = []
        for name in ("c4a", "c128a"):
            picked += [k for k in w.layers if k.name == name][:layer_sample]
        w = dataclasses.replace(w, layers=picked)
    steps = steps or args.steps
    n_layers = len(w.layers) if n_layers_arg <= 0 else min(n_layers_arg, len(w.layers))
    R = args.replicas if args.replicas > 0 else (4 if n_layers <= 2 else 1)
    log(f"workload {w.name}: B={w.B} L={w.L if w.L else 'mixed'} layers={n_layers} replicas={R}")
    layers, shared, pre = build_state(w, n_layers, torch, hca, gen, log, replicas=R)
    Lmax = shared["Lmax"]
    lens_np = shared["lens_np"]
    # workspaces (one per kind; the indexer one must start zeroed and is left zeroed)
    kinds = {l.kind.name: l.kind for l in layers}
    ws_idx = None
    ws_att = {}
    for name, kind in kinds.items():
        if kind.topk is not None:
            ws_idx = hca.workspace(hca.indexer_topk_workspace(w.B, Lmax, kind.m, kind.topk))
        ws_att[name] = hca.workspace(hca.paged_hybrid_decode_workspace(w.B, w.H, w.d, Lmax, kind.m, w.window,
                                                                       kind.topk or 0))
    torch.cuda.synchronize()
    log("capturing decode step")
    step = lambda: decode_step(w, layers, shared, ws_idx, ws_att, hca)
    t_step, wall, _g, each = time_graph(torch, step, steps, args.warmup, per_step=True)
    t_step /= R
    each = [e / R for e in each]
    log(f"step {t_step:.4f} ms")
    t_eager = time_eager(torch, step, max(2, steps // 4)) / R
    t_attn, _, _g2, _ = time_graph(torch, lambda: decode_step(w, layers, shared, ws_idx, ws_att, hca, update=False),
                                   steps, args.warmup)
    t_upd, _, _g3, _ = time_graph(torch, lambda: decode_step(w, layers, shared, ws_idx, ws_att, hca, attend=False),
                                  steps, args.warmup)
    del _g, _g2, _g3
    t_attn /= R
    t_upd /= R
    kt = kernel_table(torch, hca, w, layers, shared, ws_att, R) if per_kernel else {}
    alg = sum(layer_bytes(l.kind, lens_np, w.d, w.H, w.window) for l in layers) / R
    upd = sum(update_bytes(l.kind, w.B, w.d) for l in layers) / R
    pre_alg = pre["bytes"] / R
    out = dict(w=w, n_layers=n_layers, R=R, t_step=t_step, wall=wall, each=each, t_eager=t_eager, t_attn=t_attn,
               t_upd=t_upd, kernels=kt, alg=alg, upd=upd, lens=lens_np,
               prefill={"ms_all_layers": round(pre["ms"] / R, 3), "algorithmic_bytes": int(pre_alg),
                        "GBps": round(pre_alg / (pre["ms"] / R * 1e-3) / 1e9, 1) if pre["ms"] > 0 else None,
                        "frac": round(pre_alg / (pre["ms"] / R * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if pre["ms"] > 0
                        else None,
                        "what": ("kv_prefill_pages (fold + RMSNorm + RoPE + fp8 page write fused, no fp32 entries "
                                 "in HBM) over the whole context of every layer; algorithmic bytes = bf16 tokens + "
                                 "logits read, fp8 pages + scales written")})
    del layers, ws_att, ws_idx
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def dominant(kt):
    """The kernel with the largest time per step among the single-kernel
    entries (the score kernel and the attention split kernel of each kind)."""
    best = None
    for k, v in kt.items():
        if not (k.endswith(":score") or k.endswith(":attn_split")):
            continue
        if best is None or v["us_per_step"] > kt[best]["us_per_step"]:
            best = k
    return best


KERNEL_NAMES = {"attn_split": "attn_pair_kernel (attention split: fp8 rows of 512 dims, 16 heads per workgroup)",
                "score": "score_pages_kernel (indexer scoring)"}


def summary(r):
    """The per-workload part of the bench line."""
    w, R = r["w"], r["R"]
    each = np.array(r["each"])
    return {
        "ms_per_step": round(r["t_step"], 4),
        "tokens_per_s": round(w.B / (r["t_step"] * 1e-3), 2),
        "step_p10_ms": round(float(np.percentile(each, 10)), 4),
        "step_p50_ms": round(float(np.percentile(each, 50)), 4),
        "step_p90_ms": round(float(np.percentile(each, 90)), 4),
        "eager_ms_per_step": round(r["t_eager"], 4),
        "algorithmic_bytes_per_step": int(r["alg"]),
        "update_bytes_per_step": int(r["upd"]),
        "step_GBps_incl_update": round((r["alg"] + r["upd"]) / (r["t_step"] * 1e-3) / 1e9, 1),
        "step_frac_of_peak_incl_update": round((r["alg"] + r["upd"]) / (r["t_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "attn_only_ms": round(r["t_attn"], 4),
        "attn_only_tokens_per_s": round(w.B / (r["t_attn"] * 1e-3), 2),
        "attn_only_GBps": round(r["alg"] / (r["t_attn"] * 1e-3) / 1e9, 1),
        "attn_only_frac_of_peak": round(r["alg"] / (r["t_attn"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "update_only_ms": round(r["t_upd"], 4),
        "wall_s_timed_region": round(r["wall"], 4),
        "cache_replicas": R,
    }


def roofline_of(r, copy_gbs):
    kt = r["kernels"]
    dk = dominant(kt)
    if dk is None:
        return None
    v = kt[dk]
    kind_name, kname = dk.split(":")
    achieved = v["GBps"]
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_of(r["w"].name, kind_name, kname),
            "frac_of_measured_copy": round(achieved / copy_gbs, 4), "measured_copy_GBps": round(copy_gbs, 1),
            "kernel": f"{KERNEL_NAMES[kname]}, {kind_name} layers", "bytes_per_launch": v["bytes_per_launch"],
            "avg_launch_ms": round(v["avg_us"] * 1e-3, 5), "median_of_rounds_ms": round(v["median_of_rounds_us"] * 1e-3, 5),
            "launches": v["launches_timed"], "us_per_step": v["us_per_step"]}


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
    copy_gbs = copy_bandwidth(torch)
    r = run_workload(args, args.config, torch, hca, synth, gen, log, n_layers_arg=args.layers,
                     layer_sample=args.layer_sample)
    w = r["w"]
    extra = None
    if args.config == 4 and args.layers <= 0 and args.layer_sample <= 0 and not args.no_extra:
        # the 128K point of the metric: the c4a layer of batch 16, 4 cache replicas
        r2 = run_workload(args, 2, torch, hca, synth, gen, log)
        extra = dict(workload=r2["w"].name, **summary(r2), roofline=roofline_of(r2, copy_gbs), kernels=r2["kernels"])
    cpu = None
    if not args.no_cpu_baseline and r["n_layers"] == len(w.layers) and args.layer_sample <= 0:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w)
        cpu["cpu_model"] = cpu_model()
        # the two small workloads once more with one BLAS / NumPy thread
        from threadpoolctl import threadpool_limits

        one = {}
        with threadpool_limits(limits=1):
            for cid in (0, 1):
                w1 = synth.workload(cid)
                one[w1.name] = cpu_baseline(w1, budget_s=8.0)
        cpu["one_thread"] = one
    value = w.B / (r["t_step"] * 1e-3)
    lens = r["lens"]
    res = {
        "metric": f"decode-attn tokens/sec per GPU ({METRIC_WORKLOAD.get(args.config, w.name)})",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["t_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"{w.kv_dtype} KV" + "".join(sorted({f" / {k.idx_dtype} idx" for k in w.layers if k.idx_dtype}))
                  + ", f16+bf16 MFMA, fp32 acc"),
        "data": ("synthetic (seeded N(0,1) tokens, logits, queries, indexer keys; U(0.5, 1.5) RMSNorm gains; "
                 "random page permutation" + ("; log-uniform lengths, 16 sequences alias an 8-block prefix"
                                              if w.L is None else "") + ")"),
        "config": {"workload": w.name, "batch": w.B,
                   "context": w.L if w.L is not None else {"min": int(lens.min()), "max": int(lens.max()),
                                                            "mean": round(float(lens.mean()), 1)},
                   "layers": r["n_layers"],
                   "c4a_layers": sum(1 for k in w.layers[: r["n_layers"]] if k.name == "c4a"),
                   "c128a_layers": sum(1 for k in w.layers[: r["n_layers"]] if k.name == "c128a"), "d": w.d,
                   "heads": w.H, "window": w.window, "topk": max([k.topk or 0 for k in w.layers]) or None,
                   "cache_replicas": r["R"], "parallelism": "single GPU"},
        "roofline": roofline_of(r, copy_gbs),
        "cpu_baseline": cpu,
        "step_breakdown": summary(r),
        "kernels": r["kernels"],
        "at_128k": extra,
        "prefill": r["prefill"],
        "page_pool": pool_packing(w, hca),
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
