"""GPU parity of vq_decode_pass: every stage's output against the oracle's linear map of
the GPU's own stage input (the per-stage tolerance 1e-3 * sum|w x|), and every stage input
against the oracle's glue of the previous GPU output (within one fp16 ulp)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_guard, check_rows, guarded_buffer, need_gpu, say, upload_model

pytestmark = pytest.mark.gpu


def _stage_mats(shape, fmt, seed, stage, rows_pick=None):
    """Host copy of stage s's (fused) weight matrix, optionally only some rows."""
    L = shape.n_layers
    if stage == 4 * L:
        parts = [(L, synth.MAT_LM_HEAD)]
    else:
        l, j = divmod(stage, 4)
        parts = [[(l, synth.MAT_Q), (l, synth.MAT_K), (l, synth.MAT_V)], [(l, synth.MAT_O)],
                 [(l, synth.MAT_GATE), (l, synth.MAT_UP)], [(l, synth.MAT_DOWN)]][j]
    mats = []
    for (l, mid) in parts:
        r, c = shape.mat_shape(mid)
        mats.append(synth.weight_matrix(fmt, seed, l, mid, r, c, threads=16))
    qs = np.concatenate([m.qs for m in mats])
    sc = np.concatenate([m.scales for m in mats])
    mn = None if mats[0].mins is None else np.concatenate([m.mins for m in mats])
    if rows_pick is not None:
        qs, sc = qs[rows_pick], sc[rows_pick]
        mn = None if mn is None else mn[rows_pick]
    return synth.Q4Matrix(fmt, qs.shape[0], mats[0].cols, qs, sc, mn)


def _stage_io(model, shape, K, ws, logits, stage):
    import torch
    import speculative_decoding_verification_bit_amd as vq
    L, H, KV, FF = shape.n_layers, shape.hidden, shape.kv_dim, shape.ffn
    if stage == 4 * L:
        rows, cols = shape.vocab, H
    else:
        rows, cols = [(H + 2 * KV, H), (H, H), (2 * FF, H), (H, FF)][stage % 4]
    a, b = model.stage_ptrs(K, ws, stage)
    xin = vq.stage_tensor(ws, a, (K, cols), torch.float16).cpu().numpy()
    out = logits.cpu().numpy() if b is None else vq.stage_tensor(ws, b, (K, rows), torch.float32).cpu().numpy()
    return xin, out


def _expected_input(shape, stage, prev_out):
    """The oracle's glue applied to the previous stage's GPU output (double)."""
    H, FF = shape.hidden, shape.ffn
    j = stage % 4 if stage < 4 * shape.n_layers else 0
    if j == 1:                                   # rho(q part of q|k|v)
        return oracle.rho(prev_out[:, :H])
    if j == 3:                                   # rho(silu(gate) * up)
        K = prev_out.shape[0]
        s = np.stack([oracle.silu_mul(prev_out[k, :FF], prev_out[k, FF:]) for k in range(K)])
        return oracle.rho(s)
    return oracle.rho(prev_out)                  # rho(o), rho(down)


def _check_glue(xin, expect, what):
    e16 = expect.astype(np.float16)
    diff = np.abs(xin.astype(np.float64) - e16.astype(np.float64))
    ulp = np.spacing(np.abs(e16)).astype(np.float64)
    bad = diff > ulp
    say(f"{what}: glue inputs off the rounded oracle value: {int((diff > 0).sum())} "
        f"(one ulp), beyond one ulp: {int(bad.sum())}")
    assert not bad.any()


def _every_stage(shape, seed, fmt, K, path):
    """One pass over the stack; every row of every stage checked against the oracle, the
    workspace and the logits guarded against writes past their ends."""
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    model = upload_model(shape, fmt, seed)
    x0 = synth.activations(seed, K, shape.hidden)
    nws = model.workspace_bytes(K)
    ws, ws_whole = guarded_buffer(nws)
    nlg = K * shape.vocab * 4
    lg, lg_whole = guarded_buffer(nlg)
    logits = lg.view(torch.float32).view(K, shape.vocab)
    say(f"every stage: {shape} fmt {fmt} K {K} path {path}")
    vq.decode_pass(model, torch.from_numpy(x0).cuda(), logits, path=path, ws=ws)
    torch.cuda.synchronize()
    check_guard(ws_whole, nws, "decode workspace")
    check_guard(lg_whole, nlg, "logits")
    assert model.barrier_error(K, ws) == 0
    prev = None
    for s in range(4 * shape.n_layers + 1):
        xin, out = _stage_io(model, shape, K, ws, logits, s)
        if s == 0:
            assert np.array_equal(xin.view(np.uint16), x0.view(np.uint16))
        else:
            _check_glue(xin, _expected_input(shape, s, prev), f"stage {s}")
        W = _stage_mats(shape, fmt, seed, s)
        y_ref, a_ref = oracle.linear(W, xin, threads=8)
        check_rows(out, y_ref, a_ref, f"fmt {fmt} K {K} path {path} stage {s}")
        prev = out
    assert np.isfinite(logits.cpu().numpy()).all()


LAUNCHES = [4, 8]          # staged, persistent


@pytest.mark.parametrize("launch", LAUNCHES)
@pytest.mark.parametrize("fmt", [synth.FMT_Q4_MIN, synth.FMT_Q4, synth.FMT_MXFP4])
@pytest.mark.parametrize("K,path", [(1, 1), (2, 1), (3, 1), (4, 1), (8, 1), (4, 2), (16, 2), (1, 3), (4, 3)])
def test_mini_model_every_stage(fmt, K, path, launch):
    """A 2-layer stack (hidden 256, kv 64, ffn 512, vocab 1000): all rows of all stages."""
    if path == 3 and launch == 8:
        pytest.skip("the persistent launch rejects the row-strip kernel: run inside the cooperative "
                    "pass kernel it made an illegal memory access at K = 4 whose cause was not found, "
                    "so that combination is switched off (VQ_ERR_UNSUPPORTED, checked in test_abi)")
    _every_stage(synth.SHAPE_MINI, 4, fmt, K, path | launch)


# Two layers whose stages split into several 1024-column chunks (split-K partials, tile
# arrival counters), small enough for every row of every stage to be checked.
SHAPE_MID = synth.ModelShape(n_layers=2, hidden=2048, kv_dim=256, ffn=5120, vocab=4000)


@pytest.mark.parametrize("launch", LAUNCHES)
@pytest.mark.parametrize("K,path", [(1, 0), (2, 1), (3, 0), (4, 1), (8, 1), (8, 2), (16, 2), (2, 3)])
def test_mid_model_every_stage_split_k(K, path, launch):
    """hidden 2048, kv 256, ffn 5120, vocab 4000: 2 and 5 column chunks per row."""
    if path == 3 and launch == 8:
        pytest.skip("the persistent launch does not run the row-strip kernel")
    _every_stage(SHAPE_MID, 9, synth.FMT_Q4_MIN, K, path | launch)


STREAM_OFF = ("the stream launch is switched off: its first GPU run (mini stack, K = 1, Q4 with mins) "
              "made a memory fault whose cause is not found; host emulation of its addressing finds "
              "every access in bounds")


@pytest.mark.parametrize("fmt", [synth.FMT_Q4_MIN, synth.FMT_Q4, synth.FMT_MXFP4])
@pytest.mark.parametrize("K", [1, 2])
def test_stream_every_stage(fmt, K):
    """The stream launch on the 2-layer mini stack and on the split-K one (hidden 2048,
    ffn 5120): every row of every stage against the oracle."""
    pytest.skip(STREAM_OFF)
    import speculative_decoding_verification_bit_amd as vq
    _every_stage(synth.SHAPE_MINI, 4, fmt, K, vq.LAUNCH_STREAM)
    _every_stage(SHAPE_MID, 9, fmt, K, vq.LAUNCH_STREAM)


def test_stream_reproducible_and_close_to_staged():
    """Two stream passes give identical bits; staged and stream logits agree to rounding."""
    pytest.skip(STREAM_OFF)
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    shape, seed, K = SHAPE_MID, 11, 1
    model = upload_model(shape, synth.FMT_Q4_MIN, seed)
    x0 = torch.from_numpy(synth.activations(seed, K, shape.hidden)).cuda()
    a, _ = vq.decode_pass(model, x0, path=vq.LAUNCH_STREAM)
    b, _ = vq.decode_pass(model, x0, path=vq.LAUNCH_STREAM)
    c, _ = vq.decode_pass(model, x0, path=vq.LAUNCH_STAGED)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    rel = float((a - c).abs().max() / c.abs().max())
    say(f"stream vs staged logits: max |diff| / max |logit| = {rel:.2e}")
    assert rel < 1e-3


def test_27b_stack_stream_sampled_rows():
    """The 27B-class stack through the stream launch, sampled rows against the oracle."""
    pytest.skip(STREAM_OFF)


@pytest.mark.parametrize("fmt,runs", [(synth.FMT_Q4_MIN, ((1, 0), (4, 0), (8, 0), (1, 3))),
                                      (synth.FMT_MXFP4, ((16, 0),))])
def test_27b_stack_sampled_rows(fmt, runs):
    """The full 27B-class stack (64 layers, 5120 / 1024 / 17408, vocab 151936) in one pass;
    stages of layers 0, 31, 63 and the lm_head checked on 24 sampled rows each, every
    checked stage's input against the glue of the previous output."""
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    shape, seed = synth.SHAPE_27B, 0
    model = upload_model(shape, fmt, seed)
    say(f"27B stack fmt {fmt} uploaded: {model.nbytes / 1e9:.3f} GB")
    L = shape.n_layers
    stages = [0, 1, 2, 3, 4 * 31, 4 * 31 + 1, 4 * 31 + 2, 4 * 31 + 3, 4 * 63 + 3, 4 * L]
    rng = np.random.default_rng(1)
    picks, mats = {}, {}
    for s in stages:
        full = _stage_mats(shape, fmt, seed, s)
        pick = np.unique(np.concatenate([rng.integers(0, full.rows, 22), [0, full.rows - 1]]))
        picks[s] = pick
        mats[s] = synth.Q4Matrix(fmt, len(pick), full.cols, full.qs[pick], full.scales[pick],
                                 None if full.mins is None else full.mins[pick])
        del full
    runs_ws = []
    for K, path in runs:
        x0 = synth.activations(seed, K, shape.hidden)
        nws = model.workspace_bytes(K)
        ws, ws_whole = guarded_buffer(nws)
        logits, _ = vq.decode_pass(model, torch.from_numpy(x0).cuda(), path=path, ws=ws)
        torch.cuda.synchronize()
        check_guard(ws_whole, nws, f"K {K} path {path}: decode workspace")
        if path not in (vq.PATH_ROWS, vq.LAUNCH_STREAM):   # persistent: tile kernels, same sums
            # the other launch mode computes the same sums in the same order: identical bits
            other = vq.LAUNCH_PERSISTENT | path
            ws_st, st_whole = guarded_buffer(nws)
            logits_st, _ = vq.decode_pass(model, torch.from_numpy(x0).cuda(), path=other, ws=ws_st)
            torch.cuda.synchronize()
            check_guard(st_whole, nws, f"K {K} path {other}: decode workspace")
            assert model.barrier_error(K, ws_st) == 0
            assert model.barrier_error(K, ws) == 0
            if K < 4:
                # VALU tile kernel in both modes: the same sums in the same order
                assert torch.equal(logits, logits_st), f"K {K}: staged and persistent logits differ"
                for s in stages:
                    assert all(np.array_equal(u.view(np.uint8), v.view(np.uint8)) for u, v in
                               zip(_stage_io(model, shape, K, ws, logits, s),
                                   _stage_io(model, shape, K, ws_st, logits_st, s)))
            else:
                # MFMA: the staged launches convert each stage's input once, in workgroups
                # of their own; their per-column input scales have been seen to differ from
                # the persistent pass's by a few fp32 ulps, which flips an occasional fp16
                # input and then grows along the 257-stage chain.  Each mode is checked
                # stage by stage against the oracle instead.
                runs_ws.append((ws_st, logits_st, "persistent"))
            del st_whole
        for w_, l_, nm in [(ws, logits, "staged")] + runs_ws:
            for s in stages:
                xin, out = _stage_io(model, shape, K, w_, l_, s)
                if s > 0:
                    _, prev = _stage_io(model, shape, K, w_, l_, s - 1)
                    _check_glue(xin, _expected_input(shape, s, prev), f"K {K} {nm} stage {s}")
                y_ref, a_ref = oracle.linear(mats[s], xin, threads=8)
                check_rows(out[:, picks[s]], y_ref, a_ref, f"27B fmt {fmt} K {K} path {path} {nm} stage {s}")
        runs_ws = []
        del ws, ws_whole, logits
        torch.cuda.empty_cache()


def test_graph_replay_matches_eager():
    """A captured HIP graph of decode_pass + verify_accept, replayed several times with eager
    work in between, reproduces the eager result bitwise on every replay."""
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    shape, seed, K = synth.SHAPE_MINI, 6, 4
    model = upload_model(shape, synth.FMT_Q4_MIN, seed)
    V = shape.vocab
    x0 = torch.from_numpy(synth.activations(seed, K, shape.hidden)).cuda()
    logits = torch.empty((K, V), dtype=torch.float32, device="cuda")
    ws = torch.empty(model.workspace_bytes(K), dtype=torch.uint8, device="cuda")
    t = logits.view(1, K, V)
    d = torch.from_numpy(synth.window_logits(synth.LogitSpec(seed, K, V, 2.0, 0.5), 0)[1][None]).cuda()
    kw = dict(draft_mode=vq.DRAFT_Q_SAMPLE, T=0.8, top_p=0.9, min_p=0.02, seed=3)
    out = vq.verify_accept(vq.MODE_SAMPLE, t, d, **kw)
    aws = torch.empty(vq.workspace_bytes(vq.OP_ACCEPT, vq.accept_desc(1, t, d, out["draft_tokens"]), K),
                      dtype=torch.uint8, device="cuda")

    def step():
        vq.decode_pass(model, x0, logits, ws=ws)
        vq.verify_accept(vq.MODE_SAMPLE, t, d, draft_tokens=out["draft_tokens"], ws=aws, out=out, **kw)

    step()
    torch.cuda.synchronize()
    ref_logits = logits.clone()
    ref_tokens = out["tokens"].clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        logits.fill_(float("nan"))
        out["tokens"].fill_(-7)
        scratch = torch.randn(1 << 20, device="cuda") * 3      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(logits, ref_logits), f"replay {rep}: logits differ"
        assert torch.equal(out["tokens"], ref_tokens), f"replay {rep}: tokens differ"
        del scratch


@pytest.mark.parametrize("launch", LAUNCHES)
def test_workspace_reuse_with_new_inputs(launch):
    """A pass over a workspace that still holds another input's pass gives the same bits
    as a pass in the same launch mode over a fresh workspace: nothing stale is read back
    from the previous pass."""
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    shape, seed, K = synth.SHAPE_MINI, 7, 4
    model = upload_model(shape, synth.FMT_Q4_MIN, seed)
    xa = torch.from_numpy(synth.activations(seed, K, shape.hidden)).cuda()
    xb = torch.from_numpy(synth.activations(seed + 1, K, shape.hidden)).cuda()
    logits, ws = vq.decode_pass(model, xa, path=launch)
    for _ in range(3):
        vq.decode_pass(model, xb, logits, path=launch, ws=ws)
        torch.cuda.synchronize()
        ref, ws_ref = vq.decode_pass(model, xb, path=launch)
        torch.cuda.synchronize()
        assert torch.equal(logits, ref)
        for s in range(4 * shape.n_layers + 1):
            for u, v in zip(_stage_io(model, shape, K, ws, logits, s), _stage_io(model, shape, K, ws_ref, ref, s)):
                assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), f"stage {s}"
        xa, xb = xb, xa
