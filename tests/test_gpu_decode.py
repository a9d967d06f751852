"""GPU parity of vq_decode_pass.  Every checked stage's input is compared with the oracle's
glue applied to the GPU's previous output (bit-exact where the glue is a plain fp16
rounding; within one fp16 ulp for silu(gate) * up, which the GPU evaluates in fp32), and
its output with rho * (W x) of the oracle on the GPU's own stage input, rho in fp64 from
the GPU's previous output, to the per-row tolerance 1e-3 * rho * sum|w x|.  The staged
launch (one launch per stage) and the persistent one give identical bits."""
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
    sp = None if mats[0].supers is None else np.concatenate([m.supers for m in mats])
    full = synth.Q4Matrix(fmt, qs.shape[0], mats[0].cols, qs, sc, mn, sp)
    return full if rows_pick is None else full.take(rows_pick)


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


def _check_glue(shape, stage, xin, prev_out, what):
    """The stage's fp16 input against the oracle's glue of the previous GPU output; returns
    the oracle's rho for the stage's outputs."""
    pk = (stage - 1) % 4
    v, rho = oracle.stage_glue(prev_out, pk, shape.hidden, shape.ffn)
    e16 = v.astype(np.float16)
    if pk != oracle.STAGE_GU:
        bad = int((xin.view(np.uint16) != e16.view(np.uint16)).sum())
        assert bad == 0, f"{what}: {bad} inputs differ from the fp16 rounding of the previous output"
    else:
        diff = np.abs(xin.astype(np.float64) - e16.astype(np.float64))
        ulp = np.spacing(np.abs(e16)).astype(np.float64)
        off = int((diff > 0).sum())
        assert not (diff > ulp).any(), f"{what}: silu(gate)*up inputs beyond one fp16 ulp ({off} differ)"
        if off:
            say(f"{what}: {off} of {diff.size} silu(gate)*up inputs one fp16 ulp off the oracle's rounding")
    return rho


def _check_stage(model, shape, fmt, seed, K, ws, logits, s, x0=None, prev=None, W=None, rows_pick=None, what=""):
    xin, out = _stage_io(model, shape, K, ws, logits, s)
    if s == 0:
        assert np.array_equal(xin.view(np.uint16), x0.view(np.uint16)), f"{what}: stage 0 input is not x0"
        rho = np.ones(K)
    else:
        if prev is None:
            _, prev = _stage_io(model, shape, K, ws, logits, s - 1)
        rho = _check_glue(shape, s, xin, prev, f"{what} stage {s}")
    if W is None:
        W = _stage_mats(shape, fmt, seed, s, rows_pick)
    y_ref, a_ref = oracle.linear(W, xin, threads=8)
    got = out if rows_pick is None else out[:, rows_pick]
    check_rows(got, y_ref * rho[:, None], a_ref * rho[:, None], f"{what} stage {s}")
    return out


def _pass(model, shape, K, x0, launch):
    """One pass into guarded workspace and logits buffers; returns (logits, ws)."""
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    nws = model.workspace_bytes(K)
    ws, ws_whole = guarded_buffer(nws)
    nlg = K * shape.vocab * 4
    lg, lg_whole = guarded_buffer(nlg)
    logits = lg.view(torch.float32).view(K, shape.vocab)
    _, _, nl = vq.decode_pass_launch(model, torch.from_numpy(x0).cuda(), logits, ws=ws, launch=launch)
    torch.cuda.synchronize()
    check_guard(ws_whole, nws, f"K {K} launch {launch}: decode workspace")
    check_guard(lg_whole, nlg, f"K {K} launch {launch}: logits")
    assert model.barrier_error(K, ws) == 0, f"K {K} launch {launch}: a wait timed out"
    return logits, ws, nl


def _every_stage(shape, seed, fmt, K):
    """One pass per launch mode; every row of every stage against the oracle; the two
    launch modes bitwise equal."""
    import speculative_decoding_verification_bit_amd as vq
    model = upload_model(shape, fmt, seed)
    x0 = synth.activations(seed, K, shape.hidden)
    say(f"every stage: {shape} fmt {fmt} K {K}")
    lp, wp, nlp = _pass(model, shape, K, x0, vq.LAUNCH_AUTO)
    ls, wsg, nls = _pass(model, shape, K, x0, vq.LAUNCH_STAGED)
    assert nls == 4 * shape.n_layers + 1
    prev = None
    for s in range(4 * shape.n_layers + 1):
        prev = _check_stage(model, shape, fmt, seed, K, wp, lp, s, x0=x0, prev=prev, what=f"fmt {fmt} K {K}")
        for u, v in zip(_stage_io(model, shape, K, wp, lp, s), _stage_io(model, shape, K, wsg, ls, s)):
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), f"stage {s}: staged and persistent differ"
    assert np.isfinite(lp.cpu().numpy()).all()


@pytest.mark.parametrize("fmt", [synth.FMT_Q4_MIN, synth.FMT_Q4, synth.FMT_MXFP4, synth.FMT_Q4_K])
@pytest.mark.parametrize("K", [1, 2, 3, 4, 8, 16])
def test_mini_model_every_stage(fmt, K):
    """A 2-layer stack (hidden 256, kv 64, ffn 512, vocab 1000): all rows of all stages."""
    _every_stage(synth.SHAPE_MINI, 4, fmt, K)


# Two layers whose rows split into 5 and 16 column groups per compute wave
SHAPE_MID = synth.ModelShape(n_layers=2, hidden=2048, kv_dim=256, ffn=5120, vocab=4000)


@pytest.mark.parametrize("K", [1, 4, 8, 16])
def test_mid_model_every_stage(K):
    """hidden 2048, kv 256, ffn 5120, vocab 4000 (a partial last lm_head tile)."""
    _every_stage(SHAPE_MID, 9, synth.FMT_Q4_MIN, K)


# More layers than one persistent launch carries (16): launch boundaries inside the pass
SHAPE_DEEP = synth.ModelShape(n_layers=20, hidden=256, kv_dim=64, ffn=512, vocab=1000)


def test_deep_model_across_launches():
    import speculative_decoding_verification_bit_amd as vq
    shape, seed, fmt, K = SHAPE_DEEP, 13, synth.FMT_Q4_MIN, 4
    model = upload_model(shape, fmt, seed)
    x0 = synth.activations(seed, K, shape.hidden)
    lp, wp, nlp = _pass(model, shape, K, x0, vq.LAUNCH_AUTO)
    ls, wsg, _ = _pass(model, shape, K, x0, vq.LAUNCH_STAGED)
    assert nlp == 2, f"20 layers run as {nlp} persistent launches"
    prev = None
    for s in range(4 * shape.n_layers + 1):
        prev = _check_stage(model, shape, fmt, seed, K, wp, lp, s, x0=x0, prev=prev, what="deep")
    assert np.array_equal(lp.cpu().numpy(), ls.cpu().numpy())


@pytest.mark.parametrize("fmt,Ks", [(synth.FMT_Q4_MIN, (1, 4, 8)), (synth.FMT_MXFP4, (16,)),
                                    (synth.FMT_Q4_K, (1, 8))])
def test_27b_stack_sampled_rows(fmt, Ks):
    """The full 27B-class stack (64 layers, 5120 / 1024 / 17408, vocab 151936) in one pass;
    stages of layers 0, 31, 63 and the lm_head checked on 24 sampled rows each, every
    checked stage's input against the glue of the previous output; at every K the staged
    launch (one launch per stage) gives the same bits as the persistent one."""
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
        mats[s] = full.take(pick)
        del full
    for K in Ks:
        x0 = synth.activations(seed, K, shape.hidden)
        logits, ws, nl = _pass(model, shape, K, x0, vq.LAUNCH_AUTO)
        say(f"K {K}: {nl} persistent launches")
        for s in stages:
            _check_stage(model, shape, fmt, seed, K, ws, logits, s, x0=x0, W=mats[s], rows_pick=picks[s],
                         what=f"27B fmt {fmt} K {K}")
        ls, wsg, nls = _pass(model, shape, K, x0, vq.LAUNCH_STAGED)
        assert nls == 4 * L + 1
        assert torch.equal(logits, ls), f"K {K}: staged and persistent logits differ"
        for s in stages:
            for u, v in zip(_stage_io(model, shape, K, ws, logits, s), _stage_io(model, shape, K, wsg, ls, s)):
                assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), f"K {K} stage {s}"
        del wsg, ls
        del ws, logits
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
        assert model.barrier_error(K, ws) == 0
        del scratch


def test_workspace_reuse_with_new_inputs():
    """A pass over a workspace that still holds another input's pass gives the same bits
    as a pass over a fresh workspace: nothing stale is read back from the previous pass."""
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    shape, seed, K = synth.SHAPE_MINI, 7, 4
    model = upload_model(shape, synth.FMT_Q4_MIN, seed)
    xa = torch.from_numpy(synth.activations(seed, K, shape.hidden)).cuda()
    xb = torch.from_numpy(synth.activations(seed + 1, K, shape.hidden)).cuda()
    logits, ws = vq.decode_pass(model, xa)
    for _ in range(3):
        vq.decode_pass(model, xb, logits, ws=ws)
        torch.cuda.synchronize()
        ref, ws_ref = vq.decode_pass(model, xb)
        torch.cuda.synchronize()
        assert torch.equal(logits, ref)
        for s in range(4 * shape.n_layers + 1):
            for u, v in zip(_stage_io(model, shape, K, ws, logits, s), _stage_io(model, shape, K, ws_ref, ref, s)):
                assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), f"stage {s}"
        xa, xb = xb, xa
