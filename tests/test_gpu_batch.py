"""K columns as a batch of independent sequences (one token each): the pass applies every
stage to each column alone (the dot products, the per-column rho, silu(gate) up), so column
j of a K-column pass gives the logits of a one-column pass over column j's input.  Checked
on the mini and mid stacks at K = 8 and 16: every column within 2e-3 of its row's largest
|logit| of the one-column pass.  Where the two passes split the reductions differently (at
K = 16 the mid stack runs in column windows) the bits may differ: a stage input rounded to
fp16 can land one fp16 ulp (~5e-4 relative) apart and carry on through the stack; a column
mixed with another would differ at the size of the logits."""
import numpy as np
import pytest

import synth
from gpu_util import need_gpu, report, upload_model

pytestmark = pytest.mark.gpu

SHAPE_MID = synth.ModelShape(n_layers=2, hidden=2048, kv_dim=256, ffn=5120, vocab=4000)


@pytest.mark.parametrize("name,K", [("mini", 8), ("mini", 16), ("mid", 8), ("mid", 16)])
def test_columns_are_independent_sequences(name, K):
    torch = need_gpu()
    import speculative_decoding_verification_bit_amd as vq
    shape = synth.SHAPE_MINI if name == "mini" else SHAPE_MID
    model = upload_model(shape, synth.FMT_Q4_MIN, 21)
    x = synth.activations(21, K, shape.hidden)
    logits, ws = vq.decode_pass(model, torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert model.barrier_error(K, ws) == 0
    batch = logits.cpu().numpy()
    worst, same = 0.0, 0
    for j in range(K):
        one, ws1 = vq.decode_pass(model, torch.from_numpy(np.ascontiguousarray(x[j:j + 1])).cuda())
        torch.cuda.synchronize()
        assert model.barrier_error(1, ws1) == 0
        one = one.cpu().numpy()[0]
        scale = float(np.max(np.abs(one)))
        err = float(np.max(np.abs(batch[j] - one)))
        worst = max(worst, err / scale)
        same += int(np.array_equal(batch[j], one))
        assert err <= 2e-3 * scale, (name, K, j, err, scale)
    report(f"batch {name} K {K}: columns against one-column passes, worst {worst:.2e} of max|logit| "
           f"({same} of {K} bit-identical)")
