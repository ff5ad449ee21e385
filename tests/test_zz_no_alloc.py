"""vq_skinny_qmm_noalloc (the skinny QMM with the library's own scratch, for
callers that cannot allocate) against vq_skinny_qmm with a workspace: the same
outputs bit for bit, on two calls in a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

from synth import qmm_activations, qmm_weights
from tests.gpu_util import bf16_tensor, words_tensor

pytestmark = pytest.mark.gpu


def _case(vq, seed, bits, M, N, K, y_dtype):
    w = qmm_weights(60 + seed, N, K, bits)
    x = bf16_tensor(qmm_activations(60 + seed, M, K))
    wq, s, b = words_tensor(w["wq"]), bf16_tensor(w["scales"]), bf16_tensor(w["biases"])
    ref = vq.skinny_qmm(x, wq, s, b, bits, N, K, out_dtype=y_dtype)
    out = torch.full((M, N), float("nan"), dtype=y_dtype, device=x.device)
    vq.skinny_qmm_noalloc(x, wq, s, b, bits, N, K, out=out)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("bits,y_dtype", [(4, torch.bfloat16), (8, torch.float32)])
def test_noalloc_matches_workspace_entry(vq, bits, y_dtype):
    # first call: a 27B-shaped gate|up projection at 16 rows (10.7 MiB of scratch);
    # second call: a smaller one (config-0 shape, 3 rows) on the same scratch
    for seed, (M, N, K) in enumerate(((16, 34816, 5120), (3, 512, 1024))):
        ref, out = _case(vq, seed, bits, M, N, K, y_dtype)
        assert torch.equal(ref.view(torch.int16) if y_dtype == torch.bfloat16 else ref.view(torch.int32),
                           out.view(torch.int16) if y_dtype == torch.bfloat16 else out.view(torch.int32)), (M, N, K)


def test_noalloc_repeated_and_captured(vq):
    """Calls in order on one stream reuse the scratch; a captured graph of the
    call replays with the same result after eager calls in between."""
    M, N, K, bits = 8, 5120, 17408, 4
    w = qmm_weights(70, N, K, bits)
    x = bf16_tensor(qmm_activations(70, M, K))
    wq, s, b = words_tensor(w["wq"]), bf16_tensor(w["scales"]), bf16_tensor(w["biases"])
    ref = vq.skinny_qmm(x, wq, s, b, bits, N, K)
    out = torch.empty_like(ref)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        vq.skinny_qmm_noalloc(x, wq, s, b, bits, N, K, out=out)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vq.skinny_qmm_noalloc(x, wq, s, b, bits, N, K, out=out)
    for i in range(3):
        out.zero_()
        small = torch.empty((2, 512), dtype=torch.bfloat16, device=x.device)
        w2 = qmm_weights(71, 512, 1024, 8)
        vq.skinny_qmm_noalloc(bf16_tensor(qmm_activations(71, 2, 1024)), words_tensor(w2["wq"]),
                              bf16_tensor(w2["scales"]), bf16_tensor(w2["biases"]), 8, 512, 1024, out=small)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), i
