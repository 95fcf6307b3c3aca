"""kda_prefill_chunked_noalloc (the library's own per-GPU scratch instead of
a caller workspace) against kda_prefill_chunked on the same inputs, through
the C ABI: two calls in a row, the second smaller, each bit-identical to the
workspace call in outputs and pool rows, and both within the oracle's bar;
an input beyond the scratch is refused before any launch."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrent_amd import binding as la
from linear_attention_recurrent_amd import synth
from parity_util import assert_close_seqs, assert_close_units, f64

pytestmark = pytest.mark.gpu

D = 128


def case(lens, H, seed, dev, si, so, P):
    sh = synth.PrefillShape(seqlens=tuple(lens), Hqk=H, Hv=H, dk=D, dv=D)
    inp = synth.prefill_inputs(sh, seed, dev)
    pool = synth.normal_torch(seed, synth.S_SSM, (P + 1) * H * D * D, dev,
                              torch.float32).view(P + 1, H, D, D)
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=dev)  # noqa: E731
    return sh, inp, pool, i32(si), i32(so)


@pytest.mark.parametrize("mode", [la.LA_PREFILL_FP32, la.LA_PREFILL_BF16X3])
def test_noalloc_prefill_matches_the_workspace_call(mode, dev):
    for lens, H, seed, si, so, P in (([200, 64, 131], 4, 3500, [1, -1, 2], [3, 4, 2], 4),
                                     ([70], 2, 3501, [-1], [1], 2)):
        print(f"[noalloc] lens={lens} H={H} mode={mode}", flush=True)
        sh, inp, pool, si_t, so_t = case(lens, H, seed, dev, si, so, P)
        ref_pool = pool.clone()
        before = f64(pool)
        out = torch.empty((sh.T, H, D), dtype=torch.bfloat16, device=dev)
        args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"], si_t, so_t)
        la.kda_prefill_chunked_noalloc(*args, pool, out=out, mode=mode)
        ref = la.kda_prefill_chunked(*args, ref_pool, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(pool, ref_pool)
        q, k, v, g, beta = (f64(inp[x]) for x in ("q", "k", "v", "g", "beta"))
        o_ref, p_ref = oracle.prefill(q, k, v, g, beta, inp["cu_seqlens"].cpu().numpy(),
                                      np.array(si, np.int32), np.array(so, np.int32), before,
                                      kda=True, state_dtype="fp32", io_dtype="bf16")
        assert_close_seqs(f64(out), o_ref, inp["cu_seqlens"].cpu().numpy(), "bf16",
                          "noalloc outputs")
        assert_close_units(f64(pool)[so], p_ref[so], 2, "fp32", "noalloc states")


def test_noalloc_prefill_refuses_inputs_beyond_its_scratch(dev):
    T, H = 8192, 12   # 8192 x 12 token-heads need ~277 MB of workspace
    assert la.kda_prefill_workspace_bytes(1, T, H, H, D, D, 1) > (128 << 20)
    t = torch.empty(0, device=dev)
    q = torch.zeros((T, H, D), dtype=torch.bfloat16, device=dev)
    g = torch.zeros((T, H, D), dtype=torch.float32, device=dev)
    beta = torch.zeros((T, H), dtype=torch.float32, device=dev)
    i32 = lambda v: torch.tensor(v, dtype=torch.int32, device=dev)  # noqa: E731
    pool = torch.zeros((2, H, D, D), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    with pytest.raises(la.LAError, match="128 MiB"):
        la.kda_prefill_chunked_noalloc(q, q, q, g, beta, i32([0, T]), i32([-1]), i32([1]), pool,
                                       out=out, mode=1)
    del t
