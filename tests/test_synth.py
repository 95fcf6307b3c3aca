"""The seeded input generator: SplitMix64 reference values, numpy/torch
agreement and the workload distributions."""
import numpy as np
import torch

from linear_attention_recurrent_amd import synth


def test_splitmix64_reference_sequence():
    # SplitMix64 seeded with state 0: the published first outputs.
    base = 0
    z = []
    state = base
    for _ in range(3):
        state = (state + synth.GAMMA) & ((1 << 64) - 1)
        z.append(synth._mix64_int(state))
    assert z == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_numpy_and_torch_draws_agree():
    a = synth.raw_u64(7, 3, 1000, offset=17)
    b = synth.raw_u64_torch(7, 3, 1000, offset=17).numpy().view(np.uint64)
    assert np.array_equal(a, b)
    n = synth.normal(7, 3, (999,))
    t = synth.normal_torch(7, 3, 999, dtype=torch.float32).numpy()
    assert np.array_equal(n.astype(np.float32), t)


def test_distributions():
    z = synth.normal(1, 0, (200000,))
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    g = synth.log_decay(1, 1, (100000,))
    assert g.dtype == np.float32 and np.all(g < 0)
    b = synth.beta_gate(1, 2, (100000,))
    assert np.all((b > 0) & (b < 1))


def test_slot_permutation_is_a_permutation_of_usable_rows():
    p = synth.slot_permutation(5, 0, 80)
    assert sorted(p.tolist()) == list(range(1, 81))
    assert not np.array_equal(p, np.arange(1, 81))


def test_decode_inputs_shapes_and_determinism():
    sh = synth.DecodeShape(B=4, Hqk=2, Hv=4, dk=16, dv=16, P=6, kda=False)
    a = synth.decode_inputs(sh, 9)
    b = synth.decode_inputs(sh, 9)
    for key in a:
        assert torch.equal(a[key], b[key]), key
    assert a["x"].shape == (4, sh.C) and a["x"].dtype == torch.bfloat16
    assert a["g"].shape == (4, 4)
    assert a["ssm_pool"].shape == (7, 4, 16, 16)
    assert len(set(a["slots"].tolist())) == 4 and min(a["slots"].tolist()) >= 1
