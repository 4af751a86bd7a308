"""GPU parity of the uniforms the verifier draws for itself (Philox4x32-10,
counter (block, request, step), key seed) and of the acceptance histogram:
decisions equal the oracle's with the oracle's own generator, and equal the
same call given those uniforms explicitly."""
import numpy as np
import pytest

from oracle import oracle as O
from tests.gpu_helpers import check_verify_chain, dev, host
from workloads import synth

pytestmark = pytest.mark.gpu

SEED, OFFSET = 0x5EED5EED12345678, (3 << 32) + 17


def test_config0_rng_matches_oracle_and_explicit_uniforms():
    import torch
    import draft_verification_spec_amd as S
    c = synth.config0()
    BS, B, V = c["BS"], c["B"], c["V"]
    u_acc, u_smp = O.step_uniforms(BS, B, SEED, OFFSET)
    common = (dev(c["target"]).reshape(-1, V), dev(np.arange(BS) * (B + 1)), dev(c["tokens"]),
              dev(np.full(BS, B, np.int32)), 1.0)
    kw = dict(slot_flags=dev(np.zeros((BS, B), np.uint8)), draft_logits=dev(c["draft"]).reshape(-1, V),
              draft_row_base=dev(np.arange(BS) * B))
    hist = torch.zeros(B + 1, dtype=torch.int32, device="cuda:0")
    g = S.spec_verify_chain(*common, rng=(SEED, OFFSET), accept_hist=hist, **kw)
    e = S.spec_verify_chain(*common, u_accept=dev(u_acc), u_sample=dev(u_smp), **kw)
    torch.cuda.synchronize()
    for k in g:
        assert np.array_equal(host(g[k]), host(e[k])), k
    ref = O.verify_chain(c["target"].reshape(-1, V), np.arange(BS) * (B + 1), c["tokens"], np.zeros((BS, B), np.uint8),
                         np.full(BS, B, np.int32), u_acc, u_smp, 1.0, draft_logits=c["draft"].reshape(-1, V),
                         draft_row_base=np.arange(BS) * B)
    check_verify_chain({k: host(v) for k, v in g.items()}, ref, np.full(BS, B), "config 0 rng")
    assert np.array_equal(host(hist), np.bincount(host(g["out_accepted"]), minlength=B + 1))


def test_dense_headline_rng_and_histogram():
    """The measured step's shape (BS 128, V 151,936, bf16, T = 1) with drawn
    uniforms; two different steps draw different uniforms."""
    import torch
    import draft_verification_spec_amd as S
    c = synth.dense_headline()
    BS, V, B = c["BS"], c["V"], c["B"]
    tgt = synth.as_torch_bf16(c["target_bf16"]).to("cuda:0").reshape(-1, V)
    dft = synth.as_torch_bf16(c["draft_bf16"]).to("cuda:0").reshape(-1, V)
    common = (tgt, dev(np.arange(BS, dtype=np.int64) * (B + 1)), dev(c["tokens"]), dev(np.full(BS, B, np.int32)), 1.0)
    kw = dict(slot_flags=dev(np.zeros((BS, B), np.uint8)), draft_logits=dft,
              draft_row_base=dev(np.arange(BS, dtype=np.int64) * B))
    hist = torch.zeros(B + 1, dtype=torch.int32, device="cuda:0")
    g = S.spec_verify_chain(*common, rng=(SEED, OFFSET), accept_hist=hist, **kw)
    g2 = S.spec_verify_chain(*common, rng=(SEED, OFFSET + 1), **kw)
    torch.cuda.synchronize()
    u_acc, u_smp = O.step_uniforms(BS, B, SEED, OFFSET)
    ref = O.verify_chain(c["target_bf16"].reshape(-1, V), np.arange(BS) * (B + 1), c["tokens"],
                         np.zeros((BS, B), np.uint8), np.full(BS, B, np.int32), u_acc, u_smp, 1.0,
                         draft_logits=c["draft_bf16"].reshape(-1, V), draft_row_base=np.arange(BS) * B)
    check_verify_chain({k: host(v) for k, v in g.items()}, ref, np.full(BS, B), "dense rng")
    h = host(hist)
    assert h.sum() == BS and np.array_equal(h, np.bincount(host(g["out_accepted"]), minlength=B + 1))
    assert not np.array_equal(host(g["out_tokens"]), host(g2["out_tokens"]))
    print(f"  accepted per request {host(g['out_accepted']).mean():.2f}")
