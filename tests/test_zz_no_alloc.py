"""The chain verifier's entry point that allocates nothing
(spec_verify_chain_noalloc, scratch from the library's per-device array)
against spec_verify_chain with a caller workspace: two calls in a row, the
second on a smaller batch, each output identical."""
import numpy as np
import pytest

from tests.gpu_helpers import dev, host
from workloads import synth

pytestmark = pytest.mark.gpu


def _call(c, BS, noalloc, ngram):
    import torch
    import draft_verification_spec_amd as S
    B, V = c["B"], c["V"]
    tgt = synth.as_torch_bf16(c["target_bf16"][:BS]).to("cuda:0").reshape(-1, V)
    dft = synth.as_torch_bf16(c["draft_bf16"][:BS]).to("cuda:0").reshape(-1, V)
    ctx, ctx_len = dev(c["ctx"][:BS]), dev(c["ctx_len"][:BS])
    new_len = torch.zeros(BS, dtype=torch.int32, device="cuda:0")
    out = dict(out_tokens=torch.full((BS, B + 1), -7, dtype=torch.int32, device="cuda:0"),
               out_num=torch.zeros(BS, dtype=torch.int32, device="cuda:0"),
               out_accepted=torch.zeros(BS, dtype=torch.int32, device="cuda:0"),
               out_p=torch.zeros((BS, B + 1), dtype=torch.float32, device="cuda:0"),
               out_q=torch.zeros((BS, B), dtype=torch.float32, device="cuda:0"))
    flags = torch.zeros(BS, dtype=torch.int32, device="cuda:0")
    ng = (torch.zeros((BS, 15), dtype=torch.int32, device="cuda:0"), torch.zeros(BS, dtype=torch.int32, device="cuda:0"),
          torch.zeros((BS, 4), dtype=torch.int32, device="cuda:0")) if ngram else None
    r = S.spec_verify_chain(tgt, dev(np.arange(BS, dtype=np.int64) * (B + 1)), dev(c["tokens"][:BS]),
                            dev(np.full(BS, B, np.int32)), c["temperature"], u_accept=dev(c["u_acc"][:BS]),
                            u_sample=dev(c["u_smp"][:BS]), slot_flags=dev(np.zeros((BS, B), np.uint8)),
                            draft_logits=dft, draft_row_base=dev(np.arange(BS, dtype=np.int64) * B), out=out,
                            out_flags=flags, ctx=ctx, ctx_len=ctx_len, ctx_len_out=new_len, noalloc=noalloc,
                            ngram=(5, 15, 15, 256) if ngram else None, ngram_out=ng)
    torch.cuda.synchronize()
    res = {k: host(v) for k, v in r.items()}
    res["ctx"], res["ctx_len"] = host(ctx), host(new_len)
    return res


def test_noalloc_matches_workspace_call_twice():
    c = synth.dense_headline(BS=48, ctx_extra=64)
    for BS, ngram in ((48, True), (9, False)):   # the second call: a smaller batch over the same array
        print(f"noalloc vs workspace: BS {BS} V {c['V']} ngram {ngram}", flush=True)
        a = _call(c, BS, True, ngram)
        b = _call(c, BS, False, ngram)
        assert set(a) == set(b)
        for k in a:
            assert np.array_equal(a[k], b[k]), (BS, k)
        assert (a["out_num"] >= 1).all()


def test_noalloc_rejects_oversized_calls():
    import draft_verification_spec_amd as S
    from draft_verification_spec_amd import _lib as L
    import torch
    # fp32 rows of V 8,388,608 at BS 64 and 32 slots need 136 MB of scratch, more
    # than the array holds: the call is refused before anything is enqueued
    BS, ld, V = 64, 32, 1 << 23
    logits = torch.zeros((1, V), dtype=torch.float32, device="cuda:0")
    with pytest.raises(RuntimeError, match="workspace"):
        S.spec_verify_chain(logits, dev(np.zeros(BS, np.int64)), dev(np.zeros((BS, ld), np.int32)),
                            dev(np.zeros(BS, np.int32)), 0.0, noalloc=True)
    assert L.NOALLOC_SCRATCH_BYTES == 16 << 20
