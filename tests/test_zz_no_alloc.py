"""lattice_osr_fwd_chunked_noalloc: the chunked forward with its workspace in
the library's per-GPU scratch array instead of a caller's buffer (for callers
that cannot allocate).  Its output must equal lattice_osr_fwd_chunked's with a
caller workspace bit for bit (the same kernels on the same inputs), call after
call: the scratch keeps the last call's contents, and what must start at zero
(the hand-off counters of the state passing split over workgroups) is cleared
by each call.
"""
import sys

import pytest
import torch

from compressed_memory_linear_amd import osr, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    osr.load_library()
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _both(inp, C, **kw):
    t = osr.to_device(inp)
    args = (t["q"], t["k"], t["v"], t["gamma"], t["mu"], t["state"])
    y_ref, S_ref = osr.lattice_osr_fwd_chunked(*args, C, **kw)
    y = torch.full_like(y_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    osr.lattice_osr_fwd_chunked_noalloc(*args, C, state_out=S, y=y, **kw)
    torch.cuda.synchronize()
    return y_ref, S_ref, y, S


# (B, T, H, m, d, C): the split schedule, then a smaller one; the state passing
# split over four workgroups twice in a row (its counters must be re-zeroed);
# the token loop (no workspace at all).
CALLS = [(2, 512, 4, 64, 64, 64), (1, 256, 2, 64, 128, 64), (1, 512, 16, 128, 128, 128), (1, 256, 16, 128, 128, 128),
         (2, 64, 2, 32, 32, 4)]


def test_noalloc_matches_workspace_entry_call_after_call():
    for i, (B, T, H, m, d, C) in enumerate(CALLS):
        _say(f"no-alloc call {i}: B{B} T{T} H{H} m{m} d{d} C{C}")
        inp = synth.make_inputs(B, T, H, m, d, seed=4000 + i, in_dtype=synth.BF16)
        desc = osr.make_desc(B, T, H, m, d)
        need = osr.lattice_osr_workspace_bytes(desc, C)
        assert need <= osr.NOALLOC_SCRATCH_BYTES
        y_ref, S_ref, y, S = _both(inp, C)
        _say(f"  workspace {need} bytes; identical: {torch.equal(y, y_ref) and torch.equal(S, S_ref)}")
        assert torch.equal(y, y_ref) and torch.equal(S, S_ref)


def test_noalloc_rejects_workspace_beyond_the_scratch():
    B, T, H, m, d, C = 8, 2048, 8, 64, 64, 64   # 128 MiB of per-chunk arrays
    desc = osr.make_desc(B, T, H, m, d)
    assert osr.lattice_osr_workspace_bytes(desc, C) > osr.NOALLOC_SCRATCH_BYTES
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")
    q, v, mu = z(B, T, H, m), z(B, T, H, d), z(B, T, H)
    st = torch.zeros(B, H, m, d, device="cuda")
    with pytest.raises(osr.OSRError) as e:
        osr.lattice_osr_fwd_chunked_noalloc(q, q, v, q, mu, st, C, state_out=torch.empty_like(st),
                                            y=torch.empty(B, T, H, d, device="cuda"))
    assert e.value.status == osr.ERR_WORKSPACE
