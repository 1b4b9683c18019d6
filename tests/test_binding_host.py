"""Host-only checks of the Python binding's argument checks (no GPU needed).

Before any call into the library, every tensor is checked against the
descriptor the call builds from q and v: shapes, dtypes, layout, then the
device.  A mismatch raises ValueError instead of letting a kernel index past
a buffer.  These cases use CPU tensors: shape and dtype errors are found
first, and tensors that pass those checks are refused for not being on the
GPU, so nothing reaches the library.
"""
import pytest
import torch

from compressed_memory_linear_amd import osr

B, T, H, m, d = 2, 8, 3, 16, 32


def _inputs(dtype=torch.bfloat16, per_slot=True):
    g = (B, T, H, m) if per_slot else (B, T, H)
    return dict(q=torch.zeros(B, T, H, m, dtype=dtype), k=torch.zeros(B, T, H, m, dtype=dtype),
                v=torch.zeros(B, T, H, d, dtype=dtype), gamma=torch.zeros(g, dtype=dtype),
                mu=torch.zeros(B, T, H, dtype=dtype), state_in=torch.zeros(B, H, m, d))


def _fwd(x, **kw):
    return osr.lattice_osr_fwd_chunked(x["q"], x["k"], x["v"], x["gamma"], x["mu"], x["state_in"], 4, **kw)


BAD = [
    ("k", lambda x: torch.zeros(B, T, H, m + 16, dtype=x["q"].dtype), "k has shape"),
    ("k", lambda x: torch.zeros(B, T + 1, H, m, dtype=x["q"].dtype), "k has shape"),
    ("v", lambda x: torch.zeros(B, T, H + 1, d, dtype=x["q"].dtype), "v has shape"),
    ("gamma", lambda x: torch.zeros(B, T, H, m - 1, dtype=x["q"].dtype), "gamma has shape"),
    ("gamma", lambda x: torch.zeros(B, T, H + 1, dtype=x["q"].dtype), "gamma has shape"),
    ("mu", lambda x: torch.zeros(B, T, H, 1, dtype=x["q"].dtype), "mu has shape"),
    ("mu", lambda x: torch.zeros(B, T, dtype=x["q"].dtype), "mu has shape"),
    ("state_in", lambda x: torch.zeros(B, H, m, d + 16), "state_in has shape"),
    ("state_in", lambda x: torch.zeros(B, H, m, d, dtype=torch.bfloat16), "state_in is"),
    ("k", lambda x: torch.zeros(B, T, H, m, dtype=torch.float32), "k is"),
    ("v", lambda x: torch.zeros(B, T, H, 2 * d, dtype=x["q"].dtype)[..., :d], "v must be contiguous"),
]


@pytest.mark.parametrize("name,make,msg", BAD, ids=[f"{n}-{i}" for i, (n, _, _) in enumerate(BAD)])
def test_forward_input_checks(name, make, msg):
    x = _inputs()
    x[name] = make(x)
    with pytest.raises(ValueError, match=msg):
        _fwd(x)


@pytest.mark.parametrize("entry", ["chunked", "recurrent", "decode"])
def test_every_entry_checks_inputs(entry):
    x = _inputs()
    x["k"] = torch.zeros(B, T, H, m + 16, dtype=torch.bfloat16)
    fn = {"chunked": lambda: _fwd(x),
          "recurrent": lambda: osr.lattice_osr_fwd_recurrent(*(x[n] for n in ("q", "k", "v", "gamma", "mu",
                                                                              "state_in"))),
          "decode": lambda: osr.lattice_osr_decode_step(*(x[n] for n in ("q", "k", "v", "gamma", "mu",
                                                                         "state_in")))}[entry]
    with pytest.raises(ValueError, match="k has shape"):
        fn()


def test_output_checks():
    x = _inputs()
    with pytest.raises(ValueError, match="y has shape"):
        _fwd(x, y=torch.zeros(B, T, H, d + 1))
    with pytest.raises(ValueError, match="y is"):
        _fwd(x, y=torch.zeros(B, T, H, d, dtype=torch.bfloat16))  # y_dtype defaults to float32
    with pytest.raises(ValueError, match="state_out has shape"):
        _fwd(x, state_out=torch.zeros(B, H, m + 16, d))
    with pytest.raises(ValueError, match="y_dtype"):
        _fwd(x, y_dtype=torch.float16)


def test_host_tensors_are_refused():
    """Correct shapes on the host: refused before the library is called."""
    for per_slot in (True, False):
        with pytest.raises(ValueError, match="GPU"):
            _fwd(_inputs(per_slot=per_slot))


def test_backward_checks():
    x = _inputs()
    args = [x[n] for n in ("q", "k", "v", "gamma", "mu", "state_in")]
    with pytest.raises(ValueError, match="dy has shape"):
        osr.lattice_osr_bwd_chunked(*args, torch.zeros(B, T, H, d + 1), torch.zeros(B, H, m, d), 4)
    with pytest.raises(ValueError, match="dstate_out has shape"):
        osr.lattice_osr_bwd_chunked(*args, torch.zeros(B, T, H, d), torch.zeros(B, H, m, d + 1), 4)
    grads = {"d" + n: torch.zeros(t.shape) for n, t in zip(("q", "k", "v", "gamma", "mu", "state_in"), args)}
    grads["dk"] = torch.zeros(B, T, H, m + 1)
    with pytest.raises(ValueError, match="dk has shape"):
        osr.lattice_osr_bwd_chunked(*args, torch.zeros(B, T, H, d), torch.zeros(B, H, m, d), 4, grads=grads)


def test_glue_checks():
    xq = torch.zeros(B, T, H, m, dtype=torch.bfloat16)
    w = torch.zeros(H, m, 4)
    with pytest.raises(ValueError, match="xk has shape"):
        osr.lattice_osr_glue_pre(xq, torch.zeros(B, T, H, m + 1, dtype=torch.bfloat16), xq, w, w)
    with pytest.raises(ValueError, match="conv_wk has shape"):
        osr.lattice_osr_glue_pre(xq, xq, xq, w, torch.zeros(H, m, 3))
    with pytest.raises(ValueError, match="hist_q has shape"):
        osr.lattice_osr_glue_pre(xq, xq, xq, w, w, hist_q=torch.zeros(B, 2, H, m, dtype=torch.bfloat16),
                                 hist_k=torch.zeros(B, 3, H, m, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU"):
        osr.lattice_osr_glue_pre(xq, xq, xq, w, w)
    y = torch.zeros(B, T, H, d)
    with pytest.raises(ValueError, match="gate has shape"):
        osr.lattice_osr_glue_post(y, torch.zeros(B, T, H, d + 1))
    with pytest.raises(ValueError, match="GPU"):
        osr.lattice_osr_glue_post(y, torch.zeros(B, T, H, d))


def test_gated_forward_checks():
    x = _inputs()
    args = [x[n] for n in ("q", "k", "v", "gamma", "mu")]
    with pytest.raises(ValueError, match="gate has shape"):
        osr.lattice_osr_fwd_chunked_gated(*args, torch.zeros(B, T, H, d + 1, dtype=torch.bfloat16), x["state_in"], 4)
    with pytest.raises(ValueError, match="gate is"):
        osr.lattice_osr_fwd_chunked_gated(*args, torch.zeros(B, T, H, d), x["state_in"], 4)
    with pytest.raises(ValueError, match="GPU"):
        osr.lattice_osr_fwd_chunked_gated(*args, torch.zeros(B, T, H, d, dtype=torch.bfloat16), x["state_in"], 4)
