"""Host-side argument checks of the Python binding (no GPU): every entry point rejects
tensors that are not in device memory, and a non-contiguous q, before anything reaches
the C ABI. A tensor stand-in reports a CUDA device for the contiguity checks (its data
stays on the host and is never passed on: the checks raise first)."""
import pytest
import torch

import gated_delta_rule_48_amd as kda


class DevT:
    """A host tensor that reports device cuda:0 (the binding's checks read only its
    metadata)."""

    def __init__(self, t):
        self._t = t

    @property
    def device(self):
        return torch.device("cuda:0")

    def __getattr__(self, n):
        return getattr(self._t, n)


def _fwd_args(B=1, T=8, H=2, d=64):
    q = torch.zeros(B, T, H, d)
    return dict(q=q, k=q.clone(), v=q.clone(), log_alpha=q.clone(), beta=torch.zeros(B, T, H))


def _noncontig(shape):
    return torch.zeros(shape[:-1] + (2 * shape[-1],))[..., ::2]


def _calls(dev_wrap, q_override=None):
    """(name, thunk) for every binding entry point, with all tensors wrapped by dev_wrap
    and q replaced by q_override(shape) when given."""
    w = dev_wrap
    f = _fwd_args()
    qf = w(q_override((1, 8, 2, 64))) if q_override else w(f["q"])
    z3 = lambda *s: torch.zeros(*s)  # noqa: E731
    q3 = w(q_override((3, 2, 64))) if q_override else w(z3(3, 2, 64))
    pre = dict(a=w(z3(1, 8, 2, 64)), A_log=w(z3(2)), dt_bias=w(z3(2, 64)), b=w(z3(1, 8, 2)))
    return [
        ("chunk_fwd", lambda: kda.chunk_fwd(qf, w(f["k"]), w(f["v"]), w(f["log_alpha"]), w(f["beta"]))),
        ("chunk_fwd_preact", lambda: kda.chunk_fwd_preact(qf, w(f["k"]), w(f["v"]), pre["a"], pre["A_log"],
                                                          pre["dt_bias"], pre["b"])),
        ("recurrent_step", lambda: kda.recurrent_step(q3, w(z3(3, 2, 64)), w(z3(3, 2, 64)), w(z3(3, 2, 64)),
                                                      w(z3(3, 2)), w(z3(3, 2, 64, 64)))),
        ("recurrent_step_preact", lambda: kda.recurrent_step_preact(q3, w(z3(3, 2, 64)), w(z3(3, 2, 64)),
                                                                    w(z3(3, 2, 64)), pre["A_log"], pre["dt_bias"],
                                                                    w(z3(3, 2)), w(z3(3, 2, 64, 64)))),
        ("attn_decode", lambda: kda.attn_decode(q3, w(z3(3, 2, 10, 64)), w(z3(3, 2, 10, 64)))),
        ("chunk_bwd", lambda: kda.chunk_bwd(qf, w(f["k"]), w(f["v"]), w(f["log_alpha"]), w(f["beta"]),
                                            w(z3(1, 8, 2, 64)))),
    ]


@pytest.mark.parametrize("i", range(6))
def test_host_tensors_rejected(i):
    name, call = _calls(lambda t: t)[i]
    with pytest.raises(ValueError, match="device memory"):
        call()


@pytest.mark.parametrize("i", range(6))
def test_noncontiguous_q_rejected(i):
    name, call = _calls(DevT, q_override=_noncontig)[i]
    with pytest.raises(ValueError, match="q must be contiguous"):
        call()
