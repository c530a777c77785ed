"""The ctypes binding rejects mismatched tensors before it calls the C library (CPU only).

The C ABI takes bare pointers, so a float16 output, an int64 offset table, a
non-unit column stride or a short buffer cannot be seen on the C side; the
binding checks each tensor first and raises KattnError(KATTN_EINVAL).  Tensors
here live on the CPU; `OnGpu` wraps one so that it reports itself as a GPU
tensor, which lets the shape and stride checks run.  Every case below is
rejected before any pointer reaches the library.
"""
import numpy as np
import pytest
import torch

from transformer_attention_varlen_amd import kattn

D = 64


class OnGpu:
    """A CPU tensor that answers the binding's questions as a GPU tensor would."""

    def __init__(self, t):
        self.t = t
        self.is_cuda = True
        self.dtype = t.dtype
        self.shape = t.shape

    def data_ptr(self):
        raise AssertionError("the binding passed a pointer on before rejecting the call")

    def dim(self):
        return self.t.dim()

    def stride(self, i=None):
        return self.t.stride() if i is None else self.t.stride(i)

    def is_contiguous(self):
        return self.t.is_contiguous()

    def numel(self):
        return self.t.numel()

    def element_size(self):
        return self.t.element_size()


def g(*shape, dtype=torch.float32):
    return OnGpu(torch.zeros(shape, dtype=dtype))


S, T, H, G = 2, 128, 4, 2


def fwd_args(**kw):
    a = dict(out=g(T, H * D), q=g(T, H * D), k=g(T, G * D), v=g(T, G * D),
             cu=g(S + 1, dtype=torch.int32), workspace=g(4096, dtype=torch.uint8))
    a.update(kw)
    return a


def call_fwd(**kw):
    a = fwd_args(**kw)
    kattn.kattn_varlen_fwd(a["out"], a["q"], a["k"], a["v"], a["cu"], S, T, 91, H, G,
                           workspace=a["workspace"])


@pytest.mark.parametrize("kw,what", [
    (dict(out=g(T, H * D, dtype=torch.float16)), "out must be float32"),
    (dict(q=g(T, H * D, dtype=torch.float64)), "q must be float32"),
    (dict(cu=g(S + 1, dtype=torch.int64)), "cu must be int32"),
    (dict(cu=g(S, dtype=torch.int32)), "cu has 2 elements"),
    (dict(q=OnGpu(torch.zeros(T, 2 * H * D)[:, ::2])), "unit column stride"),
    (dict(k=g(T - 1, G * D)), "needs at least"),
    (dict(v=g(T, G * D - 4)), "needs at least"),
    (dict(out=torch.zeros(T, H * D)), "out must be on the GPU"),
    (dict(workspace=torch.zeros(4096, dtype=torch.uint8)), "workspace must be"),
    (dict(q=g(T * H * D)), "2-D"),
])
def test_varlen_fwd_rejects_mismatched_tensors(kw, what):
    with pytest.raises(kattn.KattnError) as e:
        call_fwd(**kw)
    assert e.value.code == kattn.KATTN_EINVAL
    assert what in str(e.value)


def test_f16_output_must_be_half():
    a = fwd_args()
    with pytest.raises(kattn.KattnError, match="out must be float16"):
        kattn.kattn_varlen_fwd_f16(a["out"], a["q"], a["k"], a["v"], a["cu"], S, T, 91, H, G,
                                   workspace=a["workspace"])


@pytest.mark.parametrize("cos,sin,what", [
    (g(91 * 32), g(91 * 32), "contiguous [len, 32] table"),
    (g(91, 32), None, "cos and sin must both be given"),
    (g(91, 32), g(90, 32), "different lengths"),
    (g(91, 32, dtype=torch.float64), g(91, 32), "cos must be float32"),
])
def test_rope_tables_must_be_len_by_32(cos, sin, what):
    a = fwd_args()
    with pytest.raises(kattn.KattnError) as e:
        kattn.kattn_varlen_fwd_rope(a["out"], a["q"], a["k"], a["v"], a["cu"], S, T, 91, H, G,
                                    cos, sin, workspace=a["workspace"])
    assert what in str(e.value)


B, CAP = 3, 100


def dec_args(**kw):
    a = dict(out=g(B, H * D), q=g(B, H * D), k_new=g(B, G * D), v_new=g(B, G * D),
             k_cache=g(B, G, CAP, D), v_cache=g(B, G, CAP, D),
             used=g(B, dtype=torch.int32), workspace=g(4096, dtype=torch.uint8))
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,what", [
    (dict(q=OnGpu(torch.zeros(B, H * D + 4)[:, :H * D])), "exactly 256 floats"),
    (dict(k_cache=g(B, G, CAP + 1, D)), "k_cache must be a contiguous tensor of shape"),
    (dict(v_cache=OnGpu(torch.zeros(B, CAP, G, D).transpose(1, 2))), "v_cache must be"),
    (dict(used=g(B, dtype=torch.int64)), "used must be int32"),
    (dict(used=g(B - 1, dtype=torch.int32)), "used has 2 elements"),
    (dict(out=g(B, H * D, dtype=torch.float16)), "out must be float32"),
])
def test_decode_rejects_mismatched_tensors(kw, what):
    a = dec_args(**kw)
    with pytest.raises(kattn.KattnError) as e:
        kattn.kattn_decode(a["out"], a["q"], a["k_new"], a["v_new"], a["k_cache"],
                           a["v_cache"], CAP, a["used"], CAP, B, H, G, workspace=a["workspace"])
    assert e.value.code == kattn.KATTN_EINVAL
    assert what in str(e.value)


def test_prefill_cached_rejects_an_int64_offset_table():
    a = fwd_args()
    with pytest.raises(kattn.KattnError, match="offset must be int32"):
        kattn.kattn_prefill_cached(a["out"], a["q"], a["k"], a["v"], a["cu"],
                                   g(S, dtype=torch.int64), S, T, 91, 91, g(S, G, 200, D),
                                   g(S, G, 200, D), 200, H, G, workspace=a["workspace"])


def test_rope_prologue_rejects_a_short_position_table():
    with pytest.raises(kattn.KattnError, match="pos has 10 elements"):
        kattn.kattn_rope_prologue(g(T, H * D), H, g(T, G * D), G, g(10, dtype=torch.int32),
                                  g(91, 32), g(91, 32), T=T)


def test_numpy_arrays_are_not_device_tensors():
    a = fwd_args(q=np.zeros((T, H * D), np.float32))
    with pytest.raises(kattn.KattnError, match="q must be a torch tensor"):
        call_fwd(**a)
