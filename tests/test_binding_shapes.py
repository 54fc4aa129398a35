"""The Python binding's shape checks (CPU only).

The C ABI receives bare pointers and sizes taken from q and v, so a shorter k/v/g tensor or
a smaller caller-supplied output would be read or written past its end on the device.  The
binding therefore checks every operand's shape before it calls the library; these tests
feed it wrong shapes (plain numpy arrays: the checks read only ``.shape``).
"""
import numpy as np
import pytest

from linear_attention_recurrence_gated_amd.gdn import check_norm_shapes, check_shapes

T, HK, HV, D = 40, 4, 12, 128


def _ok():
    return dict(q=np.zeros((T, HK, D)), k=np.zeros((T, HK, D)), v=np.zeros((T, HV, D)),
                g=np.zeros((T, HV)), beta=np.zeros((T, HV)), state_in=np.zeros((HV, D, D)),
                state_out=np.zeros((HV, D, D)), o=np.zeros((T, HV, D)),
                z=np.zeros((T, HV, D)), w=np.zeros((HV, D)), y=np.zeros((T, HV, D)))


def test_consistent_shapes_pass():
    assert check_shapes(**_ok()) == (T, HK, HV, D, D)
    a = _ok()
    assert check_shapes(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"]) == \
        (T, HK, HV, D, D)


@pytest.mark.parametrize("name,shape", [
    ("k", (T - 1, HK, D)),           # shorter key rows
    ("k", (T, HK + 1, D)),
    ("v", (T - 1, HV, D)),           # v shorter than q in T
    ("g", (T - 1, HV)),
    ("g", (T, HV + 1)),
    ("beta", (T, HV - 1)),
    ("state_in", (HV - 1, D, D)),
    ("state_in", (HV, D, D - 1)),
    ("state_out", (HV - 1, D, D)),   # caller-supplied outputs too small
    ("o", (T - 1, HV, D)),
    ("o", (T, HV, D - 4)),
    ("z", (T, HV - 1, D)),
    ("w", (HV, D - 1)),
    ("w", (D,)),
    ("y", (T - 1, HV, D)),
])
def test_wrong_shape_raises(name, shape):
    a = _ok()
    a[name] = np.zeros(shape)
    with pytest.raises(ValueError, match=name):
        check_shapes(**a)


def test_rank_of_q_and_v():
    a = _ok()
    a["q"] = np.zeros((T, HK * D))
    with pytest.raises(ValueError):
        check_shapes(**a)


def test_norm_shapes():
    o = np.zeros((T, HV, D))
    assert check_norm_shapes(o, np.zeros((T, HV, D)), np.zeros((HV, D))) == (T, HV, D)
    with pytest.raises(ValueError, match="z"):
        check_norm_shapes(o, np.zeros((T - 1, HV, D)), np.zeros((HV, D)))
    with pytest.raises(ValueError, match="w"):
        check_norm_shapes(o, np.zeros((T, HV, D)), np.zeros((HV - 1, D)))
    with pytest.raises(ValueError, match="y"):
        check_norm_shapes(o, np.zeros((T, HV, D)), np.zeros((HV, D)), np.zeros((T, HV, 64)))
    with pytest.raises(ValueError):
        check_norm_shapes(np.zeros((T * HV, D)), np.zeros((T, HV, D)), np.zeros((HV, D)))
