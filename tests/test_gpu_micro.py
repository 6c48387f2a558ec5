"""The measurement microbenchmarks run through the C ABI and return plausible figures."""
import pytest

import persistent_megakernel_decode_cu_amd as mk

pytestmark = pytest.mark.gpu


def test_launch_latency():
    us_stream, us_graph = mk.mkm_launch_latency(500)
    print(us_stream, us_graph)
    assert 0.0 < us_stream < 1000.0 and 0.0 < us_graph < 1000.0


@pytest.mark.parametrize("same", [False, True])
def test_dependency_hop(same):
    ns, xa, xb = mk.mkm_pingpong(2000, same_xcd=same)
    print(ns, xa, xb)
    assert 0.0 < ns < 100000.0
    assert (xa == xb) == same


def test_barrier_lds_fill_and_stream_read():
    ns = mk.mkm_barrier(10000)
    one = mk.mkm_lds_fill(16 << 20, 1, 8)
    all_ = mk.mkm_lds_fill(4 << 20, 256, 8)
    rd = mk.mkm_stream_read(1 << 30)
    print(ns, one, all_, rd)
    assert 0.0 < ns < 100000.0
    assert 1.0 < one < all_
    assert rd > 100.0


def test_arguments_out_of_range_are_rejected():
    with pytest.raises(mk.MkError):
        mk.mkm_launch_latency(0)
    with pytest.raises(mk.MkError):
        mk.mkm_lds_fill(1000, 4, 8)
    with pytest.raises(mk.MkError):
        mk.mkm_lds_fill(1 << 20, 4, 5)
