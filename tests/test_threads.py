"""The C ABI's thread-safety claim on the host (no GPU): threads create,
query and destroy groups concurrently (the same groups, so they race on the
kernel cache, and different ones), partition bodies and build tree plans;
every call succeeds and gives what a single thread gets.  ctypes releases
the GIL for the duration of each call."""
import threading

import numpy as np
import pytest

from synth import configs

P = pytest.importorskip("elementwise_reduction_groups_amd")


@pytest.fixture(scope="module")
def lib():
    return P.lib()


def _descs():
    eps = configs.f32(1e-5)
    out = []
    for C in (64, 100, 4096):
        out.append(P.GroupDesc(configs.softmax_causal_dag(0.125, C), [((32, C), "f32")], (32, C), "f32"))
        out.append(P.GroupDesc(configs.rmsnorm_gelu_dag(eps), [((8, C), "bf16"), ((8, C), "bf16"), ((C,), "bf16")],
                               (8, C), "bf16"))
    out.append(P.GroupDesc(configs.tree_sgd_dag(), [((1,), "f32"), ((1,), "f32"), ((), "f32")], (1,), "f32",
                           flags=P.PSK_GROUP_TREE))
    return out


def test_concurrent_create_query_destroy(lib):
    descs = _descs()
    want = [P.psk_group_source(d) for d in descs]
    kinds = []
    for d in descs:
        h = P.psk_group_create(d)
        kinds.append(P.psk_group_get_info(h).kind)
        P.psk_group_destroy(h)
    errors = []

    def worker(seed):
        rng = np.random.default_rng(seed)
        try:
            for _ in range(12):
                k = int(rng.integers(len(descs)))
                h = P.psk_group_create(descs[k])
                info = P.psk_group_get_info(h)
                assert info.kind == kinds[k]
                assert P.psk_group_source(descs[k]) == want[k]
                P.psk_group_destroy(h)
                off, cl, cs, cc = P.psk_tree_plan([5, 4097, int(rng.integers(1, 100000))])
                assert off[1] == 5 and int(cc.sum()) == off[-1]
        except Exception as e:          # collected and reported by the main thread
            errors.append(repr(e))

    # groups no thread has compiled yet: every thread creates them at once,
    # racing on the first compile of each
    fresh = [P.GroupDesc(configs.softmax_causal_dag(0.125, 7), [((5, 333 + k), "f32")], (5, 333 + k), "f32")
             for k in range(4)]
    barrier = threading.Barrier(8)
    names = [[None] * len(fresh) for _ in range(8)]

    def racer(t):
        try:
            barrier.wait()
            for k, d in enumerate(fresh):
                h = P.psk_group_create(d)
                names[t][k] = P.psk_group_get_info(h).kernel
                P.psk_group_destroy(h)
        except Exception as e:
            errors.append(repr(e))

    racers = [threading.Thread(target=racer, args=(t,)) for t in range(8)]
    for t in racers:
        t.start()
    for t in racers:
        t.join()
    assert not errors, errors[:3]
    assert all(n == names[0] for n in names)

    threads = [threading.Thread(target=worker, args=(s,)) for s in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
