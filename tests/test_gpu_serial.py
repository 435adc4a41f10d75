"""Record a launch, rebuild it from its YAML files and replay it on the GPU:
the replay's outputs equal the recorded launch's bit for bit and the
oracle's."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import compare, dev, host, run_oracle, to_dev
from random_commands import random_view_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", [0, 3, 7, 11])
def test_record_and_replay_random_views(tmp_path, seed):
    import elementwise_tensor_commands_amd as E
    from elementwise_tensor_commands_amd import replay
    spec, ins, outs = random_view_case(seed)
    vals = [x[0] if isinstance(x, tuple) else x for x in ins]
    host_outs = [st.copy() for _, st in outs]
    ref_views = []
    for (v, st), c in zip(outs, host_outs):
        off, strides = W.layout(v, st)
        ref_views.append(np.lib.stride_tricks.as_strided(c.reshape(-1)[off:], v.shape,
                                                         tuple(s * c.itemsize for s in strides)))
    run_oracle(spec, vals, outputs=ref_views)
    gin = []
    for x in ins:
        if isinstance(x, tuple):
            off, strides = W.layout(*x)
            gin.append(to_dev(np.ascontiguousarray(x[1]).reshape(-1)).as_strided(x[0].shape, strides, off))
        else:
            gin.append(x)
    gout, flats = [], []
    for v, st in outs:
        off, strides = W.layout(v, st)
        f = to_dev(np.ascontiguousarray(st).reshape(-1))
        flats.append(f)
        gout.append(f.as_strided(v.shape, strides, off))
    cmd = E.from_spec(spec)
    d = str(tmp_path / "rec")
    replay.record(cmd, gin + gout, d, launch=True)
    for f, r in zip(flats, host_outs):
        compare(host(f), r.reshape(-1), 0, "recorded launch seed %d" % seed)
    # replay from the files alone
    _, storages = replay.replay(d)
    assert replay.main([d]) == 0
    n_in_storages = len(storages) - len(outs)
    for k, r in enumerate(host_outs):
        # output storages follow the input ones (one storage per distinct tensor)
        compare(host(storages[n_in_storages + k]), r.reshape(-1), 0, "replay seed %d out%d" % (seed, k))


def test_replay_in_place_bf16(tmp_path):
    from elementwise_tensor_commands_amd import replay
    import elementwise_tensor_commands_amd as E
    vals, extra = W.make_inputs("axpby_bf16", 4099)
    ref = run_oracle(W.AXPBY_BF16, vals)[0]
    x, y = to_dev(vals[0]), to_dev(vals[1])
    cmd = E.from_spec(W.AXPBY_BF16)
    d = str(tmp_path / "inplace")
    replay.record(cmd, [x, y, vals[2], vals[3], y], d, launch=True)     # out is y itself
    compare(host(y), ref, 0, "in place")
    _, storages = replay.replay(d)
    assert len(storages) == 2
    compare(host(storages[1]), ref, 0, "replayed in place")
