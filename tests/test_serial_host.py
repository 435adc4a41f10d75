"""Commands to and from YAML, the lowered program's YAML and hash, and the
launch recorder (host only; replay itself runs on the GPU tests).

rocRoller serialises its Command for debugging and caching (rocRoller "Design
Overview", section "Serialization"); the document layout here is the
library's own (see cmd_to_yaml in include/ecmd.h)."""
import numpy as np
import pytest
import torch
import yaml

import elementwise_tensor_commands_amd as E
import workloads as W
from random_commands import _random_spec
from specs import SPECS


def _round_trip(c):
    text = c.to_yaml()
    c2 = E.Command.from_yaml(text)
    assert c2.to_yaml() == text
    assert c2.arg_kinds == c.arg_kinds
    return c2


@pytest.mark.parametrize("name", sorted(SPECS) + ["batched_transpose", "bias_nchw"])
def test_round_trip_of_every_spec(name):
    spec = SPECS[name] if name in SPECS else W.WORKLOADS[name]["spec"]
    c = E.from_spec(spec)
    c2 = _round_trip(c)
    assert c2.program_hash() == c.program_hash()
    assert c2.dump() == c.dump()
    assert c2.program_yaml() == c.program_yaml()


@pytest.mark.parametrize("seed", range(60))
def test_round_trip_of_random_commands(seed):
    rng = np.random.default_rng(7000 + seed)
    spec = _random_spec(rng, int(rng.integers(1, 5)), int(rng.integers(1, 20)), int(rng.integers(1, 5)))
    c = E.from_spec(spec)
    c2 = _round_trip(c)
    try:
        h = c.program_hash()
    except E.Error as e:                 # more live values than registers: both refuse alike
        with pytest.raises(E.Error) as e2:
            c2.program_hash()
        assert e2.value.name == e.name
        return
    assert c2.program_hash() == h and c2.dump() == c.dump()


def test_document_is_plain_yaml():
    """An independent YAML parser reads the document into the structure the
    header describes."""
    c = E.from_spec(W.MIXED_TWO_OUT)
    d = yaml.safe_load(c.to_yaml())
    assert d["ecmd_command"] == 1
    assert [a["role"] for a in d["arguments"]] == ["load"] * 4 + ["store"] * 2
    assert [a["dtype"] for a in d["arguments"]] == ["f16", "f16", "f16", "f32", "f16", "f32"]
    assert [o["tag"] for o in d["operations"]] == list(range(13))
    ops = [o["op"] for o in d["operations"]]
    assert ops == ["load"] * 3 + ["scalar"] + ["cvt"] * 3 + ["mul", "add", "sub", "mul", "cvt", "add"]
    assert d["stores"] == [{"tag": 11, "arg": 4}, {"tag": 12, "arg": 5}]
    p = yaml.safe_load(c.program_yaml())
    assert p["ecmd_program"] == 1 and isinstance(p["hash"], int)
    assert len(p["inputs"]) == 3 and len(p["uniforms"]) == 1 and len(p["outputs"]) == 2
    assert len(p["operations"]) == 9             # t = x*y once; fp32(u+s) needs no conversion
    assert sum(o["code"] == "mul.f32" for o in p["operations"]) == 2


def test_interleaved_stores_keep_argument_order():
    c = E.Command()
    x = c.load("f32")
    c.store(c.neg(x))                  # argument 1 is a store between two loads
    y = c.load("bf16", 3)
    s = c.scalar("i32")
    c.store(c.mul(y, y), 3)
    c.store(c.cmp("gtu", s, s))
    c2 = _round_trip(c)
    assert [k for k, _, _ in c2.arg_kinds] == [E.ARG_TENSOR, E.ARG_TENSOR, E.ARG_TENSOR, E.ARG_SCALAR,
                                              E.ARG_TENSOR, E.ARG_TENSOR]


def test_hand_written_document_with_comments():
    text = """
# out = x * 2 (scalar) ; the comment and blank lines are ignored
ecmd_command: 1

arguments:
  - {index: 0, kind: tensor, dtype: f32, rank: 2, role: load, tag: 0}
  - {index: 1, kind: scalar, dtype: f32, role: load, tag: 1}
  - {index: 2, kind: tensor, dtype: f32, rank: 2, role: store, tag: 2}
operations:
  - {tag: 0, op: load, dtype: f32, arg: 0}   # x
  - {tag: 1, op: scalar, dtype: f32, arg: 1}
  - {tag: 2, op: mul, dtype: f32, a: 0, b: 1}
stores:
  - {tag: 2, arg: 2}
"""
    c = E.Command.from_yaml(text)
    ref = E.Command()
    x = ref.load("f32", 2)
    s = ref.scalar("f32")
    ref.store(ref.mul(x, s), 2)
    assert c.to_yaml() == ref.to_yaml() and c.program_hash() == ref.program_hash()


def _bad(text, name, where):
    with pytest.raises(E.Error) as e:
        E.Command.from_yaml(text)
    assert e.value.name == name, str(e.value)
    assert where in str(e.value), str(e.value)


def test_malformed_documents_are_refused():
    good = E.from_spec(W.ADD_F32).to_yaml()
    _bad(good.replace("ecmd_command: 1", "ecmd_command: 2"), "CMD_E_ARG", "version")
    _bad(good.replace("arguments:", "args:"), "CMD_E_ARG", "line 2")
    _bad(good.replace("op: add", "op: plus"), "CMD_E_ARG", "unknown operation")
    _bad(good.replace("{tag: 2, op: add", "{tag: 5, op: add"), "CMD_E_ARG", "tags")
    _bad(good.replace("a: 0, b: 1", "a: 0, b: 1, d: 3"), "CMD_E_ARG", "field")
    _bad(good.replace("{tag: 2, arg: 2}", "{tag: 2, arg: 7}"), "CMD_E_ARG", "store")
    _bad(good.replace("- {tag: 0, op: load, dtype: f32, arg: 0}", "- {tag: 0, op: load, dtype: f32, arg: 0"),
         "CMD_E_ARG", "malformed")
    _bad(good.replace("dtype: f32, a: 0", "dtype: i32, a: 0"), "CMD_E_DTYPE", "building")
    _bad(good.replace("a: 0, b: 1", "a: 0, b: 2"), "CMD_E_TAG", "building")
    _bad(good.replace("{index: 1, kind: tensor, dtype: f32", "{index: 1, kind: tensor, dtype: i32"),
         "CMD_E_ARG", "declaration")
    _bad("", "CMD_E_ARG", "version")


def test_program_hash_identifies_programs():
    def build(order):
        c = E.Command()
        x, y = c.load("f32"), c.load("f32")
        c.store(c.add(x, y) if order else c.add(y, x))
        return c
    assert build(True).program_hash() == build(False).program_hash()      # x+y and y+x lower alike
    hashes = {E.from_spec(SPECS[n]).program_hash() for n in ("add_f32", "sub_f32", "mul_f32", "add_f16",
                                                              "add_bf16", "add_i32")}
    assert len(hashes) == 6


def test_record_writes_a_replayable_description(tmp_path):
    """record() on host tensors (no launch): the files describe every
    argument, share storages between aliased views and keep the bytes."""
    from elementwise_tensor_commands_amd import replay
    c = E.from_spec(W.AXPBY_BF16)
    x = torch.arange(12, dtype=torch.float32).to(torch.bfloat16)
    big = torch.zeros(40, dtype=torch.bfloat16)
    y = big[4:16]
    replay.record(c, [x, y, np.uint16(0x3FC0), np.uint16(0xBE80), y], str(tmp_path))
    meta = yaml.safe_load(open(tmp_path / "arguments.yaml"))
    assert meta["storages"] == 2
    a = meta["arguments"]
    assert a[1]["storage"] == a[4]["storage"] and a[1]["offset"] == 4      # in place: one storage
    assert a[2] == {"index": 2, "kind": "scalar", "dtype": "bf16", "bits": 0x3FC0}
    s0 = np.load(tmp_path / "storage0.npy")
    assert s0.dtype == np.uint16 and np.array_equal(s0, x.view(torch.int16).numpy().view(np.uint16))
    c2, values, _ = replay.load(str(tmp_path), device="cpu")
    assert c2.to_yaml() == c.to_yaml()
    assert values[1].data_ptr() == values[4].data_ptr() and values[1].stride() == (1,)
