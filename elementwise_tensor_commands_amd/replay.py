"""Record one launch of a Command to a directory and replay it later.

A debugging aid built on the Command's YAML form (rocRoller "Design
Overview", section "Serialization": serialised Commands serve debugging and
inspection).  ``record`` writes

    command.yaml     the Command (cmd_to_yaml)
    program.yaml     its lowered program (cmd_program_yaml)
    arguments.yaml   one entry per CommandArgument: scalars with their bit
                     pattern; tensors with dtype, shape, strides, element offset
                     and the storage file they view
    storage<k>.npy   every distinct storage the tensors view, whole, as it was
                     before the launch (bfloat16 as uint16 bit patterns)
    outputs/         with ``launch=True``: the storages after the launch

and ``replay`` rebuilds the Command from command.yaml, uploads the storages,
recreates every view (aliasing between arguments included) and launches it.
Nothing here computes anything: values go to the GPU library as they are.

    python -m elementwise_tensor_commands_amd.replay DIR    replay DIR and
        compare the outputs with DIR/outputs bit for bit
"""
from __future__ import annotations

import os
import struct
import sys

import numpy as np

from . import ARG_SCALAR, BF16, DTYPE_NAMES, DTYPES, F16, F32, I32, Command, scalar_bits


def _storage_of(t):
    """The whole storage a tensor views, as a flat tensor of its dtype."""
    import torch
    st = t.untyped_storage()
    n = st.nbytes() // t.element_size()
    flat = torch.empty(0, dtype=t.dtype, device=t.device)
    flat.set_(st, 0, (n,), (1,))
    return flat


def _to_numpy(flat):
    import torch
    if flat.dtype == torch.bfloat16:
        return flat.view(torch.int16).cpu().numpy().view(np.uint16)
    return flat.cpu().numpy()


def _from_numpy(a, dtype_code, device):
    import torch
    if dtype_code == BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def _scalar_from_bits(bits: int, dtype_code: int):
    if dtype_code == F32:
        return struct.unpack("<f", struct.pack("<I", bits))[0]
    if dtype_code == I32:
        return struct.unpack("<i", struct.pack("<I", bits))[0]
    if dtype_code == F16:
        return np.uint16(bits).view(np.float16)
    return np.uint16(bits)                      # bfloat16: bit pattern


def record(cmd: Command, values, directory: str, launch: bool = False, stream=None):
    """Write the Command and its argument values (in declaration order, as for
    ``cmd.launch``) to ``directory``; with ``launch`` also launch it, wait, and
    save the storages afterwards under ``outputs/``."""
    import yaml
    os.makedirs(directory, exist_ok=True)
    if len(values) != len(cmd.arg_kinds):
        raise ValueError("expected %d argument values, got %d" % (len(cmd.arg_kinds), len(values)))
    with open(os.path.join(directory, "command.yaml"), "w") as f:
        f.write(cmd.to_yaml())
    storages, keys, entries = [], {}, []
    for i, (v, (kind, dt, rank)) in enumerate(zip(values, cmd.arg_kinds)):
        if kind == ARG_SCALAR:
            entries.append({"index": i, "kind": "scalar", "dtype": DTYPE_NAMES[dt], "bits": scalar_bits(v, dt)})
            continue
        key = (v.untyped_storage().data_ptr(), str(v.device))
        if key not in keys:
            keys[key] = len(storages)
            storages.append(_storage_of(v))
        entries.append({"index": i, "kind": "tensor", "dtype": DTYPE_NAMES.get(_dtype_code(v), "?"),
                        "shape": list(v.shape), "strides": list(v.stride()), "offset": int(v.storage_offset()),
                        "storage": keys[key]})
    for k, flat in enumerate(storages):
        np.save(os.path.join(directory, "storage%d.npy" % k), _to_numpy(flat))
    with open(os.path.join(directory, "arguments.yaml"), "w") as f:
        yaml.safe_dump({"ecmd_arguments": 1, "storages": len(storages), "arguments": entries}, f,
                       default_flow_style=None, sort_keys=False)
    with open(os.path.join(directory, "program.yaml"), "w") as f:
        f.write(cmd.program_yaml())
    if launch:
        import torch
        cmd.launch(*values, stream=stream)
        torch.cuda.synchronize()
        os.makedirs(os.path.join(directory, "outputs"), exist_ok=True)
        for k, flat in enumerate(storages):
            np.save(os.path.join(directory, "outputs", "storage%d.npy" % k), _to_numpy(flat))


def _dtype_code(t) -> int:
    from . import _torch_dtype_code
    return _torch_dtype_code(t)


def load(directory: str, device="cuda"):
    """(Command, argument values, storages) rebuilt from a recording."""
    import yaml
    with open(os.path.join(directory, "command.yaml")) as f:
        cmd = Command.from_yaml(f.read())
    with open(os.path.join(directory, "arguments.yaml")) as f:
        meta = yaml.safe_load(f)
    if meta.get("ecmd_arguments") != 1:
        raise ValueError("not an argument recording")
    dts = {}
    for e in meta["arguments"]:
        if e["kind"] == "tensor":
            dts[e["storage"]] = DTYPES[e["dtype"]]
    storages = [_from_numpy(np.load(os.path.join(directory, "storage%d.npy" % k)), dts.get(k, 0), device)
                for k in range(meta["storages"])]
    values = []
    for e in meta["arguments"]:
        if e["kind"] == "scalar":
            values.append(_scalar_from_bits(int(e["bits"]), DTYPES[e["dtype"]]))
        else:
            values.append(storages[e["storage"]].as_strided(e["shape"], e["strides"], e["offset"]))
    return cmd, values, storages


def replay(directory: str, device="cuda", stream=None):
    """Rebuild and launch a recorded Command; returns (values, storages) after
    the launch has finished."""
    import torch
    cmd, values, storages = load(directory, device)
    cmd.launch(*values, stream=stream)
    torch.cuda.synchronize()
    return values, storages


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    if len(argv) != 1:
        print(__doc__)
        return 2
    directory = argv[0]
    _, storages = replay(directory)
    out = os.path.join(directory, "outputs")
    if not os.path.isdir(out):
        print("replayed %s (no recorded outputs to compare)" % directory)
        return 0
    bad = 0
    for k, flat in enumerate(storages):
        got = _to_numpy(flat)
        want = np.load(os.path.join(out, "storage%d.npy" % k))
        n = int(np.count_nonzero(got.view(np.uint8) != want.view(np.uint8)))
        print("storage%d: %s" % (k, "identical" if n == 0 else "%d bytes differ" % n))
        bad += n
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
