"""The gfx950 assembly of the payload kernels, checked on the host (no GPU).

The streaming store is written out in an asm statement (the compiler emits no
store with the write-through policy from C++), so the compiler cannot see it
as a store when it places wait states. A vector store of 128 bits needs two
wait states on gfx950 before a VALU instruction may overwrite its data
registers; the asm statement carries them (`s_nop 1`). With one, a GPU test
saw the next loop index stored in place of the data. This test compiles both libraries' device code to
assembly with the build's own flags and checks that every such store is
followed by its wait state, and that the payload kernels do use it.
"""
import os
import re
import subprocess

import pytest

from combine_ep_prepare_amd import _build

STREAM_STORE = re.compile(r"^\s*global_store_dwordx4\s.*\bsc0 sc1 nt\b")


def _device_asm(source: str, out_dir: str) -> list:
    out = os.path.join(out_dir, os.path.basename(source) + ".s")
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [_build.hipcc(), *flags, "--cuda-device-only", "-S", "-I",
           os.path.join(_build.ROOT, "include"), "-I", _build.CSRC, "-o", out, source]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return f.read().splitlines()


def _instructions(lines):
    """Instruction lines only: no comments, labels, directives or asm markers."""
    for ln in lines:
        s = ln.split(";")[0].strip()
        if not s or s.endswith(":") or s.startswith("."):
            continue
        yield s


@pytest.mark.parametrize("source,kernels", [
    ("ep_kernels.hip", ("run_rows_kernel", "scatter_rows_kernel", "reduce_rows_kernel",
                        "weighted_bwd_kernel")),
    ("ep_ceilings.hip", ("write_linear_kernel", "write_rows_kernel", "copy_linear_kernel",
                         "gather_sum_kernel")),
])
def test_stream_stores_carry_their_wait_state(tmp_path, source, kernels):
    lines = _device_asm(os.path.join(_build.CSRC, source), str(tmp_path))
    ins = list(_instructions(lines))
    stores = [i for i, s in enumerate(ins) if STREAM_STORE.match(s)]
    assert stores, "no write-through store emitted"
    for i in stores:
        assert i + 1 < len(ins) and ins[i + 1] == "s_nop 1", \
            f"store without its wait state: {ins[i]!r} then {ins[i + 1:i + 2]!r}"
    # each payload kernel's body holds at least one such store
    text = "\n".join(lines)
    for k in kernels:
        bodies = re.findall(r"^(_Z\S*" + k + r"\S*):[^\n]*\n(.*?)^\.Lfunc_end", text,
                            flags=re.M | re.S)
        assert bodies, f"{k} not found"
        for name, body in bodies:
            assert any(STREAM_STORE.match(b) for b in body.splitlines()), \
                f"{name}: no write-through store"
