"""Static checks of the decode kernels' generated gfx950 code (no GPU needed).

A decode wave fetches each k-block's activation rows, their sums and its
packed tiles into registers one k-block ahead of the matrix-core work, and
writes the rows through a small LDS buffer just before their use.  All of its
waits are placed by the compiler.  Two ways the compiler can quietly undo the
prefetch are checked here: a full `s_waitcnt vmcnt(0)` ahead of loads issued
later in the same straight-line block (the stream drains at every k-block),
and direct-to-LDS loads (whose hazard tracking forces such drains).  Also
checked: no register spills.
"""
import os
import re
import subprocess

import pytest



@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    from bit_quantized_moe_router_amd import build
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "decode.s"
    cmd = build.compile_command("decode.hip", str(out), device_asm=True)
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _functions(text, prefix):
    funcs = {}
    for m in re.finditer(r"^(_ZN5bqmoe\w+):", text, re.M):
        name = m.group(1)
        if not name.startswith(prefix):
            continue
        end = text.index("s_endpgm", m.end())
        funcs[name] = text[m.end():end]
    return funcs


def _blocks(body):
    """Straight-line pieces of a function: split at labels and branches."""
    block = []
    for line in body.splitlines():
        l = line.strip()
        if l.startswith(".LBB") or l.startswith("s_cbranch") or l.startswith("s_branch"):
            if block:
                yield block
            block = []
        elif l and not l.startswith(";"):
            block.append(l)
    if block:
        yield block


def test_no_drain_ahead_of_later_loads(asm):
    funcs = _functions(asm, "_ZN5bqmoe10k_dec_proj")
    funcs.update(_functions(asm, "_ZN5bqmoe18k_dec_down_combine"))
    assert len(funcs) >= 30
    for name, body in funcs.items():
        assert "global_load_lds" not in body, name
        for block in _blocks(body):
            loads = [i for i, l in enumerate(block) if re.match(r"global_load", l)]
            drains = [i for i, l in enumerate(block) if re.match(r"s_waitcnt vmcnt\(0\)", l)]
            if loads and drains:
                assert min(drains) > max(loads), (name, block[min(drains) - 3:min(drains) + 3])


def test_no_scratch(asm):
    meta = asm[asm.index(".amdgpu_metadata"):]
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", meta)
    assert sizes and all(int(s) == 0 for s in sizes)
