"""Static checks of the decode kernels' generated gfx950 code (no GPU needed).

Each decode wave copies its activation slice into LDS with direct-to-LDS
loads, then issues a fixed number of packed-tile loads, then waits with
`s_waitcnt vmcnt(N)` until only those N loads can be outstanding: loads
complete in issue order, so the copies have landed.  That is only right if
exactly N vector-memory loads sit between the last copy and the wait, which
depends on the compiler keeping one instruction per tile load in that order.
These tests compile the kernels to assembly and check it, along with the
absence of register spills.
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


def test_tile_loads_match_the_copy_wait(asm):
    funcs = _functions(asm, "_ZN5bqmoe10k_dec_proj")
    funcs.update(_functions(asm, "_ZN5bqmoe18k_dec_down_combine"))
    assert len(funcs) >= 30
    for name, body in funcs.items():
        lines = [l.strip() for l in body.splitlines()]
        lds = [i for i, l in enumerate(lines) if l.startswith("global_load_lds")]
        assert lds, name
        last = max(lds)
        wait = next(i for i in range(last, len(lines)) if l_wait(lines[i]) is not None)
        n = l_wait(lines[wait])
        loads = [l for l in lines[last + 1:wait] if re.match(r"global_load_(?!lds)", l)]
        assert len(loads) == n, (name, len(loads), n)
        # nothing but tile loads between the copies and the wait touches memory
        assert not any(re.match(r"(global|buffer|flat)_(store|atomic)", l)
                       for l in lines[last + 1:wait]), name


def l_wait(line):
    m = re.match(r"s_waitcnt vmcnt\((\d+)\)", line)
    return int(m.group(1)) if m else None


def test_no_scratch(asm):
    meta = asm[asm.index(".amdgpu_metadata"):]
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", meta)
    assert sizes and all(int(s) == 0 for s in sizes)
