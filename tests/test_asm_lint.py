"""Inline asm in the HIP sources: a block that issues memory loads must mark
every output early-clobber ("=&v").

Without it the compiler may give an output the register of an input that is
dead after the block, typically the address register: a load that returns
while a later load of the same block is still to be issued then overwrites
the address that load uses, and the later loads read wrong data (seen as
wrong, run-dependent backward gradients before this rule).  A plain CPU
check on the sources."""
import pathlib
import re

CSRC = pathlib.Path(__file__).resolve().parents[1] / "block_sparse_long_mean_amd" / "csrc"
LOADS = re.compile(r"\b(ds_read\w*|global_load\w*|buffer_load\w*|flat_load\w*|s_load\w*)")


def _asm_blocks(text):
    for m in re.finditer(r"asm\s+volatile\s*\(", text):
        depth, i = 1, m.end()
        while depth:
            depth += {"(": 1, ")": -1}.get(text[i], 0)
            i += 1
        yield text.count("\n", 0, m.start()) + 1, text[m.end():i - 1]


def _outputs(body):
    # the operand lists follow the template strings: template : outputs : inputs : clobbers
    parts, depth, cur, in_str = [], 0, "", False
    for ch in body:
        if ch == '"' and not cur.endswith("\\"):
            in_str = not in_str
        if not in_str and depth == 0 and ch == ":":
            parts.append(cur)
            cur = ""
            continue
        if not in_str:
            depth += {"(": 1, ")": -1}.get(ch, 0)
        cur += ch
    parts.append(cur)
    return parts[1] if len(parts) > 1 else ""


def test_asm_loads_use_early_clobber_outputs():
    checked = 0
    for f in sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.h")):
        for line, body in _asm_blocks(f.read_text()):
            template = body.split(":")[0]
            if not LOADS.search(template):
                continue
            checked += 1
            outs = re.findall(r'"(=[^"]*)"', _outputs(body))
            bad = [o for o in outs if "&" not in o]
            assert not bad, f"{f.name}:{line}: load asm outputs {bad} must be early-clobber (=&v)"
    assert checked >= 5, "expected the kernels' LDS read blocks"
