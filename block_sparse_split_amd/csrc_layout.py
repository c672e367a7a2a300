"""Schedule-image layout constants, read from ``csrc/schedule.h``.

The header is the single source of truth; this module parses its enums and
``constexpr int`` constants so that Python code (tests, diagnostics) can
decode a schedule image without restating the layout.
"""
from __future__ import annotations

import os
import re

_HDR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "schedule.h")


def _parse():
    text = open(_HDR).read()
    consts = {m.group(1): int(m.group(2))
              for m in re.finditer(r"constexpr\s+int(?:32_t)?\s+(\w+)\s*=\s*(\d+)\s*;", text)}
    enums = {}
    for body in re.findall(r"enum\s+\w+\s*:\s*int\s*\{([^}]*)\}", text):
        val = -1
        for tok in body.split(","):
            tok = tok.strip()
            if not tok:
                continue
            if "=" in tok:
                name, v = (s.strip() for s in tok.split("="))
                val = int(v)
            else:
                name = tok
                val += 1
            enums[name] = val
    return consts, enums


_CONSTS, _ENUMS = _parse()

BLOCK = _CONSTS["kBlock"]
TILE_K = _CONSTS["kTileK"]
QTILE = _CONSTS["kQTile"]
KV_GROUP = _CONSTS["kKvGroup"]
H = {k[2:]: v for k, v in _ENUMS.items() if k.startswith("H_") and k != "H_WORDS"}
H_WORDS = _ENUMS["H_WORDS"]
T_WORDS = _ENUMS["T_WORDS"]
I_WORDS = _ENUMS["I_WORDS"]
S_WORDS = _ENUMS["S_WORDS"]
K_WORDS = _ENUMS["K_WORDS"]
# word index of each item field (I_HEAD -> "HEAD", ...)
I = {k[2:]: v for k, v in _ENUMS.items() if k.startswith("I_") and k != "I_WORDS"}
# word index of each dK/dV item field (K_HEAD -> "HEAD", ...)
K = {k[2:]: v for k, v in _ENUMS.items() if k.startswith("K_") and k != "K_WORDS"}
