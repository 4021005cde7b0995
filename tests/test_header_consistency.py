"""The oracle carries its own copies of the public header's enumeration
numbers (the two share no header); check that they agree. No GPU."""
import re
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]


def _defines(path):
    out = {}
    for m in re.finditer(r"#define\s+(\w+)\s+\(?(-?\d+)\)?", path.read_text()):
        out[m.group(1)] = int(m.group(2))
    return out


def test_oracle_enums_match_public_header():
    pub = _defines(ROOT / "include" / "kvq.h")
    orc = _defines(ROOT / "oracle" / "kvq_oracle.h")
    pairs = {
        "KVQ_F16": "ORC_F16", "KVQ_BF16": "ORC_BF16", "KVQ_F32": "ORC_F32",
        "KVQ_CODE_NONE16": "ORC_CODE_NONE16", "KVQ_CODE_INT8": "ORC_CODE_INT8",
        "KVQ_CODE_FP8_E4M3": "ORC_CODE_FP8", "KVQ_CODE_INT4": "ORC_CODE_INT4",
        "KVQ_SCALE_TOKEN_SYM": "ORC_TOKEN_SYM",
        "KVQ_SCALE_GROUP_ASYM": "ORC_GROUP_ASYM",
        "KVQ_SCALE_CHANNEL_BLOCK_SYM": "ORC_CHANNEL_BLOCK",
        "KVQ_OK": "ORC_OK", "KVQ_ERR_INVALID_ARGUMENT": "ORC_ERR_INVALID",
        "KVQ_ERR_UNSUPPORTED": "ORC_ERR_UNSUPPORTED",
        "KVQ_ERR_OUT_OF_BLOCKS": "ORC_ERR_OUT_OF_BLOCKS",
    }
    for a, b in pairs.items():
        assert pub[a] == orc[b], (a, b)


def test_oracle_does_not_include_library_sources():
    src = (ROOT / "oracle" / "kvq_oracle.c").read_text()
    for inc in re.findall(r'#include\s+[<"]([^>"]+)[>"]', src):
        assert inc in ("kvq_oracle.h", "math.h", "pthread.h", "stdlib.h",
                       "string.h"), inc
