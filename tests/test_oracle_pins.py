"""The fp64 oracle against its pins, and planted mistakes against the pins (CPU only)."""
import os
import re

import pytest

import oracle
import oracle_pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(lib, check):
    check(lib)


# Plausible mistakes planted in a private copy of the oracle source.  Every one
# must make at least one pin fail.
MUTANTS = {
    "window_one_short": ("? L - j->window : 0;", "? L - j->window + 1 : 0;"),
    "window_one_long": ("? L - j->window : 0;", "? L - j->window - 1 : 0;"),
    "kv_head_modulo": ("const int g = h / G;", "const int g = h % j->KV;"),
    "softmax_sign": ("z[i] = exp(z[i] - m);", "z[i] = exp(m - z[i]);"),
    "dropped_normaliser": ("for (int d = 0; d < D; ++d) out[d] /= l;", ""),
    "kv_layout_transposed": ("return (((int64_t)b * j->cap + s) * j->KV + g) * (int64_t)j->D;",
                             "return (((int64_t)b * j->KV + g) * j->cap + s) * (int64_t)j->D;"),
    "page_slot_reversed": ("(int64_t)page * ORC_PAGE + s % ORC_PAGE",
                           "(int64_t)page * ORC_PAGE + (ORC_PAGE - 1 - s % ORC_PAGE)"),
    "block_table_stride": ("(int64_t)b * j->max_pages + s / ORC_PAGE",
                           "(int64_t)b * (j->max_pages - 1) + s / ORC_PAGE"),
    "bf16_widening_rounded": ("[idx] << 16;", "[idx] << 16 | 0x8000u;"),
    "scaled_logits": ("z[s - lo] = acc;", "z[s - lo] = acc / sqrt((double)D);"),
    "query_head_of_group": ("((size_t)b * ORC_HEADS + h) * (size_t)D",
                            "((size_t)b * ORC_HEADS + g) * (size_t)D"),
    "length_one_short": ("const int64_t L = j->seq_lens[b];",
                         "const int64_t L = j->seq_lens[b] - 1;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = oracle.build(str(path), str(tmp_path / f"libmutant_{name}.so"))
    mlib = oracle.load(so)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mlib)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(e).__name__))
            break
    assert caught, f"planted mistake {name} passed every pin"


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (x.strip() for x in line.split("=", 1))
                vals[k] = int(v)
    return vals


def test_model_constants_match_pages():
    g = _golden("model_constants.txt")
    assert oracle.HEADS == g["heads"] and oracle.PAGE == g["page_size"]
    assert oracle.VARIANTS["sliding"] == (g["sliding.kv_heads"], g["sliding.head_dim"],
                                          g["sliding.window"])
    assert oracle.VARIANTS["global"][:2] == (g["global.kv_heads"], g["global.head_dim"])
    assert g["scale_num"] == g["scale_den"] == 1
    src = open(oracle.SOURCE).read()
    assert re.search(r"#define ORC_HEADS %d\b" % g["heads"], src)
    assert re.search(r"#define ORC_PAGE %d\b" % g["page_size"], src)
