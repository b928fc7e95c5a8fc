"""Plant plausible mistakes in copies of the oracle and check that the pins catch each one.

Every mutation is a textual edit of the oracle's C source compiled into a
separate library under a temporary directory; the real oracle is untouched.
A mutation survives only if every pin still passes, which fails the test.
"""

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTATIONS = [
    ("nibble order swapped", "((c & 1) * 4)", "((1 - (c & 1)) * 4)"),
    ("neighbouring scale group", "T_E4M3[scales[c / ORC_G]]", "T_E4M3[scales[(c / ORC_G) ^ 1]]"),
    ("E2M1 exponent bias", "ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    ("E2M1 sign dropped", "double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);\n  return s ? -v : v;",
     "double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);\n  return v;"),
    ("E4M3 exponent bias", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("E4M3 subnormal scale", "ldexp(m / 8.0, -6)", "ldexp(m / 8.0, -7)"),
    ("ReLU dropped", "(dot > 0.0 ? dot : 0.0)", "dot"),
    ("head weight dropped", "I += wq[h] * (dot > 0.0 ? dot : 0.0);", "I += (dot > 0.0 ? dot : 0.0);"),
    ("visibility off by one", "q_pos[(int64_t)b * nq + t] + 1) / ORC_TPE", "q_pos[(int64_t)b * nq + t]) / ORC_TPE"),
    ("page slot reversed", "return (int64_t)page * c->page_size + s % c->page_size;",
     "return (int64_t)page * c->page_size + (c->page_size - 1 - s % c->page_size);"),
    ("tie order reversed", "return (a->id > b->id) - (a->id < b->id);", "return (a->id < b->id) - (a->id > b->id);"),
    ("selection ascending", "if (a->score > b->score) return -1;\n  if (a->score < b->score) return 1;",
     "if (a->score < b->score) return -1;\n  if (a->score > b->score) return 1;"),
    ("window dropped", "    if (win) {\n      int64_t len", "    if (0) {\n      int64_t len"),
    ("window row scale ignored", "double rs = win->row_scale ? (double)win->row_scale[(int64_t)b * win->rows + j] : 1.0;",
     "double rs = 1.0;"),
    ("window lower bound inclusive", "tok > p - win->window", "tok >= p - win->window"),
    ("softmax scale dropped", "z[r] = sm_scale * dot;", "z[r] = dot;"),
    ("max not subtracted", "L += exp(z[r] - M);", "L += exp(z[r]) * exp(-M) * exp(M) / exp(M);"),
    ("lse without log", "lse[bt * ORC_H + h] = M + log(L);", "lse[bt * ORC_H + h] = M + L;"),
    ("query head stride", "const float *qh = q + (bt * ORC_H + h) * ORC_D;", "const float *qh = q + (bt * ORC_H + (h ^ 1)) * ORC_D;"),
    ("selected entry rows skipped", "if (s < 0 || s >= c->n_entries[b]) continue;", "if (s <= 0 || s >= c->n_entries[b]) continue;"),
    ("encode ties to odd", "(d == bd && (i & 1) == 0 && (best & 1) == 1)", "(d == bd && (i & 1) == 1 && (best & 1) == 0)"),
    ("encode ties upward", "(d == bd && (i & 1) == 0 && (best & 1) == 1)", "(d == bd)"),
    ("block scale from amax/4", "int sb = orc_e4m3_encode(amax / 6.0f);", "int sb = orc_e4m3_encode(amax / 4.0f);"),
    ("encode sign dropped", "return c | (y < 0.0f ? 8 : 0);", "return c;"),
    ("encode nibble order", "cr[ch >> 1] |= (uint8_t)(code << ((ch & 1) * 4));", "cr[ch >> 1] |= (uint8_t)(code << ((1 - (ch & 1)) * 4));"),
    ("encode NaN byte allowed", "int b = nearest_even(T_E4M3, 0x7F, fabs((double)x));", "int b = nearest_even(T_E4M3, 0x7E, fabs((double)x));"),
    ("window row scale /240", "rs = amax > 0.0f ? amax / 448.0f : 1.0f;", "rs = amax > 0.0f ? amax / 240.0f : 1.0f;"),
    ("append slot reversed", "int64_t row = (int64_t)page * c->page_size + s % c->page_size;",
     "int64_t row = (int64_t)page * c->page_size + (c->page_size - 1 - s % c->page_size);"),
    ("Reindex scores the first pool columns", "const int32_t *cand = (mode == 0) ? NULL : idx_in;",
     "const int32_t *cand = NULL;"),
    ("Reindex returns pool slots", "orc_topk(sc, cand, B, nq, n, k, idx_out);", "orc_topk(sc, NULL, B, nq, n, k, idx_out);"),
    ("append indexer into main KV scales", "c->ix_codes + row * (ORC_DI / 2), c->ix_scales + row * (ORC_DI / ORC_G));",
     "c->ix_codes + row * (ORC_DI / 2), c->kv_scales + row * (ORC_D / ORC_G));"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(tmp_path, name, old, new):
    src = oracle.source()
    assert src.count(old) == 1, f"mutation anchor not found once: {name}"
    path = oracle.build_variant(src.replace(old, new), str(tmp_path / "liboracle_mut.so"))
    failed = []
    with oracle.using(path):
        for pin in ALL_PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
            except Exception as e:  # a crash or NaN-driven error also counts as caught
                failed.append(f"{pin.__name__}:{type(e).__name__}")
    assert failed, f"no pin catches: {name}"
