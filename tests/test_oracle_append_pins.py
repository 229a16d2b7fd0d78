"""Pins of the fp64 append oracle (attn.qk_norm, attn.v_norm, attn.rope of the
Model Spec page applied to the new token), CPU only.

Each check ties the oracle to something other than itself: torch's rms_norm
(a library routine), RoPE written as complex multiplication (an independent
formulation), the relative-position property RoPE is used for (the Retrofit
Plan page's "RoPE encodes relative distance" evidence), norm preservation,
the untouched inactive pairs of the global layers (the architecture page's
"zero inverse frequency" remark), values = keys on global layers, and the
zero-length case.  Planted mistakes in a copy of the oracle must each be
caught by at least one check.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

F = torch.nn.functional
GEOM = {"sliding": (16, 256, 1e4, 128), "global": (4, 512, 1e6, 64)}


def _raw(variant, B, seed, dtype="f32"):
    KV, D, _, _ = GEOM[variant]
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, 32, D, generator=g) * 3
    k = torch.randn(B, KV, D, generator=g) * 2
    v = torch.randn(B, KV, D, generator=g)
    wq = torch.empty(D).uniform_(0.2, 0.4, generator=g)
    wk = torch.empty(D).uniform_(0.2, 0.4, generator=g)
    tdt = synth.TORCH_DTYPES[dtype]
    return [t.to(tdt) for t in (q, k, v, wq, wk)]


def _run(lib, variant, q, k, v, wq, wk, lens):
    np_ = synth.to_numpy
    return oracle.gqa_append_rows(variant, np_(q), np_(k), None if variant == "global" else np_(v),
                                  np_(wq), np_(wk), np.asarray(lens, dtype=np.int32), lib=lib)


def _rope_complex(u, pos, theta, active):
    """RoPE as complex multiplication: z_i = u_i + 1j*u_{i+D/2}, z_i *= exp(1j*pos*theta^(-2i/D))."""
    D = u.shape[-1]
    h = D // 2
    z = u[..., :h] + 1j * u[..., h:]
    i = np.arange(h)
    ang = np.where(i < active, pos * theta ** (-2.0 * i / D), 0.0)
    z = z * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


def check_pos0_is_the_norm(lib):
    for variant in GEOM:
        q, k, v, wq, wk = _raw(variant, 3, 1)
        qo, ko, vo, pos = _run(lib, variant, q, k, v, wq, wk, [1, 1, 1])
        assert (pos == 0).all()
        eq = F.rms_norm(q.double(), (q.shape[-1],), weight=wq.double(), eps=1e-6).numpy()
        ek = F.rms_norm(k.double(), (k.shape[-1],), weight=wk.double(), eps=1e-6).numpy()
        src = k if variant == "global" else v
        ev = F.rms_norm(src.double(), (src.shape[-1],), eps=1e-6).numpy()
        assert np.abs(qo - eq).max() <= 1e-12
        assert np.abs(ko - ek).max() <= 1e-12
        assert np.abs(vo - ev).max() <= 1e-12


def check_rope_complex_formulation(lib):
    for variant in GEOM:
        KV, D, theta, active = GEOM[variant]
        for dtype in ("f32", "bf16"):
            q, k, v, wq, wk = _raw(variant, 4, 2, dtype)
            lens = [2, 17, 4097, 262144]
            qo, ko, _, _ = _run(lib, variant, q, k, v, wq, wk, lens)
            uq = F.rms_norm(q.double(), (D,), weight=wq.double(), eps=1e-6).numpy()
            uk = F.rms_norm(k.double(), (D,), weight=wk.double(), eps=1e-6).numpy()
            for b, L in enumerate(lens):
                eq = _rope_complex(uq[b], L - 1, theta, active)
                ek = _rope_complex(uk[b], L - 1, theta, active)
                assert np.abs(qo[b] - eq).max() <= 1e-9, (variant, dtype, L)
                assert np.abs(ko[b] - ek).max() <= 1e-9, (variant, dtype, L)


def check_relative_position(lib):
    # <rope(q, m), rope(k, n)> depends on m - n only
    for variant in GEOM:
        q, k, v, wq, wk = _raw(variant, 1, 3)
        dots = []
        for m, n in ((10, 3), (1010, 1003), (200007, 200000)):
            qo, _, _, _ = _run(lib, variant, q, k, v, wq, wk, [m + 1])
            _, ko, _, _ = _run(lib, variant, q, k, v, wq, wk, [n + 1])
            dots.append(np.einsum("hd,d->h", qo[0], ko[0, 0]))
        assert np.abs(dots[0] - dots[1]).max() <= 1e-9
        assert np.abs(dots[0] - dots[2]).max() <= 1e-8


def check_pair_norms_preserved(lib):
    for variant in GEOM:
        KV, D, _, _ = GEOM[variant]
        q, k, v, wq, wk = _raw(variant, 2, 4)
        qo1, ko1, _, _ = _run(lib, variant, q, k, v, wq, wk, [1, 1])
        qo, ko, _, _ = _run(lib, variant, q, k, v, wq, wk, [777, 131072])
        h = D // 2
        for a, a0 in ((qo, qo1), (ko, ko1)):
            n = np.hypot(a[..., :h], a[..., h:])
            n0 = np.hypot(a0[..., :h], a0[..., h:])
            assert np.abs(n - n0).max() <= 1e-12


def check_global_inactive_pairs_untouched(lib):
    q, k, v, wq, wk = _raw("global", 2, 5)
    qo1, ko1, _, _ = _run(lib, "global", q, k, v, wq, wk, [1, 1])
    qo, ko, _, _ = _run(lib, "global", q, k, v, wq, wk, [5000, 99])
    for a, a0 in ((qo, qo1), (ko, ko1)):
        for lo, hi in ((64, 256), (320, 512)):
            assert np.array_equal(a[..., lo:hi], a0[..., lo:hi])
        assert not np.array_equal(a[..., :64], a0[..., :64])  # the active pairs do rotate


def check_sliding_every_pair_rotates(lib):
    q, k, v, wq, wk = _raw("sliding", 1, 6)
    qo1, _, _, _ = _run(lib, "sliding", q, k, v, wq, wk, [1])
    qo, _, _, _ = _run(lib, "sliding", q, k, v, wq, wk, [3])
    changed = np.abs(qo - qo1)[0].max(axis=0) > 1e-12
    assert changed[:128].all() and changed[128:].all()


def check_values(lib):
    # sliding: v_norm of v_raw, unrotated; global: values = keys, unit-normalised raw keys
    for variant in GEOM:
        KV, D, _, _ = GEOM[variant]
        q, k, v, wq, wk = _raw(variant, 2, 7)
        _, _, vo, _ = _run(lib, variant, q, k, v, wq, wk, [900, 3])
        src = k if variant == "global" else v
        ev = F.rms_norm(src.double(), (D,), eps=1e-6).numpy()
        assert np.abs(vo - ev).max() <= 1e-12
        rms = np.sqrt((vo ** 2).mean(-1))
        assert np.abs(rms - 1).max() <= 1e-5  # unit RMS up to eps


def check_zero_length(lib):
    q, k, v, wq, wk = _raw("sliding", 2, 8)
    qo, ko, vo, pos = _run(lib, "sliding", q, k, v, wq, wk, [0, 5])
    assert pos[0] == -1 and pos[1] == 4
    assert not qo[0].any() and not ko[0].any() and not vo[0].any()
    assert qo[1].any()


def check_constant_vector_closed_form(lib):
    # x = c * 1  ->  rms_norm = c / sqrt(c^2 + eps) * w   (position 0: no rotation)
    KV, D, _, _ = GEOM["sliding"]
    c = 0.015625  # exact in binary
    q = torch.full((1, 32, D), c)
    k = torch.full((1, KV, D), c)
    v = torch.full((1, KV, D), c)
    wq = torch.linspace(0.2, 0.4, D)
    wk = torch.linspace(0.4, 0.2, D)
    qo, ko, vo, _ = _run(lib, "sliding", q, k, v, wq, wk, [1])
    s = c / np.sqrt(c * c + 1e-6)
    assert np.abs(qo[0] - s * wq.double().numpy()).max() <= 1e-12
    assert np.abs(ko[0] - s * wk.double().numpy()).max() <= 1e-12
    assert np.abs(vo[0] - s).max() <= 1e-12


ALL = [check_zero_length, check_constant_vector_closed_form, check_pos0_is_the_norm,
       check_values, check_rope_complex_formulation, check_relative_position,
       check_pair_norms_preserved, check_global_inactive_pairs_untouched,
       check_sliding_every_pair_rotates]


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("check", ALL, ids=lambda f: f.__name__)
def test_append_pin(lib, check):
    check(lib)


MUTANTS = {
    "rotation_sign": ("y[i] = a * c - b * s;", "y[i] = a * c + b * s;"),
    "pair_offset": ("const int h = D / 2;\n  for (int i = 0; i < active; ++i) {",
                    "const int h = D / 4;\n  for (int i = 0; i < active; ++i) {"),
    "frequency_exponent": ("pow(theta, -2.0 * i / D)", "pow(theta, -1.0 * i / D)"),
    "global_active_pairs": ("const int active = global ? 64 : 128;",
                            "const int active = global ? 128 : 128;"),
    "global_theta": ("const double theta = global ? 1e6 : 1e4;",
                     "const double theta = global ? 1e4 : 1e4;"),
    "eps_outside_sqrt": ("1.0 / sqrt(ss / D + ORC_EPS)", "1.0 / (sqrt(ss / D) + ORC_EPS)"),
    "weight_dropped": ("y[d] = x[d] * inv * (w ? w[d] : 1.0);", "y[d] = x[d] * inv;"),
    "global_values_weighted": ("orc_rms(x, D, NULL, yv);", "orc_rms(x, D, wk, yv);"),
    "position_one_late": ("const long pos = (long)seq_lens[b] - 1;",
                          "const long pos = (long)seq_lens[b];"),
    "sum_not_mean": ("sqrt(ss / D + ORC_EPS)", "sqrt(ss + ORC_EPS)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_append_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    mlib = oracle.load(oracle.build(str(path), str(tmp_path / f"libmutant_{name}.so")))
    for check in ALL:
        try:
            check(mlib)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            return
    pytest.fail(f"planted mistake {name} passed every append pin")
