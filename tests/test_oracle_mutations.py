"""Plant plausible mistakes in a private copy of the oracle (CPU only) and check that the
pins catch each one.  The copy is built from the oracle's source text with one edit; the
real oracle module is never modified.
"""
import json
import os
import types

import numpy as np
import pytest

from oracle import q4_oracle
from synth import f64_to_bf16_bits

SRC = open(q4_oracle.__file__).read()

MUTATIONS = {
    "scale denominator 16": ("dt(q_max - q_min)", "dt(q_max - q_min + 1)"),
    "alpha not extended to 0": ("np.minimum(x.min(axis=-1), dt(0))", "x.min(axis=-1)"),
    "zero-point sign": ("np.rint(dt(q_min) - ratio)", "np.rint(dt(q_min) + ratio)"),
    "round after adding z": ("r = np.clip(np.rint(quot), dt(-2.0 ** 40), dt(2.0 ** 40)).astype(np.int64)\n    q = np.clip(r + z[..., None], q_min, q_max)",
                             "q = np.clip(np.rint(quot + z[..., None]).astype(np.int64), q_min, q_max)"),
    "no fp16 scale rounding": ("s = s16.astype(dt)", "s = np.minimum(scale.astype(np.float32), F16_MAX).astype(dt)"),
    "nibble order swapped": ("(nib[:, 0::2] | (nib[:, 1::2] << 4))", "(nib[:, 1::2] | (nib[:, 0::2] << 4))"),
    "unpack order swapped": ("codes[:, 0::2] = p & 0xF\n    codes[:, 1::2] = p >> 4",
                             "codes[:, 1::2] = p & 0xF\n    codes[:, 0::2] = p >> 4"),
    "sign extension off by one": ("codes - 16", "codes - 15"),
    "dequant adds z": ("(qg - z[..., None])", "(qg + z[..., None])"),
    "symmetric q_max 8": ('quantize_groups(x, -8, 7, "sym")', 'quantize_groups(x, -8, 8, "sym")'),
    "group index off": ("s[..., None] * (qg - z[..., None])", "np.roll(s, 1, axis=-1)[..., None] * (qg - z[..., None])"),
    "abs dropped in A": ("    A = np.abs(X) @ np.abs(What).T", "    A = X @ What.T"),
    "bf16 ties away from zero": ("np.rint(np.ldexp(m, 8))", "np.trunc(np.ldexp(m, 8) + np.copysign(0.5, m))"),
    "bf16 7 significant bits": ("np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)", "np.ldexp(np.rint(np.ldexp(m, 7)), e - 7)"),
    "bf16 truncation": ("np.rint(np.ldexp(m, 8))", "np.trunc(np.ldexp(m, 8))"),
    "AWQ magnitude is the max": ("    a = np.abs(X).mean(axis=0)\n    cands", "    a = np.abs(X).max(axis=0)\n    cands"),
    "AWQ 1/s not folded back": ("cands = [qdq(W * s) / s for s", "cands = [qdq(W * s) for s"),
    "AWQ scored on weight error": ("np.linalg.norm(X @ (W - Q).T)", "np.linalg.norm(W - Q)"),
    "AWQ scales not normalised": ("    return p / np.sqrt(p.max() * p.min())", "    return p"),
    "AWQ grid misses alpha 1": ("return [i / (n_alpha - 1) if n_alpha > 1 else 0.0 for i in range(n_alpha)]", "return [i / n_alpha for i in range(n_alpha)]"),
    "AWQ last alpha wins ties": ("    k = int(np.argmin(scores))", "    k = len(scores) - 1 - int(np.argmin(scores[::-1]))"),
    "INT8 asym range 254": ('Q8_RANGE = {"asym": (0, 255), "sym": (-127, 127)}', 'Q8_RANGE = {"asym": (0, 254), "sym": (-127, 127)}'),
    "INT8 sym codes offset binary": ("return np.where(c >= 128, c - 256, c) if mode == \"sym\" else c", "return c - 128 if mode == \"sym\" else c"),
    "GPTQ toy without damping": ("    H[np.diag_indices_from(H)] += damp * np.mean(np.diag(H))\n    d = w.shape[1]", "    d = w.shape[1]"),
    "GPTQ toy compensation sign": ("w[:, i + 1:] += np.outer(w[:, i] - Q[:, i], v)", "w[:, i + 1:] -= np.outer(w[:, i] - Q[:, i], v)"),
    "GPTQ toy solves on all later rows of H": ("v = np.linalg.solve(H[i + 1:, i + 1:], H[i + 1:, i])", "v = np.linalg.lstsq(H[:, i + 1:], H[:, i], rcond=None)[0]"),
    "GPTQ toy error from the original weight": ("w[:, i + 1:] += np.outer(w[:, i] - Q[:, i], v)", "w[:, i + 1:] += np.outer(W[:, i] - Q[:, i], v)"),
    "GPTQ Cholesky of H instead of its inverse": ("np.linalg.cholesky(np.linalg.inv(H)).T", "np.linalg.cholesky(H).T"),
    "GPTQ codes from the original weights": ("quot = w[:, i].astype(np.float32) / s32[:, G]", "quot = W32[:, i] / s32[:, G]"),
    "bf16 bit rounding truncates": ("(u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)", "u >> np.uint64(16)"),
}


def _mutant(old, new):
    assert SRC.count(old) == 1, old
    mod = types.ModuleType("q4_oracle_mutant")
    exec(compile(SRC.replace(old, new), "q4_oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(orc, golden_dir):
    """The pins of test_oracle_pins / test_oracle_props in compact form; True if all hold."""
    from tests.test_oracle_props import exact_group
    try:
        ex_all = json.load(open(os.path.join(golden_dir, "hand_examples.json")))
        for mode in ("asym", "sym"):
            ex = ex_all[mode]
            W_bits = f64_to_bf16_bits(np.array([ex["x"]]))
            packed, scales, zeros = orc.quantize_rtn_ref(W_bits, g=8, mode=mode)
            if float(scales[0, 0]) != ex["scale"] or int(zeros[0, 0]) != ex["zero"]:
                return False
            if [f"0x{b:02X}" for b in packed[0]] != ex["packed_hex"]:
                return False
            if orc.unpack_codes_ref(packed, mode)[0].tolist() != ex["codes"]:
                return False
            if orc.dequantize_ref(packed, scales, zeros, 8, mode)[0].tolist() != ex["xhat"]:
                return False
        rng = np.random.default_rng(0)
        groups = np.concatenate([rng.normal(0, 0.02, (48, 32)), np.abs(rng.normal(0, 1, (16, 32))) + 0.5])
        for mode in ("asym", "sym"):
            x = orc.bf16_bits_to_f32(f64_to_bf16_bits(groups))
            qmin, qmax = (0, 15) if mode == "asym" else (-8, 7)
            q, s16, z = orc.quantize_groups(x, qmin, qmax, mode)
            for i in range(len(x)):
                es, ez, eq = exact_group(x[i], mode)
                if float(s16[i]) != float(es) or int(z[i]) != ez or q[i].tolist() != eq:
                    return False
        W_bits = f64_to_bf16_bits(rng.normal(0, 0.02, (4, 64)))
        for mode in ("asym", "sym"):
            packed, scales, zeros = orc.quantize_rtn_ref(W_bits, g=32, mode=mode)
            Y, A = orc.matmul_ref(f64_to_bf16_bits(np.eye(64)), packed, scales, zeros, 32, mode)
            if not np.array_equal(A, np.abs(Y)):
                return False
            x = orc.bf16_bits_to_f32(W_bits).astype(np.float64)
            if np.abs(Y.T - x).max() > 0.6 * np.abs(x).max() / 7 + 1e-12:
                return False
        from tests.test_oracle_pins import rounding_pins_hold
        if not rounding_pins_hold(orc):
            return False
        from tests.test_oracle_awq import awq_pins_hold
        if not awq_pins_hold(orc):
            return False
        from tests.test_oracle_w8 import w8_pins_hold
        if not w8_pins_hold(orc):
            return False
        from tests.test_oracle_gptq import gptq_pins_hold
        if not gptq_pins_hold(orc):
            return False
    except Exception:
        return False
    return True


def test_unmutated_oracle_passes(golden_dir):
    assert _pins_pass(q4_oracle, golden_dir)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, golden_dir):
    old, new = MUTATIONS[name]
    assert not _pins_pass(_mutant(old, new), golden_dir), f"pins missed: {name}"
