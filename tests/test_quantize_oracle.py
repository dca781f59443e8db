"""The quantizer oracle against its pins, and deliberately broken copies of it
against the same pins (each mistake must fail at least one)."""

import importlib.util
import sys
from pathlib import Path

import pytest

from oracle import quantize as Q
from quantize_pins import PINS

SRC = Path(Q.__file__).resolve()

MUTANTS = {
    "no_fp16_rounding": ("sd = s16.astype(np.float64)", "sd = s"),
    "ties_away": ("q = np.clip(np.rint(t), -1, 1)",
                  "q = np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -1, 1)"),
    "mean_not_max": ("s = np.abs(blocks).max(axis=2)", "s = np.abs(blocks).mean(axis=2) * 2"),
    "truncate": ("q = np.clip(np.rint(t), -1, 1)", "q = np.clip(np.trunc(t), -1, 1)"),
    "sign_flip": ("q = q.reshape(N, K).astype(np.int8)", "q = (-q).reshape(N, K).astype(np.int8)"),
    "row_group_mixup": ("blocks = w.reshape(N, K // g, g)",
                        "blocks = w.T.reshape(K // g, g, N).transpose(2, 0, 1) if N * 0 else "
                        "w.reshape(N, g, K // g).transpose(0, 2, 1)"),
    "zero_group_plus": ("q = np.where((sd == 0)[:, :, None], 0.0, q)",
                        "q = np.where((sd == 0)[:, :, None], 1.0, q)"),
    "half_scale": ("s = np.abs(blocks).max(axis=2)", "s = np.abs(blocks).max(axis=2) / 2"),
}


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_quantize_pin(pin):
    pin(Q)


def _load_mutant(name, old, new, tmp_path):
    src = SRC.read_text()
    assert old in src, name
    pkg = tmp_path / "qmut"
    pkg.mkdir()
    (pkg / "__init__.py").write_text("")
    (pkg / "dense.py").write_text((SRC.parent / "dense.py").read_text())
    (pkg / "quantize.py").write_text(src.replace(old, new))
    sys.path.insert(0, str(tmp_path))
    try:
        spec = importlib.util.spec_from_file_location(f"qmut.quantize_{name}", pkg / "quantize.py",
                                                      submodule_search_locations=None)
        import qmut  # noqa: F401
        mod = importlib.util.module_from_spec(spec)
        mod.__package__ = "qmut"
        spec.loader.exec_module(mod)
        return mod
    finally:
        sys.path.remove(str(tmp_path))
        sys.modules.pop("qmut", None)
        sys.modules.pop("qmut.dense", None)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_quantize_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    mod = _load_mutant(name, old, new, tmp_path)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except AssertionError:
            failed.append(pin.__name__)
        except Exception as e:  # a crash on the broken copy also counts as caught
            failed.append(f"{pin.__name__}:{type(e).__name__}")
    assert failed, f"mutant {name} passes every quantizer pin"
