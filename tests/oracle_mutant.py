"""Build a copy of the oracle with one planted mistake (in a temporary
directory, never touching the oracle itself or the product), for tests that
check that the oracle's pins catch it."""

import importlib.util
import shutil
import subprocess
from pathlib import Path


def build_oracle_mutant(orc, tmp_path: Path, old: str, new: str, tag: str):
    src = (Path(orc.__file__).parent / "cam_oracle.c").read_text()
    assert src.count(old) == 1, f"{tag}: the planted mistake must replace exactly one statement"
    d = tmp_path / f"oracle_{tag}"
    d.mkdir()
    (d / "cam_oracle.c").write_text(src.replace(old, new))
    shutil.copy(Path(orc.__file__), d / "__init__.py")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o", str(d / "liboracle.so"),
                    str(d / "cam_oracle.c"), "-lm"], check=True)
    spec = importlib.util.spec_from_file_location("oracle_mutant_" + tag, d / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod
