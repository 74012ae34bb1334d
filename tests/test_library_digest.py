"""The loader refuses a library built from other sources than the ones in the tree (CPU only)."""
import os
import shutil

import pytest


@pytest.fixture(scope="module")
def built():
    import __graft_entry__
    __graft_entry__._ensure_built()
    from selective_state_space_58_amd import build
    return build


def _copy_tree(build, dst):
    csrc, inc, lib = dst / "csrc", dst / "include", dst / "libssm_mi355x.so"
    shutil.copytree(build.CSRC, csrc)
    shutil.copytree(build.INCLUDE, inc)
    shutil.copy(build.LIB, lib)
    return str(lib), str(csrc), str(inc)


def test_embedded_digest_matches_the_tree(built):
    from selective_state_space_58_amd import _binding
    lib = _binding.load_library()
    assert lib.ssm_source_digest().decode() == built.source_digest()
    assert built.built_digest() == built.source_digest()
    assert built.stale_reason() is None


@pytest.mark.parametrize("edit", ["csrc/scan_host.hip", "include/ssm_mi355x.h", "csrc/new_file.hip"])
def test_loader_refuses_a_library_built_from_other_sources(built, tmp_path, edit):
    from selective_state_space_58_amd import _binding
    lib, csrc, inc = _copy_tree(built, tmp_path)
    _binding.check_library(lib, csrc, inc)       # the copy matches
    path = tmp_path / edit
    old = path.read_text() if path.exists() else ""
    path.write_text(old + "\n// one more line\n")
    assert "other sources" in built.stale_reason(lib, csrc, inc)
    with pytest.raises(RuntimeError, match="other sources"):
        _binding.check_library(lib, csrc, inc)


def test_missing_or_unmarked_library_is_refused(built, tmp_path):
    from selective_state_space_58_amd import _binding
    lib, csrc, inc = _copy_tree(built, tmp_path)
    with open(lib, "wb") as fh:
        fh.write(b"\0" * 64)
    with pytest.raises(RuntimeError, match="no source digest"):
        _binding.check_library(lib, csrc, inc)
    os.remove(lib)
    with pytest.raises(RuntimeError, match="not built"):
        _binding.check_library(lib, csrc, inc)
