"""The library the GPU tests load was built from the sources in this tree: splr_version() ends with
the hash of those sources (the build embeds it)."""
import pytest

from sparse_rank_linear_prune24_amd import binding, build

pytestmark = pytest.mark.gpu


def test_loaded_library_matches_sources():
    assert binding.version() == "0.2.0+" + build.source_hash()
