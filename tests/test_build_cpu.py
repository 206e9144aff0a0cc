"""CPU check of the build script's comparison builds: a build with tuning switches set never
replaces the plain library."""
import pytest

from paged_kv_cache_251_amd import build


def test_defines_need_an_output_of_their_own():
    with pytest.raises(ValueError):
        build.build(defines=["PA_DECODE_MFMA_WIDE_GROUPS=0"])
