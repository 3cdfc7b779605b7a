"""Load the built library for tests, building it here only when it is missing."""
import os

import paged_attention_02_amd as oxa


def ensure_built():
    if not os.path.exists(oxa.LIB_PATH):
        from paged_attention_02_amd import build
        build.build()
    return oxa.lib()
