"""Test configuration.

Tests cite the two pages that describe ISA by title and section:
[notes] is the papernotes.org ICML 2026 notes "Lightning Unified Video Editing
via In-Context Sparse Attention"; [summary] is the paperlayer.ai summary
"LIVEditor-14B: Lightning Unified Video Editing via In-Context Sparse
Attention" of arXiv 2605.04569v2.
"""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct MI355X (gfx950) device")
    config.addinivalue_line("markers", "slow: larger CPU cases")
