"""Plain, slow CPU oracle of the V-JEPA 2 / 2.1 video ViT encoder forward (and of the
V-JEPA 2 masked predictor), in float64 numpy.

THIS IS TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the HIP
library (``video_vit_encoder_amd``) and imports nothing from it; the two meet only in
the seeded inputs of the ``synth`` module.

Every function cites the passage it follows.  Sources, cited by page and section:
  [Notes]  "V-JEPA 2 / 2.1 tensor maps and RoPE derivation"
           (aselimc.github.io/jepa.cpp/vjepa-notes/)
  [Parity] "Parity -- image ViT encoders (I-JEPA, LeJEPA/hfvit, LeWM) and video encoders
           (V-JEPA 2 / V-JEPA 2.1, LeVJEPA)" (aselimc.github.io/jepa.cpp/parity/)
  [Card]   jepa.cpp V-JEPA 2 ViT-L/16 GGUF model card
           (graysoft.dev/models/jep/jepacpp-vjepa2-vitl-fpc64-256-gguf.html)
  [HFport] "V-JEPA 2.1 ViT-B/16 384 -- HuggingFace port"
           (aimarketly.com/model/apiantonio/vjepa2.1-vit-base-384)

Pinning: the pieces are pinned by ``tests/test_oracle_*.py`` against printed values,
closed forms, invariants and pure-Python brute force on tiny inputs.  The end-to-end
encoder has no printed value that can be re-run without the pages' trained weights;
it is trusted through those pins (see the test files' headers).
"""
from .vjepa import *  # noqa: F401,F403
from . import metrics  # noqa: F401
