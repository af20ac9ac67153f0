"""pytest plugin of the sanitizer run: points the state-reader binding and
the input generator at the libraries named by READY_SAN_DIR (host code built
with AddressSanitizer and UndefinedBehaviorSanitizer) before any test loads
them."""
import os

import hla_recurrent_state_amd as _ready
import synth.gen as _gen

_dir = os.environ["READY_SAN_DIR"]
_ready.LIB_PATH = os.path.join(_dir, "libready.so")
_gen.LIB_PATH = os.path.join(_dir, "libsynth.so")
