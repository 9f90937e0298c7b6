"""Runs the host-side ABI tests (argument checks, plans, size queries: no
device work) against a copy of the library whose host code was built with
AddressSanitizer and UndefinedBehaviorSanitizer.  Usage: python abi_driver.py
<library>; started with the sanitizer runtime preloaded."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, os.path.dirname(HERE))

import gated_linear_attention_rodimus_amd as R  # noqa: E402

R.LIB_PATH = sys.argv[1]
import test_abi  # noqa: E402

ran = 0
for name in sorted(dir(test_abi)):
    fn = getattr(test_abi, name)
    if name.startswith("test_") and callable(fn):
        if name == "test_binding_checks_a_supplied_workspace":
            continue                      # pure Python, no library call
        fn()
        ran += 1
print(f"abi tests under sanitizers: {ran} passed", flush=True)
