"""The pins of tests/test_oracle_pins.py on the numpy implementation of the oracle
(oracle.numpy_reference, a second and independent coding of the method): every pin that
fixes the C++ oracle fixes it too."""
import os

_SRC = open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "test_oracle_pins.py")).read()
assert "import oracle as O\n" in _SRC
exec(compile(_SRC.replace("import oracle as O\n", "from oracle import numpy_reference as O\n"), __file__, "exec"))
