"""CPU oracle of the QSA forward path (test infrastructure only; see qsa_oracle)."""
from . import qsa_oracle  # noqa: F401
