"""CPU oracle for the Q2_K decode path (test infrastructure only).

Only the tests, the smoke check and the bench's CPU baseline import this
package; the product path never does.
"""
from . import q2k_oracle  # noqa: F401
