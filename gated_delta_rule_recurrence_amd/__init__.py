"""MI355X-native gated delta rule forward pass and VJP.

Importing the package loads nothing native; the HIP library is opened on the
first call through :mod:`gated_delta_rule_recurrence_amd.ops`.
"""
__all__ = ["ops", "inputs"]
