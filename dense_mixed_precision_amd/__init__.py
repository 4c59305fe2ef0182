"""Placeholder; replaced by the binding."""
