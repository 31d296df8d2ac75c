"""Engine construction and input upload from the seeded generators (no oracle here)."""
from semantic_id_beam_amd.workloads import load_request, make_engine, native_layout, request_tensors  # noqa: F401
