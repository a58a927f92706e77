"""Device plumbing for the GPU tests (re-exported from workloads.device)."""
from workloads.device import norm_torch_dtype, norms_to_dev, to_dev  # noqa: F401
