"""MI355X-native draft step of the Gemma 4 assistant (MTP drafter): HIP kernels behind a C ABI (libmtpd.so) and a
thin ctypes binding. See include/mtpd.h for the ABI."""
from . import abi
from .drafter import Drafter, SharedKV, stream_read

__all__ = ["abi", "Drafter", "SharedKV", "stream_read"]
