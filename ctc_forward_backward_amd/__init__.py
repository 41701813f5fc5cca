"""Packed CTC loss and gradient on MI355X (gfx950): a C-ABI HIP library and its thin Python binding.

``packed_ctc_loss`` and the other entry points live in ``ctc_forward_backward_amd.api``; they are
loaded lazily so that the input generators in ``workloads`` import without the HIP library.
"""

_API = ("packed_ctc_loss", "packed_ctc_forward", "packed_ctc_backward", "packed_ctc_forward_grad",
        "packed_ctc_backward_update", "ctc_loss", "PackedCTCLoss", "packed_ctc_reduce", "packed_ctc_workspace_size",
        "PackedCTCError", "library_path", "hmm_forward")


def __getattr__(name):
    if name in _API:
        from . import api

        return getattr(api, name)
    raise AttributeError(name)
