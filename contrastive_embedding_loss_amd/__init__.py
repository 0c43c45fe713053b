"""MI355X-native fused Matryoshka contrastive loss (InfoNCE / SigLIP), fwd + bwd.

The compute runs in hand-written HIP kernels for gfx950 behind the C ABI
declared in ``include/uform_contrastive.h`` (``libuform_contrastive.so``);
``contrastive_embedding_loss_amd.binding`` marshals torch tensors into it.
Importing the package does not load the library; the first call does, and
fails loudly if it is missing.
"""

INFONCE = 0
SIGLIP = 1
INFONCE_ROWS = 2
ONESET_SIGLIP = 3
ONESET_SIGLIP_EDGES = 4

_BINDING_NAMES = ("fwd_bwd", "workspace_bytes", "supported", "status_name", "last_error", "profile", "release",
                  "library", "UformError")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
