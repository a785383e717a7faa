"""DoRA adapter hot path for AMD Instinct MI355X (gfx950).

The product is the C-ABI HIP library ``libdora_hip.so`` (declared in
``include/dora.h``): the factored weight norm and the fused magnitude compose,
forward and backward.  ``binding`` is its thin ctypes layer; ``synth`` builds the
seeded synthetic adapter inputs.  Binding names resolve lazily, so
``dora_fine_tuning_amd.synth`` imports without the built library, while any use
of the HIP entry points fails loudly if the library is missing.
"""
_BINDING = (
    "dora_norm_factored",
    "dora_compose_fwd",
    "dora_compose_bwd",
    "dora_norm_workspace_bytes",
    "dora_compose_bwd_workspace_bytes",
    "dora_last_error",
    "dora_version",
    "DoraError",
)

__all__ = list(_BINDING)


def __getattr__(name):
    if name in _BINDING:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
