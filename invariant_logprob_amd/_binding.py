"""placeholder, replaced by the ctypes binding"""
def _missing(*a, **k):
    raise RuntimeError("binding not built yet")
RlkError = RuntimeError
build_info = library_path = linear_logp = linear_logp_backward = _missing
linear_logp_workspace_size = load_library = logp_backward = logp_selected = _missing
