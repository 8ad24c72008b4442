class GdnError(RuntimeError): pass
def lib(): raise NotImplementedError
prep = recurrent = layer_core = layer_core_workspace_bytes = lib
