"""The oracle's ctypes table against its C definitions (host only).

oracle/__init__.py marshals numpy arrays into dit_oracle.c through ctypes; a
parameter added to, dropped from or retyped in a C definition without the
same change in that table would make every oracle call read wrong arguments,
and every parity verdict built on it meaningless.  This parses the exported
definitions of dit_oracle.c and compares them with what the loader binds.
"""
import ctypes
import os
import re

import oracle

_TYPES = {"int64_t": ctypes.c_int64, "int32_t": ctypes.c_int32, "int": ctypes.c_int, "double": ctypes.c_double,
          "uint16_t": ctypes.c_uint16}


def _ctype(decl):
    decl = decl.strip()
    if "*" in decl:
        return ctypes.c_void_p
    words = [w for w in decl.split() if w != "const"]
    return _TYPES[words[0]]


def exported_definitions():
    with open(oracle.SOURCE, encoding="utf-8") as fh:
        text = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    out = {}
    for m in re.finditer(r"^((?:const\s+)?\w+\s*\*?)\s*(dit_oracle_\w+)\s*\(([^)]*)\)\s*\{", text, flags=re.M):
        ret, name, params = m.groups()
        if ret.strip().startswith("static"):
            continue
        params = params.strip()
        args = [] if params in ("", "void") else [_ctype(p.rsplit(None, 1)[0] if "*" not in p else p) for p in
                                                  params.split(",")]
        out[name] = (args, _ctype(ret))
    return out


def test_every_exported_oracle_function_is_bound_with_its_c_signature():
    lib = oracle.load()
    defs = exported_definitions()
    assert len(defs) >= 15, sorted(defs)
    for name, (args, res) in defs.items():
        fn = getattr(lib, name)
        assert fn.argtypes is not None, f"{name} is not bound"
        assert [a.__name__ for a in fn.argtypes] == [a.__name__ for a in args], name
        assert fn.restype.__name__ == res.__name__, name


def test_oracle_source_is_where_the_loader_builds_from():
    assert os.path.exists(oracle.SOURCE) and oracle.SOURCE.endswith("dit_oracle.c")
