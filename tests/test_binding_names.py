"""Every global name the binding's functions load exists (CPU; no GPU call).

The binding's code paths only run on a GPU, so a misspelt or stray name in one
of them would otherwise surface there first.  This reads each function's
bytecode for global loads and checks them against the module and builtins."""
import builtins
import dis
import inspect

import kimi_delta_attention_02_amd as kda
from kimi_delta_attention_02_amd import _lib


def _global_loads(fn):
    names = set()
    todo = [fn.__code__]
    while todo:
        code = todo.pop()
        for ins in dis.get_instructions(code):
            if ins.opname == "LOAD_GLOBAL":
                names.add(ins.argval if isinstance(ins.argval, str) else ins.argrepr.split()[-1])
        todo.extend(c for c in code.co_consts if inspect.iscode(c))
    return names


def test_binding_functions_load_only_defined_globals():
    for mod in (kda, _lib):
        for name, fn in vars(mod).items():
            if not inspect.isfunction(fn) or fn.__module__ != mod.__name__:
                continue
            for g in _global_loads(fn):
                g = g.replace("NULL + ", "").strip()
                assert hasattr(mod, g) or hasattr(builtins, g), \
                    "%s.%s loads undefined global %r" % (mod.__name__, name, g)


def test_every_exported_name_exists():
    for name in kda.__all__:
        assert hasattr(kda, name), name
