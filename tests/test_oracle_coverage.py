"""Every public oracle function is reached from a pin.

A function counts as reached when a ``tests/test_oracle_*.py`` file names it,
or when a reached oracle function or module constant refers to it by name.  A helper added to the
oracle without any pin then fails here, instead of sitting "parity unpinned"
unnoticed.  (Static: names in the source, no execution of the pins.)
"""

import ast
import glob
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _refs(node):
    refs = {n.id for n in ast.walk(node) if isinstance(n, ast.Name)}
    return refs | {n.attr for n in ast.walk(node) if isinstance(n, ast.Attribute)}


def _oracle_symbols():
    """({function or class: names its body refers to}, {module constant:
    names its definition refers to}) over the oracle modules' top level."""
    funcs, consts = {}, {}
    for path in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        tree = ast.parse(open(path).read())
        for node in tree.body:
            if isinstance(node, (ast.FunctionDef, ast.ClassDef)) and not node.name.startswith("_"):
                funcs[node.name] = _refs(node)
            elif isinstance(node, ast.Assign):
                for t in node.targets:
                    if isinstance(t, ast.Name):
                        consts[t.id] = _refs(node.value)
    return funcs, consts


def _names_in_pins():
    names = set()
    for path in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")):
        if os.path.basename(path) == os.path.basename(__file__):
            continue
        tree = ast.parse(open(path).read())
        names |= {n.attr for n in ast.walk(tree) if isinstance(n, ast.Attribute)}
        names |= {n.id for n in ast.walk(tree) if isinstance(n, ast.Name)}
    return names


def test_every_oracle_function_is_reached_from_a_pin():
    funcs, consts = _oracle_symbols()
    graph = {**consts, **funcs}
    reached = set(graph) & _names_in_pins()
    grew = True
    while grew:
        grew = False
        for f in list(reached):
            for g in graph[f] & set(graph):
                if g not in reached:
                    reached.add(g)
                    grew = True
    missing = sorted(set(funcs) - reached)
    assert not missing, f"oracle functions no pin reaches: {missing}"
