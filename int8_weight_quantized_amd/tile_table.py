"""Measured per-shape tile table for the GEMM (PR #142, "What this does",
item 2: a table of benchmarked winners that the layer consults before the
heuristic, for exact shape matches, gated by the GPU it was measured on).

A table is a JSON file written by ``python -m int8_weight_quantized_amd.tune``:

    {"arch": "gfx950", "abi": 6, "entries": [
        {"m": 80666, "n": 28672, "k": 5376, "tile": 12, "group_m": 4,
         "us": ..., "heuristic_us": ..., ...}, ...]}

``load`` registers its entries with the library (ck_int8_table_set); a
table whose "arch" differs from the device's is ignored.  The torch helpers
of the package load the packaged table for the device's architecture
(``tile_table_<arch>.json`` next to this file) once per process, unless the
environment variable CK_INT8_TILE_TABLE is "off"; a path there replaces the
packaged file.  Without a table the heuristic alone decides.
"""
from __future__ import annotations

import json
import os

_loaded = False


def device_arch(device=None) -> str:
    import torch
    props = torch.cuda.get_device_properties(device if device is not None else 0)
    return props.gcnArchName.split(":")[0]


def default_path(arch: str) -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), f"tile_table_{arch}.json")


def load(path: str, arch: str) -> int:
    """Register the entries of the table at `path` if it was measured on
    `arch`; returns the number registered (0 for another architecture)."""
    from . import ck_int8_table_set
    with open(path) as fh:
        table = json.load(fh)
    if table.get("arch") != arch:
        return 0
    count = 0
    for e in table.get("entries", []):
        ck_int8_table_set(int(e["m"]), int(e["n"]), int(e["k"]), int(e["tile"]), int(e["group_m"]))
        count += 1
    return count


def ensure_loaded(device=None) -> None:
    """Load the table for this device once per process (see module doc)."""
    global _loaded
    if _loaded:
        return
    _loaded = True
    setting = os.environ.get("CK_INT8_TILE_TABLE", "")
    if setting.lower() == "off":
        return
    arch = device_arch(device)
    path = setting or default_path(arch)
    if os.path.exists(path):
        load(path, arch)
