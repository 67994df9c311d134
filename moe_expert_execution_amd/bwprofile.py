"""Measured bandwidth profiles (B_P, B_H) stored per expert format and GPU.

A profile measured by ``ft_cache_profile`` on one machine is only valid for
that GPU and that record format, so it is stored under both keys and a lookup
with another key finds nothing ("Making Large MoE Models Practical on a Single
Machine", section 7; the txtmix.com FreeToken article's quick start: one
bandwidth benchmark per GPU, profiles keyed by expert format and GPU).
"""
import json
import os
import time

DEFAULT_DIR = os.path.join(os.path.expanduser("~"), ".cache", "ftmoe", "bwprofile")


def _path(gpu_key: str, directory: str) -> str:
    safe = "".join(ch if ch.isalnum() or ch in "-_." else "_" for ch in gpu_key)
    return os.path.join(directory, safe + ".json")


def save(fmt: str, gpu_key: str, bp_mbps: int, bh_mbps: int, directory: str = DEFAULT_DIR, **extra) -> str:
    """Store the profile of `fmt` on `gpu_key`; other formats' entries are kept."""
    os.makedirs(directory, exist_ok=True)
    path = _path(gpu_key, directory)
    data = {}
    if os.path.exists(path):
        with open(path) as fh:
            data = json.load(fh)
    if data.get("gpu") != gpu_key:
        data = {"gpu": gpu_key, "formats": {}}
    data["formats"][fmt] = {"bp_mbps": int(bp_mbps), "bh_mbps": int(bh_mbps), "measured_at": time.time(), **extra}
    tmp = path + f".tmp{os.getpid()}"
    with open(tmp, "w") as fh:
        json.dump(data, fh, indent=1)
    os.replace(tmp, path)
    return path


def load(fmt: str, gpu_key: str, directory: str = DEFAULT_DIR):
    """(bp_mbps, bh_mbps) stored for `fmt` on `gpu_key`, or None."""
    path = _path(gpu_key, directory)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    if data.get("gpu") != gpu_key:
        return None
    e = data.get("formats", {}).get(fmt)
    if not e:
        return None
    return int(e["bp_mbps"]), int(e["bh_mbps"])


def gpu_key(device: int = 0) -> str:
    """A stable identity of the GPU: its UUID when the runtime reports one, else name and bus id."""
    import torch
    p = torch.cuda.get_device_properties(device)
    uuid = getattr(p, "uuid", None)
    if uuid:
        return str(uuid)
    return f"{p.name}-{getattr(p, 'pci_bus_id', device)}"
