"""Small host fixtures for the oracle self-tests: paged caches built from synth draws."""
import math
import struct

import numpy as np

import synth
from oracle import compress as oc


def pure_table(rows, rdims, theta=10000.0):
    """cos/sin table in pure Python (math.cos/sin in double, rounded to fp32 with struct)."""
    def r32(v):
        return struct.unpack("f", struct.pack("f", v))[0]
    t = []
    for p in range(rows):
        t.append([(r32(math.cos(p * theta ** (-2.0 * j / rdims))), r32(math.sin(p * theta ** (-2.0 * j / rdims))))
                  for j in range(rdims // 2)])
    return t


def empty_cache(ratio, window, dim, rdims, dtype, batch, n_blocks, n_phys, g):
    e = 256 // ratio
    if dtype == "f32":
        pages = np.full((n_phys * e, dim), np.nan, dtype=np.float32)
    elif dtype == "bf16":
        pages = np.full((n_phys * e, dim), 0x7FC0, dtype=np.uint16)
    else:
        pages = np.full((n_phys * e, dim), 0x7F, dtype=np.uint8)
    scales = np.full(n_phys * e, np.nan, dtype=np.float32) if dtype == "fp8" else None
    bt = synth.random_block_table(g, batch, n_blocks, n_phys)
    return oc.Cache(ratio, window, dim, rdims, dtype, pages, scales, bt)


def empty_state(dim, roles, dtype, bt, n_phys):
    if dtype == "f32":
        kv = np.zeros((n_phys * 256, dim), dtype=np.float32)
        lg = np.zeros((n_phys * 256, roles, dim), dtype=np.float32)
    else:
        kv = np.zeros((n_phys * 256, dim), dtype=np.uint16)
        lg = np.zeros((n_phys * 256, roles, dim), dtype=np.uint16)
    return oc.Raw(dtype, dim, roles, kv, lg, None, bt.copy())


def raw_tokens(config, n_tok, dim, roles, dtype, stream_kv=0, stream_lg=1):
    gk, gl = synth.rng(config, stream_kv), synth.rng(config, stream_lg)
    if dtype == "f32":
        return synth.normal_f32(gk, (n_tok, dim)), synth.normal_f32(gl, (n_tok, roles, dim))
    return synth.normal_bf16_bits(gk, (n_tok, dim)), synth.normal_bf16_bits(gl, (n_tok, roles, dim))
