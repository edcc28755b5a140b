"""Routed-expert MoE layer forward for AMD Instinct MI355X (gfx950).

Hot path (HIP kernels in libmoe.so, C ABI in include/moe.h): router
softmax + top-k, stable permutation by expert, grouped SwiGLU expert FFN over
bf16 / MXFP4 / INT4-group-32 weights with in-register dequant, weighted
combine, and an LRU expert-residency cache in HBM filled from pinned host
memory.  PyTorch provides device memory and streams only.
"""
from .api import (DT, FMT, ExpertCache, experts_desc, moe_combine, moe_compress_bound, moe_compress_package,
                  moe_compress_rans, moe_compress_rans_bound, moe_decompress_packages, moe_decompress_rans, moe_dequant_expert, moe_expert_ffn,
                  moe_ffn_workspace, moe_pack_expert, moe_package_bytes, moe_permute, moe_permute_workspace,
                  moe_route, moe_route_permute, moe_route_permute_workspace)
from ._lib import MoeError, header_symbols, lib

__all__ = ["DT", "FMT", "ExpertCache", "experts_desc", "moe_combine", "moe_compress_bound", "moe_compress_package",
           "moe_compress_rans", "moe_compress_rans_bound", "moe_decompress_packages", "moe_decompress_rans", "moe_dequant_expert", "moe_expert_ffn",
           "moe_ffn_workspace", "moe_pack_expert", "moe_package_bytes", "moe_permute", "moe_permute_workspace",
           "moe_route", "moe_route_permute", "moe_route_permute_workspace", "MoeError", "header_symbols", "lib"]
