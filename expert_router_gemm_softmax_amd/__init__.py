"""One GPU's share of an expert-parallel MoE layer on MI355X (gfx950).

Router softmax/top-k with capacity drop, permute into per-expert buffers,
grouped expert FFN GEMMs on bf16 MFMA, gate-weighted combine, and the full
backward, as hand-written HIP kernels behind the C-ABI of include/moe.h.
The Python side only marshals arguments; importing fails loudly when
libmoe.so has not been built.
"""
from .binding import (KERNELS, KernelProbe, MOE_BF16, MOE_FLAG_DROP_IDENTITY, MOE_FLAG_RECOMPUTE,
                      MOE_FLAG_RENORM,
                      MOE_FLAG_SLOT_PRIORITY, MOE_FP32, MOE_NO_CAPACITY,
                      MoeCfg, MoeCtx, MoeProbe,
                      MoeError, MoeGrads, MoeLibraryError, MoeWeights, LIB_PATH,
                      make_cfg, moe_capacity, moe_check_cfg, moe_combine,
                      moe_combine_bwd, moe_grouped_ffn, moe_grouped_ffn_bwd,
                      moe_layer_bwd, moe_layer_fwd, moe_permute, moe_permute_noalloc,
                      moe_route, moe_route_bwd, moe_router_aux,
                      moe_rows_max,
                      moe_unpermute_bwd, moe_workspace_bytes, status_str)
from .layer import MoeLayer

__all__ = [n for n in dir() if n.startswith(("moe_", "Moe", "MOE_"))] + [
    "KERNELS", "KernelProbe", "LIB_PATH", "make_cfg", "status_str"]
