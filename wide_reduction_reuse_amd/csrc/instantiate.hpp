// Instantiates every tile of the ladders in registry.hpp for one operator and
// storage type, plus the work-free control twin of every split tile and, for
// the operators with them, the PART and SHIFT kernels of the 16-byte held tiles,
// and the LDS-tier tiles.
#pragma once

#include "kernels.hpp"
#include "registry.hpp"

namespace credit {

template <OpKind OP, class T, int DT>
void register_op_dtype(std::vector<KernelEntry> &v)
{
    static_assert(OpTraits<OP>::kIn == op_inputs(OP), "registry.hpp's op_inputs must match the operator");
    static_assert(OpTraits<OP>::kQ == op_stats(OP), "registry.hpp's op_stats must match the operator");
    constexpr int VB = 16;
    constexpr int VS = StorageTraits<T>::kBytes;  // one-element access
#define CREDIT_K(kind, vb, block, items, ...)                                                                  \
    if constexpr (tile_enabled(OP, DT, kind, block, items, vb))                                                       \
        v.push_back(KernelEntry{kind, OP, DT, vb, block, items, reinterpret_cast<const void *>(&__VA_ARGS__)})
#define WAVE(it) CREDIT_K(kKindWave, VB, 64, it, single_wave_kernel<OP, T, VB, it>);
#define WG(b, it) CREDIT_K(kKindWg, VB, b, it, single_wg_kernel<OP, T, VB, b, it>);
#define SPLIT(b, it)                                                        \
    CREDIT_K(kKindSplit, VB, b, it, split_kernel<OP, T, VB, b, it, false>); \
    CREDIT_K(kKindControl, VB, b, it, split_kernel<OP, T, VB, b, it, true>);
#define REREAD(b, it) CREDIT_K(kKindReread, VB, b, it, reread_kernel<OP, T, VB, b, it>);
#define WAVE1E(it) CREDIT_K(kKindWave, VS, 64, it, single_wave_kernel<OP, T, VS, it>);
#define WG1E(b, it) CREDIT_K(kKindWg, VS, b, it, single_wg_kernel<OP, T, VS, b, it>);
#define SPLIT1E(b, it)                                                      \
    CREDIT_K(kKindSplit, VS, b, it, split_kernel<OP, T, VS, b, it, false>); \
    CREDIT_K(kKindControl, VS, b, it, split_kernel<OP, T, VS, b, it, true>);
#define REREAD1E(b, it) CREDIT_K(kKindReread, VS, b, it, reread_kernel<OP, T, VS, b, it>);
#define CREDIT_KP(kind, vb, block, items, ...)                                                                  \
    if constexpr (op_has_part(OP, DT) && tile_enabled(OP, DT, kind, block, items, vb))                                    \
        v.push_back(KernelEntry{kind, OP, DT, vb, block, items, reinterpret_cast<const void *>(&__VA_ARGS__), 1})
#define WAVEP(it) CREDIT_KP(kKindWave, VB, 64, it, single_wave_kernel<OP, T, VB, it, true>);
#define WGP(b, it) CREDIT_KP(kKindWg, VB, b, it, single_wg_kernel<OP, T, VB, b, it, true>);
#define SPLITP(b, it) CREDIT_KP(kKindSplit, VB, b, it, split_kernel<OP, T, VB, b, it, false, true>);
#define CREDIT_KO(kind, vb, block, items, ...)                                                                  \
    if constexpr (op_has_shift(OP, DT) && tile_enabled(OP, DT, kind, block, items, vb, 2))                            \
        v.push_back(KernelEntry{kind, OP, DT, vb, block, items, reinterpret_cast<const void *>(&__VA_ARGS__), 2})
#define CREDIT_KL(kind, block, items, lt, ...)                                                                \
    if constexpr (lds_tile_enabled(OP, DT, kind, block, items))                                                        \
        v.push_back(KernelEntry{kind, OP, DT, VB, block, items, reinterpret_cast<const void *>(&__VA_ARGS__), 0, lt})
#define WGL(b, it, lt) CREDIT_KL(kKindWg, b, it, lt, single_wg_kernel<OP, T, VB, b, it, false, false, lt>);
#define SPLITL(b, it, lt) CREDIT_KL(kKindSplit, b, it, lt, split_kernel<OP, T, VB, b, it, false, false, false, lt>);
#define WAVEO(it) CREDIT_KO(kKindWave, VB, 64, it, single_wave_kernel<OP, T, VB, it, true, true>);
#define WGO(b, it) CREDIT_KO(kKindWg, VB, b, it, single_wg_kernel<OP, T, VB, b, it, true, true>);
#define SPLITO(b, it)                                                                         \
    if constexpr (op_shifts_split(OP, DT))                                                    \
        CREDIT_KO(kKindSplit, VB, b, it, split_kernel<OP, T, VB, b, it, false, true, true>);

    CREDIT_WAVE_TILES(WAVE)
    CREDIT_WG_TILES(WG)
    CREDIT_SPLIT_TILES(SPLIT)
    CREDIT_REREAD_TILES(REREAD)
    CREDIT_WAVE_TILES_1E(WAVE1E)
    CREDIT_WG_TILES_1E(WG1E)
    CREDIT_SPLIT_TILES_1E(SPLIT1E)
    CREDIT_REREAD_TILES_1E(REREAD1E)
    CREDIT_WAVE_TILES(WAVEP)
    CREDIT_WG_TILES(WGP)
    CREDIT_SPLIT_TILES(SPLITP)
    CREDIT_WAVE_TILES(WAVEO)
    CREDIT_WG_TILES(WGO)
    CREDIT_SPLIT_TILES(SPLITO)
    CREDIT_WG_LDS_TILES(WGL)
    CREDIT_SPLIT_LDS_TILES(SPLITL)

#undef WAVE
#undef WG
#undef SPLIT
#undef REREAD
#undef WAVE1E
#undef WG1E
#undef SPLIT1E
#undef REREAD1E
#undef WAVEP
#undef WGP
#undef SPLITP
#undef WAVEO
#undef WGO
#undef SPLITO
#undef WGL
#undef SPLITL
#undef CREDIT_KL
#undef CREDIT_KO
#undef CREDIT_KP
#undef CREDIT_K
}

}  // namespace credit
