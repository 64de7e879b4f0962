// Kernel launch helper: hipLaunchKernel returns the launch's own status, so a failure is
// attributed to this call and not to whatever the caller did before.
#pragma once

#include <hip/hip_runtime.h>

namespace dh {

template <typename... Args>
inline hipError_t launch(void (*kernel)(Args...), dim3 grid, dim3 block, size_t lds,
                         hipStream_t stream, Args... args)
{
    void *argv[] = {(void *)&args..., nullptr};
    return hipLaunchKernel((const void *)kernel, grid, block, argv, lds, stream);
}

// Resident workgroups per CU of a kernel at a block size, computed once per instantiation.
template <typename K>
inline int occupancy(K kernel, int block, int &cache)
{
    int occ = __atomic_load_n(&cache, __ATOMIC_RELAXED);
    if (occ > 0)
        return occ;
    occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, block, 0) != hipSuccess ||
        occ < 1)
        occ = 1;
    __atomic_store_n(&cache, occ, __ATOMIC_RELAXED);
    return occ;
}

}  // namespace dh
