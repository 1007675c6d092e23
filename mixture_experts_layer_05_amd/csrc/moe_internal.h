// Host-side helpers shared by the entry points: argument checks and a
// kernel launcher that reports the launch's own status.
#pragma once

#include <tuple>
#include <utility>

#include "moe.h"
#include "moe_device.h"

namespace moe {

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

template <typename Tuple, size_t... I>
inline hipError_t launch_impl(const void* fn, dim3 g, dim3 b, size_t lds, hipStream_t s,
                              Tuple& t, std::index_sequence<I...>) {
  void* args[] = {static_cast<void*>(&std::get<I>(t))..., nullptr};
  return hipLaunchKernel(fn, g, b, args, lds, s);
}

// Launches `kernel` with the arguments converted to the kernel's own
// parameter types; returns hipLaunchKernel's status for this launch.
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                         hipStream_t stream, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  std::tuple<KArgs...> t(static_cast<KArgs>(args)...);
  return launch_impl(reinterpret_cast<const void*>(kernel), grid, block, lds, stream, t,
                     std::index_sequence_for<KArgs...>{});
}

// Raises a kernel's dynamic-LDS limit once when it needs more than 64 KiB.
template <typename... KArgs>
inline hipError_t allow_lds(void (*kernel)(KArgs...), size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(bytes));
}

inline moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Compute units of the current device, queried once per device and cached
// (256 on MI355X); 256 if the query fails.
int device_cu_count();

inline size_t elt_size(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }

// Router logits z[s][T][E] (fp32; s < route_logit_slabs K slabs whose sum is
// the logit, the bias in slab 0), as moe_route computes them.
int route_logit_slabs(moe_dtype dt, int64_t T, int64_t d, int32_t E);
hipError_t launch_route_logits(hipStream_t stream, moe_dtype dt, int64_t T, int64_t d, int32_t E,
                               const void* x, const void* w_router, const float* logit_bias,
                               float* z);

}  // namespace moe
