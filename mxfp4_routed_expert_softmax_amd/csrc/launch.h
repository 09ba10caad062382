// launch.h -- kernel launches of the expert-FFN stage, with optional timing.
// Internal to the HIP library.
//
// k3_launch(kernel, grid, block, stream, args...) launches like <<<>>> (every
// argument explicit, converted to the kernel's parameter types).  While the
// stage is marked (k3moe_set_stage_marks), a launch instead goes through
// hipExtLaunchKernel with the next pair of the caller's events, which then
// hold the start and end of that dispatch itself (no extra packets on the
// stream), and the kind of kernel is noted beside it.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <tuple>

namespace k3 {

constexpr int kMaxMarks = 8;  // kernels per marked stage

struct StageMarkState {
    hipEvent_t ev[2 * kMaxMarks];  // start, end of kernel i at 2i, 2i + 1
    int n;                         // kernels with events
    int* kinds;                    // host [n], may be null
    int* launched;                 // host, may be null
    bool active;                   // a stage is being enqueued with marks set
    int i;                         // kernels launched in it so far
    int kind;                      // kind of the kernels being launched now
};
extern thread_local StageMarkState g_stage_marks;

template <typename... KArgs, typename... Args>
inline void k3_launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, Args... args)
{
    static_assert(sizeof...(KArgs) == sizeof...(Args), "pass every kernel argument");
    std::tuple<KArgs...> formals{static_cast<KArgs>(args)...};
    void* argv[sizeof...(KArgs)];
    std::apply([&](auto&... v) {
        int j = 0;
        ((argv[j++] = static_cast<void*>(&v)), ...);
    }, formals);
    StageMarkState& m = g_stage_marks;
    if (m.active && m.i < m.n) {
        if (m.kinds) m.kinds[m.i] = m.kind;
        (void)hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, s, m.ev[2 * m.i],
                                 m.ev[2 * m.i + 1], 0);
    } else {
        (void)hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, s);
    }
    if (m.active) ++m.i;
}

}  // namespace k3
