// bkv_step.hpp -- launcher of a decode step's collection-phase work in one
// launch (library-internal).
#pragma once

#include "bkv_internal.hpp"

namespace bkv {

// The FPS buffer update `a` (bkv_fps_update's rule, FPS source) together with
// the key and value append `app` of the same step.
hipError_t launch_fps_step(const FpsArgs& a, const AppendArgs& app, int d, hipStream_t st);

}  // namespace bkv
