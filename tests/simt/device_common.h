// Host stand-in of the device helpers the plan kernels use (emulation only).
#pragma once
#include "simt.h"
#define MOK_DEV inline
#define MOK_HOSTDEV
#define __global__
#define __launch_bounds__(x)
#define __restrict__
inline int lane_id() { return __lane_id(); }
constexpr int kWave = 64;
