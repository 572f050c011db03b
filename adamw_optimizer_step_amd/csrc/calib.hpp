// Launcher of the MFMA calibration kernel.
#pragma once
#include "common.hpp"

namespace ma {

hipError_t launch_calib_mfma(int blocks, int iters, int changing, float* sink, hipStream_t s);

}  // namespace ma
