// ssd_stage.h -- constants shared by the kernels that stage token rows of X
// and B from HBM into LDS.
#pragma once

#include "ssd_device.h"

namespace ssd {

constexpr int kPassRows = 128;  // token rows staged per pass

}  // namespace ssd
