// Internal: the object behind the opaque sva_plan handle.
#pragma once

#include "kernels.h"
#include "plan_host.h"

struct sva_plan_s {
    sva::HostPlan host;
    sva::DevPlan dev{};
    int device = 0;
    void* dmem = nullptr;   // one allocation holding every device table
};

namespace sva {
// Resolves, once per device, the address of the library's fixed selection
// scratch on device `dev` (which must be current); called at plan creation.
hipError_t resolve_select_scratch(int dev);
}  // namespace sva
