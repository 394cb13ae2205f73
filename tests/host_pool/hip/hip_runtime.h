/* Host-only stand-in (see hip_runtime_api.h).  Test infrastructure. */
#ifndef MOE_FAKE_HIP_RUNTIME_H
#define MOE_FAKE_HIP_RUNTIME_H
#include "hip_runtime_api.h"
#endif
