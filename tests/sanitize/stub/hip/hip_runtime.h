// Host-only stand-in for <hip/hip_runtime.h>: the runtime API subset only.
#pragma once
#include "hip_runtime_api.h"
