// Host-only stand-in (see hip_runtime.h next to it).
#pragma once
#include "hip_runtime.h"
