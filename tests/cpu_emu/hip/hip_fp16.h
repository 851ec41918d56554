// CPU stand-in (test infrastructure): fp16 types live in the emulated runtime header.
#pragma once
#include "hip_runtime.h"
