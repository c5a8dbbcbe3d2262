// State of the recording launchers (fake_launch.cpp).
#pragma once
#include "launch.h"

namespace fake {
extern int launches;               // launches recorded since the last reset
extern const char* last;           // launcher of the last one
extern int64_t last_B, last_H, last_N, last_d;
extern const void* last_ws;        // workspace the backward launch received
extern hipError_t next_status;     // what every launcher returns
extern hipError_t scratch_status;  // what the workspace lookup returns
extern float scratch_stand_in[64];
}  // namespace fake
