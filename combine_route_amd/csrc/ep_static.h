// Internal interface between ep_static.hip (the static scratch array and
// ep_plan_static) and the plan code in ep_plan.cpp. Not installed.
#pragma once

#include <stddef.h>

#include "ep.h"

namespace ep {

// Devices ep_plan_static serves: one static plan object a device.
constexpr int kMaxDevices = 64;

// Sets ep_last_error's message; returns code.
int set_error(int code, const char* msg);
// cfg's checks, and whether its workspace fits scratch_bytes (EP_ERR_SIZE).
int static_plan_check(const ep_config_t* cfg, size_t scratch_bytes);
// Resets device's static plan to cfg over scratch; *out = that plan.
int static_plan_reset(const ep_config_t* cfg, void* scratch, size_t scratch_bytes, int device,
                      ep_plan_t** out);

}  // namespace ep
