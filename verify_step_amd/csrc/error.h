// Thread-local last-error message behind vs_last_error().
#pragma once

#include <string>

#include "../../include/verify_step.h"

vs_status vs_fail(vs_status code, const std::string& msg);
vs_status vs_ok();
