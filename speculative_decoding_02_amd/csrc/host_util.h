// host_util.h -- host helpers shared by the C-ABI translation units.
#pragma once
#include <string>

#include "spec.h"

namespace spec_host {

// printf-style formatting into a std::string (messages up to 511 bytes).
std::string fmt(const char* f, ...);
// The thread's last error message, returned by spec_last_error(NULL).
void set_last_error(const std::string& msg);
// Shape and pointer checks of a model description; on failure *why says which.
bool valid_model(const spec_model_desc& m, std::string* why);

}  // namespace spec_host
