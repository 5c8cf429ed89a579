// Error reporting shared by the C ABI translation units: records the
// message returned by pa_last_error() (per thread) and returns `code`.
#pragma once

namespace pa {
int record_error(int code, const char* fmt, ...);
void clear_error();
}  // namespace pa
