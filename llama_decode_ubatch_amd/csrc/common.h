// Error and log reporting shared by the library's translation units.
#pragma once

#include <string>

namespace ubd {

// Records the message for ubd_last_error() on this thread and logs it.
void set_error(const std::string &msg);
// Logs through the callback set with ubd_log_set (level 1 info, 2 error).
void log_msg(int level, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace ubd
