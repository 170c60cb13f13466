// Thread-local last-error message shared by the library's C entry points.
#pragma once

namespace pa {

// Formats the message into the calling thread's buffer and returns status.
int set_error(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Empties the message; returns PA_OK (0).
int clear_error();
const char *last_error();

}  // namespace pa
