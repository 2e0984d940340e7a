// Internal helpers shared by the host-side sources of libmlora.so.
#ifndef MLORA_INTERNAL_H_
#define MLORA_INTERNAL_H_

#include <cstdint>

namespace mlora {

// Records the message returned by mlora_last_error() and passes `code` on.
int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the last-error message at the start of a successful call.
void clear_error();

}  // namespace mlora

#endif  // MLORA_INTERNAL_H_
