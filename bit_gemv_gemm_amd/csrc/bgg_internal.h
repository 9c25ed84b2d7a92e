// Internal declarations shared by the host and device halves of libbgg.
#pragma once
#include "../../include/bgg.h"

namespace bgg {
// Record a thread-local error message and return `st`.
bgg_status fail(bgg_status st, const char* fmt, ...);
void clear_error();
// BGG_OK iff `d` is exactly what bgg_describe makes for its format and shape.
bgg_status check_desc(const bgg_weights_desc* d);
}  // namespace bgg
