// Thread-local error text and status helpers shared by the host-side entry points.
#pragma once
#include <cstdarg>
#include <cstdio>

#include "tree_attn.h"

namespace ta {

// Records a formatted message for tree_attn_last_error() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

}  // namespace ta
