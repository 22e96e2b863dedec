// Status codes and the per-thread error message shared by the C entry points.
#pragma once
#include <cstdarg>
#include <cstdio>
#include <string>

#include "orca.h"

namespace orca {

void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

}  // namespace orca

#define ORCA_CHECK_ARG(cond, ...)          \
  do {                                     \
    if (!(cond)) {                         \
      ::orca::set_error(__VA_ARGS__);      \
      return ORCA_ERR_INVALID;             \
    }                                      \
  } while (0)
