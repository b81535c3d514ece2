// Diagnostics switches of the C ABI, read once per process from the environment:
//   RBQ_LOG=1               every entry point prints its launch decision to stderr;
//   RBQ_FAULT_INJECT=launch every entry point that passed validation reports RBQ_EHIP
//                           without launching, so callers can exercise their error paths
//                           on a machine without a GPU.
// Host code only; nothing here touches the device.
#pragma once

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

namespace rbq {

inline bool diag_log() {
  static const bool on = [] {
    const char* v = getenv("RBQ_LOG");
    return v && v[0] && strcmp(v, "0") != 0;
  }();
  return on;
}

inline bool diag_fail_launch() {
  static const bool on = [] {
    const char* v = getenv("RBQ_FAULT_INJECT");
    return v && strcmp(v, "launch") == 0;
  }();
  return on;
}

}  // namespace rbq
