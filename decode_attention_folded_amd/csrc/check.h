// Launcher of the device-side precondition check (check.hip), a debugging
// aid kept apart from the attention and Quest kernels' declarations.
#pragma once

#include <stdint.h>

namespace da {

struct CheckLaunch {
  const int32_t* seqlens;     // [B]
  const int32_t* page_table;  // [B, max_pages] or nullptr
  int32_t* report;            // [4]: bad lengths, bad page entries, lowest offending batch, 0
  int32_t batch, capacity, page_shift, max_pages;
  int64_t num_pages;
};

int launch_check(const CheckLaunch& p, void* stream);

}  // namespace da
