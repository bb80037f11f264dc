// Host-side static scheduler: per-CU instruction lists for one decode step.
#pragma once
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_types.h"

struct MkPlan {
  int n_cus = 0;
  int page_bytes = 0;   // bytes per LDS page
  int slots = 0;        // pages in the LDS ring (set by the launcher for the shape's kernel)
  int s_max = 0;        // attention splits per KV head
  int min_chunk = 0;    // fewest keys one split covers
  int nch = 0;          // K-chunks of the down projection
  std::vector<int32_t> off;      // [n_cus + 1] list offsets into rec
  std::vector<MkInstr> rec;      // all lists back to back
};

// Validate `c` against the compiled shapes and the kernel's limits; on failure return
// MK_EINVAL and say why.  *nch receives the shape's down-projection chunk count.
int mk_check_config(const mk_config& c, std::string* why, int* nch = nullptr);

// Build the per-CU lists for `n_cus` compute units.  Deterministic.
int mk_build_plan(const mk_config& c, int n_cus, MkPlan* out, std::string* why);
