// Host-side static scheduler: per-CU instruction lists for one decode step.
#pragma once
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_types.h"

struct MkPlan {
  int n_cus = 0;
  int page_bytes = 0;   // bytes per LDS page
  int slots = 0;        // pages in the LDS ring
  int s_max = 0;        // attention splits per KV head
  int min_chunk = 0;    // fewest keys one split covers
  std::vector<int32_t> off;      // [n_cus + 1] list offsets into rec
  std::vector<MkInstr> rec;      // all lists back to back
};

// Validate `c` for the kernel's limits; on failure return MK_EINVAL and say why.
int mk_check_config(const mk_config& c, std::string* why);

// Build the per-CU lists for `n_cus` compute units.  Deterministic.
int mk_build_plan(const mk_config& c, int n_cus, MkPlan* out, std::string* why);
