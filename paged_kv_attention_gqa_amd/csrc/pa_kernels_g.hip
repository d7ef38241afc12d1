// GQA kernels of the group sizes that are not powers of two (3, 5, 6, 7, 12;
// e.g. 24/8, 40/8, 12/2, 28/4 and 48/4 query/KV heads), compiled apart from
// the powers of two so that the two sets build in parallel.
#include "pa_gqa_kernels.h"

namespace pa {

bool gqa_family_other(int dtype, int d, int dv, int g, GqaFamily* out) {
  return gqa_family_lookup<3, 5, 6, 7, 12>(dtype, d, dv, g, out);
}

}  // namespace pa
