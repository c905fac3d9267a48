// The Q/K-norm kernels with an fp16 cache (templates in rkv_kernels.hpp).
#include "rkv_kernels.hpp"

namespace rkv {

hipError_t launch_contig_norm(const ContigParams& p, int call, int D, int style, bool exact,
                              hipStream_t stream) {
  return detail::launch_contig_t<false, true>(p, call, D, style, exact, stream);
}

}  // namespace rkv
