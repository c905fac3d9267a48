// The Q/K-norm kernels with an fp8 (E4M3) cache (templates in rkv_kernels.hpp).
#include "rkv_kernels.hpp"

namespace rkv {

hipError_t launch_contig_norm_fp8(const ContigParams& p, int call, int D, int style, bool exact,
                                  hipStream_t stream) {
  return detail::launch_contig_t<true, true>(p, call, D, style, exact, stream);
}

}  // namespace rkv
