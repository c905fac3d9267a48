// The fp8 (E4M3) cache kernels (templates in rkv_kernels.hpp).
#include "rkv_kernels.hpp"

namespace rkv {

hipError_t launch_contig_fp8(const ContigParams& p, int call, int D, int style, bool exact,
                             hipStream_t stream) {
  return detail::launch_contig_t<true, false>(p, call, D, style, exact, stream);
}

hipError_t launch_paged_fp8(const PagedParams& p, int D, int style, bool exact, bool gather,
                            bool late_loads, hipStream_t stream) {
  return detail::launch_paged_t<true>(p, D, style, exact, gather, late_loads, stream);
}

}  // namespace rkv
