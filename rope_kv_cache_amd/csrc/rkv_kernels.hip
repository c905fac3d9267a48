// The fp16-cache kernels (templates in rkv_kernels.hpp).
#include "rkv_kernels.hpp"

namespace rkv {

hipError_t launch_contig(const ContigParams& p, int call, int D, int style, bool exact,
                         hipStream_t stream) {
  return detail::launch_contig_t<false, false>(p, call, D, style, exact, stream);
}

hipError_t launch_paged(const PagedParams& p, int D, int style, bool exact, bool gather,
                        bool late_loads, hipStream_t stream) {
  return detail::launch_paged_t<false>(p, D, style, exact, gather, late_loads, stream);
}

}  // namespace rkv
