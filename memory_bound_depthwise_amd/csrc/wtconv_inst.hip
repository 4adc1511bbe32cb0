// One instantiation unit of the layer's kernels and launch sequences: compiled
// once per kernel size (WTC_K = 3, 5, 7) and activation type (WTC_T = float,
// uint16_t for bfloat16, wtc_f16 for IEEE half), e.g.
//   hipcc -c -DWTC_K=5 -DWTC_T=uint16_t wtconv_inst.hip
// The C ABI (wtconv_api.hip) calls these instances through their declarations
// in wtconv_host.hpp.

#include "wtconv_run.hpp"

#ifndef WTC_K
#error "WTC_K (kernel size) must be defined"
#endif
#ifndef WTC_T
#error "WTC_T (activation storage type) must be defined"
#endif

namespace wtc {

template int run_forward<WTC_K, WTC_T>(const PlanSet &, const void *, const float *, const float *, const float *,
                                       const float *, const float *, void *, char *, hipStream_t, int);
template int run_backward_weight<WTC_K, WTC_T>(const PlanSet &, const void *, const void *, const float *,
                                               const float *, const float *, const float *, const float *,
                                               float *, float *, float *, float *, float *, char *, hipStream_t);
template int plane_grid<WTC_K, WTC_T>(const PlanSet &);
template int mma_grid<WTC_K, WTC_T>(const PlanSet &);
template int tile_grid<WTC_K, WTC_T>(const PlanSet &);

}  // namespace wtc
