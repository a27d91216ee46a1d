// Host-only stand-ins for the kernel launchers (sa::launch_*) so that the C
// ABI's validation code (csrc/api.hip) can be built with g++ under
// AddressSanitizer/UBSan and driven on a machine without a GPU.  Each stand-in
// records the call and returns hipSuccess; no device memory is touched.
#include "launch.h"

namespace sa {

int g_calls = 0;
Shape g_shape{};
SelectParams g_sel{};
FwdParams g_fwd{};
BwdParams g_bwd{};

hipError_t launch_pool(const Shape& s, const void*, const void*, const void*, float*, float*, float*, void*,
                       hipStream_t) {
  ++g_calls;
  g_shape = s;
  return hipSuccess;
}
hipError_t launch_select(const Shape& s, const SelectParams& p, const float*, const float*, int32_t*, int32_t*,
                         hipStream_t) {
  ++g_calls;
  g_shape = s;
  g_sel = p;
  return hipSuccess;
}
hipError_t launch_route_fused(const Shape& s, const SelectParams& p, const void*, const void*, const void*, float*,
                              float*, float*, void*, int32_t*, int32_t*, hipStream_t) {
  ++g_calls;
  g_shape = s;
  g_sel = p;
  return hipSuccess;
}
hipError_t launch_fwd(const Shape& s, const FwdParams& p, const void*, const void*, const void*, const float*,
                      const float*, const void*, const int32_t*, const int32_t*, void*, hipStream_t) {
  ++g_calls;
  g_shape = s;
  g_fwd = p;
  return hipSuccess;
}
hipError_t launch_check_lists(const Shape& s, int, int, const int32_t*, const int32_t*, uint32_t*, hipStream_t) {
  ++g_calls;
  g_shape = s;
  return hipSuccess;
}
// sizes only need to be plausible here; their values are checked against the
// built library by the ABI tests
BwdSizes bwd_sizes(const Shape& s, int approx) {
  BwdSizes z{};
  z.lse = (size_t)s.B * s.Hq * s.N * 4;
  z.delta = 2 * z.lse;
  z.sel_bits = (size_t)s.B * s.Hq * s.M * ((s.M + 31) / 32) * 4;
  z.col_idx = (size_t)s.B * s.Hq * s.M * s.M * 4;
  z.col_cnt = (size_t)s.B * s.Hkv * s.M * 4;
  z.dk_bar = approx ? (size_t)16 * s.B * s.Hkv * s.M * s.D * 4 : 0;
  z.dv_bar = z.dk_bar;
  return z;
}
hipError_t launch_bwd(const Shape& s, const BwdParams& p, const BwdPtrs&, hipStream_t) {
  ++g_calls;
  g_shape = s;
  g_bwd = p;
  return hipSuccess;
}

}  // namespace sa
