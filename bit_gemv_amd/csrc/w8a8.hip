// w8a8.hip -- INT8 x INT8 GEMM (int8 MFMA). Placeholder until the MFMA
// kernel lands: reports "not supported".
#include "launch.hpp"
namespace lq {
hipError_t launch_w8a8_gemm(const W8Args &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace lq
