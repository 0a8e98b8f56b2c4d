// gemm.hip -- W4A16 prefill GEMM (bf16 MFMA). Placeholder until the MFMA
// kernel lands: reports "not supported".
#include "launch.hpp"
namespace lq {
hipError_t launch_w4a16_gemm(const W4Args &, hipStream_t) { return hipErrorNotSupported; }
}  // namespace lq
