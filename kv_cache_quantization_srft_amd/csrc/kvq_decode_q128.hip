// Fused decode attention over the quantized cache, head dimension 128 (the kernels are in
// kvq_decode_q.h).
#include "kvq_decode_q.h"

namespace kvq_impl {
template hipError_t launch_decode_d<128>(const DecodeArgs& a, const DecodePlan& p, hipStream_t s);
}  // namespace kvq_impl
