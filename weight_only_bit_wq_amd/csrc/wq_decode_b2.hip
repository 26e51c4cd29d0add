// Decode kernels for b = 2 (one bit width per translation unit so the
// library builds in parallel).
#include "wq_decode_kernel.h"

namespace wq {
template hipError_t decode_b<2, NoGroups>(const uint16_t *, int64_t, int64_t, int64_t,
                                          const void *, bool, const uint16_t *, const uint8_t *,
                                          uint16_t *, void *, const DecodePlan &,
                                          const NoGroups &, hipStream_t);
template hipError_t decode_b<2, GroupTable>(const uint16_t *, int64_t, int64_t, int64_t,
                                            const void *, bool, const uint16_t *,
                                            const uint8_t *, uint16_t *, void *,
                                            const DecodePlan &, const GroupTable &, hipStream_t);
}  // namespace wq
