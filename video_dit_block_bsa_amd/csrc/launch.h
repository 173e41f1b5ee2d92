// Kernel launchers of libbsa.so, called by the C ABI (api.hip). Each returns
// the hipError_t of its launches.
#pragma once

#include "common.h"

namespace bsa {

hipError_t launch_pool(const Geom& g, const bf16_bits* q, const bf16_bits* k, float* qp,
                       float* kp, int blk0, hipStream_t stream);
hipError_t launch_pool_queries(const Geom& g, const bf16_bits* q, float* qp, int blk0,
                               hipStream_t stream);
hipError_t launch_pool_keys(const Geom& g, const bf16_bits* k, float* kp, int blk0, int blk_end,
                            int out_rows, hipStream_t stream);
hipError_t launch_select(const Geom& g, const float* qp, const float* kp, int mode, int k, float p,
                         int k_min, int k_max, int stride, int32_t* idx, int32_t* cnt, int row0,
                         hipStream_t stream);
hipError_t launch_attention(const Geom& g, const bf16_bits* q, const bf16_bits* k,
                            const bf16_bits* v, const int32_t* idx, const int32_t* cnt,
                            int stride, bool dense, bf16_bits* o, float* lse, int q_begin,
                            hipStream_t stream);
hipError_t launch_attention_bwd(const Geom& g, const bf16_bits* q, const bf16_bits* k,
                                const bf16_bits* v, const bf16_bits* o, const bf16_bits* dout,
                                const float* lse, const int32_t* idx, const int32_t* cnt,
                                int stride, float* stats, uint32_t* mask, bf16_bits* dq,
                                bf16_bits* dk, bf16_bits* dv, hipStream_t stream);

}  // namespace bsa
