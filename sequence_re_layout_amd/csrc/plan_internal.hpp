// plan_internal.hpp -- the plan object behind the opaque basp_plan handle.
#pragma once

#include <cstdint>

#include "basp.h"

struct basp_plan {
    // arguments
    int32_t N, B, Hq, Hkv, d;
    int64_t S;
    basp_dtype dtype;
    basp_mode mode;
    basp_layout layout;
    // derived (see basp.h for the meaning)
    int32_t es;          // element size in bytes
    int32_t G, P, Bl;
    int64_t St;
    int32_t Hl_q, Hl_kv;
    int64_t row_bytes;   // d * es: one (token, head) row, the unit every exchange moves whole
    int64_t q_elems, kv_elems;
    // launch shape per direction ([BASP_SEQ_TO_HEAD], [BASP_HEAD_TO_SEQ]);
    // zero fields mean "choose per launch"
    basp_tuning tuning[2];
};

namespace basp {

// Store s as the calling thread's last status and return it.
basp_status record(basp_status s);

// Fields of a tuning within their documented ranges.
bool tuning_in_range(const basp_tuning &t);

// Check that every launch of this plan fits the kernels' index arithmetic
// with the given tuning (the limits are the same in both directions).
basp_status check_launch_limits(const basp_plan &p, const basp_tuning &t);

}  // namespace basp
