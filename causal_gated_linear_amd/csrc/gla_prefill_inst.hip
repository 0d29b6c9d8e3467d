// gla_prefill_inst.hip -- explicit instantiations of the prefill kernel for one
// (element type, d_k) pair, selected at build time with -DGLA_INST_BF16=0|1 and
// -DGLA_INST_DK=16|32|64|128, so the instantiations compile in parallel.
#include "gla_prefill.hpp"

#ifndef GLA_INST_BF16
#error "define GLA_INST_BF16"
#endif
#ifndef GLA_INST_DK
#error "define GLA_INST_DK"
#endif

#define GLA_CAT3_(a, b, c) a##b##_##c
#define GLA_CAT3(a, b, c) GLA_CAT3_(a, b, c)

namespace gla {

#if GLA_INST_BF16
typedef bf16 InstT;
#else
typedef float InstT;
#endif

hipError_t GLA_CAT3(launch_prefill_, GLA_INST_BF16, GLA_INST_DK)(const PrefillArgs &a, int chunk,
                                                                 int dvt, int nw, hipStream_t stream)
{
    constexpr int DK = GLA_INST_DK;
#define GLA_CASE(C, DVT, NW) \
    if (chunk == C && dvt == DVT && nw == NW) return launch_prefill_inst<InstT, DK, C, DVT, NW>(a, stream);
#define GLA_CASES(C) GLA_CASE(C, 16, 4) GLA_CASE(C, 32, 4) GLA_CASE(C, 64, 4)
    GLA_CASES(16) GLA_CASES(32) GLA_CASES(64)
#if GLA_INST_DK >= 32
    GLA_CASE(16, 64, 8) GLA_CASE(32, 64, 8) GLA_CASE(64, 64, 8)
#endif
#undef GLA_CASES
#undef GLA_CASE
    return hipErrorInvalidValue;
}

}  // namespace gla
