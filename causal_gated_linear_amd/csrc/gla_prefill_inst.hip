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

template <int C, int DVT, bool SO, bool NM>
static hipError_t dispatch_gate(const PrefillArgs &a, hipStream_t stream)
{
    constexpr int DK = GLA_INST_DK;
    if (a.gate == kGateKeydim)
        return a.elu1 ? launch_prefill_inst<InstT, DK, C, DVT, kGateKeydim, true, SO, NM>(a, stream)
                      : launch_prefill_inst<InstT, DK, C, DVT, kGateKeydim, false, SO, NM>(a, stream);
    if (a.gate == kGateScalar)
        return a.elu1 ? launch_prefill_inst<InstT, DK, C, DVT, kGateScalar, true, SO, NM>(a, stream)
                      : launch_prefill_inst<InstT, DK, C, DVT, kGateScalar, false, SO, NM>(a, stream);
    return a.elu1 ? launch_prefill_inst<InstT, DK, C, DVT, kGateNone, true, SO, NM>(a, stream)
                  : launch_prefill_inst<InstT, DK, C, DVT, kGateNone, false, SO, NM>(a, stream);
}

// the outer-product gate: the plain full pass only (no segments, no normaliser), with
// chunks of at most 64 rows
template <int C, int DVT>
static hipError_t dispatch_outer(const PrefillArgs &a, hipStream_t stream)
{
    constexpr int DK = GLA_INST_DK;
    if constexpr (C > 64 || prefill_nbuf((int)sizeof(InstT), DK, C, DVT, true) == 0) {
        return hipErrorInvalidValue;               // never chosen
    } else {
        return a.elu1 ? launch_prefill_inst<InstT, DK, C, DVT, kGateOuter, true, false, false>(a, stream)
                      : launch_prefill_inst<InstT, DK, C, DVT, kGateOuter, false, false, false>(a, stream);
    }
}

template <int C, int DVT>
static hipError_t dispatch_mode(const PrefillArgs &a, bool state_only, hipStream_t stream)
{
    if (a.gate == kGateOuter)
        return state_only || a.norm ? hipErrorInvalidValue : dispatch_outer<C, DVT>(a, stream);
    if constexpr (prefill_nbuf((int)sizeof(InstT), GLA_INST_DK, C, DVT) == 0) {
        return hipErrorInvalidValue;               // does not fit in LDS; never chosen
    } else {
        // the normalised form is never segmented: no state-only normalised variant
        if (state_only) return a.norm ? hipErrorInvalidValue : dispatch_gate<C, DVT, true, false>(a, stream);
        return a.norm ? dispatch_gate<C, DVT, false, true>(a, stream) : dispatch_gate<C, DVT, false, false>(a, stream);
    }
}

hipError_t GLA_CAT3(launch_prefill_, GLA_INST_BF16, GLA_INST_DK)(const PrefillArgs &a, int chunk,
                                                                 int dvt, bool state_only,
                                                                 hipStream_t stream)
{
#define GLA_CASE(C, DVT) \
    if (chunk == C && dvt == DVT) return dispatch_mode<C, DVT>(a, state_only, stream);
#define GLA_CASES(C) GLA_CASE(C, 16) GLA_CASE(C, 32) GLA_CASE(C, 64)
    GLA_CASES(16) GLA_CASES(32) GLA_CASES(64)
#if GLA_INST_DK <= 64
    // chunks of 128 rows: only for d_k <= 64 (at d_k = 128 one operand buffer would
    // fill the LDS and the chunk's fragments would not fit in registers)
    GLA_CASES(128)
#endif
#undef GLA_CASES
#undef GLA_CASE
    return hipErrorInvalidValue;
}

}  // namespace gla
