// fa_ns.h -- the namespace of the library's internal symbols.
//
// The timeline build (FA_TRACE) puts every internal symbol -- kernels, their
// host launch stubs, the launchers -- in its own inline namespace, so that
// libfa_trace.so and libfa.so can be loaded into one process: their kernels
// then have different names, and neither library's symbols can stand in for
// the other's.
#pragma once

#ifdef FA_TRACE
#define FA_NS_BEGIN namespace fa { inline namespace traced {
#else
#define FA_NS_BEGIN namespace fa { inline namespace plain {
#endif
#define FA_NS_END } }
