// Compiled kernel instances.  Each (dtype, head dim) pair is built from
// attn_inst.hip as its own object; attn_dispatch.cpp picks one at run time.
#ifndef ATTN_LAUNCH_H_
#define ATTN_LAUNCH_H_

#include "attn_internal.h"

namespace attn {

// DT: ATTN_F16 / ATTN_BF16 with D in {32, 40, 64, 80}; ATTN_F32 with D the
// register bucket (32, 64, 128) holding the runtime head dim.
template <int DT, int D>
int launch_inst(const AttnArgs& a, void* stream);

// The backward of a validated call (half precision only).
template <int DT, int D>
int launch_bwd_inst(const AttnBwdArgs& ba, void* stream);

}  // namespace attn

#endif  // ATTN_LAUNCH_H_
