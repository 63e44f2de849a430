// Run-time choice of the compiled kernel instance for a validated call.
#include "../../include/attn.h"
#include "attn_internal.h"
#include "attn_launch.h"

namespace attn {

int launch(const AttnArgs& a, void* stream) {
  switch (a.dtype) {
    case ATTN_BF16:
      switch (a.D) {
        case 32: return launch_inst<ATTN_BF16, 32>(a, stream);
        case 40: return launch_inst<ATTN_BF16, 40>(a, stream);
        case 64: return launch_inst<ATTN_BF16, 64>(a, stream);
        case 80: return launch_inst<ATTN_BF16, 80>(a, stream);
        default: return ATTN_E_UNSUPPORTED;
      }
    case ATTN_F16:
      switch (a.D) {
        case 32: return launch_inst<ATTN_F16, 32>(a, stream);
        case 40: return launch_inst<ATTN_F16, 40>(a, stream);
        case 64: return launch_inst<ATTN_F16, 64>(a, stream);
        case 80: return launch_inst<ATTN_F16, 80>(a, stream);
        default: return ATTN_E_UNSUPPORTED;
      }
    case ATTN_F32:
      if (a.D <= 32) return launch_inst<ATTN_F32, 32>(a, stream);
      if (a.D <= 64) return launch_inst<ATTN_F32, 64>(a, stream);
      return launch_inst<ATTN_F32, 128>(a, stream);
    default:
      return ATTN_E_INVALID;
  }
}

int launch_bwd(const AttnBwdArgs& ba, void* stream) {
  const int dt = ba.a.dtype, d = ba.a.D;
  if (dt == ATTN_BF16) {
    switch (d) {
      case 32: return launch_bwd_inst<ATTN_BF16, 32>(ba, stream);
      case 40: return launch_bwd_inst<ATTN_BF16, 40>(ba, stream);
      case 64: return launch_bwd_inst<ATTN_BF16, 64>(ba, stream);
      case 80: return launch_bwd_inst<ATTN_BF16, 80>(ba, stream);
    }
  } else if (dt == ATTN_F16) {
    switch (d) {
      case 32: return launch_bwd_inst<ATTN_F16, 32>(ba, stream);
      case 40: return launch_bwd_inst<ATTN_F16, 40>(ba, stream);
      case 64: return launch_bwd_inst<ATTN_F16, 64>(ba, stream);
      case 80: return launch_bwd_inst<ATTN_F16, 80>(ba, stream);
    }
  }
  return ATTN_E_UNSUPPORTED;
}

}  // namespace attn
