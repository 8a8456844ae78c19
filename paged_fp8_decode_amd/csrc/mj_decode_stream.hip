// Decode kernel dispatch.  The generic LDS-tiled kernel serves every shape.
#include "mj_device.h"
#include "mj_internal.h"

namespace mj {

hipError_t launch_decode(const DecodeParams& p, int kv_format, int row_tiles, hipStream_t s) {
  return launch_decode_generic(p, kv_format, row_tiles, s);
}

}  // namespace mj
